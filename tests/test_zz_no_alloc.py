"""fox_attn_bwd_noalloc, the backward on the library's static scratch, against fox_attn_bwd.

Both run the same kernels, so the results must be bit-identical. Two calls in a row share the
GPU's scratch array; the second, on a smaller input, must not see the first call's contents.
"""
import numpy as np
import pytest
import torch

import fox_inputs as fi
from tests.fox_testlib import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fox():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_softmax_attention_fox_amd as f
    f.load_library()
    return f


def _inputs(fox, B, H, L, D, dtype, seed, plan=False):
    case = fi.make_case(B, H, L, D, dtype, seed=seed, with_do=True, gate="per_head",
                        head_mean_range=(-1.0, 6.0))
    q, k, v, do = (dev(getattr(case, n), dtype) for n in ("q", "k", "v", "do"))
    c = fox.fox_logf_cumsum(dev(case.log_f, "f32"))
    o, lse = fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32)
    sp = fox.fox_attn_skip_plan(q, k, c) if plan else None
    return q, k, v, c, o, lse, do, sp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_backward(fox, dtype):
    """Two calls in a row, the second smaller, each bit-identical to fox_attn_bwd."""
    shapes = [(2, 6, 3000, 128), (1, 3, 700, 64)] if dtype == "bf16" else [(1, 4, 900, 128),
                                                                           (1, 2, 300, 64)]
    for n, (B, H, L, D) in enumerate(shapes):
        say(f"noalloc call {n}: B={B} H={H} L={L} D={D} {dtype}")
        q, k, v, c, o, lse, do, _ = _inputs(fox, B, H, L, D, dtype, seed=70 + n)
        ref = fox.fox_attn_bwd(q, k, v, c, o, lse, do)
        out = tuple(torch.full_like(t, float("nan")) for t in ref)
        got = fox.fox_attn_bwd_noalloc(q, k, v, c, o, lse, do, out=out)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV", "dlog f"), ref, got):
            assert torch.equal(a, b), f"{name}: differs from fox_attn_bwd (call {n})"


def test_noalloc_with_skip_plan(fox):
    """With a skip plan, then again without one on a smaller input."""
    for n, (B, H, L, D, plan) in enumerate([(1, 4, 4097, 128, True), (1, 2, 1000, 64, False)]):
        say(f"noalloc call {n}: B={B} H={H} L={L} D={D} plan={plan}")
        q, k, v, c, o, lse, do, sp = _inputs(fox, B, H, L, D, "bf16", seed=80 + n, plan=plan)
        ref = fox.fox_attn_bwd(q, k, v, c, o, lse, do, skip_plan=sp)
        got = fox.fox_attn_bwd_noalloc(q, k, v, c, o, lse, do, skip_plan=sp)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV", "dlog f"), ref, got):
            assert torch.equal(a, b), f"{name}: differs from fox_attn_bwd (call {n})"


def test_noalloc_rejects_sizes_beyond_the_scratch(fox):
    """B*H*L above what the static array holds is refused before any launch."""
    lib = fox.load_library()
    held = int(lib.fox_attn_bwd_noalloc_max_bytes())
    assert held == 4 * (1 << 21) * 4
    B, H, L, D = 1, 2, (1 << 20) + 64, 64  # B*H*L just above 2^21
    x = torch.zeros(B, H, L, D, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(B, H, L, dtype=torch.float32, device="cuda")
    o = torch.zeros(B, H, L, D, dtype=torch.float32, device="cuda")
    with pytest.raises(fox.FoxError, match="static scratch"):
        fox.fox_attn_bwd_noalloc(x, x, x, c, o, c, x)
