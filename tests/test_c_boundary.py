"""The attention path driven from a plain C program (tests/c_abi/fox_c_smoke.c) through the C ABI
of include/fox.h: device memory from hipMalloc, no Python or PyTorch in that process. Its outputs
must equal, bit for bit, those of the Python binding on the same inputs (same kernels), and match
the fp64 oracle at the bf16 bar.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import fox_inputs as fi
import oracle
from tests.fox_testlib import check, dev

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "fox_c_smoke")

pytestmark = pytest.mark.gpu


def _bf16_bits(a):
    """bf16 bit patterns of fp32 values that bf16 represents exactly (fox_inputs rounds them)."""
    return (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("B,H,L,D", [(1, 3, 333, 64), (2, 2, 700, 128)])
def test_c_program_matches_binding_and_oracle(tmp_path, B, H, L, D):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built (python -m gated_softmax_attention_fox_amd.build)")
    import gated_softmax_attention_fox_amd as fox
    case = fi.make_case(B, H, L, D, "bf16", seed=60 + L, gate="per_head", with_do=True)
    ind, outd = tmp_path / "in", tmp_path / "out"
    ind.mkdir()
    outd.mkdir()
    for name, arr in (("q", case.q), ("k", case.k), ("v", case.v), ("do", case.do)):
        _bf16_bits(arr).tofile(ind / f"{name}.bin")
    np.ascontiguousarray(case.log_f, np.float32).tofile(ind / "logf.bin")
    print(f"C program B={B} H={H} L={L} D={D}", flush=True)
    r = subprocess.run([EXE, str(B), str(H), str(L), str(D), str(ind), str(outd)],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    shp4, shp3 = (B, H, L, D), (B, H, L)
    got = {n: np.fromfile(outd / f"{n}.bin", np.float32).reshape(shp3 if n in ("lse", "dlogf") else shp4)
           for n in ("o", "lse", "dq", "dk", "dv", "dlogf")}

    # the same calls through the binding, with the C program's scale (1.0f / sqrtf(D) in fp32)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    q, k, v, do = (dev(a, "bf16") for a in (case.q, case.k, case.v, case.do))
    c = fox.fox_logf_cumsum(dev(case.log_f, "f32"))
    o, lse = fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32, scale=scale)
    dq, dk, dv, dlf = fox.fox_attn_bwd(q, k, v, c, o, lse, do, scale=scale)
    torch.cuda.synchronize()
    for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("dlogf", dlf)):
        assert np.array_equal(got[n], t.cpu().numpy()), f"{n}: C program and binding differ"

    O, LSE = oracle.attn_fwd(case.q, case.k, case.v, case.log_f, scale=scale)
    dQ, dK, dV, dLF = oracle.attn_bwd(case.q, case.k, case.v, case.log_f, case.do, scale=scale)[:4]
    check("O", got["o"], O)
    check("LSE", got["lse"], LSE)
    check("dQ", got["dq"], dQ)
    check("dK", got["dk"], dK)
    check("dV", got["dv"], dV)
    check("d log f", got["dlogf"], dLF)
