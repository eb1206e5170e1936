"""Helpers for the GPU parity tests: upload seeded inputs, compare against the oracle."""
import math
import sys

import numpy as np
import torch

import fox_inputs as fi

# Tolerances of the path (bf16 inputs with fp32 accumulation / the fp32 workload).
BF16_MAXABS = 2e-2
BF16_RELL2 = 5e-3
F32_MAXABS = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload the exact values of a (bf16-representable for dtype == 'bf16')."""
    if dtype == "bf16":
        return torch.from_numpy(fi.bf16_bits(a)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """fp64 NumPy copy (bf16 widened exactly; fp64 kept as is)."""
    t = t.detach()
    if t.dtype != torch.float64:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    maxabs = float(np.abs(d).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)) if d.size else 0.0
    return maxabs, rel


def check(name, got, ref, maxabs=BF16_MAXABS, rel_l2=BF16_RELL2, quiet=False):
    """Assert max-abs and relative-L2 bars; quiet prints only on failure."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    m, r = errors(got, ref)
    # relative L2 is meaningless for a reference that is (numerically) zero, e.g. dQ at L = 1
    if rel_l2 is not None and np.linalg.norm(np.asarray(ref, np.float64)) < 1e-6:
        rel_l2 = None
    rl = "n/a" if rel_l2 is None else f"{rel_l2:g}"
    bad = m > maxabs or (rel_l2 is not None and r > rel_l2)
    if bad or not quiet:
        say(f"  {name}: max-abs {m:.3e} (<= {maxabs:g})  rel-L2 {r:.3e} (<= {rl})")
    assert m <= maxabs, f"{name}: max-abs {m:.3e} > {maxabs:g}"
    if rel_l2 is not None:
        assert r <= rel_l2, f"{name}: rel-L2 {r:.3e} > {rel_l2:g}"


def sample_rows(L, n, seed, tile=64):
    """Rows that cover the start, tile edges, the end and random interior rows."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, L - 1, L - 2, min(L - 1, tile - 1), min(L - 1, tile), min(L - 1, 2 * tile + 3),
             L // 2}
    rnd = set(rng.integers(0, L, size=n).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < L))


def default_scale(D):
    return 1.0 / math.sqrt(D)


def check_y(name, got, Y, O, g, eps, weight=None, y_bf16=False):
    """Check the fused output gate y = RMSNorm(O) [* w] * sigmoid(g) against the oracle's Y, where
    O is the oracle's attention output. An error e in O reaches y as r (1 + r |O_j|) |w_j|
    sigmoid(g_j) e per element (r = 1 / sqrt(mean O^2 + eps) of the row: the element's own term
    and the change of the row's RMS), so the max-abs bar is the attention bar carried through
    that factor, element by element, plus half a bf16 ulp of y when y is stored in bf16. Relative
    L2 keeps the attention bar."""
    got = np.asarray(got, np.float64)
    Y = np.asarray(Y, np.float64)
    O = np.asarray(O, np.float64)
    g = np.asarray(g, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = 1.0 / np.sqrt(np.mean(O * O, axis=-1, keepdims=True) + eps)
    w = np.ones(O.shape[-1]) if weight is None else np.abs(np.asarray(weight, np.float64))
    bound = BF16_MAXABS * r * (1.0 + r * np.abs(O)) * w / (1.0 + np.exp(-g))
    if y_bf16:
        bound = bound + 2.0 ** -9 * np.abs(Y)
    d = np.abs(got - Y)
    worst = float(np.max(d / bound))
    m, rel = errors(got, Y)
    say(f"  {name}: max-abs {m:.3e}, at most {worst:.2f} of the carried bar  rel-L2 {rel:.3e} (<= {BF16_RELL2:g})")
    assert worst <= 1.0, f"{name}: error {worst:.2f} times the bar carried from O"
    assert rel <= BF16_RELL2, f"{name}: rel-L2 {rel:.3e} > {BF16_RELL2:g}"
