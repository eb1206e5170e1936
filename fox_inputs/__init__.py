"""Seeded synthetic inputs for Forgetting Attention, shared by the tests, the bench and smoke().

This module is the only code that both the oracle side and the HIP side consume. It holds no
step of the attention path: it draws random numbers, rounds them to the storage type, and hands
back plain NumPy arrays. Both sides then receive identical bits.

Input recipes follow the workloads of the Forgetting Transformer pages (arXiv 2503.02130):
16,384-token context, head dim 64/128, 12 heads, d_model 1536, and forget-gate logits whose
per-head mean sets a memory horizon. The log forget gate handed to the path is drawn as
log f = log sigmoid(z) of a normally distributed logit z; that is the distribution of the input,
evaluated once here in fp64 and rounded to fp32, and both sides read the same fp32 values.
The gate step itself (x -> log f, Pro block Step 4) is not done here: that workload hands x,
w_f and b_f to each side, which compute log f independently.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "bf16_bits", "bf16_round", "bits_to_f32", "FoxCase", "make_case", "make_periodic_case",
    "repeat_rows", "CONFIGS", "config_case", "logsigmoid_input",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounding_bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding_bias) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to the fp32 values they encode (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 array holding the bfloat16-rounded values of x (exactly representable in bf16)."""
    return bits_to_f32(bf16_bits(x))


def logsigmoid_input(z: np.ndarray) -> np.ndarray:
    """fp32 log-forget-gate input values drawn as log sigmoid(z): fp64 evaluation, one rounding."""
    z = np.asarray(z, dtype=np.float64)
    return (-np.logaddexp(0.0, -z)).astype(np.float32)


@dataclasses.dataclass
class FoxCase:
    """One synthetic batch. Float arrays hold the exact values both sides see.

    q, k, v, do: fp32 arrays [B,H,L,D]; when dtype == "bf16" every value is bf16-representable
    and *_bits holds the uint16 encoding to upload. log_f: fp32 [B,H,L] (None for the Pro
    workload, which supplies x / w_f / b_f instead). x: [B,L,d_model] bf16 values; w_f: fp32
    [H,d_model]; b_f: fp32 [H].
    """
    name: str
    B: int
    H: int
    L: int
    D: int
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_f: np.ndarray | None = None
    do: np.ndarray | None = None
    x: np.ndarray | None = None
    w_f: np.ndarray | None = None
    b_f: np.ndarray | None = None
    qk_norm: bool = False
    seed: int = 0

    def bits(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits(a)


def _qkv(rng: np.random.Generator, shape, dtype: str):
    out = []
    for _ in range(3):
        a = rng.standard_normal(shape, dtype=np.float32)
        out.append(bf16_round(a) if dtype == "bf16" else a)
    return out


def _draw_log_f(rng: np.random.Generator, B: int, H: int, L: int, gate: str, gate_mean: float,
                gate_std: float, head_mean_range: tuple[float, float]) -> np.ndarray:
    """log f [B, H, L] fp32 by the named gate recipe (see make_case)."""
    if gate == "normal":
        z = rng.normal(gate_mean, gate_std, size=(B, H, L))
        return logsigmoid_input(z)
    if gate == "per_head":
        mu = rng.uniform(head_mean_range[0], head_mean_range[1], size=(H,))
        z = mu[None, :, None] + rng.standard_normal((B, H, L))
        return logsigmoid_input(z)
    if gate == "zero":
        return np.zeros((B, H, L), np.float32)
    if gate == "quarter_steps":
        return np.where(rng.random((B, H, L)) < 0.5, -0.25, 0.0).astype(np.float32)
    raise ValueError(gate)


def make_case(B: int, H: int, L: int, D: int, dtype: str = "bf16", *, seed: int = 0,
              gate: str = "normal", gate_mean: float = 3.0, gate_std: float = 1.5,
              head_mean_range: tuple[float, float] = (1.0, 6.0), with_do: bool = False,
              name: str = "custom") -> FoxCase:
    """Generic recipe: q, k, v ~ N(0,1); log f = log sigmoid(z).

    gate = "normal": z ~ N(gate_mean, gate_std^2) per (b, h, t).
    gate = "per_head": mu_h ~ U[head_mean_range] per head, z ~ N(mu_h, 1) per (b, h, t).
    gate = "zero": log f = 0 (f = 1, plain causal attention).
    gate = "quarter_steps": log f = -1/4 or 0 with equal odds per (b, h, t); every prefix sum is
        a multiple of 1/4 below 2^21 in size up to L = 2^23, so fp32 holds c exactly.
    """
    assert dtype in ("bf16", "f32")
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (B, H, L, D), dtype)
    log_f = _draw_log_f(rng, B, H, L, gate, gate_mean, gate_std, head_mean_range)
    do = None
    if with_do:
        r2 = np.random.default_rng(seed + 1000)
        do = r2.standard_normal((B, H, L, D), dtype=np.float32)
        do = bf16_round(do) if dtype == "bf16" else do
    return FoxCase(name, B, H, L, D, dtype, q, k, v, log_f=log_f, do=do, seed=seed)


def repeat_rows(a: np.ndarray, L: int) -> np.ndarray:
    """a [..., P, D] repeated along its row axis and cut to [..., L, D] (row r is row r mod P)."""
    P = a.shape[-2]
    reps = -(-L // P)
    return np.concatenate([a] * reps, axis=-2)[..., :L, :] if reps > 1 else a[..., :L, :].copy()


def make_periodic_case(B: int, H: int, L: int, D: int, *, period: int, seed: int = 0,
                       gate: str = "normal", with_do: bool = False,
                       name: str = "periodic") -> tuple[FoxCase, FoxCase]:
    """A long bf16 case whose q, k, v (and dO) rows repeat with the given period, for lengths at
    which drawing every value would take minutes: the rows of make_case(B, H, period, D) repeated
    along the sequence (row r is row r mod period), and log f drawn for all L positions by the
    same gate recipe from its own stream (seed + 2000), so no two positions share their decay.
    Returns (case, base): base is the period-length case whose rows repeat (its bf16 bits,
    repeated with repeat_rows, are the upload of the long case without re-rounding)."""
    base = make_case(B, H, period, D, "bf16", seed=seed, gate="zero", with_do=with_do)
    rng = np.random.default_rng(seed + 2000)
    log_f = _draw_log_f(rng, B, H, L, gate, 3.0, 1.5, (1.0, 6.0))
    q, k, v = (repeat_rows(getattr(base, n), L) for n in ("q", "k", "v"))
    do = repeat_rows(base.do, L) if with_do else None
    case = FoxCase(name, B, H, L, D, "bf16", q, k, v, log_f=log_f, do=do, seed=seed)
    return case, base


def make_pro_case(B: int, H: int, L: int, D: int, d_model: int, *, seed: int = 4,
                  name: str = "pro") -> FoxCase:
    """Pro-block workload: x ~ N(0,1) bf16 [B,L,d_model]; q, k, v ~ N(0,1) bf16;
    w_f ~ N(0, 0.02^2) fp32 [H,d_model]; b_f ~ U[1,6] fp32 [H]; QK-norm with unit weights."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (B, H, L, D), "bf16")
    x = bf16_round(rng.standard_normal((B, L, d_model), dtype=np.float32))
    w_f = (0.02 * rng.standard_normal((H, d_model))).astype(np.float32)
    b_f = rng.uniform(1.0, 6.0, size=(H,)).astype(np.float32)
    return FoxCase(name, B, H, L, D, "bf16", q, k, v, x=x, w_f=w_f, b_f=b_f, qk_norm=True,
                   seed=seed)


# The five workloads. Sizes and distributions follow the pages' setting (16K context,
# d_head 128, 12 heads, d_model 1536); config 1 is the small fp32 case.
CONFIGS = {
    1: dict(kind="fwd", B=1, H=2, L=256, D=64, dtype="f32", seed=1, gate="normal"),
    2: dict(kind="fwd", B=4, H=12, L=2048, D=128, dtype="bf16", seed=2, gate="normal"),
    3: dict(kind="fwd", B=1, H=12, L=16384, D=128, dtype="bf16", seed=3, gate="per_head"),
    4: dict(kind="pro", B=1, H=12, L=16384, D=128, d_model=1536, dtype="bf16", seed=4),
    5: dict(kind="bwd", B=1, H=12, L=16384, D=128, dtype="bf16", seed=3, gate="per_head"),
}


def config_case(n: int, L: int | None = None, B: int | None = None, H: int | None = None) -> FoxCase:
    """Inputs of workload n; L/B/H may be overridden to shrink a case with the same recipe."""
    c = dict(CONFIGS[n])
    kind = c.pop("kind")
    if L is not None:
        c["L"] = L
    if B is not None:
        c["B"] = B
    if H is not None:
        c["H"] = H
    if kind == "pro":
        return make_pro_case(c["B"], c["H"], c["L"], c["D"], c["d_model"], seed=c["seed"],
                             name=f"config{n}")
    return make_case(c["B"], c["H"], c["L"], c["D"], c["dtype"], seed=c["seed"], gate=c["gate"],
                     with_do=(kind == "bwd"), name=f"config{n}")
