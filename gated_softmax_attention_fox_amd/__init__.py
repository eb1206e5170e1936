"""Forgetting Attention on MI355X (gfx950): Python binding of libfox.so.

Argument marshalling only. Every function below checks the tensors it is given, allocates the
outputs with torch (device memory is PyTorch's plumbing here), and calls the C entry point of
the same name in libfox.so on the current HIP stream; all arithmetic runs in the library's
kernels. If libfox.so is missing, importing the binding raises: there is no fallback path.

C entry points (include/fox.h) and their wrappers:
    fox_logf_cumsum(log_f)                         -> c
    fox_gate_logf(x, w_f, b_f)                     -> log_f
    fox_qk_rmsnorm(x, eps, weight)                 -> y
    fox_attn_skip_plan(q, k, c, scale)             -> plan (uint8 device tensor)
    fox_attn_fwd(q, k, v, c, o_dtype, scale, skip_plan=None)        -> (o, lse)
    fox_attn_bwd(q, k, v, c, o, lse, dO, scale, skip_plan=None)     -> (dq, dk, dv, dlog_f)
    fox_attn_bwd_delta(dO, o)                      -> delta
    fox_attn_bwd_dq(q, k, v, c, lse, dO, delta)    -> (dq, dc_q, delta_refined)
    fox_attn_bwd_dq(q, k, v, c, lse, dO, None, o=o) -> the same, with Delta formed from o inside
    fox_attn_bwd_dkv(q, k, v, c, lse, dO, delta_refined) -> (dk, dv, dc_k)
    fox_dlogf_from_dc(dc_q, dc_k)                  -> dlog_f
    fox_attn_decode(q, k_cache, v_cache, c_cache, lens, o_dtype, scale) -> (o, lse)
    fox_attn_decode_append(k_new, v_new, log_f_new, k_cache, v_cache, c_cache, lens) (in place)
    fox_shift_gate(x, w) -> alpha;  fox_shift_gate_bwd(x, w, dalpha) -> (dx, dw)
    fox_kv_shift(x, alpha, normalize, eps, weight) -> y
    fox_kv_shift_bwd(x, alpha, dy, normalize, eps, weight) -> (dx, dalpha)
    fox_out_norm_gate(o, g, eps, weight) -> y;  fox_out_norm_gate_bwd(o, g, dy, eps, weight) -> (do, dg)
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

__all__ = [
    "FoxError", "LIB_PATH", "HEADER_PATH", "load_library", "header_functions",
    "fox_logf_cumsum", "fox_gate_logf", "fox_qk_rmsnorm", "fox_attn_fwd", "fox_attn_fwd_ex",
    "FoxFwdOpts", "fox_attn_fwd_logf",
    "fox_attn_bwd",
    "fox_attn_skip_plan_bytes", "fox_attn_skip_plan", "skip_plan_arrays",
    "fox_attn_decode_workspace_bytes", "fox_attn_decode", "fox_attn_decode_append",
    "fox_attn_decode_key_norms",
    "fox_shift_gate", "fox_shift_gate_bwd", "fox_kv_shift", "fox_kv_shift_bwd", "fox_out_norm_gate",
    "fox_out_norm_gate_bwd",
    "fox_attn_bwd_workspace_bytes", "fox_attn_bwd_noalloc", "fox_attn_bwd_delta", "fox_attn_bwd_dkv", "fox_attn_bwd_dq",
    "fox_dlogf_from_dc", "fox_version", "FOX_OK", "FOX_E_INVALID", "FOX_C_F64",
    "FOX_E_UNSUPPORTED", "FOX_E_LAUNCH", "FOX_F32", "FOX_BF16", "FOX_CAUSAL",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# FOX_LIBRARY names another build of the same library (the host tests use it to load a build
# whose host code is compiled with address and undefined-behaviour sanitizers).
LIB_PATH = os.environ.get("FOX_LIBRARY") or os.path.join(_PKG, "libfox.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "fox.h")

FOX_OK, FOX_E_INVALID, FOX_E_UNSUPPORTED, FOX_E_LAUNCH = 0, 1, 2, 3
FOX_F32, FOX_BF16 = 0, 1
FOX_CAUSAL, FOX_C_F64, FOX_QK_RMSNORM, FOX_K_RMSNORM = 1, 2, 4, 8


class FoxFwdOpts(ctypes.Structure):
    """fox_fwd_opts of include/fox.h (same field order; ctypes lays it out as the C compiler)."""
    _fields_ = [("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("q_norm_eps", ctypes.c_float), ("q_norm_weight", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("gate_dt", ctypes.c_int),
                ("out_norm_weight", ctypes.c_void_p), ("out_norm_eps", ctypes.c_float),
                ("y", ctypes.c_void_p), ("skip_plan", ctypes.c_void_p),
                ("k_shift_alpha", ctypes.c_void_p), ("v_shift_alpha", ctypes.c_void_p),
                ("k_norm_eps", ctypes.c_float), ("k_norm_weight", ctypes.c_void_p)]

_c_i64, _c_u32, _c_f32, _c_vp, _c_sz = (ctypes.c_int64, ctypes.c_uint32, ctypes.c_float,
                                         ctypes.c_void_p, ctypes.c_size_t)
_SIGS = {
    "fox_logf_cumsum": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp]),
    "fox_logf_cumsum_f64": (ctypes.c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp]),
    "fox_gate_logf": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                     _c_i64, _c_i64, _c_vp]),
    "fox_qk_rmsnorm": (ctypes.c_int, [_c_vp, _c_vp, ctypes.c_int, _c_i64, _c_i64, _c_f32, _c_vp,
                                      _c_vp]),
    "fox_gate_logf_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "fox_gate_logf_bwd": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                         _c_vp, _c_vp, _c_vp, _c_sz, _c_i64, _c_i64, _c_i64,
                                         _c_i64, _c_vp]),
    "fox_qk_rmsnorm_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64]),
    "fox_qk_rmsnorm_bwd": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                          _c_sz, _c_i64, _c_i64, _c_f32, _c_vp]),
    "fox_attn_skip_plan_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "fox_attn_skip_plan": (ctypes.c_int, [_c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_sz, _c_i64,
                                          _c_i64, _c_i64, _c_i64, _c_f32, _c_vp]),
    "fox_attn_fwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, ctypes.c_int,
                                    _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_f32, _c_u32, _c_vp,
                                    _c_vp]),
    "fox_attn_fwd_ex": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, ctypes.c_int,
                                       _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp]),
    "fox_attn_fwd_logf": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                         ctypes.c_int, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                         _c_f32, _c_u32, _c_vp]),
    "fox_attn_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "fox_attn_bwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                    _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_i64, _c_i64,
                                    _c_i64, _c_i64, _c_f32, _c_u32, _c_vp, _c_vp]),
    "fox_attn_bwd_noalloc_max_bytes": (_c_sz, []),
    "fox_attn_bwd_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                            _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                            _c_i64, _c_i64, _c_f32, _c_u32, _c_vp, _c_vp]),
    "fox_attn_bwd_delta": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp]),
    "fox_attn_bwd_dkv": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                        _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                        _c_f32, _c_u32, _c_vp, _c_vp]),
    "fox_attn_bwd_dq": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                       _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                       _c_i64, _c_i64, _c_f32, _c_u32, _c_vp, _c_vp]),
    "fox_dlogf_from_dc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp]),
    "fox_shift_gate": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                      _c_i64, _c_vp]),
    "fox_shift_gate_bwd": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                          _c_sz, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp]),
    "fox_kv_shift": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, ctypes.c_int, _c_f32, _c_vp,
                                    _c_i64, _c_i64, _c_i64, _c_vp]),
    "fox_kv_shift_bwd": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp,
                                        ctypes.c_int, _c_f32, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp]),
    "fox_out_norm_gate": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, ctypes.c_int, _c_vp, _c_f32,
                                         _c_vp, _c_i64, _c_i64, _c_vp]),
    "fox_out_norm_gate_bwd": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, ctypes.c_int, _c_vp,
                                             _c_f32, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp]),
    "fox_attn_decode_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "fox_attn_decode": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                       _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_sz, _c_i64, _c_i64,
                                       _c_i64, _c_i64, _c_f32, _c_u32, _c_vp]),
    "fox_attn_decode_key_norms": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, _c_vp, _c_i64,
                                                 _c_i64, _c_i64, _c_i64, _c_vp]),
    "fox_attn_decode_append": (ctypes.c_int, [_c_vp, _c_vp, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                              _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                              _c_vp]),
    "fox_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "fox_last_error": (ctypes.c_char_p, []),
    "fox_version": (ctypes.c_char_p, []),
}

_lib = None


class FoxError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: status {status}: {detail}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfox.so and declare the C signatures. Raises if the library is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m gated_softmax_attention_fox_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/fox.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fox_[a-z0-9_]+)\s*\(", text)))


def fox_version() -> str:
    return load_library().fox_version().decode()


def _check(status: int, fn: str):
    if status != FOX_OK:
        lib = load_library()
        raise FoxError(status, fn, lib.fox_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {t.dim()})")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t: torch.Tensor, name: str, shape) -> None:
    """Require an exact shape: the kernels index every element the sizes imply."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _code(dt: torch.dtype) -> int:
    return FOX_BF16 if dt == torch.bfloat16 else FOX_F32


def fox_logf_cumsum(log_f: torch.Tensor, c: torch.Tensor | None = None,
                    dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """c = inclusive prefix sum of log_f along the last axis (fp32 in; fp32 out, or fp64 out
    with dtype=torch.float64 or an fp64 c, for the attention calls' fp64-c mode)."""
    lib = load_library()
    pl = _dev(log_f, "log_f", (torch.float32,))
    if c is None:
        c = torch.empty(log_f.shape, dtype=dtype, device=log_f.device)
    pc = _dev(c, "c", (torch.float32, torch.float64))
    _shape(c, "c", log_f.shape)
    L = log_f.shape[-1]
    fn = lib.fox_logf_cumsum_f64 if c.dtype == torch.float64 else lib.fox_logf_cumsum
    _check(fn(pl, pc, log_f.numel() // max(L, 1), L, _stream(log_f)), "fox_logf_cumsum")
    return c


def _cflags(c: torch.Tensor) -> int:
    """FOX_CAUSAL, plus FOX_C_F64 when c holds fp64 values."""
    return FOX_CAUSAL | (FOX_C_F64 if c.dtype == torch.float64 else 0)


def fox_gate_logf(x: torch.Tensor, w_f: torch.Tensor, b_f: torch.Tensor) -> torch.Tensor:
    """log_f [B, H, L] = log sigmoid(x . w_f^T + b_f) from x [B, L, d_model]."""
    lib = load_library()
    px = _dev(x, "x", (torch.bfloat16, torch.float32), 3)
    pw = _dev(w_f, "w_f", (torch.float32,), 2)
    pb = _dev(b_f, "b_f", (torch.float32,), 1)
    B, L, dm = x.shape
    H = w_f.shape[0]
    if w_f.shape[1] != dm or b_f.shape[0] != H:
        raise ValueError("w_f must be [H, d_model] and b_f [H]")
    out = torch.empty((B, H, L), dtype=torch.float32, device=x.device)
    _check(lib.fox_gate_logf(px, _code(x.dtype), pw, pb, ctypes.c_void_p(out.data_ptr()), B, L, dm,
                             H, _stream(x)), "fox_gate_logf")
    return out


def fox_qk_rmsnorm(x: torch.Tensor, eps: float = 1e-6, weight: torch.Tensor | None = None,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """RMSNorm over the last axis (D = 64 or 128) of every row; same dtype in and out."""
    lib = load_library()
    px = _dev(x, "x", (torch.bfloat16, torch.float32))
    D = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    po = _dev(out, "out", (x.dtype,))
    _shape(out, "out", x.shape)
    pw = _wptr(weight, D)
    _check(lib.fox_qk_rmsnorm(px, po, _code(x.dtype), x.numel() // D, D, eps, pw, _stream(x)),
           "fox_qk_rmsnorm")
    return out


def fox_gate_logf_bwd(x: torch.Tensor, w_f: torch.Tensor, b_f: torch.Tensor,
                      dlog_f: torch.Tensor, log_f: torch.Tensor | None = None):
    """(dx [B, L, d_model], dw_f [H, d_model], db_f [H]), all fp32, given dlog_f [B, H, L].
    log_f: the forward's output (fox_gate_logf of the same inputs), from which the backward
    takes sigmoid(-z) instead of recomputing z from x; None recomputes."""
    lib = load_library()
    px = _dev(x, "x", (torch.bfloat16, torch.float32), 3)
    pw = _dev(w_f, "w_f", (torch.float32,), 2)
    pb = _dev(b_f, "b_f", (torch.float32,), 1)
    pg = _dev(dlog_f, "dlog_f", (torch.float32,), 3)
    B, L, dm = x.shape
    H = w_f.shape[0]
    if w_f.shape[1] != dm or b_f.shape[0] != H or tuple(dlog_f.shape) != (B, H, L):
        raise ValueError("w_f must be [H, d_model], b_f [H] and dlog_f [B, H, L]")
    pl = ctypes.c_void_p(0)
    if log_f is not None:
        pl = _dev(log_f, "log_f", (torch.float32,), 3)
        _shape(log_f, "log_f", (B, H, L))
    dx = torch.empty((B, L, dm), dtype=torch.float32, device=x.device)
    dw = torch.empty((H, dm), dtype=torch.float32, device=x.device)
    db = torch.empty((H,), dtype=torch.float32, device=x.device)
    need = int(lib.fox_gate_logf_bwd_workspace_bytes(B, L, dm, H))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib.fox_gate_logf_bwd(px, _code(x.dtype), pw, pb, pg, pl, ctypes.c_void_p(dx.data_ptr()),
                                 ctypes.c_void_p(dw.data_ptr()), ctypes.c_void_p(db.data_ptr()),
                                 ctypes.c_void_p(ws.data_ptr()), ws.numel(), B, L, dm, H,
                                 _stream(x)), "fox_gate_logf_bwd")
    return dx, dw, db


def fox_qk_rmsnorm_bwd(x: torch.Tensor, dy: torch.Tensor, eps: float = 1e-6,
                       weight: torch.Tensor | None = None, want_dweight: bool = False):
    """(dx fp32, dweight fp32 or None) of the QK-norm, given its input x and dy (fp32)."""
    lib = load_library()
    px = _dev(x, "x", (torch.bfloat16, torch.float32))
    pdy = _dev(dy, "dy", (torch.float32,))
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    D = x.shape[-1]
    rows = x.numel() // D
    dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    pw = _wptr(weight, D)
    dwt, pdw, ws, nws = None, ctypes.c_void_p(0), ctypes.c_void_p(0), 0
    if want_dweight:
        if weight is None:
            raise ValueError("want_dweight needs weight")
        dwt = torch.empty((D,), dtype=torch.float32, device=x.device)
        pdw = ctypes.c_void_p(dwt.data_ptr())
        need = int(lib.fox_qk_rmsnorm_bwd_workspace_bytes(rows, D))
        wst = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
        ws, nws = ctypes.c_void_p(wst.data_ptr()), wst.numel()
    _check(lib.fox_qk_rmsnorm_bwd(px, _code(x.dtype), pdy, ctypes.c_void_p(dx.data_ptr()), pw, pdw,
                                  ws, nws, rows, D, eps, _stream(x)), "fox_qk_rmsnorm_bwd")
    return dx, dwt


def _bhld(q, k, v):
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [B, H, L, D]")
    return q.shape


def fox_attn_skip_plan_bytes(B: int, H: int, L: int, D: int) -> int:
    return int(load_library().fox_attn_skip_plan_bytes(B, H, L, D))


def fox_attn_skip_plan(q, k, c, scale: float | None = None) -> torch.Tensor:
    """The exact tile-skipping plan of (q, k, c, scale), as a uint8 device tensor to pass as
    skip_plan to fox_attn_fwd and the backward calls made with the same inputs."""
    lib = load_library()
    B, H, L, D = _bhld(q, k, k)
    pq, pk = _dev(q, "q", (torch.bfloat16,)), _dev(k, "k", (torch.bfloat16,))
    pc = _dev(c, "c", (torch.float32,), 3)
    if tuple(c.shape) != (B, H, L):
        raise ValueError("c must be [B, H, L]")
    need = fox_attn_skip_plan_bytes(B, H, L, D)
    plan = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_skip_plan(pq, pk, FOX_BF16, pc, ctypes.c_void_p(plan.data_ptr()), need,
                                  B, H, L, D, scale, _stream(q)), "fox_attn_skip_plan")
    return plan


def skip_plan_arrays(plan: torch.Tensor, B: int, H: int, L: int):
    """Views (q_skip, kv_tiles, qn, kn, cmin, cmax, q_order, kv_order) of a plan, in the layout
    include/fox.h documents."""
    a256 = lambda x: (x + 255) // 256 * 256
    BH, n_qt, n_kb, n64 = B * H, -(-L // 256), -(-L // 128), -(-L // 64)
    o_kv = a256(4 * BH * n_qt)
    o_qn = a256(o_kv + 4 * BH * n_kb)
    o_kn = a256(o_qn + 4 * BH * n64)
    o_cmin = a256(o_kn + 4 * BH * n64)
    o_cmax = a256(o_cmin + 4 * BH * n64)
    o_qo = a256(o_cmax + 4 * BH * n64)
    o_ko = a256(o_qo + 4 * BH * n_qt)
    view = lambda off, n, dt, cols: plan[off:off + 4 * n].view(dt).view(-1, cols)
    f64 = lambda off: view(off, BH * n64, torch.float32, n64)
    return (view(0, BH * n_qt, torch.int32, n_qt), view(o_kv, BH * n_kb, torch.int32, n_kb),
            f64(o_qn), f64(o_kn), f64(o_cmin), f64(o_cmax),
            view(o_qo, BH * n_qt, torch.int32, BH * n_qt)[0],
            view(o_ko, BH * n_kb, torch.int32, BH * n_kb)[0])


def _plan_ptr(skip_plan, B: int, H: int, L: int, D: int) -> ctypes.c_void_p:
    if skip_plan is None:
        return ctypes.c_void_p(0)
    p = _dev(skip_plan, "skip_plan", (torch.uint8,))
    need = fox_attn_skip_plan_bytes(B, H, L, D)
    if skip_plan.numel() < need:
        raise ValueError(f"skip_plan holds {skip_plan.numel()} bytes; these sizes need {need} "
                         "(fox_attn_skip_plan_bytes)")
    return p


def fox_attn_fwd(q, k, v, c, o_dtype: torch.dtype | None = None, scale: float | None = None,
                 want_lse: bool = True, skip_plan: torch.Tensor | None = None):
    """(O, LSE) of causal Forgetting Attention with bias c_i - c_j (c: [B, H, L] fp32).

    skip_plan: fox_attn_skip_plan(q, k, c, scale), or None to visit every tile."""
    lib = load_library()
    B, H, L, D = _bhld(q, k, v)
    dts = (torch.bfloat16, torch.float32)
    pq, pk, pv = _dev(q, "q", dts), _dev(k, "k", (q.dtype,)), _dev(v, "v", (q.dtype,))
    pc = _dev(c, "c", (torch.float32, torch.float64), 3)
    if tuple(c.shape) != (B, H, L):
        raise ValueError("c must be [B, H, L]")
    o_dtype = o_dtype or q.dtype
    o = torch.empty((B, H, L, D), dtype=o_dtype, device=q.device)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if want_lse else None
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_fwd(pq, pk, pv, _code(q.dtype), pc, ctypes.c_void_p(o.data_ptr()),
                            _code(o_dtype), ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                            B, H, L, D, scale, _cflags(c), _plan_ptr(skip_plan, B, H, L, D),
                            _stream(q)),
           "fox_attn_fwd")
    return o, lse


def fox_attn_fwd_ex(q, k, v, c, o_dtype: torch.dtype | None = torch.float32,
                    scale: float | None = None, want_lse: bool = True,
                    q_norm_eps: float | None = None, q_norm_weight: torch.Tensor | None = None,
                    gate: torch.Tensor | None = None, out_norm_weight: torch.Tensor | None = None,
                    out_norm_eps: float = 1e-6, skip_plan: torch.Tensor | None = None,
                    k_shift_alpha: torch.Tensor | None = None,
                    v_shift_alpha: torch.Tensor | None = None,
                    k_norm_eps: float | None = None, k_norm_weight: torch.Tensor | None = None):
    """(O or None, LSE or None, y or None) of the forward with the Pro block's fusions: QK-norm
    of q as it is loaded (q_norm_eps not None); the token shift of the raw keys and values
    (k_shift_alpha, v_shift_alpha [B, H, L] fp32) and the key norm (k_norm_eps not None) as their
    tiles are loaded; and the output norm and gate y = RMSNorm(O) [* out_norm_weight] *
    sigmoid(gate) (gate [B, H, L, D] bf16 or fp32, y in its type). o_dtype=None skips O (only
    with a gate)."""
    lib = load_library()
    B, H, L, D = _bhld(q, k, v)
    pq, pk, pv = (_dev(q, "q", (torch.bfloat16,)), _dev(k, "k", (torch.bfloat16,)),
                  _dev(v, "v", (torch.bfloat16,)))
    pc = _dev(c, "c", (torch.float32, torch.float64), 3)
    _shape(c, "c", (B, H, L))
    opts = FoxFwdOpts()
    opts.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    opts.flags = (_cflags(c) | (FOX_QK_RMSNORM if q_norm_eps is not None else 0)
                  | (FOX_K_RMSNORM if k_norm_eps is not None else 0))
    opts.q_norm_eps = 0.0 if q_norm_eps is None else float(q_norm_eps)
    opts.q_norm_weight = _wptr(q_norm_weight, D).value
    opts.k_norm_eps = 0.0 if k_norm_eps is None else float(k_norm_eps)
    opts.k_norm_weight = _wptr(k_norm_weight, D).value
    for name, a in (("k_shift_alpha", k_shift_alpha), ("v_shift_alpha", v_shift_alpha)):
        if a is not None:
            _dev(a, name, (torch.float32,), 3)
            _shape(a, name, (B, H, L))
            setattr(opts, name, a.data_ptr())
    y = None
    if gate is not None:
        _dev(gate, "gate", (torch.bfloat16, torch.float32))
        _shape(gate, "gate", (B, H, L, D))
        y = torch.empty_like(gate)
        opts.gate, opts.gate_dt, opts.y = gate.data_ptr(), _code(gate.dtype), y.data_ptr()
        opts.out_norm_weight = _wptr(out_norm_weight, D).value
        opts.out_norm_eps = float(out_norm_eps)
    opts.skip_plan = _plan_ptr(skip_plan, B, H, L, D).value
    o = None if o_dtype is None else torch.empty((B, H, L, D), dtype=o_dtype, device=q.device)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if want_lse else None
    _check(lib.fox_attn_fwd_ex(pq, pk, pv, FOX_BF16, pc,
                               ctypes.c_void_p(o.data_ptr() if o is not None else 0),
                               _code(o_dtype or torch.float32),
                               ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                               B, H, L, D, ctypes.byref(opts), _stream(q)), "fox_attn_fwd_ex")
    return o, lse, y


def fox_attn_fwd_logf(q, k, v, log_f, o_dtype: torch.dtype | None = None,
                      scale: float | None = None, want_lse: bool = True,
                      c_dtype: torch.dtype = torch.float32):
    """(O, LSE, c) of the forward with the prefix sum fused in: takes log f [B, H, L] fp32 and
    returns c (fp32, or fp64 with c_dtype=torch.float64) for the backward."""
    lib = load_library()
    B, H, L, D = _bhld(q, k, v)
    dts = (torch.bfloat16, torch.float32)
    pq, pk, pv = _dev(q, "q", dts), _dev(k, "k", (q.dtype,)), _dev(v, "v", (q.dtype,))
    pl = _dev(log_f, "log_f", (torch.float32,), 3)
    _shape(log_f, "log_f", (B, H, L))
    o_dtype = o_dtype or q.dtype
    o = torch.empty((B, H, L, D), dtype=o_dtype, device=q.device)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if want_lse else None
    c = torch.empty((B, H, L), dtype=c_dtype, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_fwd_logf(pq, pk, pv, _code(q.dtype), pl, ctypes.c_void_p(c.data_ptr()),
                                 ctypes.c_void_p(o.data_ptr()), _code(o_dtype),
                                 ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                                 B, H, L, D, scale, _cflags(c), _stream(q)),
           "fox_attn_fwd_logf")
    return o, lse, c


def fox_attn_bwd_workspace_bytes(B: int, H: int, L: int, D: int) -> int:
    return int(load_library().fox_attn_bwd_workspace_bytes(B, H, L, D))


def fox_attn_bwd(q, k, v, c, o, lse, dO, scale: float | None = None, workspace=None,
                 skip_plan: torch.Tensor | None = None):
    """(dQ, dK, dV, d log f) for the loss sum(dO * O); o must be the fp32 forward output."""
    lib = load_library()
    B, H, L, D = _bhld(q, k, v)
    pq = _dev(q, "q", (torch.bfloat16, torch.float32))
    pk, pv = _dev(k, "k", (q.dtype,)), _dev(v, "v", (q.dtype,))
    pdo = _dev(dO, "dO", (q.dtype,))
    pc = _dev(c, "c", (torch.float32, torch.float64), 3)
    po = _dev(o, "o", (torch.float32,), 4)
    pl = _dev(lse, "lse", (torch.float32,), 3)
    for t, name in ((dO, "dO"), (o, "o")):
        _shape(t, name, (B, H, L, D))
    for t, name in ((c, "c"), (lse, "lse")):
        _shape(t, name, (B, H, L))
    dq = torch.empty((B, H, L, D), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    dlf = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    need = fox_attn_bwd_workspace_bytes(B, H, L, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace", (torch.uint8,))
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes; {need} needed")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_bwd(pq, pk, pv, _code(q.dtype), pc, po, pl, pdo,
                            ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()),
                            ctypes.c_void_p(dv.data_ptr()), ctypes.c_void_p(dlf.data_ptr()), pw,
                            workspace.numel(), B, H, L, D, scale, _cflags(c),
                            _plan_ptr(skip_plan, B, H, L, D), _stream(q)),
           "fox_attn_bwd")
    return dq, dk, dv, dlf


def fox_attn_bwd_noalloc(q, k, v, c, o, lse, dO, scale: float | None = None,
                         skip_plan: torch.Tensor | None = None, out=None):
    """fox_attn_bwd on the library's static scratch (no workspace). out: optional
    (dq, dk, dv, dlog_f) fp32 tensors to write; with them this call allocates nothing."""
    lib = load_library()
    B, H, L, D = _bhld(q, k, v)
    pq = _dev(q, "q", (torch.bfloat16, torch.float32))
    pk, pv = _dev(k, "k", (q.dtype,)), _dev(v, "v", (q.dtype,))
    pdo = _dev(dO, "dO", (q.dtype,))
    pc = _dev(c, "c", (torch.float32, torch.float64), 3)
    po = _dev(o, "o", (torch.float32,), 4)
    pl = _dev(lse, "lse", (torch.float32,), 3)
    for t, name in ((dO, "dO"), (o, "o")):
        _shape(t, name, (B, H, L, D))
    for t, name in ((c, "c"), (lse, "lse")):
        _shape(t, name, (B, H, L))
    if out is None:
        out = (torch.empty((B, H, L, D), dtype=torch.float32, device=q.device),
               torch.empty((B, H, L, D), dtype=torch.float32, device=q.device),
               torch.empty((B, H, L, D), dtype=torch.float32, device=q.device),
               torch.empty((B, H, L), dtype=torch.float32, device=q.device))
    dq, dk, dv, dlf = out
    ptrs = []
    for t, name, shp in ((dq, "dq", (B, H, L, D)), (dk, "dk", (B, H, L, D)),
                         (dv, "dv", (B, H, L, D)), (dlf, "dlog_f", (B, H, L))):
        ptrs.append(_dev(t, name, (torch.float32,)))
        _shape(t, name, shp)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_bwd_noalloc(pq, pk, pv, _code(q.dtype), pc, po, pl, pdo, *ptrs, B, H, L, D,
                                    scale, _cflags(c), _plan_ptr(skip_plan, B, H, L, D),
                                    _stream(q)),
           "fox_attn_bwd_noalloc")
    return dq, dk, dv, dlf


def fox_attn_bwd_delta(dO: torch.Tensor, o: torch.Tensor) -> torch.Tensor:
    """Delta = rowsum(dO * O) over the last axis; dO bf16 or fp32, o fp32."""
    lib = load_library()
    pd = _dev(dO, "dO", (torch.bfloat16, torch.float32))
    po = _dev(o, "o", (torch.float32,))
    if dO.shape != o.shape:
        raise ValueError("dO and o must have the same shape")
    D = o.shape[-1]
    delta = torch.empty(o.shape[:-1], dtype=torch.float32, device=o.device)
    _check(lib.fox_attn_bwd_delta(pd, _code(dO.dtype), po, ctypes.c_void_p(delta.data_ptr()),
                                  o.numel() // D, D, _stream(o)), "fox_attn_bwd_delta")
    return delta


def _bwd_inputs(q, k, v, c, lse, dO, delta):
    B, H, L, D = _bhld(q, k, v)
    _shape(dO, "dO", (B, H, L, D))
    for t, name in ((c, "c"), (lse, "lse"), (delta, "delta")):
        if t is not None:
            _shape(t, name, (B, H, L))
    ptrs = (_dev(q, "q", (torch.bfloat16, torch.float32)), _dev(k, "k", (q.dtype,)),
            _dev(v, "v", (q.dtype,)), _dev(c, "c", (torch.float32, torch.float64), 3),
            _dev(lse, "lse", (torch.float32,), 3), _dev(dO, "dO", (q.dtype,), 4),
            None if delta is None else _dev(delta, "delta", (torch.float32,), 3))
    return (B, H, L, D), ptrs


def fox_attn_bwd_dkv(q, k, v, c, lse, dO, delta, scale: float | None = None,
                     skip_plan: torch.Tensor | None = None):
    """(dK, dV, dc_k) of the key-stationary backward step; lse and delta are fox_attn_bwd_dq's
    lse_out and refined delta."""
    lib = load_library()
    (B, H, L, D), (pq, pk, pv, pc, pl, pdo, pdl) = _bwd_inputs(q, k, v, c, lse, dO, delta)
    dk = torch.empty((B, H, L, D), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    dck = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_bwd_dkv(pq, pk, pv, _code(q.dtype), pc, pl, pdo, pdl,
                                ctypes.c_void_p(dk.data_ptr()), ctypes.c_void_p(dv.data_ptr()),
                                ctypes.c_void_p(dck.data_ptr()), B, H, L, D, scale, _cflags(c),
                                _plan_ptr(skip_plan, B, H, L, D), _stream(q)),
           "fox_attn_bwd_dkv")
    return dk, dv, dck


def fox_attn_bwd_dq(q, k, v, c, lse, dO, delta, scale: float | None = None,
                    delta_out: torch.Tensor | None = None, skip_plan: torch.Tensor | None = None,
                    o: torch.Tensor | None = None):
    """(dQ, dc_q, refined delta, lse_out) of the query-stationary backward step (run before
    dkv, which takes lse_out and the refined delta).

    delta_out may be `delta` itself to refine it in place. With delta=None the step forms the
    row term from o (the fp32 forward output) itself, bit-identical to fox_attn_bwd_delta."""
    lib = load_library()
    (B, H, L, D), (pq, pk, pv, pc, pl, pdo, pdl) = _bwd_inputs(q, k, v, c, lse, dO, delta)
    po = None
    if delta is None:
        if o is None:
            raise ValueError("fox_attn_bwd_dq needs delta or o")
        po = _dev(o, "o", (torch.float32,), 4)
        if tuple(o.shape) != (B, H, L, D):
            raise ValueError(f"o must have shape {(B, H, L, D)}, got {tuple(o.shape)}")
    dq = torch.empty((B, H, L, D), dtype=torch.float32, device=q.device)
    dcq = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if delta_out is None:
        delta_out = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    pdn = _dev(delta_out, "delta_out", (torch.float32,), 3)
    _shape(delta_out, "delta_out", (B, H, L))
    lse_out = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib.fox_attn_bwd_dq(pq, pk, pv, _code(q.dtype), pc, pl, pdo, po, pdl,
                               ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dcq.data_ptr()), pdn,
                               ctypes.c_void_p(lse_out.data_ptr()), B, H, L, D, scale, _cflags(c),
                               _plan_ptr(skip_plan, B, H, L, D), _stream(q)),
           "fox_attn_bwd_dq")
    return dq, dcq, delta_out, lse_out


def fox_dlogf_from_dc(dc_q: torch.Tensor, dc_k: torch.Tensor) -> torch.Tensor:
    """d log f = reverse cumulative sum of dc_q + dc_k along the last axis."""
    lib = load_library()
    pa = _dev(dc_q, "dc_q", (torch.float32,))
    pb = _dev(dc_k, "dc_k", (torch.float32,))
    if dc_q.shape != dc_k.shape:
        raise ValueError("dc_q and dc_k must have the same shape")
    out = torch.empty_like(dc_q)
    L = dc_q.shape[-1]
    _check(lib.fox_dlogf_from_dc(pa, pb, ctypes.c_void_p(out.data_ptr()), dc_q.numel() // L, L,
                                 _stream(dc_q)), "fox_dlogf_from_dc")
    return out


def fox_attn_decode_workspace_bytes(B: int, H: int, T_max: int, D: int) -> int:
    return int(load_library().fox_attn_decode_workspace_bytes(B, H, T_max, D))


def fox_attn_decode(q, k_cache, v_cache, c_cache, lens, o_dtype: torch.dtype = torch.float32,
                    scale: float | None = None, workspace=None,
                    k_norms: torch.Tensor | None = None):
    """(o [B, H, D], lse [B, H]) of the newest position of each sequence against the cache.

    q: [B, H, D] bf16; k_cache, v_cache: [B, H, T_max, D] bf16; c_cache: [B, H, T_max] fp32;
    lens: [B] int32 device tensor of cached lengths (the query sits at lens[b] - 1).
    k_norms: fox_attn_decode_key_norms(...) kept current by the appends, or None; with it the
    chunks whose weights all underflow are not read (bit-identical results)."""
    lib = load_library()
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share one shape [B, H, T_max, D]")
    B, H, T, D = k_cache.shape
    if tuple(q.shape) != (B, H, D) or tuple(c_cache.shape) != (B, H, T):
        raise ValueError("q must be [B, H, D] and c_cache [B, H, T_max]")
    if tuple(lens.shape) != (B,):
        raise ValueError("lens must be [B]")
    pq = _dev(q, "q", (torch.bfloat16,), 3)
    pk, pv = _dev(k_cache, "k_cache", (torch.bfloat16,), 4), _dev(v_cache, "v_cache", (torch.bfloat16,), 4)
    pc = _dev(c_cache, "c_cache", (torch.float32,), 3)
    pl = _dev(lens, "lens", (torch.int32,), 1)
    o = torch.empty((B, H, D), dtype=o_dtype, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = fox_attn_decode_workspace_bytes(B, H, T, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    pw = _dev(workspace, "workspace", (torch.uint8,))
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes; {need} needed")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    pn = ctypes.c_void_p(0)
    if k_norms is not None:
        pn = _dev(k_norms, "k_norms", (torch.float32,), 3)
        _shape(k_norms, "k_norms", (B, H, -(-T // 64)))
    _check(lib.fox_attn_decode(pq, pk, pv, FOX_BF16, pc, pl, pn, ctypes.c_void_p(o.data_ptr()),
                               _code(o_dtype), ctypes.c_void_p(lse.data_ptr()), pw,
                               workspace.numel(), B, H, T, D, scale, FOX_CAUSAL, _stream(q)),
           "fox_attn_decode")
    return o, lse


def fox_attn_decode_key_norms(k_cache: torch.Tensor, lens: torch.Tensor) -> torch.Tensor:
    """The largest key norm of every 64 cached positions: [B, H, ceil(T_max / 64)] fp32."""
    lib = load_library()
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, H, T_max, D]")
    B, H, T, D = k_cache.shape
    _shape(lens, "lens", (B,))
    kn = torch.empty((B, H, -(-T // 64)), dtype=torch.float32, device=k_cache.device)
    _check(lib.fox_attn_decode_key_norms(_dev(k_cache, "k_cache", (torch.bfloat16,), 4), FOX_BF16,
                                         _dev(lens, "lens", (torch.int32,), 1),
                                         ctypes.c_void_p(kn.data_ptr()), B, H, T, D,
                                         _stream(k_cache)), "fox_attn_decode_key_norms")
    return kn


def fox_attn_decode_append(k_new, v_new, log_f_new, k_cache, v_cache, c_cache, lens,
                           k_norms: torch.Tensor | None = None):
    """Append one position per sequence to the cache in place (k, v, c and, when given, the key
    norms), then lens += 1."""
    lib = load_library()
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share one shape [B, H, T_max, D]")
    B, H, T, D = k_cache.shape
    _shape(c_cache, "c_cache", (B, H, T))
    if k_norms is not None:
        _shape(k_norms, "k_norms", (B, H, -(-T // 64)))
    if tuple(k_new.shape) != (B, H, D) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [B, H, D]")
    if tuple(log_f_new.shape) != (B, H) or tuple(lens.shape) != (B,):
        raise ValueError("log_f_new must be [B, H] and lens [B]")
    args = (_dev(k_new, "k_new", (torch.bfloat16,), 3), _dev(v_new, "v_new", (torch.bfloat16,), 3),
            FOX_BF16, _dev(log_f_new, "log_f_new", (torch.float32,), 2),
            _dev(k_cache, "k_cache", (torch.bfloat16,), 4),
            _dev(v_cache, "v_cache", (torch.bfloat16,), 4),
            _dev(c_cache, "c_cache", (torch.float32,), 3),
            ctypes.c_void_p(0) if k_norms is None else _dev(k_norms, "k_norms", (torch.float32,), 3),
            _dev(lens, "lens", (torch.int32,), 1))
    _check(lib.fox_attn_decode_append(*args, B, H, T, D, _stream(k_cache)),
           "fox_attn_decode_append")


def _wptr(weight, D):
    if weight is None:
        return ctypes.c_void_p(0)
    if tuple(weight.shape) != (D,):
        raise ValueError(f"weight must be [{D}]")
    return _dev(weight, "weight", (torch.float32,), 1)


def fox_shift_gate(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """Shift gate alpha [B, H, L] = sigmoid(x . w^T) (x [B, L, d_model], w [H, d_model] fp32)."""
    lib = load_library()
    B, L, dm = x.shape
    H = w.shape[0]
    px = _dev(x, "x", (torch.bfloat16, torch.float32), 3)
    pw = _dev(w, "w", (torch.float32,), 2)
    _shape(w, "w", (H, dm))
    alpha = torch.empty((B, H, L), dtype=torch.float32, device=x.device)
    _check(lib.fox_shift_gate(px, _code(x.dtype), pw, ctypes.c_void_p(alpha.data_ptr()), B, L, dm,
                              H, _stream(x)), "fox_shift_gate")
    return alpha


def fox_shift_gate_bwd(x: torch.Tensor, w: torch.Tensor, dalpha: torch.Tensor):
    """(dx, dw) of the shift gate for the upstream gradient dalpha [B, H, L]."""
    lib = load_library()
    B, L, dm = x.shape
    H = w.shape[0]
    px = _dev(x, "x", (torch.bfloat16, torch.float32), 3)
    pw = _dev(w, "w", (torch.float32,), 2)
    pd = _dev(dalpha, "dalpha", (torch.float32,), 3)
    _shape(w, "w", (H, dm))
    _shape(dalpha, "dalpha", (B, H, L))
    dx = torch.empty((B, L, dm), dtype=torch.float32, device=x.device)
    dw = torch.empty((H, dm), dtype=torch.float32, device=x.device)
    need = int(lib.fox_gate_logf_bwd_workspace_bytes(B, L, dm, H))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib.fox_shift_gate_bwd(px, _code(x.dtype), pw, pd, ctypes.c_void_p(dx.data_ptr()),
                                  ctypes.c_void_p(dw.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                  ws.numel(), B, L, dm, H, _stream(x)), "fox_shift_gate_bwd")
    return dx, dw


def fox_kv_shift(x: torch.Tensor, alpha: torch.Tensor, normalize: bool = False, eps: float = 1e-6,
                 weight: torch.Tensor | None = None) -> torch.Tensor:
    """Token shift y_t = alpha_t x_{t-1} + (1 - alpha_t) x_t over [..., L, D], RMS-normalised when
    normalize (keys); alpha [..., L] fp32."""
    lib = load_library()
    L, D = x.shape[-2], x.shape[-1]
    BH = x.numel() // (L * D)
    if tuple(alpha.shape) != tuple(x.shape[:-1]):
        raise ValueError("alpha must have x's shape without the last axis")
    px = _dev(x, "x", (torch.bfloat16, torch.float32))
    pa = _dev(alpha, "alpha", (torch.float32,))
    y = torch.empty_like(x)
    _check(lib.fox_kv_shift(px, _code(x.dtype), pa, ctypes.c_void_p(y.data_ptr()), int(normalize),
                            float(eps), _wptr(weight, D), BH, L, D, _stream(x)), "fox_kv_shift")
    return y


def fox_kv_shift_bwd(x, alpha, dy, normalize: bool = False, eps: float = 1e-6, weight=None):
    """(dx, dalpha) of fox_kv_shift for the upstream gradient dy (fp32, x's shape)."""
    lib = load_library()
    L, D = x.shape[-2], x.shape[-1]
    BH = x.numel() // (L * D)
    if dy.shape != x.shape:
        raise ValueError("dy must have x's shape")
    _shape(alpha, "alpha", x.shape[:-1])
    px = _dev(x, "x", (torch.bfloat16, torch.float32))
    pa = _dev(alpha, "alpha", (torch.float32,))
    pd = _dev(dy, "dy", (torch.float32,))
    dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    da = torch.empty(alpha.shape, dtype=torch.float32, device=x.device)
    _check(lib.fox_kv_shift_bwd(px, _code(x.dtype), pa, pd, ctypes.c_void_p(dx.data_ptr()),
                                ctypes.c_void_p(da.data_ptr()), int(normalize), float(eps),
                                _wptr(weight, D), BH, L, D, _stream(x)), "fox_kv_shift_bwd")
    return dx, da


def fox_out_norm_gate(o: torch.Tensor, g: torch.Tensor, eps: float = 1e-6,
                      weight: torch.Tensor | None = None) -> torch.Tensor:
    """y = RMSNorm(o) [* weight] * sigmoid(g) over the last axis; y has g's dtype."""
    lib = load_library()
    if o.shape != g.shape:
        raise ValueError("o and g must have the same shape")
    D = o.shape[-1]
    po = _dev(o, "o", (torch.bfloat16, torch.float32))
    pg = _dev(g, "g", (torch.bfloat16, torch.float32))
    y = torch.empty_like(g)
    _check(lib.fox_out_norm_gate(po, _code(o.dtype), pg, _code(g.dtype), _wptr(weight, D),
                                 float(eps), ctypes.c_void_p(y.data_ptr()), o.numel() // D, D,
                                 _stream(o)), "fox_out_norm_gate")
    return y


def fox_out_norm_gate_bwd(o, g, dy, eps: float = 1e-6, weight=None):
    """(d_o, dg) of fox_out_norm_gate for the upstream gradient dy (fp32)."""
    lib = load_library()
    if o.shape != g.shape or dy.shape != o.shape:
        raise ValueError("o, g and dy must have the same shape")
    D = o.shape[-1]
    po = _dev(o, "o", (torch.bfloat16, torch.float32))
    pg = _dev(g, "g", (torch.bfloat16, torch.float32))
    pd = _dev(dy, "dy", (torch.float32,))
    d_o = torch.empty(o.shape, dtype=torch.float32, device=o.device)
    dg = torch.empty(o.shape, dtype=torch.float32, device=o.device)
    _check(lib.fox_out_norm_gate_bwd(po, _code(o.dtype), pg, _code(g.dtype), _wptr(weight, D),
                                     float(eps), pd, ctypes.c_void_p(d_o.data_ptr()),
                                     ctypes.c_void_p(dg.data_ptr()), o.numel() // D, D, _stream(o)),
           "fox_out_norm_gate_bwd")
    return d_o, dg
