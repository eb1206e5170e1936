"""Host-side tests of the C ABI (CPU only: nothing here launches a kernel).

The library must load, export every function include/fox.h declares, and reject bad arguments
with the documented status codes before touching the GPU. The argument-validation cases pass
fake (never dereferenced) device addresses; they run only where no GPU is visible, so a
validation bug can never turn into a launch on fake pointers.
"""
import ctypes
import os

import pytest
import torch

import gated_softmax_attention_fox_amd as fox

NO_GPU = not torch.cuda.is_available()
host_only = pytest.mark.skipif(not NO_GPU, reason="fake-pointer validation cases run without a GPU")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fox.LIB_PATH):
        import gated_softmax_attention_fox_amd.build as b
        b.build()
    return fox.load_library()


def test_header_declares_the_boundary():
    names = fox.header_functions()
    for n in ("fox_logf_cumsum", "fox_attn_fwd", "fox_attn_bwd", "fox_attn_bwd_workspace_bytes",
              "fox_gate_logf", "fox_qk_rmsnorm", "fox_status_str", "fox_last_error", "fox_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in fox.header_functions():
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.fox_status_str(0) == b"ok"
    assert lib.fox_status_str(1) == b"invalid argument"
    assert lib.fox_status_str(2) == b"unsupported request"
    assert lib.fox_status_str(3) == b"kernel launch failed"
    assert lib.fox_version().decode().count(".") == 2


def test_workspace_size(lib):
    # four fp32 [B*H*L] regions (row term, dc^q, dc^k, row offset), each rounded up to 256 bytes
    assert lib.fox_attn_bwd_workspace_bytes(1, 12, 16384, 128) == 4 * 12 * 16384 * 4
    assert lib.fox_attn_bwd_workspace_bytes(1, 1, 1, 64) == 4 * 256
    assert lib.fox_attn_bwd_workspace_bytes(0, 1, 1, 64) == 0


P = 0x7f0000000000  # fake, 16-byte aligned, never dereferenced


def _fwd(lib, q=P, k=P, v=P, in_dt=1, c=P, o=P, o_dt=1, lse=P, B=1, H=2, L=64, D=128, scale=0.1,
         flags=1, plan=None):
    return lib.fox_attn_fwd(q, k, v, in_dt, c, o, o_dt, lse, B, H, L, D, scale, flags, plan, None)


def _bwd(lib, ws=P, ws_bytes=1 << 30, in_dt=1, B=1, H=2, L=64, D=128, flags=1, o=P, plan=None):
    return lib.fox_attn_bwd(P, P, P, in_dt, P, o, P, P, P, P, P, P, ws, ws_bytes, B, H, L, D, 0.1,
                            flags, plan, None)


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(k=P + 8), 1), (dict(c=0), 1), (dict(o=0), 1), (dict(lse=P + 4), 1),
    (dict(D=96), 1), (dict(D=256), 1), (dict(L=0), 1), (dict(L=(1 << 23) + 1), 1), (dict(B=0), 1),
    (dict(H=-1), 1), (dict(in_dt=7), 1), (dict(o_dt=3), 1), (dict(in_dt=0, o_dt=1), 1), (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1), (dict(flags=0), 2), (dict(flags=5), 2), (dict(flags=2), 2),
    (dict(flags=3, plan=P), 2), (dict(plan=P + 16), 1), (dict(in_dt=0, o_dt=0, plan=P), 2),
    (dict(flags=9), 2),
])
def test_forward_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.fox_last_error().decode() != ""


def _fwd_ex(lib, opts=None, in_dt=1, o=P, L=64, D=128, **fields):
    o_ = fox.FoxFwdOpts()
    o_.scale, o_.flags = 0.1, fox.FOX_CAUSAL
    for f, val in fields.items():
        setattr(o_, f, val)
    ref = ctypes.byref(o_) if opts is None else opts
    return lib.fox_attn_fwd_ex(P, P, P, in_dt, P, o, 1, P, 1, 2, L, D, ref, None)


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(opts=ctypes.c_void_p(0)), 1),
    (dict(flags=1 | 16), 2),
    (dict(flags=1 | 8, k_norm_eps=-1.0), 1),
    (dict(flags=1 | 8, skip_plan=P), 2),
    (dict(k_shift_alpha=P, skip_plan=P), 2),
    (dict(v_shift_alpha=P + 2), 1),
    (dict(flags=1 | 8, k_norm_weight=P + 1), 1),
    (dict(k_shift_alpha=P, in_dt=0), 2),
    (dict(k_shift_alpha=P, o=0), 1),
    (dict(flags=1 | 4, q_norm_eps=-1.0), 1),
    (dict(gate=P, y=0), 1),
    (dict(gate=P, y=P, gate_dt=5), 1),
    (dict(k_shift_alpha=P, D=96), 1),
    (dict(k_shift_alpha=P, flags=0), 2),
])
def test_forward_ex_rejects(lib, kw, status):
    """fox_attn_fwd_ex validates its options (the fused q-norm, key norm, token shift and output
    gate) before any launch."""
    assert _fwd_ex(lib, **kw) == status
    assert lib.fox_last_error().decode() != ""


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(ws=0), 1), (dict(ws=P + 16), 1), (dict(ws_bytes=100), 1), (dict(in_dt=0, plan=P), 2),
    (dict(in_dt=0, H=70000), 2), (dict(in_dt=5), 1), (dict(flags=0), 2), (dict(D=32), 1), (dict(o=0), 1),
    (dict(L=(1 << 23) + 1), 1), (dict(plan=P + 64), 1),
])
def test_backward_rejects(lib, kw, status):
    assert _bwd(lib, **kw) == status
    msg = lib.fox_last_error().decode()
    assert msg
    if kw.get("ws_bytes") == 100:
        assert "workspace too small" in msg


def _bwd_dq(lib, o=P, delta=P, in_dt=1, plan=None):
    return lib.fox_attn_bwd_dq(P, P, P, in_dt, P, P, P, o, delta, P, P, P, P + 1024, 1, 2, 64, 128,
                               0.1, 1, plan, None)


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(o=0, delta=0), 1),      # neither the row term nor the output it comes from
    (dict(o=P + 4, delta=0), 1),  # o is read with 16-byte loads
    (dict(delta=P + 4), 1), (dict(in_dt=0, plan=P), 2),
])
def test_backward_dq_step_rejects(lib, kw, status):
    assert _bwd_dq(lib, **kw) == status
    assert lib.fox_last_error().decode() != ""


@host_only
def test_scan_gate_norm_reject(lib):
    assert lib.fox_logf_cumsum(0, P, 1, 8, None) == 1
    assert lib.fox_logf_cumsum(P, P, 1, 8, None) == 1          # aliasing
    assert lib.fox_logf_cumsum(P, P + 16, 0, 8, None) == 1
    assert lib.fox_logf_cumsum(P, P + 16, 1, 0, None) == 1
    assert lib.fox_gate_logf(P, 1, P, P, P, 1, 8, 12, 2, None) == 1   # d_model % 8
    assert lib.fox_gate_logf(P, 1, P, P, P, 1, 8, 16, 65, None) == 1  # H > 64
    assert lib.fox_gate_logf(P, 2, P, P, P, 1, 8, 16, 2, None) == 1   # dtype
    assert lib.fox_qk_rmsnorm(P, P, 1, 10, 96, ctypes.c_float(1e-6), None, None) == 1
    assert lib.fox_qk_rmsnorm(P, P, 1, 10, 128, ctypes.c_float(-1.0), None, None) == 1


def test_skip_plan_size(lib):
    # int32 [12, 64] + int32 [12, 128] + 4 x fp32 [12, 256] (q and k norms, smallest and largest
    # c) + int32 [768] + int32 [1536], each rounded up to 256 bytes
    assert lib.fox_attn_skip_plan_bytes(1, 12, 16384, 128) == 4 * 12 * (64 + 128 + 4 * 256 + 64 + 128)
    assert lib.fox_attn_skip_plan_bytes(1, 1, 1, 64) == 8 * 256
    assert lib.fox_attn_skip_plan_bytes(1, 0, 1, 64) == 0


@host_only
def test_skip_plan_rejects(lib):
    def plan(q=P, k=P, in_dt=1, c=P, out=P, nbytes=1 << 20, L=300, scale=0.1):
        return lib.fox_attn_skip_plan(q, k, in_dt, c, out, nbytes, 1, 2, L, 128, scale, None)
    assert plan(q=0) == 1
    assert plan(out=0) == 1
    assert plan(out=P + 16) == 1
    assert plan(nbytes=100) == 1
    assert "plan too small" in lib.fox_last_error().decode()
    assert plan(in_dt=0) == 2
    assert plan(scale=-1.0) == 1
    assert plan(L=0) == 1
    assert lib.fox_attn_skip_plan(P, P, 1, P, P, 1 << 40, 300, 300, 64, 128, 0.1, None) == 2  # B*H


def test_decode_workspace_size(lib):
    # fp32 [B*H, ceil(T / chunk), D + 2], rounded up to 256 bytes; chunk = 512 positions here
    # (the largest power of two that keeps at least 1536 workgroups)
    assert lib.fox_attn_decode_workspace_bytes(4, 12, 16384, 128) == 4 * 12 * 32 * 130 * 4
    assert lib.fox_attn_decode_workspace_bytes(1, 1, 1, 64) == 512
    assert lib.fox_attn_decode_workspace_bytes(1, 1, 1, 96) == 0


@host_only
def test_decode_rejects(lib):
    def dec(q=P, lens=P, o=P, in_dt=1, o_dt=1, ws=P, ws_bytes=1 << 30, T=64, D=128, flags=1):
        return lib.fox_attn_decode(q, P, P, in_dt, P, lens, None, o, o_dt, None, ws, ws_bytes, 2,
                                   3, T, D, 0.1, flags, None)
    assert dec(q=0) == 1
    assert dec(lens=0) == 1
    assert dec(o=P + 8) == 1
    assert dec(in_dt=0) == 2
    assert dec(o_dt=4) == 1
    assert dec(ws=P + 16) == 1
    assert dec(ws_bytes=100) == 1
    assert "workspace too small" in lib.fox_last_error().decode()
    assert dec(T=0) == 1
    assert dec(D=96) == 1
    assert dec(flags=0) == 2
    assert lib.fox_attn_decode(P, P, P, 1, P, P, None, P, 1, None, P, 1 << 40, 300, 300, 64, 128,
                               0.1, 1, None) == 2  # B*H above the grid limit

    def app(k_new=P, lens=P, in_dt=1, T=64, D=128):
        return lib.fox_attn_decode_append(k_new, P, in_dt, P, P, P, P, None, lens, 2, 3, T, D,
                                          None)
    assert app(k_new=0) == 1
    assert app(lens=P + 4) == 1
    assert app(in_dt=0) == 2
    assert app(D=32) == 1
    assert app(T=0) == 1
    assert lib.fox_attn_decode_key_norms(P, 1, 0, P, 2, 3, 64, 128, None) == 1   # lens NULL
    assert lib.fox_attn_decode_key_norms(P, 0, P, P, 2, 3, 64, 128, None) == 2   # fp32 cache
    assert lib.fox_attn_decode_key_norms(P, 1, P, P + 8, 2, 3, 64, 128, None) == 1


@host_only
def test_pro_shift_and_output_reject(lib):
    f = ctypes.c_float
    assert lib.fox_shift_gate(0, 1, P, P, 1, 8, 16, 2, None) == 1
    assert lib.fox_shift_gate(P, 1, P, P, 1, 8, 12, 2, None) == 1      # d_model % 8
    assert lib.fox_shift_gate(P, 3, P, P, 1, 8, 16, 2, None) == 1      # dtype
    assert lib.fox_shift_gate_bwd(P, 1, P, P, P, P, P, 100, 1, 8, 16, 2, None) == 1
    assert "workspace too small" in lib.fox_last_error().decode()
    assert lib.fox_kv_shift(P, 1, P, P, 1, f(1e-6), None, 2, 8, 96, None) == 1   # D
    assert lib.fox_kv_shift(P, 1, P, P, 1, f(-1.0), None, 2, 8, 64, None) == 1   # eps
    assert lib.fox_kv_shift(P, 1, P, P + 16, 0, f(1e-6), None, 2, 0, 64, None) == 1  # L = 0
    assert lib.fox_kv_shift(P, 1, P, P, 0, f(1e-6), None, 2, 8, 64, None) == 1   # y aliases x
    assert lib.fox_kv_shift_bwd(P, 1, P, P, P, P + 16, 1, f(1e-6), None, 2, 8, 64, None) == 1
    assert lib.fox_out_norm_gate(P, 1, P, 7, None, f(1e-6), P, 4, 128, None) == 1
    assert lib.fox_out_norm_gate_bwd(P, 1, P, 1, None, f(1e-6), P, P, 0, 4, 128, None) == 1


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        fox.load_library(str(tmp_path / "missing.so"))


def test_binding_rejects_cpu_tensors(lib):
    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    c = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        fox.fox_attn_fwd(x, x, x, c)


@host_only
def test_pro_backward_rejects(lib):
    ws = 256 * 1024  # a 256-aligned stand-in address, never dereferenced
    f = lib.fox_gate_logf_bwd
    # d_model % 8, H > 64, dtype, unaligned workspace, short workspace
    assert f(P, 1, P, P, P, None, P, P, P, ws, 1 << 30, 1, 8, 12, 2, None) == 1
    assert f(P, 1, P, P, P, None, P, P, P, ws, 1 << 30, 1, 8, 16, 65, None) == 1
    assert f(P, 2, P, P, P, None, P, P, P, ws, 1 << 30, 1, 8, 16, 2, None) == 1
    assert f(P, 1, P, P, P, None, P, P, P, ws + 16, 1 << 30, 1, 8, 16, 2, None) == 1
    assert f(P, 1, P, P, P, None, P, P, P, ws, 16, 1, 8, 16, 2, None) == 1
    assert f(P, 1, P, P, P, P + 4, P, P, P, ws, 1 << 30, 1, 8, 16, 2, None) == 1  # log_f unaligned
    assert lib.fox_gate_logf_bwd_workspace_bytes(1, 16384, 1536, 12) >= 4 * 16384 * 12
    assert lib.fox_gate_logf_bwd_workspace_bytes(0, 8, 16, 2) == 0
    g = lib.fox_qk_rmsnorm_bwd
    assert g(P, 1, P, P, None, None, None, 0, 10, 96, ctypes.c_float(1e-6), None) == 1  # D
    assert g(P, 1, P, P, None, P, ws, 1 << 20, 10, 128, ctypes.c_float(1e-6), None) == 1  # dweight without weight
    assert g(P, 1, P, P, P, P, None, 0, 10, 128, ctypes.c_float(1e-6), None) == 1  # no workspace
    assert g(P, 1, P, P, None, None, None, 0, 10, 128, ctypes.c_float(-1.0), None) == 1  # eps
    assert lib.fox_qk_rmsnorm_bwd_workspace_bytes(10, 128) >= 1024 * 128 * 4


@host_only
def test_noalloc_backward_rejects(lib):
    """fox_attn_bwd_noalloc: the size limit of its static scratch and the usual validation,
    before any launch."""
    assert lib.fox_attn_bwd_noalloc_max_bytes() == 4 * (1 << 21) * 4

    def call(B=1, H=2, L=64, D=128, flags=1, in_dt=1):
        return lib.fox_attn_bwd_noalloc(P, P, P, in_dt, P, P, P, P, P, P, P, P, B, H, L, D, 0.1,
                                        flags, None, None)
    assert call(H=2, L=(1 << 20) + 64) == 1  # B*H*L above 2^21
    assert b"static scratch" in lib.fox_last_error()
    assert call(flags=0) == 2
    assert call(D=96) == 1
    assert call(in_dt=7) == 1


def test_fwd_opts_layout_matches_c():
    """The binding's fox_fwd_opts mirror has the C struct's size and field offsets (gcc on the
    header, CPU only)."""
    import shutil
    import subprocess
    import tempfile
    import gated_softmax_attention_fox_amd as fox
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    fields = [f for f, _ in fox.FoxFwdOpts._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"fox.h\"\nint main(void){printf(\"%zu\", sizeof(fox_fwd_opts));" + "".join(
        f"printf(\" %zu\", offsetof(fox_fwd_opts, {f}));" for f in fields) + "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "layout")
        subprocess.run([gcc, "-I", os.path.dirname(fox.HEADER_PATH), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(fox.FoxFwdOpts)
    assert got[1:] == [getattr(fox.FoxFwdOpts, f).offset for f in fields]


BIG = 1 << 62  # sizes whose products overflow int64


def test_size_queries_reject_extreme_sizes(lib):
    """Size queries answer 0 for sizes beyond the limits, without overflowing on the way (the
    sanitized build of this file checks the arithmetic with UBSan)."""
    for b, h, l in ((BIG, BIG, 16), (BIG, 2, 16), (2, BIG, 16), (1, 1, BIG)):
        assert lib.fox_attn_skip_plan_bytes(b, h, l, 128) == 0
        assert lib.fox_attn_bwd_workspace_bytes(b, h, l, 128) == 0
        assert lib.fox_attn_decode_workspace_bytes(b, h, l, 128) == 0
    assert lib.fox_gate_logf_bwd_workspace_bytes(BIG, 16, 128, 4) == 0
    assert lib.fox_gate_logf_bwd_workspace_bytes(1, BIG, 128, 4) == 0
    assert lib.fox_gate_logf_bwd_workspace_bytes(1, 16, BIG, 4) == 0
    assert lib.fox_qk_rmsnorm_bwd_workspace_bytes(BIG, 128) == 0
    assert lib.fox_attn_bwd_workspace_bytes(1, 12, 16384, 128) > 0  # a valid size still answers


@host_only
def test_calls_reject_extreme_sizes(lib):
    """Every entry point with int64 sizes rejects products beyond its limits with
    FOX_E_INVALID, before forming a product that could overflow."""
    e = 1e-6
    for b, h in ((BIG, BIG), (BIG, 1), (1, BIG)):
        assert _fwd(lib, B=b, H=h) == 1
        assert lib.fox_attn_skip_plan(P, P, 1, P, P, 1 << 20, b, h, 64, 128, 0.1, None) == 1
        assert lib.fox_attn_decode(P, P, P, 1, P, P, None, P, 1, P, P, 1 << 20, b, h, 64, 128,
                                   0.1, 1, None) == 1
        assert lib.fox_attn_decode_key_norms(P, 1, P, P, b, h, 64, 128, None) == 1
    assert lib.fox_gate_logf(P, 1, P, P, P, BIG, 64, 128, 4, None) == 1
    assert lib.fox_gate_logf_bwd(P, 1, P, P, P, P, P, P, P, P, 1 << 20, BIG, 64, 128, 4, None) == 1
    assert lib.fox_shift_gate(P, 1, P, P, BIG, 64, 128, 4, None) == 1
    assert lib.fox_shift_gate_bwd(P, 1, P, P, P, P, P, 1 << 20, BIG, 64, 128, 4, None) == 1
    assert lib.fox_qk_rmsnorm(P, P, 1, BIG, 128, e, None, None) == 1
    assert lib.fox_qk_rmsnorm(P, P, 1, BIG, BIG, e, None, None) == 1
    assert lib.fox_qk_rmsnorm_bwd(P, 1, P, P, None, None, None, 0, BIG, 128, e, None) == 1
    assert lib.fox_attn_bwd_delta(P, 1, P, P, BIG, 128, None) == 1
    assert lib.fox_out_norm_gate(P, 1, P, 1, None, e, P, BIG, 128, None) == 1
    assert lib.fox_out_norm_gate_bwd(P, 1, P, 1, None, e, P, P, P, BIG, 128, None) == 1
    for bh, l in ((BIG, 16), (BIG, BIG), (1 << 40, 1 << 20)):
        assert lib.fox_kv_shift(P, 1, P, P, 1, e, None, bh, l, 128, None) == 1
        assert lib.fox_kv_shift_bwd(P, 1, P, P, P, P, 1, e, None, bh, l, 128, None) == 1
    assert lib.fox_logf_cumsum(P, P + 1024, BIG, 16, None) == 1
    assert lib.fox_dlogf_from_dc(P, P + 1024, P + 2048, BIG, 16, None) == 1
