// fox_launch.h — host-side launchers of the gfx950 kernels (called by the C ABI in abi.cpp).
// Every launcher only enqueues work on `s` and returns the launch status; shapes have already
// been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fox {

// c[r, i] = sum_{l <= i} x[r, l] (fp64 accumulation, fp32 out; fp64 out for launch_cumsum64).
hipError_t launch_cumsum(const float* x, float* c, int64_t rows, int64_t L, hipStream_t s);
hipError_t launch_cumsum64(const float* x, double* c, int64_t rows, int64_t L, hipStream_t s);
// The cumulative log decay c as the attention kernels take it: fp32, or fp64 (FOX_C_F64).
struct CPtr {
  const void* p = nullptr;
  bool f64 = false;
};
// out[r, l] = sum_{t >= l} (a[r, t] + b[r, t]) (fp64 accumulation, fp32 out).
hipError_t launch_rev_cumsum2(const float* a, const float* b, float* out, int64_t rows, int64_t L,
                              hipStream_t s);
// What a per-head gate GEMV z = x . w^T + b (b may be null) returns: log sigma(z) (the forget
// gate) or sigma(z) (the Pro block's shift gates).
enum class GateKind { kLogSigmoid, kSigmoid };
// out[b, h, t] = log sigmoid(z) or sigmoid(z), z = x[b, t, :] . w_f[h, :] + b_f[h].
hipError_t launch_gate(const void* x, bool x_bf16, const float* w_f, const float* b_f, float* out,
                       int64_t B, int64_t L, int64_t d_model, int64_t H, GateKind kind,
                       hipStream_t s);
// Backward of the gate's output: dz[b, h, t] = dout[b, h, t] * (d out / dz).
hipError_t launch_gate_dz(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                          const float* dout, float* dz, int64_t B, int64_t L, int64_t d_model,
                          int64_t H, GateKind kind, hipStream_t s);
// Backward of the gate: dx, dw_f and (when not null) db_f (workspace: gate_bwd_workspace_bytes).
// log_f (forget gate only, may be null): the forward's output, from which dz is formed without
// a pass over x.
size_t gate_bwd_workspace_bytes(int64_t B, int64_t L, int64_t d_model, int64_t H);
hipError_t launch_gate_bwd(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                           const float* dout, const float* log_f, float* dx, float* dw_f,
                           float* db_f, void* ws, int64_t B, int64_t L, int64_t d_model, int64_t H,
                           GateKind kind, hipStream_t s);
// Backward of the QK-norm: dx and, when dw is not null, the weight gradient.
size_t rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t D);
hipError_t launch_rmsnorm_bwd(const void* x, bool bf16, const float* dy, const float* w, float* dx,
                              float* dw, void* ws, int64_t rows, int64_t D, float eps,
                              hipStream_t s);
// y = x / sqrt(mean(x^2) + eps) * w over rows of length D.
hipError_t launch_rmsnorm(const void* x, void* y, bool bf16, int64_t rows, int64_t D, float eps,
                          const float* w, hipStream_t s);
// Pro block token shift (optionally RMS-normalised) and output norm + gate (pro_fuse.hip).
hipError_t launch_kv_shift(const void* x, bool bf16, const float* alpha, void* y, bool norm,
                           float eps, const float* w, int64_t rows, int64_t L, int64_t D,
                           hipStream_t s);
hipError_t launch_kv_shift_bwd(const void* x, bool bf16, const float* alpha, const float* dy,
                               float* dx, float* dalpha, bool norm, float eps, const float* w,
                               int64_t rows, int64_t L, int64_t D, hipStream_t s);
hipError_t launch_out_norm_gate(const void* o, bool o_bf16, const void* g, bool g_bf16,
                                const float* w, float eps, void* y, int64_t rows, int64_t D,
                                hipStream_t s);
hipError_t launch_out_norm_gate_bwd(const void* o, bool o_bf16, const void* g, bool g_bf16,
                                    const float* w, float eps, const float* dy, float* d_o,
                                    float* dg, int64_t rows, int64_t D, hipStream_t s);
// Skip plan (skip_plan.hip): byte offsets of its four arrays and its size.
//   q_skip   : int32 [BH, ceil(L / 256)]  leading key tiles a 256-query tile skips
//   kv_tiles : int32 [BH, ceil(L / 128)]  64-query tiles a 128-key block walks
//   qn, kn   : fp32  [BH, ceil(L / 64)]   largest row norm of q / k per 64-row group
//   q_order  : int32 [BH * ceil(L / 256)] launch order of the query tiles (index bh n_qt + qt),
//                                         most work first
//   kv_order : int32 [BH * ceil(L / 128)] the same for the key blocks (index bh n_kb + kb)
struct SkipPlanLayout {
  size_t q_skip, kv_tiles, qn, kn, cmin, cmax, q_order, kv_order, bytes;
};
SkipPlanLayout skip_plan_layout(int64_t BH, int64_t L);
hipError_t launch_skip_plan(const void* q, const void* k, const float* c, void* plan, int64_t BH,
                            int64_t L, int64_t D, float scale, hipStream_t s);
// The plan's arrays the kernels read (all null without a plan).
struct SkipArgs {
  const int32_t* q_skip = nullptr;
  const int32_t* q_order = nullptr;
  const int32_t* kv_tiles = nullptr;
  const int32_t* kv_order = nullptr;
};
SkipArgs skip_args(const void* plan, int64_t BH, int64_t L);
// Pro-block options of the bf16 forward: QK-norm of q on load, output norm and gate in the
// epilogue (y = RMSNorm(O) [* out_w] * sigmoid(g), y in g's type).
struct ProFwdArgs {
  bool q_norm = false;
  const float* q_w = nullptr;
  float q_eps = 0.f;
  const void* g = nullptr;
  bool g_f32 = false;
  const float* out_w = nullptr;
  float out_eps = 0.f;
  void* y = nullptr;
  const float* k_alpha = nullptr;  // key shift gate [B, H, L] (k holds the raw candidates)
  const float* v_alpha = nullptr;  // value shift gate [B, H, L]
  bool k_norm = false;             // RMS-normalise the (shifted) key rows on load
  const float* k_w = nullptr;
  float k_eps = 0.f;
};
// Forward, bf16 inputs on MFMA; O in bf16 or fp32 (o may be null when pa->y is set).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, CPtr c, void* o,
                           bool o_f32, float* lse, int64_t BH, int64_t L, int64_t D, float scale,
                           const SkipArgs& skip, hipStream_t s, const ProFwdArgs* pa = nullptr);
// Forward from log f with the prefix sum fused in (bf16 inputs); also writes c (c_out: fp32, or
// fp64 when c_out.f64).
hipError_t launch_fwd_bf16_logf(const void* q, const void* k, const void* v, const float* log_f,
                                CPtr c_out, void* o, bool o_f32, float* lse, int64_t BH, int64_t L,
                                int64_t D, float scale, hipStream_t s);
// Forward, fp32 inputs and outputs, fp32 arithmetic throughout.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, CPtr c, float* o,
                          float* lse, int64_t BH, int64_t L, int64_t D, float scale, hipStream_t s);
// Workspace bytes of the bf16 backward.
size_t bwd_workspace_bytes(int64_t BH, int64_t L);
// The static scratch array of noalloc.hip: its size, and its device address on the current
// device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);
// Backward steps: Delta = rowsum(dO * O); query-stationary dQ, dc^q, the refined Delta
// (delta_out may equal delta; with delta null the step forms Delta from o itself, bit-identical
// to launch_bwd_delta) and the normalised row offset lse_out; key-stationary dK, dV, dc^k from
// the refined Delta and lse_out.
hipError_t launch_bwd_delta(const void* dO, const float* o, float* delta, int64_t rows, int64_t D,
                            hipStream_t s);
hipError_t launch_bwd_dkv(const void* q, const void* k, const void* v, CPtr c,
                          const float* lse, const void* dO, const float* delta, float* dk,
                          float* dv, float* dck, int64_t BH, int64_t L, int64_t D, float scale,
                          const SkipArgs& skip, hipStream_t s);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, CPtr c,
                         const float* lse, const void* dO, const float* delta, const float* o,
                         float* dq, float* dcq, float* delta_out, float* lse_out, int64_t BH,
                         int64_t L, int64_t D, float scale, const SkipArgs& skip, hipStream_t s);
// Single-token decode against a KV cache [BH, T, D] (bf16) with c [BH, T] and per-sequence
// lengths lens [B]: o [BH, D] (bf16 or fp32) and lse [BH]; workspace decode_workspace_bytes.
// k_norms [BH, ceil(T / 64)] (largest key norm per 64 positions) or null: with it, chunks
// whose weights all underflow are not read.
size_t decode_workspace_bytes(int64_t BH, int64_t T, int64_t D);
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* c,
                         const int32_t* lens, const float* k_norms, void* o, bool o_f32,
                         float* lse, void* ws, int64_t B, int64_t H, int64_t T, int64_t D,
                         float scale, hipStream_t s);
hipError_t launch_decode_key_norms(const void* k, const int32_t* lens, float* k_norms, int64_t B,
                                   int64_t H, int64_t T, int64_t D, hipStream_t s);
// Append one position per sequence at lens[b] (k, v, c = c_prev + log f and, when k_norms is not
// null, the group's key norm), then lens += 1.
hipError_t launch_decode_append(const void* k_new, const void* v_new, const float* logf_new,
                                void* k, void* v, float* c, float* k_norms, int32_t* lens,
                                int64_t B, int64_t H, int64_t T, int64_t D, hipStream_t s);
// Backward, bf16 inputs, fp32 O / gradients: the four steps in order (plan: a skip plan or
// null).
// The fp32 backward (vector ALU): the same four steps and workspace as the bf16 path.
hipError_t launch_bwd_delta_f32(const float* dO, const float* o, float* delta, int64_t rows,
                                int64_t D, hipStream_t s);
hipError_t launch_bwd_dq_f32(const float* q, const float* k, const float* v, CPtr c,
                             const float* lse, const float* dO, const float* delta, float* dq,
                             float* dcq, float* delta_out, float* lse_out, int64_t BH, int64_t L,
                             int64_t D, float scale, hipStream_t s);
hipError_t launch_bwd_dkv_f32(const float* q, const float* k, const float* v, CPtr c,
                              const float* lse, const float* dO, const float* delta, float* dk,
                              float* dv, float* dck, int64_t BH, int64_t L, int64_t D, float scale,
                              hipStream_t s);
hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, CPtr c,
                          const float* o, const float* lse, const float* dO, float* dq, float* dk,
                          float* dv, float* dlog_f, void* ws, int64_t BH, int64_t L, int64_t D,
                          float scale, hipStream_t s);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, CPtr c,
                           const float* o, const float* lse, const void* dO, float* dq, float* dk,
                           float* dv, float* dlog_f, void* ws, int64_t BH, int64_t L, int64_t D,
                           float scale, const void* plan, hipStream_t s);

}  // namespace fox
