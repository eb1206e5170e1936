// fox_launch.h — host-side launchers of the gfx950 kernels (called by the C ABI in abi.cpp).
// Every launcher only enqueues work on `s` and returns the launch status; shapes have already
// been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fox {

// c[r, i] = sum_{l <= i} x[r, l] (fp64 accumulation, fp32 out).
hipError_t launch_cumsum(const float* x, float* c, int64_t rows, int64_t L, hipStream_t s);
// out[r, l] = sum_{t >= l} (a[r, t] + b[r, t]) (fp64 accumulation, fp32 out).
hipError_t launch_rev_cumsum2(const float* a, const float* b, float* out, int64_t rows, int64_t L,
                              hipStream_t s);
// log_f[b, h, t] = log sigmoid(x[b, t, :] . w_f[h, :] + b_f[h]).
hipError_t launch_gate(const void* x, bool x_bf16, const float* w_f, const float* b_f, float* log_f,
                       int64_t B, int64_t L, int64_t d_model, int64_t H, hipStream_t s);
// Backward of the gate: dz[b, t, h] = dlog_f[b, h, t] * sigma(-z) (token-major).
hipError_t launch_gate_dz(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                          const float* dlog_f, float* dz, int64_t B, int64_t L, int64_t d_model,
                          int64_t H, hipStream_t s);
// Backward of the gate: dx, dw_f, db_f (workspace: gate_bwd_workspace_bytes).
size_t gate_bwd_workspace_bytes(int64_t B, int64_t L, int64_t d_model, int64_t H);
hipError_t launch_gate_bwd(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                           const float* dlog_f, float* dx, float* dw_f, float* db_f, void* ws,
                           int64_t B, int64_t L, int64_t d_model, int64_t H, hipStream_t s);
// Backward of the QK-norm: dx and, when dw is not null, the weight gradient.
size_t rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t D);
hipError_t launch_rmsnorm_bwd(const void* x, bool bf16, const float* dy, const float* w, float* dx,
                              float* dw, void* ws, int64_t rows, int64_t D, float eps,
                              hipStream_t s);
// y = x / sqrt(mean(x^2) + eps) * w over rows of length D.
hipError_t launch_rmsnorm(const void* x, void* y, bool bf16, int64_t rows, int64_t D, float eps,
                          const float* w, hipStream_t s);
// Forward, bf16 inputs on MFMA; O in bf16 or fp32.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, const float* c, void* o,
                           bool o_f32, float* lse, int64_t BH, int64_t L, int64_t D, float scale,
                           hipStream_t s);
// Forward, fp32 inputs and outputs, fp32 arithmetic throughout.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, const float* c, float* o,
                          float* lse, int64_t BH, int64_t L, int64_t D, float scale, hipStream_t s);
// Workspace bytes of the bf16 backward.
size_t bwd_workspace_bytes(int64_t BH, int64_t L);
// Backward steps: Delta = rowsum(dO * O); query-stationary dQ, dc^q and the refined Delta
// (delta_out may equal delta); key-stationary dK, dV, dc^k from the refined Delta.
hipError_t launch_bwd_delta(const void* dO, const float* o, float* delta, int64_t rows, int64_t D,
                            hipStream_t s);
hipError_t launch_bwd_dkv(const void* q, const void* k, const void* v, const float* c,
                          const float* lse, const void* dO, const float* delta, float* dk,
                          float* dv, float* dck, int64_t BH, int64_t L, int64_t D, float scale,
                          hipStream_t s);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* c,
                         const float* lse, const void* dO, const float* delta, float* dq,
                         float* dcq, float* delta_out, int64_t BH, int64_t L, int64_t D,
                         float scale, hipStream_t s);
// Backward, bf16 inputs, fp32 O / gradients: the four steps in order.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const float* c,
                           const float* o, const float* lse, const void* dO, float* dq, float* dk,
                           float* dv, float* dlog_f, void* ws, int64_t BH, int64_t L, int64_t D,
                           float scale, hipStream_t s);

}  // namespace fox
