// pro_fuse.hip — the Pro block's token shift and output normalisation + gate, fused passes.
//
// Paper-graph-ui summary, section 3.4, "The Pro Block Architecture":
//   Steps 2-3 (data-dependent token shift): the shift gate alpha_t in (0, 1) interpolates between
//     the previous position's key (value) candidate and the current one,
//       y_t = alpha_t x_{t-1} + (1 - alpha_t) x_t   (x_{-1} = 0),
//     and keys are then RMS-normalised (QK-norm) while values are not;
//   Steps 5 and 7 (output gate and output normalisation): y = RMSNorm(o) [* w] * sigma(g), g the
//     per-dimension output-gate pre-activation W_g x, before the output projection.
// The page's equations are missing; these are the plainest readings of its words. The
// projections (W_k x, W_v x, W_g x, W_o) are plain GEMMs outside this library.
//
// All four kernels are bound by HBM. D / 8 lanes share one row (8 elements each, so a load is
// 16 or 32 bytes per lane and a row group reads whole rows); row sums are shuffles within the
// group. The shift's backward recomputes the shifted rows t and t + 1 (dx_t needs the gradient
// of row t + 1), so it reads x once more from cache rather than storing the pre-norm rows.
#include <type_traits>

#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

template <typename T>
__device__ __forceinline__ void load_row8(const T* p, float (&v)[8]) {
  if constexpr (std::is_same<T, float>::value) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const bf16x8 x = ld8(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  }
}

template <typename T>
__device__ __forceinline__ void store_row8(T* p, const float (&v)[8]) {
  if constexpr (std::is_same<T, float>::value) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Sum over the D / 8 lanes of a row group.
template <int D>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int m = 1; m < D / 8; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + expf(-z)); }

// Shifted row v = a prev + (1 - a) cur, optionally RMS-normalised (weight w or unit).
template <int D, typename T, bool kNorm>
__global__ __launch_bounds__(256) void kv_shift_kernel(const T* __restrict__ x,
                                                       const float* __restrict__ alpha,
                                                       T* __restrict__ y, const float* __restrict__ w,
                                                       float eps, int64_t rows, int L) {
  constexpr int CPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / CPR) + threadIdx.x / CPR;
  const int c = (threadIdx.x % CPR) * 8;
  if (row >= rows) return;  // a whole row group (the groups never mix in a shuffle)
  const int t = (int)(row % L);
  float cur[8], prev[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  load_row8(x + row * D + c, cur);
  if (t > 0) load_row8(x + (row - 1) * D + c, prev);
  const float a = alpha[row];
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = shift_mix(a, prev[e], cur[e]);
  if constexpr (kNorm) rms_norm8<D>(v, w, c, eps);
  store_row8(y + row * D + c, v);
}

// Gradient with respect to the pre-norm shifted row v, given dy for the row's output.
template <int D, bool kNorm>
__device__ __forceinline__ void pre_norm_grad(const float (&v)[8], const float (&dy)[8],
                                              const float* w, int c, float eps, float (&g)[8]) {
  if constexpr (kNorm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    const float r = rms_scale<D>(row_sum<D>(ss), eps);
    float gw[8], dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gw[e] = dy[e] * (w ? w[c + e] : 1.0f);
      dot = fmaf(gw[e], v[e] * r, dot);
    }
    const float mean = row_sum<D>(dot) / D;
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = (gw[e] - v[e] * r * mean) * r;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = dy[e];
  }
}

// dx_t = (1 - a_t) g_t + a_{t+1} g_{t+1},  dalpha_t = sum g_t (x_{t-1} - x_t), g the gradient of
// the pre-norm shifted row.
template <int D, typename T, bool kNorm>
__global__ __launch_bounds__(256) void kv_shift_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ alpha, const float* __restrict__ dy,
    float* __restrict__ dx, float* __restrict__ dalpha, const float* __restrict__ w, float eps,
    int64_t rows, int L) {
  constexpr int CPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / CPR) + threadIdx.x / CPR;
  const int c = (threadIdx.x % CPR) * 8;
  if (row >= rows) return;
  const int t = (int)(row % L);
  float cur[8], prev[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, d0[8];
  load_row8(x + row * D + c, cur);
  if (t > 0) load_row8(x + (row - 1) * D + c, prev);
  load_row8(dy + row * D + c, d0);
  const float a = alpha[row];
  float v[8], g0[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = shift_mix(a, prev[e], cur[e]);
  pre_norm_grad<D, kNorm>(v, d0, w, c, eps, g0);
  float out[8], da = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    out[e] = (1.0f - a) * g0[e];
    da = fmaf(g0[e], prev[e] - cur[e], da);
  }
  if (t + 1 < L) {
    float nxt[8], d1[8], v1[8], g1[8];
    load_row8(x + (row + 1) * D + c, nxt);
    load_row8(dy + (row + 1) * D + c, d1);
    const float a1 = alpha[row + 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) v1[e] = shift_mix(a1, cur[e], nxt[e]);
    pre_norm_grad<D, kNorm>(v1, d1, w, c, eps, g1);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = fmaf(a1, g1[e], out[e]);
  }
  store_row8(dx + row * D + c, out);
  da = row_sum<D>(da);
  if (c == 0) dalpha[row] = da;
}

// y = o / sqrt(mean(o^2) + eps) [* w] * sigma(g).
template <int D, typename TO, typename TG>
__global__ __launch_bounds__(256) void out_norm_gate_kernel(const TO* __restrict__ o,
                                                            const TG* __restrict__ g,
                                                            const float* __restrict__ w, float eps,
                                                            TG* __restrict__ y, int64_t rows) {
  constexpr int CPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / CPR) + threadIdx.x / CPR;
  const int c = (threadIdx.x % CPR) * 8;
  if (row >= rows) return;
  float v[8], gg[8];
  load_row8(o + row * D + c, v);
  load_row8(g + row * D + c, gg);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  const float r = rsqrtf(row_sum<D>(ss) / D + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = v[e] * r * (w ? w[c + e] : 1.0f) * sigm(gg[e]);
  store_row8(y + row * D + c, v);
}

// dg = dy n s (1 - s) with n = RMSNorm(o) [* w], s = sigma(g); do = RMSNorm backward of dy s.
template <int D, typename TO, typename TG>
__global__ __launch_bounds__(256) void out_norm_gate_bwd_kernel(
    const TO* __restrict__ o, const TG* __restrict__ g, const float* __restrict__ w, float eps,
    const float* __restrict__ dy, float* __restrict__ d_o, float* __restrict__ dg, int64_t rows) {
  constexpr int CPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / CPR) + threadIdx.x / CPR;
  const int c = (threadIdx.x % CPR) * 8;
  if (row >= rows) return;
  float v[8], gg[8], d[8];
  load_row8(o + row * D + c, v);
  load_row8(g + row * D + c, gg);
  load_row8(dy + row * D + c, d);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  const float r = rsqrtf(row_sum<D>(ss) / D + eps);
  float gw[8], dgo[8], dot = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float we = w ? w[c + e] : 1.0f;
    const float s = sigm(gg[e]);
    dgo[e] = d[e] * v[e] * r * we * s * sigm(-gg[e]);
    gw[e] = d[e] * s * we;
    dot = fmaf(gw[e], v[e] * r, dot);
  }
  const float mean = row_sum<D>(dot) / D;
  float out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (gw[e] - v[e] * r * mean) * r;
  store_row8(d_o + row * D + c, out);
  store_row8(dg + row * D + c, dgo);
}

template <int D>
dim3 row_grid(int64_t rows) {
  return dim3((unsigned)((rows + 256 / (D / 8) - 1) / (256 / (D / 8))));
}

template <int D, typename T>
void go_shift(const void* x, const float* alpha, void* y, bool norm, float eps, const float* w,
              int64_t rows, int64_t L, hipStream_t s) {
  if (norm)
    hipLaunchKernelGGL((kv_shift_kernel<D, T, true>), row_grid<D>(rows), dim3(256), 0, s,
                       (const T*)x, alpha, (T*)y, w, eps, rows, (int)L);
  else
    hipLaunchKernelGGL((kv_shift_kernel<D, T, false>), row_grid<D>(rows), dim3(256), 0, s,
                       (const T*)x, alpha, (T*)y, w, eps, rows, (int)L);
}

template <int D, typename T>
void go_shift_bwd(const void* x, const float* alpha, const float* dy, float* dx, float* dalpha,
                  bool norm, float eps, const float* w, int64_t rows, int64_t L, hipStream_t s) {
  if (norm)
    hipLaunchKernelGGL((kv_shift_bwd_kernel<D, T, true>), row_grid<D>(rows), dim3(256), 0, s,
                       (const T*)x, alpha, dy, dx, dalpha, w, eps, rows, (int)L);
  else
    hipLaunchKernelGGL((kv_shift_bwd_kernel<D, T, false>), row_grid<D>(rows), dim3(256), 0, s,
                       (const T*)x, alpha, dy, dx, dalpha, w, eps, rows, (int)L);
}

template <int D, typename TO, typename TG>
void go_out(const void* o, const void* g, const float* w, float eps, void* y, const float* dy,
            float* d_o, float* dg, int64_t rows, bool bwd, hipStream_t s) {
  if (bwd)
    hipLaunchKernelGGL((out_norm_gate_bwd_kernel<D, TO, TG>), row_grid<D>(rows), dim3(256), 0, s,
                       (const TO*)o, (const TG*)g, w, eps, dy, d_o, dg, rows);
  else
    hipLaunchKernelGGL((out_norm_gate_kernel<D, TO, TG>), row_grid<D>(rows), dim3(256), 0, s,
                       (const TO*)o, (const TG*)g, w, eps, (TG*)y, rows);
}

template <int D>
void go_out_d(const void* o, bool o_bf16, const void* g, bool g_bf16, const float* w, float eps,
              void* y, const float* dy, float* d_o, float* dg, int64_t rows, bool bwd,
              hipStream_t s) {
  if (o_bf16 && g_bf16) go_out<D, bf16_t, bf16_t>(o, g, w, eps, y, dy, d_o, dg, rows, bwd, s);
  else if (o_bf16) go_out<D, bf16_t, float>(o, g, w, eps, y, dy, d_o, dg, rows, bwd, s);
  else if (g_bf16) go_out<D, float, bf16_t>(o, g, w, eps, y, dy, d_o, dg, rows, bwd, s);
  else go_out<D, float, float>(o, g, w, eps, y, dy, d_o, dg, rows, bwd, s);
}

}  // namespace

hipError_t launch_kv_shift(const void* x, bool bf16, const float* alpha, void* y, bool norm,
                           float eps, const float* w, int64_t rows, int64_t L, int64_t D,
                           hipStream_t s) {
  if (D == 64) {
    if (bf16) go_shift<64, bf16_t>(x, alpha, y, norm, eps, w, rows, L, s);
    else go_shift<64, float>(x, alpha, y, norm, eps, w, rows, L, s);
  } else {
    if (bf16) go_shift<128, bf16_t>(x, alpha, y, norm, eps, w, rows, L, s);
    else go_shift<128, float>(x, alpha, y, norm, eps, w, rows, L, s);
  }
  return hipGetLastError();
}

hipError_t launch_kv_shift_bwd(const void* x, bool bf16, const float* alpha, const float* dy,
                               float* dx, float* dalpha, bool norm, float eps, const float* w,
                               int64_t rows, int64_t L, int64_t D, hipStream_t s) {
  if (D == 64) {
    if (bf16) go_shift_bwd<64, bf16_t>(x, alpha, dy, dx, dalpha, norm, eps, w, rows, L, s);
    else go_shift_bwd<64, float>(x, alpha, dy, dx, dalpha, norm, eps, w, rows, L, s);
  } else {
    if (bf16) go_shift_bwd<128, bf16_t>(x, alpha, dy, dx, dalpha, norm, eps, w, rows, L, s);
    else go_shift_bwd<128, float>(x, alpha, dy, dx, dalpha, norm, eps, w, rows, L, s);
  }
  return hipGetLastError();
}

hipError_t launch_out_norm_gate(const void* o, bool o_bf16, const void* g, bool g_bf16,
                                const float* w, float eps, void* y, int64_t rows, int64_t D,
                                hipStream_t s) {
  if (D == 64) go_out_d<64>(o, o_bf16, g, g_bf16, w, eps, y, nullptr, nullptr, nullptr, rows, false, s);
  else go_out_d<128>(o, o_bf16, g, g_bf16, w, eps, y, nullptr, nullptr, nullptr, rows, false, s);
  return hipGetLastError();
}

hipError_t launch_out_norm_gate_bwd(const void* o, bool o_bf16, const void* g, bool g_bf16,
                                    const float* w, float eps, const float* dy, float* d_o,
                                    float* dg, int64_t rows, int64_t D, hipStream_t s) {
  if (D == 64) go_out_d<64>(o, o_bf16, g, g_bf16, w, eps, nullptr, dy, d_o, dg, rows, true, s);
  else go_out_d<128>(o, o_bf16, g, g_bf16, w, eps, nullptr, dy, d_o, dg, rows, true, s);
  return hipGetLastError();
}

}  // namespace fox
