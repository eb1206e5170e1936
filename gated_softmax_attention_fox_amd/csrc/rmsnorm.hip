// rmsnorm.hip — QK-norm of the Pro block (paper-graph-ui summary of arXiv 2503.02130, section 3.4,
// "The Pro Block Architecture", Steps 1-2: RMSNorm over the head dimension of every query and key).
//
// y = x / sqrt(mean_d x^2 + eps) * w, per row of length D (64 or 128). HBM-bound: D/8 lanes own
// a row, each loads 8 elements (16 B for bf16), squares are summed in fp32 across the lane group
// with shuffles, and the row is scaled and stored with one rounding.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

template <int D, bool kBf16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* xv, void* yv,
                                                      int64_t rows, float eps,
                                                      const float* __restrict__ w) {
  constexpr int G = D / 8;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / G;
  const int part = (int)(gid % G);
  const bool ok = row < rows;
  float v[8];
  const size_t off = (size_t)(ok ? row : 0) * D + part * 8;
  if (kBf16) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (ok) raw = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(xv) + off);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w4[e] << 16);
      v[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
    }
  } else {
    float4 a = make_float4(0, 0, 0, 0), b = a;
    if (ok) {
      a = *reinterpret_cast<const float4*>(static_cast<const float*>(xv) + off);
      b = *reinterpret_cast<const float4*>(static_cast<const float*>(xv) + off + 4);
    }
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
  for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = v[e] * r * (w ? w[part * 8 + e] : 1.0f);
  if (!ok) return;
  if (kBf16) {
    uint32_t o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o4[e] = (uint32_t)f2bf(y[2 * e]) | ((uint32_t)f2bf(y[2 * e + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(yv) + off) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(yv) + off) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(static_cast<float*>(yv) + off + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
}

template <int D, bool kBf16>
hipError_t go(const void* x, void* y, int64_t rows, float eps, const float* w, hipStream_t s) {
  const int64_t threads = rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((rmsnorm_kernel<D, kBf16>), dim3(blocks), dim3(256), 0, s, x, y, rows, eps, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, void* y, bool bf16, int64_t rows, int64_t D, float eps,
                          const float* w, hipStream_t s) {
  if (D == 64) return bf16 ? go<64, true>(x, y, rows, eps, w, s) : go<64, false>(x, y, rows, eps, w, s);
  return bf16 ? go<128, true>(x, y, rows, eps, w, s) : go<128, false>(x, y, rows, eps, w, s);
}

}  // namespace fox
