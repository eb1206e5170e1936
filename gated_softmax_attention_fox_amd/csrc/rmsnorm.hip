// rmsnorm.hip — QK-norm of the Pro block (paper-graph-ui summary of arXiv 2503.02130, section 3.4,
// "The Pro Block Architecture", Steps 1-2: RMSNorm over the head dimension of every query and key).
//
// y = x / sqrt(mean_d x^2 + eps) * w, per row of length D (64 or 128). HBM-bound: D/8 lanes own
// a row, each loads 8 elements (16 B for bf16), squares are summed in fp32 across the lane group
// with shuffles, and the row is scaled and stored with one rounding. Each thread serves four
// rows and issues all four loads first, so enough bytes are in flight to cover HBM latency.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kNormRowsPerThread = 4;  // row slots per thread, loaded before any is used

template <int D, bool kBf16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* xv, void* yv,
                                                      int64_t rows, float eps,
                                                      const float* __restrict__ w) {
  constexpr int G = D / 8;          // lanes per row
  constexpr int RB = 256 / G;       // rows per workgroup slot
  constexpr int R = kNormRowsPerThread;
  const int part = threadIdx.x % G;
  // slot r of this workgroup covers RB consecutive rows, so every load and store is coalesced
  int64_t row[R];
  bool ok[R];
  float v[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = ((int64_t)blockIdx.x * R + r) * RB + threadIdx.x / G;
    ok[r] = row[r] < rows;
    const size_t off = (size_t)(ok[r] ? row[r] : 0) * D + part * 8;
    if (kBf16) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (ok[r]) raw = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(xv) + off);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[r][2 * e] = __uint_as_float(w4[e] << 16);
        v[r][2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
      }
    } else {
      float4 a = make_float4(0, 0, 0, 0), b = a;
      if (ok[r]) {
        a = *reinterpret_cast<const float4*>(static_cast<const float*>(xv) + off);
        b = *reinterpret_cast<const float4*>(static_cast<const float*>(xv) + off + 4);
      }
      v[r][0] = a.x; v[r][1] = a.y; v[r][2] = a.z; v[r][3] = a.w;
      v[r][4] = b.x; v[r][5] = b.y; v[r][6] = b.z; v[r][7] = b.w;
    }
  }
  float wv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wv[e] = w ? w[part * 8 + e] : 1.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[r][e], v[r][e], ss);
#pragma unroll
    for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = v[r][e] * rs * wv[e];
    if (!ok[r]) continue;
    const size_t off = (size_t)row[r] * D + part * 8;
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
}

template <int D, bool kBf16>
hipError_t go(const void* x, void* y, int64_t rows, float eps, const float* w, hipStream_t s) {
  const int64_t rows_per_block = (int64_t)(256 / (D / 8)) * kNormRowsPerThread;
  const unsigned blocks = (unsigned)((rows + rows_per_block - 1) / rows_per_block);
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
