// scan.hip — prefix sums along the sequence axis.
//
// Forward: c_i = sum_{l<=i} log f_l, the cumulative log decay that Forgetting Attention needs
// once per head before attention (paper-graph-ui summary of arXiv 2503.02130, section 3.4,
// "Hardware-Aware Implementation (Modified FlashAttention)": precompute c = cumsum(log f)).
// Reverse: d log f_l = sum_{t>=l} dc_t, the adjoint of that sum, which turns the gradient of c
// into the gradient of log f (same section, backward pass).
//
// One 1024-thread workgroup per row, in tiles of 16384 elements. Each thread owns 16 consecutive
// positions of the scan order and keeps them in registers as fp64 (the reverse sum adds its two
// inputs exactly there); a row whose length is a multiple of 4 moves them as four 16-byte loads
// and stores per thread. Each thread sums its 16 values, the workgroup scans the 1024 thread
// totals with 64-wide wavefront shuffles plus one LDS step across the 16 waves, each thread
// rewrites its values with the running fp64 sum, and the result is rounded once to fp32 (or kept
// in fp64 for the fp64 form of c); the tile total carries into the next tile. fp64 keeps
// c_i - c_j free of accumulated rounding: the only error left is the single rounding of each
// c_i to the output type. The rows are short (a few hundred KB), so the time is latency: the
// dependent chain per thread is 16 adds, not a full segment walk.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;                        // consecutive scan positions per thread
constexpr int kScanTile = kScanThreads * kScanPer;  // positions per pass of the workgroup
constexpr int kScanWaves = kScanThreads / 64;

template <bool kReverse>
__device__ __forceinline__ double scan_load(const float* __restrict__ a, const float* __restrict__ b,
                                            int64_t L, int64_t i) {
  if (kReverse) {
    const int64_t p = L - 1 - i;
    return (double)a[p] + (double)b[p];
  }
  return (double)a[i];
}

// 16-byte store of four consecutive outputs (two for fp64 values, done twice).
__device__ __forceinline__ void store4(float* p, const float (&r)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ void store4(double* p, const double (&r)[4]) {
  reinterpret_cast<double2*>(p)[0] = make_double2(r[0], r[1]);
  reinterpret_cast<double2*>(p)[1] = make_double2(r[2], r[3]);
}

// Forward: out[i] = sum_{l<=i} a[l]. Reverse: out[l] = sum_{t>=l} (a[t] + b[t]). Scan position
// k is memory position k (forward) or L-1-k (reverse). OutT: float, or double for the fp64 c.
template <bool kReverse, typename OutT>
__global__ __launch_bounds__(kScanThreads) void scan_rows_kernel(const float* __restrict__ a,
                                                                 const float* __restrict__ b,
                                                                 OutT* __restrict__ out,
                                                                 int64_t L) {
  __shared__ double wave_tot[2][kScanWaves];  // two copies: a pass never waits for the last reads
  const int64_t row = blockIdx.x;
  a += row * L;
  if (kReverse) b += row * L;
  out += row * L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // 16-byte moves where every row pointer is 16-byte aligned (then so is each thread's block)
  const uintptr_t align = (uintptr_t)a | (uintptr_t)out | (kReverse ? (uintptr_t)b : (uintptr_t)0);
  const bool vec = (L & 3) == 0 && (align & 15) == 0;
  double carry = 0.0;
  int par = 0;
  for (int64_t t0 = 0; t0 < L; t0 += kScanTile, par ^= 1) {
    const int64_t k0 = t0 + (int64_t)tid * kScanPer;  // this thread's first scan position
    const int cnt = L - k0 <= 0 ? 0 : (L - k0 < kScanPer ? (int)(L - k0) : kScanPer);
    const bool full = vec && cnt == kScanPer;
    // memory position of this thread's block (the lowest address it touches when full)
    const int64_t p0 = kReverse ? L - kScanPer - k0 : k0;
    double v[kScanPer];
    if (full) {
#pragma unroll
      for (int g = 0; g < kScanPer / 4; ++g) {
        const float4 x = *reinterpret_cast<const float4*>(a + p0 + 4 * g);
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kReverse) y = *reinterpret_cast<const float4*>(b + p0 + 4 * g);
        const double m[4] = {(double)x.x + (double)y.x, (double)x.y + (double)y.y,
                             (double)x.z + (double)y.z, (double)x.w + (double)y.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[kReverse ? kScanPer - 1 - (4 * g + e) : 4 * g + e] = m[e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j) v[j] = j < cnt ? scan_load<kReverse>(a, b, L, k0 + j) : 0.0;
    }
    double tot = 0.0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) tot += v[j];
    // inclusive scan of the thread totals inside the wave, then across the waves
    double x = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[par][wave] = x;
    __syncthreads();
    double before = carry, tile_tot = 0.0;
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) {
      const double t = wave_tot[par][w];
      if (w < wave) before += t;
      tile_tot += t;
    }
    double run = before + x - tot;  // exclusive prefix of this thread's block
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      run += v[j];
      v[j] = run;
    }
    carry += tile_tot;
    if (full) {
#pragma unroll
      for (int g = 0; g < kScanPer / 4; ++g) {
        OutT r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (OutT)v[kReverse ? kScanPer - 1 - (4 * g + e) : 4 * g + e];
        store4(out + p0 + 4 * g, r);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j) {
        if (j < cnt) out[kReverse ? (L - 1 - (k0 + j)) : (k0 + j)] = (OutT)v[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_cumsum(const float* x, float* c, int64_t rows, int64_t L, hipStream_t s) {
  hipLaunchKernelGGL((scan_rows_kernel<false, float>), dim3((unsigned)rows), dim3(kScanThreads), 0,
                     s, x, (const float*)nullptr, c, L);
  return hipGetLastError();
}

hipError_t launch_cumsum64(const float* x, double* c, int64_t rows, int64_t L, hipStream_t s) {
  hipLaunchKernelGGL((scan_rows_kernel<false, double>), dim3((unsigned)rows), dim3(kScanThreads),
                     0, s, x, (const float*)nullptr, c, L);
  return hipGetLastError();
}

hipError_t launch_rev_cumsum2(const float* a, const float* b, float* out, int64_t rows, int64_t L,
                              hipStream_t s) {
  hipLaunchKernelGGL((scan_rows_kernel<true, float>), dim3((unsigned)rows), dim3(kScanThreads), 0, s,
                     a, b, out, L);
  return hipGetLastError();
}

}  // namespace fox
