// scan.hip — prefix sums along the sequence axis.
//
// Forward: c_i = sum_{l<=i} log f_l, the cumulative log decay that Forgetting Attention needs
// once per head before attention (paper-graph-ui summary of arXiv 2503.02130, section 3.4,
// "Hardware-Aware Implementation (Modified FlashAttention)": precompute c = cumsum(log f)).
// Reverse: d log f_l = sum_{t>=l} dc_t, the adjoint of that sum, which turns the gradient of c
// into the gradient of log f (same section, backward pass).
//
// One 256-thread workgroup per row, in tiles of 16384 elements staged through LDS. Each tile is
// loaded with coalesced reads (in fp64; the reverse sum adds its two inputs exactly there) into
// 256 contiguous segments of 64, padded by one slot so that the threads' segment walks do not
// collide on a bank. Each thread sums its segment in fp64, the workgroup scans the 256 segment
// totals with 64-wide wavefront shuffles plus one LDS step across the 4 waves, each thread
// rewrites its segment with the running fp64 sum, and the tile is stored with coalesced writes,
// rounded once to fp32; the tile total carries into the next tile. fp64 keeps c_i - c_j free
// of accumulated rounding: the only error left is the single fp32 rounding of each c_i.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanPer = 64;                          // elements per thread segment
constexpr int kScanTile = kScanThreads * kScanPer;    // elements per LDS tile
constexpr int kScanPad = kScanPer + 1;                // LDS stride of a segment (bank spread)

template <bool kReverse>
__device__ __forceinline__ double scan_load(const float* __restrict__ a, const float* __restrict__ b,
                                            int64_t L, int64_t i) {
  if (kReverse) {
    const int64_t p = L - 1 - i;
    return (double)a[p] + (double)b[p];
  }
  return (double)a[i];
}

template <bool kReverse>
__global__ __launch_bounds__(kScanThreads) void scan_rows_kernel(const float* __restrict__ a,
                                                                 const float* __restrict__ b,
                                                                 float* __restrict__ out,
                                                                 int64_t L) {
  __shared__ double tile[kScanThreads * kScanPad];
  __shared__ double wave_tot[kScanThreads / 64];
  const int64_t row = blockIdx.x;
  a += row * L;
  if (kReverse) b += row * L;
  out += row * L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double carry = 0.0;
  for (int64_t t0 = 0; t0 < L; t0 += kScanTile) {
    const int n = L - t0 < kScanTile ? (int)(L - t0) : kScanTile;
    // coalesced loads in scan order (i = t0 + k), scattered into padded segments; unrolled so
    // that many loads are in flight at once (the inputs usually come cold from HBM)
#pragma unroll 16
    for (int k = tid; k < n; k += kScanThreads)
      tile[(k / kScanPer) * kScanPad + k % kScanPer] = scan_load<kReverse>(a, b, L, t0 + k);
    __syncthreads();
    const int cnt = n - tid * kScanPer < 0 ? 0 : (n - tid * kScanPer < kScanPer ? n - tid * kScanPer : kScanPer);
    double* seg = tile + tid * kScanPad;
    double tot = 0.0;
    for (int j = 0; j < cnt; ++j) tot += seg[j];
    // inclusive scan of segment totals inside the wave, then across the 4 waves
    double x = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    double before = carry, tile_tot = 0.0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      if (w < wave) before += wave_tot[w];
      tile_tot += wave_tot[w];
    }
    double run = before + x - tot;  // exclusive prefix of this thread's segment
    for (int j = 0; j < cnt; ++j) {
      run += seg[j];
      seg[j] = run;
    }
    carry += tile_tot;
    __syncthreads();
#pragma unroll 16
    for (int k = tid; k < n; k += kScanThreads) {
      const int64_t i = t0 + k;
      out[kReverse ? (L - 1 - i) : i] = (float)tile[(k / kScanPer) * kScanPad + k % kScanPer];
    }
    __syncthreads();  // the next tile reuses the LDS
  }
}

}  // namespace

hipError_t launch_cumsum(const float* x, float* c, int64_t rows, int64_t L, hipStream_t s) {
  hipLaunchKernelGGL(scan_rows_kernel<false>, dim3((unsigned)rows), dim3(kScanThreads), 0, s, x,
                     (const float*)nullptr, c, L);
  return hipGetLastError();
}

hipError_t launch_rev_cumsum2(const float* a, const float* b, float* out, int64_t rows, int64_t L,
                              hipStream_t s) {
  hipLaunchKernelGGL(scan_rows_kernel<true>, dim3((unsigned)rows), dim3(kScanThreads), 0, s, a, b,
                     out, L);
  return hipGetLastError();
}

}  // namespace fox
