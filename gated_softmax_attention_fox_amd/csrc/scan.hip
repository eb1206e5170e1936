// scan.hip — prefix sums along the sequence axis.
//
// Forward: c_i = sum_{l<=i} log f_l, the cumulative log decay that Forgetting Attention needs
// once per head before attention (paper-graph-ui summary of arXiv 2503.02130, section 3.4,
// "Hardware-Aware Implementation (Modified FlashAttention)": precompute c = cumsum(log f)).
// Reverse: d log f_l = sum_{t>=l} dc_t, the adjoint of that sum, which turns the gradient of c
// into the gradient of log f (same section, backward pass).
//
// One 256-thread workgroup per row. Each thread owns a contiguous segment, sums it in fp64,
// the workgroup scans the 256 segment totals with 64-wide wavefront shuffles plus one LDS step
// across the 4 waves, and each thread then rewrites its segment with the running fp64 sum,
// rounding once to fp32. fp64 keeps c_i - c_j free of accumulated rounding: the only error
// left is the single fp32 rounding of each c_i.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kScanThreads = 256;

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
  __shared__ double wave_tot[kScanThreads / 64];
  const int64_t row = blockIdx.x;
  a += row * L;
  if (kReverse) b += row * L;
  out += row * L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = (L + kScanThreads - 1) / kScanThreads;
  const int64_t s = (int64_t)tid * n;
  const int64_t e = s + n < L ? s + n : L;

  double tot = 0.0;
  for (int64_t i = s; i < e; ++i) tot += scan_load<kReverse>(a, b, L, i);

  // inclusive scan of segment totals inside the wave
  double x = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  double run = before + x - tot;  // exclusive prefix of this thread's segment

  for (int64_t i = s; i < e; ++i) {
    run += scan_load<kReverse>(a, b, L, i);
    out[kReverse ? (L - 1 - i) : i] = (float)run;
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
