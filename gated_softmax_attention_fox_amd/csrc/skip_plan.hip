// skip_plan.hip — which tiles of the attention kernels carry no weight at all.
//
// The forget gate makes the weight of a key decay with its distance from the query: the logit
// carries the bias c_i - c_j, and c falls by -log f per position. The pages name pruning of
// computation by the gate values as future work (paperlayer.ai summary, section 6
// "CONCLUSION", limitations and future work; paper-graph-ui summary, "Follow-Up Research",
// KV-cache eviction before sharp forget gates). This file does it without changing any result:
// a tile is skipped only when every weight in it is provably below 2^-160 of the row's
// reference, where exp2 in fp32 already returns exactly zero.
//
// The bound. For a query i and an earlier key j (natural-log units)
//   logit_ij - logit_ii = scale q_i.(k_j - k_i) - (c_j - c_i)
//                      <= scale |q_i| (|k_j| + |k_i|) - (c_j - c_i).
// The kernels subtract at least logit_ii from every logit of row i before the exponential:
// the forward's running max is set on the diagonal block first and only rises, and the
// backward subtracts LSE_i >= logit_ii. Over a query range and an earlier key range,
// c_j - c_i >= Cmin - Cmax with Cmin the smallest c of the key range and Cmax the largest c of
// the query range, so
//   log2(weight) <= log2(e) (scale Qmax (Kmax + Kdiag) - (Cmin - Cmax))
// with Qmax the largest |q_i| of the range, Kmax the largest |k_j| and Kdiag the largest
// |k_i| at the query positions. A tile is skipped when this bound, plus a slack for the fp32
// rounding of c, is below -160. A forget gate in (0, 1) makes c non-increasing, and then Cmin
// and Cmax are c at the key range's last and the query range's first position; the extremes
// are taken over every 64-position group all the same, so the plan stays exact for any finite c.
//
// The plan holds, per (b, h): the largest row norm of q and of k and the smallest and largest c
// in every 64-row group; per
// 256-query tile, the number of leading key tiles the forward and the query-stationary
// backward skip (the oldest keys, a prefix of the key tiles that lie before the tile's diagonal
// band); per 128-key block, the number of 64-query tiles the key-stationary backward walks
// from its diagonal (the skipped query tiles are the last ones); and, for both kinds of item, a
// launch order by decreasing work, so that the longest items start first once skipping has
// made the work per item uneven across heads.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr float kSkipLog2 = -160.f;

// Largest row norm of every 64-row group of q (blockIdx.z = 0) and k (1), and the smallest and
// largest c of every group (2). One wave per group; each load instruction covers 1 KiB
// (64 / (D / 8) whole rows), so the reads are contiguous.
template <int D>
__global__ __launch_bounds__(256) void group_norm_kernel(const bf16_t* __restrict__ q,
                                                         const bf16_t* __restrict__ k,
                                                         const float* __restrict__ C,
                                                         float* __restrict__ qn,
                                                         float* __restrict__ kn,
                                                         float* __restrict__ cmin,
                                                         float* __restrict__ cmax, int L,
                                                         int n64) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  if (g >= n64) return;  // a whole wave; the kernel has no barrier
  if (blockIdx.z == 2) {
    const int j = g * 64 + lane;
    const float cj = j < L ? C[(size_t)bh * L + j] : C[(size_t)bh * L + L - 1];
    float lo = cj, hi = cj;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, m, 64));
      hi = fmaxf(hi, __shfl_xor(hi, m, 64));
    }
    if (lane == 0) {
      cmin[(size_t)bh * n64 + g] = lo;
      cmax[(size_t)bh * n64 + g] = hi;
    }
    return;
  }
  const bf16_t* x = (blockIdx.z == 0 ? q : k) + (size_t)bh * L * D;
  float mx = 0.f;
#pragma unroll 4
  for (int it = 0; it < 64 / RPI; ++it) {
    const int row = g * 64 + it * RPI + lane / CPR;
    float ss = 0.f;
    if (row < L) {
      const bf16x8 v = ld8(x + (size_t)row * D + (lane % CPR) * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)v[e];
        ss = fmaf(f, f, ss);
      }
    }
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    mx = fmaxf(mx, sqrtf(ss));
  }
#pragma unroll
  for (int m = CPR; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  // Round up: fp32 sums of squares and the square root are within a few ulp.
  if (lane == 0) (blockIdx.z == 0 ? qn : kn)[(size_t)bh * n64 + g] = mx * (1.f + 1e-5f);
}

// True when every weight between a key range whose smallest c is ck_min and a query range
// whose largest c is cq_max is below 2^kSkipLog2; a = scale Qmax (Kmax + Kdiag).
__device__ __forceinline__ bool decayed(float a, float ck_min, float cq_max) {
  const float slack = 1e-6f * (fabsf(ck_min) + fabsf(cq_max)) + 1.f;
  return (a - (ck_min - cq_max) + slack) * kLog2e < kSkipLog2;
}

// One wave per plan entry: entries [0, BH n_qt) are the 256-query tiles, the rest the 128-key
// blocks. Candidates are tested 64 at a time, one per lane.
__global__ __launch_bounds__(256) void skip_plan_kernel(const float* __restrict__ cmin,
                                                        const float* __restrict__ cmax,
                                                        const float* __restrict__ qn,
                                                        const float* __restrict__ kn,
                                                        int32_t* __restrict__ q_skip,
                                                        int32_t* __restrict__ kv_tiles, int L,
                                                        int BH, int n64, int n_qt, int n_kb,
                                                        float scale) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_q = BH * n_qt;
  if (e >= n_q + BH * n_kb) return;  // a whole wave; the kernel has no barrier
  if (e < n_q) {
    const int bh = e / n_qt, qt = e % n_qt;
    const float* cmn = cmin + (size_t)bh * n64;
    const float* cmx = cmax + (size_t)bh * n64;
    const float* qnh = qn + (size_t)bh * n64;
    const float* knh = kn + (size_t)bh * n64;
    const int q0 = qt * 256;
    const int q_last = min(q0 + 255, L - 1);
    const int n_old = q_last / 64 - 3;  // key tiles 0 .. n_old - 1 lie before the diagonal band
    int skip = 0;
    if (n_old > 0) {
      float qmax = 0.f, kdiag = 0.f, cq = -INFINITY;
      for (int g = q0 / 64; g <= q_last / 64; ++g) {
        qmax = fmaxf(qmax, qnh[g]);
        kdiag = fmaxf(kdiag, knh[g]);
        cq = fmaxf(cq, cmx[g]);
      }
      skip = n_old;
      for (int base = 0; base < n_old; base += 64) {
        const int t = base + lane;
        const bool keep = t < n_old && !decayed(scale * qmax * (knh[t] + kdiag), cmn[t], cq);
        const uint64_t m = __ballot(keep);
        if (m) {
          skip = base + __builtin_ctzll(m);
          break;
        }
      }
    }
    if (lane == 0) q_skip[e] = skip;
  } else {
    const int e2 = e - n_q;
    const int bh = e2 / n_kb, kb = e2 % n_kb;
    const float* cmn = cmin + (size_t)bh * n64;
    const float* cmx = cmax + (size_t)bh * n64;
    const float* qnh = qn + (size_t)bh * n64;
    const float* knh = kn + (size_t)bh * n64;
    const int k0 = kb * 128;
    const int n_full = (L - k0 + 63) / 64;  // query tiles from the diagonal to the sequence end
    int walk = n_full;
    if (n_full > 2) {  // tiles 0 and 1 hold the block's diagonal and are always walked
      const float kmax = fmaxf(knh[2 * kb], 2 * kb + 1 < n64 ? knh[2 * kb + 1] : 0.f);
      const float ck = fminf(cmn[2 * kb], 2 * kb + 1 < n64 ? cmn[2 * kb + 1] : INFINITY);
      int last_keep = 1;
      for (int base = 2; base < n_full; base += 64) {
        const int t = base + lane;
        bool keep = false;
        if (t < n_full) {
          const int g = 2 * kb + t;
          keep = !decayed(scale * qnh[g] * (kmax + knh[g]), ck, cmx[g]);
        }
        const uint64_t m = __ballot(keep);
        if (m) last_keep = base + 63 - __builtin_clzll(m);
      }
      walk = last_keep + 1;
    }
    if (lane == 0) kv_tiles[e2] = walk;
  }
}

// Launch order by decreasing work: a counting sort of the items on the number of tiles each
// walks (clamped to kOrderBins - 1). One workgroup per kind of item (blockIdx.x = 0: the
// 256-query tiles, 1: the 128-key blocks). Items of equal work land in an arbitrary order; each
// item writes only its own outputs, so the order never changes a result.
constexpr int kOrderBins = 4096;
__global__ __launch_bounds__(1024) void skip_order_kernel(const int32_t* __restrict__ q_skip,
                                                          const int32_t* __restrict__ kv_tiles,
                                                          int32_t* __restrict__ q_order,
                                                          int32_t* __restrict__ kv_order, int L,
                                                          int BH, int n_qt, int n_kb) {
  __shared__ int cnt[kOrderBins];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const bool kv = blockIdx.x == 1;
  const int n = BH * (kv ? n_kb : n_qt);
  int32_t* order = kv ? kv_order : q_order;
  auto bin = [&](int e) {
    int w;
    if (kv) {
      w = kv_tiles[e];
    } else {
      const int q_last = min((e % n_qt) * 256 + 255, L - 1);
      w = q_last / 64 + 1 - q_skip[e];
    }
    return kOrderBins - 1 - min(w, kOrderBins - 1);  // most work first
  };
  for (int b = tid; b < kOrderBins; b += 1024) cnt[b] = 0;
  __syncthreads();
  for (int e = tid; e < n; e += 1024) atomicAdd(&cnt[bin(e)], 1);
  __syncthreads();
  // exclusive prefix sum: four bins per thread, then a scan of the 1024 partial sums
  constexpr int PER = kOrderBins / 1024;
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += cnt[PER * tid + i];
  part[tid] = local;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int add = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - local;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = cnt[PER * tid + i];
    cnt[PER * tid + i] = run;
    run += c;
  }
  __syncthreads();
  for (int e = tid; e < n; e += 1024) order[atomicAdd(&cnt[bin(e)], 1)] = e;
}

}  // namespace

SkipPlanLayout skip_plan_layout(int64_t BH, int64_t L) {
  auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_qt = (size_t)((L + 255) / 256), n_kb = (size_t)((L + 127) / 128);
  const size_t n64 = (size_t)((L + 63) / 64);
  SkipPlanLayout p;
  p.q_skip = 0;
  p.kv_tiles = a256(p.q_skip + 4 * (size_t)BH * n_qt);
  p.qn = a256(p.kv_tiles + 4 * (size_t)BH * n_kb);
  p.kn = a256(p.qn + 4 * (size_t)BH * n64);
  p.cmin = a256(p.kn + 4 * (size_t)BH * n64);
  p.cmax = a256(p.cmin + 4 * (size_t)BH * n64);
  p.q_order = a256(p.cmax + 4 * (size_t)BH * n64);
  p.kv_order = a256(p.q_order + 4 * (size_t)BH * n_qt);
  p.bytes = a256(p.kv_order + 4 * (size_t)BH * n_kb);
  return p;
}

SkipArgs skip_args(const void* plan, int64_t BH, int64_t L) {
  SkipArgs a;
  if (!plan) return a;
  const SkipPlanLayout p = skip_plan_layout(BH, L);
  const unsigned char* base = static_cast<const unsigned char*>(plan);
  a.q_skip = reinterpret_cast<const int32_t*>(base + p.q_skip);
  a.q_order = reinterpret_cast<const int32_t*>(base + p.q_order);
  a.kv_tiles = reinterpret_cast<const int32_t*>(base + p.kv_tiles);
  a.kv_order = reinterpret_cast<const int32_t*>(base + p.kv_order);
  return a;
}

hipError_t launch_skip_plan(const void* q, const void* k, const float* c, void* plan, int64_t BH,
                            int64_t L, int64_t D, float scale, hipStream_t s) {
  const SkipPlanLayout p = skip_plan_layout(BH, L);
  unsigned char* base = static_cast<unsigned char*>(plan);
  float* qn = reinterpret_cast<float*>(base + p.qn);
  float* kn = reinterpret_cast<float*>(base + p.kn);
  float* cmn = reinterpret_cast<float*>(base + p.cmin);
  float* cmx = reinterpret_cast<float*>(base + p.cmax);
  const int n64 = (int)((L + 63) / 64), n_qt = (int)((L + 255) / 256), n_kb = (int)((L + 127) / 128);
  const dim3 g1((unsigned)((n64 + 3) / 4), (unsigned)BH, 3);
  if (D == 64)
    hipLaunchKernelGGL(group_norm_kernel<64>, g1, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)k, c, qn, kn, cmn, cmx, (int)L, n64);
  else
    hipLaunchKernelGGL(group_norm_kernel<128>, g1, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)k, c, qn, kn, cmn, cmx, (int)L, n64);
  const int64_t entries = BH * (n_qt + n_kb);
  hipLaunchKernelGGL(skip_plan_kernel, dim3((unsigned)((entries + 3) / 4)), dim3(256), 0, s, cmn,
                     cmx, qn, kn, reinterpret_cast<int32_t*>(base + p.q_skip),
                     reinterpret_cast<int32_t*>(base + p.kv_tiles), (int)L, (int)BH, n64, n_qt,
                     n_kb, scale);
  hipLaunchKernelGGL(skip_order_kernel, dim3(2), dim3(1024), 0, s,
                     reinterpret_cast<const int32_t*>(base + p.q_skip),
                     reinterpret_cast<const int32_t*>(base + p.kv_tiles),
                     reinterpret_cast<int32_t*>(base + p.q_order),
                     reinterpret_cast<int32_t*>(base + p.kv_order), (int)L, (int)BH, n_qt, n_kb);
  return hipGetLastError();
}

}  // namespace fox
