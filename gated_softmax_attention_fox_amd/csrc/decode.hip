// decode.hip — one new token per sequence against a KV cache (single-token decode).
//
// At the last position t of a sequence, Forgetting Attention is
//   o_t = sum_{j<=t} softmax_j(scale q_t.k_j + c_t - c_j) v_j
// (paper-graph-ui summary, section 3.4, "The Mathematical Form of Forgetting Attention": the
// bias is the sum of log f over (j, t], here c_t - c_j with c the cumulative log forget gate of
// the cached positions). Appending a token extends c by c_t = c_{t-1} + log f_t, the recurrent
// form of the same prefix sum ("Hardware-Aware Implementation": c is the cumulative sum of
// log f).
//
// The step reads every cached key and value once, so it is bound by HBM. A workgroup of four
// waves takes a chunk of cached positions of one (b, h) and each wave streams a quarter of it
// with an online softmax, double-buffering its K and V rows in registers (decode_partial_kernel).
// The chunk writes (o, m, l) to the workspace; a second kernel combines the chunks of each
// (b, h) (m = max over chunks, l and o rescaled by exp2(m_c - m)) and normalises.
//
// Exact skipping (optional). With the largest key norm of every 64 cached positions at hand
// (kept beside the cache), a chunk whose every weight is provably below 2^-160 of the query's
// own-key weight is not read: for a key j of the chunk, scale q_t.(k_j - k_t) - (c_j - c_t)
// <= scale |q_t| (|k_j| + |k_t|) - (c_min - c_t), c_min the chunk's smallest c (its last one
// when the gates lie in (0, 1); the chunk's c values are read to find it, 4 bytes per position
// against the 4 D bytes of its key and value rows, so the test holds for any finite c). The
// combine would scale such a chunk by exp2(m_c - m) with m at least the own-key logit, which is
// exactly 0 in fp32, so skipping it changes no bit of the result.
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecRows = 4;  // rows per lane and tensor in one step of a wave

// Positions per workgroup: the largest power of two from 256 to 4096 that still gives at least
// 12 D workgroups (1536 at D = 128, six per compute unit), so short batches spread over the
// chip and long ones stream long ranges per wave. Measured on the decode shapes of the bench:
// smaller chunks pay the per-workgroup start and combine; larger ones leave units idle.
int decode_chunk(int64_t BH, int64_t T, int64_t D) {
  int64_t chunk = 256;
  while (chunk < 4096 && BH * ((T + 2 * chunk - 1) / (2 * chunk)) >= 12 * D) chunk *= 2;
  return (int)chunk;
}

// One workgroup per (chunk of positions, b, h); wave w streams positions
// [j0 + w chunk/4, j0 + (w + 1) chunk/4) in steps of 4 rows per lane (16 positions at D = 128,
// 32 at D = 64) with its own online softmax (reference
// m, sum l, weighted values acc), reading the next step's K and V rows into a second register
// buffer while it computes on the current one. D / 8 lanes share a row, so each load
// instruction reads whole rows (1 KiB contiguous). The waves are combined once at the end.
template <int D, bool kSkip>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ C, const int32_t* __restrict__ lens, const float* __restrict__ KN,
    float* __restrict__ part, int H, int T, int n_ch, int chunk, float sl2e) {
  constexpr int CPR = D / 8;          // lanes per row (16 bytes each)
  constexpr int RPI = 64 / CPR;       // rows per load instruction
  constexpr int IT = kDecRows;        // load instructions per tensor and step
  constexpr int kDecStep = IT * RPI;  // positions per step
  __shared__ float red[kDecWaves][D + 2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ch = blockIdx.x, bh = blockIdx.y;
  const int len = min(lens[bh / H], T);
  const int j0 = ch * chunk;
  if (len < 1 || j0 >= len) return;  // uniform over the workgroup, before the barrier
  const int t = len - 1;
  const int cw = chunk / kDecWaves;
  const int a = j0 + wave * cw;
  const int b = min(a + cw, len);  // this wave's positions [a, b); may be empty
  const int n_steps = b > a ? (b - a + kDecStep - 1) / kDecStep : 0;
  const int grp = lane / CPR, col = (lane % CPR) * 8;
  const size_t rows = (size_t)bh * T;
  const bf16_t* Kb = K + rows * D;
  const bf16_t* Vb = V + rows * D;
  const float* Cb = C + rows;
  const float ct = Cb[t];
  const bf16x8 qv = ld8(Q + (size_t)bh * D + col);
  float* out = part + ((size_t)bh * n_ch + ch) * (D + 2);

  // A separate instantiation: the bound's code in the dense kernel measured 9% slower even
  // when not taken.
  if constexpr (kSkip) {  // the bound of this chunk; every thread evaluates the same values
    const int n64 = (T + 63) / 64;
    const float* kn = KN + (size_t)bh * n64;
    float qq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qq = fmaf((float)qv[e], (float)qv[e], qq);
#pragma unroll
    for (int mk = 1; mk < CPR; mk <<= 1) qq += __shfl_xor(qq, mk, 64);
    const int g0 = j0 / 64, g1 = (min(j0 + chunk, len) - 1) / 64;
    float km = 0.f;
    for (int g = g0 + lane; g <= g1; g += 64) km = fmaxf(km, kn[g]);
#pragma unroll
    for (int mk = 1; mk < 64; mk <<= 1) km = fmaxf(km, __shfl_xor(km, mk, 64));
    const int j_end = min(j0 + chunk, len);
    float ce = INFINITY;  // the chunk's smallest c; 16 loads in flight per lane
#pragma unroll 16
    for (int j = j0 + lane; j < j_end; j += 64) ce = fminf(ce, Cb[j]);
#pragma unroll
    for (int mk = 1; mk < 64; mk <<= 1) ce = fminf(ce, __shfl_xor(ce, mk, 64));
    const float slack = 1e-6f * (fabsf(ce) + fabsf(ct)) + 1.f;
    const float bound = sl2e * sqrtf(qq) * 1.00001f * (km + kn[t / 64]) + (slack - (ce - ct)) * kLog2e;
    if (bound < -160.f) {  // nothing in this chunk can carry weight: an empty partial
      for (int d = threadIdx.x; d < D + 2; d += 256) out[d] = d == D ? -INFINITY : 0.f;
      return;
    }
  }

  auto load = [&](bf16x8 (&kr)[IT], bf16x8 (&vr)[IT], int step) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int j = a + step * kDecStep + i * RPI + grp;
      if (j < b) {  // read once: non-temporal loads (measured 8-13% faster than cached ones)
        kr[i] = __builtin_bit_cast(
            bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kb + (size_t)j * D + col)));
        vr[i] = __builtin_bit_cast(
            bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vb + (size_t)j * D + col)));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kr[i][e] = vr[i][e] = (__bf16)0.f;
      }
    }
  };
  float m = -INFINITY, l = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto process = [&](const bf16x8 (&kr)[IT], const bf16x8 (&vr)[IT], int step)
      __attribute__((always_inline)) {
    // logits in log2 units, log2(e) (scale q.k_j + c_t - c_j)
    float s[IT];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int j = a + step * kDecStep + i * RPI + grp;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf((float)qv[e], (float)kr[i][e], dot);
#pragma unroll
      for (int mk = 1; mk < CPR; mk <<= 1) dot += __shfl_xor(dot, mk, 64);
      s[i] = j < b ? fmaf(dot, sl2e, (ct - Cb[min(j, t)]) * kLog2e) : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
#pragma unroll
    for (int mk = CPR; mk < 64; mk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, mk, 64));
    const float mn = fmaxf(m, mx);  // finite: every step holds a position of [a, b)
    const float r = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    l *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[i] - m);  // 0 past b
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, (float)vr[i][e], acc[e]);
      l += p;
    }
  };
  bf16x8 k0[IT], v0[IT], k1[IT], v1[IT];
  if (n_steps > 0) load(k0, v0, 0);
  for (int st = 0; st < n_steps; st += 2) {
    if (st + 1 < n_steps) load(k1, v1, st + 1);
    process(k0, v0, st);
    if (st + 1 < n_steps) {
      if (st + 2 < n_steps) load(k0, v0, st + 2);
      process(k1, v1, st + 1);
    }
  }
  // sum over the row groups of the wave (all hold the same m), then combine the waves
#pragma unroll
  for (int mk = CPR; mk < 64; mk <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], mk, 64);
    l += __shfl_xor(l, mk, 64);
  }
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][col + e] = acc[e];
    if (lane == 0) {
      red[wave][D] = m;
      red[wave][D + 1] = l;
    }
  }
  __syncthreads();
  float mt = red[0][D];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) mt = fmaxf(mt, red[w][D]);  // wave 0 is never empty
  for (int d = threadIdx.x; d < D + 2; d += 256) {
    if (d == D) {
      out[d] = mt;
    } else {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float sw = red[w][D] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red[w][D] - mt);
        v = fmaf(sw, red[w][d], v);
      }
      out[d] = v;
    }
  }
}

// One workgroup of D threads per (b, h): combine the chunks, normalise, write o and lse.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ part,
                                                           const int32_t* __restrict__ lens,
                                                           void* __restrict__ O, int o_f32,
                                                           float* __restrict__ LSE, int H, int T,
                                                           int n_ch, int chunk) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const int len = min(lens[bh / H], T);
  const int n = (len + chunk - 1) / chunk;
  const float* p = part + (size_t)bh * n_ch * (D + 2);
  // unrolled so that eight chunks' loads are in flight at once
  float mt = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < n; ++c) mt = fmaxf(mt, p[(size_t)c * (D + 2) + D]);
  float l = 0.f, o = 0.f;
#pragma unroll 8
  for (int c = 0; c < n; ++c) {
    const float* pc = p + (size_t)c * (D + 2);
    const float a = __builtin_amdgcn_exp2f(pc[D] - mt);  // 0 for a skipped chunk (m = -inf)
    l = fmaf(a, pc[D + 1], l);
    o = fmaf(a, pc[d], o);
  }
  // len = 0 (an empty cache) has no defined output: it is written as zeros with lse = -inf
  const float y = n > 0 ? o / l : 0.f;
  if (o_f32)
    static_cast<float*>(O)[(size_t)bh * D + d] = y;
  else
    static_cast<bf16_t*>(O)[(size_t)bh * D + d] = f2bf(y);
  if (d == 0 && LSE) LSE[bh] = n > 0 ? (mt + __log2f(l)) * kLn2 : -INFINITY;
}

// Append one position per sequence at index lens[b]: k, v copied, c extended by log f.
template <int D>
__global__ __launch_bounds__(64) void decode_append_kernel(
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    const float* __restrict__ logf_new, bf16_t* __restrict__ K, bf16_t* __restrict__ V,
    float* __restrict__ C, float* __restrict__ KN, const int32_t* __restrict__ lens, int H,
    int T) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int pos = lens[bh / H];
  if (pos < 0 || pos >= T) return;  // a full cache is left unchanged (uniform: one wave)
  const size_t row = (size_t)bh * T + pos;
  float ss = 0.f;
  if (tid < D / 8) {
    const uint4 kw = *reinterpret_cast<const uint4*>(k_new + (size_t)bh * D + tid * 8);
    *reinterpret_cast<uint4*>(K + row * D + tid * 8) = kw;
    *reinterpret_cast<uint4*>(V + row * D + tid * 8) =
        *reinterpret_cast<const uint4*>(v_new + (size_t)bh * D + tid * 8);
    const bf16x8 kv = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf((float)kv[e], (float)kv[e], ss);
  }
#pragma unroll
  for (int mk = 1; mk < 64; mk <<= 1) ss += __shfl_xor(ss, mk, 64);
  if (tid == 0) {
    C[row] = (pos > 0 ? C[row - 1] : 0.f) + logf_new[bh];
    if (KN) {  // the group's largest key norm, restarted at a group's first position
      float* kn = KN + (size_t)bh * ((T + 63) / 64) + pos / 64;
      const float nk = sqrtf(ss) * 1.00001f;
      *kn = pos % 64 == 0 ? nk : fmaxf(*kn, nk);
    }
  }
}

// Largest key norm of every 64 cached positions (positions at or past the length count as 0).
template <int D>
__global__ __launch_bounds__(256) void decode_key_norms_kernel(const bf16_t* __restrict__ K,
                                                               const int32_t* __restrict__ lens,
                                                               float* __restrict__ KN, int H,
                                                               int T) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int lane = threadIdx.x & 63;
  const int n64 = (T + 63) / 64;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  if (g >= n64) return;  // a whole wave; the kernel has no barrier
  const int len = min(lens[bh / H], T);
  const bf16_t* Kb = K + (size_t)bh * T * D;
  float mx = 0.f;
  for (int it = 0; it < 64 / RPI; ++it) {
    const int row = g * 64 + it * RPI + lane / CPR;
    float ss = 0.f;
    if (row < len) {
      const bf16x8 v = ld8(Kb + (size_t)row * D + (lane % CPR) * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)v[e], (float)v[e], ss);
    }
#pragma unroll
    for (int mk = 1; mk < CPR; mk <<= 1) ss += __shfl_xor(ss, mk, 64);
    mx = fmaxf(mx, sqrtf(ss));
  }
#pragma unroll
  for (int mk = CPR; mk < 64; mk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, mk, 64));
  if (lane == 0) KN[(size_t)bh * n64 + g] = mx * 1.00001f;  // rounded up
}

__global__ void decode_advance_kernel(int32_t* __restrict__ lens, int B, int T) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B && lens[b] >= 0 && lens[b] < T) lens[b] += 1;
}

}  // namespace

size_t decode_workspace_bytes(int64_t BH, int64_t T, int64_t D) {
  const int64_t chunk = decode_chunk(BH, T, D);
  const size_t n_ch = (size_t)((T + chunk - 1) / chunk);
  return ((size_t)BH * n_ch * (size_t)(D + 2) * sizeof(float) + 255) & ~size_t(255);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* c,
                         const int32_t* lens, const float* k_norms, void* o, bool o_f32,
                         float* lse, void* ws, int64_t B, int64_t H, int64_t T, int64_t D,
                         float scale, hipStream_t s) {
  const int chunk = decode_chunk(B * H, T, D);
  const int n_ch = (int)((T + chunk - 1) / chunk);
  const dim3 g1((unsigned)n_ch, (unsigned)(B * H));
  float* part = static_cast<float*>(ws);
  if (D == 64) {
    if (k_norms)
      hipLaunchKernelGGL((decode_partial_kernel<64, true>), g1, dim3(256), 0, s, (const bf16_t*)q,
                         (const bf16_t*)k, (const bf16_t*)v, c, lens, k_norms, part, (int)H,
                         (int)T, n_ch, chunk, scale * kLog2e);
    else
      hipLaunchKernelGGL((decode_partial_kernel<64, false>), g1, dim3(256), 0, s, (const bf16_t*)q,
                         (const bf16_t*)k, (const bf16_t*)v, c, lens, k_norms, part, (int)H,
                         (int)T, n_ch, chunk, scale * kLog2e);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)(B * H)), dim3(64), 0, s, part,
                       lens, o, (int)o_f32, lse, (int)H, (int)T, n_ch, chunk);
  } else {
    if (k_norms)
      hipLaunchKernelGGL((decode_partial_kernel<128, true>), g1, dim3(256), 0, s,
                         (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, c, lens, k_norms,
                         part, (int)H, (int)T, n_ch, chunk, scale * kLog2e);
    else
      hipLaunchKernelGGL((decode_partial_kernel<128, false>), g1, dim3(256), 0, s,
                         (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, c, lens, k_norms,
                         part, (int)H, (int)T, n_ch, chunk, scale * kLog2e);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)(B * H)), dim3(128), 0, s,
                       part, lens, o, (int)o_f32, lse, (int)H, (int)T, n_ch, chunk);
  }
  return hipGetLastError();
}

hipError_t launch_decode_key_norms(const void* k, const int32_t* lens, float* k_norms, int64_t B,
                                   int64_t H, int64_t T, int64_t D, hipStream_t s) {
  const int n64 = (int)((T + 63) / 64);
  const dim3 grid((unsigned)((n64 + 3) / 4), (unsigned)(B * H));
  if (D == 64)
    hipLaunchKernelGGL(decode_key_norms_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)k, lens,
                       k_norms, (int)H, (int)T);
  else
    hipLaunchKernelGGL(decode_key_norms_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)k,
                       lens, k_norms, (int)H, (int)T);
  return hipGetLastError();
}

hipError_t launch_decode_append(const void* k_new, const void* v_new, const float* logf_new,
                                void* k, void* v, float* c, float* k_norms, int32_t* lens,
                                int64_t B, int64_t H, int64_t T, int64_t D, hipStream_t s) {
  if (D == 64)
    hipLaunchKernelGGL(decode_append_kernel<64>, dim3((unsigned)(B * H)), dim3(64), 0, s,
                       (const bf16_t*)k_new, (const bf16_t*)v_new, logf_new, (bf16_t*)k,
                       (bf16_t*)v, c, k_norms, lens, (int)H, (int)T);
  else
    hipLaunchKernelGGL(decode_append_kernel<128>, dim3((unsigned)(B * H)), dim3(64), 0, s,
                       (const bf16_t*)k_new, (const bf16_t*)v_new, logf_new, (bf16_t*)k,
                       (bf16_t*)v, c, k_norms, lens, (int)H, (int)T);
  hipLaunchKernelGGL(decode_advance_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s,
                     lens, (int)B, (int)T);
  return hipGetLastError();
}

}  // namespace fox
