// gate.hip — the scalar per-head forget gate in log space.
//
// log f[b, h, t] = log sigmoid(z), z = sum_d x[b, t, d] w_f[h, d] + b_f[h]  (paper-graph-ui summary
// of arXiv 2503.02130, section 3.4, "Forget Gate Computation": one weight vector and one bias per
// head applied to the layer input; Pro block Step 4 keeps the same gate).
//
// HBM-bound contraction with H (~12) outputs per token, done on the vector ALU: a workgroup owns
// 64 tokens, stages x through LDS in coalesced 256-column slabs, and each of its 4 waves walks a
// quarter of every slab with one token per lane. The gate weights are read with wave-uniform
// addresses (scalar loads), so the inner loop is one FMA per (token, head, column). It runs in
// fp64: the products of fp32 x and w are exact there and the sum rounds only at fp64, so z is
// the fp64 sum rounded once to fp32 whatever d_model and sum |x w| are (an fp32 running sum over
// a wave's 384 columns at d_model 1536 moved log f by up to 1.5e-5 where sum |x w| reached ~200).
// The
// four per-wave partial sums meet in LDS and lane t writes log f for token t, evaluated stably
// as -log1p(exp(-z)) for z >= 0 and z - log1p(exp(z)) otherwise.
//
// The same kernel serves the backward (kBwd): it recomputes z and writes
// dz[b, h, t] = dlog_f[b, h, t] * sigma(-z), since d log sigma(z) / dz = 1 - sigma(z) = sigma(-z);
// sigma(-z) = 1 / (1 + exp(z)) goes to 0 or 1 in the limits without a NaN.
//
// With kSig the output is sigma(z) itself and the bias may be absent: the Pro block's shift gates
// (Steps 2-3, one learned vector per head), whose backward takes dz = dalpha sigma(z) sigma(-z).
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kGateTok = 64;       // tokens per workgroup
constexpr int kGateSlab = 256;     // x columns staged per step
constexpr int kGatePitch = kGateSlab + 8;
constexpr int kGateHeads = 16;     // heads handled per workgroup (blockIdx.y walks head groups)
constexpr int kGateSB = 3;         // 32-column steps per load batch of the matrix-core gate

__device__ __forceinline__ float log_sigmoid(float z) {
  return z >= 0.f ? -log1pf(expf(-z)) : z - log1pf(expf(z));
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

template <bool kBf16, bool kBwd, bool kSig>
__global__ __launch_bounds__(256) void gate_kernel(const void* __restrict__ xv,
                                                   const float* __restrict__ w_f,
                                                   const float* __restrict__ b_f,
                                                   const float* __restrict__ dlog_f,
                                                   float* __restrict__ out, int L, int dm, int H,
                                                   int tok_blocks) {
  __shared__ bf16_t xs_b[kBf16 ? kGateTok * kGatePitch : 1];
  __shared__ float xs_f[kBf16 ? 1 : kGateTok * kGatePitch];
  __shared__ double red[4][kGateHeads][kGateTok];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / tok_blocks;
  const int t0 = (blockIdx.x % tok_blocks) * kGateTok;
  const int h0 = blockIdx.y * kGateHeads;
  const int nh = H - h0 < kGateHeads ? H - h0 : kGateHeads;

  double acc[kGateHeads];
#pragma unroll
  for (int h = 0; h < kGateHeads; ++h) acc[h] = 0.0;

  for (int d0 = 0; d0 < dm; d0 += kGateSlab) {
    const int width = dm - d0 < kGateSlab ? dm - d0 : kGateSlab;  // multiple of 8
    __syncthreads();
    // stage x[b, t0 .. t0+63, d0 .. d0+width) into LDS, 8 columns per thread-step
    for (int idx = tid; idx < kGateTok * (kGateSlab / 8); idx += 256) {
      const int r = idx / (kGateSlab / 8), c8 = (idx % (kGateSlab / 8)) * 8;
      const int t = t0 + r;
      const bool ok = t < L && c8 < width;
      const size_t g = ((size_t)b * L + t) * dm + d0 + c8;
      if (kBf16) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(xv) + g);
        *reinterpret_cast<uint4*>(&xs_b[r * kGatePitch + c8]) = v;
      } else {
        float4 v0 = make_float4(0, 0, 0, 0), v1 = v0;
        if (ok) {
          v0 = *reinterpret_cast<const float4*>(static_cast<const float*>(xv) + g);
          v1 = *reinterpret_cast<const float4*>(static_cast<const float*>(xv) + g + 4);
        }
        *reinterpret_cast<float4*>(&xs_f[r * kGatePitch + c8]) = v0;
        *reinterpret_cast<float4*>(&xs_f[r * kGatePitch + c8 + 4]) = v1;
      }
    }
    __syncthreads();
    // wave w covers columns [64w, 64w+64) of the slab; lane = token
    const int cw0 = wave * 64;
    for (int c8 = 0; c8 < 64; c8 += 8) {
      const int col = cw0 + c8;
      if (col >= width) break;  // wave-uniform
      float xv8[8];
      if (kBf16) {
        const uint4 raw = *reinterpret_cast<const uint4*>(&xs_b[lane * kGatePitch + col]);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv8[2 * e] = __uint_as_float(w4[e] << 16);
          xv8[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv8[e] = xs_f[lane * kGatePitch + col + e];
      }
#pragma unroll
      for (int h = 0; h < kGateHeads; ++h) {
        if (h < nh) {
          const float* wr = w_f + (size_t)(h0 + h) * dm + d0 + col;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h] = fma((double)xv8[e], (double)wr[e], acc[h]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kGateHeads; ++h) red[wave][h][lane] = acc[h];
  __syncthreads();
  if (wave == 0) {
    const int t = t0 + lane;
    for (int h = 0; h < nh; ++h) {
      const float z = (float)(((red[0][h][lane] + red[1][h][lane]) +
                               (red[2][h][lane] + red[3][h][lane])) +
                              (b_f ? (double)b_f[h0 + h] : 0.0));
      if (t < L) {
        if constexpr (kBwd) {
          const float g = dlog_f[((size_t)b * H + h0 + h) * L + t];
          out[((size_t)b * H + h0 + h) * L + t] =
              kSig ? g * sigmoid(z) / (1.0f + expf(z)) : g / (1.0f + expf(z));
        } else {
          out[((size_t)b * H + h0 + h) * L + t] = kSig ? sigmoid(z) : log_sigmoid(z);
        }
      }
    }
  }
}

// bf16 x on the matrix cores: z[16 tokens][16 heads] = x[16 tokens][:] . w_f[16 heads][:]^T with
// v_mfma_f32_16x16x32_bf16. A workgroup of 8 waves takes NTT tiles of 16 tokens (blockIdx.y picks
// the group of 16 heads). Wave w takes the 32-column steps d0 = 32 (w + 8 s); lane l supplies
// A = x[token l % 16][d0 + 8 (l / 16) .. +7] straight from HBM and B = w_f[head l % 16][same
// columns]. w_f is split into three bf16 parts (hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid)) that together hold all 24 bits of its significand, and all three are
// multiplied: the products are exact, so z carries only the fp32 accumulation's rounding (two
// parts, 16 bits of w, leave z off by up to 2^-17 of sum |x w|: 4e-5 in log f at d_model 1536
// and |w| ~ 0.1). Lane l receives z for head l % 16 and tokens 4 (l / 16) .. +3. Needs
// d_model % 32 == 0.
// Measured on the Pro shape (x [16384, 1536]), the costs beyond the bare x stream were the w_f
// reads (each workgroup reads all of w_f for its heads: with 64 tokens per workgroup that stream
// is half of what 32 tokens cost) and a one-wave epilogue of scattered stores. So every load of a
// batch of kGateSB steps is issued before its first product, padded heads load nothing, and the
// epilogue spreads the (head, token) outputs over all 512 threads, each head's 64 tokens stored
// contiguously.
template <bool kBwd, bool kSig, int NTT>
__global__ __launch_bounds__(512) void gate_mfma_kernel(const bf16_t* __restrict__ x,
                                                        const float* __restrict__ w_f,
                                                        const float* __restrict__ b_f,
                                                        const float* __restrict__ dlog_f,
                                                        float* __restrict__ out, int L, int dm,
                                                        int H, int tiles_per_b, int n_tiles) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __shared__ f32x4v part[8][NTT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int h0 = blockIdx.y * 16;
  const int hh = h0 + r;
  const bool head_ok = hh < H;
  const float* wr = w_f + (size_t)(head_ok ? hh : 0) * dm + 8 * grp;
  // The workgroup's NTT token tiles (flattened over batch rows; tiles past the end are skipped).
  const bf16_t* xr[NTT];
  bool tok_ok[NTT];
#pragma unroll
  for (int u = 0; u < NTT; ++u) {
    const int tile = blockIdx.x * NTT + u;
    const int tl = tile < n_tiles ? tile : 0;
    const int b = tl / tiles_per_b, t = (tl % tiles_per_b) * 16 + r;
    tok_ok[u] = tile < n_tiles && t < L;
    xr[u] = x + ((size_t)b * L + (t < L ? t : L - 1)) * dm + 8 * grp;
  }
  f32x4v acc[NTT];
#pragma unroll
  for (int u = 0; u < NTT; ++u) acc[u] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int n_steps = (dm / 32 - wave + 7) / 8;  // this wave's 32-column steps
  for (int s0 = 0; s0 < n_steps; s0 += kGateSB) {
    u32x4 xa[kGateSB][NTT];
    float4 wa[kGateSB][2];
#pragma unroll
    for (int j = 0; j < kGateSB; ++j) {
      if (s0 + j < n_steps) {  // wave-uniform
        const int d0 = 32 * (wave + 8 * (s0 + j));
#pragma unroll
        for (int u = 0; u < NTT; ++u) xa[j][u] = *reinterpret_cast<const u32x4*>(xr[u] + d0);
        if (head_ok) {
          wa[j][0] = *reinterpret_cast<const float4*>(wr + d0);
          wa[j][1] = *reinterpret_cast<const float4*>(wr + d0 + 4);
        } else {
          wa[j][0] = make_float4(0.f, 0.f, 0.f, 0.f);
          wa[j][1] = wa[j][0];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kGateSB; ++j) {
      if (s0 + j >= n_steps) break;
      const float wv[8] = {wa[j][0].x, wa[j][0].y, wa[j][0].z, wa[j][0].w,
                           wa[j][1].x, wa[j][1].y, wa[j][1].z, wa[j][1].w};
      bf16x8 bh, bm, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hi = (__bf16)wv[e];
        const float r1 = wv[e] - (float)hi;
        const __bf16 mid = (__bf16)r1;
        bh[e] = hi;
        bm[e] = mid;
        bl[e] = (__bf16)(r1 - (float)mid);
      }
#pragma unroll
      for (int u = 0; u < NTT; ++u) {  // one load and split of w_f serves all the tiles
        const bf16x8 a = __builtin_bit_cast(bf16x8, tok_ok[u] ? xa[j][u] : zero4);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[u], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NTT; ++u) part[wave][u][lane] = acc[u];
  __syncthreads();
  // Output (head h, token tok) of the workgroup's 16 NTT tokens: tile u = tok / 16; inside the
  // tile, accumulator lane h + 16 g holds tokens 4 g .. 4 g + 3 in its four slots. The eight wave
  // sums are added in wave order.
  const int nh = H - h0 < 16 ? H - h0 : 16;
  constexpr int kTok = 16 * NTT;
  const float* pf = reinterpret_cast<const float*>(part);
  for (int i = threadIdx.x; i < nh * kTok; i += 512) {
    const int h = i / kTok, tok = i % kTok;
    const int u = tok >> 4, tin = tok & 15, g = tin >> 2, j = tin & 3;
    const int tile = blockIdx.x * NTT + u;
    if (tile >= n_tiles) continue;
    const int b = tile / tiles_per_b, tt = (tile % tiles_per_b) * 16 + tin;
    if (tt >= L) continue;
    float zs = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) zs += pf[((w * NTT + u) * 64 + h + 16 * g) * 4 + j];
    const float z = zs + (b_f ? b_f[h0 + h] : 0.f);
    const size_t o = ((size_t)b * H + h0 + h) * L + tt;
    if constexpr (kBwd) {
      const float gd = dlog_f[o];
      out[o] = kSig ? gd * sigmoid(z) / (1.0f + expf(z)) : gd / (1.0f + expf(z));
    } else {
      out[o] = kSig ? sigmoid(z) : log_sigmoid(z);
    }
  }
}

constexpr int kGateTiles = 4;  // token tiles per workgroup of the matrix-core gate

template <bool kBwd, bool kSig>
void go_gate_mfma(const void* x, const float* w_f, const float* b_f, const float* dlog_f,
                  float* out, int64_t B, int64_t L, int64_t d_model, int64_t H, hipStream_t s) {
  const int tiles_per_b = (int)((L + 15) / 16);
  const int64_t n_tiles = B * tiles_per_b;
  const dim3 grid((unsigned)((n_tiles + kGateTiles - 1) / kGateTiles), (unsigned)((H + 15) / 16));
  hipLaunchKernelGGL((gate_mfma_kernel<kBwd, kSig, kGateTiles>), grid, dim3(512), 0, s,
                     static_cast<const bf16_t*>(x), w_f, b_f, dlog_f, out, (int)L, (int)d_model,
                     (int)H, tiles_per_b, (int)n_tiles);
}

}  // namespace

namespace {
template <bool kBwd, bool kSig>
hipError_t go_gate(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                   const float* dlog_f, float* out, int64_t B, int64_t L, int64_t d_model,
                   int64_t H, hipStream_t s) {
  if (x_bf16 && d_model % 32 == 0) {
    go_gate_mfma<kBwd, kSig>(x, w_f, b_f, dlog_f, out, B, L, d_model, H, s);
    return hipGetLastError();
  }
  const int tok_blocks = (int)((L + kGateTok - 1) / kGateTok);
  const dim3 grid((unsigned)(B * tok_blocks), (unsigned)((H + kGateHeads - 1) / kGateHeads));
  if (x_bf16)
    hipLaunchKernelGGL((gate_kernel<true, kBwd, kSig>), grid, dim3(256), 0, s, x, w_f, b_f,
                       dlog_f, out, (int)L, (int)d_model, (int)H, tok_blocks);
  else
    hipLaunchKernelGGL((gate_kernel<false, kBwd, kSig>), grid, dim3(256), 0, s, x, w_f, b_f,
                       dlog_f, out, (int)L, (int)d_model, (int)H, tok_blocks);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gate(const void* x, bool x_bf16, const float* w_f, const float* b_f, float* out,
                       int64_t B, int64_t L, int64_t d_model, int64_t H, GateKind kind,
                       hipStream_t s) {
  return kind == GateKind::kSigmoid
             ? go_gate<false, true>(x, x_bf16, w_f, b_f, nullptr, out, B, L, d_model, H, s)
             : go_gate<false, false>(x, x_bf16, w_f, b_f, nullptr, out, B, L, d_model, H, s);
}

hipError_t launch_gate_dz(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                          const float* dout, float* dz, int64_t B, int64_t L, int64_t d_model,
                          int64_t H, GateKind kind, hipStream_t s) {
  return kind == GateKind::kSigmoid
             ? go_gate<true, true>(x, x_bf16, w_f, b_f, dout, dz, B, L, d_model, H, s)
             : go_gate<true, false>(x, x_bf16, w_f, b_f, dout, dz, B, L, d_model, H, s);
}

}  // namespace fox
