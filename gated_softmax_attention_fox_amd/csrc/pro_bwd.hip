// pro_bwd.hip — backward of the Pro block's preprocessing: the forget gate's GEMV and the
// QK-norm (paper-graph-ui summary of arXiv 2503.02130, section 3.4, "Forget Gate Computation" and
// "The Pro Block Architecture", Steps 1-2 and 4). Both are HBM-bound; every reduction runs in a
// fixed order (per-chunk partials, then a second pass), so the results are deterministic.
//
// Gate: given dz[b, h, t] (from gate.hip's backward mode, which recomputes z from x; or, for the
// forget gate, from the forward's own output: d log sigma(z) / dz = 1 - sigma(z) = 1 - f, so
// dz = dlog_f (1 - f) = -dlog_f expm1(log f), which needs no pass over x),
//   dx[b, t, :] = sum_h dz[b, t, h] w_f[h, :]        (one pass over the tokens; on the matrix
//                                                    cores when H <= 16, d_model % 128 == 0)
//   dw_f[h, :]  = sum_{b,t} dz[b, t, h] x[b, t, :]   (partials per 256-token chunk, then a sum;
//                                                    on the matrix cores for bf16 x)
//   db_f[h]     = sum_{b,t} dz[b, t, h]
// QK-norm: with r = 1 / sqrt(mean x^2 + eps), xh = x r and g = dy w (w = 1 when absent),
//   dx = r (g - xh mean(g xh)),  dw = sum over rows of dy xh  (partials per workgroup, then a sum).
#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kChunk = 256;   // tokens per dw_f partial
constexpr int kHGroup = 16;   // heads per dw_f partial workgroup
constexpr int kRmsBlocks = 1024;

__device__ __forceinline__ float load_x(const void* x, bool bf16, size_t i) {
  return bf16 ? bf2f(static_cast<const bf16_t*>(x)[i]) : static_cast<const float*>(x)[i];
}

// dz[b, h, t] for the flattened token row = b L + t: stored, or formed from dlog_f and log f.
struct DzSrc {
  const float* dz;    // [B, H, L], or null
  const float* dout;  // dlog_f [B, H, L] (used with logf)
  const float* logf;  // the forward's log f [B, H, L]
  int64_t L;
  int H;
  __device__ __forceinline__ float operator()(int64_t row, int h) const {
    const int64_t b = row / L;
    const size_t i = (size_t)(b * H + h) * L + (row - b * L);
    return dz ? dz[i] : dout[i] * -expm1f(logf[i]);
  }
};

// dx[r, d .. d+7] for token r (one thread per 8 columns).
__global__ __launch_bounds__(256) void gate_dx_kernel(const DzSrc dz,
                                                      const float* __restrict__ w_f,
                                                      float* __restrict__ dx, int64_t rows, int dm,
                                                      int H) {
  const int groups = dm / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= rows * groups) return;
  const int64_t r = gid / groups;
  const int d = (int)(gid % groups) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int h = 0; h < H; ++h) {
    const float g = dz(r, h);
    const float4 w0 = *reinterpret_cast<const float4*>(w_f + (size_t)h * dm + d);
    const float4 w1 = *reinterpret_cast<const float4*>(w_f + (size_t)h * dm + d + 4);
    acc[0] = fmaf(g, w0.x, acc[0]); acc[1] = fmaf(g, w0.y, acc[1]);
    acc[2] = fmaf(g, w0.z, acc[2]); acc[3] = fmaf(g, w0.w, acc[3]);
    acc[4] = fmaf(g, w1.x, acc[4]); acc[5] = fmaf(g, w1.y, acc[5]);
    acc[6] = fmaf(g, w1.z, acc[6]); acc[7] = fmaf(g, w1.w, acc[7]);
  }
  *reinterpret_cast<float4*>(dx + r * dm + d) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(dx + r * dm + d + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// dx for up to 16 heads: a workgroup owns 16 tokens and thread c the columns 8c .. 8c + 7 of all
// of them, so its slice of w_f (16 heads x 8 columns) is read once and stays in registers.
__global__ __launch_bounds__(256) void gate_dx16_kernel(const DzSrc dz,
                                                        const float* __restrict__ w_f,
                                                        float* __restrict__ dx, int64_t rows,
                                                        int dm, int H) {
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  for (int grp = threadIdx.x; grp < dm / 8; grp += 256) {
    const int d = grp * 8;
    float w[16][8];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
      if (h < H) {
        a = *reinterpret_cast<const float4*>(w_f + (size_t)h * dm + d);
        c = *reinterpret_cast<const float4*>(w_f + (size_t)h * dm + d + 4);
      }
      w[h][0] = a.x; w[h][1] = a.y; w[h][2] = a.z; w[h][3] = a.w;
      w[h][4] = c.x; w[h][5] = c.y; w[h][6] = c.z; w[h][7] = c.w;
    }
    for (int i = 0; i < 16; ++i) {
      const int64_t r = r0 + i;
      if (r >= rows) break;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h < H) {
          const float g = dz(r, h);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(g, w[h][e], acc[e]);
        }
      }
      *reinterpret_cast<float4*>(dx + r * dm + d) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(dx + r * dm + d + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// Partial dw_f and db_f of one 256-token chunk, one 256-column slab and up to 16 heads: thread c
// owns column slab * 256 + c and walks the chunk's tokens (coalesced rows of x).
// dx on the matrix cores (d_model a multiple of 128, H <= 16): workgroup (token block, slab) owns
// 128 tokens x 128 columns, each wave 32 columns; the workgroup's dz goes through LDS first,
// already split into its bf16 parts. dx^T[32 columns x 32 tokens] is one
// v_mfma_f32_32x32x16_bf16 per operand pair, k = the (zero-padded) 16 heads: A = w_f^T (the
// wave's columns, loaded once), B = dz^T of 32 tokens. Both are split into three bf16 parts and
// the six products that reach fp32 accuracy are summed smallest first; the hi x hi product is
// exact, so the result matches an fp32 dot product of 16 terms to its rounding.
__global__ __launch_bounds__(256) void gate_dx_mfma_kernel(const DzSrc dz,
                                                           const float* __restrict__ w_f,
                                                           float* __restrict__ dx, int64_t rows,
                                                           int dm, int H) {
  constexpr int TB = 128;  // tokens per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hl = lane >> 5, l32 = lane & 31;
  const int64_t t_blk = (int64_t)blockIdx.x * TB;
  const int d0 = blockIdx.y * 128 + 32 * wave;
  auto split3 = [](const float (&v)[8], bf16x8& p0, bf16x8& p1, bf16x8& p2) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 a = (__bf16)v[e];
      const float r1 = v[e] - (float)a;
      const __bf16 b = (__bf16)r1;
      p0[e] = a;
      p1[e] = b;
      p2[e] = (__bf16)(r1 - (float)b);
    }
  };
  // The workgroup's dz as B operands, split once: thread (token tt, half hb) loads the 8 heads
  // 8 hb .. 8 hb + 7 of its token (coalesced over tokens) and stores their three bf16 parts in
  // operand order, so each wave's step reads one 16-byte chunk per part instead of splitting.
  __shared__ __attribute__((aligned(16))) bf16x8 dzp[3][TB / 32][2][32];
  {
    const int tt = threadIdx.x % TB, hb = threadIdx.x / TB;  // 256 threads: 128 tokens x 2 halves
    const int64_t t = t_blk + tt;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = 8 * hb + e;
      v[e] = (h < H && t < rows) ? dz(t, h) : 0.f;
    }
    bf16x8 p0, p1, p2;
    split3(v, p0, p1, p2);
    dzp[0][tt >> 5][hb][tt & 31] = p0;
    dzp[1][tt >> 5][hb][tt & 31] = p1;
    dzp[2][tt >> 5][hb][tt & 31] = p2;
  }
  // A[m = column d0 + l32][k = head 8 hl + e]
  bf16x8 wa0, wa1, wa2;
  {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = 8 * hl + e;
      v[e] = h < H ? w_f[(size_t)h * dm + d0 + l32] : 0.f;
    }
    split3(v, wa0, wa1, wa2);
  }
  __syncthreads();
  for (int tb = 0; tb < TB; tb += 32) {
    const int64_t t = t_blk + tb + l32;  // B[k = head 8 hl + e][n = token t]
    const bf16x8 b0 = dzp[0][tb >> 5][hl][l32], b1 = dzp[1][tb >> 5][hl][l32],
                 b2 = dzp[2][tb >> 5][hl][l32];
    f32x16 acc = zero16();
    acc = mfma32(wa2, b0, acc);
    acc = mfma32(wa1, b1, acc);
    acc = mfma32(wa0, b2, acc);
    acc = mfma32(wa1, b0, acc);
    acc = mfma32(wa0, b1, acc);
    acc = mfma32(wa0, b0, acc);
    if (t < rows) {  // C[m = 8 i + 4 hl + j][n = l32] in slot 4 i + j: 4 consecutive columns
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(dx + t * dm + d0 + 8 * i + 4 * hl) =
            make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    }
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void gate_dw_partial_kernel(const void* __restrict__ x,
                                                              const DzSrc dz,
                                                              float* __restrict__ part,
                                                              float* __restrict__ part_db,
                                                              int64_t rows, int dm, int H) {
  __shared__ float dzs[kChunk][kHGroup + 1];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, slab = blockIdx.y, h0 = blockIdx.z * kHGroup;
  const int nh = H - h0 < kHGroup ? H - h0 : kHGroup;
  const int64_t r0 = (int64_t)chunk * kChunk;
  const int n = rows - r0 < kChunk ? (int)(rows - r0) : kChunk;
  for (int i = tid; i < kChunk * kHGroup; i += 256) {  // token fastest: coalesced per head
    const int r = i % kChunk, h = i / kChunk;
    dzs[r][h] = (r < n && h < nh) ? dz(r0 + r, h0 + h) : 0.f;
  }
  __syncthreads();
  const int d = slab * 256 + tid;
  if (d < dm) {
    float acc[kHGroup];
#pragma unroll
    for (int h = 0; h < kHGroup; ++h) acc[h] = 0.f;
    for (int r = 0; r < n; ++r) {
      const float xv = load_x(x, kBf16, (size_t)(r0 + r) * dm + d);
#pragma unroll
      for (int h = 0; h < kHGroup; ++h) acc[h] = fmaf(dzs[r][h], xv, acc[h]);
    }
    for (int h = 0; h < nh; ++h) part[((size_t)chunk * H + h0 + h) * dm + d] = acc[h];
  }
  if (slab == 0 && tid < nh) {
    double sum = 0.0;  // fp64, as in the matrix-core kernel
    for (int r = 0; r < n; ++r) sum += (double)dzs[r][tid];
    part_db[(size_t)chunk * H + h0 + tid] = (float)sum;
  }
}

// dw_f[h, d] and db_f[h] as the chunk partials summed in chunk order.
// dw_f partials on the matrix cores (bf16 x, d_model a multiple of 128; heads in groups of 32).
// Workgroup (chunk, slab, head group) accumulates dw_f^T[128 columns x 32 heads] over the chunk's
// kChunk tokens, staging 64 tokens of x and dz at a time in LDS (the next stage's x is already in
// flight in registers while the current one is multiplied). Each wave owns 32 columns:
// v_mfma_f32_32x32x16_bf16 with A = x^T from transposed reads of the swizzled x tile (k = token)
// and B = dz of the same 16 tokens for head n = lane % 32, split into three bf16 parts
// (hi + mid + lo carries all 24 bits of the fp32 value), so every product is exact and only the
// fp32 accumulation rounds. The partials have gate_dw_partial_kernel's layout.
__global__ __launch_bounds__(256) void gate_dw_mfma_kernel(const bf16_t* __restrict__ x,
                                                           const DzSrc dz,
                                                           float* __restrict__ part,
                                                           float* __restrict__ part_db,
                                                           int64_t rows, int dm, int H) {
  constexpr int TS = 64;  // tokens per LDS stage
  constexpr int HG = 32;  // heads per workgroup (the MFMA's n dimension)
  constexpr int XV = TS * 16 / 256;  // 16-byte pieces of x per thread and stage
  constexpr int DV = TS * HG / 256;  // dz values per thread and stage
  __shared__ __attribute__((aligned(16))) bf16_t xs[TS * 128];
  // dz of the stage, split once into three bf16 parts (hi + mid + lo carries all 24 bits) and
  // stored in B-operand order: part p, 16-token block ks, half hl, head n -> the 8 bf16 of B's k
  // slots, so the product loop reads each part with one 16-byte read.
  __shared__ __attribute__((aligned(16))) bf16_t dzp[3][TS / 16][2][HG][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5;
  const int chunk = blockIdx.x, slab = blockIdx.y, h0 = blockIdx.z * HG;
  const int nh = H - h0 < HG ? H - h0 : HG;
  const int64_t r0 = (int64_t)chunk * kChunk;
  const int n = rows - r0 < kChunk ? (int)(rows - r0) : kChunk;
  const int n_st = (n + TS - 1) / TS;
  const uint32_t xb = lds_addr(xs);
  const uint32_t a0 = xb + col8_off<128>(lane, 32 * wave, 0);
  const uint32_t a1 = xb + col8_off<128>(lane, 32 * wave, 1);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  u32x4 xv[XV];
  float dv[DV];
  auto load_stage = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < XV; ++q) {
      const int i = tid + 256 * q, row = i >> 4, c = i & 15;
      const int tok = st * TS + row;
      const bool ok = tok < n;  // rows past the chunk read token r0 and are zeroed
      const u32x4 v = *reinterpret_cast<const u32x4*>(x + (size_t)(ok ? r0 + tok : r0) * dm +
                                                      slab * 128 + c * 8);
      xv[q] = ok ? v : zero4;
    }
#pragma unroll
    for (int q = 0; q < DV; ++q) {  // token fastest: coalesced per head
      const int i = tid + 256 * q, row = i % TS, hh = i / TS;
      const int tok = st * TS + row;
      dv[q] = (tok < n && hh < nh) ? dz(r0 + tok, h0 + hh) : 0.f;
    }
  };

  f32x16 acc = zero16();
  // db partial: thread tid holds dz of token tid % TS and heads tid / TS + 4 q (q < DV) in every
  // stage, so each wave sums its lanes' values over the stages and reduces across lanes at the
  // end (a fixed butterfly order). The sums run in fp64: db_f is a sum over every token whose
  // terms may cancel, and an fp32 running sum left it off by 1.4-1.9e-5 relative where it did.
  double dba[DV];
#pragma unroll
  for (int q = 0; q < DV; ++q) dba[q] = 0.0;
  load_stage(0);
  for (int st = 0; st < n_st; ++st) {
#pragma unroll
    for (int q = 0; q < XV; ++q) {
      const int i = tid + 256 * q;
      lds_store8<128>(xs, i >> 4, (i & 15) * 8, xv[q]);
    }
#pragma unroll
    for (int q = 0; q < DV; ++q) {
      const int i = tid + 256 * q, row = i % TS, hh = i / TS;
      // token row of the stage sits in k slot e of half hb of block ks (the slot order of the
      // transposed x reads: tokens 16 ks + 4 hb + 0..3 in slots 0..3, 16 ks + 8 + 4 hb + 0..3 in 4..7)
      const int ks = row >> 4, tin = row & 15, hb = (tin >> 2) & 1, e = (tin & 3) + ((tin >> 3) << 2);
      const float v = dv[q];
      const __bf16 p1 = (__bf16)v;
      const float r1 = v - (float)p1;
      const __bf16 p2 = (__bf16)r1;
      dzp[0][ks][hb][hh][e] = __builtin_bit_cast(bf16_t, p1);
      dzp[1][ks][hb][hh][e] = __builtin_bit_cast(bf16_t, p2);
      dzp[2][ks][hb][hh][e] = __builtin_bit_cast(bf16_t, (__bf16)(r1 - (float)p2));
      dba[q] += (double)v;
    }
    __syncthreads();
    if (st + 1 < n_st) load_stage(st + 1);
#pragma unroll
    for (int ks = 0; ks < TS / 16; ++ks) {
      const uint32_t ro = (uint32_t)ks * 16 * 128 * 2;  // 16-row blocks keep the swizzle key
      const bf16x8 a = lds_tr8(a0 + ro, a1 + ro);
      const int hd = lane & 31;
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&dzp[0][ks][hl][hd][0]);
      const bf16x8 bm = *reinterpret_cast<const bf16x8*>(&dzp[1][ks][hl][hd][0]);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&dzp[2][ks][hl][hd][0]);
      acc = mfma32(a, bh, acc);
      acc = mfma32(a, bm, acc);
      acc = mfma32(a, bl, acc);
    }
    __syncthreads();
  }
  const int head = lane & 31;  // C[m = 8 i + 4 hl + j][n = head] sits in slot 4 i + j
  if (head < nh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = slab * 128 + 32 * wave + 8 * i + 4 * hl;
      *reinterpret_cast<float4*>(part + ((size_t)chunk * H + h0 + head) * dm + d) =
          make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    }
  }
  if (slab == 0) {
    static_assert(TS == 64, "one wave holds one head's tokens of a stage");
#pragma unroll
    for (int q = 0; q < DV; ++q) {
      double v = dba[q];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      const int hh = wave + 4 * q;  // (tid + 256 q) / TS
      if (lane == 0 && hh < nh) part_db[(size_t)chunk * H + h0 + hh] = (float)v;
    }
  }
}

// dw_f[h, d] and db_f[h]: the chunk partials summed in a fixed order, in fp64. A workgroup owns
// 64 consecutive entries of the flattened [H, d_model] array; wave w sums the chunks
// [w n / 4, (w + 1) n / 4) of every entry (16 loads in flight), and the four wave sums are added
// in wave order. The last workgroup sums the db_f partials the same way.
__global__ __launch_bounds__(256) void gate_dw_reduce_kernel(const float* __restrict__ part,
                                                             const float* __restrict__ part_db,
                                                             float* __restrict__ dw_f,
                                                             float* __restrict__ db_f, int n_chunk,
                                                             int dm, int H) {
  __shared__ double red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_w = (int64_t)H * dm;
  const bool db_blk = blockIdx.x == gridDim.x - 1;
  const int64_t e = db_blk ? lane : (int64_t)blockIdx.x * 64 + lane;
  const int64_t n_e = db_blk ? H : n_w;
  const float* src = db_blk ? part_db : part;
  const int64_t stride = db_blk ? H : n_w;
  const int c0 = (int)((int64_t)n_chunk * wave / 4), c1 = (int)((int64_t)n_chunk * (wave + 1) / 4);
  double s = 0.0;
  if (e < n_e) {
#pragma unroll 16
    for (int c = c0; c < c1; ++c) s += (double)src[(size_t)c * stride + e];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && e < n_e) {
    const float t = (float)(((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
    if (!db_blk) dw_f[e] = t;
    else if (db_f) db_f[e] = t;
  }
}

// QK-norm backward, D / 8 lanes per row, grid-stride over rows; with kDw each workgroup also sums
// dy * xh over its rows into one partial row of length D.
template <int D, bool kBf16, bool kDw>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ dy,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ dx,
                                                          float* __restrict__ part, int64_t rows,
                                                          float eps) {
  constexpr int G = D / 8, RPB = 256 / G;
  __shared__ float red[kDw ? RPB : 1][kDw ? D : 1];
  const int tid = threadIdx.x, sub = tid / G, pc = (tid % G) * 8;
  float wv[8], dwp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wv[e] = w ? w[pc + e] : 1.0f;
    dwp[e] = 0.f;
  }
  for (int64_t row = (int64_t)blockIdx.x * RPB + sub; row < rows; row += (int64_t)gridDim.x * RPB) {
    // the G lanes of a row are consecutive in one wave and share `row`, so they stay together
    const size_t off = (size_t)row * D + pc;
    float v[8], g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = load_x(x, kBf16, off + e);
    const float4 d0 = *reinterpret_cast<const float4*>(dy + off);
    const float4 d1 = *reinterpret_cast<const float4*>(dy + off + 4);
    const float dyv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
    for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    float sg = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] *= r;  // xh
      g[e] = dyv[e] * wv[e];
      sg = fmaf(g[e], v[e], sg);
    }
#pragma unroll
    for (int m = 1; m < G; m <<= 1) sg += __shfl_xor(sg, m, 64);
    const float mean = sg / (float)D;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = r * (g[e] - v[e] * mean);
      if (kDw) dwp[e] = fmaf(dyv[e], v[e], dwp[e]);
    }
    *reinterpret_cast<float4*>(dx + off) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dx + off + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
  if constexpr (kDw) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[sub][pc + e] = dwp[e];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
      for (int i = 0; i < RPB; ++i) s += red[i][tid];
      part[(size_t)blockIdx.x * D + tid] = s;
    }
  }
}

__global__ __launch_bounds__(128) void rmsnorm_dw_reduce_kernel(const float* __restrict__ part,
                                                                float* __restrict__ dw, int nblk,
                                                                int D) {
  const int d = threadIdx.x;
  if (d >= D) return;
  float s = 0.f;
  for (int b = 0; b < nblk; ++b) s += part[(size_t)b * D + d];
  dw[d] = s;
}

size_t granule(size_t floats) { return (floats + 63) / 64 * 64; }  // 256-byte granules

template <int D, bool kBf16>
hipError_t go_rms_bwd(const void* x, const float* dy, const float* w, float* dx, float* dw,
                      float* part, int64_t rows, float eps, hipStream_t s) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t need = (rows + RPB - 1) / RPB;
  if (dw) {
    const int nblk = (int)(need < kRmsBlocks ? need : kRmsBlocks);
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<D, kBf16, true>), dim3((unsigned)nblk), dim3(256), 0, s,
                       x, dy, w, dx, part, rows, eps);
    hipLaunchKernelGGL(rmsnorm_dw_reduce_kernel, dim3(1), dim3(128), 0, s, part, dw, nblk, D);
  } else {
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<D, kBf16, false>), dim3((unsigned)need), dim3(256), 0,
                       s, x, dy, w, dx, nullptr, rows, eps);
  }
  return hipGetLastError();
}

}  // namespace

size_t gate_bwd_workspace_bytes(int64_t B, int64_t L, int64_t d_model, int64_t H) {
  const int64_t rows = B * L;
  const int64_t n_chunk = (rows + kChunk - 1) / kChunk;
  return 4 * (granule((size_t)(rows * H)) + granule((size_t)(n_chunk * H * d_model)) +
              granule((size_t)(n_chunk * H)));
}

hipError_t launch_gate_bwd(const void* x, bool x_bf16, const float* w_f, const float* b_f,
                           const float* dout, const float* log_f, float* dx, float* dw_f,
                           float* db_f, void* ws, int64_t B, int64_t L, int64_t d_model, int64_t H,
                           GateKind kind, hipStream_t s) {
  const int64_t rows = B * L;
  const int n_chunk = (int)((rows + kChunk - 1) / kChunk);
  float* dzbuf = static_cast<float*>(ws);
  float* part = dzbuf + granule((size_t)(rows * H));
  float* part_db = part + granule((size_t)((int64_t)n_chunk * H * d_model));
  DzSrc dz{nullptr, dout, log_f, L, (int)H};
  if (kind != GateKind::kLogSigmoid || log_f == nullptr) {  // recompute z from x
    hipError_t e = launch_gate_dz(x, x_bf16, w_f, b_f, dout, dzbuf, B, L, d_model, H, kind, s);
    if (e != hipSuccess) return e;
    dz.dz = dzbuf;
  }
  if (H <= 16 && d_model % 128 == 0) {
    hipLaunchKernelGGL(gate_dx_mfma_kernel, dim3((unsigned)((rows + 127) / 128), (unsigned)(d_model / 128)),
                       dim3(256), 0, s, dz, w_f, dx, rows, (int)d_model, (int)H);
  } else if (H <= 16) {
    hipLaunchKernelGGL(gate_dx16_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, dz,
                       w_f, dx, rows, (int)d_model, (int)H);
  } else {
    const int64_t dx_threads = rows * (d_model / 8);
    hipLaunchKernelGGL(gate_dx_kernel, dim3((unsigned)((dx_threads + 255) / 256)), dim3(256), 0,
                       s, dz, w_f, dx, rows, (int)d_model, (int)H);
  }
  const dim3 pg((unsigned)n_chunk, (unsigned)((d_model + 255) / 256),
                (unsigned)((H + kHGroup - 1) / kHGroup));
  if (x_bf16 && d_model % 128 == 0)
    hipLaunchKernelGGL(gate_dw_mfma_kernel,
                       dim3((unsigned)n_chunk, (unsigned)(d_model / 128), (unsigned)((H + 31) / 32)),
                       dim3(256), 0, s, static_cast<const bf16_t*>(x), dz, part, part_db, rows,
                       (int)d_model, (int)H);
  else if (x_bf16)
    hipLaunchKernelGGL((gate_dw_partial_kernel<true>), pg, dim3(256), 0, s, x, dz, part, part_db,
                       rows, (int)d_model, (int)H);
  else
    hipLaunchKernelGGL((gate_dw_partial_kernel<false>), pg, dim3(256), 0, s, x, dz, part, part_db,
                       rows, (int)d_model, (int)H);
  const int64_t n_w = H * d_model;
  hipLaunchKernelGGL(gate_dw_reduce_kernel, dim3((unsigned)((n_w + 63) / 64 + 1)), dim3(256), 0, s,
                     part, part_db, dw_f, db_f, n_chunk, (int)d_model, (int)H);
  return hipGetLastError();
}

size_t rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t D) {
  (void)rows;
  return 4 * granule((size_t)kRmsBlocks * (size_t)D);
}

hipError_t launch_rmsnorm_bwd(const void* x, bool bf16, const float* dy, const float* w, float* dx,
                              float* dw, void* ws, int64_t rows, int64_t D, float eps,
                              hipStream_t s) {
  float* part = static_cast<float*>(ws);
  if (D == 64)
    return bf16 ? go_rms_bwd<64, true>(x, dy, w, dx, dw, part, rows, eps, s)
                : go_rms_bwd<64, false>(x, dy, w, dx, dw, part, rows, eps, s);
  return bf16 ? go_rms_bwd<128, true>(x, dy, w, dx, dw, part, rows, eps, s)
              : go_rms_bwd<128, false>(x, dy, w, dx, dw, part, rows, eps, s);
}

}  // namespace fox
