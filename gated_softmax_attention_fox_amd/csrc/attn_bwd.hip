// attn_bwd.hip — Forgetting Attention backward on gfx950 (bf16 inputs, fp32 gradients).
//
// The pages' backward (paper-graph-ui summary of arXiv 2503.02130, section 3.4, "Hardware-Aware
// Implementation (Modified FlashAttention)", the backward pass; paperlayer.ai summary, section E)
// is the FlashAttention-2 backward with the same bias added when P is recomputed from the saved
// log-sum-exp, plus the gradient of c: every dS_ij adds to dc_i and subtracts from dc_j; the two
// partial vectors dc^q and dc^k are summed and a reverse cumulative sum gives d log f. The pages
// note the work may be split over two kernels; here it is split so that no output needs atomics:
//
//   1. delta_kernel : Delta_i = dO_i . O_i from the fp32 forward output. Given O instead of
//                     Delta, dq_pipe_kernel forms the same values (same bits) in its prologue,
//                     which saves the launch and a second read of dO.
//   2. dq_pipe_kernel  : query-stationary. A workgroup owns 256 queries (32 per wave) and walks
//                        the key tiles from its diagonal backwards: S^T = K Q^T, P,
//                        dP^T = V dO^T, dS = P (dP - Delta_i), dQ^T += K^T dS^T. It also sums P
//                        and dS along each row and replaces Delta_i by the value that makes the
//                        row of dS sum to zero under this P and dP; dc^q_i is that row sum.
//   3. dkv_pipe_kernel : key-stationary. A workgroup owns 128 keys (32 per wave, held in
//                        registers as MFMA operands) and walks the query tiles from its diagonal
//                        to the end: S = Q K^T, P = exp(S*scale + c_i - c_j - LSE_i), dP = dO V^T,
//                        dS = P (dP - Delta'_i), dV^T += dO^T P, dK^T += Q^T dS,
//                        dc^k_j -= sum_i dS_ij.
//   4. reverse scan : d log f_l = sum_{t>=l} (dc^q_t + dc^k_t), fp64 accumulation.
//
// d log f_l telescopes to the sum of dS over rows >= l and columns < l, so the row and column
// sums must come from one consistent dS: both are taken in fp32 before dS is rounded to bf16 for
// the MFMA, and both kernels use the refined row term (a Delta from the forward's O, whose P
// was rounded to bf16, leaves a per-row residual that the reverse scan would accumulate).
// Every output element is written by exactly one lane, so the backward is deterministic. The C-tile / operand conventions are those of
// fox_device.h: in dkv_pipe_kernel the C tiles are [query x key] with one key per lane, so P
// and dS are B operands of products that contract over queries; in dq_pipe_kernel they are
// [key x query].
#include <type_traits>
#include <utility>

#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const bf16_t* __restrict__ dO,
                                                    const float* __restrict__ O,
                                                    float* __restrict__ delta, int64_t rows) {
  constexpr int G = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / G;
  const int part = (int)(gid % G);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + part * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(dO + off);
    const float4 a = *reinterpret_cast<const float4*>(O + off);
    const float4 b = *reinterpret_cast<const float4*>(O + off + 4);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
    const float o8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(w4[e] << 16), o8[2 * e], acc);
      acc = fmaf(__uint_as_float(w4[e] & 0xffff0000u), o8[2 * e + 1], acc);
    }
  }
#pragma unroll
  for (int m = 1; m < G; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && part == 0) delta[row] = acc;
}

// Instruction order of one software-pipelined step (scheduler groups, filled in this order): kD0
// LDS reads, then each of the step's kNM matrix products followed by kDs LDS reads (for the
// first kNd products) and kV vector instructions.
template <int I, int kDs, int kV, int kNd>
__device__ __forceinline__ void interleave_bwd_one() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (I < kNd) __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
}
template <int kD0, int kDs, int kV, int kNd, int... I>
__device__ __forceinline__ void interleave_bwd_all(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, kD0, 0);
  (interleave_bwd_one<I, kDs, kV, kNd>(), ...);
}
template <int kD0, int kDs, int kV, int kNd, int kNM>
__device__ __forceinline__ void interleave_bwd() {
  interleave_bwd_all<kD0, kDs, kV, kNd>(std::make_integer_sequence<int, kNM>{});
}
// A block of kNM matrix products fed by one LDS read each: kD0 reads first, then one read after
// each product, so that every operand is read kD0 products ahead.
template <int I>
__device__ __forceinline__ void readahead_one() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}
template <int kD0, int... I>
__device__ __forceinline__ void readahead_all(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, kD0, 0);
  (readahead_one<I>(), ...);
}
template <int kD0, int kNM>
__device__ __forceinline__ void readahead() {
  readahead_all<kD0>(std::make_integer_sequence<int, kNM - kD0>{});
}

// Key-stationary step with the forward kernel's memory pipeline. 4 waves, one per SIMD, 32 keys
// per wave (K^T and V^T held as MFMA operands, dK^T and dV^T accumulated in registers), 128 keys
// per workgroup. Queries are walked upwards from the diagonal in 64-query tiles (tile t =
// queries k0 + 64 t .., two 32-query sub-tiles). Q and dO of tile t and its raw c, LSE and
// Delta values sit in LDS ring slot t % 4, the converted row terms m_i =
// (LSE_i - (c_i - c_ref)) log2 e and Delta_i in slot t % 2; iteration t reads tile t, starts the
// untracked copies of Q(t + 2), dO(t + 2) and the raw row values of tile t + 3, converts those of
// tile t + 1, and its barrier waits only for the copies started one iteration earlier. Past the
// sequence end the copies read zeros and m_i is +inf, so P is zero there. Per 32-query sub-tile
// a wave computes S = Q K^T and dP = dO V^T (one key per lane), P = exp2(scale log2(e) s -
// (k_j + m_i)) with k_j = (c_j - c_ref) log2 e (the two terms added first), dS = P (dP - Delta_i),
// dc^k_j -= sum_i dS_ij from the fp32 dS, and dV^T += dO^T P, dK^T += Q^T dS with the transposes
// read from the row-major tiles. Tiles 0 and 1 hold every wave's diagonal and evaluate the
// causal mask; from tile 2 on the loop is unrolled over four tiles for compile-time slots.
// Occupancy: at D = 128 a wave needs about 400 registers, so each SIMD runs one. At D = 64 the
// kernel fits in 256 (128 VGPRs and 128 AGPRs, no spill) and its LDS in 69 KB, so two
// workgroups share a compute unit and each SIMD interleaves two waves.
template <int D, typename CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1))) void dkv_pipe_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const CT* __restrict__ C, const float* __restrict__ LSE,
    const float* __restrict__ Delta, float* __restrict__ dK, float* __restrict__ dV,
    float* __restrict__ dck_out, const int32_t* __restrict__ kv_tiles,
    const int32_t* __restrict__ kv_order, int L, int BH, float sl2e, float scale) {
  constexpr int NW = 4, BK = NW * 32, BQ = 64;
  constexpr int TILE = BQ * D;
  constexpr int CPR = D / 8;
  constexpr int BLK = TILE * 2 / 1024 / NW;  // 1 KiB copies per wave per tensor and tile
  constexpr int RW = BQ / NW;                // row values each wave copies per array and tile
  constexpr int NCOPY = 2 * BLK + 3;
  static_assert(BLK >= 1, "tile must split evenly over the waves");
  constexpr uint32_t TB = TILE * 2;
  constexpr uint32_t CS = sizeof(CT);        // bytes of one raw c value (fp32 or fp64)
  constexpr uint32_t RS = BQ * (CS + 8);     // raw c, LSE and Delta of one tile (one ring slot)
  constexpr uint32_t Q_OFF = 0, O_OFF = 4 * TB, R_OFF = 8 * TB, M_OFF = 8 * TB + 4 * RS;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[8 * TB + 4 * RS + 2 * 2 * BQ * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  // Key tile 0 sees every query tile and is issued first, or a skip plan's order of decreasing
  // work.
  const int bid = blockIdx.x;
  const int n_kb = (L + BK - 1) / BK;
  int bh, kt;
  if (kv_order) {
    const int item = kv_order[bid];
    bh = item / n_kb;
    kt = item % n_kb;
  } else {  // key blocks from the first, each head kept to one XCD where possible
    xcd_item(bid, BH, bh, kt);
  }
  const int k0 = kt * BK;
  const size_t base = (size_t)bh * L * D;
  Q += base;
  K += base;
  V += base;
  dO += base;
  C += (size_t)bh * L;
  LSE += (size_t)bh * L;
  Delta += (size_t)bh * L;
  const CT c_ref = C[k0];
  const int kw = k0 + wave * 32;
  const int kj = kw + l32;
  const bool kok = kj < L;
  const bool active = kw < L;
  // Query tiles walked from the diagonal: to the sequence end, or to the last tile whose weights
  // a skip plan could not rule out (the later ones would add exact zeros).
  const int n_t = kv_tiles ? kv_tiles[(size_t)bh * n_kb + kt] : (L - k0 + BQ - 1) / BQ;
  const int j0 = wave;                     // the wave's diagonal sub-tile (queries kw .. kw + 31)
  const i32x4 q_rs = buffer_words(Q, (uint32_t)L * (uint32_t)(D * 2));
  const i32x4 o_rs = buffer_words(dO, (uint32_t)L * (uint32_t)(D * 2));
  const i32x4 c_rs = buffer_words(C, (uint32_t)L * CS);
  const i32x4 l_rs = buffer_words(LSE, (uint32_t)L * 4u);
  const i32x4 d_rs = buffer_words(Delta, (uint32_t)L * 4u);
  const uint32_t sbase = lds_addr(smem);

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (kok) {
      kf[c] = ld8(K + (size_t)kj * D + 16 * c + 8 * h);
      vf[c] = ld8(V + (size_t)kj * D + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[c][e] = (__bf16)0.f;
        vf[c][e] = (__bf16)0.f;
      }
    }
    // Only the matrix cores read K^T and V^T: AGPRs, which leaves the vector registers free.
    pin_agpr(kf[c]);
    pin_agpr(vf[c]);
  }
  const float kterm = kok ? cbias(C[kj], c_ref) : 0.f;
  f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    dvacc[d] = zero16();
    dkacc[d] = zero16();
  }
  float dck = 0.f;

  auto copy_tile = [&](const i32x4& rs, uint32_t region, int t, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const int blk = wave * BLK + k;
      const int r = blk * (512 / D) + lane / CPR;
      const int lc = (lane % CPR) ^ swz_key<D>(r);
      const uint32_t voff = (uint32_t)((k0 + t * BQ + r) * D + lc * 8) * 2;
      copy16_to_lds(sbase + region + slot * TB + blk * 1024, voff, rs);
    }
  };
  auto copy_rows = [&](int t, int slot) __attribute__((always_inline)) {  // raw c, LSE, Delta
    const uint32_t row0 = (uint32_t)(k0 + t * BQ + wave * RW);
    const uint32_t dst = sbase + R_OFF + slot * RS;
    if (lane < RW * (int)CS / 4)  // c: one 4-byte word per lane
      copy4_to_lds(dst + wave * RW * CS, row0 * CS + lane * 4, c_rs);
    if (lane < RW) {
      copy4_to_lds(dst + BQ * CS + wave * RW * 4, (row0 + lane) * 4, l_rs);
      copy4_to_lds(dst + BQ * (CS + 4) + wave * RW * 4, (row0 + lane) * 4, d_rs);
    }
  };
  auto start_copies = [&](int t, int sqo, int sr) __attribute__((always_inline)) {
    if (t + 2 < n_t) {
      copy_tile(q_rs, Q_OFF, t + 2, sqo);
      copy_tile(o_rs, O_OFF, t + 2, sqo);
    }
    if (t + 3 < n_t) copy_rows(t + 3, sr);
  };
  // Row terms of tile t + 1 from its raw values (wave 0, one query per lane).
  auto convert_rows = [&](int t, int sr, int sm) __attribute__((always_inline)) {
    if (wave == 0 && t + 1 < n_t) {
      typedef __attribute__((address_space(3))) float lds_f;
      typedef __attribute__((address_space(3))) CT lds_c;
      const uint32_t src = sbase + R_OFF + sr * RS;
      const CT ci = *(const lds_c*)(uintptr_t)(src + lane * CS);
      const float li = *(const lds_f*)(uintptr_t)(src + BQ * CS + lane * 4);
      const float di = *(const lds_f*)(uintptr_t)(src + BQ * (CS + 4) + lane * 4);
      const bool ok = k0 + (t + 1) * BQ + lane < L;
      const uint32_t dst = sbase + M_OFF + sm * 2 * BQ * 4 + lane * 4;
      *(lds_f*)(uintptr_t)dst = ok ? (li - cdiff(ci, c_ref)) * kLog2e : INFINITY;
      *(lds_f*)(uintptr_t)(dst + BQ * 4) = ok ? di : 0.f;
    }
  };

  uint32_t qp[D / 16], op[D / 16], qtp[D / 32][2], otp[D / 32][2];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    qp[c] = opaque(sbase + Q_OFF + row8_off<D>(lane, 16 * c + 8 * h));
    op[c] = opaque(sbase + O_OFF + row8_off<D>(lane, 16 * c + 8 * h));
  }
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    qtp[d][0] = opaque(sbase + Q_OFF + col8_off<D>(lane, d * 32, 0));
    qtp[d][1] = opaque(sbase + Q_OFF + col8_off<D>(lane, d * 32, 1));
    otp[d][0] = opaque(sbase + O_OFF + col8_off<D>(lane, d * 32, 0));
    otp[d][1] = opaque(sbase + O_OFF + col8_off<D>(lane, d * 32, 1));
  }
  const uint32_t mp = opaque(sbase + M_OFF + 16 * h);

  // The three parts of one 32-query sub-tile (Q / dO rows at byte offset ro of a slot, row terms
  // at mo, first query q0s, masking only with kMask):
  //   sd   : S = Q K^T and dP = dO V^T (one key per lane);
  //   grad : P = exp2(scale log2(e) s - (k_j + m_i)), dS = P (dP - Delta_i), dc^k_j -= sum_i dS_ij,
  //          and P, dS as bf16 B operands;
  //   dvdk : dV^T += dO^T P, dK^T += Q^T dS.
  auto sd = [&](f32x16& s, f32x16& dp, uint32_t ro) __attribute__((always_inline)) {
    s = zero16();
    dp = zero16();
#pragma unroll
    for (int c = 0; c < D / 16; ++c) s = mfma32(lds_ld16(qp[c] + ro), kf[c], s);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) dp = mfma32(lds_ld16(op[c] + ro), vf[c], dp);
    pin_vgpr(s);
    pin_vgpr(dp);
  };
  auto rows = [&](f32x4 (&m4)[4], f32x4 (&d4)[4], uint32_t mo) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m4[i] = lds_ldf4(mp + mo + 32 * i);
      d4[i] = lds_ldf4(mp + mo + BQ * 4 + 32 * i);
    }
  };
  auto grad = [&](f32x16& s, f32x16& dp, const f32x4 (&m4)[4], const f32x4 (&d4)[4], int q0s,
                  auto mask_tag, bf16x8 (&pb)[2], bf16x8 (&sb)[2]) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = fmaf(s[4 * i + e], sl2e, -(kterm + m4[i][e]));
        if constexpr (kMask) {
          if (kj > q0s + 8 * i + 4 * h + e) x = -INFINITY;
        }
        const float p = __builtin_amdgcn_exp2f(x);
        const float ds = p * (dp[4 * i + e] - d4[i][e]);
        dck -= ds;
        s[4 * i + e] = p;
        dp[4 * i + e] = ds;
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pb[t] = pack_c_half(s, t);
      sb[t] = pack_c_half(dp, t);
    }
  };
  auto grad_h = [&](f32x16& s, f32x16& dp, const f32x4 (&m4)[4], const f32x4 (&d4)[4], int hf,
                    bf16x8 (&pb)[2], bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hf + ii;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = fmaf(s[4 * i + e], sl2e, -(kterm + m4[i][e]));
        const float p = __builtin_amdgcn_exp2f(x);
        const float ds = p * (dp[4 * i + e] - d4[i][e]);
        dck -= ds;
        s[4 * i + e] = p;
        dp[4 * i + e] = ds;
      }
    }
    pb[hf] = pack_c_half(s, hf);
    sb[hf] = pack_c_half(dp, hf);
  };
  auto dvdk = [&](uint32_t ro, const bf16x8 (&pb)[2], const bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        dvacc[d] = mfma32(lds_tr8(otp[d][0] + ro + t * 16 * D * 2, otp[d][1] + ro + t * 16 * D * 2),
                          pb[t], dvacc[d]);
        dkacc[d] = mfma32(lds_tr8(qtp[d][0] + ro + t * 16 * D * 2, qtp[d][1] + ro + t * 16 * D * 2),
                          sb[t], dkacc[d]);
      }
    }
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
      pin_agpr(dvacc[d]);
      pin_agpr(dkacc[d]);
    }
  };
  auto sub_tile = [&](uint32_t ro, uint32_t mo, int q0s, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    f32x16 s, dp;
    bf16x8 pb[2], sb[2];
    f32x4 m4[4], d4[4];
    rows(m4, d4, mo);
    sd(s, dp, ro);
    readahead<8, 16>();
    __builtin_amdgcn_sched_barrier(0);
    grad(s, dp, m4, d4, q0s, mask_tag, pb, sb);
    dvdk(ro, pb, sb);
    if constexpr (kMask) {
      // The diagonal tiles hold the queries that give a key its largest weights whenever a few
      // keys dominate their rows, and there P and dS are large: their bf16 rounding alone can
      // move dV and dK by ~2^-9 of their size. These products therefore also take the rounding
      // remainders P - bf16(P) and dS - bf16(dS), so they see both to ~2^-17.
      bf16x8 pl[2], sl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pl[t][e] = (__bf16)(s[8 * t + e] - (float)pb[t][e]);
          sl[t][e] = (__bf16)(dp[8 * t + e] - (float)sb[t][e]);
        }
      }
      dvdk(ro, pl, sl);
    }
  };

  // prologue: copies of Q(0), dO(0), Q(1), dO(1) and the raw rows of tiles 0..2; convert tile 0
  copy_tile(q_rs, Q_OFF, 0, 0);
  copy_tile(o_rs, O_OFF, 0, 0);
  copy_rows(0, 0);
  if (1 < n_t) {
    copy_tile(q_rs, Q_OFF, 1, 1);
    copy_tile(o_rs, O_OFF, 1, 1);
    copy_rows(1, 1);
  }
  if (2 < n_t) copy_rows(2, 2);
  bar_vm<0>();
  convert_rows(-1, 0, 0);
  bar_vm<0>();

  auto generic_tile = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    start_copies(t, (t + 2) & 3, (t + 3) & 3);
    convert_rows(t, (t + 1) & 3, (t + 1) & 1);
    if (active) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int j = 2 * t + sub;
        const uint32_t ro = (uint32_t)(t & 3) * TB + (uint32_t)sub * 32 * D * 2;
        const uint32_t mo = (uint32_t)(t & 1) * 2 * BQ * 4 + (uint32_t)sub * 32 * 4;
        if (j >= j0) sub_tile(ro, mo, k0 + 32 * j, mask_tag);
      }
    }
    bar_vm<0>();
  };
  // Steady tile t (slot S = t % 4), software-pipelined so that the vector work of one sub-tile runs
  // under the matrix products of its neighbours: S, dP of sub-tile 2t under the second half of
  // the gradient arithmetic of 2t - 1; then (step A) the arithmetic of 2t under dV, dK of 2t - 1
  // (from pc, sc) and S, dP of 2t + 1; then (step B) the first half of the arithmetic of 2t + 1
  // under dV, dK of 2t. Each of the three product blocks then carries about 3-4 vector
  // instructions per product (before, the first carried none and the last 8). The P and dS of
  // 2t + 1 are carried to the next tile. Every tile read here (t - 1 and t) has landed.
  bf16x8 pc[2], sc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pc[i][e] = (__bf16)0.f;
      sc[i][e] = (__bf16)0.f;
    }
  }
  // The second half of sub-tile 2t + 1's arithmetic runs under the next tile's first products
  // (its S and dP, which carry no vector work otherwise); s1c, dp1c and the row terms m4c, d4c
  // carry it across the barrier (the row-term slot is rewritten by the next conversion).
  f32x16 s1c, dp1c;
  f32x4 m4c[4], d4c[4];
  auto steady_tile = [&](int t, auto slot_tag, auto first_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;  // t % 4
    constexpr bool kFirst = decltype(first_tag)::value;
    constexpr uint32_t cur = S * TB, prev = ((S + 3) & 3) * TB, half = 32 * D * 2;
    constexpr uint32_t mo0 = (S & 1) * 2 * BQ * 4, mo1 = mo0 + 32 * 4;
    start_copies(t, (S + 2) & 3, (S + 3) & 3);
    convert_rows(t, (S + 1) & 3, (S + 1) & 1);
    if (active) {
      f32x16 s0, dp0;
      bf16x8 p0[2], q0[2];
      f32x4 m4[4], d4[4];
      sd(s0, dp0, cur);
      if constexpr (kFirst) {
        readahead<8, 16>();
      } else {
        grad_h(s1c, dp1c, m4c, d4c, 1, pc, sc);
        interleave_bwd<8, 1, 3, 8, 16>();
      }
      __builtin_amdgcn_sched_barrier(0);
      rows(m4, d4, mo0);
      dvdk(prev + half, pc, sc);
      sd(s1c, dp1c, cur + half);
      grad(s0, dp0, m4, d4, 0, std::false_type{}, p0, q0);
      interleave_bwd<14, 2, 4, 21, 32>();
      __builtin_amdgcn_sched_barrier(0);
      rows(m4c, d4c, mo1);
      dvdk(cur, p0, q0);
      grad_h(s1c, dp1c, m4c, d4c, 0, pc, sc);
      interleave_bwd<14, 2, 4, 13, 16>();
    }
    bar_vm<NCOPY>();
  };
  int t = 0;
  for (; t < n_t && t < 2; ++t) generic_tile(t, std::true_type{});
  const bool ran = t + 6 < n_t;
  if (ran) {
    steady_tile(t, std::integral_constant<int, 2>{}, std::true_type{});
    ++t;
    for (; t + 6 < n_t; t += 4) {  // t % 4 == 3; every copy of the four iterations exists
      steady_tile(t, std::integral_constant<int, 3>{}, std::false_type{});
      steady_tile(t + 1, std::integral_constant<int, 0>{}, std::false_type{});
      steady_tile(t + 2, std::integral_constant<int, 1>{}, std::false_type{});
      steady_tile(t + 3, std::integral_constant<int, 2>{}, std::false_type{});
    }
    if (active) grad_h(s1c, dp1c, m4c, d4c, 1, pc, sc);  // the carried half
  }
  // the last steady tile's carried sub-tile (zero operands when the loop did not run)
  if (active) dvdk((uint32_t)((t + 3) & 3) * TB + 32 * D * 2, pc, sc);
  for (; t < n_t; ++t) generic_tile(t, std::false_type{});

  const float dck_tot = xhalf_sum(dck);
  if (!kok) return;
  const size_t row = base + (size_t)kj * D;
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = d * 32 + 8 * i + 4 * h;
      *reinterpret_cast<float4*>(dV + row + col) =
          make_float4(dvacc[d][4 * i], dvacc[d][4 * i + 1], dvacc[d][4 * i + 2], dvacc[d][4 * i + 3]);
      *reinterpret_cast<float4*>(dK + row + col) =
          make_float4(dkacc[d][4 * i] * scale, dkacc[d][4 * i + 1] * scale,
                      dkacc[d][4 * i + 2] * scale, dkacc[d][4 * i + 3] * scale);
    }
  }
  if (h == 0) dck_out[(size_t)bh * L + kj] = dck_tot;
}

// Query-stationary step with the forward kernel's memory pipeline. NB 32-query blocks per wave
// share every K / V operand read; 8 / NB waves cover 256 queries (NB = 1: 8 waves, two per
// SIMD, within 256 registers each; NB = 2: 4 waves, within 256 registers at D = 64, where two
// workgroups share a compute unit). Keys are walked in 64-key tiles (two 32-key sub-tiles):
// the diagonal band (the last four key tiles, where sub-tile j is key block
// 2 kt_last + 1 - j) from the diagonal backwards, then the older tiles in ascending order.
// K, V and raw c of tile t sit in LDS
// ring slot t % 4 (the bias slice (c_j - c_ref) log2 e of tile t in slot t % 2); iteration t
// reads K(t), V(t) and the bias of tile t, starts the untracked copies of K(t + 2), V(t + 2)
// and c(t + 3), converts c(t + 1) into the bias of tile t + 1, and its barrier waits only for
// the copies started one iteration earlier. Tile 0 (holding the sequence end) goes through
// registers with zero fill. Per 32-key sub-tile and query block a wave computes S^T = K Q^T
// and dP^T = V dO^T, then P = exp2(scale log2(e) s - (bias_j + m_i)) with
// m_i = (LSE_i - (c_i - c_ref)) log2 e (bias and m added first, as in the forward),
// dS = P (dP - Delta_i), and dQ^T += K^T dS^T with K^T from transposed reads of the K tile.
// Tiles 0..3 hold every wave's diagonal and evaluate the causal mask; from tile 4 on the loop
// is unrolled over four tiles so that every LDS address is a per-lane base plus an immediate.
template <int D, int NB, typename CT>
__global__ __launch_bounds__(512 / NB) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 3 - NB, D == 64 ? 2 : 3 - NB))) void dq_pipe_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const CT* __restrict__ C, const float* __restrict__ LSE,
    const float* Delta, const float* __restrict__ O, float* __restrict__ dQ,
    float* __restrict__ dcq_out, float* delta_out, float* lse_out,
    const int32_t* __restrict__ q_skip,
    const int32_t* __restrict__ q_order, int L, int BH, int n_qt, float sl2e, float scale) {
  constexpr int NW = 8 / NB, BM = 256, NT = NW * 64, BN = 64;
  constexpr int TILE = BN * D;
  constexpr int CPR = D / 8;
  constexpr int CPT = TILE / 8 / NT;
  constexpr int BLK = TILE * 2 / 1024 / NW;  // 1 KiB copies per wave per tensor and tile
  constexpr int CW = BN / NW;                // c values each wave copies per tile
  constexpr int NCOPY = 2 * BLK + 1;
  static_assert(CPT >= 1 && BLK >= 1, "tile must split evenly over the waves");
  constexpr uint32_t TB = TILE * 2;
  constexpr uint32_t CS = sizeof(CT);  // bytes of one raw c value (fp32 or fp64)
  constexpr uint32_t K_OFF = 0, V_OFF = 4 * TB, R_OFF = 8 * TB, C_OFF = 8 * TB + 4 * BN * CS;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[8 * TB + 4 * BN * CS + 2 * BN * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  // Longest-first: by query tile, or in a skip plan's order of decreasing work.
  const int bid = blockIdx.x;
  int bh, qt;
  if (q_order) {
    const int item = q_order[bid];
    bh = item / n_qt;
    qt = item % n_qt;
  } else {  // query tiles from the last, each head kept to one XCD where possible
    int level;
    xcd_item(bid, BH, bh, level);
    qt = n_qt - 1 - level;
  }
  const int q0 = qt * BM;
  const size_t base = (size_t)bh * L * D;
  Q += base;
  K += base;
  V += base;
  dO += base;
  C += (size_t)bh * L;
  const CT c_ref = C[q0];
  const int qw = q0 + wave * 32 * NB;
  const int q_last = (q0 + BM - 1 < L - 1) ? q0 + BM - 1 : L - 1;
  const int kt_last = q_last / BN;
  // Key tiles kt_last down to the oldest one a skip plan could not rule out.
  const int kt_skip = q_skip ? q_skip[(size_t)bh * n_qt + qt] : 0;
  const int n_t = kt_last + 1 - kt_skip;
  const bool active = qw <= q_last;
  const int j0 = max(2 * kt_last + 2 - NB - qw / 32, 0);  // first sub-tile with a key <= a query of the wave
  const i32x4 k_rs = buffer_words(K, (uint32_t)L * (uint32_t)(D * 2));
  const i32x4 v_rs = buffer_words(V, (uint32_t)L * (uint32_t)(D * 2));
  const i32x4 c_rs = buffer_words(C, (uint32_t)L * CS);
  const uint32_t sbase = lds_addr(smem);

  int qi[NB];
  bool qok[NB];
  bf16x8 qf[NB][D / 16], dof[NB][D / 16];
  float mrow[NB], dl[NB], dcq[NB], psum[NB];
  f32x16 dqacc[NB][D / 32];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    qi[b] = qw + 32 * b + l32;
    qok[b] = qi[b] < L;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (qok[b]) {
        qf[b][c] = ld8(Q + (size_t)qi[b] * D + 16 * c + 8 * h);
        dof[b][c] = ld8(dO + (size_t)qi[b] * D + 16 * c + 8 * h);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qf[b][c][e] = (__bf16)0.f;
          dof[b][c][e] = (__bf16)0.f;
        }
      }
    }
    // rows past the end get P = 0 through an infinite row offset
    mrow[b] = qok[b] ? (LSE[(size_t)bh * L + qi[b]] - cdiff(C[qi[b]], c_ref)) * kLog2e : INFINITY;
    if (O) {
      // Delta_i = dO_i . O_i from the fp32 output, summed in delta_kernel's order: each group of
      // eight consecutive elements in order, then the D/8 groups as a balanced pairwise tree
      // (group 2c + h is this lane's chunk c; the partner half sits in lane ^ 32). The fused
      // and the separate row term therefore agree bit for bit.
      float g[D / 16];
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        float acc = 0.f;
        if (qok[b]) {
          const float* orow = O + base + (size_t)qi[b] * D + 16 * c + 8 * h;
          const float4 x0 = *reinterpret_cast<const float4*>(orow);
          const float4 x1 = *reinterpret_cast<const float4*>(orow + 4);
          const float o8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf((float)dof[b][c][e], o8[e], acc);
        }
        g[c] = acc;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) g[c] += __shfl_xor(g[c], 32, 64);
#pragma unroll
      for (int w = 1; w < D / 16; w <<= 1) {
#pragma unroll
        for (int c = 0; c < D / 16; c += 2 * w) g[c] += g[c + w];
      }
      dl[b] = g[0];  // 0 for rows past the end
    } else {
      dl[b] = qok[b] ? Delta[(size_t)bh * L + qi[b]] : 0.f;
    }
    dcq[b] = 0.f;
    psum[b] = 0.f;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) dqacc[b][d] = zero16();
  }

  // Key tile of visit t: the diagonal band (the last four key tiles) from the diagonal
  // backwards, then the older tiles in ascending order, so that the workgroups of one head that
  // run at the same time stream the same K and V tiles through the cache.
  auto key_tile = [&](int t) __attribute__((always_inline)) {
    return t < 4 ? kt_last - t : t - 4 + kt_skip;
  };
  auto copy_kv = [&](const i32x4& rs, uint32_t region, int t, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const int blk = wave * BLK + k;
      const int r = blk * (512 / D) + lane / CPR;
      const int lc = (lane % CPR) ^ swz_key<D>(r);
      const uint32_t voff = (uint32_t)((key_tile(t) * BN + r) * D + lc * 8) * 2;
      copy16_to_lds(sbase + region + slot * TB + blk * 1024, voff, rs);
    }
  };
  auto copy_c = [&](int t, int slot) __attribute__((always_inline)) {
    if (lane < CW * (int)CS / 4) {  // one 4-byte word per lane
      const uint32_t voff = (uint32_t)(key_tile(t) * BN + wave * CW) * CS + lane * 4;
      copy4_to_lds(sbase + R_OFF + slot * BN * CS + wave * CW * CS, voff, c_rs);
    }
  };
  auto start_copies = [&](int t, int skv, int sc) __attribute__((always_inline)) {
    if (t + 2 < n_t) {
      copy_kv(k_rs, K_OFF, t + 2, skv);
      copy_kv(v_rs, V_OFF, t + 2, skv);
    }
    if (t + 3 < n_t) copy_c(t + 3, sc);
  };
  auto convert_c = [&](int t, int sr, int sb) __attribute__((always_inline)) {
    if (wave == 0 && t + 1 < n_t) {
      const CT cj = *(const __attribute__((address_space(3))) CT*)(uintptr_t)(
          sbase + R_OFF + sr * BN * CS + lane * CS);
      *(__attribute__((address_space(3))) float*)(uintptr_t)(sbase + C_OFF + sb * BN * 4 + lane * 4) =
          cbias(cj, c_ref);
    }
  };

  uint32_t kp[D / 16], vq[D / 16], kt[D / 32][2];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    kp[c] = opaque(sbase + K_OFF + row8_off<D>(lane, 16 * c + 8 * h));
    vq[c] = opaque(sbase + V_OFF + row8_off<D>(lane, 16 * c + 8 * h));
  }
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    kt[d][0] = opaque(sbase + K_OFF + col8_off<D>(lane, d * 32, 0));
    kt[d][1] = opaque(sbase + K_OFF + col8_off<D>(lane, d * 32, 1));
  }
  const uint32_t cp = opaque(sbase + C_OFF + 16 * h);

  // One 32-key sub-tile for both query blocks: rows at byte offset ro of a K / V slot, bias
  // slice at co, first key key0 (masking only with kMask).
  auto sub_tile = [&](uint32_t ro, uint32_t co, int key0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    f32x16 s[NB], dp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s[b] = zero16();
      dp[b] = zero16();
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 a = lds_ld16(kp[c] + ro);
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = mfma32(a, qf[b][c], s[b]);
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 a = lds_ld16(vq[c] + ro);
#pragma unroll
      for (int b = 0; b < NB; ++b) dp[b] = mfma32(a, dof[b][c], dp[b]);
    }
    bf16x8 sb[NB][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 ck = lds_ldf4(cp + co + 32 * i);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = fmaf(s[b][4 * i + e], sl2e, -(ck[e] + mrow[b]));
          if constexpr (kMask) {
            if ((key0 + 8 * i + 4 * h + e) > qi[b]) x = -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(x);
          const float ds = p * (dp[b][4 * i + e] - dl[b]);
          dcq[b] += ds;
          psum[b] += p;
          s[b][4 * i + e] = ds;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      sb[b][0] = pack_c_half(s[b], 0);
      sb[b][1] = pack_c_half(s[b], 1);
    }
    // The diagonal band (the masked sub-tiles) holds the keys that carry a row's largest weights
    // whenever a few keys dominate it (early rows, strong decay), and there dS is large: its
    // bf16 rounding alone can move dQ by ~2^-9 |dQ|. The band's products therefore also take the
    // rounding remainder dS - bf16(dS), so they see dS to ~2^-17.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 sl[NB];
      if constexpr (kMask) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sl[b][e] = (__bf16)(s[b][8 * t + e] - (float)sb[b][t][e]);
        }
      }
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const bf16x8 a = lds_tr8(kt[d][0] + ro + t * 16 * D * 2, kt[d][1] + ro + t * 16 * D * 2);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          dqacc[b][d] = mfma32(a, sb[b][t], dqacc[b][d]);
          if constexpr (kMask) dqacc[b][d] = mfma32(a, sl[b], dqacc[b][d]);
        }
      }
    }
  };

  // prologue: tile 0 through registers (zero fill past the end), copies of K(1), V(1), c(1), c(2)
  {
    const int k0 = kt_last * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int key = k0 + idx / CPR, cc = idx % CPR;
      lds_store8<D>((bf16_t*)(smem + K_OFF), idx / CPR, cc * 8, ld16_or_zero<D>(K, key, L, cc * 8));
      lds_store8<D>((bf16_t*)(smem + V_OFF), idx / CPR, cc * 8, ld16_or_zero<D>(V, key, L, cc * 8));
    }
    if (tid < BN) {
      const int key = k0 + tid;
      ((float*)(smem + C_OFF))[tid] = key < L ? cbias(C[key], c_ref) : 0.f;
    }
    if (1 < n_t) {
      copy_kv(k_rs, K_OFF, 1, 1);
      copy_kv(v_rs, V_OFF, 1, 1);
      copy_c(1, 1);
    }
    if (2 < n_t) copy_c(2, 2);
    bar_vm<0>();
  }

  // tiles 0..3 (the diagonal band, masked) and the last few tiles: run-time slots
  auto generic_tile = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    start_copies(t, (t + 2) & 3, (t + 3) & 3);
    convert_c(t, (t + 1) & 3, (t + 1) & 1);
    if (active) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int j = 2 * t + sub;
        const uint32_t ro = (uint32_t)(t & 3) * TB + (uint32_t)(1 - sub) * 32 * D * 2;
        const uint32_t co = (uint32_t)(t & 1) * BN * 4 + (uint32_t)(1 - sub) * 32 * 4;
        if (j >= j0) sub_tile(ro, co, (2 * kt_last + 1 - j) * 32, mask_tag);
      }
    }
    bar_vm<0>();
  };
  auto steady_tile = [&](int t, auto slot_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;  // t % 4
    start_copies(t, (S + 2) & 3, (S + 3) & 3);
    convert_c(t, (S + 1) & 3, (S + 1) & 1);
    if (active) {
      sub_tile(S * TB + 32 * D * 2, (S & 1) * BN * 4 + 32 * 4, 0, std::false_type{});
      sub_tile(S * TB, (S & 1) * BN * 4, 0, std::false_type{});
    }
    bar_vm<NCOPY>();
  };
  int t = 0;
  for (; t < n_t && t < 4; ++t) generic_tile(t, std::true_type{});
  for (; t + 6 < n_t; t += 4) {  // t % 4 == 0; every copy of the four iterations exists
    steady_tile(t, std::integral_constant<int, 0>{});
    steady_tile(t + 1, std::integral_constant<int, 1>{});
    steady_tile(t + 2, std::integral_constant<int, 2>{});
    steady_tile(t + 3, std::integral_constant<int, 3>{});
  }
  for (; t < n_t; ++t) generic_tile(t, std::false_type{});

  // Row terms consistent with this kernel's own P and dP.
  // Normalisation: the forward's LSE is the log of the sum of the bf16-rounded weights that built
  // O (and carries the rounding of c_i - c_ref), so exp(s - LSE) sums over a row to
  // S = sum_j P_ij = 1 + O(2^-9), most off where a few keys dominate (after a hard reset). A
  // row-constant error like that cancels in S: P_ij / S is the softmax to fp32 rounding. dQ and
  // dc^q are scaled by 1 / S here, and LSE' = LSE + ln S goes to the key-stationary step, whose
  // P then sums to one in every row; otherwise sum_i P_ij (...) in dc^k inherits the row errors
  // and d log f accumulates them.
  // Row term: the forward's O was built from P rounded to bf16, so dO.O differs from
  // sum_j P_ij dP_ij by ~1e-3 relative, and that residual would accumulate in d log f over every
  // row that still attends across a position. With eps = sum_j P_ij (dP_ij - Delta_i),
  // Delta'_i = Delta_i + eps / S makes sum_j P_ij (dP_ij - Delta'_i) vanish; the key-stationary
  // step uses Delta', and dc^q is that (rounding-level) row sum. dQ keeps Delta: its error from
  // the residual is ~scale*eps*|k| / S.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float eps = xhalf_sum(dcq[b]);
    const float ptot = xhalf_sum(psum[b]);
    const float dl_new = dl[b] + eps / ptot;
    const float inv = 1.0f / ptot;
    const float dcq_tot = (eps - (dl_new - dl[b]) * ptot) * inv;
    if (qok[b]) {
      const size_t row = base + (size_t)qi[b] * D;
      const float sc = scale * inv;
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = d * 32 + 8 * i + 4 * h;
          *reinterpret_cast<float4*>(dQ + row + col) =
              make_float4(dqacc[b][d][4 * i] * sc, dqacc[b][d][4 * i + 1] * sc,
                          dqacc[b][d][4 * i + 2] * sc, dqacc[b][d][4 * i + 3] * sc);
        }
      }
      if (h == 0) {
        const size_t r = (size_t)bh * L + qi[b];
        dcq_out[r] = dcq_tot;
        delta_out[r] = dl_new;
        lse_out[r] = LSE[r] + __logf(ptot);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 path (vector ALU, no down-conversion; the counterpart of fwd_f32_kernel). A wave owns 16
// rows (queries in f32_dq_kernel, keys in f32_dkv_kernel) with 4 lanes per row, each lane holding
// a quarter of the head dimension; the other side's rows stream through LDS 32 at a time. Both
// kernels form every dS element with the same instructions in the same order (f32_dot and
// f32_ds), so the row sums dc^q and the column sums dc^k come from bit-identical dS and the
// reverse scan telescopes, as in the bf16 path; those sums and the row-term refinement run in
// fp64.
constexpr int kF32Rows = 16;  // rows per wave (4 lanes each)
constexpr int kF32Tile = 32;  // streamed rows per LDS tile

// Dot product of a row quarter held by this lane with the matching quarter of b, summed over the
// row's 4 lanes (lane bits 4 and 5) as (q0 + q1) + (q2 + q3) in every lane.
template <int DQ>
__device__ __forceinline__ float f32_dot(const float (&a)[DQ], const float* b) {
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < DQ; ++d) s = fmaf(a[d], b[d], s);
  s += __shfl_xor(s, 16, 64);
  return s + __shfl_xor(s, 32, 64);
}
// P_ij and dS_ij from the two dot products and the row / column terms.
template <typename CT>
__device__ __forceinline__ void f32_ds(float qk, float dp, float scale, CT ci, CT cj,
                                       float lse_i, float delta_i, float& p, float& ds) {
  p = expf(fmaf(qk, scale, cdiff(ci, cj)) - lse_i);
  ds = p * (dp - delta_i);
}

template <int D>
__global__ __launch_bounds__(256) void delta_f32_kernel(const float* __restrict__ dO,
                                                        const float* __restrict__ O,
                                                        float* __restrict__ delta, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  if (row < rows)
    for (int d = lane; d < D; d += 64) acc = fmaf(dO[(size_t)row * D + d], O[(size_t)row * D + d], acc);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && lane == 0) delta[row] = acc;
}

// dQ, dc^q and the refined row term (as dq_pipe_kernel: Delta' makes the kernel's own row of dS
// sum to zero; dc^q is the remaining rounding-level sum).
template <int D, typename CT>
__global__ __launch_bounds__(64) void f32_dq_kernel(const float* __restrict__ Q,
                                                    const float* __restrict__ K,
                                                    const float* __restrict__ V,
                                                    const float* __restrict__ dO,
                                                    const CT* __restrict__ C,
                                                    const float* __restrict__ LSE,
                                                    const float* Delta, float* __restrict__ dQ,
                                                    float* __restrict__ dcq_out,
                                                    float* delta_out, float* lse_out, int L,
                                                    float scale) {
  constexpr int DQ = D / 4;
  __shared__ float k_s[kF32Tile][D], v_s[kF32Tile][D];
  __shared__ CT c_s[kF32Tile];
  const int tid = threadIdx.x, part = tid >> 4;
  const int64_t bh = blockIdx.y;
  const int qi = blockIdx.x * kF32Rows + (tid & 15);
  const bool qok = qi < L;
  const size_t base = (size_t)bh * L * D, rbase = (size_t)bh * L;
  float q[DQ], g[DQ], acc[DQ];
#pragma unroll
  for (int d = 0; d < DQ; ++d) {
    q[d] = qok ? Q[base + (size_t)qi * D + part * DQ + d] : 0.f;
    g[d] = qok ? dO[base + (size_t)qi * D + part * DQ + d] : 0.f;
    acc[d] = 0.f;
  }
  const CT ci = qok ? C[rbase + qi] : (CT)0;
  const float lse = qok ? LSE[rbase + qi] : 0.f;
  const float dl = qok ? Delta[rbase + qi] : 0.f;
  double eps = 0.0, ptot = 0.0;
  const int q_last = min(blockIdx.x * kF32Rows + kF32Rows - 1, L - 1);
  for (int k0 = 0; k0 <= q_last; k0 += kF32Tile) {
    __syncthreads();
    for (int i = tid; i < kF32Tile * D; i += 64) {
      const int r = i / D, d = i % D, key = k0 + r;
      k_s[r][d] = key < L ? K[base + (size_t)key * D + d] : 0.f;
      v_s[r][d] = key < L ? V[base + (size_t)key * D + d] : 0.f;
    }
    if (tid < kF32Tile) c_s[tid] = k0 + tid < L ? C[rbase + k0 + tid] : (CT)0;
    __syncthreads();
    for (int j = 0; j < kF32Tile; ++j) {
      const float qk = f32_dot<DQ>(q, &k_s[j][part * DQ]);
      const float dp = f32_dot<DQ>(g, &v_s[j][part * DQ]);
      if (qok && k0 + j <= qi) {
        float p, ds;
        f32_ds(qk, dp, scale, ci, c_s[j], lse, dl, p, ds);
        eps += (double)ds;
        ptot += (double)p;
#pragma unroll
        for (int d = 0; d < DQ; ++d) acc[d] = fmaf(ds, k_s[j][part * DQ + d], acc[d]);
      }
    }
  }
  if (!qok) return;
#pragma unroll
  for (int d = 0; d < DQ; ++d) dQ[base + (size_t)qi * D + part * DQ + d] = acc[d] * scale;
  if (part == 0) {
    const double dl_new = (double)dl + eps / ptot;
    dcq_out[rbase + qi] = (float)(eps - (dl_new - (double)dl) * ptot);
    delta_out[rbase + qi] = (float)dl_new;
    // this path's forward sums the fp32 weights, so its rows already sum to one to fp32
    // rounding: the row offset passes unchanged, and both steps form bit-identical dS
    lse_out[rbase + qi] = lse;
  }
}

// dK, dV and dc^k (keys stationary; queries from the key's own onwards).
template <int D, typename CT>
__global__ __launch_bounds__(64) void f32_dkv_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     const float* __restrict__ dO,
                                                     const CT* __restrict__ C,
                                                     const float* __restrict__ LSE,
                                                     const float* __restrict__ Delta,
                                                     float* __restrict__ dK, float* __restrict__ dV,
                                                     float* __restrict__ dck_out, int L,
                                                     float scale) {
  constexpr int DQ = D / 4;
  __shared__ float q_s[kF32Tile][D], o_s[kF32Tile][D], l_s[kF32Tile], d_s[kF32Tile];
  __shared__ CT c_s[kF32Tile];
  const int tid = threadIdx.x, part = tid >> 4;
  const int64_t bh = blockIdx.y;
  const int k0 = blockIdx.x * kF32Rows;
  const int kj = k0 + (tid & 15);
  const bool kok = kj < L;
  const size_t base = (size_t)bh * L * D, rbase = (size_t)bh * L;
  float kr[DQ], vr[DQ], dk[DQ], dv[DQ];
#pragma unroll
  for (int d = 0; d < DQ; ++d) {
    kr[d] = kok ? K[base + (size_t)kj * D + part * DQ + d] : 0.f;
    vr[d] = kok ? V[base + (size_t)kj * D + part * DQ + d] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const CT cj = kok ? C[rbase + kj] : (CT)0;
  double dck = 0.0;
  for (int i0 = k0 / kF32Tile * kF32Tile; i0 < L; i0 += kF32Tile) {
    __syncthreads();
    for (int i = tid; i < kF32Tile * D; i += 64) {
      const int r = i / D, d = i % D, qq = i0 + r;
      q_s[r][d] = qq < L ? Q[base + (size_t)qq * D + d] : 0.f;
      o_s[r][d] = qq < L ? dO[base + (size_t)qq * D + d] : 0.f;
    }
    if (tid < kF32Tile) {
      const int qq = i0 + tid;
      c_s[tid] = qq < L ? C[rbase + qq] : (CT)0;
      l_s[tid] = qq < L ? LSE[rbase + qq] : 0.f;
      d_s[tid] = qq < L ? Delta[rbase + qq] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < kF32Tile; ++r) {
      const float qk = f32_dot<DQ>(kr, &q_s[r][part * DQ]);
      const float dp = f32_dot<DQ>(vr, &o_s[r][part * DQ]);
      if (kok && i0 + r >= kj && i0 + r < L) {
        float p, ds;
        f32_ds(qk, dp, scale, c_s[r], cj, l_s[r], d_s[r], p, ds);
        dck -= (double)ds;
#pragma unroll
        for (int d = 0; d < DQ; ++d) {
          dv[d] = fmaf(p, o_s[r][part * DQ + d], dv[d]);
          dk[d] = fmaf(ds, q_s[r][part * DQ + d], dk[d]);
        }
      }
    }
  }
  if (!kok) return;
#pragma unroll
  for (int d = 0; d < DQ; ++d) {
    dK[base + (size_t)kj * D + part * DQ + d] = dk[d] * scale;
    dV[base + (size_t)kj * D + part * DQ + d] = dv[d];
  }
  if (part == 0) dck_out[rbase + kj] = (float)dck;
}

inline size_t region_floats(int64_t BH, int64_t L) {
  return (size_t)((BH * L + 63) / 64 * 64);  // 256-byte granules
}

template <int D>
void go_delta(const bf16_t* dO, const float* o, float* delta, int64_t rows, hipStream_t s) {
  hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0,
                     s, dO, o, delta, rows);
}

template <int D, typename CT>
void go_dkv(const bf16_t* q, const bf16_t* k, const bf16_t* v, const void* c, const float* lse,
            const bf16_t* dO, const float* delta, float* dk, float* dv, float* dck, int64_t BH,
            int64_t L, float scale, const SkipArgs& skip, hipStream_t s) {
  const int n_kt = (int)((L + 127) / 128);
  hipLaunchKernelGGL((dkv_pipe_kernel<D, CT>), dim3((unsigned)(n_kt * BH)), dim3(256), 0, s, q, k,
                     v, dO, (const CT*)c, lse, delta, dk, dv, dck, skip.kv_tiles, skip.kv_order,
                     (int)L, (int)BH, scale * kLog2e, scale);
}

template <int D, typename CT>
void go_dq(const bf16_t* q, const bf16_t* k, const bf16_t* v, const void* c, const float* lse,
           const bf16_t* dO, const float* delta, const float* o, float* dq, float* dcq,
           float* delta_out, float* lse_out, int64_t BH, int64_t L, float scale,
           const SkipArgs& skip,
           hipStream_t s) {
  const int n_qt = (int)((L + 255) / 256);
  // D = 128: one 32-query block per wave, 8 waves (two per SIMD): measured 18% faster than 4
  // waves with two blocks each, whose halved LDS traffic does not make up for the lost latency
  // hiding. D = 64: two blocks per wave, 4 waves in 253 registers and 67 KB of LDS, so two
  // workgroups share a compute unit and each SIMD still runs two waves, each K and V operand
  // read now feeding two products (6% faster than one block per wave).
  constexpr int NB = D == 64 ? 2 : 1;
  hipLaunchKernelGGL((dq_pipe_kernel<D, NB, CT>), dim3((unsigned)(n_qt * BH)), dim3(512 / NB), 0, s, q, k,
                     v, dO, (const CT*)c, lse, delta, o, dq, dcq, delta_out, lse_out, skip.q_skip,
                     skip.q_order, (int)L, (int)BH, n_qt, scale * kLog2e, scale);
}

}  // namespace

// Four fp32 [BH, L] regions: the refined row term, dc^q, dc^k and the row offset LSE' that the
// query-stationary step hands to the key-stationary one.
size_t bwd_workspace_bytes(int64_t BH, int64_t L) { return 4 * region_floats(BH, L) * sizeof(float); }

hipError_t launch_bwd_delta(const void* dO, const float* o, float* delta, int64_t rows, int64_t D,
                            hipStream_t s) {
  if (D == 64) go_delta<64>((const bf16_t*)dO, o, delta, rows, s);
  else go_delta<128>((const bf16_t*)dO, o, delta, rows, s);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const void* q, const void* k, const void* v, CPtr c,
                          const float* lse, const void* dO, const float* delta, float* dk,
                          float* dv, float* dck, int64_t BH, int64_t L, int64_t D, float scale,
                          const SkipArgs& skip, hipStream_t s) {
  const auto* Q = (const bf16_t*)q;
  const auto* K = (const bf16_t*)k;
  const auto* V = (const bf16_t*)v;
  const auto* G = (const bf16_t*)dO;
  if (D == 64) {
    if (c.f64) go_dkv<64, double>(Q, K, V, c.p, lse, G, delta, dk, dv, dck, BH, L, scale, skip, s);
    else go_dkv<64, float>(Q, K, V, c.p, lse, G, delta, dk, dv, dck, BH, L, scale, skip, s);
  } else {
    if (c.f64) go_dkv<128, double>(Q, K, V, c.p, lse, G, delta, dk, dv, dck, BH, L, scale, skip, s);
    else go_dkv<128, float>(Q, K, V, c.p, lse, G, delta, dk, dv, dck, BH, L, scale, skip, s);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, CPtr c,
                         const float* lse, const void* dO, const float* delta, const float* o,
                         float* dq, float* dcq, float* delta_out, float* lse_out, int64_t BH,
                         int64_t L,
                         int64_t D, float scale, const SkipArgs& skip, hipStream_t s) {
  const auto* Q = (const bf16_t*)q;
  const auto* K = (const bf16_t*)k;
  const auto* V = (const bf16_t*)v;
  const auto* G = (const bf16_t*)dO;
  if (D == 64) {
    if (c.f64)
      go_dq<64, double>(Q, K, V, c.p, lse, G, delta, o, dq, dcq, delta_out, lse_out, BH, L, scale,
                        skip, s);
    else
      go_dq<64, float>(Q, K, V, c.p, lse, G, delta, o, dq, dcq, delta_out, lse_out, BH, L, scale,
                       skip, s);
  } else {
    if (c.f64)
      go_dq<128, double>(Q, K, V, c.p, lse, G, delta, o, dq, dcq, delta_out, lse_out, BH, L, scale,
                         skip, s);
    else
      go_dq<128, float>(Q, K, V, c.p, lse, G, delta, o, dq, dcq, delta_out, lse_out, BH, L, scale,
                        skip, s);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_delta_f32(const float* dO, const float* o, float* delta, int64_t rows,
                                int64_t D, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (D == 64) hipLaunchKernelGGL(delta_f32_kernel<64>, grid, dim3(256), 0, s, dO, o, delta, rows);
  else hipLaunchKernelGGL(delta_f32_kernel<128>, grid, dim3(256), 0, s, dO, o, delta, rows);
  return hipGetLastError();
}

template <int D, typename CT>
void go_dq_f32(const float* q, const float* k, const float* v, const void* c, const float* lse,
               const float* dO, const float* delta, float* dq, float* dcq, float* delta_out,
               float* lse_out, int64_t BH, int64_t L, float scale, hipStream_t s) {
  const dim3 grid((unsigned)((L + kF32Rows - 1) / kF32Rows), (unsigned)BH);
  hipLaunchKernelGGL((f32_dq_kernel<D, CT>), grid, dim3(64), 0, s, q, k, v, dO, (const CT*)c, lse,
                     delta, dq, dcq, delta_out, lse_out, (int)L, scale);
}

hipError_t launch_bwd_dq_f32(const float* q, const float* k, const float* v, CPtr c,
                             const float* lse, const float* dO, const float* delta, float* dq,
                             float* dcq, float* delta_out, float* lse_out, int64_t BH, int64_t L,
                             int64_t D, float scale, hipStream_t s) {
  if (D == 64) {
    if (c.f64)
      go_dq_f32<64, double>(q, k, v, c.p, lse, dO, delta, dq, dcq, delta_out, lse_out, BH, L, scale,
                                     s);
    else go_dq_f32<64, float>(q, k, v, c.p, lse, dO, delta, dq, dcq, delta_out, lse_out, BH, L, scale,
                                     s);
  } else {
    if (c.f64)
      go_dq_f32<128, double>(q, k, v, c.p, lse, dO, delta, dq, dcq, delta_out, lse_out, BH, L, scale,
                                     s);
    else go_dq_f32<128, float>(q, k, v, c.p, lse, dO, delta, dq, dcq, delta_out, lse_out, BH, L, scale,
                                     s);
  }
  return hipGetLastError();
}

template <int D, typename CT>
void go_dkv_f32(const float* q, const float* k, const float* v, const void* c, const float* lse,
                const float* dO, const float* delta, float* dk, float* dv, float* dck, int64_t BH,
                int64_t L, float scale, hipStream_t s) {
  const dim3 grid((unsigned)((L + kF32Rows - 1) / kF32Rows), (unsigned)BH);
  hipLaunchKernelGGL((f32_dkv_kernel<D, CT>), grid, dim3(64), 0, s, q, k, v, dO, (const CT*)c, lse,
                     delta, dk, dv, dck, (int)L, scale);
}

hipError_t launch_bwd_dkv_f32(const float* q, const float* k, const float* v, CPtr c,
                              const float* lse, const float* dO, const float* delta, float* dk,
                              float* dv, float* dck, int64_t BH, int64_t L, int64_t D, float scale,
                              hipStream_t s) {
  if (D == 64) {
    if (c.f64) go_dkv_f32<64, double>(q, k, v, c.p, lse, dO, delta, dk, dv, dck, BH, L, scale, s);
    else go_dkv_f32<64, float>(q, k, v, c.p, lse, dO, delta, dk, dv, dck, BH, L, scale, s);
  } else {
    if (c.f64)
      go_dkv_f32<128, double>(q, k, v, c.p, lse, dO, delta, dk, dv, dck, BH, L, scale, s);
    else go_dkv_f32<128, float>(q, k, v, c.p, lse, dO, delta, dk, dv, dck, BH, L, scale, s);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, CPtr c,
                          const float* o, const float* lse, const float* dO, float* dq, float* dk,
                          float* dv, float* dlog_f, void* ws, int64_t BH, int64_t L, int64_t D,
                          float scale, hipStream_t s) {
  const size_t R = region_floats(BH, L);
  float* delta = (float*)ws;
  float* dcq = delta + R;
  float* dck = delta + 2 * R;
  float* lse2 = delta + 3 * R;
  hipError_t e = launch_bwd_delta_f32(dO, o, delta, BH * L, D, s);
  if (e != hipSuccess) return e;
  e = launch_bwd_dq_f32(q, k, v, c, lse, dO, delta, dq, dcq, delta, lse2, BH, L, D, scale, s);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkv_f32(q, k, v, c, lse2, dO, delta, dk, dv, dck, BH, L, D, scale, s);
  if (e != hipSuccess) return e;
  return launch_rev_cumsum2(dcq, dck, dlog_f, BH, L, s);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, CPtr c,
                           const float* o, const float* lse, const void* dO, float* dq, float* dk,
                           float* dv, float* dlog_f, void* ws, int64_t BH, int64_t L, int64_t D,
                           float scale, const void* plan, hipStream_t s) {
  const size_t R = region_floats(BH, L);
  const SkipArgs skip = skip_args(plan, BH, L);
  float* delta = (float*)ws;
  float* dcq = delta + R;
  float* dck = delta + 2 * R;
  float* lse2 = delta + 3 * R;
  // the query-stationary step forms the row term from O itself and writes the refined value and
  // the normalised row offset; the key-stationary step reads both
  hipError_t e = launch_bwd_dq(q, k, v, c, lse, dO, nullptr, o, dq, dcq, delta, lse2, BH, L, D,
                               scale, skip, s);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkv(q, k, v, c, lse2, dO, delta, dk, dv, dck, BH, L, D, scale, skip, s);
  if (e != hipSuccess) return e;
  return launch_rev_cumsum2(dcq, dck, dlog_f, BH, L, s);
}

}  // namespace fox
