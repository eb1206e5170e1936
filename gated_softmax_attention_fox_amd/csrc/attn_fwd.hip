// attn_fwd.hip — Forgetting Attention forward on gfx950.
//
// Computes, for every (b, h) and query i,
//   O_i = sum_{j<=i} softmax_j(scale q_i.k_j + c_i - c_j) v_j,  LSE_i = log sum_j exp(...),
// tile by tile, without materialising the L x L bias (paper-graph-ui summary of arXiv 2503.02130,
// section 3.4, "Hardware-Aware Implementation (Modified FlashAttention)", the forward pass: load
// the c slices with the Q and K/V blocks, add the rank-1 bias c^q 1^T - 1 c^k^T to the logit
// block on chip, mask causally, run the online softmax, normalise at the end; paperlayer.ai
// summary, section E).
//
// bf16 path (MFMA). A workgroup owns 256 queries of one (b, h); each of its 8 waves owns 32 of
// them. The score block is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so
// that every lane holds one query's column of scores: the row max and row sum of the online
// softmax are then in-lane reductions plus one exchange with the partner half-wave. The
// probabilities stay in registers and feed O^T += V^T P^T directly as the B operand; V^T comes
// from transposed reads (ds_read_b64_tr_b16) of the row-major V tile in LDS. The diagonal band
// of keys is visited first: it fixes a running max that the decaying bias rarely lets older keys
// beat, so O is rescaled only when a row max rises by more than kFwdLazy; the older keys then
// follow in ascending order, which keeps the workgroups of one head on the same K and V tiles at
// the same time. Workgroups are issued longest-first (the last query tiles, which see the most keys,
// start first) to even out the causal triangle. The memory pipeline, the three-stage software
// pipeline per wave and the phases are described at the kernel.
//
// Bias and precision: the softmax runs in base 2 on
//   y = scale*log2(e)*(q.k) - (ck_j + m_i),  ck_j = log2(e)*(c_j - c_r),
// with c_r = c at the workgroup's first query and m_i the row's running reference. The row
// constant c_i - c_r cancels in the softmax and is added back only to LSE. ck_j and m_i are
// summed before the fma: both grow large when c_r is far from the row's own c, and for every
// key with weight they nearly cancel, so the sum is exact.
//
// fp32 path (vector ALU, no down-conversion): one wave owns 32 queries, two lanes per query
// (each half of the head dimension), K/V tiles of 32 keys in LDS; the logit is
// scale*(q.k) + (c_i - c_j) in fp32 and the softmax uses expf.
#include <type_traits>
#include <utility>

#include "fox_device.h"
#include "fox_launch.h"

namespace fox {
namespace {

constexpr int kFwdBN = 64;  // keys per LDS tile
constexpr float kFwdLazy = 8.0f;  // rescale O only when a row max rises by more than this (log2)
constexpr float kFwdLazyW = 256.0f;  // 2^kFwdLazy: the weight a row max above kFwdLazy exceeds
struct First { static constexpr bool value = true; };   // tag: a wave's first (diagonal) tile
struct Rest { static constexpr bool value = false; };   // tag: every later tile

// Instruction order of one pipelined step (scheduler groups, filled in this order): kD0 LDS reads,
// then each of the step's 16 matrix products followed by kDs LDS reads (for the first kNd
// products) and kV vector instructions.
template <int I, int kDs, int kV, int kNd>
__device__ __forceinline__ void interleave_one() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (I < kNd) __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
}
template <int kD0, int kDs, int kV, int kNd, int... I>
__device__ __forceinline__ void interleave_all(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, kD0, 0);
  (interleave_one<I, kDs, kV, kNd>(), ...);
}
template <int kD0, int kDs, int kV, int kNd>
__device__ __forceinline__ void interleave_step() {
  interleave_all<kD0, kDs, kV, kNd>(std::make_integer_sequence<int, 16>{});
}

// ---------------------------------------------------------------------------------------------
// bf16 kernel: 8 waves x 32 queries (256 queries of one (b, h) per workgroup), diagonal band first
// with lazy rescaling (see the head of this file). Each wave overlaps three 32-key sub-tiles:
// while it turns the scores of sub-tile j into probabilities (VALU), the matrix cores work on
// O += V(j-1)^T P(j-1)^T and on S(j+1)^T = K(j+1) Q^T. The workgroup visits n_t 64-key tiles:
// visit t < 4 is key tile kt_last - t (the band), visit t >= 4 is key tile t - 4; visit t holds
// sub-tiles 2t (its rows 32..63) and 2t + 1 (rows 0..31).
//
// Memory pipeline. K, V and the raw c values of tile t live in LDS ring slot t % 4 (the bias
// slice of tile t, (c_j - c_ref) log2 e, in slot t % 2). Iteration t reads K(t), K(t + 1),
// V(t - 1), V(t) and the bias of tile t; it starts the global -> LDS copies of K(t + 3),
// V(t + 2) and c(t + 3), converts c(t + 1) into the bias of tile t + 1, and ends with a barrier
// that waits only for the copies started one iteration earlier, so every copy has two
// iterations to land. The copies are inline-assembly buffer loads the compiler does not track
// (fox_device.h), which keeps it from stalling the first LDS read after each copy. Tile 0 (the
// one holding the sequence end, possibly partial) goes through registers with zero fill.
//
// Phases. Every wave's diagonal 32-key block lies in tiles 0..3 (the diagonal band); there the
// waves run P(j-1)V, S(j), softmax(j) one after another from their own first sub-tile, which is
// the only one that evaluates the causal mask. From tile 4 on all waves are in step and run the
// pipelined body; its main loop is unrolled over four tiles so that every ring slot is a
// compile-time constant and every LDS address is a per-lane base register plus an immediate.
//
// Fused scan (kLogF). The kernel then takes log f (LF) instead of c and forms the prefix sums
// itself, in fp64: a workgroup sums log f over every position before its window (the 256
// positions of its diagonal band, which hold its own queries), scans the window, and writes c
// for its queries (Cout, fp32 or fp64) for the backward. For the older key tiles, walked in
// ascending order, the converting wave carries the running prefix from tile to tile and scans
// each tile's 64 values. Every bias is an fp64 difference of prefix sums, rounded once.
//
// Pro-block options (runtime, outside the hot loop; the Pro Block Architecture of the
// paper-graph-ui summary, section 3.4). FwdPro::q_norm: each query row is RMS-normalised in
// registers when it is loaded (Step 1, QK-norm of the queries; the keys come normalised from the
// key shift). FwdPro::y: the epilogue writes y = RMSNorm(O) [* out_w] * sigmoid(g) (Steps 5 and 7,
// output norm and output gate) from the fp32 O still in registers; O itself may then be skipped.
// FwdPro::k_alpha, v_alpha, k_norm (the kPre instantiation; Steps 2-3, token shift, and Step 1 for
// the keys): K and V arrive as the raw key and value candidates, and every tile goes through
// registers on its way to LDS, where each row t becomes a_t x_{t-1} + (1 - a_t) x_t (x_{-1} = 0)
// and, for keys, is RMS-normalised: the arithmetic of the separate shift pass, element for
// element, so the tiles hold the bits that pass would have written. Every workgroup whose queries
// see a key tile repeats that work for it.
struct FwdPro {
  const float* q_w = nullptr;  // QK-norm weight [D] or null (unit)
  float q_eps = 0.f;
  int q_norm = 0;
  const void* g = nullptr;     // output gate pre-activation [B, H, L, D] (bf16 or fp32)
  int g_f32 = 0;
  const float* out_w = nullptr;  // output-norm weight [D] or null (unit)
  float out_eps = 0.f;
  void* y = nullptr;           // [B, H, L, D] in g's type, or null: no output gate
  const float* k_alpha = nullptr;  // key shift gate [B, H, L] or null (no key shift)
  const float* v_alpha = nullptr;  // value shift gate [B, H, L] or null (no value shift)
  int k_norm = 0;                  // RMS-normalise each key row (after its shift)
  const float* k_w = nullptr;      // its weight [D] or null (unit)
  float k_eps = 0.f;
};

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

template <int D, typename CT, bool kLogF, bool kPre>
__global__ __launch_bounds__(512) void fwd_bf16_pipe_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const CT* __restrict__ C, const float* __restrict__ LF, CT* __restrict__ Cout,
    void* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ q_skip,
    const int32_t* __restrict__ q_order, int L, int BH, int n_qt, float sl2e, int o_f32,
    FwdPro pro) {
  constexpr int NW = 8, BM = NW * 32, NT = NW * 64, BN = kFwdBN;
  constexpr int TILE = BN * D;
  constexpr int CPR = D / 8;
  constexpr int CPT = TILE / 8 / NT;         // 16-byte chunks per thread per tensor (register path)
  constexpr int BLK = TILE * 2 / 1024 / NW;  // 1 KiB copies per wave per tensor and tile
  // untracked copies a wave starts per iteration: K, V and c, or only c when K and V go through
  // registers (kPre)
  constexpr int NCOPY = kPre ? 1 : 2 * BLK + 1;
  static_assert(CPT >= 1 && BLK >= 1, "tile must split evenly over the waves");
  constexpr uint32_t TB = TILE * 2;  // bytes of one K or V tile
  // bytes of one raw value in the copy ring: c (fp32 or fp64), or log f (fp32) when fused
  constexpr uint32_t CS = kLogF ? 4 : sizeof(CT);
  constexpr uint32_t K_OFF = 0, V_OFF = 4 * TB, R_OFF = 8 * TB, C_OFF = 8 * TB + 4 * BN * CS;
  // fused scan: the window's fp64 prefix sums and eight per-wave partial sums
  constexpr uint32_t W_OFF = C_OFF + 2 * BN * 4, RED_OFF = W_OFF + (kLogF ? 256 * 8 : 0);
  __shared__ __attribute__((aligned(1024))) unsigned char
      smem[8 * TB + 4 * BN * CS + 2 * BN * 4 + (kLogF ? 256 * 8 + 16 * 8 : 0)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy addresses need it
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
  if constexpr (kLogF) {
    LF += (size_t)bh * L;
    Cout += (size_t)bh * L;
  } else {
    C += (size_t)bh * L;
  }
  const float* k_alpha = (kPre && pro.k_alpha) ? pro.k_alpha + (size_t)bh * L : nullptr;
  const float* v_alpha = (kPre && pro.v_alpha) ? pro.v_alpha + (size_t)bh * L : nullptr;
  const CT c_ref = kLogF ? (CT)0 : C[q0];
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  const int q_last = (q0 + BM - 1 < L - 1) ? q0 + BM - 1 : L - 1;
  const int kt_last = q_last / BN;
  // Leading key tiles a skip plan rules out (every weight in them underflows to zero).
  const int kt_skip = q_skip ? q_skip[(size_t)bh * n_qt + qt] : 0;
  const int n_t = kt_last + 1 - kt_skip;     // tiles this workgroup visits
  const int n_j = 2 * n_t;                   // sub-tiles
  const bool active = qw <= q_last;          // the wave holds at least one real query
  const int j0 = 2 * kt_last + 1 - qw / 32;  // the wave's diagonal sub-tile
  const i32x4 k_rs = buffer_words(K, (uint32_t)L * (uint32_t)(D * 2));
  const i32x4 v_rs = buffer_words(V, (uint32_t)L * (uint32_t)(D * 2));
  const i32x4 c_rs = kLogF ? buffer_words(LF, (uint32_t)L * 4u) : buffer_words(C, (uint32_t)L * CS);
  const uint32_t sbase = lds_addr(smem);
  typedef __attribute__((address_space(3))) double lds_d;
  const int w0 = kt_last >= 3 ? (kt_last - 3) * BN : 0;  // first position of the window
  // fused scan: the prefix sum at q0 sits in the window at P_REF; the converting wave keeps the
  // running prefix before the next older tile at CARRY (LDS, so no fp64 stays live in registers)
  const uint32_t P_REF = sbase + W_OFF + (uint32_t)(q0 - w0) * 8, CARRY = sbase + RED_OFF + 128;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (qi < L) {
      qf[c] = ld8(Q + (size_t)qi * D + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.f;
    }
  }
  if (pro.q_norm) {  // QK-norm of the query: this lane holds half its row, the partner the rest
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)qf[c][e], (float)qf[c][e], ss);
    }
    const float rs = 1.0f / sqrtf(xhalf_sum(ss) / (float)D + pro.q_eps);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qf[c][e] = (__bf16)((float)qf[c][e] * rs * (pro.q_w ? pro.q_w[16 * c + 8 * h + e] : 1.0f));
    }
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) oacc[d] = zero16();
  float m = 0.f, lsum = 0.f;
  bf16x8 pb[2];  // P of the previous sub-tile as B operands (two 16-key halves)

  // ---- copies -------------------------------------------------------------------------------
  // Key tile of visit t: the diagonal band (the last four key tiles) first, from the diagonal
  // backwards; then every earlier key tile not skipped, in ascending order, so that the
  // workgroups of one head that run at the same time stream the same K and V tiles through the
  // cache.
  auto key_tile = [&](int t) __attribute__((always_inline)) {
    return t < 4 ? kt_last - t : t - 4 + kt_skip;
  };
  auto copy_kv = [&](const i32x4& rs, uint32_t region, int t, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < BLK; ++b) {
      const int blk = wave * BLK + b;
      const int r = blk * (512 / D) + lane / CPR;
      const int lc = (lane % CPR) ^ swz_key<D>(r);
      const uint32_t voff = (uint32_t)((key_tile(t) * BN + r) * D + lc * 8) * 2;
      copy16_to_lds(sbase + region + slot * TB + blk * 1024, voff, rs);
    }
  };
  auto copy_c = [&](int t, int slot) __attribute__((always_inline)) {  // 8 values per wave
    if (kLogF && t < 4) return;  // fused: the band's prefix sums come from the window scan
    if (lane < 2 * (int)CS) {  // one 4-byte word per lane
      const uint32_t voff = (uint32_t)(key_tile(t) * BN + wave * 8) * CS + lane * 4;
      copy4_to_lds(sbase + R_OFF + slot * BN * CS + wave * 8 * CS, voff, c_rs);
    }
  };
  // kPre: tile t of K or V through registers into ring slot `slot`, shifted (A non-null) and,
  // for keys, normalised (rows past the sequence end are zero, as in the copies).
  auto stage_tile = [&](const bf16_t* X, const float* A, bool norm, uint32_t region, int t,
                        int slot) __attribute__((always_inline)) {
    const int k0 = key_tile(t) * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, cc = idx % CPR, key = k0 + r;
      float x[8];
      unpack8(ld16_or_zero<D>(X, key, L, cc * 8), x);
      if (A) {
        const bool has_prev = key >= 1 && key < L;  // x_{-1} = 0; rows past the end stay zero
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 pv = *reinterpret_cast<const u32x4*>(X + (size_t)(has_prev ? key - 1 : 0) * D + cc * 8);
        float p[8];
        unpack8(has_prev ? pv : z, p);
        const float a = key < L ? A[key] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = shift_mix(a, p[e], x[e]);
      }
      if (norm) {
        rms_norm8<D>(x, pro.k_w, cc * 8, pro.k_eps);
        if (key >= L) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
      }
      lds_store8<D>((bf16_t*)(smem + region + slot * TB), r, cc * 8, pack8(x));
    }
  };
  // Iteration t's copies: K(t + 3), V(t + 2), c(t + 3) (full tiles only: t >= 1). kPre: the
  // staged tiles first, so that no tracked load follows the untracked copy of c.
  auto start_copies = [&](int t, int sk, int sv, int sc) __attribute__((always_inline)) {
    if constexpr (kPre) {
      if (t + 3 < n_t) stage_tile(K, k_alpha, pro.k_norm != 0, K_OFF, t + 3, sk);
      if (t + 2 < n_t) stage_tile(V, v_alpha, false, V_OFF, t + 2, sv);
      if (t + 3 < n_t) copy_c(t + 3, sc);
    } else {
      if (t + 3 < n_t) {
        copy_kv(k_rs, K_OFF, t + 3, sk);
        copy_c(t + 3, sc);
      }
      if (t + 2 < n_t) copy_kv(v_rs, V_OFF, t + 2, sv);
    }
  };
  // Bias slice of tile t + 1 from its raw c values (wave 0). Fused: from the window's prefix
  // sums for the band, else from the running prefix and a scan of the tile's log f.
  auto convert_c = [&](int t, int sr, int sb) __attribute__((always_inline)) {
    if (wave == 0 && t + 1 < n_t) {
      float bias;
      if constexpr (kLogF) {
        const double p_ref = *(const lds_d*)(uintptr_t)P_REF;
        if (t + 1 < 4) {
          const double pj =
              *(const lds_d*)(uintptr_t)(sbase + W_OFF + (key_tile(t + 1) * BN - w0 + lane) * 8);
          bias = (float)((pj - p_ref) * 1.4426950408889634);
        } else {
          // the tile's own prefix in fp32 on DPP moves (its partial sums are small; the carry
          // across tiles and the reference stay fp64)
          const float x = wave_scan_incl(*(const __attribute__((address_space(3))) float*)(uintptr_t)(
              sbase + R_OFF + sr * BN * 4 + lane * 4));
          const double carry = *(const lds_d*)(uintptr_t)CARRY;
          bias = (float)(((carry - p_ref) + (double)x) * 1.4426950408889634);
          const float tot =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
          if (lane == 0) *(lds_d*)(uintptr_t)CARRY = carry + (double)tot;
        }
      } else {
        const CT cj = *(const __attribute__((address_space(3))) CT*)(uintptr_t)(
            sbase + R_OFF + sr * BN * CS + lane * CS);
        bias = cbias(cj, c_ref);
      }
      *(__attribute__((address_space(3))) float*)(uintptr_t)(sbase + C_OFF + sb * BN * 4 + lane * 4) =
          bias;
    }
  };

  // ---- compute stages -----------------------------------------------------------------------
  uint32_t kp[D / 16], vp[D / 32][2];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kp[c] = opaque(sbase + K_OFF + row8_off<D>(lane, 16 * c + 8 * h));
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    vp[d][0] = opaque(sbase + V_OFF + col8_off<D>(lane, d * 32, 0));
    vp[d][1] = opaque(sbase + V_OFF + col8_off<D>(lane, d * 32, 1));
  }
  const uint32_t cp = opaque(sbase + C_OFF + 16 * h);

  // Byte offsets of sub-tile j's rows (K and V share the layout) and bias slice.
  auto kofs = [&](int j) __attribute__((always_inline)) {
    return (uint32_t)((j >> 1) & 3) * TB + (uint32_t)(1 - (j & 1)) * 32 * D * 2;
  };
  auto cofs = [&](int j) __attribute__((always_inline)) {
    return (uint32_t)((j >> 1) & 1) * BN * 4 + (uint32_t)(1 - (j & 1)) * 32 * 4;
  };
  auto qk = [&](f32x16& sacc, uint32_t ko) __attribute__((always_inline)) {
    sacc = zero16();
#pragma unroll
    for (int c = 0; c < D / 16; ++c) sacc = mfma32(lds_ld16(kp[c] + ko), qf[c], sacc);
  };
  auto pv = [&](uint32_t vo) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
        oacc[d] = mfma32(lds_tr8(vp[d][0] + vo + t * 16 * D * 2, vp[d][1] + vo + t * 16 * D * 2),
                         pb[t], oacc[d]);
    }
  };
  // The bias values a lane needs for one sub-tile (keys 8i + 4h + e of its bias slice at co).
  auto bias_vals = [&](f32x4 (&ck)[4], uint32_t co) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ck[i] = lds_ldf4(cp + co + 32 * i);
  };
  // Scores of one sub-tile (bias values ck, first key key0) -> P (bf16 B operands) and the
  // running max / sum, in log2 units relative to m: y = scale log2(e) q.k - (ck + m). The bias
  // and m are added first: both can be large when c_ref lies far from the row's own c (a
  // sequence of strongly closed gates), and for every key that carries weight they nearly
  // cancel, so their sum is exact and the fma rounds only the small result. First: the wave's
  // diagonal sub-tile, which is also its first: mask keys after the query, set m from scratch.
  auto softmax = [&](f32x16& sacc, const f32x4 (&ck)[4], int key0, auto first_tag)
      __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    float mx = -INFINITY;
    if constexpr (kFirst) {  // a rough pass for the row max, then the exact form below
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = fmaf(sacc[4 * i + e], sl2e, -ck[i][e]);
          if ((key0 + 8 * i + 4 * h + e) > qi) x = -INFINITY;
          mx = fmaxf(mx, x);
        }
      }
      m = xhalf_max(mx);
      mx = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = fmaf(sacc[4 * i + e], sl2e, -(ck[i][e] + m));
        if constexpr (kFirst) {
          if ((key0 + 8 * i + 4 * h + e) > qi) x = -INFINITY;
        }
        sacc[4 * i + e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = xhalf_max(mx);
    if constexpr (!kFirst) {
      // scores are already relative to m; raise m only when a row exceeds it by kFwdLazy
      const bool raise = mx > kFwdLazy;
      if (__any(raise)) {
        const float dm = raise ? mx : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-dm);
        m += dm;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] -= dm;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = __builtin_amdgcn_exp2f(sacc[e]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pb[t] = pack_c_half(sacc, t);
      lsum = rowsum_bf16x8(pb[t], lsum);  // l sums the same rounded P that meets V
    }
  };

  // ---- fused scan: prefix sums of the window [w0, q_last], c of this workgroup's queries --------
  // (all of its global loads and stores complete before the first untracked copy is issued)
  if constexpr (kLogF) {
    double part = 0.0;  // sum of log f over [0, w0), then over the wave's 64 window positions
#pragma unroll 8
    for (int l = tid; l < w0; l += NT) part += (double)LF[l];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) part += __shfl_xor(part, off, 64);
    double x = (tid < 256 && w0 + tid <= q_last) ? (double)LF[w0 + tid] : 0.0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 0) *(lds_d*)(uintptr_t)(sbase + RED_OFF + wave * 8) = part;
    if (tid == 0) *(lds_d*)(uintptr_t)CARRY = 0.0;  // older tiles start from key 0
    if (lane == 63 && wave < 4) *(lds_d*)(uintptr_t)(sbase + RED_OFF + 64 + wave * 8) = x;
    __syncthreads();
    double base = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) base += *(const lds_d*)(uintptr_t)(sbase + RED_OFF + w * 8);
    if (tid < 256) {
      double pre = base;
      for (int w = 0; w < wave; ++w) pre += *(const lds_d*)(uintptr_t)(sbase + RED_OFF + 64 + w * 8);
      *(lds_d*)(uintptr_t)(sbase + W_OFF + tid * 8) = pre + x;
    }
    __syncthreads();
    if (tid < 256 && q0 + tid <= q_last)
      Cout[q0 + tid] = (CT)*(const lds_d*)(uintptr_t)(sbase + W_OFF + (q0 - w0 + tid) * 8);
  }

  // ---- prologue: tile 0 through registers; copies of K(1), K(2), V(1), c(1), c(2) -------------
  {
    const int k0 = kt_last * BN;
    if constexpr (kPre) {
      stage_tile(K, k_alpha, pro.k_norm != 0, K_OFF, 0, 0);
      stage_tile(V, v_alpha, false, V_OFF, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int idx = tid + i * NT;
        const int key = k0 + idx / CPR, cc = idx % CPR;
        lds_store8<D>((bf16_t*)(smem + K_OFF), idx / CPR, cc * 8, ld16_or_zero<D>(K, key, L, cc * 8));
        lds_store8<D>((bf16_t*)(smem + V_OFF), idx / CPR, cc * 8, ld16_or_zero<D>(V, key, L, cc * 8));
      }
    }
    if (tid < BN) {
      const int key = k0 + tid;
      float bias = 0.f;
      if constexpr (kLogF) {
        if (key < L)
          bias = (float)((*(const lds_d*)(uintptr_t)(sbase + W_OFF + (key - w0) * 8) -
                          *(const lds_d*)(uintptr_t)P_REF) * 1.4426950408889634);
      } else {
        bias = key < L ? cbias(C[key], c_ref) : 0.f;
      }
      ((float*)(smem + C_OFF))[tid] = bias;
    }
    if constexpr (kPre) {
      if (1 < n_t) {
        stage_tile(K, k_alpha, pro.k_norm != 0, K_OFF, 1, 1);
        stage_tile(V, v_alpha, false, V_OFF, 1, 1);
      }
      if (2 < n_t) stage_tile(K, k_alpha, pro.k_norm != 0, K_OFF, 2, 2);
      if (1 < n_t) copy_c(1, 1);
      if (2 < n_t) copy_c(2, 2);
    } else {
      if (1 < n_t) {
        copy_kv(k_rs, K_OFF, 1, 1);
        copy_kv(v_rs, V_OFF, 1, 1);
        copy_c(1, 1);
      }
      if (2 < n_t) {
        copy_kv(k_rs, K_OFF, 2, 2);
        copy_c(2, 2);
      }
    }
    bar_vm<0>();
  }

  // ---- phase A: the diagonal band, tiles 0..3 -----------------------------------------------
  f32x16 sa, sb;
  const int n_a = n_t < 4 ? n_t : 4;
  for (int t = 0; t < n_a; ++t) {
    start_copies(t, (t + 3) & 3, (t + 2) & 3, (t + 3) & 3);
    convert_c(t, (t + 1) & 3, (t + 1) & 1);
    if (active) {
#pragma unroll 1
      for (int s = 0; s < 2; ++s) {
        const int j = 2 * t + s;
        if (j > j0) pv(kofs(j - 1));
        if (j >= j0) {
          f32x4 ck[4];
          bias_vals(ck, cofs(j));
          qk(sa, kofs(j));
          const int key0 = (2 * kt_last + 1 - j) * 32;
          if (j == j0) softmax(sa, ck, key0, First{});
          else softmax(sa, ck, key0, Rest{});
        }
      }
    }
    bar_vm<0>();
  }

  // ---- phase B: tiles 4..n_t-1, every wave past its diagonal --------------------------------
  // One step: P(j-1)V into O, softmax of sub-tile j (scores in sc, bias values ck), S(j+1) into
  // sn. The exponentials are taken against the current m before the lazy-raise test; only when a
  // row max rose by more than kFwdLazy (rare) are they taken again after the raise. The common
  // path is one straight-line block, so the scheduler can interleave the softmax arithmetic with
  // the step's matrix products.
  auto step = [&](f32x16& sc, f32x16& sn, const f32x4 (&ck)[4], uint32_t vo, uint32_t ko, bool next)
      __attribute__((always_inline)) {
    pv(vo);
    f32x16 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = fmaf(sc[4 * i + e], sl2e, -(ck[i][e] + m));
        sc[4 * i + e] = x;
        p[4 * i + e] = __builtin_amdgcn_exp2f(x);
      }
    }
    bf16x8 nb[2];
    float ps = 0.f;  // this lane's sum of the step's rounded weights
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      nb[t] = pack_c_half(p, t);
      ps = rowsum_bf16x8(nb[t], ps);
    }
    if (next) qk(sn, ko);
    // Keep the common-path exponentials above the branch (the compiler would otherwise sink them
    // into the fall-through path, which splits the block again).
    asm volatile("" : "+v"(nb[0]), "+v"(nb[1]), "+v"(ps));
    interleave_step<6, 2, 4, 11>();
    // The lazy-raise test without a row max: a weight above 2^kFwdLazy (x > kFwdLazy) rounds to
    // at least 2^kFwdLazy in bf16, and a sum of non-negative terms is at least each term, so a
    // lane whose row needs a raise always has ps >= 2^kFwdLazy. The branch then takes the exact
    // row max and raises only the rows whose max exceeds kFwdLazy, as the max test would; a
    // lane let through by the sum alone gets dm = 0, which leaves its values unchanged.
    if (__any(ps >= kFwdLazyW)) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      mx = xhalf_max(mx);
      const bool raise = mx > kFwdLazy;
      const float dm = raise ? mx : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-dm);
      m += dm;
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(sc[e] - dm);
      lsum *= alpha;
      ps = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        nb[t] = pack_c_half(p, t);
        ps = rowsum_bf16x8(nb[t], ps);
      }
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
      }
    }
    pb[0] = nb[0];
    pb[1] = nb[1];
    lsum += ps;
  };
  // Iteration t: sub-tiles 2t (rows 32..63 of tile t) and 2t + 1 (rows 0..31).
  auto tile_body = [&](uint32_t ko_t, uint32_t ko_t1, uint32_t vo_tm1, uint32_t co_t, bool next)
      __attribute__((always_inline)) {
    f32x4 ck[4];
    bias_vals(ck, co_t + 32 * 4);
    step(sa, sb, ck, vo_tm1, ko_t, true);
    bias_vals(ck, co_t);
    step(sb, sa, ck, ko_t + 32 * D * 2, ko_t1 + 32 * D * 2, next);
  };
  auto steady = [&](int t, auto slot_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;  // t % 4
    start_copies(t, (S + 3) & 3, (S + 2) & 3, (S + 3) & 3);
    convert_c(t, (S + 1) & 3, (S + 1) & 1);
    if (active) tile_body(S * TB, ((S + 1) & 3) * TB, ((S + 3) & 3) * TB, (S & 1) * BN * 4, true);
    bar_vm<NCOPY>();
  };
  if (n_t > 4) {
    if (active) qk(sa, kofs(8));
    int t = 4;
    for (; t + 6 < n_t; t += 4) {  // all copies of the four iterations exist; t % 4 == 0
      steady(t, std::integral_constant<int, 0>{});
      steady(t + 1, std::integral_constant<int, 1>{});
      steady(t + 2, std::integral_constant<int, 2>{});
      steady(t + 3, std::integral_constant<int, 3>{});
    }
    for (; t < n_t; ++t) {  // the last few tiles, run-time slots
      start_copies(t, (t + 3) & 3, (t + 2) & 3, (t + 3) & 3);
      convert_c(t, (t + 1) & 3, (t + 1) & 1);
      if (active)
        tile_body(kofs(2 * t + 1), kofs(2 * t + 3), kofs(2 * t - 1), cofs(2 * t + 1), t + 1 < n_t);
      bar_vm<0>();
    }
  }
  if (active) pv(kofs(n_j - 1));

  if (!active) return;
  const float ltot = xhalf_sum(lsum);
  const float inv = 1.0f / ltot;
  if (qi < L && pro.y) {  // output norm and gate (both halves of the row take this branch)
    float ss = 0.f;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) ss = fmaf(oacc[d][e] * inv, oacc[d][e] * inv, ss);
    }
    const float rs = 1.0f / sqrtf(xhalf_sum(ss) / (float)D + pro.out_eps);
    const size_t orow = base + (size_t)qi * D;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = d * 32 + 8 * i + 4 * h;
        float g4[4], y4[4];
        if (pro.g_f32) {
          const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(pro.g) + orow + col);
          g4[0] = t.x; g4[1] = t.y; g4[2] = t.z; g4[3] = t.w;
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(pro.g) + orow + col);
          g4[0] = __uint_as_float(t.x << 16); g4[1] = __uint_as_float(t.x & 0xffff0000u);
          g4[2] = __uint_as_float(t.y << 16); g4[3] = __uint_as_float(t.y & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          y4[j] = oacc[d][4 * i + j] * inv * rs * (pro.out_w ? pro.out_w[col + j] : 1.0f) *
                  sigmoid_f(g4[j]);
        if (pro.g_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(pro.y) + orow + col) =
              make_float4(y4[0], y4[1], y4[2], y4[3]);
        } else {
          const uint32_t lo = (uint32_t)f2bf(y4[0]) | ((uint32_t)f2bf(y4[1]) << 16);
          const uint32_t hi = (uint32_t)f2bf(y4[2]) | ((uint32_t)f2bf(y4[3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(pro.y) + orow + col) = make_uint2(lo, hi);
        }
      }
    }
  }
  if (qi < L) {
    const size_t orow = base + (size_t)qi * D;
#pragma unroll
    for (int d = 0; d < D / 32 && O; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = d * 32 + 8 * i + 4 * h;
        const float y0 = oacc[d][4 * i] * inv, y1 = oacc[d][4 * i + 1] * inv;
        const float y2 = oacc[d][4 * i + 2] * inv, y3 = oacc[d][4 * i + 3] * inv;
        if (o_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(O) + orow + col) = make_float4(y0, y1, y2, y3);
        } else {
          const uint32_t lo = (uint32_t)f2bf(y0) | ((uint32_t)f2bf(y1) << 16);
          const uint32_t hi = (uint32_t)f2bf(y2) | ((uint32_t)f2bf(y3) << 16);
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(O) + orow + col) = make_uint2(lo, hi);
        }
      }
    }
    if (h == 0 && LSE) {
      float crel;  // c_qi - c_q0
      if constexpr (kLogF)
        crel = (float)(*(const lds_d*)(uintptr_t)(sbase + W_OFF + (qi - w0) * 8) -
                       *(const lds_d*)(uintptr_t)P_REF);
      else
        crel = cdiff(C[qi], c_ref);
      LSE[(size_t)bh * L + qi] = (m + __log2f(ltot)) * kLn2 + crel;
    }
  }
}

// ---------------------------------------------------------------------------------------------
constexpr int kF32BM = 32;  // queries per workgroup (one wave, two lanes per query)
constexpr int kF32BN = 32;  // keys per LDS tile

template <int D, typename CT>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     const CT* __restrict__ C,
                                                     float* __restrict__ O, float* __restrict__ LSE,
                                                     int L, float scale) {
  constexpr int DH = D / 2;
  __shared__ float k_s[kF32BN][D];
  __shared__ float v_s[kF32BN][D];
  __shared__ CT c_s[kF32BN];
  const int tid = threadIdx.x;
  const int half = tid >> 5;
  const int bh = blockIdx.y;
  const int q0 = blockIdx.x * kF32BM;
  const int qi = q0 + (tid & 31);
  const size_t base = (size_t)bh * L * D;
  Q += base;
  K += base;
  V += base;
  C += (size_t)bh * L;
  const bool qok = qi < L;
  const CT ci = qok ? C[qi] : (CT)0;
  float q[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    q[d] = qok ? Q[(size_t)qi * D + half * DH + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int q_last = (q0 + kF32BM - 1 < L - 1) ? q0 + kF32BM - 1 : L - 1;
  for (int k0 = 0; k0 <= q_last; k0 += kF32BN) {
    __syncthreads();
    for (int idx = tid; idx < kF32BN * D; idx += 64) {
      const int r = idx / D, d = idx % D;
      const int key = k0 + r;
      k_s[r][d] = key < L ? K[(size_t)key * D + d] : 0.f;
      v_s[r][d] = key < L ? V[(size_t)key * D + d] : 0.f;
    }
    if (tid < kF32BN) c_s[tid] = (k0 + tid) < L ? C[k0 + tid] : (CT)0;
    __syncthreads();
    float s[kF32BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) dot = fmaf(q[d], k_s[j][half * DH + d], dot);
      dot += __shfl_xor(dot, 32, 64);
      const float x = (k0 + j <= qi) ? fmaf(dot, scale, cdiff(ci, c_s[j])) : -INFINITY;
      s[j] = x;
      mx = fmaxf(mx, x);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = expf(m - mnew);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      s[j] = expf(s[j] - mnew);
      ps += s[j];
    }
    l = l * alpha + ps;
    m = mnew;
#pragma unroll
    for (int d = 0; d < DH; ++d) {
      float acc = o[d] * alpha;
#pragma unroll
      for (int j = 0; j < kF32BN; ++j) acc = fmaf(s[j], v_s[j][half * DH + d], acc);
      o[d] = acc;
    }
  }
  if (!qok) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < DH; ++d) O[base + (size_t)qi * D + half * DH + d] = o[d] * inv;
  if (half == 0 && LSE) LSE[(size_t)bh * L + qi] = m + logf(l);
}

template <int D, typename CT>
void go_fwd_bf16(const void* q, const void* k, const void* v, const void* c, void* o, bool o_f32,
                 float* lse, int64_t BH, int64_t L, float scale, const SkipArgs& skip,
                 const FwdPro& pro, hipStream_t s) {
  const int n_qt = (int)((L + 255) / 256);
  if (pro.k_alpha || pro.v_alpha || pro.k_norm)
    hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, CT, false, true>), dim3((unsigned)(n_qt * BH)),
                       dim3(512), 0, s, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                       (const CT*)c, (const float*)nullptr, (CT*)nullptr, o, lse, skip.q_skip,
                       skip.q_order, (int)L, (int)BH, n_qt, scale * kLog2e, (int)o_f32, pro);
  else
    hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, CT, false, false>), dim3((unsigned)(n_qt * BH)),
                       dim3(512), 0, s, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                       (const CT*)c, (const float*)nullptr, (CT*)nullptr, o, lse, skip.q_skip,
                       skip.q_order, (int)L, (int)BH, n_qt, scale * kLog2e, (int)o_f32, pro);
}

template <int D, typename CT>
void go_fwd_bf16_logf(const void* q, const void* k, const void* v, const float* log_f, void* c_out,
                      void* o, bool o_f32, float* lse, int64_t BH, int64_t L, float scale,
                      hipStream_t s) {
  const int n_qt = (int)((L + 255) / 256);
  hipLaunchKernelGGL((fwd_bf16_pipe_kernel<D, CT, true, false>), dim3((unsigned)(n_qt * BH)), dim3(512),
                     0, s, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const CT*)nullptr,
                     log_f, (CT*)c_out, o, lse, (const int32_t*)nullptr, (const int32_t*)nullptr,
                     (int)L, (int)BH, n_qt, scale * kLog2e, (int)o_f32, FwdPro());
}

template <int D, typename CT>
void go_fwd_f32(const float* q, const float* k, const float* v, const void* c, float* o,
                float* lse, int64_t BH, int64_t L, float scale, hipStream_t s) {
  const dim3 grid((unsigned)((L + kF32BM - 1) / kF32BM), (unsigned)BH);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CT>), grid, dim3(64), 0, s, q, k, v, (const CT*)c, o, lse,
                     (int)L, scale);
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, CPtr c, void* o,
                           bool o_f32, float* lse, int64_t BH, int64_t L, int64_t D, float scale,
                           const SkipArgs& skip, hipStream_t s, const ProFwdArgs* pa) {
  FwdPro pro;
  if (pa) {
    pro.q_w = pa->q_w;
    pro.q_eps = pa->q_eps;
    pro.q_norm = pa->q_norm ? 1 : 0;
    pro.g = pa->g;
    pro.g_f32 = pa->g_f32 ? 1 : 0;
    pro.out_w = pa->out_w;
    pro.out_eps = pa->out_eps;
    pro.y = pa->y;
    pro.k_alpha = pa->k_alpha;
    pro.v_alpha = pa->v_alpha;
    pro.k_norm = pa->k_norm ? 1 : 0;
    pro.k_w = pa->k_w;
    pro.k_eps = pa->k_eps;
  }
  if (D == 64) {
    if (c.f64) go_fwd_bf16<64, double>(q, k, v, c.p, o, o_f32, lse, BH, L, scale, skip, pro, s);
    else go_fwd_bf16<64, float>(q, k, v, c.p, o, o_f32, lse, BH, L, scale, skip, pro, s);
  } else {
    if (c.f64) go_fwd_bf16<128, double>(q, k, v, c.p, o, o_f32, lse, BH, L, scale, skip, pro, s);
    else go_fwd_bf16<128, float>(q, k, v, c.p, o, o_f32, lse, BH, L, scale, skip, pro, s);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_logf(const void* q, const void* k, const void* v, const float* log_f,
                                CPtr c_out, void* o, bool o_f32, float* lse, int64_t BH, int64_t L,
                                int64_t D, float scale, hipStream_t s) {
  void* co = const_cast<void*>(c_out.p);
  if (D == 64) {
    if (c_out.f64) go_fwd_bf16_logf<64, double>(q, k, v, log_f, co, o, o_f32, lse, BH, L, scale, s);
    else go_fwd_bf16_logf<64, float>(q, k, v, log_f, co, o, o_f32, lse, BH, L, scale, s);
  } else {
    if (c_out.f64) go_fwd_bf16_logf<128, double>(q, k, v, log_f, co, o, o_f32, lse, BH, L, scale, s);
    else go_fwd_bf16_logf<128, float>(q, k, v, log_f, co, o, o_f32, lse, BH, L, scale, s);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, CPtr c, float* o,
                          float* lse, int64_t BH, int64_t L, int64_t D, float scale, hipStream_t s) {
  if (D == 64) {
    if (c.f64) go_fwd_f32<64, double>(q, k, v, c.p, o, lse, BH, L, scale, s);
    else go_fwd_f32<64, float>(q, k, v, c.p, o, lse, BH, L, scale, s);
  } else {
    if (c.f64) go_fwd_f32<128, double>(q, k, v, c.p, o, lse, BH, L, scale, s);
    else go_fwd_f32<128, float>(q, k, v, c.p, o, lse, BH, L, scale, s);
  }
  return hipGetLastError();
}

}  // namespace fox
