// fox_device.h — device-side building blocks shared by the gfx950 kernels of libfox.
//
// Matrix-core conventions (CDNA4, wave64). For v_mfma_f32_32x32x16_bf16, lane l with
// h = l / 32 supplies
//   A[m = l % 32][k = 8h .. 8h+7]     (8 bf16)
//   B[k = 8h .. 8h+7][n = l % 32]     (8 bf16)
// and receives the fp32 accumulator values
//   C[m = 8i + 4h + j][n = l % 32]    in slot 4i + j   (i, j = 0..3).
// Only two facts are relied on: A and B pair their k slots identically, and the C layout above.
// A C tile therefore already sits in B-operand form with k = its row index: the 8 values of
// slots 8t .. 8t+7 (t = 0, 1) are B's k slots for rows {16t + 4h + 0..3, 16t + 8 + 4h + 0..3}.
// Any A operand paired with such a B must present the same rows in the same slots; the
// helpers below read exactly that row set.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fox {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage type of bfloat16 in global memory and LDS

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// c_a - c_b, and log2(e) (c_a - c_b), from the cumulative log decay in fp32 or fp64: the fp64
// form subtracts exactly and rounds once, so the difference keeps its precision however large
// |c| has grown (hard resets drive c to -1e5 and beyond, where fp32 values are 2^-6 apart).
__device__ __forceinline__ float cdiff(float a, float b) { return a - b; }
__device__ __forceinline__ float cdiff(double a, double b) { return (float)(a - b); }
__device__ __forceinline__ float cbias(float a, float b) { return (a - b) * kLog2e; }
__device__ __forceinline__ float cbias(double a, double b) {
  return (float)((a - b) * 1.4426950408889634);
}

// bf16 <-> fp32 (round to nearest even on the way down, via the gfx950 convert instruction).
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

// 8 consecutive bf16 from memory (global or LDS) as an MFMA operand.
__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Pack slots 8t .. 8t+7 of a C tile into a bf16 B operand.
__device__ __forceinline__ bf16x8 pack_c_half(const f32x16& c, int t) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[8 * t + e];
  return r;
}

// ---------------------------------------------------------------------------------------------
// LDS tiles of D bf16 columns (D = 64 or 128), unpadded and XOR-swizzled in 16-byte chunks:
// logical chunk c of row r lives at physical chunk c ^ swz_key(r). The key is chosen so that
// both access patterns the kernels use are free of bank conflicts:
//   row reads   - 16 lanes read the same 16-byte chunk of 16 consecutive rows (ds_read_b128);
//   column reads - 32 lanes read a 4-row x 64-byte block in 8-byte pieces (ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Element offset of logical (row, col) in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 3) ^ swz_key<D>(row))) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte register chunk. A native vector (not HIP's uint4 struct): selects between two chunks
// then stay in registers instead of going through scratch memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Row `row` (0-based, < rows) of a dense [rows x D] bf16 matrix, 8 elements from column col,
// or zeros when row >= rows. The load itself is clamped to the last row, so it is always in
// bounds, and the zero fill is a value select.
template <int D>
__device__ __forceinline__ u32x4 ld16_or_zero(const bf16_t* m, int row, int rows, int col) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(m + (row < rows ? row : rows - 1) * D + col);
  const u32x4 z = {0u, 0u, 0u, 0u};
  return row < rows ? v : z;
}

// Store 16 bytes (8 elements, col a multiple of 8) into a swizzled tile.
template <int D>
__device__ __forceinline__ void lds_store8(bf16_t* base, int row, int col, const u32x4& v) {
  *reinterpret_cast<u32x4*>(base + swz<D>(row, col)) = v;
}

// The Pro block's token shift and key RMSNorm on one 8-element chunk of a row. The separate
// shift pass and the forward's fused tile loads both use these, so their rows hold the same bits:
// the shifted row is a prev + (1 - a) cur, and the norm multiplies it by
// 1 / sqrt(mean of squares + eps) [* w], the sum of squares taken over the D / 8 consecutive
// lanes that hold the row (a butterfly, which leaves the same sum in every lane of the group).
__device__ __forceinline__ float shift_mix(float a, float prev, float cur) {
  return fmaf(a, prev, (1.0f - a) * cur);
}
template <int D>
__device__ __forceinline__ float row_group_sum(float v) {
#pragma unroll
  for (int m = 1; m < D / 8; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
template <int D>
__device__ __forceinline__ float rms_scale(float ss_row, float eps) {
  return rsqrtf(fmaf(ss_row, 1.0f / D, eps));
}
template <int D>
__device__ __forceinline__ void rms_norm8(float (&v)[8], const float* w, int col, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  const float r = rms_scale<D>(row_group_sum<D>(ss), eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= r * (w ? w[col + e] : 1.0f);
}
__device__ __forceinline__ void unpack8(const u32x4& x, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(x[i] << 16);
    v[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack8(const float (&v)[8]) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
  return r;
}

// acc + sum of the 8 bf16 values of v, with v_dot2_f32_bf16 against packed ones (fp32 sums).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float rowsum_bf16x8(const bf16x8& v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// Sum / max across the two half-waves (lanes l and l ^ 32). v_permlane32_swap on two copies of
// v returns, in every lane, the pair {v[l % 32], v[l % 32 + 32]}.
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xhalf_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// ---------------------------------------------------------------------------------------------
// LDS reads from a per-lane base address plus a compile-time offset. A kernel computes each
// lane's swizzled byte address once, hides it from the optimiser with opaque(), and adds only
// constants inside its loops: the constant then folds into the 16-bit offset field of the DS
// instruction, so a read costs no address arithmetic.
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {  // LDS byte address of a __shared__ object
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
__device__ __forceinline__ bf16x8 lds_ld16(uint32_t a) { return *(const lds_bf16x8*)(uintptr_t)a; }
__device__ __forceinline__ f32x4 lds_ldf4(uint32_t a) { return *(const lds_f32x4*)(uintptr_t)a; }
// Per-lane byte offsets inside a swizzled tile, relative to its first row (adding 2 D bytes per
// row moves them down; row blocks of 16 keep the swizzle key, so whole blocks can be added):
//
// row8_off(lane, col): 8 consecutive elements of row lane % 32 from column col (a multiple of
// 8), read with ds_read_b128 - an A operand with m = row and k = column, or a B operand with
// n = row.
//
// col8_off(lane, cbase, second): the two ds_read_b64_tr_b16 reads (second = 0, 1) that form an
// A operand whose k slots are the rows {4h + 0..3, 8 + 4h + 0..3} of the tile at column
// cbase + lane % 32 (cbase a multiple of 32): the transpose of a row read. It pairs with
// pack_c_half(., t) of a C tile whose rows are the tile rows 16 t ... ds_read_b64_tr_b16 works on
// groups of 16 lanes: lane 4a + b of a group receives element b of the 8-byte pieces read by the
// group's lanes a, a + 4, a + 8, a + 12 (in that order). So when group lane s reads columns
// col0 + 4 (s % 4) .. + 3 of row row0 + s / 4, group lane i receives column col0 + i of rows
// row0 .. row0 + 3.
template <int D>
__device__ __forceinline__ uint32_t row8_off(int lane, int col) {
  return (uint32_t)swz<D>(lane & 31, col) * 2;
}
template <int D>
__device__ __forceinline__ uint32_t col8_off(int lane, int cbase, int second) {
  const int row = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * second;
  const int col = cbase + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return (uint32_t)swz<D>(row, col) * 2;
}
// The two col8 reads as one operand. Whole-vector shuffle and bit cast only: a
// __builtin_bit_cast of a single element of a __bf16 vector is miscompiled by this toolchain
// (every element reads element 0).
__device__ __forceinline__ bf16x8 lds_tr8(uint32_t a0, uint32_t a1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
  const i16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

// Inclusive prefix sum of one float per lane over the wave (lane 0 first), on DPP moves only (no
// LDS round trips): a Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8, lanes
// without a source reading 0), then row 0's total added to row 1 and row 2's to row 3
// (row_bcast:15), then lane 31's prefix added to rows 2 and 3 (row_bcast:31). Lanes a step does
// not write read the zero passed as the old value.
template <int kCtrl, int kRowMask, bool kBound>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                               kRowMask, 0xf, kBound));
}
__device__ __forceinline__ float wave_scan_incl(float x) {
  x += dpp_move<0x111, 0xf, true>(x);  // row_shr:1
  x += dpp_move<0x112, 0xf, true>(x);  // row_shr:2
  x += dpp_move<0x114, 0xf, true>(x);  // row_shr:4
  x += dpp_move<0x118, 0xf, true>(x);  // row_shr:8
  x += dpp_move<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_move<0x143, 0xc, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Register-file hints for the allocator (no instruction is emitted): accumulators only the
// matrix cores touch stay in AGPRs, MFMA results the vector ALU reads stay in VGPRs, so no
// v_accvgpr moves are needed between them.
__device__ __forceinline__ void pin_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void pin_vgpr(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_agpr(bf16x8& x) { asm volatile("" : "+a"(x)); }

// ---------------------------------------------------------------------------------------------
// Global -> LDS copies issued as inline assembly. The compiler does not track them, so it never
// inserts the conservative vmcnt(0) it would place before every LDS read that might alias a
// tracked copy; the kernel instead waits explicitly with bar_vm<N>(), which lets the N most
// recently issued copies stay in flight across the barrier (vector memory loads complete in
// issue order). A compiler-visible vector memory load issued after a copy leaves this correct,
// since the loads still complete in order, but the compiler's wait for that load's data then
// also waits for the copy; the kernels keep such loads out of their pipelined loops, or issue
// them before the iteration's copies.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: `bytes` bytes from `base`, reads at or past the end return zero.
__device__ __forceinline__ i32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);  // stride 0
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}
// Each active lane copies 16 bytes from byte offset voff of the buffer to LDS byte address
// lds + 16 * lane (lds must be wave-uniform). M0 is saved and restored.
__device__ __forceinline__ void copy16_to_lds(uint32_t lds, uint32_t voff, i32x4 rs) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}
// Same with 4 bytes per lane (LDS byte address lds + 4 * lane).
__device__ __forceinline__ void copy4_to_lds(uint32_t lds, uint32_t voff, i32x4 rs) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}
// Workgroup barrier after this wave's LDS accesses have completed and all but its N most recent
// copies have landed.
template <int N>
__device__ __forceinline__ void bar_vm() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------------------------
// XCD-aware work order. The hardware places workgroup `bid` on XCD bid % 8, and each XCD has its
// own L2. A grid of n_levels x BH items (levels issued one after another, most work first; a level
// holds one item per (b, h)) is mapped so that every head keeps to one XCD where the level's
// positions allow it: head h's home XCD is h % 8; a level position on XCD x takes the next head
// at home on x, and the positions left over (when BH is not a multiple of 8) take the heads left
// over, both in order. Within each level this is a bijection between positions and heads, so the
// grid covers every item once whatever the placement; only the cache reuse depends on it. With
// 12 heads, heads 0..7 stay on their XCD and heads 8..11 alternate between two XCDs level by level
// (instead of every head alternating and every XCD streaming three heads).
__device__ __forceinline__ void xcd_item(int bid, int BH, int& bh, int& level) {
  constexpr int NX = 8;
  level = bid / BH;
  const int p = bid - level * BH;  // position within the level
  const int b8 = (level * BH) % NX;  // XCD of the level's first position
  auto first_pos = [&](int y) { return (y - b8 + NX) % NX; };  // first position on XCD y
  auto n_pos = [&](int y) { const int q = first_pos(y); return BH > q ? (BH - q + NX - 1) / NX : 0; };
  auto n_home = [&](int y) { return y < BH ? (BH - 1 - y) / NX + 1 : 0; };
  const int x = (b8 + p) % NX;
  const int k = (p - first_pos(x)) / NX;  // rank of p among the level's positions on XCD x
  if (k < n_home(x)) {
    bh = x + NX * k;
    return;
  }
  int r = 0;  // rank of p among the left-over positions before it
  for (int y = 0; y < NX; ++y) {
    const int q = first_pos(y);
    const int before = p > q ? (p - q + NX - 1) / NX : 0;
    r += before > n_home(y) ? before - n_home(y) : 0;
  }
  for (int y = 0; y < NX; ++y) {  // the r-th left-over head: y + NX j for n_pos(y) <= j < n_home(y)
    const int extra = n_home(y) - n_pos(y);
    if (extra > 0) {
      if (r < extra) {
        bh = y + NX * (n_pos(y) + r);
        return;
      }
      r -= extra;
    }
  }
  bh = p;  // not reached: the left-over positions and heads are equal in number
}

}  // namespace fox
