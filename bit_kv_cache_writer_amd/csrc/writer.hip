// Fused cache writer for gfx950 (QuantMLA Figure 8 caption: a packed copy of
// every incoming token plus BF16 retention of sink/recent tokens; RAQ-MLA
// appendix Table 5: per-token 128-channel latent groups with FP16 scale/min,
// 0.94-quantile |x| clipping for the 2-bit latent, per-(channel, page) 4-bit
// k_R with FP16 scale/min).
//
// One workgroup (8 waves) per (sequence, cache page touched by the call), or
// three / five per page when a call brings many tokens into few pages (a
// page's tokens are then dealt to them in runs of 8, and the first one of a
// page does all of its k_R and tail work below, and no tokens when the page
// completes):
//   * without the clip each wave quantizes two whole latent tokens at a
//     time, one per half-wave, two pairs per loop trip, each pair's rows
//     requested one pair ahead: lane l owns channels 16c..16c+15 (c = l mod
//     32) of its half's token, so a 128-channel group is 8 lanes and its
//     min/max take three DPP steps, and the group's metadata arithmetic is
//     shared by the two tokens; codes are packed in registers and stored as
//     two dwords (4-bit) or one dword (2-bit) per lane;
//   * with the INT2 clip each wave quantizes one whole token at a time (three
//     per loop trip, rows requested two tokens ahead), lane l owning channels
//     8l..8l+7: a group is 16 lanes, and the clip takes its order statistics
//     by a binary search over each lane's sorted keys, counting with one
//     ballot per column;
//   * if the page becomes full in this call the workgroup quantizes its k_R
//     per channel over the P tokens (tail buffer for tokens written by earlier
//     calls, input rows for the new ones);
//   * only the workgroup of the sequence's first touched page reads the tail
//     buffer, and it alone then writes the tail rows of a page left
//     incomplete, after a barrier -- so no workgroup reads tail rows another
//     one overwrites.
// With the latent transform and no clipping, a page has four workgroups, one
// per 128-channel latent group: each forms its quarter of y = A_c x (a quarter
// of A_c) and caches that group, which is quantized on its own; the first of
// them also does the page's k_R work.
// The quantizer's arithmetic is IEEE fp32 with each operation rounded on its
// own (contraction off), so codes and metadata are reproducible bit for bit.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "geometry.h"

#pragma clang fp contract(off)

namespace mla {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

struct WriterParams {
  const uint16_t* a_c;  // latent transform, bf16 [512][512] row-major (transforming writer only)
  const uint16_t* c_kv;
  const uint16_t* k_r;
  const int32_t* cu_new;
  const int32_t* seqlens_before;
  const int32_t* block_table;
  uint8_t* pool;
  uint16_t* sink;
  uint16_t* ring;
  uint16_t* tail;
  int32_t batch, total_new, max_pages, num_pool_pages, pages_per_seq_grid;
  int32_t token_split;  // plain writer: workgroups per page (1, 3 or 5), tokens dealt between them
  int32_t P, bits, sink_n, local;
  int32_t clip_lo, clip_hi;
  float clip_frac;
  int64_t latent_row, latent_meta_off, rope_codes_off, rope_meta_off, page_bytes;
};

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// Workgroup barrier for LDS traffic only (__syncthreads would also wait for
// every outstanding global load, prefetches included).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// fp32 -> bf16 bits, nearest with ties to even (finite values)
__device__ inline uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// -0 -> +0, every other value unchanged: -0 + +0 is +0 under round to
// nearest, x + 0 = x otherwise (one add; contraction is off in this file).
__device__ inline float canon_zero(float x) { return x + 0.0f; }

__device__ inline float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Directed fp16 rounding by the conversion itself: the wave's MODE register
// (its four round-mode bits: fp32 and fp16/fp64, 0 nearest-even, 1 toward
// +inf, 2 toward -inf) is set for one v_cvt_f16_f32 and put back to
// nearest-even, all inside one asm block so that no other instruction runs
// under the directed mode; two wait states follow each mode change.  The
// unsigned min takes an infinity (a value beyond 65504 in that direction)
// back to the largest finite fp16.  x is not -0 (the callers normalize it).
#define MLA_CVT_F16_DIRECTED(MODE)                                   \
  "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), " MODE "\n\t"     \
  "s_nop 1\n\t"                                                    \
  "v_cvt_f16_f32_e32 %0, %1\n\t"                                   \
  "s_nop 1\n\t"                                                    \
  "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 4), 0"

// Largest fp16 <= x (-65504 for x below it).
__device__ inline uint16_t f16_round_down(float x) {
  uint32_t h;
  asm volatile(MLA_CVT_F16_DIRECTED("10") : "=v"(h) : "v"(x));
  return static_cast<uint16_t>(min(h & 0xFFFFu, 0xFBFFu));
}

// Smallest fp16 >= x (x >= 0; 65504 for x above it).
__device__ inline uint16_t f16_round_up(float x) {
  uint32_t h;
  asm volatile(MLA_CVT_F16_DIRECTED("5") : "=v"(h) : "v"(x));
  return static_cast<uint16_t>(min(h & 0xFFFFu, 0x7BFFu));
}
#undef MLA_CVT_F16_DIRECTED

// span / d, correctly rounded, for d = 3 or 15 (rd = rn(1 / d)) and
// 0 <= span <= 2^20: the product with rd and one FMA correction of it give
// the IEEE quotient for every fp32 span in that range (checked against the
// division one by one).  Spans of in-range inputs stay below 2^18, and above
// 15 * 65504 the scale saturates whatever the last bit.
__device__ inline float div_levels(float span, float d, float rd) {
  const float q0 = span * rd;
  const float e = __builtin_fmaf(-q0, d, span);
  return __builtin_fmaf(e, rd, q0);
}

// rint of the correctly rounded quotient d / s (d >= 0, s > 0, the quotient
// below 32 in every use).  d times the hardware reciprocal is within 2 ulp of
// the correctly rounded quotient; more than 1e-5 (over 4 ulp below 32) from a
// half-integer, both round to the same integer; otherwise (rare) the IEEE
// division decides.  Bit-identical to rintf(d / s).
__device__ inline float rint_div(float d, float s, float rcp_s) {
  const float qa = d * rcp_s;
  float r = rintf(qa);
  if (__builtin_expect(fabsf(qa - floorf(qa) - 0.5f) <= 1e-5f, 0)) r = rintf(d / s);
  return r;
}

// Eight 4-bit codes (integer-valued floats in [0, 15]) packed, code i in
// bits 4i .. 4i + 3: the even codes go to the bytes of one dword and the odd
// ones to another by v_cvt_pk_u8_f32 (exact for integers), then one shift-or
// interleaves them.
__device__ inline uint32_t pack_nibbles(const float (&c)[8]) {
  uint32_t even = 0, odd = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    even = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * k], k, even);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * k + 1], k, odd);
  }
  return even | (odd << 4);
}

// Codes of 8 values v[i] with offset m and step s: for s > 0 the same codes
// as min(max(rint_div(v - m, s), 0), levels); s = 0 gives 0 (the reciprocal
// is replaced by 0, so every quotient is 0).  The fast quotient is checked
// for nearness to a half-integer once for the 8 values (|qa - rint(qa)| at
// least 0.5 - 1e-5 is the same set as rint_div's test), and only a row with
// such a value takes the IEEE division.  Codes are packed `bits` apiece.
// The clamp to [0, levels] is never active for finite values in the stated
// range, so none is applied: m is at most the group's minimum (rounded
// down), so v - m >= 0; and s is at least fl(span / levels) (rounded up to
// fp16), span = fl(max - m) bounds every fl(v - m), so each quotient, fast
// (a reciprocal within 1 ulp) or divided, is at most levels (1 + 2^-22)
// and rounds to at most levels.
__device__ inline uint32_t pack_codes(const float (&v)[8], float m, float s, float rcp_s, int bits) {
  const float rc = s > 0.0f ? rcp_s : 0.0f;
  float r[8];
  float dev = 0.0f;  // largest |qa - rint(qa)| of the 8 (a max3 chain)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float qa = (v[i] - m) * rc;
    r[i] = rintf(qa);
    dev = fmaxf(dev, fabsf(qa - r[i]));
  }
  if (__builtin_expect(dev >= 0.49999f, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = rint_div(v[i] - m, s, rcp_s);
  }
  if (bits == 4) return pack_nibbles(r);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= static_cast<uint32_t>(r[i]) << (bits * i);
  return packed;
}

// DPP lane move within 16-lane rows (bound_ctrl set: the fused form).
template <int kCtrl>
__device__ inline int dpp_key(int k) {
  return __builtin_amdgcn_mov_dpp(k, kCtrl, 0xF, 0xF, true);
}

// Min and max of a lane's 8 values, then over each 16-lane row by DPP lane
// moves fused into v_min_f32 / v_max_f32 (swap neighbours, swap pairs, rotate
// the row by 4 and by 8): 16 VALU instructions.  Written out so that no
// canonicalizing copies are inserted around the float min / max (the values
// are never NaN); the s_nop keep two wait states between a VGPR's write and
// its DPP read.  Which zero a min or max of -0 and +0 returns is left open
// (the callers normalize it).
__device__ inline void group_minmax(const float (&x)[8], float& mn, float& mx) {
#define MLA_DPP_STEP(CTRL)                                                   \
  "s_nop 0\n\t"                                                             \
  "v_min_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_max_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
  asm volatile("v_min3_f32 %0, %2, %3, %4\n\t"
               "v_max3_f32 %1, %2, %3, %4\n\t"
               "v_min3_f32 %0, %0, %5, %6\n\t"
               "v_max3_f32 %1, %1, %5, %6\n\t"
               "v_min3_f32 %0, %0, %7, %8\n\t"
               "v_max3_f32 %1, %1, %7, %8\n\t"
               "v_min_f32 %0, %0, %9\n\t"
               "v_max_f32 %1, %1, %9\n\t"
               "s_nop 0\n\t"
               MLA_DPP_STEP("quad_perm:[1,0,3,2]") MLA_DPP_STEP("quad_perm:[2,3,0,1]")
               MLA_DPP_STEP("row_ror:4") MLA_DPP_STEP("row_ror:8")
               : "=&v"(mn), "=&v"(mx)
               : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
#undef MLA_DPP_STEP
}
// The same for 16 values a lane and 8-lane groups (two tokens per wave, 16
// channels a lane): swap neighbours, swap pairs, mirror the half-row; 22 VALU
// instructions for two tokens.
__device__ inline void group_minmax16(const float (&x)[16], float& mn, float& mx) {
#define MLA_DPP_STEP(CTRL)                                                   \
  "s_nop 0\n\t"                                                             \
  "v_min_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_max_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
  asm volatile("v_min3_f32 %0, %2, %3, %4\n\t"
               "v_max3_f32 %1, %2, %3, %4\n\t"
               "v_min3_f32 %0, %0, %5, %6\n\t"
               "v_max3_f32 %1, %1, %5, %6\n\t"
               "v_min3_f32 %0, %0, %7, %8\n\t"
               "v_max3_f32 %1, %1, %7, %8\n\t"
               "v_min3_f32 %0, %0, %9, %10\n\t"
               "v_max3_f32 %1, %1, %9, %10\n\t"
               "v_min3_f32 %0, %0, %11, %12\n\t"
               "v_max3_f32 %1, %1, %11, %12\n\t"
               "v_min3_f32 %0, %0, %13, %14\n\t"
               "v_max3_f32 %1, %1, %13, %14\n\t"
               "v_min3_f32 %0, %0, %15, %16\n\t"
               "v_max3_f32 %1, %1, %15, %16\n\t"
               "v_min_f32 %0, %0, %17\n\t"
               "v_max_f32 %1, %1, %17\n\t"
               "s_nop 0\n\t"
               MLA_DPP_STEP("quad_perm:[1,0,3,2]") MLA_DPP_STEP("quad_perm:[2,3,0,1]")
               MLA_DPP_STEP("row_half_mirror")
               : "=&v"(mn), "=&v"(mx)
               : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
                 "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]));
#undef MLA_DPP_STEP
}
// Packed signed 16-bit pairs, reduced over the whole wave per half: DPP lane
// moves within 16-lane rows, then the swaps of rows and of 32-lane halves.
// (The swapped dwords are taken out as plain 32-bit values before they are
// reinterpreted: a bit cast straight from an element of the returned pair
// reads the first element.)
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
template <int kCtrl>
__device__ inline i16x2 dpp_i16x2(i16x2 v) {
  return __builtin_bit_cast(i16x2, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
// Minimum over a lane and its DPP partner of one of two packed-key dwords:
// the lane keeps `hi` when `up` is set, else `lo`, and sends the other to the
// partner, whose `up` is the opposite (one step of a reduce-scatter).
template <int kCtrl>
__device__ inline uint32_t scatter_min(bool up, uint32_t lo, uint32_t hi) {
  const uint32_t keep = up ? hi : lo, send = up ? lo : hi;
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(i16x2, keep),
                                                                dpp_i16x2<kCtrl>(__builtin_bit_cast(i16x2, send))));
}
// Packed 16-bit minimum over the lanes l, l ^ 8, l ^ 16, ... (the lanes that
// agree in their three low bits): the 8-lane step inside a row, then the
// swaps of 16-lane rows and of 32-lane halves.
__device__ inline uint32_t min_over_octets(uint32_t u) {
  u = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(i16x2, u),
                                                             dpp_i16x2<0x128>(__builtin_bit_cast(i16x2, u))));
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  u = __builtin_bit_cast(uint32_t,
                         __builtin_elementwise_min(__builtin_bit_cast(i16x2, a0), __builtin_bit_cast(i16x2, a1)));
  const auto c = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t c0 = c[0], c1 = c[1];
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_min(__builtin_bit_cast(i16x2, c0), __builtin_bit_cast(i16x2, c1)));
}

// Min / max of integers over the whole wave: the row steps of group_minmax,
// then the swaps of 16-lane rows and of 32-lane halves.
__device__ inline int wave_min_i32(int v) {
  v = min(v, dpp_key<0xB1>(v));
  v = min(v, dpp_key<0x4E>(v));
  v = min(v, dpp_key<0x124>(v));
  v = min(v, dpp_key<0x128>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  v = min(static_cast<int>(a[0]), static_cast<int>(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  return min(static_cast<int>(c[0]), static_cast<int>(c[1]));
}
__device__ inline int wave_max_i32(int v) {
  v = max(v, dpp_key<0xB1>(v));
  v = max(v, dpp_key<0x4E>(v));
  v = max(v, dpp_key<0x124>(v));
  v = max(v, dpp_key<0x128>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  v = max(static_cast<int>(a[0]), static_cast<int>(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  return max(static_cast<int>(c[0]), static_cast<int>(c[1]));
}

// A lane's 8 clip keys, two per dword: 15-bit keys (|x| as bf16 bits), so
// that each packed 16-bit min / max handles two of them.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ inline void ce_u16x2(u16x2& a, u16x2& b) {
  const u16x2 hi = __builtin_elementwise_max(a, b), lo = __builtin_elementwise_min(a, b);
  a = hi;
  b = lo;
}

// Sorts a lane's 8 keys into descending order: column j (0..7) is the low
// half of u[j] for j < 4, the high half of u[j - 4] otherwise.  The low and
// the high halves are first sorted each on their own (one 5-comparator
// network running on both), then merged by one bitonic step (each low key
// against the high keys in reverse order: the larger four and the smaller
// four), and both fours are finished by a bitonic half-cleaner, again side by
// side.  (Checked on all 256 zero-one inputs and on random inputs with ties.)
__device__ inline void sort8_packed(u16x2 (&u)[4]) {
  ce_u16x2(u[0], u[1]);
  ce_u16x2(u[2], u[3]);
  ce_u16x2(u[0], u[2]);
  ce_u16x2(u[1], u[3]);
  ce_u16x2(u[1], u[2]);
  const u16x2 r3 = u[3].yx, r2 = u[2].yx;
  const u16x2 m0 = __builtin_elementwise_max(u[0], r3), n0 = __builtin_elementwise_min(u[0], r3);
  const u16x2 m1 = __builtin_elementwise_max(u[1], r2), n1 = __builtin_elementwise_min(u[1], r2);
  u[0] = __builtin_shufflevector(m0, n0, 0, 2);
  u[1] = __builtin_shufflevector(m1, n1, 0, 2);
  u[2] = __builtin_shufflevector(m1, n1, 1, 3);
  u[3] = __builtin_shufflevector(m0, n0, 1, 3);
  ce_u16x2(u[0], u[2]);
  ce_u16x2(u[1], u[3]);
  ce_u16x2(u[0], u[1]);
  ce_u16x2(u[2], u[3]);
}
__device__ inline uint32_t key_column(const u16x2 (&u)[4], int j) { return j < 4 ? u[j].x : u[j - 4].y; }
__device__ inline uint32_t packed_bits(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// The smallest key v in [lo, hi] with fewer than `need` (>= 1) of the
// wave's 512 keys above it (lo, hi wave-uniform and enclosing that key, with
// at least `need` keys at or above lo), by binary lifting: base, starting at
// lo - 1, is the largest key known to have at least `need` keys above it;
// steps of 2^(k-1), ..., 1 with 2^k >= hi - lo + 1 probe base + step and move
// base there when the probe has at least `need` keys above it, and the answer
// is base + 1.  Probes stay below 2 hi - lo <= 0xFFFE, inside the 16-bit
// compares.  Each probe counts the keys above it with one ballot per column
// of the lanes' sorted keys: column j's set of lanes is part of column
// j - 1's, so an empty column ends the count (fewer than need), and so does
// the count reaching need.  Per column: a 16-bit compare into a lane mask
// (low halves of u, then of uh = u >> 16), its popcount (SCC: any lane set)
// and the popcount taken from the remaining need - 1 (SCC: borrow, i.e. the
// count reached need).  The step's shift sets SCC while a step is left, so
// the loop needs no compare of its own.
#define MLA_GT_COLUMN(V)                              \
  "v_cmp_gt_u16_e64 %[m], %[" V "], %[t]\n\t"          \
  "s_bcnt1_i32_b64 %[pc], %[m]\n\t"                  \
  "s_cbranch_scc0 .Lnext%=\n\t"                      \
  "s_sub_u32 %[r], %[r], %[pc]\n\t"                  \
  "s_cbranch_scc1 .Labove%=\n\t"
__device__ inline uint32_t wave_bisect_rank(const u16x2 (&u)[4], uint32_t lo, uint32_t hi, int need) {
  const uint32_t need_m1 = static_cast<uint32_t>(need - 1);
  uint32_t uh[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) uh[j] = u[j].y;
  // 2^(k-1) for the smallest k with 2^k >= hi - lo + 1 (0: lo is the answer)
  uint32_t step = hi > lo ? 1u << (31 - __builtin_clz(hi - lo)) : 0u;
  uint32_t base = lo - 1u;
  if (step != 0) {
    uint32_t t, pc, r;
    uint64_t m;
    asm volatile(".Lprobe%=:\n\t"
                 "s_add_u32 %[t], %[base], %[step]\n\t"
                 "v_cmp_gt_u16_e64 %[m], %[u0], %[t]\n\t"
                 "s_bcnt1_i32_b64 %[pc], %[m]\n\t"
                 "s_sub_u32 %[r], %[nm1], %[pc]\n\t"
                 "s_cbranch_scc1 .Labove%=\n\t"
                 MLA_GT_COLUMN("u1") MLA_GT_COLUMN("u2") MLA_GT_COLUMN("u3")
                 MLA_GT_COLUMN("h0") MLA_GT_COLUMN("h1") MLA_GT_COLUMN("h2") MLA_GT_COLUMN("h3")
                 ".Lnext%=:\n\t"
                 "s_lshr_b32 %[step], %[step], 1\n\t"
                 "s_cbranch_scc1 .Lprobe%=\n\t"
                 "s_branch .Ldone%=\n"
                 ".Labove%=:\n\t"
                 "s_mov_b32 %[base], %[t]\n\t"
                 "s_lshr_b32 %[step], %[step], 1\n\t"
                 "s_cbranch_scc1 .Lprobe%=\n"
                 ".Ldone%=:"
                 : [base] "+s"(base), [step] "+s"(step), [t] "=&s"(t), [pc] "=&s"(pc), [r] "=&s"(r), [m] "=&s"(m)
                 : [u0] "v"(packed_bits(u[0])), [u1] "v"(packed_bits(u[1])), [u2] "v"(packed_bits(u[2])),
                   [u3] "v"(packed_bits(u[3])), [h0] "v"(uh[0]), [h1] "v"(uh[1]), [h2] "v"(uh[2]), [h3] "v"(uh[3]),
                   [nm1] "s"(need_m1)
                 : "scc");
  }
  return base + 1u;
}
#undef MLA_GT_COLUMN

// k-th smallest (0-based) of the 512 keys, held 8 per lane in descending
// order: the smallest v with fewer than 512 - k keys above it, by a binary
// search between two keys that enclose it.  Each lane holds j + 1 keys at or above
// its column j, so with j = (511 - k) / 64 at least 512 - k keys lie at or
// above the wave minimum of column j; the wave maximum bounds it above.
__device__ inline uint32_t wave_kth_smallest(const u16x2 (&u)[4], int k) {
  const int need = kLatentDim - k;
  const int col = (need - 1) >> 6;
  uint32_t sc = u[0].x;
  if (col != 0) {
#pragma unroll
    for (int j = 1; j < 8; ++j) sc = col == j ? key_column(u, j) : sc;
  }
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave_min_i32(static_cast<int>(sc))));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave_max_i32(static_cast<int>(u[0].x))));
  return wave_bisect_rank(u, lo, hi, need);
}

// Quantizes one latent token (one wave; lane l holds channels 8l..8l+7), or,
// without clipping, one 128-channel group of a token per 16-lane row: the
// reductions stay inside each row, and col (= lane for whole tokens) is the
// channel octet the lane holds, which places its codes and its group's
// metadata word.
template <bool kClip>
__device__ void write_latent_token(const WriterParams& p, const uint4 raw, uint8_t* page, int slot, int col) {
  const int lane = col;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  // (a -0 among the values changes no code; the group's min and max are
  // made +0 below)
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  if constexpr (kClip) {
    // |x| as 15-bit bf16 keys (the input words with their sign bits
    // cleared), each lane's sorted in descending order
    u16x2 u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
    sort8_packed(u);
    const uint32_t lo = wave_kth_smallest(u, p.clip_lo);
    // order statistic clip_hi: the smallest key above lo if at least
    // 512 - clip_hi keys lie above lo, else lo itself.  The columns holding
    // keys above lo come first (each column's lanes are part of the previous
    // one's), so the first empty column ends the pass; a lane's smallest key
    // above lo is the last of its sorted keys that is.
    uint32_t above = 0x7FFFFFFFu;
    int n_above = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t key = key_column(u, j);
      const uint64_t m = __ballot(key > lo);
      if (m == 0) break;
      n_above += __popcll(m);
      above = key > lo ? key : above;
    }
    uint32_t hi = lo;
    if (n_above >= kLatentDim - p.clip_hi)
      hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave_min_i32(static_cast<int>(above))));
    const float flo = bf16_to_f32(lo), fhi = bf16_to_f32(hi);
    const float d = fhi - flo;
    const float prod = p.clip_frac * d;
    const float c = flo + prod;
    // clamp to [-c, c] (c >= 0)
    const float nc = -c;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_fmed3f(x[i], nc, c);
  }
  float mn, mx;
  group_minmax(x, mn, mx);
  mn = canon_zero(mn);
  mx = canon_zero(mx);
  const uint16_t mh = f16_round_down(mn);
  const float minf = f16_to_f32(mh);
  const float span = mx - minf;
  const float s = p.bits == 4 ? div_levels(span, 15.0f, 1.0f / 15.0f) : div_levels(span, 3.0f, 1.0f / 3.0f);
  const uint16_t sh = f16_round_up(s);
  const float sf = f16_to_f32(sh);
  const float rs = __builtin_amdgcn_rcpf(sf);
  const uint32_t packed = pack_codes(x, minf, sf, rs, p.bits);
  uint8_t* row = page + static_cast<int64_t>(slot) * p.latent_row;
  if (p.bits == 4) {
    reinterpret_cast<uint32_t*>(row)[lane] = packed;
  } else {
    reinterpret_cast<uint16_t*>(row)[lane] = static_cast<uint16_t>(packed);
  }
  if ((lane & 15) == 0) {
    const uint32_t meta = static_cast<uint32_t>(sh) | (static_cast<uint32_t>(mh) << 16);
    uint8_t* m = page + p.latent_meta_off + static_cast<int64_t>(slot) * (kGroups * 4);
    reinterpret_cast<uint32_t*>(m)[lane >> 4] = meta;
  }
}

// Stores one token's BF16 row [c_KV 512 | k_R 64] (1152 B) with one wave:
// lane l holds c_KV bytes 16 l .. 16 l + 15 and (l < 8) k_R bytes 16 l ...
__device__ inline void copy_row(uint16_t* dst, const uint4 ckv, const uint4 kr, int lane) {
  reinterpret_cast<uint4*>(dst)[lane] = ckv;
  if (lane < 8) reinterpret_cast<uint4*>(dst + kLatentDim)[lane] = kr;
}

// One token's latent row as a wave holds it (see copy_row).
__device__ inline uint4 load_latent(const WriterParams& p, int64_t row, int lane) {
  return reinterpret_cast<const uint4*>(p.c_kv + row * kLatentDim)[lane];
}

// The BF16 copies of sequence b's token at position t (input row `row`,
// latent bf16 row `ckv` as a wave holds it) in the sink and the window ring,
// for a token that belongs there (end: the sequence length after the call);
// its k_R row is read only then.
__device__ inline void retain_token(const WriterParams& p, int b, int t, int end, int64_t row, const uint4 ckv,
                                    int lane) {
  const bool to_sink = t < p.sink_n, to_ring = p.local > 0 && t >= end - p.local;
  if (!to_sink && !to_ring) return;
  const uint4 kr = reinterpret_cast<const uint4*>(p.k_r + row * kRopeDim)[lane & 7];
  if (to_sink) copy_row(p.sink + (static_cast<int64_t>(b) * p.sink_n + t) * kRowElems, ckv, kr, lane);
  if (to_ring) copy_row(p.ring + (static_cast<int64_t>(b) * p.local + t % p.local) * kRowElems, ckv, kr, lane);
}

// Quantizes two latent tokens with one wave (no clip): lanes 0..31 hold
// one token and lanes 32..63 the other, lane l channels 16 c .. 16 c + 15
// (c = l mod 32), so a 128-channel group is 8 lanes and the group's min / max
// and metadata are worked out once per lane for both tokens.  x holds the
// lane's 32 bytes of its token's row; the codes go to row slot `slot` of the
// page (two dwords a lane at 4 bits, one at 2), and nothing is stored where
// `store` is false (a half-wave without a token).  The stores address the
// first token's code row and metadata (`rows`, `metas`, the same in every
// lane) plus per-lane byte offsets that also step to the second token.
__device__ void write_latent_pair(const WriterParams& p, const uint4 (&raw)[2], uint8_t* rows, uint8_t* metas,
                                  uint32_t code_off, uint32_t meta_off, int col, bool store) {
  const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float mn, mx;
  group_minmax16(x, mn, mx);
  mn = canon_zero(mn);
  mx = canon_zero(mx);
  const uint16_t mh = f16_round_down(mn);
  const float minf = f16_to_f32(mh);
  const float span = mx - minf;
  const float s = p.bits == 4 ? div_levels(span, 15.0f, 1.0f / 15.0f) : div_levels(span, 3.0f, 1.0f / 3.0f);
  const uint16_t sh = f16_round_up(s);
  const float sf = f16_to_f32(sh);
  const float rs = __builtin_amdgcn_rcpf(sf);
  float a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = x[i];
    b[i] = x[8 + i];
  }
  const uint32_t ca = pack_codes(a, minf, sf, rs, p.bits), cb = pack_codes(b, minf, sf, rs, p.bits);
  if (!store) return;
  if (p.bits == 4) {
    *reinterpret_cast<uint2*>(rows + code_off) = make_uint2(ca, cb);
  } else {
    *reinterpret_cast<uint32_t*>(rows + code_off) = ca | (cb << 16);
  }
  if ((col & 7) == 0)
    *reinterpret_cast<uint32_t*>(metas + meta_off) = static_cast<uint32_t>(sh) | (static_cast<uint32_t>(mh) << 16);
}

// retain_token for a half-wave holding its token's row 32 bytes a lane
// (lane c = l mod 32 holds c_KV bytes 32 c .. 32 c + 31, k_R by c < 8).
__device__ inline void retain_half(const WriterParams& p, int b, int t, int end, int64_t row, const uint4 (&x)[2],
                                   int col) {
  const bool to_sink = t < p.sink_n, to_ring = p.local > 0 && t >= end - p.local;
  if (!to_sink && !to_ring) return;
  const uint4 kr = reinterpret_cast<const uint4*>(p.k_r + row * kRopeDim)[col & 7];
  const auto put = [&](uint16_t* dst) {
    reinterpret_cast<uint4*>(dst)[2 * col] = x[0];
    reinterpret_cast<uint4*>(dst)[2 * col + 1] = x[1];
    if (col < 8) reinterpret_cast<uint4*>(dst + kLatentDim)[col] = kr;
  };
  if (to_sink) put(p.sink + (static_cast<int64_t>(b) * p.sink_n + t) * kRowElems);
  if (to_ring) put(p.ring + (static_cast<int64_t>(b) * p.local + t % p.local) * kRowElems);
}

// Columns k0 .. k0 + 63 of the latent transform for N tokens: acc[w] of
// token w continues its fp32 fma chain over A_c row `arow` (64 staged bf16
// values) times the token's inputs xs[w][k0 ..] (fp32, broadcast from LDS),
// in ascending order.  N is a compile-time count so that the pass has no
// branches and its LDS reads can all be issued ahead of the chain.
template <int N>
__device__ inline void transform_pass(float (&acc)[kWaves], const uint8_t* arow, const float (*xs)[kLatentDim],
                                      int k0) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const uint4 a8 = *reinterpret_cast<const uint4*>(arow + 16 * kb);
    const float a[8] = {bf16_to_f32(a8.x & 0xFFFFu), bf16_to_f32(a8.x >> 16), bf16_to_f32(a8.y & 0xFFFFu),
                        bf16_to_f32(a8.y >> 16),     bf16_to_f32(a8.z & 0xFFFFu), bf16_to_f32(a8.z >> 16),
                        bf16_to_f32(a8.w & 0xFFFFu), bf16_to_f32(a8.w >> 16)};
    const int k = k0 + 8 * kb;
#pragma unroll
    for (int w = 0; w < N; ++w) {
      const float4 x0 = *reinterpret_cast<const float4*>(&xs[w][k]);
      const float4 x1 = *reinterpret_cast<const float4*>(&xs[w][k + 4]);
      float s = acc[w];
      s = fmaf(a[0], x0.x, s);
      s = fmaf(a[1], x0.y, s);
      s = fmaf(a[2], x0.z, s);
      s = fmaf(a[3], x0.w, s);
      s = fmaf(a[4], x1.x, s);
      s = fmaf(a[5], x1.y, s);
      s = fmaf(a[6], x1.z, s);
      s = fmaf(a[7], x1.w, s);
      acc[w] = s;
    }
  }
}

// kMode 0: plain writer; 1: with the latent transform, one workgroup per
// page; 2: with the latent transform, four workgroups per page (latent group
// g = blockIdx.x % 4).  kClip: the INT2 latent's quantile clip (never with
// kMode 2); a separate instantiation keeps its code out of the others.  The
// plain writer is held to 80 VGPRs (6 waves per SIMD, 3 workgroups per CU:
// its two-token path needs 79), the clip writer to 64 (8 waves per SIMD).
template <int kMode, bool kClip>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kMode == 0 ? (kClip ? 8 : 6) : 1))) writer_kernel(WriterParams p) {
  constexpr bool kTransform = kMode != 0;
  // kMode 2: latent group g of the page; kMode 0: token share g of
  // p.token_split (share 0 also does the page's k_R work)
  const int split = kMode == 2 ? 4 : (kMode == 0 ? p.token_split : 1);
  const int g = static_cast<int>(blockIdx.x % static_cast<uint32_t>(split));
  const int blk = static_cast<int>(blockIdx.x / static_cast<uint32_t>(split));
  const int b = blk / p.pages_per_seq_grid;
  const int pi = blk % p.pages_per_seq_grid;
  if (b >= p.batch) return;
  const int r0 = p.cu_new[b], r1 = p.cu_new[b + 1];
  const int sb = p.seqlens_before[b];
  if (r0 < 0 || r1 < r0 || r1 > p.total_new || sb < 0) return;
  const int n_new = r1 - r0;
  if (n_new == 0) return;
  const int P = p.P;
  const int end = sb + n_new;
  const int p0 = sb / P;
  const int pg = p0 + pi;
  if (static_cast<int64_t>(pg) * P >= end) return;
  const int last_page = (end - 1) / P;
  if (last_page >= p.max_pages) return;  // positions beyond the block table
  const int tb = max(sb, pg * P), te = min(end, (pg + 1) * P);
  // (the wave index is the same in every lane: read from lane 0, it is a
  // scalar, and so are the token indices and loop bounds derived from it)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint16_t* tail = p.tail + static_cast<int64_t>(b) * P * kRopeDim;

  // k_R rows of a page that becomes full in this call (tail buffer for tokens
  // of earlier calls, input rows for new ones) go straight from global memory
  // into LDS, all at once (16 bytes per lane and load), before the page id is
  // looked up: they do not depend on it.  The barrier before their reduction
  // waits for them.  Row s's channel octet q sits in 16-byte unit
  // 8 s + (q ^ (s % 8)), so that a wave reading one octet of 64 rows (a row
  // per lane) spreads over every bank.
  __shared__ uint4 s_rows[256 * kRopeDim / 8];  // P x 64 bf16
  const bool completes = g == 0 && (pg + 1) * P <= end;  // (the group-0 workgroup does the k_R work)
  if (completes) {
    for (int k = 0; k * kThreads < P * (kRopeDim / 8); ++k) {
      const int i = static_cast<int>(threadIdx.x) + k * kThreads;
      if (k * kThreads + 64 * wave >= P * (kRopeDim / 8)) break;  // whole waves (P * 8 is a multiple of 256)
      const int slot = i >> 3, q = (i & 7) ^ (slot & 7);
      const int t = pg * P + slot;
      const uint4* src = t < sb ? reinterpret_cast<const uint4*>(tail + static_cast<int64_t>(slot) * kRopeDim) + q
                                : reinterpret_cast<const uint4*>(p.k_r + (r0 + (t - sb)) * static_cast<int64_t>(kRopeDim)) + q;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(s_rows + k * kThreads + 64 * wave),
                                       16, 0, 0);
    }
  }
  // this wave's first token goes out with them (its row index is clamped
  // into the input: a wave without a token reads a row it does not use)
  uint4 cur{};
  // kMode 0 with the tokens of a page dealt to `split` workgroups: on a page
  // that this call completes, the first workgroup only does the page's k_R
  // work and the others take its tokens (its share would otherwise run after
  // theirs); token runs of kWaves go round the token workgroups in turn.
  const bool finalize_only = kMode == 0 && split > 1 && (pg + 1) * P <= end;  // same in every workgroup of the page
  const int tok_wgs = finalize_only ? split - 1 : split, tok_g = finalize_only ? g - 1 : g;
  const int t_first = kMode != 0 ? tb + wave : (tok_g < 0 ? te : tb + tok_g * kWaves + wave);
  const int t_step = kWaves * (kMode == 0 ? tok_wgs : 1);
  // (the plain writer without the clip takes two tokens a wave: half-wave
  // h = lane / 32 has token t_first + h t_step of each pair)
  constexpr bool kPairs = kMode == 0 && !kClip;
  const int half = lane >> 5, col2 = lane & 31;
  uint4 pa[2] = {};
  // byte offsets of the lane's part of its half-wave's token from the pair's
  // first token: input row, code row, metadata (same in every pair)
  const uint32_t step_h = static_cast<uint32_t>(half * t_step);
  const uint32_t in_off = step_h * (kLatentDim * 2) + 32u * static_cast<uint32_t>(col2);
  const uint32_t code_off = step_h * static_cast<uint32_t>(p.latent_row) + (p.bits == 4 ? 8u : 4u) * col2;
  const uint32_t meta_off = step_h * (kGroups * 4) + 4u * static_cast<uint32_t>(col2 >> 3);
  const auto load_pair = [&](uint4(&x)[2], int t) {  // t: the pair's first token
    const uint8_t* src =
        reinterpret_cast<const uint8_t*>(p.c_kv + static_cast<int64_t>(r0 + (t - sb)) * kLatentDim) + in_off;
    x[0] = reinterpret_cast<const uint4*>(src)[0];
    x[1] = reinterpret_cast<const uint4*>(src)[1];
  };
  if constexpr (kPairs) {
    // (a half-wave past the page's last token reads that token's row instead)
    if (t_first + half * t_step < te) {
      load_pair(pa, t_first);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(p.c_kv + static_cast<int64_t>(r0 + (te - 1 - sb)) * kLatentDim) + 2 * col2;
      pa[0] = src[0];
      pa[1] = src[1];
    }
  } else if constexpr (!kTransform) {
    cur = load_latent(p, r0 + (min(t_first, te - 1) - sb), lane);
  }
  const int page_id = p.block_table[static_cast<int64_t>(b) * p.max_pages + pg];
  if (page_id < 0 || page_id >= p.num_pool_pages) {
    __syncthreads();  // no direct load outlives the workgroup
    return;
  }
  uint8_t* page = p.pool + static_cast<int64_t>(page_id) * p.page_bytes;

  if constexpr (kMode == 2) {
    // The latent transform split by latent group: thread (j, o) forms output
    // channel 128 g + o of token slot j (of up to 4 tokens at a time) as the
    // same ascending fp32 fma chain as below, over rows 128 g .. 128 g + 127
    // of A_c (64 input columns per LDS pass, loaded two passes ahead); row q
    // of wave 0 then caches group g of token q: its codes and metadata word,
    // and its 256 bytes of the BF16 sink / ring rows (plus the k_R bytes in
    // the group-0 workgroup).
    constexpr int kTok = 4;
    constexpr int kAChunk = 64;
    constexpr int kAPitch = 2 * kAChunk + 16;
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kGroup * kAPitch];
    __shared__ __attribute__((aligned(16))) float s_x[kTok][kLatentDim];
    __shared__ __attribute__((aligned(16))) uint16_t s_y[kTok][kGroup];
    const int o = static_cast<int>(threadIdx.x) & (kGroup - 1), j = static_cast<int>(threadIdx.x) >> 7;
    // staging: 16-byte piece st_part of rows st_row and st_row + 64 of a pass
    const int st_row = static_cast<int>(threadIdx.x) >> 3, st_part = static_cast<int>(threadIdx.x) & 7;
    const uint4* const a_src =
        reinterpret_cast<const uint4*>(p.a_c + static_cast<int64_t>(kGroup * g + st_row) * kLatentDim) + st_part;
    uint8_t* const a_dst = s_a + st_row * kAPitch + 16 * st_part;
    constexpr int kRowStep = 64 * kLatentDim / 8;  // uint4 elements from row st_row to row st_row + 64
    const uint8_t* const arow = s_a + o * kAPitch;
    for (int t0 = tb; t0 < te; t0 += kTok) {
      const int n = min(kTok, te - t0);
      if (wave < n) {
        const uint4 raw =
            reinterpret_cast<const uint4*>(p.c_kv + (r0 + (t0 + wave - sb)) * static_cast<int64_t>(kLatentDim))[lane];
        const float4 lo = {bf16_to_f32(raw.x & 0xFFFFu), bf16_to_f32(raw.x >> 16), bf16_to_f32(raw.y & 0xFFFFu),
                           bf16_to_f32(raw.y >> 16)};
        const float4 hi = {bf16_to_f32(raw.z & 0xFFFFu), bf16_to_f32(raw.z >> 16), bf16_to_f32(raw.w & 0xFFFFu),
                           bf16_to_f32(raw.w >> 16)};
        *reinterpret_cast<float4*>(&s_x[wave][8 * lane]) = lo;
        *reinterpret_cast<float4*>(&s_x[wave][8 * lane + 4]) = hi;
      }
      float acc[kWaves];
      acc[0] = 0.0f;
      uint4 a0 = a_src[0], a1 = a_src[kRowStep];
      uint4 b0 = a_src[kAChunk / 8], b1 = a_src[kRowStep + kAChunk / 8];
      static_assert(kLatentDim % (2 * kAChunk) == 0, "passes go in pairs");
#pragma unroll 1
      for (int k0 = 0; k0 < kLatentDim; k0 += 2 * kAChunk) {
        lds_barrier();  // the previous pass's reads of s_a are done
        *reinterpret_cast<uint4*>(a_dst) = a0;
        *reinterpret_cast<uint4*>(a_dst + 64 * kAPitch) = a1;
        lds_barrier();  // s_a (and, on the first pass, s_x) filled
        if (k0 + 2 * kAChunk < kLatentDim) {
          a0 = a_src[(k0 + 2 * kAChunk) / 8];
          a1 = a_src[kRowStep + (k0 + 2 * kAChunk) / 8];
        }
        if (j < n) transform_pass<1>(acc, arow, &s_x[j], k0);
        lds_barrier();
        *reinterpret_cast<uint4*>(a_dst) = b0;
        *reinterpret_cast<uint4*>(a_dst + 64 * kAPitch) = b1;
        lds_barrier();
        if (k0 + 3 * kAChunk < kLatentDim) {
          b0 = a_src[(k0 + 3 * kAChunk) / 8];
          b1 = a_src[kRowStep + (k0 + 3 * kAChunk) / 8];
        }
        if (j < n) transform_pass<1>(acc, arow, &s_x[j], k0 + kAChunk);
      }
      if (j < n) s_y[j][o] = static_cast<uint16_t>(f32_to_bf16_rne(acc[0]));
      lds_barrier();
      const int q = lane >> 4, l16 = lane & 15;
      if (wave == 0 && q < n) {
        const int t = t0 + q;
        const uint4 y = *reinterpret_cast<const uint4*>(&s_y[q][8 * l16]);
        write_latent_token<false>(p, y, page, t - pg * P, 16 * g + l16);
        // this group's slice of the BF16 rows (the group-0 workgroup adds k_R)
        auto copy_slice = [&](uint16_t* dst) {
          reinterpret_cast<uint4*>(dst + kGroup * g)[l16] = y;
          if (g == 0 && l16 < 8)
            reinterpret_cast<uint4*>(dst + kLatentDim)[l16] =
                reinterpret_cast<const uint4*>(p.k_r + (r0 + (t - sb)) * static_cast<int64_t>(kRopeDim))[l16];
        };
        if (t < p.sink_n) copy_slice(p.sink + (static_cast<int64_t>(b) * p.sink_n + t) * kRowElems);
        if (p.local > 0 && t >= end - p.local)
          copy_slice(p.ring + (static_cast<int64_t>(b) * p.local + t % p.local) * kRowElems);
      }
      lds_barrier();  // s_x and s_y are refilled for the next tokens
    }
  } else if constexpr (kTransform) {
    // The latent transform (RAQ-MLA Figure 4 caption; appendix Table 9, the
    // fused variant): y = A_c x per token, for up to kWaves tokens at a time.
    // Thread c forms output channel c of each token as an fp32 fma chain over
    // the 512 inputs in ascending order, rounded once to bf16; wave w then
    // caches token t0 + w from that bf16 row exactly as it caches an
    // untransformed one (codes, metadata, sink and ring copies).  A_c passes
    // through LDS 64 input columns at a time, read as whole 128-byte row
    // segments (coalesced) and stored with a padded row pitch so that each
    // thread's reads of its own row do not collide; the inputs are broadcast
    // from LDS.
    constexpr int kAChunk = 64;                // input columns per LDS pass
    constexpr int kAPitch = 2 * kAChunk + 16;  // bytes per staged row
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kLatentDim * kAPitch];
    __shared__ __attribute__((aligned(16))) float s_x[kWaves][kLatentDim];
    __shared__ uint4 s_y[kWaves][kLatentDim / 8];
    const int c = static_cast<int>(threadIdx.x);
    const int st_row = c >> 3, st_part = c & 7;  // staging: 16 bytes of row st_row + 64 j
    for (int t0 = tb; t0 < te; t0 += kWaves) {
      const int n = min(kWaves, te - t0);
      if (wave < n) {
        const uint4 raw =
            reinterpret_cast<const uint4*>(p.c_kv + (r0 + (t0 + wave - sb)) * static_cast<int64_t>(kLatentDim))[lane];
        const float4 lo = {bf16_to_f32(raw.x & 0xFFFFu), bf16_to_f32(raw.x >> 16), bf16_to_f32(raw.y & 0xFFFFu),
                           bf16_to_f32(raw.y >> 16)};
        const float4 hi = {bf16_to_f32(raw.z & 0xFFFFu), bf16_to_f32(raw.z >> 16), bf16_to_f32(raw.w & 0xFFFFu),
                           bf16_to_f32(raw.w >> 16)};
        *reinterpret_cast<float4*>(&s_x[wave][8 * lane]) = lo;
        *reinterpret_cast<float4*>(&s_x[wave][8 * lane + 4]) = hi;
      }
      float acc[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) acc[w] = 0.0f;
      // this thread's 16-byte pieces of a pass's A_c columns, loaded two
      // passes ahead (two register sets in turn) so that they arrive while
      // the passes between compute; the barriers here wait for LDS traffic
      // only (__syncthreads would also drain these loads)
      const uint4* const a_src = reinterpret_cast<const uint4*>(p.a_c + static_cast<int64_t>(st_row) * kLatentDim) + st_part;
      uint8_t* const a_dst = s_a + st_row * kAPitch + 16 * st_part;
      constexpr int kRowStep = 64 * kLatentDim / 8;  // uint4 elements between rows st_row + 64 j
      uint4 a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3, b4, b5, b6, b7;
      a0 = a_src[0 * kRowStep]; a1 = a_src[1 * kRowStep]; a2 = a_src[2 * kRowStep]; a3 = a_src[3 * kRowStep];
      a4 = a_src[4 * kRowStep]; a5 = a_src[5 * kRowStep]; a6 = a_src[6 * kRowStep]; a7 = a_src[7 * kRowStep];
      {
        constexpr int o = kAChunk / 8;
        b0 = a_src[0 * kRowStep + o]; b1 = a_src[1 * kRowStep + o]; b2 = a_src[2 * kRowStep + o];
        b3 = a_src[3 * kRowStep + o]; b4 = a_src[4 * kRowStep + o]; b5 = a_src[5 * kRowStep + o];
        b6 = a_src[6 * kRowStep + o]; b7 = a_src[7 * kRowStep + o];
      }
      auto run_pass = [&](int k0) {
        static_assert(kAChunk == 64, "transform_pass takes 64 columns");
        const uint8_t* const arow = s_a + c * kAPitch;
        switch (n) {
          case 1: transform_pass<1>(acc, arow, s_x, k0); break;
          case 2: transform_pass<2>(acc, arow, s_x, k0); break;
          case 3: transform_pass<3>(acc, arow, s_x, k0); break;
          case 4: transform_pass<4>(acc, arow, s_x, k0); break;
          case 5: transform_pass<5>(acc, arow, s_x, k0); break;
          case 6: transform_pass<6>(acc, arow, s_x, k0); break;
          case 7: transform_pass<7>(acc, arow, s_x, k0); break;
          default: transform_pass<8>(acc, arow, s_x, k0); break;
        }
      };
      static_assert(kLatentDim % (2 * kAChunk) == 0, "passes go in pairs");
#pragma unroll 1
      for (int k0 = 0; k0 < kLatentDim; k0 += 2 * kAChunk) {
        // a pass's pieces into LDS between two LDS-only barriers, then the
        // set is reloaded for the pass two ahead
        lds_barrier();  // the previous pass's reads of s_a are done
        *reinterpret_cast<uint4*>(a_dst + 0 * 64 * kAPitch) = a0;
        *reinterpret_cast<uint4*>(a_dst + 1 * 64 * kAPitch) = a1;
        *reinterpret_cast<uint4*>(a_dst + 2 * 64 * kAPitch) = a2;
        *reinterpret_cast<uint4*>(a_dst + 3 * 64 * kAPitch) = a3;
        *reinterpret_cast<uint4*>(a_dst + 4 * 64 * kAPitch) = a4;
        *reinterpret_cast<uint4*>(a_dst + 5 * 64 * kAPitch) = a5;
        *reinterpret_cast<uint4*>(a_dst + 6 * 64 * kAPitch) = a6;
        *reinterpret_cast<uint4*>(a_dst + 7 * 64 * kAPitch) = a7;
        lds_barrier();  // s_a (and, on the first pass, s_x) filled
        if (k0 + 2 * kAChunk < kLatentDim) {
          const int o = (k0 + 2 * kAChunk) / 8;
          a0 = a_src[0 * kRowStep + o]; a1 = a_src[1 * kRowStep + o]; a2 = a_src[2 * kRowStep + o];
          a3 = a_src[3 * kRowStep + o]; a4 = a_src[4 * kRowStep + o]; a5 = a_src[5 * kRowStep + o];
          a6 = a_src[6 * kRowStep + o]; a7 = a_src[7 * kRowStep + o];
        }
        run_pass(k0);
        lds_barrier();
        *reinterpret_cast<uint4*>(a_dst + 0 * 64 * kAPitch) = b0;
        *reinterpret_cast<uint4*>(a_dst + 1 * 64 * kAPitch) = b1;
        *reinterpret_cast<uint4*>(a_dst + 2 * 64 * kAPitch) = b2;
        *reinterpret_cast<uint4*>(a_dst + 3 * 64 * kAPitch) = b3;
        *reinterpret_cast<uint4*>(a_dst + 4 * 64 * kAPitch) = b4;
        *reinterpret_cast<uint4*>(a_dst + 5 * 64 * kAPitch) = b5;
        *reinterpret_cast<uint4*>(a_dst + 6 * 64 * kAPitch) = b6;
        *reinterpret_cast<uint4*>(a_dst + 7 * 64 * kAPitch) = b7;
        lds_barrier();
        if (k0 + 3 * kAChunk < kLatentDim) {
          const int o = (k0 + 3 * kAChunk) / 8;
          b0 = a_src[0 * kRowStep + o]; b1 = a_src[1 * kRowStep + o]; b2 = a_src[2 * kRowStep + o];
          b3 = a_src[3 * kRowStep + o]; b4 = a_src[4 * kRowStep + o]; b5 = a_src[5 * kRowStep + o];
          b6 = a_src[6 * kRowStep + o]; b7 = a_src[7 * kRowStep + o];
        }
        run_pass(k0 + kAChunk);
      }
      uint16_t* const ys = reinterpret_cast<uint16_t*>(&s_y[0][0]);
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (w < n) ys[w * kLatentDim + c] = static_cast<uint16_t>(f32_to_bf16_rne(acc[w]));
      lds_barrier();
      if (wave < n) {
        const int t = t0 + wave;
        const uint4 y = s_y[wave][lane];
        write_latent_token<kClip>(p, y, page, t - pg * P, lane);
        retain_token(p, b, t, end, r0 + (t - sb), y, lane);
      }
      lds_barrier();  // s_x and s_y are refilled for the next tokens
    }
  } else if constexpr (kPairs) {
    // Two tokens a wave (one a half-wave), two pairs per trip in two register
    // sets: each pair's rows are requested before the previous pair is
    // written (no register copies).
    const auto pair = [&](const uint4(&x)[2], int t) {
      const int my = t + half * t_step;
      const bool ok = my < te;
      uint8_t* const rows = page + static_cast<int64_t>(t - pg * P) * p.latent_row;
      uint8_t* const metas = page + p.latent_meta_off + static_cast<int64_t>(t - pg * P) * (kGroups * 4);
      if (ok) retain_half(p, b, my, end, r0 + (my - sb), x, col2);  // (first: the raw row is then dead)
      write_latent_pair(p, x, rows, metas, code_off, meta_off, col2, ok);
    };
    const auto fetch2 = [&](uint4(&x)[2], int t) {
      if (t + half * t_step < te) load_pair(x, t);
    };
    uint4 pb[2] = {};
    for (int t = t_first; t < te; t += 4 * t_step) {
      fetch2(pb, t + 2 * t_step);
      pair(pa, t);
      if (t + 2 * t_step >= te) break;
      fetch2(pa, t + 4 * t_step);
      pair(pb, t + 2 * t_step);
    }
  } else {
    // Latent codes + metadata, BF16 sink / ring copies.  Three tokens per
    // trip in three register sets, each token's row requested two tokens
    // before it is written (no register copies).
    const auto token = [&](const uint4 x, int t) {
      write_latent_token<kClip>(p, x, page, t - pg * P, lane);
      retain_token(p, b, t, end, r0 + (t - sb), x, lane);
    };
    const auto fetch = [&](uint4& x, int t) {
      if (t < te) x = load_latent(p, r0 + (t - sb), lane);
    };
    uint4 nx1{}, nx2{};
    fetch(nx1, t_first + t_step);
    for (int t = t_first; t < te; t += 3 * t_step) {
      fetch(nx2, t + 2 * t_step);
      token(cur, t);
      if (t + t_step >= te) break;
      fetch(cur, t + 3 * t_step);
      token(nx1, t + t_step);
      if (t + 2 * t_step >= te) break;
      fetch(nx1, t + 4 * t_step);
      token(nx2, t + 2 * t_step);
    }
  }

  // k_R of a page that becomes full: per channel over its P tokens.  Wave w
  // takes channels 8w .. 8w + 7 (octet w) of rows lane, lane + 64, ...: the
  // octet's minimum and maximum are reduced inside the wave as packed 16-bit
  // order keys of the bf16 values (two channels per dword), lanes 0..7 form
  // one channel's metadata each, and every lane then codes its rows' octet
  // (one dword: row s, channels 8w .. 8w + 7 is dword 8 s + w).  No data
  // crosses waves, so one barrier (the rows in LDS) is all it takes.
  if (completes) {
    __syncthreads();
    const int q = wave;
    const int rows_per_lane = (P + 63) >> 6;
    // order keys: a bf16 b as a signed 16-bit k = b, or b ^ 0x7FFF for a
    // negative b (the map is its own inverse; -0 sorts just below +0)
    const auto keys = [](uint32_t w) {
      const i16x2 neg = __builtin_bit_cast(i16x2, w) >> i16x2{15, 15};  // -1 in a negative half
      return w ^ (__builtin_bit_cast(uint32_t, neg) & 0x7FFF7FFFu);
    };
    i16x2 kmn[4], kmx[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      kmn[d] = i16x2{0x7FFF, 0x7FFF};
      kmx[d] = i16x2{-0x8000, -0x8000};
    }
    for (int k = 0; k < rows_per_lane; ++k) {
      const int s = lane + 64 * k;
      if (s < P) {
        const uint4 w = s_rows[s * 8 + (q ^ (s & 7))];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const i16x2 kk = __builtin_bit_cast(i16x2, keys(ww[d]));
          kmn[d] = __builtin_elementwise_min(kmn[d], kk);
          kmx[d] = __builtin_elementwise_max(kmx[d], kk);
        }
      }
    }
    // The eight dwords (minimum keys of the channel pairs 0..3, then the
    // maximum keys complemented, so that all eight reduce by minimum) are
    // reduced by a reduce-scatter: the partners l ^ 1, l ^ 2 (quad permutes)
    // and l ^ 7 (half-row mirror) each halve the lane's dwords by a lane bit
    // in which the partners differ and agree in the others (a = b0 ^ b2,
    // b = b1 ^ b2, c = b2), so that lane l ends with dword 4a + 2b + c over
    // its 8 lanes; the lanes agreeing in their low three bits then finish it.
    uint32_t dw[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      dw[d] = __builtin_bit_cast(uint32_t, kmn[d]);
      dw[4 + d] = ~__builtin_bit_cast(uint32_t, kmx[d]);
    }
    const bool ua = ((lane ^ (lane >> 2)) & 1) != 0, ub = (((lane >> 1) ^ (lane >> 2)) & 1) != 0,
               uc = ((lane >> 2) & 1) != 0;
    uint32_t e4[4], e2[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) e4[i] = scatter_min<0xB1>(ua, dw[i], dw[i + 4]);
#pragma unroll
    for (int j = 0; j < 2; ++j) e2[j] = scatter_min<0x4E>(ub, e4[j], e4[j + 2]);
    const uint32_t g = min_over_octets(scatter_min<0x141>(uc, e2[0], e2[1]));
    // Lanes l and l ^ 1 hold the minimum and the (complemented) maximum of the
    // channel pair k = 2b + c; lane l < 8 takes channel 2k + (l & 1) of the
    // octet, so lanes 0..7 hold channels 0, 1, 4, 5, 6, 7, 2, 3.
    const uint32_t other = __builtin_bit_cast(uint32_t, dpp_i16x2<0xB1>(__builtin_bit_cast(i16x2, g)));
    const uint32_t pmn = ua ? other : g, pmx = ~(ua ? g : other);
    const int e = 4 * static_cast<int>(ub) + 2 * static_cast<int>(uc) + (lane & 1);
    const uint32_t bmn = keys((lane & 1) ? pmn >> 16 : pmn & 0xFFFFu) & 0xFFFFu;
    const uint32_t bmx = keys((lane & 1) ? pmx >> 16 : pmx & 0xFFFFu) & 0xFFFFu;
    const float cmn = canon_zero(bf16_to_f32(bmn)), cmx = canon_zero(bf16_to_f32(bmx));
    const uint16_t mh = f16_round_down(cmn);
    const float minf = f16_to_f32(mh);
    const float span = cmx - minf;
    const uint16_t sh = f16_round_up(div_levels(span, 15.0f, 1.0f / 15.0f));
    const float sf = f16_to_f32(sh);
    if (lane < 8) {
      uint16_t* meta = reinterpret_cast<uint16_t*>(page + p.rope_meta_off);
      meta[8 * q + e] = sh;
      meta[kRopeDim + 8 * q + e] = mh;
    }
    // every lane gets the octet's offsets, steps and reciprocals (0 for a
    // zero step: its codes are 0)
    float mo[8], so[8], ro[8];
    const float rc = sf > 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int src = 4 * ((c >> 1) & 1) + 2 * ((c >> 2) ^ ((c >> 1) & 1)) + (c & 1);  // the lane of channel c
      mo[c] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, minf), src));
      so[c] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sf), src));
      ro[c] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rc), src));
    }
    uint32_t* const codes = reinterpret_cast<uint32_t*>(page + p.rope_codes_off);
    for (int k = 0; k < rows_per_lane; ++k) {
      const int s = lane + 64 * k;
      if (s < P) {
        const uint4 w = s_rows[s * 8 + (q ^ (s & 7))];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float d[8], r[8];
        float dev = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          d[c] = bf16_to_f32((c & 1) ? ww[c >> 1] >> 16 : ww[c >> 1] & 0xFFFFu) - mo[c];
          const float qa = d[c] * ro[c];
          r[c] = rintf(qa);
          dev = fmaxf(dev, fabsf(qa - r[c]));
        }
        if (__builtin_expect(dev >= 0.49999f, 0)) {
#pragma unroll
          for (int c = 0; c < 8; ++c)
            if (so[c] > 0.0f) r[c] = rint_div(d[c], so[c], ro[c]);
        }
        codes[s * 8 + q] = pack_nibbles(r);  // (in [0, 15] without a clamp, as in pack_codes)
      }
    }
  }

  // Tail rows of the page left incomplete, written by the first page's
  // workgroup after every read of the old tail rows above.
  if (g == 0 && pi == 0 && end % P != 0) {
    __syncthreads();
    const int t0 = max(sb, (end / P) * P);
    for (int i = threadIdx.x; i < (end - t0) * (kRopeDim / 8); i += kThreads) {
      const int t = t0 + i / (kRopeDim / 8), q = i % (kRopeDim / 8);
      const uint4* src = reinterpret_cast<const uint4*>(p.k_r + (r0 + (t - sb)) * static_cast<int64_t>(kRopeDim)) + q;
      reinterpret_cast<uint4*>(tail + static_cast<int64_t>(t % P) * kRopeDim)[q] = *src;
    }
  }
}

}  // namespace
}  // namespace mla

namespace mla {
namespace {

int write_impl(const mla_lowbit_layout* layout, const void* a_c, const void* c_kv, const void* k_r,
                                const int32_t* cu_new, const int32_t* seqlens_before, int32_t batch,
                                int32_t total_new, int32_t max_new_per_seq,
                                const int32_t* block_table, int32_t max_pages,
                                int32_t num_pool_pages, void* page_pool, void* sink_buf,
                                void* ring_buf, void* rope_tail, hipStream_t stream) {
  Geometry g;
  int rc = make_geometry(layout, &g);
  if (rc) return rc;
  if (batch < 0 || total_new < 0 || max_new_per_seq < 0 || max_pages < 0 || num_pool_pages < 0)
    return MLA_LOWBIT_ERR_ARG;
  if (batch == 0 || total_new == 0 || max_new_per_seq == 0) return MLA_LOWBIT_OK;
  if (!c_kv || !k_r || !cu_new || !seqlens_before || !block_table || !page_pool || !rope_tail)
    return MLA_LOWBIT_ERR_ARG;
  if (g.sink > 0 && !sink_buf) return MLA_LOWBIT_ERR_ARG;
  if (g.local > 0 && !ring_buf) return MLA_LOWBIT_ERR_ARG;
  if (!aligned16(c_kv) || !aligned16(k_r) || !aligned16(page_pool) || !aligned16(rope_tail) ||
      (sink_buf && !aligned16(sink_buf)) || (ring_buf && !aligned16(ring_buf)))
    return MLA_LOWBIT_ERR_ARG;
  if (max_pages == 0 || num_pool_pages == 0) return MLA_LOWBIT_ERR_ARG;
  if (a_c && !aligned16(a_c)) return MLA_LOWBIT_ERR_ARG;
  WriterParams p{};
  p.a_c = static_cast<const uint16_t*>(a_c);
  p.c_kv = static_cast<const uint16_t*>(c_kv);
  p.k_r = static_cast<const uint16_t*>(k_r);
  p.cu_new = cu_new;
  p.seqlens_before = seqlens_before;
  p.block_table = block_table;
  p.pool = static_cast<uint8_t*>(page_pool);
  p.sink = static_cast<uint16_t*>(sink_buf);
  p.ring = static_cast<uint16_t*>(ring_buf);
  p.tail = static_cast<uint16_t*>(rope_tail);
  p.batch = batch;
  p.total_new = total_new;
  p.max_pages = max_pages;
  p.num_pool_pages = num_pool_pages;
  p.P = g.page_size;
  p.bits = g.latent_bits;
  p.sink_n = g.sink;
  p.local = g.local;
  p.clip_lo = g.clip_lo;
  p.clip_hi = g.clip_hi;
  p.clip_frac = g.clip_frac;
  p.latent_row = g.latent_row;
  p.latent_meta_off = g.latent_meta_off;
  p.rope_codes_off = g.rope_codes_off;
  p.rope_meta_off = g.rope_meta_off;
  p.page_bytes = g.page_bytes;
  // pages a call of n tokens can touch: (n - 1) / P + 2
  p.pages_per_seq_grid = (max_new_per_seq - 1) / g.page_size + 2;
  // with the transform and no clipping, four workgroups per page (one per
  // latent group); the clip needs all 512 channels of a token in one wave.
  // The plain writer deals a page's tokens to 3 or 5 workgroups when a call
  // writes many tokens into few pages (chunked prefill of a few sequences),
  // so that the chip holds more than one workgroup per CU; on a page the call
  // completes the first of them only does the page's k_R work.
  const bool split = a_c && !g.clip;
  p.token_split = 1;
  if (!a_c && max_new_per_seq >= 4 * kWaves) {
    const int64_t pages = static_cast<int64_t>(batch) * ((max_new_per_seq + g.page_size - 1) / g.page_size);
    p.token_split = pages <= 256 ? 5 : (pages <= 1024 ? 3 : 1);
  }
  const int64_t blocks = static_cast<int64_t>(batch) * p.pages_per_seq_grid * (split ? 4 : p.token_split);
  if (blocks > 0x7FFFFFFF) return MLA_LOWBIT_ERR_UNSUPPORTED;
  if (split)
    hipLaunchKernelGGL((writer_kernel<2, false>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, p);
  else if (a_c)  // with the transform only the clip keeps one workgroup per page
    hipLaunchKernelGGL((writer_kernel<1, true>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, p);
  else if (g.clip)
    hipLaunchKernelGGL((writer_kernel<0, true>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((writer_kernel<0, false>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ERR_HIP;
}

}  // namespace
}  // namespace mla

extern "C" int mla_lowbit_write(const mla_lowbit_layout* layout, const void* c_kv, const void* k_r,
                                const int32_t* cu_new, const int32_t* seqlens_before, int32_t batch,
                                int32_t total_new, int32_t max_new_per_seq,
                                const int32_t* block_table, int32_t max_pages,
                                int32_t num_pool_pages, void* page_pool, void* sink_buf,
                                void* ring_buf, void* rope_tail, hipStream_t stream) {
  return mla::write_impl(layout, nullptr, c_kv, k_r, cu_new, seqlens_before, batch, total_new, max_new_per_seq,
                         block_table, max_pages, num_pool_pages, page_pool, sink_buf, ring_buf, rope_tail, stream);
}

extern "C" int mla_lowbit_write_transformed(const mla_lowbit_layout* layout, const void* a_c, const void* c_kv,
                                            const void* k_r, const int32_t* cu_new,
                                            const int32_t* seqlens_before, int32_t batch, int32_t total_new,
                                            int32_t max_new_per_seq, const int32_t* block_table,
                                            int32_t max_pages, int32_t num_pool_pages, void* page_pool,
                                            void* sink_buf, void* ring_buf, void* rope_tail,
                                            hipStream_t stream) {
  if (!a_c) return MLA_LOWBIT_ERR_ARG;
  return mla::write_impl(layout, a_c, c_kv, k_r, cu_new, seqlens_before, batch, total_new, max_new_per_seq,
                         block_table, max_pages, num_pool_pages, page_pool, sink_buf, ring_buf, rope_tail, stream);
}
