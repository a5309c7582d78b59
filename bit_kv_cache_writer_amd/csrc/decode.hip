// Decode attention over the dual-path low-bit MLA cache, for gfx950.
//
// What is computed (QuantMLA Figure 8 caption; RAQ-MLA abstract and
// Figure 4 caption): per sequence and head, one softmax over all valid
// tokens of score = q_lat . c_KV + q_rope . k_R, output sum_j p_j c_KV_j in
// latent space; protected (sink / recent) tokens from BF16, the others from
// codes dequantized inside the loop -- the same reconstructed content tile
// feeds both the score (matching) and the output (aggregation).
//
// How.  Each (sequence, 16-head block) is cut into workgroups of 4 waves (one
// per SIMD, two workgroups per CU): a few BF16-path workgroups take the
// protected tokens, the rest split the packed pages.  Each writes a partial
// (unnormalized output, max, sum); a second kernel merges them with
// log-sum-exp weights (the kernel boundary makes every XCD's partials
// visible without cache flushes inside the kernel).
//
// Packed workgroup.  Each wave owns a contiguous run of 16-token tiles
// (consecutive tiles share a page) and keeps a ring of three tile slots in LDS
// filled by direct global->LDS loads two tiles ahead; the slots hold the codes
// as stored (XOR-swizzled 16-byte units, so row reads and transposed reads are
// bank-conflict free).  The waves advance in lockstep rounds, one tile each:
//  1. Scores: codes come out of LDS in the lanes that feed
//     v_mfma_f32_16x16x32_f16 (M = 16 tokens, N = 16 heads, K = 32 channels;
//     lane (t, g) holds 8 channels of token t) and are unpacked in registers
//     by masking alone: a code left in the low mantissa bits of an fp16 with
//     a zero exponent is the subnormal code * 2^-24 * sigma, sigma the power
//     of two of its bit position (the matrix cores take fp16 subnormals
//     exactly).  The query operand carries q / sigma per slot, so the MFMA
//     sums 2^-24 q_g . code_g; group scale s and minimum m are folded after it:
//       q.c = 2^24 sum_g s_g (q_g . code_g 2^-24) + sum_g m_g Q_g,
//     Q_g = sum of the query over group g; the second sum is one more MFMA on
//     the raw fp16 (scale, min) words.  The positional key's per-(channel,
//     page) scale/min is folded into a per-page query q' = q s / sigma
//     against the same masked codes, and a bias sum_c q_c m_c, rebuilt only
//     when the page changes.
//  2. Softmax: the four tile maxima meet in LDS; every wave raises the same
//     running max and publishes fp16 weights P'_g = p s_g / sigma per latent
//     group.  Sums of p and of p m_g stay per lane until the end.
//  3. Output: wave w owns latent group w (128 output channels).  Its B operand
//     comes straight from the four code tiles of the round with
//     ds_read_b64_tr_b4 (16 tokens of one 4-bit channel, or of a 2-bit channel
//     pair, per lane) and the same masking unpack; A = P'_w, whose 1/sigma
//     per token slot cancels the slot's sigma.  The output accumulates
//     2^-24 sum_j fp16(p_j s_j) code_j; 2^24 and sum_j p_j m_j are applied at
//     the end.
// BF16-path workgroup: the same rounds over the protected tokens (sink,
// recent window and, when the window is shorter than a page, tokens of the
// unfinished page); their rows are converted to fp16 on their way into an fp16
// x tile that both the score MFMAs and the transposed output reads use.
// Tile, page and address arithmetic is wave-uniform (scalar registers).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "decode_plan.h"
#include "mla_bf16.h"
#include "geometry.h"

namespace mla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kStatW = 5;      // per head: sum p, sum p m_g (4)
constexpr float kCodeScale = 16777216.0f;   // 2^24: undoes the subnormal unpack
constexpr float kNegInf = -INFINITY;

// The power of two that brings magnitude x into the binade [2^(top-1), 2^top)
// (1 for x = 0): fp16 operands are scaled by it so that they neither overflow
// nor lose bits to the subnormal range, and the fp32 results are scaled back.
__device__ inline float pow2_to_binade(float x, int top) {
  if (!(x > 0.f)) return 1.f;
  int k = top - __builtin_amdgcn_frexp_expf(x);  // x = f 2^e, f in [0.5, 1)
  k = k < -100 ? -100 : (k > 100 ? 100 : k);
  return __builtin_amdgcn_ldexpf(1.f, k);
}

// Largest |bf16| among the 8 halves of a 16-byte row piece (bf16 magnitudes
// order like their bit patterns).
__device__ inline uint32_t bf16_absmax8(u32x4 w) {
  uint32_t a = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) a = max(a, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
  return a;
}

// BF16-path workgroup LDS map (bytes).  x-tile row: 512 fp16 + 16 B pad (260
// dwords: rows land 4 banks apart, so row writes and transposed reads are
// conflict-free).
constexpr int kXRow = 1040;
constexpr int kXTile = kTile * kXRow;
constexpr int kOffX = 0;                                   // [wave] x tiles
constexpr int kPTile = 4 * 64 * 8;                         // [group][lane] fp16 x 4
constexpr int kOffP = kOffX + kWaves * kXTile;             // [wave] P' tiles
constexpr int kOffMax = kOffP + kWaves * kPTile;           // [head][wave] tile maxima
constexpr int kOffQr = kOffMax + kHeadBlock * kWaves * 4;  // [head] q_rope, bf16 x 64
constexpr int kDenseLds = kOffQr + kHeadBlock * kRopeDim * 2;
static_assert(kTile * 128 <= kPTile, "a BF16 tile's k_R rows fit the P' area");

// Packed workgroup LDS map.  A tile slot: latent codes (16 rows, 16-byte
// units XOR-swizzled by row), k_R codes [16][32 B], latent metadata
// [16][16 B], the page's k_R metadata (256 B); +64 B so that the slots of
// consecutive waves start on different banks.
constexpr int kSlots = 3;
constexpr int kSlotBytes = 4096 + 512 + 256 + 256 + 64;
constexpr int kPkOffStage = 0;                                  // [slot][wave]
constexpr int kPkOffP = kPkOffStage + kSlots * kWaves * kSlotBytes;  // [kb][g][gq][head] x 16 B
constexpr int kPkPBytes = 2 * 4 * 4 * kHeadBlock * 16;
constexpr int kPkOffMax = kPkOffP + kPkPBytes;
constexpr int kPkOffQr = kPkOffMax + kHeadBlock * kWaves * 4;
constexpr int kPkOffPid = kPkOffQr + kHeadBlock * kRopeDim * 2;
constexpr int kPackedLds = kPkOffPid + kPageWin * 4;

constexpr int kLdsBytes = kDenseLds > kPackedLds ? kDenseLds : kPackedLds;
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per gfx950 CU");
static_assert(kWaves * kHeadBlock * kStatW * 4 <= kWaves * kPTile, "final sums fit the P' area");
static_assert(kWaves * kHeadBlock * kStatW * 4 <= kPkPBytes, "final sums fit the P' area");

struct DecodeParams {
  const uint16_t* q_lat;
  const uint16_t* q_rope;
  const uint8_t* pool;
  const int32_t* block_table;
  const int32_t* seqlens;
  const uint16_t* sink;
  const uint16_t* ring;
  const uint16_t* tail;
  const uint8_t* fallback;  // load source for a tile without a page (see dma_tile)
  uint32_t off_mask;        // ~0, or 0 when there is no page pool (max_seqlen = 0)
  uint8_t* parts;
  float* out;
  float* lse;
  int32_t batch, heads, max_pages, num_pool_pages, max_seqlen;
  int32_t n_hb, n_dense, n_splits;
  int32_t P, log2P, sink_n, local;
  int32_t t_lo, t_count;  // packed tiles of the longest possible sequence: [t_lo, t_lo + t_count)
  int64_t latent_meta_off, rope_codes_off, rope_meta_off, page_bytes;
  float c_log2;  // softmax_scale * log2(e)
};

// Channel (within a lane group's 32-channel span) of slot s of chunk d, in
// the order the unpack below produces.
template <int BITS>
__device__ constexpr int chan_off(int d, int s) {
  return BITS == 4 ? 8 * d + (s >> 1) + 4 * (s & 1)
                   : 16 * (d >> 1) + 4 * (d & 1) + (s >> 1) + 8 * (s & 1);
}

// x-tile column (slot order) -> latent channel.
template <int BITS>
__device__ inline int col_to_channel(int c) {
  return (c & ~31) + chan_off<BITS>((c >> 3) & 3, c & 7);
}

// Latent-code unpack by masking: slot value = code * 2^-24 * sigma (an fp16
// subnormal, the code sitting at bit log2(sigma) of a zero-exponent half).
// 8 nibbles -> slots [n0 n4 n1 n5 n2 n6 n3 n7], sigma = 16 in slots 2, 3, 6, 7.
// (A nibble can sit only at bits 0-3 or 4-7 of a half: bits 10-14 are the
// exponent, so the upper two nibbles of each half are shifted down first.)
__device__ inline half8 unpack4(uint32_t w) {
  const uint32_t t = w >> 8;
  const u32x4 v = {w & 0x000F000Fu, w & 0x00F000F0u, t & 0x000F000Fu, t & 0x00F000F0u};
  return __builtin_bit_cast(half8, v);
}

// 8 of the 16 crumbs of w; hi = 0: crumbs [0 8 1 9 2 10 3 11], sigma 1, 4,
// 16, 64 per slot pair; hi = 1: crumbs [4 12 5 13 6 14 7 15], sigma 256, 4,
// 16, 64.
__device__ inline half8 unpack2(uint32_t w, int hi) {
  u32x4 v;
  if (hi == 0) {
    v = u32x4{w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
  } else {
    const uint32_t t = w >> 8;
    v = u32x4{w & 0x03000300u, t & 0x000C000Cu, t & 0x00300030u, t & 0x00C000C0u};
  }
  return __builtin_bit_cast(half8, v);
}

// sigma of slot sl of latent chunk d (the unpacks above).
template <int BITS>
__device__ constexpr float slot_sigma(int d, int sl) {
  if constexpr (BITS == 4) {
    return (sl & 2) ? 16.f : 1.f;
  } else {
    return (sl >> 1) == 0 ? ((d & 1) ? 256.f : 1.f) : ((sl >> 1) == 1 ? 4.f : ((sl >> 1) == 2 ? 16.f : 64.f));
  }
}

__device__ inline float bf16f(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ inline float lo_f16(uint32_t w) { return static_cast<float>(__builtin_bit_cast(half2, w)[0]); }
__device__ inline float hi_f16(uint32_t w) { return static_cast<float>(__builtin_bit_cast(half2, w)[1]); }

__device__ inline f32x4 mfma(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ inline T ldg(const void* p) {
  return *reinterpret_cast<const T*>(p);
}
template <typename T>
__device__ inline T lds_ld(const uint8_t* p) {
  return *reinterpret_cast<const T*>(p);
}
template <typename T>
__device__ inline void lds_st(uint8_t* p, T v) {
  *reinterpret_cast<T*>(p) = v;
}

__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load, which would drain the next tile's prefetch.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 32-bit LDS address of a pointer into shared memory.
__device__ inline uint32_t lds_addr(const void* ptr) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)ptr));
}

// Sum / max over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the
// row-swap permutes (no LDS traffic); every row gets the same result.
__device__ inline float row_allsum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
__device__ inline float row_allmax(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// ---------------------------------------------------------------------------
// query operands

template <int BITS>
struct QueryOps {
  half8 lat[4][4];  // [group][chunk], slot order of the unpack
  half8 meta;       // (scale, min) slots of the metadata MFMA, scaled by 1 / meta_mul
  float meta_mul;   // per head (lane & 15): undoes the metadata operand's scale
};

// Query staging.  Wave w fetches latent group w of the 16 heads of a head
// block straight into the operand layout (lane (h, gq): channels
// 128 w + 32 gq .. + 31 of head h) and the q_rope rows (lane: head lane / 4,
// 16 channels).  Heads past the last one read a copy of the
// last head.
struct QueryRows {
  u32x4 lat[4], rope[2];
};

__device__ inline void fetch_query(QueryRows& qr, const DecodeParams& p, int b, int hb, int wave, int lane) {
  const int n16 = lane & 15, gq = lane >> 4;
  const int h = hb * kHeadBlock + n16;
  const int hc = h < p.heads ? h : p.heads - 1;
  const uint16_t* ql = p.q_lat + (static_cast<int64_t>(b) * p.heads + hc) * kLatentDim + 128 * wave + 32 * gq;
#pragma unroll
  for (int u = 0; u < 4; ++u) qr.lat[u] = ldg<u32x4>(ql + 8 * u);
  // every wave loads them (no branch, so that the loads' waits stay counted
  // in order); only wave 0 stores them
  const int hr = hb * kHeadBlock + (lane >> 2);
  const int hrc = hr < p.heads ? hr : p.heads - 1;
  const uint16_t* qp = p.q_rope + (static_cast<int64_t>(b) * p.heads + hrc) * kRopeDim + 16 * (lane & 3);
  qr.rope[0] = ldg<u32x4>(qp);
  qr.rope[1] = ldg<u32x4>(qp + 8);
}

// 16 bytes from global memory straight into LDS at lds_base + 16 * lane.
__device__ inline void load_to_lds(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
// 4 bytes per lane: lds_base + 4 * lane.
__device__ inline void load4_to_lds(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// Query rows of a packed workgroup by direct loads: wave w brings latent
// group w of the 16 heads into qraw ([group][head][128 channels] bf16, four
// loads) and the q_rope rows of heads 8 (w % 2) .. + 7 into qr_lds
// ([head][64] bf16; waves w and w + 2 write the same bytes).  Heads past the
// last one read a copy of the last head.
__device__ inline void dma_query(const DecodeParams& p, int b, int hb, uint8_t* qraw, uint8_t* qr_lds, int wave,
                                 int lane) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int h = hb * kHeadBlock + 4 * c + (lane >> 4);
    const int hc = h < p.heads ? h : p.heads - 1;
    const uint16_t* src = p.q_lat + (static_cast<int64_t>(b) * p.heads + hc) * kLatentDim + 128 * wave + 8 * (lane & 15);
    load_to_lds(src, qraw + wave * 4096 + 1024 * c);
  }
  const int h = hb * kHeadBlock + 8 * (wave & 1) + (lane >> 3);
  const int hc = h < p.heads ? h : p.heads - 1;
  load_to_lds(p.q_rope + (static_cast<int64_t>(b) * p.heads + hc) * kRopeDim + 8 * (lane & 7),
              qr_lds + 1024 * (wave & 1));
}

// LDS image of the converted query: [group][chunk][lane] fp16 x 8 operands,
// then [head][group] fp32 group sums.
constexpr int kQopsSums = 4 * 4 * 64 * 16;
constexpr int kQopsBytes = kQopsSums + kHeadBlock * 4 * 4;

// Wave w converts its latent group: fp16 operands in the unpack's slot order
// (times qscale, a power of two per head, and divided by the slot's sigma for
// the masking unpack when kSigma) and Q_w = sum of the group's 128 channels
// (unscaled), both into the LDS image; wave 0 also stores the q_rope rows as
// [head][128 B].
template <int BITS, bool kSigma, bool kRope = true>
__device__ inline void publish_query(const QueryRows& qr, uint8_t* qops, uint8_t* qr_lds, int wave, int lane,
                                     float qscale = 1.f) {
  const int n16 = lane & 15, gq = lane >> 4;
  float v[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * u + 2 * e] = bf16f(qr.lat[u][e] & 0xFFFFu);
      v[8 * u + 2 * e + 1] = bf16f(qr.lat[u][e] >> 16);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) s += v[c];
  const float qsum = row_allsum(s);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    half8 x;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl)
      x[sl] = static_cast<_Float16>(kSigma ? v[chan_off<BITS>(d, sl)] * (qscale / slot_sigma<BITS>(d, sl))
                                           : v[chan_off<BITS>(d, sl)]);
    lds_st<half8>(qops + ((wave * 4 + d) * 64 + lane) * 16, x);
  }
  if (gq == 0) lds_st<float>(qops + kQopsSums + (n16 * 4 + wave) * 4, qsum);
  if (kRope && wave == 0) {
    lds_st<u32x4>(qr_lds + (lane >> 2) * 128 + 32 * (lane & 3), qr.rope[0]);
    lds_st<u32x4>(qr_lds + (lane >> 2) * 128 + 32 * (lane & 3) + 16, qr.rope[1]);
  }
}

// MFMA operands of the whole query from the LDS image; Q_g enters the
// metadata operand (min slots; the scale slots stay zero) as fp16 hi + lo,
// scaled per head so that the largest |Q_g| lies in [2^13, 2^14).
template <int BITS>
__device__ inline void load_query(QueryOps<BITS>& q, const uint8_t* qops, int lane) {
  const int n16 = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 0; d < 4; ++d) q.lat[i][d] = lds_ld<half8>(qops + ((i * 4 + d) * 64 + lane) * 16);
  }
  const f32x4 qg = lds_ld<f32x4>(qops + kQopsSums + n16 * 16);
  const float mscale =
      pow2_to_binade(fmaxf(fmaxf(fabsf(qg[0]), fabsf(qg[1])), fmaxf(fabsf(qg[2]), fabsf(qg[3]))), 14);
  q.meta_mul = 1.f / mscale;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float c = qg[i] * mscale;
    const _Float16 ch = static_cast<_Float16>(c);
    const _Float16 cl = static_cast<_Float16>(c - static_cast<float>(ch));
    const _Float16 z = static_cast<_Float16>(0.f);
    q.meta[2 * i] = z;
    q.meta[2 * i + 1] = gq == 0 ? ch : (gq == 1 ? cl : z);
  }
}

// Per-page positional-key operands for channels 16*gq + 8e + slot order
// (masking unpack, as the latent codes): q' = q s r / sigma as fp16 hi + lo
// (a bf16 times an fp16 needs more bits than one fp16 holds), r a power of two
// per (head, page) that puts the largest |q s| of the head into [2^13, 2^14);
// mul = 2^24 / r undoes it and the unpack; bias = sum_c q_c m_c over the lane
// row's 64 channels.
struct RopeOps {
  half8 hi[2], lo[2];
  float bias, mul;
};

__device__ inline void rope_ops(RopeOps& r, const uint8_t* qr_row, const uint8_t* rmeta, int gq) {
  const u32x4 q0 = lds_ld<u32x4>(qr_row + 32 * gq), q1 = lds_ld<u32x4>(qr_row + 32 * gq + 16);
  const u32x4 s0 = lds_ld<u32x4>(rmeta + 32 * gq);
  const u32x4 s1 = lds_ld<u32x4>(rmeta + 32 * gq + 16);
  const u32x4 m0 = lds_ld<u32x4>(rmeta + 128 + 32 * gq);
  const u32x4 m1 = lds_ld<u32x4>(rmeta + 128 + 32 * gq + 16);
  float sc[16], mn[16], qv[16];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sc[2 * e] = lo_f16(s0[e]);
    sc[2 * e + 1] = hi_f16(s0[e]);
    sc[8 + 2 * e] = lo_f16(s1[e]);
    sc[8 + 2 * e + 1] = hi_f16(s1[e]);
    mn[2 * e] = lo_f16(m0[e]);
    mn[2 * e + 1] = hi_f16(m0[e]);
    mn[8 + 2 * e] = lo_f16(m1[e]);
    mn[8 + 2 * e + 1] = hi_f16(m1[e]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    qv[2 * k] = bf16f(q0[k] & 0xFFFFu);
    qv[2 * k + 1] = bf16f(q0[k] >> 16);
    qv[8 + 2 * k] = bf16f(q1[k] & 0xFFFFu);
    qv[8 + 2 * k + 1] = bf16f(q1[k] >> 16);
  }
  float bias = 0.f, qs[16], big = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    bias = fmaf(qv[c], mn[c], bias);
    qs[c] = qv[c] * sc[c];
    big = fmaxf(big, fabsf(qs[c]));
  }
  r.bias = row_allsum(bias);
  const float rs = pow2_to_binade(row_allmax(big), 14);
  r.mul = kCodeScale / rs;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int c = 8 * e + chan_off<4>(0, sl);
      const float v = qs[c] * (rs / slot_sigma<4>(0, sl));
      const _Float16 vh = static_cast<_Float16>(v);
      r.hi[e][sl] = vh;
      r.lo[e][sl] = static_cast<_Float16>(v - static_cast<float>(vh));
    }
  }
}

// ---------------------------------------------------------------------------
// packed tiles, staged in LDS by direct loads

template <int BITS>
struct TileGeom {
  static constexpr int kLatRow = kLatentDim * BITS / 8;  // bytes of one token's codes
  static constexpr int kLatBytes = kTile * kLatRow;     // 4096 or 2048
  static constexpr int kLatLoads = kLatBytes / 1024;    // direct loads of the latent codes
  static constexpr int kLoads = kLatLoads + 1;          // + k_R codes, latent and k_R metadata
  static constexpr int kOffRope = kLatBytes;            // [16][32 B]
  static constexpr int kOffMeta = kLatBytes + 512;      // [16][4 x (fp16 scale, fp16 min)]
  static constexpr int kOffRMeta = kLatBytes + 768;     // 64 fp16 scales, 64 fp16 mins
};

// Offset inside a slot of 16-byte unit u of latent row `row` (XOR swizzle).
template <int BITS>
__device__ inline int lat_unit(int row, int u) {
  if constexpr (BITS == 4) return row * 256 + ((u ^ row) << 4);
  else return row * 128 + ((u ^ (row & 7)) << 4);
}


// Source offset (inside the tile's latent rows) of the 16 bytes lane `lane`
// moves with direct load c: the lane writes slot unit 64 c + lane, which
// holds source unit (that unit) XOR row.
template <int BITS>
__device__ inline uint32_t lat_src(int c, int lane) {
  if constexpr (BITS == 4) {
    const int row = 4 * c + (lane >> 4);
    return static_cast<uint32_t>(row * 256 + (((lane & 15) ^ row) << 4));
  } else {
    const int pos = 64 * c + lane, row = pos >> 3;
    return static_cast<uint32_t>(row * 128 + (((pos & 7) ^ (row & 7)) << 4));
  }
}

// Per-lane byte offsets of a tile's direct loads: the latent-code loads
// relative to the tile's first code row, and the side load (lanes 0-31: k_R
// codes, 32-47: latent metadata, 48-63: the page's k_R metadata) relative to
// the page as side_a + slot0 * side_k.  All fit 32 bits (a page is < 64 KB),
// so every load takes a wave-uniform 64-bit base plus a 32-bit lane offset and
// the per-tile address work is one multiply-add.
struct TileSrc {
  uint32_t lat[4];
  uint32_t side_a, side_k;
};

template <int BITS>
__device__ inline TileSrc tile_src(const DecodeParams& p, int lane) {
  TileSrc t;
#pragma unroll
  for (int c = 0; c < 4; ++c) t.lat[c] = lat_src<BITS>(c, lane) & p.off_mask;
  uint32_t a = static_cast<uint32_t>(p.rope_meta_off) + 16u * static_cast<uint32_t>(lane - 48), k = 0;
  if (lane < 48) {
    a = static_cast<uint32_t>(p.latent_meta_off) + 16u * static_cast<uint32_t>(lane - 32);
    k = 16;
  }
  if (lane < 32) {
    a = static_cast<uint32_t>(p.rope_codes_off) + 16u * static_cast<uint32_t>(lane);
    k = kRopeRowBytes;
  }
  t.side_a = a & p.off_mask;
  t.side_k = k & p.off_mask;
  return t;
}

// Issues the direct loads of one 16-token tile (first slot slot0 of a
// wave-uniform page) into an LDS slot: always TileGeom<BITS>::kLoads
// vector-memory instructions, so the waits below can count them.
template <int BITS>
__device__ inline void dma_tile(uint8_t* slot, const uint8_t* page, int slot0, const TileSrc& ts,
                                const DecodeParams& p) {
  using G = TileGeom<BITS>;
  // a page missing from the block table loads from the fallback buffer instead
  // (page 0 of the pool, or the query when there is no pool and the offsets are
  // all zero; the tile is skipped); selected rather than branched, so that later
  // waits can count these loads
  const bool ok = page != nullptr;
  const uint8_t* const lat_base = ok ? page + slot0 * G::kLatRow : p.fallback;
  const uint8_t* const side_base = ok ? page : p.fallback;
  const uint32_t s0 = ok ? static_cast<uint32_t>(slot0) : 0u;
#pragma unroll
  for (int c = 0; c < G::kLatLoads; ++c) load_to_lds(lat_base + ts.lat[c], slot + 1024 * c);
  load_to_lds(side_base + (ts.side_a + s0 * ts.side_k), slot + G::kOffRope);
}

// Waits until at most `after` tiles' direct loads are still in flight (the
// loads of older tiles have landed in LDS).  Only direct loads are in flight
// in the packed loop, so the count is exact.
template <int BITS>
__device__ inline void wait_tiles_after(int after) {
  constexpr int K = TileGeom<BITS>::kLoads;
  if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * K) : "memory");
  else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Per-head multipliers that undo the operand scalings of the score MFMAs:
// latent (2^24 / the query's scale), metadata and positional key.
struct ScoreMul {
  float lat, meta, rope;
};

// Score from the MFMA sums: latent sum_g s_g q_g.code_g (v), metadata
// sum_g m_g Q_g (meta), positional q s.code (rope), each scaled as its
// operands were; bias = sum_c q_R,c m_R,c.
__device__ inline float score_of(float v, float meta, float rope, float bias, const ScoreMul& k) {
  return fmaf(rope, k.rope, fmaf(v, k.lat, fmaf(meta, k.meta, bias)));
}

// Score inputs of one packed tile from its LDS slot: lane (t, gq) gets the
// latent codes of channels 32 gq .. + 31 of every 128-channel group of token
// t, its k_R codes (channels 16 gq .. + 15) and its latent metadata.
template <int BITS>
struct ScoreIn {
  uint32_t lat[BITS == 4 ? 16 : 8];
  u32x2 rope;
  u32x4 ma;
};

template <int BITS>
__device__ inline void load_score_in(ScoreIn<BITS>& si, const uint8_t* slot, int n16, int gq) {
  using G = TileGeom<BITS>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BITS == 4) {
      const u32x4 v = lds_ld<u32x4>(slot + lat_unit<4>(n16, 4 * i + gq));
#pragma unroll
      for (int e = 0; e < 4; ++e) si.lat[4 * i + e] = v[e];
    } else {
      const u32x2 v = lds_ld<u32x2>(slot + lat_unit<2>(n16, 2 * i + (gq >> 1)) + 8 * (gq & 1));
      si.lat[2 * i] = v[0];
      si.lat[2 * i + 1] = v[1];
    }
  }
  si.rope = lds_ld<u32x2>(slot + G::kOffRope + n16 * kRopeRowBytes + 8 * gq);
  si.ma = lds_ld<u32x4>(slot + G::kOffMeta + 16 * n16);
}

// Score MFMAs of one packed tile: acc[g] = q_g . code_g per latent group g,
// acc[4] = sum_g m_g Q_g (metadata), acc[5] = q_R s . code_R (positional
// key), each scaled as its operands are (ScoreMul undoes it).
template <int BITS>
__device__ inline void score_mfma(f32x4 (&acc)[6], const ScoreIn<BITS>& si, const QueryOps<BITS>& q,
                                  const RopeOps& ro) {
#pragma unroll
  for (int g = 0; g < 6; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half8 x = BITS == 4 ? unpack4(si.lat[4 * i + d]) : unpack2(si.lat[2 * i + (d >> 1)], d & 1);
      acc[i] = mfma(x, q.lat[i][d], acc[i]);
    }
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const half8 xr = unpack4(si.rope[e]);
    acc[5] = mfma(xr, ro.hi[e], acc[5]);
    acc[5] = mfma(xr, ro.lo[e], acc[5]);
  }
  acc[4] = mfma(__builtin_bit_cast(half8, si.ma), q.meta, acc[4]);
}

// Scores (log2 domain: km and bias carry softmax_scale log2(e)) of one packed
// tile (tokens j0 .. j0+15 of a complete page, valid in [vlo, vhi); none when
// !has) from its MFMA sums: lane (h, gq) gets tokens 4 gq + r of head h.
// md[r] = the metadata words of token 4 gq + r.
// The metadata words of tokens 4 gq + r of a packed tile (loaded with the
// tile's score inputs, ahead of the score MFMAs).
template <int BITS>
__device__ inline void load_tile_meta(u32x4 (&md)[4], const uint8_t* slot, int gq) {
#pragma unroll
  for (int r = 0; r < 4; ++r) md[r] = lds_ld<u32x4>(slot + TileGeom<BITS>::kOffMeta + 16 * (4 * gq + r));
}

template <int BITS>
__device__ inline void score_finish(float (&sc)[4], const u32x4 (&md)[4], const f32x4 (&acc)[6], float bias,
                                    const ScoreMul& km, bool has, int j0, int vlo, int vhi, int gq) {
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = fmaf(lo_f16(md[r][g]), acc[g][r], v[r]);
  }
  if (has && j0 >= vlo && j0 + kTile <= vhi) {  // whole tile valid
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = score_of(v[r], acc[4][r], acc[5][r], bias, km);
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = j0 + 4 * gq + r;
    const float z = score_of(v[r], acc[4][r], acc[5][r], bias, km);
    sc[r] = (has && t >= vlo && t < vhi) ? z : kNegInf;
  }
}

// P' entry of (K block kb, latent group g, reader lane row gq, head h): the 8
// tokens 8 gq .. 8 gq + 7 of the K block (tiles 2 kb, 2 kb + 1), fp16.
__device__ inline int p_entry(int kb, int g, int gq, int h) { return (((kb * 4 + g) * 4 + gq) * kHeadBlock + h) * 16; }

// Headroom of the four tokens 4 gq .. 4 gq + 3 of a packed tile: k = E - 7,
// E the exponent with max_g s_g < 2^E over the tokens' latent scales (fp16
// bit patterns: field 0 gives E = -14, the subnormal bound).  The running max
// m of a packed workgroup is raised so that t + k <= m + 8 for every token (t
// its score), hence p = 2^(t - m) <= 2^(8 - k) and p s_g < 2^15: the fp16
// weights P'_g below never overflow, and the largest of a tile sits near
// 2^14, far above the subnormal range, at any latent magnitude.  k >= -21
// bounds p by 2^29, which fp32 sums hold.
// Lane (n16, gq) reads the scale word of token 4 gq + n16 % 4, group n16 / 4
// (with the tile's score inputs), and the row's 16 lanes take their maximum
// by rotations within the row.
template <int BITS>
__device__ inline uint32_t headroom_word(const uint8_t* slot, int n16, int gq) {
  return lds_ld<uint32_t>(slot + TileGeom<BITS>::kOffMeta + 16 * (4 * gq + (n16 & 3)) + 4 * (n16 >> 2));
}
__device__ inline float scale_headroom(uint32_t word) {
  uint32_t a = word & 0x7FFFu;
  a = max(a, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(a), 0x128, 0xF, 0xF, true)));  // row_ror:8
  a = max(a, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(a), 0x124, 0xF, 0xF, true)));  // row_ror:4
  a = max(a, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(a), 0x122, 0xF, 0xF, true)));  // row_ror:2
  a = max(a, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(a), 0x121, 0xF, 0xF, true)));  // row_ror:1
  return static_cast<float>(a >> 10) - 21.f;
}

// Two fp16 weights in one register: p0 s0 and p1 s1 (+ 0), each one
// v_fma_mix{lo,hi}_f16 rounded to fp16, with the scale s taken as the fp16 low
// half of its metadata word w.
__device__ inline uint32_t weight_pair(float p0, uint32_t w0, float p1, uint32_t w1) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0 op_sel_hi:[0,1,0]"
      : "=&v"(d)
      : "v"(p0), "v"(w0), "v"(p1), "v"(w1));
  return d;
}

// Weights of this wave's packed tile: P'_g = fp16(p s_g / sigma) into the P'
// entries its tokens fall in (tokens 4 gq + 2, 4 gq + 3 land in the output
// unpack's sigma = 16 slots); adds this lane's sums of p and of p m_g (fp32)
// to st.
__device__ inline void packed_weights(const float (&pr)[4], const u32x4 (&md)[4], uint8_t* pbase,
                                      float (&st)[kStatW], int wave, int n16, int gq) {
  st[0] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const float pw[4] = {pr[0], pr[1], pr[2] * 0.0625f, pr[3] * 0.0625f};
  const int at = 8 * (gq & 1);  // tokens 4 gq .. 4 gq + 3 of the tile
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float ms = st[1 + g];
#pragma unroll
    for (int r = 0; r < 4; ++r) ms = fmaf(pr[r], hi_f16(md[r][g]), ms);
    const u32x2 pa = {weight_pair(pw[0], md[0][g], pw[1], md[1][g]), weight_pair(pw[2], md[2][g], pw[3], md[3][g])};
    lds_st<u32x2>(pbase + p_entry(wave >> 1, g, 2 * (wave & 1) + (gq >> 1), n16) + at, pa);
    st[1 + g] = ms;
  }
}

// 8 crumbs (parity par of 8 nibbles) of w by masking, slots
// [n0 n4 n1 n5 n2 n6 n3 n7] of the nibbles, sigma = 16 in slots 2, 3, 6, 7
// (as unpack4).
__device__ inline half8 unpack2_pairs(uint32_t w, int par) {
  const uint32_t u = par == 0 ? w : w >> 2, t = u >> 8;
  const u32x4 v = {u & 0x00030003u, u & 0x00300030u, t & 0x00030003u, t & 0x00300030u};
  return __builtin_bit_cast(half8, v);
}

// Output MFMAs of latent group `wave` over the round's four tiles (slot s of
// every wave).  ds_read_b64_tr_b4: within each 16-lane row, lane i receives
// nibble i of the 8 bytes each of the row's lanes addressed.  Lane (j, gq)
// addresses token 8 gq + sigma(j) (j < 8, K block 0) or 32 + 8 gq +
// sigma(j - 8) (K block 1); sigma undoes the unpack's slot order, so slot k of
// the unpacked B operand is token 8 gq + k of its K block, as in P'.
// 4-bit codes: column n16 of block kk = channel 128 g + 16 kk + n16.
// 2-bit codes: chunk c, parity par -> o[2 c + par], channel 128 g + 32 c +
// 2 n16 + par.
template <int BITS>
__device__ inline void packed_pv(f32x4 (&o)[8], const uint8_t* smem, int s, int wave, int n16, int gq) {
  const half8 pa0 = lds_ld<half8>(smem + kPkOffP + p_entry(0, wave, gq, n16));
  const half8 pa1 = lds_ld<half8>(smem + kPkOffP + p_entry(1, wave, gq, n16));
  const int j = n16 & 7;
  const int tau = (n16 < 8 ? 0 : 32) + 8 * gq + (((j & 3) << 1) | (j >> 2));
  const int row = tau & 15;
  const uint8_t* base = smem + kPkOffStage + (s * kWaves + (tau >> 4)) * kSlotBytes;
  // The transposed reads go through inline assembly: for an LDS intrinsic the
  // compiler would first wait for every direct load in flight (the slots being
  // filled are not the ones read here).  One lgkmcnt wait covers all reads.
  if constexpr (BITS == 4) {
    // unit 4 wave + k2 of row `row` at (4 wave ^ (row & 12)) + (k2 ^ (row & 3))
    uint32_t a[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
      a[k2] = lds_addr(base + lat_unit<4>(row, 4 * wave + k2));
    i32x2 r[8];
    asm volatile(
        "ds_read_b64_tr_b4 %0, %8\n\t"
        "ds_read_b64_tr_b4 %1, %8 offset:8\n\t"
        "ds_read_b64_tr_b4 %2, %9\n\t"
        "ds_read_b64_tr_b4 %3, %9 offset:8\n\t"
        "ds_read_b64_tr_b4 %4, %10\n\t"
        "ds_read_b64_tr_b4 %5, %10 offset:8\n\t"
        "ds_read_b64_tr_b4 %6, %11\n\t"
        "ds_read_b64_tr_b4 %7, %11 offset:8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) o[kk] = mfma(pa0, unpack4(static_cast<uint32_t>(r[kk][0])), o[kk]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) o[kk] = mfma(pa1, unpack4(static_cast<uint32_t>(r[kk][1])), o[kk]);
  } else {
    uint32_t a[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      a[c2] = lds_addr(base + lat_unit<2>(row, 2 * wave + c2));
    i32x2 r[4];
    asm volatile(
        "ds_read_b64_tr_b4 %0, %4\n\t"
        "ds_read_b64_tr_b4 %1, %4 offset:8\n\t"
        "ds_read_b64_tr_b4 %2, %5\n\t"
        "ds_read_b64_tr_b4 %3, %5 offset:8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1])
        : "memory");
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int par = 0; par < 2; ++par)
        o[2 * c + par] = mfma(pa0, unpack2_pairs(static_cast<uint32_t>(r[c][0]), par), o[2 * c + par]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int par = 0; par < 2; ++par)
        o[2 * c + par] = mfma(pa1, unpack2_pairs(static_cast<uint32_t>(r[c][1]), par), o[2 * c + par]);
    }
  }
}

// ---------------------------------------------------------------------------
// BF16-path tiles

struct SeqRanges {
  int L, lo_p, hi_p;  // packed tokens are [lo_p, hi_p)
};

__device__ inline SeqRanges seq_ranges(const DecodeParams& p, int b) {
  SeqRanges r;
  int L = uniform(p.seqlens[b]);
  const int cap = min(p.max_seqlen, p.max_pages * p.P);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  r.L = L;
  r.lo_p = min(p.sink_n, L);
  const int full = (L >> p.log2P) << p.log2P;
  r.hi_p = max(r.lo_p, min(L - p.local, full));
  return r;
}

__device__ inline const uint8_t* page_of_id(const DecodeParams& p, int id) {
  if (id < 0 || id >= p.num_pool_pages) return nullptr;
  return p.pool + static_cast<int64_t>(id) * p.page_bytes;
}

__device__ inline const uint8_t* page_ptr(const DecodeParams& p, int b, int pidx) {
  if (pidx < 0 || pidx >= p.max_pages) return nullptr;
  return page_of_id(p, p.block_table[static_cast<int64_t>(b) * p.max_pages + pidx]);
}

// Source of BF16-path token k: its BF16 row ([c_KV | k_R]) or, for a token of
// the unfinished page outside the window, its packed latent and the BF16 k_R
// of the tail buffer.  kind: 0 none, 1 row, 2 packed latent.
struct DenseSrc {
  int kind;
  const uint16_t* row;
  const uint8_t* page;
  const uint16_t* rope;
  int slot;
};

__device__ inline DenseSrc dense_src(const DecodeParams& p, int b, const SeqRanges& sr, int k) {
  DenseSrc s{0, nullptr, nullptr, nullptr, 0};
  const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
  if (k < 0 || k >= n_dense) return s;
  const int j = k < sr.lo_p ? k : sr.hi_p + (k - sr.lo_p);
  if (j < p.sink_n) {
    s.kind = 1;
    s.row = p.sink + (static_cast<int64_t>(b) * p.sink_n + j) * kRowElems;
  } else if (p.local > 0 && j >= sr.L - p.local) {
    s.kind = 1;
    s.row = p.ring + (static_cast<int64_t>(b) * p.local + j % p.local) * kRowElems;
  } else {
    s.page = page_ptr(p, b, j >> p.log2P);
    if (s.page) {
      s.kind = 2;
      s.slot = j & (p.P - 1);
      s.rope = p.tail + (static_cast<int64_t>(b) * p.P + s.slot) * kRopeDim;
    }
  }
  if (s.kind == 1) s.rope = s.row + kLatentDim;
  return s;
}

// Scores of one BF16-path tile (dense indices k0 .. k0+15).  Rows are
// converted to fp16 in the unpack's slot order into the x tile (latent) and
// copied raw into rbuf (k_R), then fed to the same MFMAs.  (Loads go through
// registers: an LDS-direct load would make every later LDS read of the kernel
// wait for all outstanding global loads, prefetches included.)
template <int BITS>
__device__ void dense_scores(float (&sc)[4], const QueryOps<BITS>& q, const uint8_t* qr_row, int b,
                             const SeqRanges& sr, int k0, uint8_t* xt, uint8_t* rbuf, int lane, int n16, int gq,
                             const DecodeParams& p) {
  // k_R rows: token 8 u + lane / 8, bytes 16 (lane % 8) .. +15
#pragma unroll
  for (int u = 0; u < kTile / 8; ++u) {
    const DenseSrc s = dense_src(p, b, sr, k0 + 8 * u + (lane >> 3));
    const u32x4 w = s.kind ? ldg<u32x4>(s.rope + 8 * (lane & 7)) : u32x4{0, 0, 0, 0};
    lds_st<u32x4>(rbuf + u * 1024 + 16 * lane, w);
  }
  // latent rows: lane handles channels 16 part .. 16 part + 15 of rows
  // lane / 32 + 2 m, all eight of its rows requested before any is converted
  const int part = lane & 31;
  {
    constexpr int m0 = 0;
    u32x4 ra[kTile / 2], rc[kTile / 2];
    int kind[kTile / 2];
#pragma unroll
    for (int u = 0; u < kTile / 2; ++u) {
      const int t = 2 * (m0 + u) + (lane >> 5);
      const DenseSrc s = dense_src(p, b, sr, k0 + t);
      kind[u] = s.kind;
      ra[u] = u32x4{0, 0, 0, 0};
      rc[u] = u32x4{0, 0, 0, 0};
      if (s.kind == 1) {
        ra[u] = ldg<u32x4>(s.row + 16 * part);
        rc[u] = ldg<u32x4>(s.row + 16 * part + 8);
      } else if (s.kind == 2) {
        const uint8_t* row = s.page + s.slot * (kLatentDim * BITS / 8);
        if constexpr (BITS == 4) {
          const u32x2 w = ldg<u32x2>(row + 8 * part);
          ra[u][0] = w[0];
          ra[u][1] = w[1];
        } else {
          ra[u][0] = ldg<uint32_t>(row + 4 * part);
        }
        ra[u][2] = ldg<uint32_t>(s.page + p.latent_meta_off + s.slot * 16 + 4 * (part >> 3));
      }
    }
#pragma unroll
    for (int u = 0; u < kTile / 2; ++u) {
      const int t = 2 * (m0 + u) + (lane >> 5);
      float v[16];
      if (kind[u] == 2) {
        const float scl = lo_f16(ra[u][2]), mn = hi_f16(ra[u][2]);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const uint32_t code = BITS == 4 ? (ra[u][c >> 3] >> (4 * (c & 7))) & 15u : (ra[u][0] >> (2 * c)) & 3u;
          v[c] = fmaf(static_cast<float>(code), scl, mn);
        }
      } else {  // BF16 row, or zeros for a token past the end
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf16f(ra[u][e] & 0xFFFFu);
          v[2 * e + 1] = bf16f(ra[u][e] >> 16);
          v[8 + 2 * e] = bf16f(rc[u][e] & 0xFFFFu);
          v[8 + 2 * e + 1] = bf16f(rc[u][e] >> 16);
        }
      }
      // columns 16 part .. 16 part + 15 are chunks 2 (part & 1) and 2 (part & 1) + 1
      // of lane group (part >> 1) & 3 in latent group part >> 3
      half8 x0, x1;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        x0[sl] = static_cast<_Float16>(v[chan_off<BITS>(0, sl)]);
        x1[sl] = static_cast<_Float16>(v[chan_off<BITS>(1, sl)]);
      }
      uint8_t* cell = xt + t * kXRow + 32 * part;
      lds_st<half8>(cell, x0);
      lds_st<half8>(cell + 16, x1);
    }
  }
  lds_wait();
  // score MFMAs from LDS
  half8 qrp[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const u32x4 w = lds_ld<u32x4>(qr_row + 32 * gq + 16 * e);
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int c = chan_off<4>(0, sl);
      qrp[e][sl] = static_cast<_Float16>(bf16f((c & 1) ? (w[c >> 1] >> 16) : (w[c >> 1] & 0xFFFFu)));
    }
  }
  const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* lrow = xt + n16 * kXRow + 64 * gq;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int d = 0; d < 4; ++d) acc = mfma(lds_ld<half8>(lrow + 256 * i + 16 * d), q.lat[i][d], acc);
  }
  const uint8_t* rrow = rbuf + n16 * 128 + 32 * gq;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const u32x4 w = lds_ld<u32x4>(rrow + 16 * e);
    half8 xr;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int c = chan_off<4>(0, sl);
      xr[sl] = static_cast<_Float16>(bf16f((c & 1) ? (w[c >> 1] >> 16) : (w[c >> 1] & 0xFFFFu)));
    }
    acc = mfma(xr, qrp[e], acc);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = k0 + 4 * gq + r < n_dense;
    sc[r] = ok ? acc[r] * p.c_log2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// workgroups

struct WgCtx {
  int b, hb, grp, split, lane, wave, n16, gq;
};

// Common round step 2 bookkeeping: the tile maxima of the four waves meet in
// LDS (smax [head][wave]); returns the rescale factor of head n16 (score
// layout) and updates m_run, and the factors ah of heads 4 gq + r (output
// layout) and m_o.  The reference max only moves when a tile max exceeds it
// by more than kMaxSlack (log2 units): weights stay below 2^kMaxSlack, and
// most rounds keep every factor at exactly 1 so that the rescale is skipped.
// (Packed workgroups publish t + k, k the tiles' scale headroom, instead of
// the score t: see scale_headroom.)  Both layouts apply the same rule to the
// same maxima, so they agree.
constexpr float kMaxSlack = 8.f;
__device__ inline float lazy_max(float m, float tile_max) { return tile_max > m + kMaxSlack ? tile_max : m; }

// 2^x on the transcendental unit; results below the fp32 normal range flush
// to zero, which only drops softmax weights under 2^-126.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Every head of the wave keeps its max (all factors 1) unless `raised`; the
// output-layout maxima are only touched then.
__device__ inline float raise_max(float& m_run, float (&m_o)[4], float (&ah)[4], bool& raised, const float* smax,
                                  int n16, int gq) {
  const f32x4 mv = lds_ld<f32x4>(reinterpret_cast<const uint8_t*>(smax + n16 * kWaves));
  const float rmax = lazy_max(m_run, fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
  raised = __any(rmax != m_run);
  const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - rmax);
  m_run = rmax;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) ah[rr] = 1.f;
  if (raised) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x4 mo = lds_ld<f32x4>(reinterpret_cast<const uint8_t*>(smax + (4 * gq + rr) * kWaves));
      const float ro = lazy_max(m_o[rr], fmaxf(fmaxf(mo[0], mo[1]), fmaxf(mo[2], mo[3])));
      ah[rr] = m_o[rr] == kNegInf ? 0.f : fast_exp2(m_o[rr] - ro);
      m_o[rr] = ro;
    }
  }
  return alpha;
}

__device__ inline void rescale_stats(float (&st)[kStatW], float alpha, bool raised) {
  if (raised) {
#pragma unroll
    for (int k = 0; k < kStatW; ++k) st[k] *= alpha;
  }
}

__device__ inline void rescale_out(f32x4 (&o)[8], const float (&ah)[4], bool raised) {
  if (raised) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) o[k][rr] *= ah[rr];
    }
  }
}

// BF16-path workgroup `ds` of n_dense: BF16 tiles (dense token indices, see
// dense_src) split evenly; fp16 x tiles in LDS serve both MFMAs.
template <int BITS>
__device__ void dense_wg(f32x4 (&o)[8], float (&st)[kStatW], float (&m_o)[4], const DecodeParams& p, uint8_t* smem,
                         const SeqRanges& sr, const WgCtx& cx, int ds) {
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  const int lane = cx.lane, wave = cx.wave, n16 = cx.n16, gq = cx.gq;
  uint8_t* const xt_own = smem + kOffX + wave * kXTile;
  uint8_t* const p_own = smem + kOffP + wave * kPTile;
  float* const smax = reinterpret_cast<float*>(smem + kOffMax);
  const uint8_t* const qr_row = smem + kOffQr + n16 * 128;
  uint8_t* const qops = smem + kOffX;  // converted query, until round 0 writes x tiles

  const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
  const int D = (n_dense + kTile - 1) / kTile;
  const int per = (D + p.n_dense - 1) / p.n_dense;
  const int i0 = min(D, ds * per), i1 = min(D, i0 + per);
  const int rounds = (i1 - i0 + kWaves - 1) / kWaves;
  const int my0 = i0 + wave * rounds, my1 = min(i1, my0 + rounds);
  // Round 0's BF16 rows (9 lines of 128 bytes each; lane: token lane / 4,
  // lines lane % 4 + 4 j) are touched before the query is requested: loads
  // complete in order, so the query's wait also covers them, and round 0
  // then finds them in cache instead of waiting a second HBM round trip.
  uint32_t touch = 0;
  if (my0 < my1) {
    const DenseSrc s = dense_src(p, cx.b, sr, my0 * kTile + (lane >> 2));
    if (s.kind == 1) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int line = (lane & 3) + 4 * j;
        if (line < kRowElems * 2 / 128) touch ^= ldg<uint32_t>(reinterpret_cast<const uint8_t*>(s.row) + 128 * line);
      }
    }
  }
  {
    QueryRows qrows;
    fetch_query(qrows, p, cx.b, cx.hb, wave, lane);
    publish_query<BITS, false>(qrows, qops, smem + kOffQr, wave, lane);
  }
  static_assert(kQopsBytes <= kWaves * kXTile, "the converted query fits the x tiles");
  asm volatile("" ::"v"(touch));  // keeps the touching loads
  lds_barrier();  // query converted
  QueryOps<BITS> q;
  load_query<BITS>(q, qops, lane);
  lds_barrier();  // query read: the x tiles may be written
  if (my0 >= my1) {  // a wave without tiles still feeds zeros to the output MFMAs
    for (int off = 16 * lane; off < kXTile; off += 64 * 16) lds_st<u32x4>(xt_own + off, u32x4{0, 0, 0, 0});
  }
  float m_run = kNegInf;
  for (int r = 0; r < rounds; ++r) {
    const int it = my0 + r;
    const bool has = it < my1;
    float sc[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
    if (has) dense_scores<BITS>(sc, q, qr_row, cx.b, sr, it * kTile, xt_own, p_own, lane, n16, gq, p);
    const float tmax = row_allmax(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    if (gq == 0) smax[n16 * kWaves + wave] = tmax;
    lds_barrier();

    float ah[4];
    bool raised;
    const float alpha = raise_max(m_run, m_o, ah, raised, smax, n16, gq);
    rescale_stats(st, alpha, raised);
    half4 pa = {};
    if (has) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float pr = sc[k] == kNegInf ? 0.f : fast_exp2(sc[k] - m_run);
        st[0] += pr;
        pa[k] = static_cast<_Float16>(pr * (1.f / kappa));
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) lds_st<half4>(p_own + g * 512 + 8 * lane, pa);
    lds_barrier();

    // output of latent group `wave`, tiles in pairs: A slots 0-3 tile t
    // (tokens 4 gq + j), slots 4-7 tile t + 1
    rescale_out(o, ah, raised);
#pragma unroll
    for (int t = 0; t < kWaves; t += 2) {
      const half4 p0 = lds_ld<half4>(smem + kOffP + t * kPTile + wave * 512 + 8 * lane);
      const half4 p1 = lds_ld<half4>(smem + kOffP + (t + 1) * kPTile + wave * 512 + 8 * lane);
      const half8 pa8 = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
      const uint8_t* b0 = smem + kOffX + t * kXTile + (4 * gq + (n16 >> 2)) * kXRow + 8 * (n16 & 3) + 256 * wave;
      const uint8_t* b1 = b0 + kXTile;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const i16x4 r1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(b0 + 32 * kk));
        const i16x4 r2 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(b1 + 32 * kk));
        // whole-vector shuffle + bit cast: assembling the operand element by
        // element from the transposed reads produced wrong code with this compiler
        const half8 vb = __builtin_bit_cast(half8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
        o[kk] = mfma(pa8, vb, o[kk]);
      }
    }
    lds_barrier();
  }
}

// Packed workgroup `ps` of n_ps: packed tiles split evenly, each wave a
// contiguous run; per wave a ring of kSlots LDS slots filled by direct loads.
// Rounds of three phases and two barriers:
//   A: the scores of this wave's tile r (slot r % 3)
//   B: the common running max, P' of round r, the rescale of the output
//      accumulators
//   C: the output MFMAs of round r (P' and every wave's slot r % 3), then
//      the direct loads of tile r+2 into slot (r+2) % 3 = (r-1) % 3 (free:
//      every wave's round r-1 output MFMAs ran before this round's first
//      barrier)
// so each slot is busy for one round and the next tiles stay in flight.
template <int BITS>
__device__ void packed_wg(f32x4 (&o)[8], float (&st)[kStatW], float (&m_o)[4], const DecodeParams& p, uint8_t* smem,
                          const SeqRanges& sr, const WgCtx& cx, int ps, int n_ps) {
  const int lane = cx.lane, wave = cx.wave, n16 = cx.n16, gq = cx.gq;
  float* const smax = reinterpret_cast<float*>(smem + kPkOffMax);
  int* const s_pid = reinterpret_cast<int*>(smem + kPkOffPid);
  const uint8_t* const qr_row = smem + kPkOffQr + n16 * 128;
  uint8_t* const qops = smem + kPkOffStage + 2 * kWaves * kSlotBytes;  // slot 2 of every wave
  static_assert(kQopsBytes <= kWaves * kSlotBytes, "the converted query fits one slot row");
  auto slot_ptr = [&](int s, int w) { return smem + kPkOffStage + (s * kWaves + w) * kSlotBytes; };

  // The tiles are split by the batch's longest possible packed range
  // (p.t_lo, p.t_count, from max_seqlen), not by this sequence's length, so
  // that the first page id, the page-id window and the query rows are all
  // requested at once; tiles past the sequence's own packed range are skipped.
  const int t_lo = p.t_lo, T = p.t_count;
  const int per = (T + n_ps - 1) / n_ps;
  const int k0 = min(T, ps * per), k1 = min(T, k0 + per);
  int rounds = (k1 - k0 + kWaves - 1) / kWaves;
  {
    // Long runs are rounded up to whole pages per wave, when that costs at
    // most 1/16 more rounds: then every wave changes page in the same round
    // and the positional-key operands are rebuilt in one round of every P/16,
    // instead of some wave rebuilding (and holding the barriers) in most
    // rounds.
    const int tpp = p.P / kTile;
    const int r_al = (rounds + tpp - 1) / tpp * tpp;
    if ((r_al - rounds) * 16 <= rounds) rounds = r_al;
  }
  const int my0 = k0 + wave * rounds, my1 = min(k1, my0 + rounds);
  // The opening loads carry no branch (clamped indices; a block table that
  // may be absent is replaced by the seqlens array), so the compiler's waits
  // for the query and page ids leave the first tile's loads in flight.
  const int32_t* const bt_seq =
      p.max_pages > 0 ? p.block_table + static_cast<int64_t>(cx.b) * p.max_pages : p.seqlens;
  const int last_pg = max(p.max_pages - 1, 0);
  // page id of this wave's first tile (a wave without tiles loads one anyway)
  const int id0 = uniform(bt_seq[min(((t_lo + my0) * kTile) >> p.log2P, last_pg)]);

  // page ids of this workgroup's tiles (the launch sizes splits so that they
  // fit the window); loaded together with the query rows
  int pg_first = 0, n_pg = 0;
  if (k1 > k0) {
    pg_first = ((t_lo + k0) * kTile) >> p.log2P;
    n_pg = min((((t_lo + k1 - 1) * kTile) >> p.log2P) - pg_first + 1, kPageWin);
  }
  // The page-id window and the query rows come by direct loads (entries past
  // n_pg repeat an in-range one and are never used): with only direct loads
  // in flight, the counted wait below leaves the first tile's loads flying
  // while the query is converted.
  constexpr int kPidPerWave = kPageWin / kWaves;
  static_assert(kPidPerWave % 64 == 0, "whole 4-byte direct loads per wave");
#pragma unroll
  for (int i = 0; i < kPidPerWave / 64; ++i) {
    const int k = wave * kPidPerWave + 64 * i + lane;
    load4_to_lds(bt_seq + min(pg_first + min(k, max(n_pg - 1, 0)), last_pg),
                 reinterpret_cast<uint8_t*>(s_pid) + 4 * (wave * kPidPerWave + 64 * i));
  }
  uint8_t* const qraw = smem + kPkOffStage + 1 * kWaves * kSlotBytes;  // slot 1 of every wave
  static_assert(kWaves * 4096 <= kWaves * kSlotBytes, "the raw query rows fit one slot row");
  dma_query(p, cx.b, cx.hb, qraw, smem + kPkOffQr, wave, lane);
  const TileSrc src = tile_src<BITS>(p, lane);
  // the first tile goes out as soon as its page id is in; only it joins the
  // opening burst (every workgroup starts at once), the second follows round
  // 0's scores
  // this sequence's packed tiles end at my_end (the sequence may be shorter
  // than the longest one)
  const int t_end = max((sr.hi_p + kTile - 1) / kTile - t_lo, 0) * (sr.hi_p > sr.lo_p);
  const int my_end = min(my1, t_end);
  dma_tile<BITS>(slot_ptr(0, wave), page_of_id(p, id0), ((t_lo + my0) * kTile) & (p.P - 1), src, p);
  wait_tiles_after<BITS>(1);  // this wave's page ids and query rows are in
  lds_barrier();              // every wave's are
  // staged page id of tile it (not yet wave-uniform: read early, used later)
  auto pid_at = [&](int it) { return s_pid[min(max((((t_lo + it) * kTile) >> p.log2P) - pg_first, 0), kPageWin - 1)]; };
  auto issue = [&](int it, int id, int s) {
    dma_tile<BITS>(slot_ptr(s, wave), page_of_id(p, id), ((t_lo + it) * kTile) & (p.P - 1), src, p);
  };
  // the query is converted while the first tile is in flight; slot 2, which
  // holds it, is first filled after the round-0 barrier
  // The fp16 query operands carry q / sigma (sigma up to 16 for 4-bit and 256
  // for 2-bit codes), so each head's query is first scaled by a power of two
  // that puts its largest |q| into [2^14, 2^15): the operands then stay exact
  // (no subnormals) for any query magnitude.  The waves' group maxima meet in
  // the (still unused) tile-maxima area.
  float qscale;
  {
    QueryRows qrows;
    const int n16 = lane & 15, gq = lane >> 4;
    uint32_t big = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qrows.lat[u] = lds_ld<u32x4>(qraw + wave * 4096 + n16 * 256 + 64 * gq + 16 * u);
      big = max(big, bf16_absmax8(qrows.lat[u]));
    }
    const float gmax = row_allmax(bf16f(big));
    if (gq == 0) smax[n16 * kWaves + wave] = gmax;
    lds_barrier();  // every group's maximum is in
    const f32x4 mv = lds_ld<f32x4>(reinterpret_cast<const uint8_t*>(smax + n16 * kWaves));
    qscale = pow2_to_binade(fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])), 15);
    publish_query<BITS, true, false>(qrows, qops, nullptr, wave, lane, qscale);
  }
  lds_barrier();  // query converted
  QueryOps<BITS> q;
  load_query<BITS>(q, qops, lane);
  // the multipliers carry the softmax scale in the log2 domain, so the
  // scores leave score_finish ready for exp2
  ScoreMul km;
  km.lat = kCodeScale / qscale * p.c_log2;
  km.meta = q.meta_mul * p.c_log2;

  float m_run = kNegInf;
  RopeOps ro;
  int ro_page = -1;
  for (int r = 0; r < rounds; ++r) {
    // A: scores of tile r (tile r+1, and after round 0 tile r+2, may still
    // be in flight)
    const int it = my0 + r;
    bool has = it < my_end;
    if (has) wait_tiles_after<BITS>(r > 0 && it + 1 < my_end ? 1 : 0);
    const uint8_t* const slot = slot_ptr(r % kSlots, wave);
    const int pidx = ((t_lo + it) * kTile) >> p.log2P;
    if (has && pidx != ro_page) {  // (a page missing from the block table only spoils its own tiles)
      rope_ops(ro, qr_row, slot + TileGeom<BITS>::kOffRMeta, gq);
      ro.mul *= p.c_log2;
      ro.bias *= p.c_log2;
      ro_page = pidx;
    }
    // page ids of this tile and of the tiles issued this round, read with
    // the tile's LDS inputs
    const int id_cur = pid_at(it), id_1 = pid_at(it + 1), id_2 = pid_at(it + 2);
    // every LDS input of the tile's scores is requested before the MFMAs
    ScoreIn<BITS> si;
    load_score_in<BITS>(si, slot, n16, gq);
    u32x4 md[4];
    load_tile_meta<BITS>(md, slot, gq);
    const uint32_t hw = headroom_word<BITS>(slot, n16, gq);
    has = has && page_of_id(p, uniform(id_cur)) != nullptr;
    f32x4 acc[6];
    score_mfma<BITS>(acc, si, q, ro);
    float sc[4];
    km.rope = ro.mul;
    score_finish<BITS>(sc, md, acc, ro.bias, km, has, (t_lo + it) * kTile, sr.lo_p, sr.hi_p, gq);
    if (r == 0 && it + 1 < my_end) issue(it + 1, uniform(id_1), 1);
    const float tmax = row_allmax(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) + scale_headroom(hw));
    if (gq == 0) smax[n16 * kWaves + wave] = tmax;
    lds_barrier();

    // B: the common running max and P' of round r
    float ah[4];
    bool raised;
    const float alpha = raise_max(m_run, m_o, ah, raised, smax, n16, gq);
    rescale_stats(st, alpha, raised);
    if (has) {
      float pr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pr[k] = sc[k] == kNegInf ? 0.f : fast_exp2(sc[k] - m_run);
      packed_weights(pr, md, smem + kPkOffP, st, wave, n16, gq);
    } else {  // no tile: zero weights (the slot's stale codes unpack to finite values)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        lds_st<u32x2>(smem + kPkOffP + p_entry(wave >> 1, g, 2 * (wave & 1) + (gq >> 1), n16) + 8 * (gq & 1),
                      u32x2{0, 0});
    }
    rescale_out(o, ah, raised);
    lds_barrier();

    // C: output MFMAs of round r (P' and every wave's slot r % 3), then tile
    // r+2 into slot (r+2) % 3 = (r-1) % 3, which every wave's output MFMAs of
    // round r-1 have left (they ran before this round's first barrier)
    packed_pv<BITS>(o, smem, r % kSlots, wave, n16, gq);
    if (it + 2 < my_end) issue(it + 2, uniform(id_2), (r + 2) % kSlots);
  }
  // no direct load outlives the workgroup, and every wave's last reads of P'
  // and of the slots are done before finish reuses that LDS
  __syncthreads();
}

// Per-head sums of every wave meet in LDS (sums_lds, [wave][sum][head]); each
// lane then turns its accumulators (heads 4 gq + r of one channel per column
// block kk) into the split's partial, stored straight from registers in the
// channel-major layout [channel][16 heads] fp16 (four heads = 8 bytes per
// lane and block), or, with one split, into the normalized output and lse.
// chan(kk, n16) maps an accumulator column to its latent channel.
template <int BITS, bool kPackedMap>
__device__ void finish(const DecodeParams& p, uint8_t* sums_lds, const f32x4 (&o)[8], const float (&st)[kStatW],
                       const float (&m_o)[4], const WgCtx& cx) {
  // packed: output MFMAs summed 2^-24 fp16(p s) code; BF16 path: p / kappa x
  constexpr float out_scale = kPackedMap ? kCodeScale : (BITS == 4 ? 16.f : 4.f);
  const int wave = cx.wave, n16 = cx.n16, gq = cx.gq;
#pragma unroll
  for (int k = 0; k < kStatW; ++k) {
    const float v = row_allsum(st[k]);
    if (gq == 0) lds_st<float>(sums_lds + ((wave * kStatW + k) * kHeadBlock + n16) * 4, v);
  }
  lds_barrier();
  // sums over the waves for heads 4 gq .. 4 gq + 3: l and sum p m_g of this
  // wave's latent group g = wave
  f32x4 lq = {0.f, 0.f, 0.f, 0.f}, mq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    lq += lds_ld<f32x4>(sums_lds + ((w * kStatW) * kHeadBlock + 4 * gq) * 4);
    mq += lds_ld<f32x4>(sums_lds + ((w * kStatW + 1 + wave) * kHeadBlock + 4 * gq) * 4);
  }
  float inv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) inv[rr] = lq[rr] > 0.f ? 1.f / lq[rr] : 0.f;
  const bool direct = p.n_splits == 1;
  uint8_t* const part = p.parts + (static_cast<int64_t>(cx.grp) * p.n_splits + cx.split) * kPartBytes;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    int ch;
    if constexpr (kPackedMap)
      ch = BITS == 4 ? 128 * wave + 16 * kk + n16 : 128 * wave + 32 * (kk >> 1) + 2 * n16 + (kk & 1);
    else
      ch = col_to_channel<BITS>(128 * wave + 16 * kk + n16);
    float v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) v[rr] = fmaf(out_scale, o[kk][rr], mq[rr]) * inv[rr];
    if (direct) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int hg = cx.hb * kHeadBlock + 4 * gq + rr;
        if (hg < p.heads) p.out[(static_cast<int64_t>(cx.b) * p.heads + hg) * kLatentDim + ch] = v[rr];
      }
    } else {
      const half4 h = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
                       static_cast<_Float16>(v[3])};
      *reinterpret_cast<half4*>(part + 2 * (ch * kHeadBlock + 4 * gq)) = h;
    }
  }
  if (wave == 0 && n16 == 0) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int hh = 4 * gq + rr, hg = cx.hb * kHeadBlock + hh;
      if (direct) {
        if (hg < p.heads)
          p.lse[static_cast<int64_t>(cx.b) * p.heads + hg] =
              lq[rr] > 0.f ? (m_o[rr] + log2f(lq[rr])) * 0.69314718055994531f : kNegInf;
      } else {
        float* const ml = reinterpret_cast<float*>(part + kPartRowBytes);
        ml[hh] = m_o[rr];
        ml[kHeadBlock + hh] = lq[rr];
      }
    }
  }
}

template <int BITS>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  WgCtx cx;
  // Workgroups are dealt to the 8 XCDs of the chip in turn (block i on XCD
  // i mod 8); order the work so that each XCD's blocks take consecutive
  // items, which keeps the splits of a sequence on one XCD, sharing its L2 for
  // the query rows, block-table window and (with several head blocks) pages.
  // (Any dispatch order gives the same results; this only places the work.)
  const int n_blocks = gridDim.x, xcd = blockIdx.x & 7, per_xcd = n_blocks >> 3, extra = n_blocks & 7;
  const int item = xcd * per_xcd + min(xcd, extra) + (blockIdx.x >> 3);
  // items are ordered (sequence, split, head block): the head blocks of one
  // (sequence, split) read the same pages, and as consecutive items they run
  // on one XCD at the same time, so the XCD's L2 serves the repeats
  cx.hb = item % p.n_hb;
  cx.split = (item / p.n_hb) % p.n_splits;
  cx.b = item / (p.n_hb * p.n_splits);
  cx.grp = cx.b * p.n_hb + cx.hb;
  cx.lane = threadIdx.x & 63;
  cx.wave = uniform(threadIdx.x >> 6);
  cx.n16 = cx.lane & 15;
  cx.gq = cx.lane >> 4;
  const SeqRanges sr = seq_ranges(p, cx.b);
  // running max of heads 4 gq + r (identical in every wave), this wave's
  // output (latent group `wave`: heads 4 gq + r, columns 16 kk + n16) and
  // per-lane sums (head n16)
  float m_o[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  f32x4 o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float st[kStatW];
#pragma unroll
  for (int k = 0; k < kStatW; ++k) st[k] = 0.f;
  if (cx.split < p.n_dense) {
    dense_wg<BITS>(o, st, m_o, p, smem, sr, cx, cx.split);
    finish<BITS, false>(p, smem + kOffP, o, st, m_o, cx);
  } else {
    packed_wg<BITS>(o, st, m_o, p, smem, sr, cx, cx.split - p.n_dense, p.n_splits - p.n_dense);
    finish<BITS, true>(p, smem + kPkOffP, o, st, m_o, cx);
  }
}

// Merge of the split partials of one (sequence, head block).  A workgroup
// takes CB channels: its 2 CB columns are (channel, heads 8 (col % 2) .. + 7),
// 16 bytes of the channel-major partial rows each, and its SG split groups
// take the splits g, g + SG, ... of every column with up to 16 row loads in
// flight per thread; the split groups' sums meet in LDS at the end (summed in
// two stages by all the threads).  Grid =
// (sequence, head block) x 512 / CB.  A partial holds the split's normalized
// output O_s / l_s (fp16) and (m_s, l_s); the merge weights split s by
// 2^(m_s - M) l_s / sum over splits, M = max_s m_s, per head (formed by all
// threads: head t % 16, splits t / 16 (mod threads / 16)).
template <int CB, int SG>
struct Cmb {
  static constexpr int kThreads = 2 * CB * SG;
  static constexpr int kQ = kThreads / kHeadBlock;  // split groups of the weights
  static constexpr int kBlocks = kLatentDim / CB;   // workgroups per (sequence, head block)
  static constexpr int kMaxS = SG == 1 ? 32 : kMaxSplits;  // splits it is launched for
  static constexpr int kOut = 2 * CB * 8;                  // outputs of a workgroup (channel, head)
  static constexpr int kParts = kThreads / kOut;          // threads per output in the final sum
  static_assert(SG == 1 || (kThreads % kOut == 0 && SG % kParts == 0), "final sum layout");
};

// Dynamic LDS of combine_kernel<CB, SG> for n splits: s_ml [split][m 16, l 16],
// s_w [split][head], s_red [2][kQ][head] + [head], s_acc [thread][8].
template <int CB, int SG>
constexpr size_t combine_lds_bytes(int n_splits) {
  return static_cast<size_t>(n_splits) * 3 * kHeadBlock * 4 + (2 * Cmb<CB, SG>::kQ + 1) * kHeadBlock * 4 +
         (SG > 1 ? Cmb<CB, SG>::kThreads * 8 * 4 : 0);
}

template <int CB, int SG>
__global__ void __launch_bounds__((Cmb<CB, SG>::kThreads)) combine_kernel(const uint8_t* __restrict__ parts,
                                                                       float* __restrict__ out, float* __restrict__ lse,
                                                                       int heads, int n_hb, int n_splits) {
  using C = Cmb<CB, SG>;
  extern __shared__ __attribute__((aligned(16))) float cmb_lds[];
  float* const s_ml = cmb_lds;
  float* const s_w = s_ml + n_splits * 2 * kHeadBlock;
  float* const s_red = s_w + n_splits * kHeadBlock;
  float* const s_acc = s_red + (2 * C::kQ + 1) * kHeadBlock;
  const int grp = blockIdx.x / C::kBlocks, cb = blockIdx.x % C::kBlocks;
  const int b = grp / n_hb, hb = grp % n_hb;
  const uint8_t* const base = parts + static_cast<int64_t>(grp) * n_splits * kPartBytes;
  const int t = threadIdx.x, col = t % (2 * CB), sg = t / (2 * CB);
  const int c = CB * cb + (col >> 1), h0 = 8 * (col & 1);
  const uint8_t* const row = base + 2 * (c * kHeadBlock + h0);
  // every split's (max, sum) block (8 x 16 bytes) goes out first, all at once,
  // then this split group's first rows; the weights are formed while the rows
  // fly (the (max, sum) addresses are clamped to the last split rather than
  // branched around, so that every load is in flight before the wait)
  const int n_ml = (n_splits * 8 + C::kThreads - 1) / C::kThreads;  // pieces per thread
  constexpr int kMlPieces = C::kMaxS * 8 / C::kThreads;
  u32x4 ml[kMlPieces];
#pragma unroll
  for (int k = 0; k < kMlPieces; ++k) {
    const int i = min(t + C::kThreads * k, n_splits * 8 - 1);  // piece i: split i / 8, floats 4 (i % 8) .. + 3
    if (k < n_ml) ml[k] = ldg<u32x4>(base + static_cast<int64_t>(i >> 3) * kPartBytes + kPartRowBytes + 16 * (i & 7));
  }
  constexpr int kEarly = 16;
  u32x4 v[kEarly];
#pragma unroll
  for (int j = 0; j < kEarly; ++j)  // clamped, not branched: all 16 go out back to back
    v[j] = ldg<u32x4>(row + static_cast<int64_t>(min(sg + SG * j, n_splits - 1)) * kPartBytes);
#pragma unroll
  for (int k = 0; k < kMlPieces; ++k) {
    if (k < n_ml) *reinterpret_cast<u32x4*>(s_ml + 4 * min(t + C::kThreads * k, n_splits * 8 - 1)) = ml[k];
  }
  __syncthreads();
  const int wh = t & 15, wq = t >> 4;
  float mp = kNegInf;
  for (int sp = wq; sp < n_splits; sp += C::kQ) mp = fmaxf(mp, s_ml[sp * 32 + wh]);
  s_red[wq * kHeadBlock + wh] = mp;
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int q = 0; q < C::kQ; ++q) M = fmaxf(M, s_red[q * kHeadBlock + wh]);
  float lp = 0.f;
  for (int sp = wq; sp < n_splits; sp += C::kQ) {
    const float m = s_ml[sp * 32 + wh];
    const float w = m == kNegInf ? 0.f : fast_exp2(m - M) * s_ml[sp * 32 + kHeadBlock + wh];
    s_w[sp * kHeadBlock + wh] = w;
    lp += w;
  }
  s_red[(C::kQ + wq) * kHeadBlock + wh] = lp;
  __syncthreads();
  if (t < kHeadBlock) {
    float L = 0.f;
#pragma unroll
    for (int q = 0; q < C::kQ; ++q) L += s_red[(C::kQ + q) * kHeadBlock + t];
    s_red[2 * C::kQ * kHeadBlock + t] = L > 0.f ? 1.f / L : 0.f;
    const int hg = hb * kHeadBlock + t;
    if (cb == 0 && hg < heads)
      lse[static_cast<int64_t>(b) * heads + hg] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
  }
  __syncthreads();
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](int sp, const u32x4& x) {
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(s_w + sp * kHeadBlock + h0);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(s_w + sp * kHeadBlock + h0 + 4);
    const half8 hv = __builtin_bit_cast(half8, x);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(w0[e], static_cast<float>(hv[e]), acc[e]);
      acc[4 + e] = fmaf(w1[e], static_cast<float>(hv[4 + e]), acc[4 + e]);
    }
  };
#pragma unroll
  for (int j = 0; j < kEarly; ++j) {
    const int sp = sg + SG * j;
    if (sp < n_splits) add(sp, v[j]);
  }
#pragma unroll 16
  for (int sp = sg + SG * kEarly; sp < n_splits; sp += SG) add(sp, ldg<u32x4>(row + static_cast<int64_t>(sp) * kPartBytes));
  if constexpr (SG > 1) {
    // the split groups' sums meet in LDS, then in two stages over all the
    // threads: output o (column o / 8, head h0 + o % 8 of it) is summed over
    // every C::kParts-th split group by C::kParts threads, whose parts meet
    // once more
    float* const mine = s_acc + t * 8;
    *reinterpret_cast<f32x4*>(mine) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(mine + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    const int o = t % C::kOut, part = t / C::kOut;
    float sum = 0.f;
#pragma unroll
    for (int g = part; g < SG; g += C::kParts) sum += s_acc[(g * 2 * CB + (o >> 3)) * 8 + (o & 7)];
    __syncthreads();
    s_acc[part * C::kOut + o] = sum;
    __syncthreads();
    if (t >= C::kOut) return;
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < C::kParts; ++q) tot += s_acc[q * C::kOut + t];
    const int oc = CB * cb + (t >> 4), oh = 8 * ((t >> 3) & 1) + (t & 7);
    const int hg = hb * kHeadBlock + oh;
    if (hg < heads)
      out[(static_cast<int64_t>(b) * heads + hg) * kLatentDim + oc] = tot * s_red[2 * C::kQ * kHeadBlock + oh];
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int hg = hb * kHeadBlock + h0 + e;
    if (hg < heads)
      out[(static_cast<int64_t>(b) * heads + hg) * kLatentDim + c] = acc[e] * s_red[2 * C::kQ * kHeadBlock + h0 + e];
  }
}

// Launches the merge kernel in one shape (CB channels per workgroup, SG
// split groups); launch_merge picks the shape.
template <int CB, int SG>
int launch_combine(const DecodeParams& p, int64_t groups, int heads, int n_hb, int n_splits, hipStream_t stream) {
  static const bool attr_ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&combine_kernel<CB, SG>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(combine_lds_bytes<CB, SG>(Cmb<CB, SG>::kMaxS))) == hipSuccess;
  if (!attr_ok) return MLA_LOWBIT_ERR_HIP;
  using C = Cmb<CB, SG>;
  const dim3 grid(static_cast<uint32_t>(groups * C::kBlocks)), block(C::kThreads);
  const size_t lds = combine_lds_bytes<CB, SG>(n_splits);
  hipLaunchKernelGGL((combine_kernel<CB, SG>), grid, block, lds, stream, p.parts, p.out, p.lse, heads, n_hb,
                     n_splits);
  return hipGetLastError() == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ERR_HIP;
}

// The merge shape for n_splits partials of `groups` (sequence, head block)
// groups: one wave per 32 channels when the splits are few (up to 32); else
// 8-channel blocks of 16 split groups, or, when so few groups would leave
// most of the chip idle (under 256 workgroups), 4-channel blocks of 32 split
// groups (twice the workgroups, every row of a thread in flight at once).
int launch_merge(const DecodeParams& p, int64_t groups, int heads, int n_hb, int n_splits, hipStream_t stream) {
  if (n_splits <= 32) return launch_combine<32, 1>(p, groups, heads, n_hb, n_splits, stream);
  if (groups * (kLatentDim / 8) < 256) return launch_combine<4, 32>(p, groups, heads, n_hb, n_splits, stream);
  return launch_combine<8, 16>(p, groups, heads, n_hb, n_splits, stream);
}

#include "decode_bf16.h"

// Validation and launches of the BF16-cache entry points.
int bf16_decode_impl(const void* q_lat, const void* q_rope, int32_t batch, int32_t heads, float softmax_scale,
                     const void* pool, int32_t num_pool_pages, int32_t page_size, const int32_t* block_table,
                     int32_t max_pages, const int32_t* seqlens, int32_t max_seqlen, float* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch < 0 || heads < 1 || heads > kMaxHeads || max_seqlen < 0 || max_pages < 0 || num_pool_pages < 0 ||
      page_size < 16 || page_size > 1024 || (page_size & (page_size - 1)) || !std::isfinite(softmax_scale))
    return MLA_LOWBIT_ERR_ARG;
  if (batch == 0) return MLA_LOWBIT_OK;
  if (static_cast<int64_t>(max_seqlen) > static_cast<int64_t>(max_pages) * page_size) return MLA_LOWBIT_ERR_ARG;
  if (!q_lat || !q_rope || !seqlens || !out || !lse) return MLA_LOWBIT_ERR_ARG;
  if (max_seqlen > 0 && (!pool || !block_table || num_pool_pages == 0)) return MLA_LOWBIT_ERR_ARG;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(out) || (pool && !aligned16(pool)) ||
      (workspace && !aligned16(workspace)))
    return MLA_LOWBIT_ERR_ARG;
  const bf16c::Plan plan = bf16c::plan(page_size, batch, heads, max_seqlen);
  if (!plan.ok) return MLA_LOWBIT_ERR_UNSUPPORTED;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return MLA_LOWBIT_ERR_WORKSPACE;
  const int64_t groups = static_cast<int64_t>(batch) * plan.n_hb;
  const int64_t blocks = groups * plan.n_splits;
  if (blocks > 0x7FFFFFFF || groups * 64 > 0x7FFFFFFF) return MLA_LOWBIT_ERR_UNSUPPORTED;
  static const bool attr_ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&bf16c::decode_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bf16c::kLdsBytes) == hipSuccess;
  if (!attr_ok) return MLA_LOWBIT_ERR_HIP;
  bf16c::Params p{};
  p.q_lat = static_cast<const uint16_t*>(q_lat);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.pool = static_cast<const uint8_t*>(pool);
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.parts = static_cast<uint8_t*>(workspace);
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.heads = heads;
  p.max_pages = max_pages;
  p.num_pool_pages = num_pool_pages;
  p.n_hb = plan.n_hb;
  p.n_splits = plan.n_splits;
  p.per = plan.per;
  p.log2P = 0;
  while ((1 << p.log2P) < page_size) ++p.log2P;
  p.page_bytes = static_cast<int64_t>(page_size) * bf16c::kRowBytes;
  p.c_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(bf16c::decode_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(bf16c::kThreads),
                     bf16c::kLdsBytes, stream, p);
  if (hipGetLastError() != hipSuccess) return MLA_LOWBIT_ERR_HIP;
  if (plan.n_splits > 1) {
    DecodeParams cp{};
    cp.parts = p.parts;
    cp.out = out;
    cp.lse = lse;
    return launch_merge(cp, groups, heads, plan.n_hb, plan.n_splits, stream);
  }
  return MLA_LOWBIT_OK;
}

// The no-allocation entry point's split partials: one fixed array per GPU
// (each device holds its own copy at its own address for the life of the
// process).  Host code never uses this name as an address: it takes the
// device's address from hipGetSymbolAddress once per device (scratch_of).
static __device__ __align__(256) uint8_t scratch[MLA_LOWBIT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call made on that device; nullptr if the lookup fails.
void* scratch_of_current_device() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

// Sets the decode kernels' dynamic-LDS limits once per process (thread-safe
// static initialization).
int set_decode_attributes() {
  static const int rc = [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<4>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) == hipSuccess &&
                   hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<2>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) == hipSuccess
               ? MLA_LOWBIT_OK
               : MLA_LOWBIT_ERR_HIP;
  }();
  return rc;
}

// Validation, work split and launches shared by both decode entry points.
// With noalloc the partials go to the device's fixed scratch array instead of
// the caller's workspace.
int decode_impl(const mla_lowbit_layout* layout, const void* q_lat, const void* q_rope, int32_t batch,
                int32_t heads, float softmax_scale, const void* page_pool, int32_t num_pool_pages,
                const int32_t* block_table, int32_t max_pages, const int32_t* seqlens, int32_t max_seqlen,
                const void* sink_buf, const void* ring_buf, const void* rope_tail, float* out, float* lse,
                void* workspace, size_t workspace_bytes, bool noalloc, hipStream_t stream) {
  Geometry g;
  int rc = make_geometry(layout, &g);
  if (rc) return rc;
  if (batch < 0 || heads < 1 || heads > kMaxHeads || max_seqlen < 0 || max_pages < 0 ||
      num_pool_pages < 0 || !std::isfinite(softmax_scale))
    return MLA_LOWBIT_ERR_ARG;
  if (batch == 0) return MLA_LOWBIT_OK;
  if (static_cast<int64_t>(max_seqlen) > static_cast<int64_t>(max_pages) * g.page_size)
    return MLA_LOWBIT_ERR_ARG;
  if (!q_lat || !q_rope || !seqlens || !out || !lse || !rope_tail) return MLA_LOWBIT_ERR_ARG;
  if (max_seqlen > 0 && (!page_pool || !block_table || num_pool_pages == 0)) return MLA_LOWBIT_ERR_ARG;
  if (g.sink > 0 && !sink_buf) return MLA_LOWBIT_ERR_ARG;
  if (g.local > 0 && !ring_buf) return MLA_LOWBIT_ERR_ARG;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(out) || !aligned16(rope_tail) ||
      (page_pool && !aligned16(page_pool)) || (sink_buf && !aligned16(sink_buf)) ||
      (ring_buf && !aligned16(ring_buf)) || (workspace && !aligned16(workspace)))
    return MLA_LOWBIT_ERR_ARG;
  const DecodePlan plan = plan_decode(g, batch, heads, max_seqlen);
  if (!plan.ok) return MLA_LOWBIT_ERR_UNSUPPORTED;
  if (noalloc) {
    if (plan.workspace_bytes > MLA_LOWBIT_NOALLOC_SCRATCH_BYTES) return MLA_LOWBIT_ERR_SCRATCH;
    workspace = nullptr;
    workspace_bytes = 0;
    if (plan.workspace_bytes > 0) {
      workspace = scratch_of_current_device();
      if (!workspace) return MLA_LOWBIT_ERR_HIP;
      workspace_bytes = MLA_LOWBIT_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return MLA_LOWBIT_ERR_WORKSPACE;
  DecodeParams p{};
  p.q_lat = static_cast<const uint16_t*>(q_lat);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.pool = static_cast<const uint8_t*>(page_pool);
  {
    const bool pool_ok = page_pool != nullptr && num_pool_pages > 0;
    p.fallback = pool_ok ? p.pool : static_cast<const uint8_t*>(q_lat);
    p.off_mask = pool_ok ? ~0u : 0u;
  }
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.sink = static_cast<const uint16_t*>(sink_buf);
  p.ring = static_cast<const uint16_t*>(ring_buf);
  p.tail = static_cast<const uint16_t*>(rope_tail);
  p.parts = static_cast<uint8_t*>(workspace);
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.heads = heads;
  p.max_pages = max_pages;
  p.num_pool_pages = num_pool_pages;
  p.max_seqlen = max_seqlen;
  p.n_hb = plan.n_hb;
  p.n_dense = plan.n_dense;
  p.n_splits = plan.n_splits;
  p.P = g.page_size;
  p.log2P = 0;
  while ((1 << p.log2P) < g.page_size) ++p.log2P;
  p.sink_n = g.sink;
  p.local = g.local;
  p.latent_meta_off = g.latent_meta_off;
  p.rope_codes_off = g.rope_codes_off;
  p.rope_meta_off = g.rope_meta_off;
  p.page_bytes = g.page_bytes;
  p.c_log2 = softmax_scale * 1.44269504088896341f;
  {  // packed range of a sequence of max_seqlen tokens (the longest one)
    const int64_t ml = max_seqlen;
    const int64_t lo = std::min<int64_t>(g.sink, ml);
    const int64_t hi = std::max<int64_t>(lo, std::min<int64_t>(ml - g.local, (ml / g.page_size) * g.page_size));
    p.t_lo = static_cast<int32_t>(lo / kTile);
    p.t_count = hi > lo ? static_cast<int32_t>((hi + kTile - 1) / kTile - p.t_lo) : 0;
  }
  const int64_t groups = static_cast<int64_t>(batch) * plan.n_hb;
  const int64_t blocks = groups * plan.n_splits;
  if (blocks > 0x7FFFFFFF || groups * 64 > 0x7FFFFFFF) return MLA_LOWBIT_ERR_UNSUPPORTED;
  if ((rc = set_decode_attributes()) != MLA_LOWBIT_OK) return rc;
  if (g.latent_bits == 4)
    hipLaunchKernelGGL(decode_kernel<4>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), kLdsBytes,
                       stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<2>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), kLdsBytes,
                       stream, p);
  if (hipGetLastError() != hipSuccess) return MLA_LOWBIT_ERR_HIP;
  if (plan.n_splits > 1) {
    rc = launch_merge(p, groups, heads, plan.n_hb, plan.n_splits, stream);
    if (rc) return rc;
  }
  return MLA_LOWBIT_OK;
}

}  // namespace
}  // namespace mla

extern "C" int mla_lowbit_decode(const mla_lowbit_layout* layout, const void* q_lat, const void* q_rope,
                                 int32_t batch, int32_t heads, float softmax_scale, const void* page_pool,
                                 int32_t num_pool_pages, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seqlens, int32_t max_seqlen, const void* sink_buf,
                                 const void* ring_buf, const void* rope_tail, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mla::decode_impl(layout, q_lat, q_rope, batch, heads, softmax_scale, page_pool, num_pool_pages,
                          block_table, max_pages, seqlens, max_seqlen, sink_buf, ring_buf, rope_tail, out, lse,
                          workspace, workspace_bytes, false, stream);
}

extern "C" int mla_lowbit_decode_noalloc(const mla_lowbit_layout* layout, const void* q_lat, const void* q_rope,
                                         int32_t batch, int32_t heads, float softmax_scale, const void* page_pool,
                                         int32_t num_pool_pages, const int32_t* block_table, int32_t max_pages,
                                         const int32_t* seqlens, int32_t max_seqlen, const void* sink_buf,
                                         const void* ring_buf, const void* rope_tail, float* out, float* lse,
                                         hipStream_t stream) {
  return mla::decode_impl(layout, q_lat, q_rope, batch, heads, softmax_scale, page_pool, num_pool_pages,
                          block_table, max_pages, seqlens, max_seqlen, sink_buf, ring_buf, rope_tail, out, lse,
                          nullptr, 0, true, stream);
}

extern "C" int mla_bf16_decode_workspace(int32_t page_size, int32_t batch, int32_t heads, int32_t max_seqlen,
                                         size_t* bytes) {
  if (!bytes || batch < 0 || heads < 1 || heads > mla::kMaxHeads || max_seqlen < 0 || page_size < 16 ||
      page_size > 1024 || (page_size & (page_size - 1)))
    return MLA_LOWBIT_ERR_ARG;
  const mla::bf16c::Plan plan = mla::bf16c::plan(page_size, batch, heads, max_seqlen);
  if (!plan.ok) return MLA_LOWBIT_ERR_UNSUPPORTED;
  *bytes = batch == 0 ? 0 : plan.workspace_bytes;
  return MLA_LOWBIT_OK;
}

extern "C" int mla_bf16_decode(const void* q_lat, const void* q_rope, int32_t batch, int32_t heads,
                               float softmax_scale, const void* pool, int32_t num_pool_pages, int32_t page_size,
                               const int32_t* block_table, int32_t max_pages, const int32_t* seqlens,
                               int32_t max_seqlen, float* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return mla::bf16_decode_impl(q_lat, q_rope, batch, heads, softmax_scale, pool, num_pool_pages, page_size,
                               block_table, max_pages, seqlens, max_seqlen, out, lse, workspace, workspace_bytes,
                               stream);
}

extern "C" int mla_bf16_append(const void* c_kv, const void* k_r, const int32_t* cu_new,
                               const int32_t* seqlens_before, int32_t batch, int32_t total_new,
                               int32_t max_new_per_seq, int32_t page_size, const int32_t* block_table,
                               int32_t max_pages, int32_t num_pool_pages, void* pool, hipStream_t stream) {
  if (batch < 0 || total_new < 0 || max_new_per_seq < 0 || max_pages < 0 || num_pool_pages < 0 ||
      page_size < 16 || page_size > 1024 || (page_size & (page_size - 1)))
    return MLA_LOWBIT_ERR_ARG;
  if (batch == 0 || total_new == 0 || max_new_per_seq == 0) return MLA_LOWBIT_OK;
  if (!c_kv || !k_r || !cu_new || !seqlens_before || !block_table || !pool || max_pages == 0 ||
      num_pool_pages == 0)
    return MLA_LOWBIT_ERR_ARG;
  if (!mla::aligned16(c_kv) || !mla::aligned16(k_r) || !mla::aligned16(pool)) return MLA_LOWBIT_ERR_ARG;
  int log2P = 0;
  while ((1 << log2P) < page_size) ++log2P;
  const dim3 grid(static_cast<uint32_t>((max_new_per_seq + 3) / 4), static_cast<uint32_t>(batch));
  if (grid.y > 65535u) return MLA_LOWBIT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mla::bf16c::append_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(c_kv),
                     static_cast<const uint16_t*>(k_r), cu_new, seqlens_before, log2P, block_table, max_pages,
                     num_pool_pages, static_cast<uint16_t*>(pool));
  return hipGetLastError() == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ERR_HIP;
}
