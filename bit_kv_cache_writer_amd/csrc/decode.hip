// Decode attention over the dual-path low-bit MLA cache, for gfx950.
//
// What is computed (QuantMLA Figure 8 caption; RAQ-MLA abstract and
// Figure 4 caption): per sequence and head, one softmax over all valid
// tokens of score = q_lat . c_KV + q_rope . k_R, output sum_j p_j c_KV_j in
// latent space; protected (sink / recent) tokens from BF16, the others from
// codes dequantized inside the loop -- the same reconstructed content tile
// feeds both the score (matching) and the output (aggregation).
//
// How.  One workgroup of 4 waves (one per SIMD) per (sequence, 16-head block,
// split of the sequence); two workgroups share a CU, so one fills the other's
// barrier and memory waits.  Each wave owns a contiguous run of 16-token
// tiles (consecutive tiles of a wave share a page); the waves advance in
// lockstep rounds, one tile each:
//  1. Scores.  The wave's codes arrive straight in the lanes that feed
//     v_mfma_f32_16x16x32_f16 (M = 16 tokens, N = 16 heads, K = 32 channels;
//     lane (t, g) holds 8 channels of token t); the next tile's codes are
//     requested as soon as these are unpacked.  Codes are unpacked in
//     registers to fp16 x = 1 + code/kappa by OR-ing the code into the top of
//     an fp16 mantissa (kappa = 16 for 4-bit codes, 4 for 2-bit codes); the x
//     tile also goes to LDS.  Group scale s and minimum m are folded after the
//     MFMA:
//       q.c = sum_g kappa s_g (q_g . x_g) + sum_g (m_g - kappa s_g) Q_g,
//     Q_g = sum of the query over group g; the second sum is one more MFMA on
//     the raw fp16 (scale, min) metadata.  The positional key's per-(channel,
//     page) scale/min is folded into a per-page query q' = q s (fp16 hi + lo)
//     and bias sum_c q_c (m_c - 16 s_c), rebuilt only when the page changes.
//  2. Softmax.  The four tile maxima meet in LDS; every wave raises the same
//     running max and turns its scores into fp16 weights P'_g = p s_g per
//     latent group.  Sums of p, of P'_g and of p m_g stay per lane until the
//     end.
//  3. Output.  Wave w owns latent group w (128 output channels) for the four
//     tiles of the round, taken in pairs (K = 32 tokens): A = P'_w, B = the x
//     tiles read back with ds_read_b64_tr_b16 (one channel of 4 tokens per
//     lane).  The output accumulates sum_j fp16(p_j s_j) x_j; the offsets
//     -kappa sum_j fp16(p_j s_j) and sum_j p_j m_j are applied at the end --
//     the same rounded fp16 products enter both, so they cancel.
// Tile, page and address arithmetic is wave-uniform (scalar registers); the
// page ids a workgroup needs are staged in LDS once.  BF16 tokens (sink,
// recent window and, when the window is shorter than a page, tokens of the
// unfinished page) are tiles of the same rounds: their rows are converted to
// fp16 on their way into the x tile.  With several splits each workgroup
// writes a partial (unnormalized output, max, sum) and a second kernel merges
// them with log-sum-exp weights (the kernel boundary makes the partials of
// every XCD visible without cache flushes inside the kernel).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "decode_plan.h"
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

constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = 64 * kWaves;
// x-tile row: 512 fp16 + 16 B pad (260 dwords: rows land 4 banks apart, so
// both the row-wise writes and the transposed reads are conflict-free)
constexpr int kXRow = 1040;
constexpr int kXTile = kTile * kXRow;
// LDS map (bytes)
constexpr int kOffX = 0;                              // [wave] x tiles
constexpr int kPTile = 4 * 64 * 8;                    // [group][lane] fp16 x 4
constexpr int kOffP = kOffX + kWaves * kXTile;        // [wave] P' tiles
constexpr int kOffMeta = kOffP + kWaves * kPTile;     // [wave][group][16 tokens] dwords
constexpr int kOffRMeta = kOffMeta + kWaves * 256;    // [wave] k_R metadata of a page
constexpr int kOffMax = kOffRMeta + kWaves * 256;     // [head][wave] tile maxima
constexpr int kOffQr = kOffMax + kHeadBlock * kWaves * 4;  // [head] q_rope, bf16 x 64
constexpr int kPageWin = 256;                              // page ids staged per workgroup
constexpr int kOffPid = kOffQr + kHeadBlock * kRopeDim * 2;
constexpr int kLdsBytes = kOffPid + kPageWin * 4;
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per gfx950 CU");
constexpr int kStatW = 9;  // per head: sum p, sum P'_g (4), sum p m_g (4)
static_assert(kWaves * kHeadBlock * kStatW * 4 <= kWaves * kPTile, "final sums reuse the P' area");
static_assert(kTile * 128 <= kPTile, "a BF16 tile's k_R rows fit the P' area");
constexpr float kPrescale = 1.0f / 256.0f;  // keeps q' and Q_g inside fp16 range
constexpr float kNegInf = -INFINITY;

struct DecodeParams {
  const uint16_t* q_lat;
  const uint16_t* q_rope;
  const uint8_t* pool;
  const int32_t* block_table;
  const int32_t* seqlens;
  const uint16_t* sink;
  const uint16_t* ring;
  const uint16_t* tail;
  float* parts;
  float* out;
  float* lse;
  int32_t batch, heads, max_pages, num_pool_pages, max_seqlen;
  int32_t n_hb, n_splits;
  int32_t P, log2P, sink_n, local;
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

// Constants kept in VGPRs so that shift-and-merge compiles to one v_and_or_b32
// per pair (a VOP3 instruction cannot encode two literal constants).
struct UnpackK {
  uint32_t m4, m2, e;
};
__device__ inline UnpackK unpack_k() {
  UnpackK k;
  asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(k.e));
  k.m4 = 0x03C003C0u;
  k.m2 = 0x03000300u;
  return k;
}

// 8 nibbles -> fp16 1 + code/16, slots [n0 n4 n1 n5 n2 n6 n3 n7].
__device__ inline half8 unpack4(uint32_t w, const UnpackK& k) {
  u32x4 v;
  v[0] = ((w << 6) & k.m4) | k.e;
  v[1] = ((w << 2) & k.m4) | k.e;
  v[2] = ((w >> 2) & k.m4) | k.e;
  v[3] = ((w >> 6) & k.m4) | k.e;
  return __builtin_bit_cast(half8, v);
}

// 8 of the 16 crumbs of w -> fp16 1 + code/4; hi = 0: crumbs [0 8 1 9 2 10 3 11],
// hi = 1: crumbs [4 12 5 13 6 14 7 15].
__device__ inline half8 unpack2(uint32_t w, int hi, const UnpackK& k) {
  u32x4 v;
  if (hi == 0) {
    v[0] = ((w << 8) & k.m2) | k.e;
    v[1] = ((w << 6) & k.m2) | k.e;
    v[2] = ((w << 4) & k.m2) | k.e;
    v[3] = ((w << 2) & k.m2) | k.e;
  } else {
    v[0] = (w & k.m2) | k.e;
    v[1] = ((w >> 2) & k.m2) | k.e;
    v[2] = ((w >> 4) & k.m2) | k.e;
    v[3] = ((w >> 6) & k.m2) | k.e;
  }
  return __builtin_bit_cast(half8, v);
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
  half8 meta;       // (scale, min) slots of the metadata MFMA, prescaled
};

// Query rows of the 16 heads of a head block, staged in LDS as [head][1024 B]
// (q_lat) plus [head][128 B] (q_rope): wave w fetches latent group w of every
// head (lane: head lane / 4, 32 channels), wave 0 also the q_rope rows.
// Heads past the last one read a copy of the last head.
__device__ inline void stage_query(uint8_t* ql_lds, uint8_t* qr_lds, const DecodeParams& p, int b, int hb, int wave,
                                   int lane) {
  const int h = hb * kHeadBlock + (lane >> 2), part = lane & 3;
  const int hc = h < p.heads ? h : p.heads - 1;
  const uint16_t* ql = p.q_lat + (static_cast<int64_t>(b) * p.heads + hc) * kLatentDim + 128 * wave + 32 * part;
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = ldg<u32x4>(ql + 8 * u);
  u32x4 r[2];
  if (wave == 0) {
    const uint16_t* qr = p.q_rope + (static_cast<int64_t>(b) * p.heads + hc) * kRopeDim + 16 * part;
    r[0] = ldg<u32x4>(qr);
    r[1] = ldg<u32x4>(qr + 8);
  }
  uint8_t* row = ql_lds + (lane >> 2) * 1024 + 2 * (128 * wave + 32 * part);
#pragma unroll
  for (int u = 0; u < 4; ++u) lds_st<u32x4>(row + 16 * u, v[u]);
  if (wave == 0) {
    lds_st<u32x4>(qr_lds + (lane >> 2) * 128 + 32 * part, r[0]);
    lds_st<u32x4>(qr_lds + (lane >> 2) * 128 + 32 * part + 16, r[1]);
  }
}

// MFMA operands of the query from the staged rows: lane (h, gq) takes channels
// 128 i + 32 gq .. + 31 of head h, in the unpack's slot order; Q_g = sum of
// the query over group g enters the metadata operand.
template <int BITS>
__device__ inline void load_query(QueryOps<BITS>& q, const uint8_t* ql_lds, int n16, int gq) {
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  float qg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* row = ql_lds + n16 * 1024 + 2 * (128 * i + 32 * gq);
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 w = lds_ld<u32x4>(row + 16 * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * u + 2 * e] = bf16f(w[e] & 0xFFFFu);
        v[8 * u + 2 * e + 1] = bf16f(w[e] >> 16);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) s += v[c];
    qg[i] = row_allsum(s);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) q.lat[i][d][sl] = static_cast<_Float16>(v[chan_off<BITS>(d, sl)]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = -kappa * qg[i] * kPrescale, c = qg[i] * kPrescale;
    const _Float16 ah = static_cast<_Float16>(a), ch = static_cast<_Float16>(c);
    const _Float16 al = static_cast<_Float16>(a - static_cast<float>(ah));
    const _Float16 cl = static_cast<_Float16>(c - static_cast<float>(ch));
    const _Float16 z = static_cast<_Float16>(0.f);
    q.meta[2 * i] = gq == 0 ? ah : (gq == 1 ? al : z);
    q.meta[2 * i + 1] = gq == 0 ? ch : (gq == 1 ? cl : z);
  }
}

// Per-page positional-key operands for channels 16*gq + 8e + slot order:
// q' = q s * 16 / 256 as fp16 hi + lo, and bias sum_c q_c (m_c - 16 s_c).
struct RopeOps {
  half8 hi[2], lo[2];
  float bias;
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
  float bias = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) bias += qv[c] * (mn[c] - 16.f * sc[c]);
  r.bias = row_allsum(bias);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int c = 8 * e + chan_off<4>(0, sl);
      const float v = qv[c] * sc[c] * (16.f * kPrescale);
      const _Float16 vh = static_cast<_Float16>(v);
      r.hi[e][sl] = vh;
      r.lo[e][sl] = static_cast<_Float16>(v - static_cast<float>(vh));
    }
  }
}

// ---------------------------------------------------------------------------
// packed tiles

template <int BITS>
struct Stage {
  uint32_t lat[BITS == 4 ? 16 : 8];  // dwords of the 4 groups
  u32x2 rope;
  u32x4 ma;        // latent metadata of token n16
  uint32_t rmeta;  // 4 bytes of the page's k_R metadata (first tile of a page)
};

// Per-lane byte offsets inside a tile (constant over the kernel).
struct LaneOffs {
  uint32_t lat, rope, meta;
};

// Loads the 16-token tile whose first slot is slot0 of `page` (a wave-uniform
// pointer); every address is page base (scalar) + 32-bit lane offset.
template <int BITS>
__device__ inline void load_stage(Stage<BITS>& sg, const uint8_t* page, int slot0, bool new_page,
                                  const LaneOffs& lo, int lane, const DecodeParams& p) {
  constexpr int kLatRow = kLatentDim * BITS / 8;
  const uint8_t* lat = page + slot0 * kLatRow;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BITS == 4) {
      const u32x4 v = ldg<u32x4>(lat + lo.lat + 64 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) sg.lat[4 * i + e] = v[e];
    } else {
      const u32x2 v = ldg<u32x2>(lat + lo.lat + 32 * i);
      sg.lat[2 * i + 0] = v[0];
      sg.lat[2 * i + 1] = v[1];
    }
  }
  sg.rope = ldg<u32x2>(page + p.rope_codes_off + slot0 * kRopeRowBytes + lo.rope);
  sg.ma = ldg<u32x4>(page + p.latent_meta_off + slot0 * 16 + lo.meta);
  if (new_page) sg.rmeta = ldg<uint32_t>(page + p.rope_meta_off + 4 * lane);
}

template <int BITS>
__device__ inline half8 chunk_of(const Stage<BITS>& sg, int i, int d, const UnpackK& k) {
  if constexpr (BITS == 4) return unpack4(sg.lat[4 * i + d], k);
  else return unpack2(sg.lat[2 * i + (d >> 1)], d & 1, k);
}

// Score MFMAs of one packed tile: acc[g] = q_g . x_g per latent group,
// acc[4] = rope and metadata terms / 256.  The x tile goes to LDS.  After
// this the stage registers are free for the next tile.
template <int BITS>
__device__ void packed_mfma(f32x4 (&acc)[5], const QueryOps<BITS>& q, RopeOps& ro, const Stage<BITS>& sg,
                            bool new_page, uint8_t* xt, uint8_t* meta_lds, uint8_t* rmeta_lds, const uint8_t* qr_row,
                            int lane, int n16, int gq) {
  const UnpackK uk = unpack_k();
  if (gq == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) lds_st<uint32_t>(meta_lds + (g * kTile + n16) * 4, sg.ma[g]);
  }
  if (new_page) {
    lds_st<uint32_t>(rmeta_lds + 4 * lane, sg.rmeta);
    lds_wait();
    rope_ops(ro, qr_row, rmeta_lds, gq);
  }
#pragma unroll
  for (int g = 0; g < 5; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint8_t* lrow = xt + n16 * kXRow + 64 * gq;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half8 x = chunk_of<BITS>(sg, i, d, uk);
      acc[i] = mfma(x, q.lat[i][d], acc[i]);
      lds_st<half8>(lrow + 256 * i + 16 * d, x);
    }
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const half8 xr = unpack4(sg.rope[e], uk);
    acc[4] = mfma(xr, ro.hi[e], acc[4]);
    acc[4] = mfma(xr, ro.lo[e], acc[4]);
  }
  acc[4] = mfma(__builtin_bit_cast(half8, sg.ma), q.meta, acc[4]);
}

// Scores (log2 domain) of the tile tokens j0 .. j0+15, valid in [vlo, vhi):
// lane (h, gq) gets tokens 4 gq + r of head h.
template <int BITS>
__device__ inline void packed_fold(float (&sc)[4], const f32x4 (&acc)[5], float bias, int j0, int vlo, int vhi,
                                   const uint8_t* meta_lds, int gq, float c_log2) {
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  lds_wait();
  u32x4 mg[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) mg[g] = lds_ld<u32x4>(meta_lds + (g * kTile + 4 * gq) * 4);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = fmaf(lo_f16(mg[g][r]), acc[g][r], v[r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = j0 + 4 * gq + r;
    const float z = fmaf(v[r], kappa, fmaf(acc[4][r], 256.f, bias));
    sc[r] = (t >= vlo && t < vhi) ? z * c_log2 : kNegInf;
  }
}

// Weights of a packed tile: P'_g = fp16(fp16(p) s_g) per latent group into
// LDS [group][lane]; adds this lane's sums of p, of the fp16 P'_g and of
// p m_g to st.
__device__ inline void packed_weights(const float (&pr)[4], const uint8_t* meta_lds, uint8_t* ptile,
                                      float (&st)[kStatW], int lane, int gq) {
  const half2 ph[2] = {half2{static_cast<_Float16>(pr[0]), static_cast<_Float16>(pr[1])},
                       half2{static_cast<_Float16>(pr[2]), static_cast<_Float16>(pr[3])}};
  st[0] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const half2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  u32x4 mg[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) mg[g] = lds_ld<u32x4>(meta_lds + (g * kTile + 4 * gq) * 4);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    half4 pa;
    float cs = st[1 + g], ms = st[5 + g];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t w0 = mg[g][2 * k], w1 = mg[g][2 * k + 1];
      const half2 s2 = {__builtin_bit_cast(half2, w0)[0], __builtin_bit_cast(half2, w1)[0]};
      const half2 m2 = {__builtin_bit_cast(half2, w0)[1], __builtin_bit_cast(half2, w1)[1]};
      const half2 ps = ph[k] * s2;
      cs = __builtin_amdgcn_fdot2(ps, ones, cs, false);
      ms = __builtin_amdgcn_fdot2(ph[k], m2, ms, false);
      pa[2 * k] = ps[0];
      pa[2 * k + 1] = ps[1];
    }
    lds_st<half4>(ptile + g * 512 + 8 * lane, pa);
    st[1 + g] = cs;
    st[5 + g] = ms;
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
  // lane / 32 + 2 m, four rows per batch
  const int part = lane & 31;
#pragma unroll 1
  for (int m0 = 0; m0 < kTile / 2; m0 += 4) {
    u32x4 ra[4], rc[4];
    int kind[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
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
    for (int u = 0; u < 4; ++u) {
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

// First item whose cost prefix reaches c (items: D BF16 tiles of cost
// kDenseCost, then packed tiles of cost 1).
__device__ inline int item_of_cost(int c, int D) {
  return c <= kDenseCost * D ? (c + kDenseCost - 1) / kDenseCost : D + (c - kDenseCost * D);
}

// ---------------------------------------------------------------------------

template <int BITS>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  const int split = blockIdx.x % p.n_splits;
  const int grp = blockIdx.x / p.n_splits;  // b * n_hb + hb
  const int hb = grp % p.n_hb, b = grp / p.n_hb;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n16 = lane & 15, gq = lane >> 4;
  uint8_t* const xt_own = smem + kOffX + wave * kXTile;
  uint8_t* const p_own = smem + kOffP + wave * kPTile;
  uint8_t* const meta_own = smem + kOffMeta + wave * 256;
  uint8_t* const rmeta_own = smem + kOffRMeta + wave * 256;
  float* const smax = reinterpret_cast<float*>(smem + kOffMax);
  int* const s_pid = reinterpret_cast<int*>(smem + kOffPid);
  const uint8_t* const qr_row = smem + kOffQr + n16 * 128;
  uint8_t* const ql_stage = smem + kOffX;  // query rows, until round 0 writes x tiles

  stage_query(ql_stage, smem + kOffQr, p, b, hb, wave, lane);
  const SeqRanges sr = seq_ranges(p, b);

  // this workgroup's items: BF16 tiles first (cost kDenseCost), then packed;
  // wave w takes the contiguous run [my0, my1)
  const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
  const int D = (n_dense + kTile - 1) / kTile;
  const int t_lo = sr.lo_p / kTile;
  const int T = sr.hi_p > sr.lo_p ? (sr.hi_p + kTile - 1) / kTile - t_lo : 0;
  const int cost = kDenseCost * D + T;
  const int cs = (cost + p.n_splits - 1) / p.n_splits;
  const int c0 = min(cost, split * cs), c1 = min(cost, c0 + cs);
  const int i0 = item_of_cost(c0, D), i1 = item_of_cost(c1, D);
  const int rounds = (i1 - i0 + kWaves - 1) / kWaves;
  const int my0 = i0 + wave * rounds, my1 = min(i1, my0 + rounds);

  // page ids of the packed items, staged once
  const int ip0 = max(i0, D);
  int pg_first = 0, n_pg = 0;
  if (i1 > ip0) {
    pg_first = ((t_lo + ip0 - D) * kTile) >> p.log2P;
    n_pg = (((t_lo + i1 - 1 - D) * kTile) >> p.log2P) - pg_first + 1;
  }
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  for (int k = threadIdx.x; k < min(n_pg, kPageWin); k += kThreads) s_pid[k] = bt_row[pg_first + k];
  bool pid_staged = false;  // the first tile reads the block table directly
  auto page_ptr_of = [&](int pidx) -> const uint8_t* {
    const int k = pidx - pg_first;
    const int id = uniform(pid_staged && k < kPageWin ? *reinterpret_cast<volatile int*>(s_pid + k) : bt_row[pidx]);
    return page_of_id(p, id);
  };

  const LaneOffs lo{static_cast<uint32_t>(n16 * (kLatentDim * BITS / 8) + (BITS == 4 ? 16 : 8) * gq),
                    static_cast<uint32_t>(n16 * kRopeRowBytes + 8 * gq), static_cast<uint32_t>(n16 * 16)};

  // running max: m_run for head n16 (score layout), m_o[r] for heads 4 gq + r
  // (output layout); identical in every wave.  Output of latent group `wave`:
  // heads 4 gq + r, columns 16 kk + n16.  Per-lane sums (head n16): st.
  float m_run = kNegInf;
  float m_o[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  f32x4 o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float st[kStatW];
#pragma unroll
  for (int k = 0; k < kStatW; ++k) st[k] = 0.f;

  Stage<BITS> cur;
  RopeOps ro;
  int ro_page = -1;
  // Loads packed item `it` into sg; returns its page index, -1 for a BF16
  // item or none, -2 for a page missing from the block table.
  auto stage_for = [&](Stage<BITS>& sg, int it, int prev_page) -> int {
    if (it >= my1 || it < D) return -1;
    const int j0 = (t_lo + (it - D)) * kTile;
    const int pidx = j0 >> p.log2P;
    const uint8_t* page = page_ptr_of(pidx);
    if (!page) return -2;
    load_stage<BITS>(sg, page, j0 & (p.P - 1), pidx != prev_page, lo, lane, p);
    return pidx;
  };
  int cur_pidx = stage_for(cur, my0, ro_page);
  pid_staged = true;
  __syncthreads();  // query rows and page ids staged
  QueryOps<BITS> q;
  load_query<BITS>(q, ql_stage, n16, gq);
  __syncthreads();  // query rows read: the x tiles may be written
  if (my0 >= my1) {  // a wave without tiles still feeds zeros to the output MFMAs
    for (int o = 16 * lane; o < kXTile; o += 64 * 16) lds_st<u32x4>(xt_own + o, u32x4{0, 0, 0, 0});
  }

  for (int r = 0; r < rounds; ++r) {
    const int it = my0 + r;

    // 1. scores of this wave's tile
    float sc[4];
    bool has = it < my1;
    const bool dense = has && it < D;
    if (dense) {
      dense_scores<BITS>(sc, q, qr_row, b, sr, it * kTile, xt_own, p_own, lane, n16, gq, p);
    } else if (has && cur_pidx >= 0) {
      const int j0 = (t_lo + (it - D)) * kTile;
      const bool new_page = cur_pidx != ro_page;
      f32x4 acc[5];
#pragma unroll
      for (int g = 0; g < 5; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      packed_mfma<BITS>(acc, q, ro, cur, new_page, xt_own, meta_own, rmeta_own, qr_row, lane, n16, gq);
      ro_page = cur_pidx;
      // the codes of this wave's next tile, in flight while the round finishes
      cur_pidx = stage_for(cur, it + 1, ro_page);
      packed_fold<BITS>(sc, acc, ro.bias, j0, sr.lo_p, sr.hi_p, meta_own, gq, p.c_log2);
    } else {
      has = false;
    }
    if (!has || dense) cur_pidx = stage_for(cur, it + 1, ro_page);
    if (!has) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sc[k] = kNegInf;
    }
    float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tmax = row_allmax(tmax);
    if (gq == 0) smax[n16 * kWaves + wave] = tmax;
    lds_barrier();

    // 2. softmax: common running max, this tile's weights
    {
      const f32x4 mv = lds_ld<f32x4>(reinterpret_cast<const uint8_t*>(smax + n16 * kWaves));
      const float rmax = fmaxf(m_run, fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
      const float alpha = m_run == kNegInf ? 0.f : exp2f(m_run - rmax);
      m_run = rmax;
#pragma unroll
      for (int k = 0; k < kStatW; ++k) st[k] *= alpha;
    }
    if (has) {
      float pr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pr[k] = sc[k] == kNegInf ? 0.f : exp2f(sc[k] - m_run);
      if (dense) {
        half4 pa;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          st[0] += pr[k];
          pa[k] = static_cast<_Float16>(pr[k] * (1.f / kappa));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) lds_st<half4>(p_own + g * 512 + 8 * lane, pa);
      } else {
        packed_weights(pr, meta_own, p_own, st, lane, gq);
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) lds_st<u32x2>(p_own + g * 512 + 8 * lane, u32x2{0, 0});
    }
    // output-layout copy of the running max: heads 4 gq + rr
    float ah[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x4 mv = lds_ld<f32x4>(reinterpret_cast<const uint8_t*>(smax + (4 * gq + rr) * kWaves));
      const float rmax = fmaxf(m_o[rr], fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
      ah[rr] = m_o[rr] == kNegInf ? 0.f : exp2f(m_o[rr] - rmax);
      m_o[rr] = rmax;
    }
    lds_barrier();

    // 3. output of latent group `wave` for the four tiles of the round, in
    //    pairs: A slots 0-3 tile t (tokens 4 gq + j), slots 4-7 tile t + 1
    if (__any(ah[0] != 1.f || ah[1] != 1.f || ah[2] != 1.f || ah[3] != 1.f)) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[k][rr] *= ah[rr];
      }
    }
#pragma unroll
    for (int t = 0; t < kWaves; t += 2) {
      const half4 p0 = lds_ld<half4>(smem + kOffP + t * kPTile + wave * 512 + 8 * lane);
      const half4 p1 = lds_ld<half4>(smem + kOffP + (t + 1) * kPTile + wave * 512 + 8 * lane);
      const half8 pa = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
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
        o[kk] = mfma(pa, vb, o[kk]);
      }
    }
    lds_barrier();
  }

  // per-head sums of every wave, through the (now idle) P' area
  float* const sfin = reinterpret_cast<float*>(smem + kOffP);
#pragma unroll
  for (int k = 0; k < kStatW; ++k) {
    const float v = row_allsum(st[k]);
    if (gq == 0) sfin[(wave * kHeadBlock + n16) * kStatW + k] = v;
  }
  __syncthreads();
  const bool direct = p.n_splits == 1;
  // partial layout (per split): O as [group][kk][lane] f32x4 over heads
  // 4 gq + r (the MFMA accumulator layout, so every store is 16 B), then the
  // running max and the sum of the 16 heads
  float* part = p.parts + (static_cast<int64_t>(grp) * p.n_splits + split) * kPartFloats;
  float l_h[4], c_h[4], m_h[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int hh = 4 * gq + rr;
    float l = 0.f, c = 0.f, m = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* f = sfin + (w * kHeadBlock + hh) * kStatW;
      l += f[0];
      c += f[1 + wave];
      m += f[5 + wave];
    }
    l_h[rr] = l;
    c_h[rr] = c;
    m_h[rr] = m;
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    f32x4 v;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) v[rr] = fmaf(kappa, o[kk][rr] - c_h[rr], m_h[rr]);
    if (direct) {
      const int ch = col_to_channel<BITS>(128 * wave + 16 * kk + n16);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int hg = hb * kHeadBlock + 4 * gq + rr;
        if (hg < p.heads)
          p.out[(static_cast<int64_t>(b) * p.heads + hg) * kLatentDim + ch] = l_h[rr] > 0.f ? v[rr] / l_h[rr] : 0.f;
      }
    } else {
      reinterpret_cast<f32x4*>(part)[(wave * 8 + kk) * 64 + lane] = v;
    }
  }
  if (wave == 0 && n16 == 0) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int hh = 4 * gq + rr, hg = hb * kHeadBlock + hh;
      if (direct) {
        if (hg < p.heads)
          p.lse[static_cast<int64_t>(b) * p.heads + hg] =
              l_h[rr] > 0.f ? (m_o[rr] + log2f(l_h[rr])) * 0.69314718055994531f : kNegInf;
      } else {
        part[kHeadBlock * kLatentDim + hh] = m_o[rr];
        part[kHeadBlock * kLatentDim + kHeadBlock + hh] = l_h[rr];
      }
    }
  }
}

// Merge of the per-split partials of one sequence and head block.  Split s
// holds O_s = sum_j p_j c_j with p_j = 2^(z_j - m_s) and l_s = sum_j p_j; the
// result is sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
// One workgroup of 64 threads per (sequence, head block, latent group g,
// 16-column block kk); thread = MFMA lane (n16, gq): column 128 g + 16 kk +
// n16 of heads 4 gq + r.
template <int BITS>
__global__ void __launch_bounds__(64) combine_kernel(const float* __restrict__ parts, float* __restrict__ out,
                                                     float* __restrict__ lse, int heads, int n_hb, int n_splits) {
  __shared__ float s_ml[kMaxSplits][2 * kHeadBlock];  // per split: max of the 16 heads, then sums
  __shared__ float s_M[kHeadBlock], s_L[kHeadBlock];
  const int grp = blockIdx.x >> 5, gk = blockIdx.x & 31;  // gk = 8 g + kk
  const int b = grp / n_hb, hb = grp % n_hb;
  const int t = threadIdx.x, n16 = t & 15, gq = t >> 4;
  const float* base = parts + static_cast<int64_t>(grp) * n_splits * kPartFloats;
  // this thread's partials of the first splits go out before the (max, sum)
  // staging, so both latencies overlap
  constexpr int kEarly = 16;
  f32x4 v[kEarly];
#pragma unroll
  for (int s = 0; s < kEarly; ++s)
    v[s] = s < n_splits ? ldg<f32x4>(base + static_cast<int64_t>(s) * kPartFloats + 4 * (gk * 64 + t))
                        : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = t; k < n_splits * 2 * kHeadBlock; k += 64)
    s_ml[k >> 5][k & 31] = base[(k >> 5) * kPartFloats + kHeadBlock * kLatentDim + (k & 31)];
  __syncthreads();
  if (t < kHeadBlock) {
    float M = kNegInf;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, s_ml[s][t]);
    float L = 0.f;
    for (int s = 0; s < n_splits; ++s) L = fmaf(s_ml[s][t] == kNegInf ? 0.f : exp2f(s_ml[s][t] - M), s_ml[s][16 + t], L);
    s_M[t] = M;
    s_L[t] = L;
  }
  __syncthreads();
  float Mh[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) Mh[rr] = s_M[4 * gq + rr];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](int s, const f32x4& x) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float m_s = s_ml[s][4 * gq + rr];
      const float f = m_s == kNegInf ? 0.f : exp2f(m_s - Mh[rr]);
      acc[rr] = fmaf(f, x[rr], acc[rr]);
    }
  };
#pragma unroll
  for (int s = 0; s < kEarly; ++s)
    if (s < n_splits) add(s, v[s]);
#pragma unroll 8
  for (int s = kEarly; s < n_splits; ++s)
    add(s, ldg<f32x4>(base + static_cast<int64_t>(s) * kPartFloats + 4 * (gk * 64 + t)));
  const int ch = col_to_channel<BITS>(16 * gk + n16);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int hg = hb * kHeadBlock + 4 * gq + rr;
    const float L = s_L[4 * gq + rr];
    if (hg < heads) out[(static_cast<int64_t>(b) * heads + hg) * kLatentDim + ch] = L > 0.f ? acc[rr] / L : 0.f;
  }
  if (gk == 0 && t < kHeadBlock && hb * kHeadBlock + t < heads)
    lse[static_cast<int64_t>(b) * heads + hb * kHeadBlock + t] =
        s_L[t] > 0.f ? (s_M[t] + log2f(s_L[t])) * 0.69314718055994531f : kNegInf;
}

}  // namespace
}  // namespace mla

extern "C" int mla_lowbit_decode(const mla_lowbit_layout* layout, const void* q_lat, const void* q_rope,
                                 int32_t batch, int32_t heads, float softmax_scale, const void* page_pool,
                                 int32_t num_pool_pages, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seqlens, int32_t max_seqlen, const void* sink_buf,
                                 const void* ring_buf, const void* rope_tail, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace mla;
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
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return MLA_LOWBIT_ERR_WORKSPACE;
  DecodeParams p{};
  p.q_lat = static_cast<const uint16_t*>(q_lat);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.pool = static_cast<const uint8_t*>(page_pool);
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.sink = static_cast<const uint16_t*>(sink_buf);
  p.ring = static_cast<const uint16_t*>(ring_buf);
  p.tail = static_cast<const uint16_t*>(rope_tail);
  p.parts = static_cast<float*>(workspace);
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.heads = heads;
  p.max_pages = max_pages;
  p.num_pool_pages = num_pool_pages;
  p.max_seqlen = max_seqlen;
  p.n_hb = plan.n_hb;
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
  const int64_t groups = static_cast<int64_t>(batch) * plan.n_hb;
  const int64_t blocks = groups * plan.n_splits;
  if (blocks > 0x7FFFFFFF || groups * 32 > 0x7FFFFFFF) return MLA_LOWBIT_ERR_UNSUPPORTED;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess)
      return MLA_LOWBIT_ERR_HIP;
    attr_set = true;
  }
  if (g.latent_bits == 4)
    hipLaunchKernelGGL(decode_kernel<4>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), kLdsBytes,
                       stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<2>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), kLdsBytes,
                       stream, p);
  if (hipGetLastError() != hipSuccess) return MLA_LOWBIT_ERR_HIP;
  if (plan.n_splits > 1) {
    const dim3 grid(static_cast<uint32_t>(groups * 32));
    if (g.latent_bits == 4)
      hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(64), 0, stream, p.parts, out, lse, heads, plan.n_hb,
                         plan.n_splits);
    else
      hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(64), 0, stream, p.parts, out, lse, heads, plan.n_hb,
                         plan.n_splits);
    if (hipGetLastError() != hipSuccess) return MLA_LOWBIT_ERR_HIP;
  }
  return MLA_LOWBIT_OK;
}
