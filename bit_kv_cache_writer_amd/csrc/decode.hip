// Decode attention over the dual-path low-bit MLA cache, for gfx950.
//
// What is computed (QuantMLA Figure 8 caption; RAQ-MLA abstract and
// Figure 4 caption): per sequence and head, one softmax over all valid
// tokens of score = q_lat . c_KV + q_rope . k_R, output sum_j p_j c_KV_j in
// latent space; protected (sink / recent) tokens from BF16, the others from
// codes dequantized inside the loop -- the same reconstructed content tile
// feeds both the score (matching) and the output (aggregation).
//
// How (one workgroup = 4 waves per (sequence, 16-head block, token split);
// every wave walks its own 32-token tiles and keeps its own softmax state):
//  * Codes are loaded straight from the page into the lanes that feed the
//    score MFMA (v_mfma_f32_16x16x32_f16, M = 16 tokens, N = 16 heads,
//    K = 32 channels): lane (t, g) holds 8 channels of token t.  They are
//    unpacked in registers to fp16 x = 1 + code/kappa by OR-ing the code into
//    the top of an fp16 mantissa (kappa = 16 for 4-bit codes, 4 for 2-bit).
//  * The per-token group scale s and minimum m are folded after the MFMA:
//    c = kappa s (x - 1) + m, so
//      q.c = sum_g kappa s_g (q_g . x_g) + sum_g (m_g - kappa s_g) Q_g,
//    with Q_g = sum of the query over group g.  The second sum is one more
//    MFMA whose token operand is the raw fp16 (scale, min) metadata.
//  * The positional key has a scale/min per channel and page, folded into a
//    per-page query q' = q s (split into fp16 hi + lo halves) plus a per-page
//    bias sum_c q_c (m_c - 16 s_c).
//  * Scores come out of the MFMA with one head per lane, so the softmax
//    probabilities are already laid out as the A operand of the output MFMA
//    (M = heads, K = tokens); no transpose of P is needed.
//  * The unpacked fp16 tile is also written to LDS (token-major rows) and read
//    back with ds_read_b64_tr_b16, which hands every lane one channel of 4
//    tokens -- the token-contiguous B operand of the output MFMA.
//  * The output accumulates sum_j (p_j s_j) x_j per channel; the offset terms
//    -kappa sum_j fp16(p_j s_j) and sum_j p_j m_j are kept per (head, group)
//    in fp32 and applied once at the end.  The same rounded fp16 products
//    enter both sums, so the offset cancels exactly.
//  * The BF16 tokens (sink, recent window, and -- when the window is shorter
//    than a page -- the k_R of an unfinished page) run through the same MFMA
//    pipeline in one extra workgroup per (sequence, head block).
//  * Each workgroup merges its 4 waves in LDS and writes one partial
//    (unnormalized output, running max, sum) per head; a second kernel merges
//    the partials with log-sum-exp weights.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "decode_plan.h"
#include "geometry.h"

namespace mla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 64 * kDecodeWaves;
constexpr int kLdsRow = 1056;                    // bytes per token row: 512 fp16 + pad
constexpr int kWaveLds = kTile * kLdsRow;        // 33792 B per wave
constexpr float kPrescale = 1.0f / 256.0f;      // keeps q' and Q_g inside fp16 range
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
  float* ws;
  int32_t batch, heads, max_pages, num_pool_pages, max_seqlen;
  int32_t n_hb, n_splits, n_parts;
  int32_t P, sink_n, local;
  int64_t latent_row, latent_meta_off, rope_codes_off, rope_meta_off, page_bytes;
  float c_log2;  // softmax_scale * log2(e)
};

// Channel (within a lane group's 32-channel span) of slot s of chunk d, in
// the order the unpack below produces.
template <int BITS>
__device__ constexpr int chan_off(int d, int s) {
  return BITS == 4 ? 8 * d + (s >> 1) + 4 * (s & 1)
                   : 16 * (d >> 1) + 4 * (d & 1) + (s >> 1) + 8 * (s & 1);
}

// LDS column (slot order) -> latent channel.
template <int BITS>
__device__ inline int col_to_channel(int c) {
  return (c & ~31) + chan_off<BITS>((c >> 3) & 3, c & 7);
}

// 8 nibbles -> fp16 1 + code/16, slots [n0 n4 n1 n5 n2 n6 n3 n7].
__device__ inline half8 unpack4(uint32_t w) {
  const uint32_t M = 0x03C003C0u, E = 0x3C003C00u;
  u32x4 v;
  v[0] = ((w << 6) & M) | E;
  v[1] = ((w << 2) & M) | E;
  v[2] = ((w >> 2) & M) | E;
  v[3] = ((w >> 6) & M) | E;
  return __builtin_bit_cast(half8, v);
}

// 8 of the 16 crumbs of w -> fp16 1 + code/4; hi = 0: crumbs [0 8 1 9 2 10 3 11],
// hi = 1: crumbs [4 12 5 13 6 14 7 15].
__device__ inline half8 unpack2(uint32_t w, int hi) {
  const uint32_t M = 0x03000300u, E = 0x3C003C00u;
  u32x4 v;
  if (hi == 0) {
    v[0] = ((w << 8) & M) | E;
    v[1] = ((w << 6) & M) | E;
    v[2] = ((w << 4) & M) | E;
    v[3] = ((w << 2) & M) | E;
  } else {
    v[0] = (w & M) | E;
    v[1] = ((w >> 2) & M) | E;
    v[2] = ((w >> 4) & M) | E;
    v[3] = ((w >> 6) & M) | E;
  }
  return __builtin_bit_cast(half8, v);
}

__device__ inline float bf16f(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ inline float h2f(uint32_t h16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

__device__ inline f32x4 mfma(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ inline T ldg(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ inline float lane_group_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}
__device__ inline float lane_group_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Codes of one 32-token tile in the score-MFMA lane layout.
template <int BITS>
struct TileCodes {
  uint32_t lat[2][BITS == 4 ? 16 : 8];  // [token block][dwords of 4 groups]
  u32x2 rope[2];
};

template <int BITS>
__device__ inline void load_codes(TileCodes<BITS>& tc, const uint8_t* page, int slot0, int n16, int gq,
                                  const DecodeParams& p) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const uint8_t* row = page + static_cast<int64_t>(slot0 + 16 * kb + n16) * p.latent_row;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BITS == 4) {
        const u32x4 v = ldg<u32x4>(row + 64 * i + 16 * gq);
        tc.lat[kb][4 * i + 0] = v[0];
        tc.lat[kb][4 * i + 1] = v[1];
        tc.lat[kb][4 * i + 2] = v[2];
        tc.lat[kb][4 * i + 3] = v[3];
      } else {
        const u32x2 v = ldg<u32x2>(row + 32 * i + 8 * gq);
        tc.lat[kb][2 * i + 0] = v[0];
        tc.lat[kb][2 * i + 1] = v[1];
      }
    }
    tc.rope[kb] = ldg<u32x2>(page + p.rope_codes_off + static_cast<int64_t>(slot0 + 16 * kb + n16) * kRopeRowBytes + 8 * gq);
  }
}

template <int BITS>
__device__ inline half8 chunk_of(const TileCodes<BITS>& tc, int kb, int i, int d) {
  if constexpr (BITS == 4) return unpack4(tc.lat[kb][4 * i + d]);
  else return unpack2(tc.lat[kb][2 * i + (d >> 1)], d & 1);
}

// Per-lane softmax / output state of one wave.
struct WaveState {
  f32x4 o[32];     // output accumulators: heads 4*gq + r, LDS columns 16k + n16
  float m;         // running max (log2 domain) of head n16
  float l;         // partial sum of p over this lane's tokens
  float csum[4];   // partial sum of fp16(p * s_g) per group
  float msum[4];   // partial sum of p * m_g per group
};

__device__ inline void state_init(WaveState& st) {
#pragma unroll
  for (int k = 0; k < 32; ++k) st.o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) st.csum[g] = st.msum[g] = 0.f;
}

// Raises the running max to cover a tile with max mt (per head, already
// reduced over the lane groups) and rescales everything accumulated so far.
__device__ inline void softmax_raise(WaveState& st, float mt, int gq) {
  if (!__any(mt > st.m)) return;
  const float mn = fmaxf(st.m, mt);
  const float alpha = (mn == kNegInf || st.m == kNegInf) ? (st.m == kNegInf ? 0.f : 1.f) : exp2f(st.m - mn);
  st.m = mn;
  st.l *= alpha;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    st.csum[g] *= alpha;
    st.msum[g] *= alpha;
  }
  float ah[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ah[r] = __shfl(alpha, 4 * gq + r, 64);
#pragma unroll
  for (int k = 0; k < 32; ++k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[k][r] *= ah[r];
  }
}

// Output MFMAs of one tile: B operand = LDS tile rows read transposed.
__device__ inline void pv_tile(WaveState& st, const half8 (&pa)[4], const uint8_t* lds, int n16, int gq) {
  const uint8_t* base = lds + (4 * gq + (n16 >> 2)) * kLdsRow + 8 * (n16 & 3);
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint8_t* a1 = base + 32 * k;
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(a1));
    const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(a1 + 16 * kLdsRow));
    // whole-vector shuffle + bit cast (element-wise casts of the transposed
    // result were mis-assembled by the compiler)
    const half8 vb = __builtin_bit_cast(half8, __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7));
    st.o[k] = mfma(pa[k >> 3], vb, st.o[k]);
  }
}

// Query operands of one 16-head block, in the slot order of the unpack.
template <int BITS>
struct QueryOps {
  half8 lat[4][4];  // [group][chunk]
  half8 meta;       // (scale, min) slots of the metadata MFMA, prescaled
  float qg[4];      // sum of q over each group (full, all lanes)
  float qr[16];     // q_rope channels 16*gq .. 16*gq+15 (fp32)
};

template <int BITS>
__device__ inline void load_query(QueryOps<BITS>& q, const DecodeParams& p, int b, int h, int gq) {
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  const bool hv = h < p.heads;
  const uint16_t* ql = p.q_lat + (static_cast<int64_t>(b) * p.heads + (hv ? h : 0)) * kLatentDim;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 w = hv ? ldg<u32x4>(ql + 128 * i + 32 * gq + 8 * u) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * u + 2 * e] = bf16f(w[e] & 0xFFFFu);
        v[8 * u + 2 * e + 1] = bf16f(w[e] >> 16);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) s += v[c];
    q.qg[i] = lane_group_sum(s);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) q.lat[i][d][sl] = static_cast<_Float16>(v[chan_off<BITS>(d, sl)]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = -kappa * q.qg[i] * kPrescale, c = q.qg[i] * kPrescale;
    const _Float16 ah = static_cast<_Float16>(a), ch = static_cast<_Float16>(c);
    const _Float16 al = static_cast<_Float16>(a - static_cast<float>(ah));
    const _Float16 cl = static_cast<_Float16>(c - static_cast<float>(ch));
    q.meta[2 * i] = gq == 0 ? ah : (gq == 1 ? al : static_cast<_Float16>(0.f));
    q.meta[2 * i + 1] = gq == 0 ? ch : (gq == 1 ? cl : static_cast<_Float16>(0.f));
  }
  const uint16_t* qr = p.q_rope + (static_cast<int64_t>(b) * p.heads + (hv ? h : 0)) * kRopeDim + 16 * gq;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const u32x4 w = hv ? ldg<u32x4>(qr + 8 * u) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q.qr[8 * u + 2 * e] = bf16f(w[e] & 0xFFFFu);
      q.qr[8 * u + 2 * e + 1] = bf16f(w[e] >> 16);
    }
  }
}

// Per-page positional-key operands: q' = q s / 16 prescaled (hi, lo) and the
// bias sum_c q_c (m_c - 16 s_c), for channels 16*gq + 8e + slot order.
struct RopeOps {
  half8 hi[2], lo[2];
  float bias;
};

__device__ inline void rope_ops(RopeOps& r, const float (&qr)[16], const uint8_t* page, int gq,
                                const DecodeParams& p) {
  const uint16_t* meta = reinterpret_cast<const uint16_t*>(page + p.rope_meta_off);
  const u32x4 s0 = ldg<u32x4>(meta + 16 * gq), s1 = ldg<u32x4>(meta + 16 * gq + 8);
  const u32x4 m0 = ldg<u32x4>(meta + kRopeDim + 16 * gq), m1 = ldg<u32x4>(meta + kRopeDim + 16 * gq + 8);
  float sc[16], mn[16];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sc[2 * e] = h2f(s0[e] & 0xFFFFu);
    sc[2 * e + 1] = h2f(s0[e] >> 16);
    sc[8 + 2 * e] = h2f(s1[e] & 0xFFFFu);
    sc[8 + 2 * e + 1] = h2f(s1[e] >> 16);
    mn[2 * e] = h2f(m0[e] & 0xFFFFu);
    mn[2 * e + 1] = h2f(m0[e] >> 16);
    mn[8 + 2 * e] = h2f(m1[e] & 0xFFFFu);
    mn[8 + 2 * e + 1] = h2f(m1[e] >> 16);
  }
  float bias = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) bias += qr[c] * (mn[c] - 16.f * sc[c]);
  r.bias = lane_group_sum(bias);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int c = 8 * e + chan_off<4>(0, sl);
      const float v = qr[c] * sc[c] * (16.f * kPrescale);
      const _Float16 vh = static_cast<_Float16>(v);
      r.hi[e][sl] = vh;
      r.lo[e][sl] = static_cast<_Float16>(v - static_cast<float>(vh));
    }
  }
}

// Token ranges of sequence b: packed [lo_p, hi_p); BF16 / tail otherwise.
struct SeqRanges {
  int L, lo_p, hi_p;
};

__device__ inline SeqRanges seq_ranges(const DecodeParams& p, int b) {
  SeqRanges r;
  int L = p.seqlens[b];
  const int cap = min(p.max_seqlen, p.max_pages * p.P);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  r.L = L;
  r.lo_p = min(p.sink_n, L);
  const int full = (L / p.P) * p.P;
  r.hi_p = max(r.lo_p, min(L - p.local, full));
  return r;
}

__device__ inline const uint8_t* page_ptr(const DecodeParams& p, int b, int pidx) {
  if (pidx < 0 || pidx >= p.max_pages) return nullptr;
  const int id = p.block_table[static_cast<int64_t>(b) * p.max_pages + pidx];
  if (id < 0 || id >= p.num_pool_pages) return nullptr;
  return p.pool + static_cast<int64_t>(id) * p.page_bytes;
}

// One packed tile: tokens j0 .. j0+31 of one page, valid in [vlo, vhi).
// Latent metadata of a tile: the MFMA operand rows (token n16 of each block)
// and the values the fold needs (tokens 4*gq + r of each block).
struct TileMeta {
  u32x4 ma[2], ms[2][4];
};

__device__ inline void load_meta(TileMeta& tm, const uint8_t* page, int slot0, int n16, int gq,
                                 const DecodeParams& p) {
  const uint8_t* meta = page + p.latent_meta_off;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    tm.ma[kb] = gq < 2 ? ldg<u32x4>(meta + (slot0 + 16 * kb + n16) * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) tm.ms[kb][r] = ldg<u32x4>(meta + (slot0 + 16 * kb + 4 * gq + r) * 16);
  }
}

template <int BITS>
__device__ void packed_tile(WaveState& st, const QueryOps<BITS>& q, const RopeOps& ro,
                            const TileCodes<BITS>& tc, const TileMeta& tm, int j0, int vlo, int vhi,
                            uint8_t* lds, int n16, int gq, const DecodeParams& p) {
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  const u32x4(&ma)[2] = tm.ma;
  const u32x4(&ms)[2][4] = tm.ms;
  f32x4 acc[2][5];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int g = 0; g < 5; ++g) acc[kb][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint8_t* lrow = lds + (16 * kb + n16) * kLdsRow + 64 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const half8 x = chunk_of<BITS>(tc, kb, i, d);
        acc[kb][i] = mfma(x, q.lat[i][d], acc[kb][i]);
        *reinterpret_cast<half8*>(lrow + 256 * i + 16 * d) = x;
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const half8 xr = unpack4(tc.rope[kb][e]);
      acc[kb][4] = mfma(xr, ro.hi[e], acc[kb][4]);
      acc[kb][4] = mfma(xr, ro.lo[e], acc[kb][4]);
    }
    acc[kb][4] = mfma(__builtin_bit_cast(half8, ma[kb]), q.meta, acc[kb][4]);
  }
  // fold the group scales, mask, online softmax
  float sc[8];
  bool valid[8];
  float tmax = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = j0 + 16 * kb + 4 * gq + r;
      const u32x4 mm = ms[kb][r];
      float v = h2f(mm[0] & 0xFFFFu) * acc[kb][0][r];
      v = fmaf(h2f(mm[1] & 0xFFFFu), acc[kb][1][r], v);
      v = fmaf(h2f(mm[2] & 0xFFFFu), acc[kb][2][r], v);
      v = fmaf(h2f(mm[3] & 0xFFFFu), acc[kb][3][r], v);
      v = fmaf(v, kappa, fmaf(acc[kb][4][r], 256.f, ro.bias));
      const bool ok = t >= vlo && t < vhi;
      valid[4 * kb + r] = ok;
      sc[4 * kb + r] = ok ? v * p.c_log2 : kNegInf;
      tmax = fmaxf(tmax, sc[4 * kb + r]);
    }
  }
  tmax = lane_group_max(tmax);
  softmax_raise(st, tmax, gq);
  float pr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    pr[k] = valid[k] ? exp2f(sc[k] - st.m) : 0.f;
    st.l += pr[k];
  }
  half8 pa[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t w = ms[k >> 2][k & 3][g];
      const float ps = valid[k] ? pr[k] * h2f(w & 0xFFFFu) : 0.f;
      pa[g][k] = static_cast<_Float16>(ps);
      st.csum[g] += static_cast<float>(pa[g][k]);
      st.msum[g] += valid[k] ? pr[k] * h2f(w >> 16) : 0.f;
    }
  }
  lds_wait();
  pv_tile(st, pa, lds, n16, gq);
}

// Source of one BF16-path token (sink row, ring slot, or packed latent with
// the k_R of an unfinished page from the tail buffer).
struct DenseSrc {
  const uint16_t* row;    // bf16 [576] row, or nullptr
  const uint8_t* page;    // packed latent page when row == nullptr
  const uint16_t* rope;   // bf16 k_R [64]
  int slot;
};

__device__ inline DenseSrc dense_src(const DecodeParams& p, int b, const SeqRanges& sr, int k) {
  DenseSrc s{nullptr, nullptr, nullptr, 0};
  const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
  if (k >= n_dense) return s;
  const int j = k < sr.lo_p ? k : sr.hi_p + (k - sr.lo_p);
  if (j < p.sink_n) {
    s.row = p.sink + (static_cast<int64_t>(b) * p.sink_n + j) * kRowElems;
  } else if (p.local > 0 && j >= sr.L - p.local) {
    s.row = p.ring + (static_cast<int64_t>(b) * p.local + j % p.local) * kRowElems;
  } else {
    s.page = page_ptr(p, b, j / p.P);
    s.slot = j % p.P;
    s.rope = p.tail + (static_cast<int64_t>(b) * p.P + j % p.P) * kRopeDim;
    if (!s.page) s.rope = nullptr;
  }
  if (s.row) s.rope = s.row + kLatentDim;
  return s;
}

// fp32 values of latent channels 128 i + 32 gq + (0..31) of a BF16-path token.
template <int BITS>
__device__ inline void dense_latent(float (&v)[32], const DenseSrc& s, int i, int gq, const DecodeParams& p) {
  if (s.row) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 w = ldg<u32x4>(s.row + 128 * i + 32 * gq + 8 * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * u + 2 * e] = bf16f(w[e] & 0xFFFFu);
        v[8 * u + 2 * e + 1] = bf16f(w[e] >> 16);
      }
    }
  } else if (s.page) {
    const uint32_t mw = ldg<uint32_t>(s.page + p.latent_meta_off + s.slot * 16 + 4 * i);
    const float sc = h2f(mw & 0xFFFFu), mn = h2f(mw >> 16);
    const uint8_t* row = s.page + static_cast<int64_t>(s.slot) * p.latent_row;
    if constexpr (BITS == 4) {
      const u32x4 w = ldg<u32x4>(row + 64 * i + 16 * gq);
#pragma unroll
      for (int c = 0; c < 32; ++c) v[c] = fmaf(static_cast<float>((w[c >> 3] >> (4 * (c & 7))) & 15u), sc, mn);
    } else {
      const u32x2 w = ldg<u32x2>(row + 32 * i + 8 * gq);
#pragma unroll
      for (int c = 0; c < 32; ++c) v[c] = fmaf(static_cast<float>((w[c >> 4] >> (2 * (c & 15))) & 3u), sc, mn);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] = 0.f;
  }
}

// One tile of BF16-path tokens (dense indices k0 .. k0+31).
template <int BITS>
__device__ void dense_tile(WaveState& st, const QueryOps<BITS>& q, const half8 (&qrp)[2], int b,
                           const SeqRanges& sr, int k0, uint8_t* lds, int n16, int gq,
                           const DecodeParams& p) {
  constexpr float inv_kappa = BITS == 4 ? 1.f / 16.f : 1.f / 4.f;
  f32x4 acc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const DenseSrc s = dense_src(p, b, sr, k0 + 16 * kb + n16);
    uint8_t* lrow = lds + (16 * kb + n16) * kLdsRow + 64 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[32];
      dense_latent<BITS>(v, s, i, gq, p);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        half8 x;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) x[sl] = static_cast<_Float16>(v[chan_off<BITS>(d, sl)]);
        acc[kb] = mfma(x, q.lat[i][d], acc[kb]);
        *reinterpret_cast<half8*>(lrow + 256 * i + 16 * d) = x;
      }
    }
    float r[16];
    if (s.rope) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 w = ldg<u32x4>(s.rope + 16 * gq + 8 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[8 * u + 2 * e] = bf16f(w[e] & 0xFFFFu);
          r[8 * u + 2 * e + 1] = bf16f(w[e] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) r[c] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      half8 xr;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) xr[sl] = static_cast<_Float16>(r[8 * e + chan_off<4>(0, sl)]);
      acc[kb] = mfma(xr, qrp[e], acc[kb]);
    }
  }
  const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
  float sc[8];
  bool valid[8];
  float tmax = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = k0 + 16 * kb + 4 * gq + r;
      const bool ok = k < n_dense;
      valid[4 * kb + r] = ok;
      sc[4 * kb + r] = ok ? acc[kb][r] * p.c_log2 : kNegInf;
      tmax = fmaxf(tmax, sc[4 * kb + r]);
    }
  }
  tmax = lane_group_max(tmax);
  softmax_raise(st, tmax, gq);
  half8 pa1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float pr = valid[k] ? exp2f(sc[k] - st.m) : 0.f;
    st.l += pr;
    pa1[k] = static_cast<_Float16>(pr * inv_kappa);
  }
  const half8 pa[4] = {pa1, pa1, pa1, pa1};
  lds_wait();
  pv_tile(st, pa, lds, n16, gq);
}

template <int BITS>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr float kappa = BITS == 4 ? 16.f : 4.f;
  const int part = blockIdx.x % p.n_parts;
  const int hb = (blockIdx.x / p.n_parts) % p.n_hb;
  const int b = blockIdx.x / (p.n_parts * p.n_hb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, gq = lane >> 4;
  const int h = hb * kHeadBlock + n16;
  uint8_t* lds = smem + wave * kWaveLds;

  QueryOps<BITS> q;
  load_query<BITS>(q, p, b, h, gq);
  WaveState st;
  state_init(st);
  const SeqRanges sr = seq_ranges(p, b);

  if (part < p.n_splits) {
    // packed tokens: absolute 32-token tiles [t_lo, t_hi) of [lo_p, hi_p)
    const int t_lo = sr.lo_p / kTile, t_hi = (sr.hi_p + kTile - 1) / kTile;
    const int n_t = sr.hi_p > sr.lo_p ? t_hi - t_lo : 0;
    const int per = (n_t + p.n_splits - 1) / p.n_splits;
    const int s_lo = t_lo + part * per, s_hi = min(t_hi, s_lo + per);
    RopeOps ro;
    int ro_page = -1;
    TileCodes<BITS> cur, nxt;
    const uint8_t* cur_page = nullptr;
    int tt = s_lo + wave;
    if (n_t > 0 && tt < s_hi) {
      cur_page = page_ptr(p, b, (tt * kTile) / p.P);
      if (cur_page) load_codes<BITS>(cur, cur_page, (tt * kTile) % p.P, n16, gq, p);
    }
    for (; n_t > 0 && tt < s_hi; tt += kDecodeWaves) {
      const int j0 = tt * kTile;
      const int pidx = j0 / p.P;
      if (cur_page && pidx != ro_page) {
        rope_ops(ro, q.qr, cur_page, gq, p);
        ro_page = pidx;
      }
      TileMeta tm;
      if (cur_page) load_meta(tm, cur_page, j0 % p.P, n16, gq, p);
      // prefetch the next tile's codes after this tile's metadata, so that
      // waiting for the metadata never waits for the prefetch
      const uint8_t* nxt_page = nullptr;
      const int tn = tt + kDecodeWaves;
      if (tn < s_hi) {
        nxt_page = page_ptr(p, b, (tn * kTile) / p.P);
        if (nxt_page) load_codes<BITS>(nxt, nxt_page, (tn * kTile) % p.P, n16, gq, p);
      }
      if (cur_page) packed_tile<BITS>(st, q, ro, cur, tm, j0, sr.lo_p, sr.hi_p, lds, n16, gq, p);
      cur = nxt;
      cur_page = nxt_page;
    }
  } else {
    // BF16 path: plain fp16 rope query
    half8 qrp[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) qrp[e][sl] = static_cast<_Float16>(q.qr[8 * e + chan_off<4>(0, sl)]);
    }
    const int n_dense = sr.lo_p + (sr.L - sr.hi_p);
    for (int k0 = wave * kTile; k0 < n_dense; k0 += kDecodeWaves * kTile)
      dense_tile<BITS>(st, q, qrp, b, sr, k0, lds, n16, gq, p);
  }

  // finish this wave: offsets of the output, totals per head
  st.l = lane_group_sum(st.l);
  float cs[4], msum[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    cs[g] = lane_group_sum(st.csum[g]);
    msum[g] = lane_group_sum(st.msum[g]);
  }
  float corr_c[4][4], corr_m[4][4];  // [row r][group]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      corr_c[r][g] = __shfl(cs[g], 4 * gq + r, 64);
      corr_m[r][g] = __shfl(msum[g], 4 * gq + r, 64);
    }
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[k][r] = fmaf(kappa, st.o[k][r] - corr_c[r][k >> 3], corr_m[r][k >> 3]);
  }
  float mr[4], lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mr[r] = __shfl(st.m, 4 * gq + r, 64);
    lr[r] = __shfl(st.l, 4 * gq + r, 64);
  }

  // merge the waves of the workgroup in LDS (reusing the tile buffers)
  __syncthreads();
  float* mine = reinterpret_cast<float*>(smem + wave * kWaveLds);
  if (wave > 0) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) mine[(4 * k + r) * 64 + lane] = st.o[k][r];
    }
    if (n16 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mine[8192 + 4 * gq + r] = mr[r];
        mine[8192 + 16 + 4 * gq + r] = lr[r];
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float mtot[4], f[kDecodeWaves][4], ltot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) mtot[r] = mr[r];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) {
    const float* other = reinterpret_cast<const float*>(smem + w * kWaveLds);
#pragma unroll
    for (int r = 0; r < 4; ++r) mtot[r] = fmaxf(mtot[r], other[8192 + 4 * gq + r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f[0][r] = mr[r] == kNegInf ? 0.f : exp2f(mr[r] - mtot[r]);
    ltot[r] = f[0][r] * lr[r];
  }
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) {
    const float* other = reinterpret_cast<const float*>(smem + w * kWaveLds);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mw = other[8192 + 4 * gq + r];
      f[w][r] = mw == kNegInf ? 0.f : exp2f(mw - mtot[r]);
      ltot[r] += f[w][r] * other[8192 + 16 + 4 * gq + r];
    }
  }
  float* out = p.ws + ((static_cast<int64_t>(b) * p.n_parts + part) * p.n_hb + hb) * kPartFloats;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int ch = col_to_channel<BITS>(16 * k + n16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = f[0][r] * st.o[k][r];
#pragma unroll
      for (int w = 1; w < kDecodeWaves; ++w) {
        const float* other = reinterpret_cast<const float*>(smem + w * kWaveLds);
        v = fmaf(f[w][r], other[(4 * k + r) * 64 + lane], v);
      }
      out[(4 * gq + r) * kLatentDim + ch] = v;
    }
  }
  if (n16 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      out[kHeadBlock * kLatentDim + 4 * gq + r] = mtot[r];
      out[kHeadBlock * kLatentDim + kHeadBlock + 4 * gq + r] = ltot[r];
    }
  }
}

// Merges the partials of every (sequence, head): log-sum-exp weights.
__global__ void __launch_bounds__(128) combine_kernel(const float* ws, float* out, float* lse, int heads,
                                                      int n_hb, int n_parts) {
  const int bh = blockIdx.x;
  const int b = bh / heads, h = bh % heads;
  const int hb = h / kHeadBlock, hl = h % kHeadBlock;
  const int tid = threadIdx.x;
  float mtot = kNegInf;
  for (int s = 0; s < n_parts; ++s) {
    const float* part = ws + ((static_cast<int64_t>(b) * n_parts + s) * n_hb + hb) * kPartFloats;
    mtot = fmaxf(mtot, part[kHeadBlock * kLatentDim + hl]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ltot = 0.f;
  for (int s = 0; s < n_parts; ++s) {
    const float* part = ws + ((static_cast<int64_t>(b) * n_parts + s) * n_hb + hb) * kPartFloats;
    const float ms = part[kHeadBlock * kLatentDim + hl];
    if (ms == kNegInf) continue;
    const float f = exp2f(ms - mtot);
    ltot = fmaf(f, part[kHeadBlock * kLatentDim + kHeadBlock + hl], ltot);
    const f32x4 o = *reinterpret_cast<const f32x4*>(part + hl * kLatentDim + 4 * tid);
    acc += f * o;
  }
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(bh) * kLatentDim + 4 * tid) = acc * inv;
  if (tid == 0) lse[bh] = ltot > 0.f ? (mtot + log2f(ltot)) * 0.69314718055994531f : kNegInf;
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
  if (!q_lat || !q_rope || !seqlens || !out || !lse || !workspace || !rope_tail) return MLA_LOWBIT_ERR_ARG;
  if (max_seqlen > 0 && (!page_pool || !block_table || num_pool_pages == 0)) return MLA_LOWBIT_ERR_ARG;
  if (g.sink > 0 && !sink_buf) return MLA_LOWBIT_ERR_ARG;
  if (g.local > 0 && !ring_buf) return MLA_LOWBIT_ERR_ARG;
  if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(out) || !aligned16(rope_tail) ||
      (page_pool && !aligned16(page_pool)) || (sink_buf && !aligned16(sink_buf)) ||
      (ring_buf && !aligned16(ring_buf)) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return MLA_LOWBIT_ERR_ARG;
  const DecodePlan plan = plan_decode(g, batch, heads, max_seqlen);
  if (workspace_bytes < plan.workspace_bytes) return MLA_LOWBIT_ERR_WORKSPACE;
  DecodeParams p{};
  p.q_lat = static_cast<const uint16_t*>(q_lat);
  p.q_rope = static_cast<const uint16_t*>(q_rope);
  p.pool = static_cast<const uint8_t*>(page_pool);
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.sink = static_cast<const uint16_t*>(sink_buf);
  p.ring = static_cast<const uint16_t*>(ring_buf);
  p.tail = static_cast<const uint16_t*>(rope_tail);
  p.ws = static_cast<float*>(workspace);
  p.batch = batch;
  p.heads = heads;
  p.max_pages = max_pages;
  p.num_pool_pages = num_pool_pages;
  p.max_seqlen = max_seqlen;
  p.n_hb = plan.n_hb;
  p.n_splits = plan.n_splits;
  p.n_parts = plan.n_parts;
  p.P = g.page_size;
  p.sink_n = g.sink;
  p.local = g.local;
  p.latent_row = g.latent_row;
  p.latent_meta_off = g.latent_meta_off;
  p.rope_codes_off = g.rope_codes_off;
  p.rope_meta_off = g.rope_meta_off;
  p.page_bytes = g.page_bytes;
  p.c_log2 = softmax_scale * 1.44269504088896341f;
  const int64_t blocks = static_cast<int64_t>(batch) * plan.n_hb * plan.n_parts;
  if (blocks > 0x7FFFFFFF) return MLA_LOWBIT_ERR_UNSUPPORTED;
  const size_t lds = static_cast<size_t>(kDecodeWaves) * kWaveLds;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess)
      return MLA_LOWBIT_ERR_HIP;
    attr_set = true;
  }
  if (g.latent_bits == 4)
    hipLaunchKernelGGL(decode_kernel<4>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<2>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), lds, stream, p);
  if (hipGetLastError() != hipSuccess) return MLA_LOWBIT_ERR_HIP;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<uint32_t>(batch * heads)), dim3(128), 0, stream,
                     p.ws, out, lse, heads, plan.n_hb, plan.n_parts);
  return hipGetLastError() == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ERR_HIP;
}
