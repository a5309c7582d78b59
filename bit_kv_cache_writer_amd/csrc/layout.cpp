// Host side of the C ABI: layout validation, byte geometry, workspace sizing
// and error strings.  The page layout reads RAQ-MLA appendix Table 5 (bits,
// grouping and FP16 metadata per path) into bytes; see mla_lowbit.h.
#include <cmath>

#include "geometry.h"
#include "decode_plan.h"

namespace mla {

int make_geometry(const mla_lowbit_layout* L, Geometry* g) {
  if (!L || !g) return MLA_LOWBIT_ERR_ARG;
  if (L->version != MLA_LOWBIT_LAYOUT_VERSION || L->reserved != 0) return MLA_LOWBIT_ERR_LAYOUT;
  if (L->latent_dim != kLatentDim || L->rope_dim != kRopeDim || L->latent_group != kGroup ||
      L->rope_bits != 4)
    return MLA_LOWBIT_ERR_LAYOUT;
  if (L->latent_bits != 2 && L->latent_bits != 4) return MLA_LOWBIT_ERR_LAYOUT;
  const int P = L->page_size;
  if (P != 32 && P != 64 && P != 128 && P != 256) return MLA_LOWBIT_ERR_LAYOUT;
  if (L->sink < 0 || L->sink > kMaxSink || L->local < 0 || L->local > kMaxLocal)
    return MLA_LOWBIT_ERR_LAYOUT;
  const double q = L->latent_clip_q;
  if (!(q >= 0.0 && q <= 1.0)) return MLA_LOWBIT_ERR_LAYOUT;  // also rejects NaN
  g->page_size = P;
  g->latent_bits = L->latent_bits;
  g->sink = L->sink;
  g->local = L->local;
  g->clip = q > 0.0;
  // Quantile of n = 512 order statistics with linear interpolation:
  // position h = (n - 1) q, ranks floor(h) and floor(h) + 1, weight h - floor(h).
  const double h = (kLatentDim - 1) * q;
  int lo = static_cast<int>(std::floor(h));
  if (lo > kLatentDim - 1) lo = kLatentDim - 1;
  g->clip_lo = lo;
  g->clip_hi = lo + 1 < kLatentDim ? lo + 1 : kLatentDim - 1;
  g->clip_frac = static_cast<float>(h - lo);
  g->latent_row = static_cast<int64_t>(kLatentDim) * L->latent_bits / 8;
  g->latent_meta_off = g->latent_row * P;
  g->rope_codes_off = g->latent_meta_off + static_cast<int64_t>(P) * kGroups * 4;
  g->rope_meta_off = g->rope_codes_off + static_cast<int64_t>(P) * kRopeRowBytes;
  g->page_bytes = g->rope_meta_off + kRopeDim * 4;
  return MLA_LOWBIT_OK;
}

}  // namespace mla

extern "C" int mla_lowbit_layout_query(const mla_lowbit_layout* layout, mla_lowbit_sizes* s) {
  if (!layout || !s) return MLA_LOWBIT_ERR_ARG;
  mla::Geometry g;
  int rc = mla::make_geometry(layout, &g);
  if (rc) return rc;
  s->page_bytes = g.page_bytes;
  s->latent_row_bytes = g.latent_row;
  s->latent_meta_offset = g.latent_meta_off;
  s->rope_codes_offset = g.rope_codes_off;
  s->rope_row_bytes = mla::kRopeRowBytes;
  s->rope_meta_offset = g.rope_meta_off;
  s->bf16_row_bytes = mla::kRowElems * 2;
  s->sink_bytes_per_seq = static_cast<uint64_t>(g.sink) * mla::kRowElems * 2;
  s->ring_bytes_per_seq = static_cast<uint64_t>(g.local) * mla::kRowElems * 2;
  s->tail_bytes_per_seq = static_cast<uint64_t>(g.page_size) * mla::kRopeDim * 2;
  return MLA_LOWBIT_OK;
}

extern "C" int mla_lowbit_decode_workspace(const mla_lowbit_layout* layout, int32_t batch,
                                           int32_t heads, int32_t max_seqlen, size_t* bytes) {
  if (!layout || !bytes) return MLA_LOWBIT_ERR_ARG;
  mla::Geometry g;
  int rc = mla::make_geometry(layout, &g);
  if (rc) return rc;
  if (batch < 0 || heads < 1 || heads > mla::kMaxHeads || max_seqlen < 0) return MLA_LOWBIT_ERR_ARG;
  mla::DecodePlan plan = mla::plan_decode(g, batch, heads, max_seqlen);
  if (!plan.ok) return MLA_LOWBIT_ERR_UNSUPPORTED;
  *bytes = plan.workspace_bytes;
  return MLA_LOWBIT_OK;
}

extern "C" const char* mla_lowbit_strerror(int code) {
  switch (code) {
    case MLA_LOWBIT_OK: return "ok";
    case MLA_LOWBIT_ERR_LAYOUT: return "invalid or unsupported cache-layout descriptor";
    case MLA_LOWBIT_ERR_ARG: return "invalid argument (null or misaligned pointer, or bad size)";
    case MLA_LOWBIT_ERR_UNSUPPORTED: return "valid request the library does not run";
    case MLA_LOWBIT_ERR_WORKSPACE: return "workspace smaller than mla_lowbit_decode_workspace()";
    case MLA_LOWBIT_ERR_HIP: return "HIP kernel launch failed";
    case MLA_LOWBIT_ERR_SCRATCH:
      return "shape needs more split-partial memory than MLA_LOWBIT_NOALLOC_SCRATCH_BYTES (use mla_lowbit_decode)";
    default: return "unknown error code";
  }
}
