// Work split of the decode (internal; shared by the workspace query and the
// launch so that both always agree).
#pragma once
#include <cstddef>
#include <cstdint>

#include "geometry.h"

namespace mla {

constexpr int kTile = 16;          // tokens per wave and round (the MFMA M dimension)
constexpr int kHeadBlock = 16;     // heads per MFMA block
constexpr int kDecodeWaves = 4;    // waves per workgroup (one per SIMD)
// A split's partial: O / l as fp16 [16 heads][512], then fp32 m[16], l[16].
constexpr int kPartRowBytes = kHeadBlock * kLatentDim * 2;
constexpr int kPartBytes = kPartRowBytes + 2 * kHeadBlock * 4;
constexpr int kTargetGroups = 512;  // two workgroups per CU of an MI355X
constexpr int kDenseTilesPerWg = 8;  // BF16-path tiles per workgroup (two rounds)
constexpr int kMaxSplits = 128;     // workgroups per (sequence, head block)
constexpr int kPageWin = 512;       // page ids a packed workgroup stages in LDS

// Every (sequence, head block) gets n_dense BF16-path workgroups (sink,
// recent window and unfinished-page tokens, bounded by sink + local + P - 1)
// and n_splits - n_dense packed-page workgroups.
struct DecodePlan {
  bool ok;         // false: max_seqlen needs more pages per workgroup than kPageWin
  int n_hb;        // head blocks of 16
  int n_dense;     // BF16-path workgroups per (sequence, head block)
  int n_splits;    // workgroups per (sequence, head block)
  size_t workspace_bytes;
};

inline DecodePlan plan_decode(const Geometry& g, int batch, int heads, int max_seqlen) {
  DecodePlan p;
  p.n_hb = (heads + kHeadBlock - 1) / kHeadBlock;
  const long groups = static_cast<long>(batch > 0 ? batch : 1) * p.n_hb;
  long dense_tokens = static_cast<long>(g.sink) + g.local + g.page_size - 1;
  if (dense_tokens > max_seqlen) dense_tokens = max_seqlen;
  const long dense_tiles = (dense_tokens + kTile - 1) / kTile;
  p.n_dense = static_cast<int>((dense_tiles + kDenseTilesPerWg - 1) / kDenseTilesPerWg);
  const long packed_tiles = (max_seqlen + kTile - 1) / kTile + 1;
  long s = (kTargetGroups + groups - 1) / groups - p.n_dense;
  long cap = packed_tiles / (2L * kDecodeWaves);  // >= 2 tiles per wave
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  // pages a packed workgroup spans must fit its LDS window of page ids
  auto pages_spanned = [&](long n_ps) {
    const long tiles = (packed_tiles + n_ps - 1) / n_ps;
    return (tiles * kTile + g.page_size - 1) / g.page_size + 1;
  };
  while (pages_spanned(s) > kPageWin && s + p.n_dense < kMaxSplits) ++s;
  if (s + p.n_dense > kMaxSplits) s = kMaxSplits - p.n_dense;
  p.ok = pages_spanned(s) <= kPageWin;
  p.n_splits = p.n_dense + static_cast<int>(s);
  p.workspace_bytes = 0;
  if (p.n_splits > 1)
    p.workspace_bytes = static_cast<size_t>(groups) * p.n_splits * kPartBytes;
  return p;
}

}  // namespace mla
