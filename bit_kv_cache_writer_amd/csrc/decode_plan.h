// Work split of the decode (internal; shared by the workspace query and the
// launch so that both always agree).
#pragma once
#include <cstddef>
#include <cstdint>

#include "geometry.h"

namespace mla {

constexpr int kTile = 32;         // tokens per MFMA tile
constexpr int kHeadBlock = 16;    // heads per MFMA M/N block
constexpr int kDecodeWaves = 4;   // waves per workgroup, one tile each at a time
constexpr int kPartFloats = kHeadBlock * kLatentDim + 2 * kHeadBlock;  // O, m, l

struct DecodePlan {
  int n_hb;        // head blocks of 16
  int n_splits;    // packed-token splits per (sequence, head block); +1 BF16 part
  int n_parts;     // n_splits + 1
  size_t workspace_bytes;
};

inline DecodePlan plan_decode(const Geometry& g, int batch, int heads, int max_seqlen) {
  (void)g;
  DecodePlan p;
  p.n_hb = (heads + kHeadBlock - 1) / kHeadBlock;
  const int tiles = (max_seqlen + kTile - 1) / kTile + 1;
  // Enough workgroups to cover 256 CUs twice, but every split keeps at least
  // 2 tiles per wave so the partial (16 x 512 fp32) stays small next to the
  // cache bytes it summarizes.
  const int min_tiles = 2 * kDecodeWaves;
  const long groups = static_cast<long>(batch > 0 ? batch : 1) * p.n_hb;
  int s = static_cast<int>((512 + groups - 1) / groups);
  int cap = tiles / min_tiles;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  p.n_splits = s;
  p.n_parts = s + 1;
  p.workspace_bytes = static_cast<size_t>(batch) * p.n_parts * p.n_hb * kPartFloats * sizeof(float);
  return p;
}

}  // namespace mla
