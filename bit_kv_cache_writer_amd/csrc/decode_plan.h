// Work split of the decode (internal; shared by the workspace query and the
// launch so that both always agree).
#pragma once
#include <cstddef>
#include <cstdint>

#include "geometry.h"

namespace mla {

constexpr int kTile = 16;         // tokens per wave and round (the MFMA M dimension)
constexpr int kHeadBlock = 16;    // heads per MFMA block
constexpr int kDecodeWaves = 4;   // waves per workgroup (one per SIMD)
constexpr int kPartFloats = kHeadBlock * kLatentDim + 2 * kHeadBlock;  // O, m, l
constexpr int kTargetGroups = 512;  // two workgroups per CU of an MI355X
constexpr int kDenseCost = 2;       // a BF16 tile costs about two packed tiles
constexpr int kMaxSplits = 128;     // splits per (sequence, head block): the merge stages their (max, sum)

struct DecodePlan {
  int n_hb;        // head blocks of 16
  int n_splits;    // workgroups per (sequence, head block)
  size_t workspace_bytes;
};

inline DecodePlan plan_decode(const Geometry& g, int batch, int heads, int max_seqlen) {
  (void)g;
  DecodePlan p;
  p.n_hb = (heads + kHeadBlock - 1) / kHeadBlock;
  const long groups = static_cast<long>(batch > 0 ? batch : 1) * p.n_hb;
  // Cost bound of one sequence: every token in a packed tile, plus the BF16
  // tiles' extra cost.
  const long tiles = (max_seqlen + kTile - 1) / kTile + 2;
  long s = (kTargetGroups + groups - 1) / groups;
  long cap = tiles / (2L * kDecodeWaves);  // >= 2 tiles per wave
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  p.n_splits = static_cast<int>(s);
  p.workspace_bytes = 0;
  if (p.n_splits > 1)
    p.workspace_bytes = static_cast<size_t>(groups) * p.n_splits * kPartFloats * sizeof(float);
  return p;
}

}  // namespace mla
