// Work split of the decode (internal; shared by the workspace query and the
// launch so that both always agree).
#pragma once
#include <cstddef>
#include <algorithm>
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
constexpr int kMaxSplits = 512;     // workgroups per (sequence, head block)
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
  const long packed_tiles = (max_seqlen + kTile - 1) / kTile + 1;
  long cap = packed_tiles / (2L * kDecodeWaves);  // >= 2 tiles per wave
  if (cap < 1) cap = 1;
  // pages a packed workgroup spans must fit its LDS window of page ids
  auto pages_spanned = [&](long n_ps) {
    const long tiles = (packed_tiles + n_ps - 1) / n_ps;
    return (tiles * kTile + g.page_size - 1) / g.page_size + 1;
  };
  auto ceil_div = [](long a, long b) { return (a + b - 1) / b; };
  // packed tiles of a sequence of max_seqlen tokens (as the kernel splits
  // them) and its BF16-path tiles: the estimate the split is chosen for (a
  // shorter sequence may have up to dense_tiles BF16-path tiles; its BF16-path
  // workgroups then take more rounds, with the same results)
  long t_count = 0, dense_est = 0;
  {
    const long lo = std::min<long>(g.sink, max_seqlen);
    const long hi = std::max<long>(lo, std::min<long>(static_cast<long>(max_seqlen) - g.local,
                                                      (max_seqlen / g.page_size) * static_cast<long>(g.page_size)));
    if (hi > lo) t_count = ceil_div(hi, kTile) - lo / kTile;
    dense_est = ceil_div(lo + (max_seqlen - hi), kTile);
  }
  // BF16-path and packed workgroups of a (sequence, head block) share the
  // groups' slots of two workgroups per CU; the count of BF16-path ones is
  // chosen to minimize the longer of the two kinds of workgroup, a BF16-path
  // round (latency-bound row loads) costing about two packed rounds.
  const long slots = (kTargetGroups + groups - 1) / groups;
  long best_cost = -1, best_nd = 0, best_s = 1;
  // (no BF16-path workgroup when no token can need one: max_seqlen = 0)
  for (long nd = dense_tiles > 0 ? 1 : 0; nd <= dense_tiles && nd <= kMaxSplits - 1; ++nd) {
    long s = slots - nd;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    while (pages_spanned(s) > kPageWin && s + nd < kMaxSplits) ++s;
    if (s + nd > kMaxSplits) s = kMaxSplits - nd;
    if (s < 1) continue;
    const long dense_rounds = nd > 0 ? ceil_div(ceil_div(dense_est, nd), kDecodeWaves) : 0;
    const long packed_rounds = ceil_div(ceil_div(t_count, s), kDecodeWaves);
    const long cost = std::max(2 * dense_rounds, packed_rounds);
    // ties: fewer partials to merge, then fewer BF16-path rounds
    if (best_cost < 0 || cost < best_cost ||
        (cost == best_cost && (s + nd < best_s + best_nd || (s + nd == best_s + best_nd && nd > best_nd)))) {
      best_cost = cost;
      best_nd = nd;
      best_s = s;
    }
  }
  p.n_dense = static_cast<int>(best_nd);
  p.ok = pages_spanned(best_s) <= kPageWin;
  p.n_splits = p.n_dense + static_cast<int>(best_s);
  p.workspace_bytes = 0;
  if (p.n_splits > 1)
    p.workspace_bytes = static_cast<size_t>(groups) * p.n_splits * kPartBytes;
  return p;
}

}  // namespace mla
