// Validated cache geometry shared by the host side of the writer and the
// decode (internal; not part of the C ABI).
#pragma once
#include <cstddef>
#include <cstdint>

#include "mla_lowbit.h"

namespace mla {

constexpr int kLatentDim = 512;
constexpr int kRopeDim = 64;
constexpr int kGroup = 128;
constexpr int kGroups = kLatentDim / kGroup;
constexpr int kRowElems = kLatentDim + kRopeDim;  // BF16 side-buffer row
constexpr int kRopeRowBytes = kRopeDim * 4 / 8;   // 32
constexpr int kMaxHeads = 128;
constexpr int kMaxSink = 64;
constexpr int kMaxLocal = 4096;

struct Geometry {
  int page_size;
  int latent_bits;
  int sink, local;
  bool clip;
  int clip_lo, clip_hi;  // order-statistic ranks of |x| for the clip value
  float clip_frac;       // interpolation weight between them
  int64_t latent_row;    // bytes
  int64_t latent_meta_off, rope_codes_off, rope_meta_off, page_bytes;
};

// Returns MLA_LOWBIT_OK and fills *g, or MLA_LOWBIT_ERR_LAYOUT.
int make_geometry(const mla_lowbit_layout* layout, Geometry* g);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace mla
