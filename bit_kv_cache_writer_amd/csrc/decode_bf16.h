// The plain BF16 paged cache (declared in mla_bf16.h; included by decode.hip,
// whose helpers and split merge it uses): an append kernel and a split-KV
// decode, the baseline the low-bit cache is measured against (QuantMLA,
// Table 9 caption: BF16 attention with native partitioning).
//
// Decode.  A workgroup of four waves serves 16 heads of one (sequence,
// split); its 16-token tiles (16 rows of 1152 bytes, always inside one page)
// go into a four-slot LDS ring by direct global->LDS loads, three tiles
// ahead.  Wave w owns the channel quarter w: latent channels 128 w .. +127
// and positional channels 16 w .. +15.
//   scores  D[token][head] over the quarter on the bf16 matrix cores (rows
//           as the A operand straight from LDS, the query as B from
//           registers: 16x16x32 for the latent, 16x16x16 for the positional
//           part); the four waves add their partials through LDS in a fixed
//           order, so all hold identical scores;
//   softmax online, base 2, the reference max moving only by more than 2^8
//           (as the packed-cache kernels);
//   output  O[head][channel] += P V for the wave's 128 channels: P from the
//           score registers (their layout is the A operand's), as bf16 high
//           and low parts (two products, so the weights keep 16 bits), V
//           read transposed from the same LDS rows with ds_read_b64_tr_b16.
// Split partials (O / l in fp16, max, sum) are merged by the packed cache's
// merge kernel.

namespace bf16c {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 16;                       // tokens per tile
constexpr int kRowBytes = 1152;              // (c_KV 512, k_R 64) bf16
constexpr int kRowUnits = kRowBytes / 16;    // 16-byte units per row
constexpr int kSlotBytes = kT * kRowBytes;   // 18432
constexpr int kLoads = kSlotBytes / 1024;    // direct loads of 64 x 16 B per tile
constexpr int kSlots = 4;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPageWin = 512;                // page ids a workgroup stages
constexpr int kOffXch = kSlots * kSlotBytes;  // partial scores [wave][lane] f32x4
constexpr int kOffPid = kOffXch + kWaves * 64 * 16;
constexpr int kLdsBytes = kOffPid + kPageWin * 4;
constexpr int kTargetWgs = 512;              // two workgroups per CU
constexpr int kMinTiles = 4;                 // tiles per split at least
constexpr int kMaxSplitsB = kMaxSplits;      // the merge's limit
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU");
static_assert(kSlotBytes % 1024 == 0, "a tile is whole direct loads");

// Work split: enough workgroups for two per CU, each with at least kMinTiles
// tiles and at most kPageWin - 1 pages.
struct Plan {
  bool ok;
  int n_hb, n_splits, per;  // head blocks, splits per (sequence, head block), tiles per split
  size_t workspace_bytes;
};

inline Plan plan(int page_size, int batch, int heads, int max_seqlen) {
  Plan p{};
  auto ceil_div = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  p.n_hb = static_cast<int>(ceil_div(heads, kHeadBlock));
  const int64_t groups = static_cast<int64_t>(batch > 0 ? batch : 1) * p.n_hb;
  const int64_t tiles = ceil_div(max_seqlen, kT);
  int64_t s = std::max<int64_t>(1, std::min(ceil_div(kTargetWgs, groups), ceil_div(tiles, kMinTiles)));
  const int64_t max_tiles = static_cast<int64_t>(kPageWin - 2) * page_size / kT;  // keeps pages <= kPageWin - 1
  if (tiles > 0) s = std::max(s, ceil_div(tiles, max_tiles));
  s = std::min<int64_t>(s, kMaxSplitsB);
  p.n_splits = static_cast<int>(s);
  p.per = static_cast<int>(std::max<int64_t>(1, ceil_div(tiles, s)));
  p.ok = p.per <= max_tiles;
  p.workspace_bytes = p.n_splits > 1 ? static_cast<size_t>(groups) * p.n_splits * kPartBytes : 0;
  return p;
}

struct Params {
  const uint16_t* q_lat;
  const uint16_t* q_rope;
  const uint8_t* pool;
  const int32_t* block_table;
  const int32_t* seqlens;
  uint8_t* parts;
  float* out;
  float* lse;
  int32_t batch, heads, max_pages, num_pool_pages, n_hb, n_splits, per, log2P;
  int64_t page_bytes;
  float c_log2;
};

// Unit u of token row r of a tile sits at position u ^ swz(r) of the row
// (inside its aligned group of 8 units): the 16 rows of one score read and
// the 4 rows x 2 units of one transposed read fall on distinct bank groups.
__device__ constexpr int swz(int r) { return (r >> 1) & 7; }
__device__ constexpr int unit_at(int r, int u) { return r * kRowUnits + (u ^ swz(r)); }

// Wait until at most n of this wave's vector-memory operations are in flight.
__device__ inline void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
  }
}

__device__ inline f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ inline f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}

// bf16 of an fp32 value, rounded to nearest even (finite inputs).
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ void __launch_bounds__(kThreads, 2) decode_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // block i -> (sequence, split, head block), XCD-major as the packed-cache
  // kernel: the head blocks of a split run side by side on one XCD and share
  // its L2
  const int n_blocks = gridDim.x, xcd = blockIdx.x & 7, per_xcd = n_blocks >> 3, extra = n_blocks & 7;
  const int item = xcd * per_xcd + min(xcd, extra) + (blockIdx.x >> 3);
  const int hb = item % p.n_hb, split = (item / p.n_hb) % p.n_splits, b = item / (p.n_hb * p.n_splits);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int n16 = lane & 15, gq = lane >> 4;
  uint8_t* const ring = smem;
  f32x4* const xch = reinterpret_cast<f32x4*>(smem + kOffXch);
  int* const s_pid = reinterpret_cast<int*>(smem + kOffPid);

  const int L = uniform(p.seqlens[b]);
  const int tiles = (L + kT - 1) / kT;
  const int k0 = min(tiles, split * p.per), k1 = min(tiles, k0 + p.per);
  const int n = p.max_pages > 0 ? max(0, k1 - k0) : 0;  // (no page table: nothing to read)
  const int P = 1 << p.log2P;

  // query operands of this wave's quarter (heads past the last read a copy of
  // the last): B of the latent products (channels 128 w + 32 s + 8 gq .. + 7
  // of head n16) and of the positional one (channels 16 w + 4 gq .. + 3)
  const int hq = min(hb * kHeadBlock + n16, p.heads - 1);
  u32x4 qv[4];
  {
    const uint16_t* ql = p.q_lat + (static_cast<int64_t>(b) * p.heads + hq) * kLatentDim + 128 * wave + 8 * gq;
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[s] = ldg<u32x4>(ql + 32 * s);
  }
  const u32x2 qr = ldg<u32x2>(p.q_rope + (static_cast<int64_t>(b) * p.heads + hq) * kRopeDim + 16 * wave + 4 * gq);

  // page ids of the split's tiles into LDS
  const int pg_first = (k0 * kT) >> p.log2P;
  const int n_pg = n > 0 ? (((k1 * kT - 1) >> p.log2P) - pg_first + 1) : 0;
  const int32_t* const bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  for (int i = wave; i * 64 < n_pg; i += kWaves)
    load4_to_lds(bt + max(0, min(pg_first + min(64 * i + lane, n_pg - 1), p.max_pages - 1)),
                 reinterpret_cast<uint8_t*>(s_pid) + 4 * 64 * i);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  auto page_id = [&](int k) { return uniform(s_pid[(((k0 + k) * kT) >> p.log2P) - pg_first]); };
  auto page_ok = [&](int id) { return id >= 0 && id < p.num_pool_pages; };
  // direct loads of tile k: load i (of kLoads) by wave i % 4, lane l to LDS
  // unit 64 i + l of the slot (the swizzle's inverse picks its source)
  auto issue = [&](int k) {
    const int id = page_id(k);
    const uint8_t* const base =
        page_ok(id) ? p.pool + id * p.page_bytes + static_cast<int64_t>(((k0 + k) * kT) & (P - 1)) * kRowBytes
                    : p.pool;  // a missing page: any valid rows (the tile is masked)
    uint8_t* const slot = ring + (k % kSlots) * kSlotBytes;
#pragma unroll
    for (int i = wave; i < kLoads; i += kWaves) {
      const int U = 64 * i + lane, r = U / kRowUnits, u = (U % kRowUnits) ^ swz(r);
      load_to_lds(base + r * kRowBytes + 16 * u, slot + 1024 * i);
    }
  };
  const int my_loads = (kLoads - wave + kWaves - 1) / kWaves;
#pragma unroll
  for (int k = 0; k < kSlots - 1; ++k)
    if (k < n) issue(k);

  f32x4 o[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) o[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, lsum = 0.f;
  // transposed reads: lane j of row group gq points at token 4 gq + j / 4,
  // channels 4 (j % 4) .. + 3 of each 16-channel block, so that lane i gets
  // channel i of tokens 4 gq .. 4 gq + 3 (the B operand of the output)
  const int tr_tok = 4 * gq + (n16 >> 2);
  const int tr_unit = 16 * wave + ((n16 & 3) >> 1), tr_half = 8 * (n16 & 1);

  for (int k = 0; k < n; ++k) {
    // tile k has landed once this wave's loads of it are done and every wave
    // has passed the barrier; every wave is then also done with tile k - 1
    // (its slot and the exchange)
    wait_vm(min(n - 1 - k, kSlots - 2) * my_loads);
    lds_barrier();
    if (k + kSlots - 1 < n) issue(k + kSlots - 1);
    const uint8_t* const slot = ring + (k % kSlots) * kSlotBytes;
    // this wave's partial scores: token 4 gq + r, head n16 (the two MFMA
    // shapes accumulate apart: one never reads the other's result as its
    // accumulator input)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = mfma_k32(lds_ld<u32x4>(slot + 16 * unit_at(n16, 16 * wave + 4 * s + gq)), qv[s], acc);
    const f32x4 acc_r = mfma_k16(lds_ld<u32x2>(slot + 16 * unit_at(n16, 64 + 2 * wave + (gq >> 1)) + 8 * (gq & 1)),
                                 qr, f32x4{0.f, 0.f, 0.f, 0.f});
    xch[wave * 64 + lane] = acc + acc_r;
    lds_barrier();
    f32x4 sc = xch[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sc += xch[w * 64 + lane];
    const bool ok = page_ok(page_id(k));
    float t[4], tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = (k0 + k) * kT + 4 * gq + r;
      t[r] = ok && tok < L ? sc[r] * p.c_log2 : kNegInf;
      tmax = fmaxf(tmax, t[r]);
    }
    tmax = row_allmax(tmax);  // head n16 over the tile's 16 tokens
    const float m_new = tmax > m_run + kMaxSlack ? tmax : m_run;
    if (__any(m_new != m_run)) {  // rescale the output rows of the raised heads
      const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - m_new);
      lsum *= alpha;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * gq + r);  // output row r is head 4 gq + r
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[kk][r] *= ar[r];
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(t[r] - m_use);  // a masked token gives 0
      lsum += pr[r];
    }
    // weights as bf16 high + low: A[head n16][token 4 gq + e] is this lane's pr[e]
    u32x2 ph, pl;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t h0 = bf16_rne(pr[2 * e]), h1 = bf16_rne(pr[2 * e + 1]);
      ph[e] = h0 | (h1 << 16);
      pl[e] = bf16_rne(pr[2 * e] - __uint_as_float(h0 << 16)) | (bf16_rne(pr[2 * e + 1] - __uint_as_float(h1 << 16)) << 16);
    }
    // the wave's 8 blocks of 16 channels, transposed, in one block of reads
    // (a load written in asm is waited for inside it)
    uint32_t addr[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) addr[kk] = lds_addr(slot + 16 * unit_at(tr_tok, tr_unit + 2 * kk) + tr_half);
    i32x2 v[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
          "v"(addr[7])
        : "memory");
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x2 vb = __builtin_bit_cast(u32x2, v[kk]);
      o[kk] = mfma_k16(ph, vb, o[kk]);
      o[kk] = mfma_k16(pl, vb, o[kk]);
    }
  }

  // finish: output row r of this lane is head 4 gq + r, channel
  // 128 w + 16 kk + n16
  const float l_h = row_allsum(lsum);  // head n16
  float lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lr[r] = __shfl(l_h, 4 * gq + r);
  const bool direct = p.n_splits == 1;
  uint8_t* const part =
      p.parts + (static_cast<int64_t>(b * p.n_hb + hb) * p.n_splits + split) * kPartBytes;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int ch = 128 * wave + 16 * kk + n16;
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = lr[r] > 0.f ? o[kk][r] / lr[r] : 0.f;
    if (direct) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = hb * kHeadBlock + 4 * gq + r;
        if (h < p.heads) p.out[(static_cast<int64_t>(b) * p.heads + h) * kLatentDim + ch] = y[r];
      }
    } else {
      const half4 hv = {static_cast<_Float16>(y[0]), static_cast<_Float16>(y[1]), static_cast<_Float16>(y[2]),
                        static_cast<_Float16>(y[3])};
      *reinterpret_cast<half4*>(part + 2 * (ch * kHeadBlock + 4 * gq)) = hv;
    }
  }
  if (wave == 0 && gq == 0) {
    const int h = hb * kHeadBlock + n16;
    if (direct) {
      if (h < p.heads)
        p.lse[static_cast<int64_t>(b) * p.heads + h] =
            l_h > 0.f ? (m_run + log2f(l_h)) * 0.69314718055994531f : kNegInf;
    } else {
      float* const ml = reinterpret_cast<float*>(part + kPartRowBytes);
      ml[n16] = m_run;
      ml[kHeadBlock + n16] = l_h;
    }
  }
}

// One wave per new token: its 576-value row into the pool.
__global__ void __launch_bounds__(256) append_kernel(const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_r,
                                                     const int32_t* __restrict__ cu_new,
                                                     const int32_t* __restrict__ seqlens_before, int log2P,
                                                     const int32_t* __restrict__ block_table, int max_pages,
                                                     int num_pool_pages, uint16_t* __restrict__ pool) {
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = cu_new[b];
  if (i >= cu_new[b + 1] - n0) return;
  const int j = seqlens_before[b] + i;
  const int pidx = j >> log2P;
  if (j < 0 || pidx >= max_pages) return;
  const int id = block_table[static_cast<int64_t>(b) * max_pages + pidx];
  if (id < 0 || id >= num_pool_pages) return;
  uint16_t* const dst = pool + (static_cast<int64_t>(id) * (1 << log2P) + (j & ((1 << log2P) - 1))) * 576;
  const int64_t row = static_cast<int64_t>(n0) + i;
  reinterpret_cast<u32x4*>(dst)[lane] = ldg<u32x4>(c_kv + row * kLatentDim + 8 * lane);
  if (lane < 8) reinterpret_cast<u32x4*>(dst + kLatentDim)[lane] = ldg<u32x4>(k_r + row * kRopeDim + 8 * lane);
}

}  // namespace bf16c
