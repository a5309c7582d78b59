/*
 * mla_lowbit.h -- C ABI of the MI355X (gfx950) dual-path low-bit MLA cache:
 * a fused cache writer and a decode-attention kernel over the packed cache.
 *
 * The method (QuantMLA page, Figure 8 caption; RAQ-MLA page, appendix
 * Table 5): every incoming token's compressed latent c_KV (512 channels) and
 * post-RoPE positional key k_R (64 channels) are stored as low-bit codes with
 * asymmetric FP16 scale/minimum metadata -- the latent per token in groups of
 * 128 channels (2- or 4-bit), k_R per channel within a cache page (4-bit).
 * Protected sink tokens and the recent window are also kept in BF16 and are
 * attended from BF16.  Decode uses absorbed queries (RAQ-MLA abstract and
 * Figure 4 caption): per head, score = q_lat . c_KV + q_rope . k_R, one
 * softmax over every valid token, output = sum_j p_j c_KV_j in latent space.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronizes, and keeps no state between
 *     calls.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and runs asynchronously: a device-side fault surfaces at the
 *     caller's next synchronization.
 *   - bf16 tensors are raw 16-bit patterns, row-major, densely packed.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and returned as a negative MLA_LOWBIT_ERR_* code; nothing is launched
 *     then.
 *   - Device-side indices (block-table entries, positions, lengths) that fall
 *     outside the sizes passed on the host are skipped/clamped by the kernels,
 *     never dereferenced; results for such sequences are unspecified.
 */
#ifndef MLA_LOWBIT_H
#define MLA_LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_LOWBIT_LAYOUT_VERSION 1

/* Error codes. */
#define MLA_LOWBIT_OK 0
#define MLA_LOWBIT_ERR_LAYOUT (-1)      /* invalid or unsupported layout descriptor */
#define MLA_LOWBIT_ERR_ARG (-2)         /* null / misaligned pointer, bad size */
#define MLA_LOWBIT_ERR_UNSUPPORTED (-3) /* valid request the library does not run */
#define MLA_LOWBIT_ERR_WORKSPACE (-4)   /* workspace smaller than required */
#define MLA_LOWBIT_ERR_HIP (-5)         /* a HIP launch failed */
#define MLA_LOWBIT_ERR_SCRATCH (-6)     /* shape needs more than the fixed no-allocation scratch */

/*
 * Cache-layout descriptor (RAQ-MLA appendix Table 5: bits, grouping,
 * clipping and metadata per path; appendix Table 6: page size per model;
 * QuantMLA Figure 5 caption: sink/local protection).
 */
typedef struct mla_lowbit_layout {
  int32_t version;      /* MLA_LOWBIT_LAYOUT_VERSION */
  int32_t latent_dim;   /* c_KV channels; must be 512 */
  int32_t rope_dim;     /* k_R channels; must be 64 */
  int32_t page_size;    /* P tokens per cache page: 32, 64, 128 or 256 */
  int32_t latent_bits;  /* 2 or 4 */
  int32_t rope_bits;    /* must be 4 */
  int32_t latent_group; /* channels per latent scale/min group; must be 128 */
  int32_t sink;         /* leading tokens kept in BF16: 0..64 */
  int32_t local;        /* most recent tokens kept in BF16: 0..4096 */
  int32_t reserved;     /* must be 0 */
  double latent_clip_q; /* 0: no clipping; in (0, 1]: clip each latent token
                           to +-(the q-quantile of its |x|, linear
                           interpolation between order statistics) */
} mla_lowbit_layout;

/*
 * Byte geometry of the layout.  A cache page of P tokens is
 *   [latent codes : P rows x latent_row_bytes]   row t = token slot t
 *   [latent meta  : P rows x 4 groups x (fp16 scale, fp16 min)]
 *   [rope codes   : P rows x rope_row_bytes]
 *   [rope meta    : 64 fp16 scales, then 64 fp16 minimums]
 * In a code row, channel c occupies bits [(c*b) % 8, +b) of byte (c*b)/8.
 * Per sequence the BF16 side buffers are
 *   sink : [sink ][576] bf16  (row = [c_KV 512 | k_R 64] of token t < sink)
 *   ring : [local][576] bf16  (slot t % local holds token t of the window)
 *   tail : [P    ][64]  bf16  (k_R of the tokens of the page being filled;
 *                              a page's k_R codes exist once it is full)
 */
typedef struct mla_lowbit_sizes {
  uint64_t page_bytes;
  uint64_t latent_row_bytes;
  uint64_t latent_meta_offset;
  uint64_t rope_codes_offset;
  uint64_t rope_row_bytes;
  uint64_t rope_meta_offset;
  uint64_t bf16_row_bytes;     /* 1152 */
  uint64_t sink_bytes_per_seq; /* sink * 1152 */
  uint64_t ring_bytes_per_seq; /* local * 1152 */
  uint64_t tail_bytes_per_seq; /* P * 128 */
} mla_lowbit_sizes;

/* Validate `layout` and fill `sizes`.  Host only. */
int mla_lowbit_layout_query(const mla_lowbit_layout* layout, mla_lowbit_sizes* sizes);

/*
 * Fused cache writer (QuantMLA Figure 8 caption; RAQ-MLA appendix Table 5).
 * Appends new tokens: the rows cu_new[b] .. cu_new[b+1]-1 of c_kv / k_r are
 * sequence b's tokens at positions seqlens_before[b] + i.  For each token:
 *   - the latent is clipped (if latent_clip_q > 0), quantized per group of
 *     128 with FP16 (scale, min), packed into page block_table[b][t / P],
 *     slot t % P;
 *   - its BF16 row is stored in sink[b][t] if t < sink and in ring slot
 *     t % local if it is among the last `local` positions written by the call;
 *   - its k_R goes to the tail buffer while its page is incomplete; when the
 *     page becomes full its k_R is quantized per channel over the page
 *     (FP16 scale/min per channel and page) and packed.
 * Codes, metadata and the BF16 copies equal, bit for bit, those of appending
 * the same tokens one at a time.  `seqlens_before` is not modified.
 * Inputs must be finite bf16 with |x| <= 65280 (the largest bf16 below the
 * fp16 limit), as mla_lowbit_decode also requires.  The FP16 minimum is
 * rounded toward -inf and the scale toward +inf; within that range every
 * code falls in [0, levels] without a clamp, and the codes are not clamped
 * (values beyond it give codes that differ from a clamped quantizer's).
 *
 *   c_kv           bf16 [total_new][512], 16-B aligned
 *   k_r            bf16 [total_new][64],  16-B aligned
 *   cu_new         int32 [batch+1], cu_new[0] = 0, non-decreasing, last = total_new
 *   seqlens_before int32 [batch], tokens already written per sequence
 *   max_new_per_seq host bound on cu_new[b+1]-cu_new[b] (grid sizing)
 *   block_table    int32 [batch][max_pages] page ids in [0, num_pool_pages)
 *   page_pool      [num_pool_pages][page_bytes], 16-B aligned
 *   sink_buf / ring_buf / rope_tail  per-sequence BF16 buffers (may be NULL
 *                  when sink / local is 0; rope_tail is required)
 */
int mla_lowbit_write(const mla_lowbit_layout* layout, const void* c_kv, const void* k_r,
                     const int32_t* cu_new, const int32_t* seqlens_before, int32_t batch,
                     int32_t total_new, int32_t max_new_per_seq, const int32_t* block_table,
                     int32_t max_pages, int32_t num_pool_pages, void* page_pool, void* sink_buf,
                     void* ring_buf, void* rope_tail, hipStream_t stream);

/*
 * The same writer with the latent transform applied inside it (RAQ-MLA
 * Figure 4 caption: A_c acts on the latent before quantization, its inverse
 * is folded into the read-side weights; appendix Table 9: the transform
 * fused into the write kernel).  Every token's latent is replaced by
 *   y[c] = bf16( sum over k = 0..511 of A_c[c][k] * c_kv[k] )
 * with the sum an fp32 fused multiply-add chain in ascending k, rounded once
 * to the nearest bf16 (ties to even); y is then cached exactly as
 * mla_lowbit_write caches a latent row (codes, metadata, sink and ring
 * copies).  k_R is not transformed.  The result equals mla_lowbit_write on
 * the rows y, bit for bit.
 *
 *   a_c            bf16 [512][512] row-major ([output][input]), 16-B aligned,
 *                  read only; required (NULL is an argument error)
 *   other arguments, errors and ownership as mla_lowbit_write.
 */
int mla_lowbit_write_transformed(const mla_lowbit_layout* layout, const void* a_c, const void* c_kv,
                                 const void* k_r, const int32_t* cu_new, const int32_t* seqlens_before,
                                 int32_t batch, int32_t total_new, int32_t max_new_per_seq,
                                 const int32_t* block_table, int32_t max_pages, int32_t num_pool_pages,
                                 void* page_pool, void* sink_buf, void* ring_buf, void* rope_tail,
                                 hipStream_t stream);

/* Bytes of device workspace mla_lowbit_decode needs for this shape. Host only. */
int mla_lowbit_decode_workspace(const mla_lowbit_layout* layout, int32_t batch, int32_t heads,
                                int32_t max_seqlen, size_t* bytes);

/*
 * Decode attention over the packed cache (QuantMLA Figure 8 caption;
 * RAQ-MLA abstract and Figure 4 caption), one query token per sequence.
 * For sequence b with L = seqlens[b] valid tokens and every head h:
 *   token j is read from BF16 if j < sink or j >= L - local, otherwise from
 *   its dequantized codes (x = code * scale + min; the k_R of a page that is
 *   not yet full comes from the BF16 tail);
 *   z_j = softmax_scale * (q_lat[b][h] . c_j + q_rope[b][h] . k_j)
 *   out[b][h] = sum_j softmax(z)_j c_j        (fp32, latent space, 512)
 *   lse[b][h] = log sum_j exp(z_j)            (fp32, natural log)
 * L = 0 gives out = 0 and lse = -inf.  The buffers must hold what
 * mla_lowbit_write produced for exactly L tokens per sequence.
 *
 *   q_lat          bf16 [batch][heads][512];  q_rope bf16 [batch][heads][64]
 *   heads          1..128
 *   seqlens        int32 [batch] (device), each <= max_seqlen
 *   max_seqlen     host bound used for the work split; <= max_pages * P
 *   out            fp32 [batch][heads][512];  lse fp32 [batch][heads]
 *   workspace      device scratch of at least mla_lowbit_decode_workspace()
 *                  bytes, 16-B aligned, contents ignored (it holds the
 *                  per-split partial results between the attention kernel
 *                  and the merge kernel of one call; calls that share a
 *                  workspace must not run concurrently).  May be NULL when
 *                  the query returns 0 (one split per sequence).
 * Value range.  Queries and cached values must be finite with |x| <= 65280
 * (the largest bf16 below the fp16 limit): queries, BF16 rows and split
 * partials are carried as fp16.  Within that range the packed tokens'
 * scores and weights are exact-product MFMA sums scaled into fp16 range per
 * head, per page and per tile (no overflow at any magnitude).  BF16-path
 * values (sink, window) and queries of magnitude below 2^-14 keep an
 * absolute accuracy of 2^-25 rather than a relative one.
 */
int mla_lowbit_decode(const mla_lowbit_layout* layout, const void* q_lat, const void* q_rope,
                      int32_t batch, int32_t heads, float softmax_scale, const void* page_pool,
                      int32_t num_pool_pages, const int32_t* block_table, int32_t max_pages,
                      const int32_t* seqlens, int32_t max_seqlen, const void* sink_buf,
                      const void* ring_buf, const void* rope_tail, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_lowbit_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid hipMalloc).
 * Arguments, results and errors are those of mla_lowbit_decode without the
 * workspace: the per-split partials go to a fixed device array inside the
 * library, MLA_LOWBIT_NOALLOC_SCRATCH_BYTES long, of which every GPU the
 * library runs on holds its own copy until the process ends (its address is
 * looked up on the first call made on a device, with that device current).
 * The call allocates, frees and synchronizes nothing.
 *   - A shape whose mla_lowbit_decode_workspace() exceeds the scratch size
 *     returns MLA_LOWBIT_ERR_SCRATCH and launches nothing.
 *   - All calls on one GPU share its array and it keeps the last call's
 *     contents (nothing in it needs to start at zero): calls that may overlap
 *     on one GPU (different streams, or different threads without ordering)
 *     race; calls enqueued on one stream are ordered and safe.
 *   - The calling thread's current device must be the device of `stream`.
 */
#define MLA_LOWBIT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mla_lowbit_decode_noalloc(const mla_lowbit_layout* layout, const void* q_lat, const void* q_rope,
                              int32_t batch, int32_t heads, float softmax_scale, const void* page_pool,
                              int32_t num_pool_pages, const int32_t* block_table, int32_t max_pages,
                              const int32_t* seqlens, int32_t max_seqlen, const void* sink_buf,
                              const void* ring_buf, const void* rope_tail, float* out, float* lse,
                              hipStream_t stream);

/* Static description of an error code. */
const char* mla_lowbit_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LOWBIT_H */
