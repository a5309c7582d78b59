/*
 * mla_bf16.h -- the plain BF16 paged cache of libmla_lowbit.so: the baseline
 * the low-bit cache is measured against (QuantMLA, Table 9 caption: BF16
 * attention with native partitioning, i.e. split-KV plus a log-sum-exp merge;
 * Figure 5 caption (b): attention latency normalized to BF16).
 *
 * Layout.  A pool of pages [num_pool_pages][P][576] bf16: token j of
 * sequence b is the row (c_KV[0..511], k_R[0..63]) at page
 * block_table[b][j / P], slot j % P.  P is a power of two in 16..1024.
 *
 * All pointers are device pointers owned by the caller, 16-byte aligned;
 * nothing is allocated, freed or synchronized.  Calls enqueue on `stream` and
 * return MLA_LOWBIT_OK or a negative MLA_LOWBIT_ERR_* code (mla_lowbit.h);
 * argument errors are found on the host before anything is launched.
 */
#ifndef MLA_BF16_H
#define MLA_BF16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Appends new tokens: rows cu_new[b] .. cu_new[b+1]-1 of c_kv / k_r are
 * sequence b's tokens at positions seqlens_before[b] + i, stored bit for bit
 * as rows of the pool.
 *   c_kv           bf16 [total_new][512];  k_r bf16 [total_new][64]
 *   cu_new         int32 [batch+1] (device), cu_new[0] = 0, non-decreasing,
 *                  last = total_new
 *   seqlens_before int32 [batch] (device), not modified
 *   max_new_per_seq host bound on cu_new[b+1] - cu_new[b] (grid sizing)
 *   block_table    int32 [batch][max_pages] (device), page ids in
 *                  [0, num_pool_pages); a row whose page id is outside that
 *                  range is dropped
 *   pool           bf16 [num_pool_pages][page_size][576]
 */
int mla_bf16_append(const void* c_kv, const void* k_r, const int32_t* cu_new, const int32_t* seqlens_before,
                    int32_t batch, int32_t total_new, int32_t max_new_per_seq, int32_t page_size,
                    const int32_t* block_table, int32_t max_pages, int32_t num_pool_pages, void* pool,
                    hipStream_t stream);

/* Bytes of device workspace mla_bf16_decode needs for this shape.  Host only. */
int mla_bf16_decode_workspace(int32_t page_size, int32_t batch, int32_t heads, int32_t max_seqlen,
                              size_t* bytes);

/*
 * Decode attention over the BF16 cache, one query token per sequence, the
 * same function as mla_lowbit_decode with every token read from its row:
 *   z_j = softmax_scale * (q_lat[b][h] . c_j + q_rope[b][h] . k_j)
 *   out[b][h] = sum_j softmax(z)_j c_j        (fp32, 512)
 *   lse[b][h] = log sum_j exp(z_j)            (fp32, natural log)
 * L = seqlens[b] = 0 gives out = 0 and lse = -inf.
 *   q_lat          bf16 [batch][heads][512];  q_rope bf16 [batch][heads][64]
 *   heads          1..128
 *   seqlens        int32 [batch] (device), each <= max_seqlen
 *   max_seqlen     host bound used for the work split; <= max_pages * P
 *   pool, block_table, num_pool_pages, max_pages, page_size  as above; a
 *                  page id outside [0, num_pool_pages) masks its tokens
 *   out            fp32 [batch][heads][512];  lse fp32 [batch][heads]
 *   workspace      device scratch of at least mla_bf16_decode_workspace()
 *                  bytes (split partials), 16-B aligned, contents ignored;
 *                  may be NULL when that is 0.  Concurrent calls must not
 *                  share it.
 * Values must be finite with |x| <= 65280 (split partials are fp16).
 */
int mla_bf16_decode(const void* q_lat, const void* q_rope, int32_t batch, int32_t heads, float softmax_scale,
                    const void* pool, int32_t num_pool_pages, int32_t page_size, const int32_t* block_table,
                    int32_t max_pages, const int32_t* seqlens, int32_t max_seqlen, float* out, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_BF16_H */
