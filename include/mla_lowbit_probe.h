/*
 * mla_lowbit_probe.h -- measurement probes of libmla_lowbit.so.
 *
 * Not part of the cache method: two kernels that measure what this GPU
 * sustains, so that the decode's rates can be reported against measured
 * peaks next to the published ones (HBM 8 TB/s, fp16 matrix 2.5 PFLOP/s).
 * Both take device pointers owned by the caller, enqueue on `stream`, and
 * return MLA_LOWBIT_OK or a negative MLA_LOWBIT_ERR_* code (argument errors
 * are found on the host before anything is launched).
 */
#ifndef MLA_LOWBIT_PROBE_H
#define MLA_LOWBIT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups (of 256 threads) each probe launches. */
#define MLA_LOWBIT_PROBE_BLOCKS 2048

/*
 * Streams `bytes` (a multiple of 64, 16-B aligned) of `src` once with 16-byte
 * vector loads and writes one 32-bit digest per thread to `sink`
 * (MLA_LOWBIT_PROBE_BLOCKS * 256 uint32, 4 B aligned), so the loads cannot be
 * dropped.  Achieved read rate = bytes / elapsed.
 */
int mla_lowbit_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * Runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_f16 chains in
 * every wave of MLA_LOWBIT_PROBE_BLOCKS workgroups of 4 waves, and writes one
 * float per thread to `sink` (MLA_LOWBIT_PROBE_BLOCKS * 256 floats).  *flops
 * receives the dense flop count of the launch:
 *   MLA_LOWBIT_PROBE_BLOCKS * 4 * iters * 8 * (2 * 32 * 32 * 16).
 * iters must be in 1 .. 1,000,000.
 */
int mla_lowbit_probe_mfma(float* sink, int32_t iters, double* flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LOWBIT_PROBE_H */
