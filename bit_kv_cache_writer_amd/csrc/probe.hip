// Measurement probes for gfx950 (declared in mla_lowbit_probe.h): the HBM
// read rate and the fp16 matrix-core rate the GPU sustains.  Not part of the
// cache method; the benchmark reports the decode's rates against them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_lowbit.h"
#include "mla_lowbit_probe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Grid-stride stream of 16-byte loads, four in flight per thread per step.
__global__ void __launch_bounds__(kThreads) read_probe(const u32x4* __restrict__ src, size_t n16,
                                                       uint32_t* __restrict__ sink) {
  const size_t tid = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= (a ^ b) ^ (c ^ d);
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Eight independent accumulator chains of v_mfma_f32_32x32x16_f16 (the
// fastest fp16 form on gfx950) per wave, so the matrix core never waits on a
// previous result.
__global__ void __launch_bounds__(kThreads) mfma_probe(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = static_cast<_Float16>(0.001f * static_cast<float>((lane + k) & 7));
    b[k] = static_cast<_Float16>(0.001f * static_cast<float>((lane * 3 + k) & 7));
  }
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[k][r];
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int mla_lowbit_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 64 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u))
    return MLA_LOWBIT_ERR_ARG;
  hipLaunchKernelGGL(read_probe, dim3(MLA_LOWBIT_PROBE_BLOCKS), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ERR_HIP;
}

extern "C" int mla_lowbit_probe_mfma(float* sink, int32_t iters, double* flops, hipStream_t stream) {
  if (!sink || !flops || iters < 1 || iters > 1000000 || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return MLA_LOWBIT_ERR_ARG;
  *flops = static_cast<double>(MLA_LOWBIT_PROBE_BLOCKS) * 4.0 * iters * 8.0 * (2.0 * 32 * 32 * 16);
  hipLaunchKernelGGL(mfma_probe, dim3(MLA_LOWBIT_PROBE_BLOCKS), dim3(kThreads), 0, stream, sink, iters);
  return hipGetLastError() == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ERR_HIP;
}
