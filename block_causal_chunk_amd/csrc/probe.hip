// probe.hip -- probes for the measurement side (libwfprobe.so, loaded by the benchmark only; not
// part of the attention library):
//   * how many v_exp_f32 the chip retires per second when nothing else runs: the ceiling against
//     which the attention's exponentials per second (one per visible (query row, key, head)
//     triple, the online softmax's weights) are read;
//   * a plain device copy of known size, the reference that scales the memory counters
//     (FETCH_SIZE, WRITE_SIZE) of a profiling run to bytes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "wfprobe.h"

namespace {

constexpr int kChains = 8;  // independent dependency chains per lane: enough to hide the latency

// Each lane iterates x <- 2^(-x) on kChains values; from [0, 1) the values stay in [0.5, 1], so
// no chain reaches a denormal or an infinity whatever the iteration count.  One store per lane
// keeps the chains live.
__global__ __launch_bounds__(256) void exp_rate_kernel(float* __restrict__ out, int iters) {
  float x[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) x[k] = 0.1f * k + 1e-4f * threadIdx.x;
#pragma unroll 4
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += x[k];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride copy of n16 16-byte granules: every granule read once and written once.
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

}  // namespace

extern "C" int32_t wfprobe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes <= 0 || (bytes & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return -1;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + 255) / 256 < 8192 ? (n16 + 255) / 256 : 8192;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int64_t wfprobe_exp_rate(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(exp_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  if (hipGetLastError() != hipSuccess) return -1;
  return (int64_t)blocks * 256 * kChains * iters;
}
