// probe.hip -- issue-rate probe for the measurement side (libwfprobe.so, loaded by the benchmark
// only; not part of the attention library).  It measures how many v_exp_f32 the chip retires per
// second when nothing else runs: the ceiling against which the attention's exponentials per second
// (one per visible (query row, key, head) triple, the online softmax's weights) are read.
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

}  // namespace

extern "C" int64_t wfprobe_exp_rate(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(exp_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  if (hipGetLastError() != hipSuccess) return -1;
  return (int64_t)blocks * 256 * kChains * iters;
}
