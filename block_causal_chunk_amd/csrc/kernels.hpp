// kernels.hpp -- launch parameters and launchers of the wfattn HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wfattn {

struct FwdParams {
  const uint16_t* q;       // bf16 [Lq, H, D]
  const uint16_t* k;       // bf16 pool [pool_rows, H, D]
  const uint16_t* v;       // bf16 pool [pool_rows, H, D]
  const uint8_t* q8;       // e4m3 [Lq, H, D]               (fp8 path)
  const float* q_scale;    // [nqb, H]                      (fp8 path)
  const uint8_t* k8;       // e4m3 pool                     (fp8 path)
  const float* k_scale;    // [pool_rows / 64, H]           (fp8 path)
  void* out;               // bf16 or fp32 [Lq, H, D]
  float* lse;              // [H, Lq] or nullptr
  const int32_t* blob;     // uploaded work list (device)
  float* part_o;           // [n_partials, BM, D]
  float* part_lse;         // [n_partials, BM]
  int32_t H;
  int32_t lq;
  float c;                 // softmax scale * log2(e)
  float scale;             // softmax scale
  uint32_t nonce_lo, nonce_hi;
};

hipError_t launch_attn_bf16(const FwdParams& p, int head_dim, bool out_f32, int grid, hipStream_t s);
hipError_t launch_attn_fp8(const FwdParams& p, int head_dim, int grid, hipStream_t s);
hipError_t launch_combine(const FwdParams& p, int head_dim, bool out_f32, int groups, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int32_t heads, int32_t head_dim,
                               uint8_t* x8, float* scales, hipStream_t s);

}  // namespace wfattn
