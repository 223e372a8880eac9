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
  const uint8_t* v8;       // e4m3 V pool [pool_rows / 64, H, D, 64] (e4m3 K/V storage)
  const float* v_scale;    // [pool_rows / 64, H]           (e4m3 K/V storage)
  void* out;               // bf16 or fp32 [Lq, H, D]
  float* lse;              // [H, Lq] or nullptr
  const int32_t* blob;     // uploaded work list (device)
  uint16_t* part_o;        // fp16 [n_partials, BM, D]: row r holds O_r * 2^-e_r
  float* part_lse;         // [n_partials, BM, 2]: the row's LSE, then e_r (int32 bits)
  int32_t H;
  int32_t lq;
  float c;                 // softmax scale * log2(e)
  float scale;             // softmax scale
  uint32_t nonce_lo, nonce_hi;
  // Optional gate: before a work item reads keys, every chunk it sees must have
  // gate_flags[c] >= gate_need[c]; polled at most gate_spin times, else the item is skipped and
  // bit 0 of *gate_status is set.  gate_flags == nullptr: no gate.
  const uint32_t* gate_flags;
  const uint32_t* gate_need;
  uint32_t* gate_status;
  int32_t gate_spin;
};

struct PublishParams {
  const uint16_t* k_src;   // bf16 [tokens, H, D], projection layout
  const uint16_t* v_src;
  uint16_t* k_pool;        // bf16 [pool_rows, H, D]
  uint16_t* v_pool;
  const int32_t* blob;     // uploaded work list (device): chunk table and key tiles
  int32_t chunk;
  int32_t row_granules;    // 16-byte granules per token row (H * D * 2 / 16)
  uint32_t nonce_lo, nonce_hi;
  uint32_t* flags;         // nullptr, or flags[chunk] = generation after the copy
  uint32_t generation;
};

struct PublishFp8Params {
  const uint16_t* k_src;   // bf16 [tokens, H, D], projection layout
  const uint16_t* v_src;
  uint8_t* k8_pool;        // e4m3 [pool_rows, H, D]
  float* k_scale;          // [pool_rows / 64, H]
  uint16_t* v_pool;        // bf16 [pool_rows, H, D]
  const int32_t* blob;
  int32_t chunk;
  int32_t heads;
  uint32_t nonce_lo, nonce_hi;
  uint32_t* flags;
  uint32_t generation;
};

struct RopeParams {
  const uint16_t* qkv;     // bf16 [tokens, 3, H, D]: q, k, v of a token side by side
  const float* cos_t;      // [tokens, D/2]
  const float* sin_t;      // [tokens, D/2]
  uint16_t* q_out;         // bf16 [tokens, H, D] or nullptr
  uint8_t* q8;             // e4m3 [tokens, H, D] or nullptr
  float* q_scale;          // [ceil(tokens/64), H]
  uint16_t* k_pool;        // bf16 pool, or nullptr when k8_pool is set
  uint8_t* k8_pool;        // e4m3 pool, or nullptr
  float* k_scale;          // [pool_rows / 64, H]
  uint16_t* v_pool;        // bf16 pool
  const int32_t* blob;
  int32_t chunk;
  int32_t heads;
  uint32_t nonce_lo, nonce_hi;
  uint32_t* flags;
  uint32_t generation;
};

struct QkvParams {
  const uint16_t* x;       // bf16 [tokens, hidden]: the chunk's hidden states
  const uint16_t* w;       // bf16 [hidden, 3 * H * D]: columns (role, head, channel), role q, k, v
  int32_t tokens;
  int32_t hidden;          // a multiple of 64
  const float* cos_t;      // [tokens, D/2]
  const float* sin_t;      // [tokens, D/2]
  uint16_t* q_out;         // bf16 [tokens, H, D] or nullptr
  uint8_t* q8;             // e4m3 [tokens, H, D] or nullptr
  float* q_scale;          // [ceil(tokens/64), H]
  uint16_t* k_pool;        // bf16 pool, or nullptr when k8_pool is set
  uint8_t* k8_pool;        // e4m3 pool, or nullptr
  float* k_scale;          // [pool_rows / 64, H]
  uint16_t* v_pool;        // bf16 pool
  const int32_t* blob;
  int32_t chunk;
  int32_t heads;
  uint32_t nonce_lo, nonce_hi;
  uint32_t* flags;
  uint32_t generation;
};

hipError_t launch_attn_bf16(const FwdParams& p, int head_dim, bool out_f32, int grid, hipStream_t s);
hipError_t launch_attn_fp8(const FwdParams& p, int head_dim, int grid, hipStream_t s);
hipError_t launch_attn_fp8kv(const FwdParams& p, int head_dim, int grid, hipStream_t s);
hipError_t launch_quantize_v_fp8(const uint16_t* v, int64_t rows, int32_t heads, int32_t head_dim, uint8_t* v8,
                                 float* scales, hipStream_t s);
hipError_t launch_combine(const FwdParams& p, int head_dim, bool out_f32, int groups, hipStream_t s);
hipError_t launch_publish(const PublishParams& p, int64_t tokens, hipStream_t s);
// flags[chunk] = generation, release-ordered after everything before it on the stream
hipError_t launch_flag(uint32_t* flags, int32_t chunk, uint32_t generation, hipStream_t s);
hipError_t launch_publish_fp8(const PublishFp8Params& p, int64_t tokens, int32_t head_dim, hipStream_t s);
hipError_t launch_rope_publish(const RopeParams& p, int64_t tokens, int32_t head_dim, hipStream_t s);
hipError_t launch_qkv_rope_publish(const QkvParams& p, int32_t head_dim, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
// the rows of key tiles 0 .. n_tiles-1 of a plan's tile list (device), row_elems values per row
hipError_t launch_f32_tiles_to_bf16(const float* in, uint16_t* out, const int32_t* tiles, int n_tiles, int64_t row_elems,
                                    hipStream_t s);
hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int32_t heads, int32_t head_dim,
                               uint8_t* x8, float* scales, hipStream_t s);

}  // namespace wfattn
