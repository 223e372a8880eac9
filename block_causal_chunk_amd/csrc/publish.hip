// publish.hip -- write one chunk's K/V from projection layout into its pages of the paged pools,
// then raise the chunk's generation flag.
//
// The producers of the Wave Forcing pipeline write their K/V straight into the slots the consumer
// reads, and the consumer reads its prefix in place with no assembly (Wave Forcing project page,
// "03 - End-to-end KV transport", panel "03 - Layout"; KipQuest paper page, "The deep dive", on
// the paged variant).  The consumer uses a chunk's states only once they are complete: here a
// per-chunk generation counter, raised after the copy, which the gated forward checks.
#include "blockq.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace wfattn {
namespace {

constexpr int kParts = 8;  // workgroups per 64-token tile: one chunk's copy spreads over the CUs

// Workgroup (tile t, part): tile t of the chunk holds tokens 64t .. 64t+nv-1, and its pool rows
// row0 .. row0+nv-1 are contiguous (a tile never crosses a page), as are those tokens' rows of the
// projection layout.  So the tile is one contiguous block in both, copied in 16-byte granules.
__global__ __launch_bounds__(256) void publish_kernel(PublishParams p) {
  const int32_t* hdr = p.blob;
  if (hdr[H_NONCE_LO] != (int32_t)p.nonce_lo || hdr[H_NONCE_HI] != (int32_t)p.nonce_hi) return;
  const int t = blockIdx.x / kParts, part = blockIdx.x % kParts;
  const int first_tile = p.blob[hdr[H_OFF_CHUNKS] + p.chunk * kChunkInts];
  const int32_t* tile = p.blob + hdr[H_OFF_TILES] + (first_tile + t) * kTileInts;
  const int64_t row0 = tile[0], nv = tile[1];
  const int64_t G = nv * p.row_granules;
  const uint4* sk = reinterpret_cast<const uint4*>(p.k_src) + (int64_t)t * 64 * p.row_granules;
  const uint4* sv = reinterpret_cast<const uint4*>(p.v_src) + (int64_t)t * 64 * p.row_granules;
  uint4* dk = reinterpret_cast<uint4*>(p.k_pool) + row0 * p.row_granules;
  uint4* dv = reinterpret_cast<uint4*>(p.v_pool) + row0 * p.row_granules;
  for (int64_t i = (int64_t)part * 256 + threadIdx.x; i < G; i += kParts * 256) {
    const uint4 a = sk[i], b = sv[i];
    dk[i] = a;
    dv[i] = b;
  }
}

// Rotate channel pairs (2i, 2i+1) of eight values by angles with cosines c[0..3], sines s[0..3]:
// (x0, x1) -> (x0 c - x1 s, x0 s + x1 c), each product and sum rounded to fp32 on its own (no
// fused multiply-add), then each result rounded to bf16 (RNE); o holds the bf16 values widened
// back to fp32, w the packed bf16.
__device__ __forceinline__ void rotate8(const float (&x)[8], const float4 c, const float4 s, float (&o)[8], uint4& w) {
#pragma clang fp contract(off)
  const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
  uint32_t u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x0 = x[2 * j], x1 = x[2 * j + 1];
    const float a = x0 * cc[j], b = x1 * ss[j], e = x0 * ss[j], f = x1 * cc[j];
    const float y0 = a - b, y1 = e + f;
    u[j] = pack2_bf16(y0, y1);
    o[2 * j] = __uint_as_float(u[j] << 16);
    o[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
  }
  w = make_uint4(u[0], u[1], u[2], u[3]);
}

// Fused pre-attention epilogue of one chunk.  Workgroup (tile t, head): the tile's tokens 64t ..
// 64t+nv-1 (one page-aligned 64-row block of the pool, and one 64-row Q-scale block of the chunk).
// Q and K are rotated (rotate8), V passes through; Q goes to q_out and/or, quantized as one block,
// to q8; K goes to the tile's pool rows in bf16, or quantized as one block into the e4m3 pool; V to
// its pool rows.  The quantizer sees the bf16-rounded rotated values, so the e4m3 result equals
// rotating, rounding to bf16 and then calling the block quantizer.
template <int D>
__global__ __launch_bounds__(256) void rope_publish_kernel(RopeParams p) {
  using L = BlockLayout<D>;
  const int32_t* hdr = p.blob;
  if (hdr[H_NONCE_LO] != (int32_t)p.nonce_lo || hdr[H_NONCE_HI] != (int32_t)p.nonce_hi) return;
  const int H = p.heads;
  const int t = blockIdx.x / H, head = blockIdx.x % H;
  const int first_tile = p.blob[hdr[H_OFF_CHUNKS] + p.chunk * kChunkInts];
  const int32_t* tile = p.blob + hdr[H_OFF_TILES] + (first_tile + t) * kTileInts;
  const int64_t row0 = tile[0];
  const int nv = tile[1];
  const int g = threadIdx.x % L::GPR, rsub = threadIdx.x / L::GPR;
  float qv[L::ITER][8], kv[L::ITER][8];
#pragma unroll
  for (int it = 0; it < L::ITER; ++it) {
    const int r = it * L::RPI + rsub;
    if (r >= nv) continue;
    const int64_t tok = (int64_t)t * 64 + r;
    const uint16_t* src = p.qkv + (tok * 3 * H + head) * D + 8 * g;
    // the row's q, k, v and angles are all loaded before its first store (the compiler would
    // otherwise keep the k and v loads behind the q store, which may alias them as far as it knows)
    const uint4 xq = *reinterpret_cast<const uint4*>(src);
    const uint4 xk = *reinterpret_cast<const uint4*>(src + (size_t)H * D);
    const uint4 xv = *reinterpret_cast<const uint4*>(src + (size_t)2 * H * D);
    const float4 c = *reinterpret_cast<const float4*>(p.cos_t + tok * (D / 2) + 4 * g);
    const float4 s = *reinterpret_cast<const float4*>(p.sin_t + tok * (D / 2) + 4 * g);
    float x[8];
    uint4 w;
    unpack8(xq, x);
    rotate8(x, c, s, qv[it], w);
    if (p.q_out) *reinterpret_cast<uint4*>(p.q_out + (tok * H + head) * D + 8 * g) = w;
    unpack8(xk, x);
    rotate8(x, c, s, kv[it], w);
    const size_t prow = ((size_t)(row0 + r) * H + head) * D + 8 * g;
    if (p.k_pool) *reinterpret_cast<uint4*>(p.k_pool + prow) = w;
    *reinterpret_cast<uint4*>(p.v_pool + prow) = xv;
  }
  if (p.q8)
    quantize_regs<D>(qv, nv, (size_t)H * D, p.q8 + ((size_t)t * 64 * H + head) * D, p.q_scale + (size_t)t * H + head);
  if (p.k8_pool)
    quantize_regs<D>(kv, nv, (size_t)H * D, p.k8_pool + ((size_t)row0 * H + head) * D, p.k_scale + (row0 / 64) * H + head);
}

// Runs after the copy on the same stream, so every granule of it is visible device-wide first.
__global__ void flag_kernel(uint32_t* flags, int chunk, uint32_t generation) {
  __hip_atomic_store(flags + chunk, generation, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_publish(const PublishParams& p, int64_t tokens, hipStream_t s) {
  const int64_t n_tiles = (tokens + 63) / 64;
  if (n_tiles > 0) {
    hipLaunchKernelGGL(publish_kernel, dim3((unsigned)(n_tiles * kParts)), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return p.flags ? launch_flag(p.flags, p.chunk, p.generation, s) : hipSuccess;
}

hipError_t launch_rope_publish(const RopeParams& p, int64_t tokens, int32_t head_dim, hipStream_t s) {
  const int64_t grid = (tokens + 63) / 64 * p.heads;
  if (grid > 0) {
    if (head_dim == 128) hipLaunchKernelGGL(rope_publish_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(rope_publish_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return p.flags ? launch_flag(p.flags, p.chunk, p.generation, s) : hipSuccess;
}

hipError_t launch_flag(uint32_t* flags, int32_t chunk, uint32_t generation, hipStream_t s) {
  hipLaunchKernelGGL(flag_kernel, dim3(1), dim3(1), 0, s, flags, chunk, generation);
  return hipGetLastError();
}

}  // namespace wfattn
