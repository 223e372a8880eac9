// publish.hip -- write one chunk's K/V from projection layout into its pages of the paged pools,
// then raise the chunk's generation flag.
//
// The producers of the Wave Forcing pipeline write their K/V straight into the slots the consumer
// reads, and the consumer reads its prefix in place with no assembly (Wave Forcing project page,
// "03 - End-to-end KV transport", panel "03 - Layout"; KipQuest paper page, "The deep dive", on
// the paged variant).  The consumer uses a chunk's states only once they are complete: here a
// per-chunk generation counter, raised after the copy, which the gated forward checks.
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

hipError_t launch_flag(uint32_t* flags, int32_t chunk, uint32_t generation, hipStream_t s) {
  hipLaunchKernelGGL(flag_kernel, dim3(1), dim3(1), 0, s, flags, chunk, generation);
  return hipGetLastError();
}

}  // namespace wfattn
