// quant.hip -- bf16 -> e4m3 (OCP E4M3FN) block quantizer with one fp32 scale per (64 rows, head).
//
// The reduced-precision K/V transport is the project page's "03 - End-to-end KV transport",
// "Precision" panel; the block shape (64 rows x all head_dim channels of one head) is the one the
// fp8 attention consumes.  Every decision is taken in fp32: amax = max |x| (NaN ignored),
// scale = amax/448, multiplier = 448/amax (both correctly rounded), y = x * multiplier clamped to
// [-448, 448] (NaN kept), then the hardware round-to-nearest-even conversion, which is exact RNE
// inside the clamp range; amax == 0 gives scale 1 and multiplier 1.
#include "blockq.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace wfattn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const uint16_t* __restrict__ x, int64_t rows, int heads,
                                                            uint8_t* __restrict__ x8, float* __restrict__ scales) {
  const int64_t blk = blockIdx.x / heads;
  const int head = blockIdx.x % heads;
  const int64_t r0 = blk * 64;
  const int nrows = (int)((rows - r0) < 64 ? (rows - r0) : 64);
  quantize_block<D>(x + ((size_t)r0 * heads + head) * D, nrows, heads, x8 + ((size_t)r0 * heads + head) * D,
                    scales + blk * heads + head);
}

// Publish for the e4m3 path: workgroup (tile t, head) quantizes the chunk's K rows 64t .. 64t+nv-1
// of that head as one block (a tile is a whole 64-row scale block of the pool: chunks start on
// fresh pages and pages hold a multiple of 64 rows), writes the codes to the tile's pool rows and
// the scale to its block, and copies the same rows of V.  Only valid rows enter the block's amax.
template <int D>
__global__ __launch_bounds__(256) void publish_e4m3_kernel(PublishFp8Params p) {
  const int32_t* hdr = p.blob;
  if (hdr[H_NONCE_LO] != (int32_t)p.nonce_lo || hdr[H_NONCE_HI] != (int32_t)p.nonce_hi) return;
  const int H = p.heads;
  const int t = blockIdx.x / H, head = blockIdx.x % H;
  const int first_tile = p.blob[hdr[H_OFF_CHUNKS] + p.chunk * kChunkInts];
  const int32_t* tile = p.blob + hdr[H_OFF_TILES] + (first_tile + t) * kTileInts;
  const int64_t row0 = tile[0];
  const int nv = tile[1];
  const size_t src = ((size_t)t * 64 * H + head) * D;
  const size_t dst = ((size_t)row0 * H + head) * D;
  quantize_block<D>(p.k_src + src, nv, H, p.k8_pool + dst, p.k_scale + (row0 / 64) * H + head);
  // V rows of this head: 16-byte granules, D/8 per row
  for (int i = threadIdx.x; i < nv * (D / 8); i += 256) {
    const int r = i / (D / 8), g = i % (D / 8);
    reinterpret_cast<uint4*>(p.v_pool + dst + (size_t)r * H * D)[g] =
        reinterpret_cast<const uint4*>(p.v_src + src + (size_t)r * H * D)[g];
  }
}

// e4m3 V pool for e4m3 K/V storage: workgroup (64-row block, head) quantizes the block exactly as
// quantize_e4m3_kernel (amax over the finite values, the same scale and RNE codes), except that a
// NaN value is padding (a slot past a chunk's end) and gets code 0, and writes the codes
// transposed, [channel][64 key slots], into the block's 64*D bytes of v8 (layout [rows/64, H, D,
// 64]).  Within each 32-key half the slots hold the 8-key groups in the order 0, 2, 1, 3, so that
// one 16-byte read of a channel gives a lane of the attention's P.V the keys of both its 16-key
// steps.  The transpose goes through LDS so that the stores are whole 16-byte granules.
template <int D>
__global__ __launch_bounds__(256) void quantize_v8_kernel(const uint16_t* __restrict__ x, int heads,
                                                          uint8_t* __restrict__ v8, float* __restrict__ scales) {
  using L = BlockLayout<D>;
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * 64];
  const int64_t blk = blockIdx.x / heads;
  const int head = blockIdx.x % heads;
  const int g = threadIdx.x % L::GPR, rsub = threadIdx.x / L::GPR;
  const uint16_t* src = x + ((size_t)blk * 64 * heads + head) * D;
  float v[L::ITER][8];
#pragma unroll
  for (int it = 0; it < L::ITER; ++it)
    unpack8(*reinterpret_cast<const uint4*>(src + (size_t)(it * L::RPI + rsub) * heads * D + g * 8), v[it]);
  float scale, mult;
  block_scale<D>(v, 64, scale, mult);
  if (threadIdx.x == 0) scales[blk * heads + head] = scale;
#pragma unroll
  for (int it = 0; it < L::ITER; ++it) {
    const int r = it * L::RPI + rsub;
    const int grp = (r >> 3) & 3;
    const int slot = (r & ~31) | ((grp == 1 ? 2 : grp == 2 ? 1 : grp) << 3) | (r & 7);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float t = __fmul_rn(v[it][j], mult);
      t = (t > 448.f) ? 448.f : t;
      t = (t < -448.f) ? -448.f : t;
      y[j] = (v[it][j] == v[it][j]) ? t : 0.f;  // NaN: padding, code 0
    }
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      tile[(8 * g + j) * 64 + slot] = (uint8_t)(((j < 4 ? (uint32_t)w0 : (uint32_t)w1) >> (8 * (j & 3))) & 0xff);
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(v8 + ((size_t)blk * heads + head) * (size_t)(64 * D));
  for (int i = threadIdx.x; i < D * 4; i += 256) dst[i] = reinterpret_cast<const uint4*>(tile)[i];
}

}  // namespace

hipError_t launch_quantize_v_fp8(const uint16_t* v, int64_t rows, int32_t heads, int32_t head_dim, uint8_t* v8,
                                 float* scales, hipStream_t s) {
  const int64_t grid = rows / 64 * heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(quantize_v8_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, v, heads, v8, scales);
  else
    hipLaunchKernelGGL(quantize_v8_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, v, heads, v8, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int32_t heads, int32_t head_dim, uint8_t* x8,
                               float* scales, hipStream_t s) {
  const int64_t nblk = (rows + 63) / 64;
  const int64_t grid = nblk * heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(quantize_e4m3_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, x, rows, heads, x8, scales);
  else
    hipLaunchKernelGGL(quantize_e4m3_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, x, rows, heads, x8, scales);
  return hipGetLastError();
}

hipError_t launch_publish_fp8(const PublishFp8Params& p, int64_t tokens, int32_t head_dim, hipStream_t s) {
  const int64_t grid = (tokens + 63) / 64 * p.heads;
  if (grid > 0) {
    if (head_dim == 128) hipLaunchKernelGGL(publish_e4m3_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(publish_e4m3_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return p.flags ? launch_flag(p.flags, p.chunk, p.generation, s) : hipSuccess;
}

}  // namespace wfattn
