// quant.hip -- bf16 -> e4m3 (OCP E4M3FN) block quantizer with one fp32 scale per (64 rows, head).
//
// The reduced-precision K/V transport is the project page's "03 - End-to-end KV transport",
// "Precision" panel; the block shape (64 rows x all head_dim channels of one head) is the one the
// fp8 attention consumes.  Every decision is taken in fp32: amax = max |x| (NaN ignored),
// scale = amax/448, multiplier = 448/amax (both correctly rounded), y = x * multiplier clamped to
// [-448, 448] (NaN kept), then the hardware round-to-nearest-even conversion, which is exact RNE
// inside the clamp range; amax == 0 gives scale 1 and multiplier 1.
#include "device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace wfattn {
namespace {

// One (64-row block, head): rows [0, nrows) of the block, row r of the source at
// x + r * heads * D and of the codes at x8 + r * heads * D (this head's channels); the scale goes
// to *scale.  Called by a whole 256-thread workgroup.
template <int D>
__device__ __forceinline__ void quantize_block(const uint16_t* __restrict__ x, int nrows, int heads,
                                               uint8_t* __restrict__ x8, float* __restrict__ scale_out) {
  constexpr int GPR = D / 8;            // 16-byte groups per row
  constexpr int RPI = 256 / GPR;        // rows covered by the block per iteration
  constexpr int ITER = 64 / RPI;
  const int g = threadIdx.x % GPR, rsub = threadIdx.x / GPR;
  float v[ITER][8];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int r = it * RPI + rsub;
    if (r < nrows) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + (size_t)r * heads * D + g * 8);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[it][2 * j] = __uint_as_float(u[j] << 16);
        v[it][2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = fabsf(v[it][j]);
        amax = (a > amax) ? a : amax;  // a NaN compares false and is ignored
      }
    }
  }
  // block max: wave shuffle, then across the 4 waves through LDS
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(amax, off);
    amax = (o > amax) ? o : amax;
  }
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) amax = (wmax[w] > amax) ? wmax[w] : amax;
  float scale = 1.f, mult = 1.f;
  if (amax > 0.f) {
    scale = __fdiv_rn(amax, 448.f);
    mult = __fdiv_rn(448.f, amax);
  }
  if (threadIdx.x == 0) *scale_out = scale;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int r = it * RPI + rsub;
    if (r < nrows) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float t = __fmul_rn(v[it][j], mult);
        t = (t > 448.f) ? 448.f : t;
        t = (t < -448.f) ? -448.f : t;
        y[j] = t;
      }
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
      *reinterpret_cast<uint2*>(x8 + (size_t)r * heads * D + g * 8) = make_uint2((uint32_t)w0, (uint32_t)w1);
    }
  }
}

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

}  // namespace

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
