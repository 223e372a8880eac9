// blockq.hpp -- e4m3 block quantization of one (64-row block, head) by a 256-thread workgroup,
// shared by the quantizer, the e4m3 publish and the fused pre-attention epilogue.
//
// The reduced-precision K/V transport is the project page's "03 - End-to-end KV transport",
// "Precision" panel; the block shape (64 rows x all head_dim channels of one head) is the one the
// e4m3 attention consumes.  Every decision is taken in fp32.
#pragma once

#include "device.hpp"

namespace wfattn {

// Thread layout shared by the block routines: a 256-thread workgroup covers one (64-row block,
// head); thread (rsub, g) holds channels 8g .. 8g+7 of rows it*RPI + rsub, it < ITER.
template <int D>
struct BlockLayout {
  static constexpr int GPR = D / 8;      // 16-byte groups per row
  static constexpr int RPI = 256 / GPR;  // rows covered by the workgroup per iteration
  static constexpr int ITER = 64 / RPI;
};

// Quantize the block held in registers (v: this thread's values, rows >= nrows ignored): amax over
// the block (NaN ignored), scale = amax/448 and multiplier 448/amax (both correctly rounded),
// codes = RNE e4m3 of v * multiplier clamped to [-448, 448] (NaN kept); amax == 0 gives scale 1.
// Row r of the codes goes to x8 + r * row_stride; the scale to *scale_out.
// The block's scale and multiplier (amax over rows < nrows, NaN ignored; amax == 0 gives 1, 1).
template <int D>
__device__ __forceinline__ void block_scale(const float (&v)[BlockLayout<D>::ITER][8], int nrows, float& scale,
                                            float& mult) {
  using L = BlockLayout<D>;
  const int rsub = threadIdx.x / L::GPR;
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < L::ITER; ++it) {
    if (it * L::RPI + rsub < nrows) {
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
  __syncthreads();  // wmax is reused by the next block of this workgroup
  scale = 1.f;
  mult = 1.f;
  if (amax > 0.f) {
    scale = __fdiv_rn(amax, 448.f);
    mult = __fdiv_rn(448.f, amax);
  }
}

template <int D>
__device__ __forceinline__ void quantize_regs(const float (&v)[BlockLayout<D>::ITER][8], int nrows, size_t row_stride,
                                              uint8_t* __restrict__ x8, float* __restrict__ scale_out) {
  using L = BlockLayout<D>;
  const int g = threadIdx.x % L::GPR, rsub = threadIdx.x / L::GPR;
  float scale, mult;
  block_scale<D>(v, nrows, scale, mult);
  if (threadIdx.x == 0) *scale_out = scale;
#pragma unroll
  for (int it = 0; it < L::ITER; ++it) {
    const int r = it * L::RPI + rsub;
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
      *reinterpret_cast<uint2*>(x8 + (size_t)r * row_stride + g * 8) = make_uint2((uint32_t)w0, (uint32_t)w1);
    }
  }
}

// Eight bf16 values (one 16-byte group) widened exactly to fp32.
__device__ __forceinline__ void unpack8(const uint4 w, float (&o)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = __uint_as_float(u[j] << 16);
    o[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
  }
}

// One (64-row block, head) from memory: row r of the source at x + r * heads * D (this head's
// channels), codes at x8 + r * heads * D, the scale to *scale_out.
template <int D>
__device__ __forceinline__ void quantize_block(const uint16_t* __restrict__ x, int nrows, int heads,
                                               uint8_t* __restrict__ x8, float* __restrict__ scale_out) {
  using L = BlockLayout<D>;
  const int g = threadIdx.x % L::GPR, rsub = threadIdx.x / L::GPR;
  float v[L::ITER][8];
#pragma unroll
  for (int it = 0; it < L::ITER; ++it) {
    const int r = it * L::RPI + rsub;
    if (r < nrows) unpack8(*reinterpret_cast<const uint4*>(x + (size_t)r * heads * D + g * 8), v[it]);
  }
  quantize_regs<D>(v, nrows, (size_t)heads * D, x8, scale_out);
}

}  // namespace wfattn
