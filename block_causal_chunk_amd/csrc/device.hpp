// device.hpp -- gfx950 device helpers shared by the wfattn kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wfattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define WF_LDS __attribute__((address_space(3)))

// Physical 16-byte granule of logical granule g in row r of an LDS tile whose rows are D bf16
// (D/8 granules).  XOR swizzle f(r) = 4*(r%4) + (r/4)%4 makes both access patterns of the
// attention kernel conflict-free: 16 lanes reading one granule column over 16 consecutive rows
// (f is a bijection on r%16), and the transposed reads that touch 4 consecutive rows x 4
// consecutive granules (low two bits of f(r) fixed, bits 2-3 distinct).
template <int D>
__device__ __forceinline__ int swz(int r, int g) {
  return g ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (D / 8 - 1));
}

// Element offset of (row, col) inside a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * D + swz<D>(r, c >> 3) * 8 + (c & 7);
}

// max of three scores in one v_max3_f32.  fmaxf would add a canonicalising v_max per operand
// (IEEE signalling-NaN handling); scores are never NaN here.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap exchanges the upper 32 lanes of
// its first operand with the lower 32 lanes of its second; called with x twice, one result holds
// x of this lane and the other x of the partner lane, so the symmetric max/sum of the two results
// is the pair's max/sum on every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// O += A.B on v_mfma_f32_32x32x16_bf16 with the accumulator pinned in AGPRs.  The attention's O
// tile (128 fp32 per lane for two 32-row blocks at d = 128) cannot share the 256 VGPRs with Q,
// the scores and P; held in AGPRs it is only touched by MFMAs in the key loop.  The compiler does
// not know this instruction's latency, so every VALU access to such an accumulator must follow
// mfma_drain() on it.
__device__ __forceinline__ void mfma_acc_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// 24 wait states, ordered after the MFMAs that write `acc` and before any VALU use of it (an
// 8-pass XDL result needs 11 before a VALU or v_accvgpr_read may touch it); also separates a
// VALU write of `acc` from the next MFMA that reads it.
__device__ __forceinline__ void mfma_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Load through the constant address space: uniform indices become scalar loads (s_load), which
// wait on lgkmcnt and so never stall on the vmcnt of in-flight global->LDS tile fills.
template <class T>
__device__ __forceinline__ T ld_const(const T* p, int i) {
  return ((const __attribute__((address_space(4))) T*)(p))[i];
}

// Pack 8 fp32 into bf16x8 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // v_cvt_pk_bf16_f32
}

// Pack 2 fp32 into fp16x2 with round-to-nearest-even.
__device__ __forceinline__ uint32_t pack2_f16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

}  // namespace wfattn
