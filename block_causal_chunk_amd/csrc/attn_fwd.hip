// attn_fwd.hip -- block-causal chunk attention forward, bf16 MFMA (gfx950).
//
// What one workgroup computes: one work item = (head, query tile of up to 128 rows of one query
// chunk, a contiguous range of that chunk's visible key tiles).  The visible keys are the chunk's
// own tokens and every earlier, cleaner chunk's tokens (Wave Forcing project page, "01 - The
// design gap", directed frontier and "Key observation"); the planner has already reduced them to
// a list of 64-key tiles that never cross a page, so nothing here tests chunk visibility: masked
// tiles are simply not in the list.  Keys are read from the paged pool in place (project page,
// "03 - End-to-end KV transport", "Layout" panel).
//
// Data flow per key tile (4 waves, 32 query rows each):
//   K, V tile [64 x d] : global (16 B per lane, coalesced rows) -> registers -> swizzled LDS,
//                        double-buffered so the next tile's loads fly during this tile's math
//   S^T = K . Q^T      : v_mfma_f32_32x32x16_bf16, K rows read from LDS in a bit-swapped order
//                        so each lane ends up owning 8 consecutive keys of one query
//   online softmax     : fp32 in registers; one lane pair (l, l^32) per query, exp2 with the
//                        softmax scale folded into log2(e)
//   O^T += V^T . P^T   : P stays in registers as the B operand; V^T comes from LDS through
//                        ds_read_b64_tr_b16 transposed reads
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace wfattn {
namespace {

constexpr int BM = kBlockM;  // 128 query rows per workgroup
constexpr int BN = kBlockN;  // 64 keys per tile
constexpr int NTHR = 256;    // 4 waves of 64

// Row of the K tile that lane row r of the S^T A-operand reads: bits 2 and 3 swapped.  With it,
// accumulator register i of lane l holds key 16*(i/8) + 8*(l/32) + i%8 of the 32-key block.
__device__ __forceinline__ int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Global -> register -> LDS staging of one key tile: K (bf16 rows of 2*D bytes, or e4m3 rows of D
// bytes) and V (bf16).  Rows past the tile's valid keys are zero-filled, so the pool's padding
// slots are never read.
template <int D, bool FP8>
struct TileLoader {
  static constexpr int KB = FP8 ? D : 2 * D;           // bytes per K row
  static constexpr int KG = KB / 16;                   // 16-byte granules per K row
  static constexpr int KPER = BN * KG / NTHR;          // K granules per thread
  static constexpr int VPER = BN * D / 8 / NTHR;       // V granules per thread
  uint4 kr[KPER], vr[VPER];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ k, const uint16_t* __restrict__ v, int row0,
                                       int nvalid, int head, int H) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int ci = threadIdx.x + NTHR * i;
      const int row = ci / KG, g = ci % KG;
      kr[i] = make_uint4(0, 0, 0, 0);
      if (row < nvalid) kr[i] = *reinterpret_cast<const uint4*>(k + ((size_t)(row0 + row) * H + head) * KB + g * 16);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int ci = threadIdx.x + NTHR * i;
      const int row = ci / (D / 8), g = ci % (D / 8);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (row < nvalid) vr[i] = *reinterpret_cast<const uint4*>(v + ((size_t)(row0 + row) * H + head) * D + g * 8);
    }
  }
  __device__ __forceinline__ void store(uint8_t* sk, uint16_t* sv) const {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int ci = threadIdx.x + NTHR * i;
      const int row = ci / KG, g = ci % KG;
      *reinterpret_cast<uint4*>(sk + kswz_off(row, g)) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int ci = threadIdx.x + NTHR * i;
      const int row = ci / (D / 8), g = ci % (D / 8);
      *reinterpret_cast<uint4*>(sv + row * D + swz<D>(row, g) * 8) = vr[i];
    }
  }
  // Byte offset of granule g of K row r.  bf16: the same swizzle as V.  e4m3: rows are D bytes,
  // so 256/D rows share one 64-bank line; XOR with (r / (256/D)) spreads 16 rows of one granule
  // column over distinct banks.
  __device__ __forceinline__ static int kswz_off(int r, int g) {
    if constexpr (FP8) return r * KB + ((g ^ ((r / (256 / D)) & (KG - 1))) * 16);
    else return r * KB + swz<D>(r, g) * 16;
  }
};

// One work item (see the top of this file).  FP8: Q and K are e4m3 codes with one fp32 scale per
// (64-row block, head); the product of the two block scales and the softmax scale is applied
// once to the fp32 accumulator, P.V stays bf16.
template <int D, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(NTHR, 2) void attn_fwd_kernel(FwdParams p) {
  using Loader = TileLoader<D, FP8>;
  constexpr int KTILE = BN * Loader::KB;  // bytes of one K tile in LDS
  __shared__ __attribute__((aligned(16))) uint8_t smem_k[2][KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t smem_v[2][BN * D];
  const int32_t* hdr = p.blob;
  if (hdr[H_NONCE_LO] != (int32_t)p.nonce_lo || hdr[H_NONCE_HI] != (int32_t)p.nonce_hi) return;
  const int32_t* it = p.blob + hdr[H_OFF_ITEMS] + (size_t)blockIdx.x * kItemInts;
  const int head = it[0];
  if (head < 0) return;  // idle slot of the XCD interleave
  const int q_row0 = it[1], q_rows = it[2], kt0 = it[3], kt1 = it[4], slot = it[5], qsb = it[6];
  const int32_t* tiles = p.blob + hdr[H_OFF_TILES];
  const int H = p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int qr = wave * 32 + l32;  // this lane's query row inside the tile
  const bool wave_active = wave * 32 < q_rows;
  const bool ok = qr < q_rows;

  // Q^T as the B operand of S^T = K.Q^T.  bf16: lane holds query qr, channels 16*ks + 8*hi .. +7.
  // e4m3: channels 64*ks + 32*hi .. +31.
  constexpr int QREGS = FP8 ? D / 64 : D / 16;
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type QVec;
  QVec qf[QREGS];
  float c_lane = p.c;  // per-lane score multiplier: softmax scale * log2(e) [* Q block scale]
  {
    const size_t qoff = ((size_t)(q_row0 + (ok ? qr : 0)) * H + head) * D;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      QVec z = {};
      if constexpr (FP8) {
        if (ok) {
          const i32x4* src = reinterpret_cast<const i32x4*>(p.q8 + qoff + 64 * ks + 32 * hi);
          z = __builtin_shufflevector(src[0], src[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
        qf[ks] = z;
      } else {
        qf[ks] = ok ? *reinterpret_cast<const bf16x8*>(p.q + qoff + 16 * ks + 8 * hi) : z;
      }
    }
    if constexpr (FP8) c_lane *= ok ? p.q_scale[(size_t)(qsb + qr / 64) * H + head] : 1.f;
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[cb][i] = 0.f;
  // Running max m is kept in exp2 units (already multiplied by the score multiplier).
  float m = -INFINITY, l = 0.f;
  const uint8_t* kbase = FP8 ? p.k8 : reinterpret_cast<const uint8_t*>(p.k);

  Loader ld;
  ld.load(kbase, p.v, tiles[2 * kt0], tiles[2 * kt0 + 1], head, H);
  ld.store(smem_k[0], smem_v[0]);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool has_next = kt + 1 < kt1;
    if (has_next) ld.load(kbase, p.v, tiles[2 * kt + 2], tiles[2 * kt + 3], head, H);
    const int nvalid = tiles[2 * kt + 1];
    float cm = c_lane;
    if constexpr (FP8) cm *= p.k_scale[(size_t)(tiles[2 * kt] / 64) * H + head];
    if (wave_active) {
      const uint8_t* sk = smem_k[buf];
      const uint16_t* sv = smem_v[buf];
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
        const int krow = 32 * kb + sigma(l32);
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks) {
          if constexpr (FP8) {
            const int g0 = 4 * ks + 2 * hi;
            const i32x4 a0 = *reinterpret_cast<const i32x4*>(sk + Loader::kswz_off(krow, g0));
            const i32x4 a1 = *reinterpret_cast<const i32x4*>(sk + Loader::kswz_off(krow, g0 + 1));
            const i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
            s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 0, 0, 0, 0);
          } else {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sk + Loader::kswz_off(krow, 2 * ks + hi));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
          }
        }
      }
      if (nvalid < BN) {  // ragged last tile of a chunk: keys past its end do not exist
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb + 16 * (i / 8) + 8 * hi + (i % 8) >= nvalid) s[kb][i] = -INFINITY;
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = pair_max(mx) * cm;  // cm > 0, so scaling commutes with the max
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      // P = exp2(s * cm - m) rounded to bf16; the row sum is taken over the same rounded values
      // (v_dot2 with ones), so the weights that multiply V sum exactly to the normaliser.
      float rs0 = 0.f, rs1 = 0.f;
      bf16x8 pb[4];
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const int kb = k2 >> 1, b = 8 * (k2 & 1);
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = fast_exp2(fmaf(s[kb][b + j], cm, -m_new));
        pb[k2] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[k2], pb[k2], 0, 1), ones, rs0, false);
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[k2], pb[k2], 2, 3), ones, rs1, false);
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[k2], pb[k2], 4, 5), ones, rs0, false);
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[k2], pb[k2], 6, 7), ones, rs1, false);
      }
      l = l * alpha + (rs0 + rs1);
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
      const int t = lane & 15, G = lane >> 4;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const int row = 16 * k2 + 8 * hi + (t >> 2);
          const int col = 32 * cb + 16 * (G & 1) + 4 * (t & 3);
          const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(sv + lds_off<D>(row, col)));
          const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(sv + lds_off<D>(row + 4, col)));
          // whole-vector concatenation: element-wise 16-bit inserts are lowered wrongly by this
          // compiler (they reuse the first dword of each transposed read)
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[k2], o[cb], 0, 0, 0);
        }
      }
    }
    if (has_next) ld.store(smem_k[buf ^ 1], smem_v[buf ^ 1]);
    __syncthreads();
  }

  if (!wave_active) return;
  const float lt = pair_sum(l);
  const float inv = 1.f / lt;
  if (!ok) return;
  // m is log2 of the largest exp(scale * s); lse = m * ln(2) + ln(l)
  const float lse_val = m * 0.6931471805599453f + logf(lt);
  if (slot < 0) {
    const size_t rowoff = ((size_t)(q_row0 + qr) * H + head) * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * cb + 8 * g4 + 4 * hi;
        const float v0 = o[cb][4 * g4] * inv, v1 = o[cb][4 * g4 + 1] * inv;
        const float v2 = o[cb][4 * g4 + 2] * inv, v3 = o[cb][4 * g4 + 3] * inv;
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + rowoff + d0) = make_float4(v0, v1, v2, v3);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + rowoff + d0) =
              make_uint2(pack2_bf16(v0, v1), pack2_bf16(v2, v3));
        }
      }
    if (p.lse && hi == 0) p.lse[(size_t)head * p.lq + q_row0 + qr] = lse_val;
  } else {
    float* po = p.part_o + ((size_t)slot * BM + qr) * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * cb + 8 * g4 + 4 * hi;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(o[cb][4 * g4] * inv, o[cb][4 * g4 + 1] * inv, o[cb][4 * g4 + 2] * inv, o[cb][4 * g4 + 3] * inv);
      }
    if (hi == 0) p.part_lse[(size_t)slot * BM + qr] = lse_val;
  }
}

// Merge of split key ranges (a9): out = sum_k exp(lse_k - lse) * O_k, lse = log sum_k exp(lse_k).
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
  const int32_t* hdr = p.blob;
  if (hdr[H_NONCE_LO] != (int32_t)p.nonce_lo || hdr[H_NONCE_HI] != (int32_t)p.nonce_hi) return;
  const int32_t* g = p.blob + hdr[H_OFF_GROUPS] + (size_t)blockIdx.x * kGroupInts;
  const int head = g[0], q_row0 = g[1], rows = g[2], slot0 = g[3], parts = g[4];
  for (int idx = threadIdx.x; idx < rows * (D / 4); idx += blockDim.x) {
    const int r = idx / (D / 4), d4 = idx % (D / 4);
    float mx = -INFINITY;
    for (int k = 0; k < parts; ++k) mx = fmaxf(mx, p.part_lse[(size_t)(slot0 + k) * BM + r]);
    float z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < parts; ++k) {
      const float w = expf(p.part_lse[(size_t)(slot0 + k) * BM + r] - mx);
      const float4 v = *reinterpret_cast<const float4*>(p.part_o + ((size_t)(slot0 + k) * BM + r) * D + 4 * d4);
      z += w;
      acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
    }
    const float iz = 1.f / z;
    const size_t off = ((size_t)(q_row0 + r) * p.H + head) * D + 4 * d4;
    if constexpr (OUT_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) = make_float4(acc.x * iz, acc.y * iz, acc.z * iz, acc.w * iz);
    } else {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) =
          make_uint2(pack2_bf16(acc.x * iz, acc.y * iz), pack2_bf16(acc.z * iz, acc.w * iz));
    }
    if (p.lse && d4 == 0) p.lse[(size_t)head * p.lq + q_row0 + r] = mx + logf(z);
  }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(in)[i];
    reinterpret_cast<uint2*>(out)[i] = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
  }
}

}  // namespace

hipError_t launch_attn_bf16(const FwdParams& p, int head_dim, bool out_f32, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<128, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false, false>), dim3(grid), dim3(NTHR), 0, s, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<64, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false, false>), dim3(grid), dim3(NTHR), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const FwdParams& p, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((attn_fwd_kernel<128, true, false>), dim3(grid), dim3(NTHR), 0, s, p);
  else hipLaunchKernelGGL((attn_fwd_kernel<64, true, false>), dim3(grid), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine(const FwdParams& p, int head_dim, bool out_f32, int groups, hipStream_t s) {
  if (groups <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(groups), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<128, false>), dim3(groups), dim3(256), 0, s, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(groups), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<64, false>), dim3(groups), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;  // n is a multiple of head_dim, hence of 4
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, in, out, n4);
  return hipGetLastError();
}

}  // namespace wfattn
