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

constexpr int BM = kBlockM;  // 256 query rows per workgroup
constexpr int BN = kBlockN;  // 64 keys per tile
constexpr int NTHR = 256;    // 4 waves of 64

// Row of the K tile that lane row r of the S^T A-operand reads: bits 2 and 3 swapped.  With it,
// accumulator register i of lane l holds key 16*(i/8) + 8*(l/32) + i%8 of the 32-key block.
__device__ __forceinline__ int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Global -> LDS staging of one key tile, K (bf16 rows of 2*D bytes, or e4m3 rows of D bytes) and
// V (bf16), with global_load_lds_dwordx4: lane i of a wave's load fills bytes [16i, 16i+16) of a
// contiguous 1 KB run of the tile, so the swizzle is applied on the global side (the lane that
// fills physical granule p of row r fetches logical granule p ^ f(r)).  Rows past the tile's valid
// keys re-read the last valid row: finite data whose scores are masked to -inf and whose V rows
// then carry weight 0, so the pool's padding slots are never read.
template <int D, bool FP8>
struct TileLoader {
  static constexpr int KB = FP8 ? D : 2 * D;    // bytes per K row
  static constexpr int KG = KB / 16;            // 16-byte granules per K row
  static constexpr int VG = D / 8;              // 16-byte granules per V row
  static constexpr int KI = BN * KB / 1024 / 4; // 1 KB loads per wave for K
  static constexpr int VI = BN * D * 2 / 1024 / 4;

  // Byte offset of granule g of K row r.  bf16: the same swizzle as V.  e4m3: rows are D bytes,
  // so 256/D rows share one 64-bank line; XOR with (r / (256/D)) spreads 16 rows of one granule
  // column over distinct banks.
  __device__ __forceinline__ static int kswz(int r, int g) {
    if constexpr (FP8) return g ^ ((r / (256 / D)) & (KG - 1));
    else return swz<D>(r, g);
  }
  __device__ __forceinline__ static int kswz_off(int r, int g) { return r * KB + kswz(r, g) * 16; }

  // The fills are written as inline asm so that the compiler does not treat them as LDS stores:
  // it would otherwise wait for every in-flight fill (of the other buffer) before each LDS read
  // of this tile.  Completion is awaited explicitly by lds_fill_barrier().  M0 carries the LDS
  // destination of global_load_lds; nothing else in these kernels uses M0.
  __device__ __forceinline__ static void dma16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory");
  }
  __device__ __forceinline__ static void issue(const uint8_t* __restrict__ k, const uint16_t* __restrict__ v, int row0,
                                               int nvalid, int head, int H, uint32_t sk, uint32_t sv) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int chunk = (wave * KI + j) * 64 + lane;
      const int row = chunk / KG, g = kswz(row, chunk % KG);
      const int src_row = row < nvalid ? row : nvalid - 1;
      dma16(k + ((size_t)(row0 + src_row) * H + head) * KB + g * 16, __builtin_amdgcn_readfirstlane(sk + (wave * KI + j) * 1024));
    }
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int chunk = (wave * VI + j) * 64 + lane;
      const int row = chunk / VG, g = swz<D>(row, chunk % VG);
      const int src_row = row < nvalid ? row : nvalid - 1;
      dma16(v + ((size_t)(row0 + src_row) * H + head) * D + g * 8, __builtin_amdgcn_readfirstlane(sv + (wave * VI + j) * 1024));
    }
  }
};

// Wait for this wave's outstanding global loads (the LDS fills), then the workgroup barrier.
__device__ __forceinline__ void lds_fill_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// One segment: the key tiles [kt0, kt1) of one item (head, query tile of up to 256 rows).  Wave w
// owns query rows 64w .. 64w+63 as two 32-row blocks; every K and V^T operand read from LDS feeds
// one MFMA per block.  FP8: Q and K are e4m3 codes with one fp32 scale per (64-row block, head);
// the product of the two block scales and the softmax scale multiplies the fp32 accumulator
// once, and P.V stays bf16.
//
// Softmax reference.  P = exp2(s*c - m) against a per-row reference m in exp2 units, fixed from
// the first tile of the segment (that tile computes its max before its exponentials).  Later
// tiles therefore need no max before P, so their exponentials overlap the score MFMAs, and O is
// never rescaled inside the key loop.  Any reference works as long as no P overflows: the true
// running max is tracked, and if some score exceeded m by more than 2^64 (P could have
// overflowed, which needs scores to jump by more than 44 natural-log units after the first
// tile) the whole segment is recomputed with m set to that max, which no score exceeds.
template <int D, bool FP8, bool OUT_F32>
__device__ __forceinline__ void run_segment(const FwdParams& p, const int32_t* items, int item, int kt0, int kt1,
                                            int slot, const int32_t* tiles,
                                            uint8_t (*smem_k)[BN * TileLoader<D, FP8>::KB], uint16_t (*smem_v)[BN * D],
                                            int* redo_flags) {
  using Loader = TileLoader<D, FP8>;
  const int head = ld_const(items, item * kItemInts + 0), q_row0 = ld_const(items, item * kItemInts + 1);
  const int q_rows = ld_const(items, item * kItemInts + 2), qsb = ld_const(items, item * kItemInts + 3);
  const int H = p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const bool wave_active = 64 * wave < q_rows;

  // Q^T as the B operand of S^T = K.Q^T.  bf16: lane holds query row r, channels 16*ks + 8*hi .. +7;
  // e4m3: channels 64*ks + 32*hi .. +31.
  constexpr int QREGS = FP8 ? D / 64 : D / 16;
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type QVec;
  QVec qf[2][QREGS];
  float cq[2];  // per-lane score multiplier: softmax scale * log2(e) [* Q block scale]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = 64 * wave + 32 * qb + l32;
    const bool ok = r < q_rows;
    const size_t qoff = ((size_t)(q_row0 + (ok ? r : 0)) * H + head) * D;
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) {
      QVec z = {};
      if constexpr (FP8) {
        if (ok) {
          const i32x4* src = reinterpret_cast<const i32x4*>(p.q8 + qoff + 64 * ks + 32 * hi);
          z = __builtin_shufflevector(src[0], src[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
        qf[qb][ks] = z;
      } else {
        qf[qb][ks] = ok ? *reinterpret_cast<const bf16x8*>(p.q + qoff + 16 * ks + 8 * hi) : z;
      }
    }
    cq[qb] = p.c;
    if constexpr (FP8) cq[qb] *= ok ? p.q_scale[(size_t)(qsb + r / 64) * H + head] : 1.f;
  }
  const uint8_t* kbase = FP8 ? p.k8 : reinterpret_cast<const uint8_t*>(p.k);

  f32x16 o[2][D / 32];  // in AGPRs (see mfma_acc_agpr)
  float m[2], l[2];     // reference max (exp2 units) and this lane's half of the row sum
  float mr[2];          // running max of the scaled scores, for the overflow check
  // LDS byte addresses of the two buffers, for the fills
  const uint32_t ska0 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_k[0], ska1 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_k[1];
  const uint32_t sva0 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_v[0], sva1 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_v[1];

  // S^T = K.Q^T for both query blocks over one 64-key tile in LDS; keys past nvalid get -inf.
  auto scores = [&](const uint8_t* sk, int nvalid, f32x16 (&s)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[qb][kb][i] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int krow = 32 * kb + sigma(l32);
      if constexpr (FP8) {
        i32x8 a[QREGS];
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks) {
          const int g0 = 4 * ks + 2 * hi;
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(sk + Loader::kswz_off(krow, g0));
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(sk + Loader::kswz_off(krow, g0 + 1));
          a[ks] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks) {
          s[0][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[ks], qf[0][ks], s[0][kb], 0, 0, 0, 0, 0, 0);
          s[1][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[ks], qf[1][ks], s[1][kb], 0, 0, 0, 0, 0, 0);
        }
      } else {
        bf16x8 a[QREGS];
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks)
          a[ks] = *reinterpret_cast<const bf16x8*>(sk + Loader::kswz_off(krow, 2 * ks + hi));
#pragma unroll
        for (int ks = 0; ks < QREGS; ++ks) {
          s[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[0][ks], s[0][kb], 0, 0, 0);
          s[1][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[1][ks], s[1][kb], 0, 0, 0);
        }
      }
    }
    if (nvalid < BN) {  // last tile of a chunk: keys past its end do not exist
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb + 16 * (i / 8) + 8 * hi + (i % 8) >= nvalid) s[qb][kb][i] = -INFINITY;
    }
  };
  // max over this lane's 32 scores of one query block, times the score multiplier
  auto lane_max = [&](const f32x16 (&sq)[2], float mult) {
    float a0 = max3(sq[0][0], sq[0][1], sq[0][2]), a1 = max3(sq[0][3], sq[0][4], sq[0][5]);
    float a2 = max3(sq[1][0], sq[1][1], sq[1][2]), a3 = max3(sq[1][3], sq[1][4], sq[1][5]);
#pragma unroll
    for (int i = 6; i < 16; i += 2) {
      a0 = max3(a0, sq[0][i], sq[0][i + 1]);
      a2 = max3(a2, sq[1][i], sq[1][i + 1]);
    }
    return max3(a1, a3, fmaxf(a0, a2)) * mult;
  };

  int cur_row0, cur_nv, nxt_row0, nxt_nv;  // tile descriptors, read one tile ahead

  // One key tile: compute from buffer `buf` while the other buffer fills with the next tile.
  // Order inside the tile (one wave, two query blocks):
  //   scores of keys 0-31, then keys 32-63 (K operands shared by both blocks)
  //   P of keys 0-31 (overlaps the second half of the score MFMAs)
  //   P.V of keys 0-31, interleaved region by region with P of keys 32-63
  //   P.V of keys 32-63
  // The P.V MFMAs are inline asm (see mfma_acc_agpr), which the scheduler cannot interleave with
  // VALU on its own, so the regions are fenced with sched_barrier.
  auto tile = [&](int kt, int buf) {
    const bool has_next = kt + 1 < kt1;
    // the other buffer was last read before the previous barrier: refill it now, wait at the end
    if (has_next) Loader::issue(kbase, p.v, nxt_row0, nxt_nv, head, H, buf ? ska0 : ska1, buf ? sva0 : sva1);
    int n2_row0 = 0, n2_nv = 0;
    if (kt + 2 < kt1) {
      n2_row0 = ld_const(tiles, 2 * kt + 4);
      n2_nv = ld_const(tiles, 2 * kt + 5);
    }
    float ksc = 1.f;
    if constexpr (FP8) ksc = ld_const(p.k_scale, (cur_row0 / 64) * H + head);
    if (wave_active) {
      f32x16 s[2][2];  // [query block][32-key block]
      float cm[2];
      // P = exp2(s * cm - m) rounded to bf16, 8 keys (one MFMA k-step) at a time; the row sum is
      // taken over the same rounded values (v_dot2 with ones), so the weights that multiply V
      // sum exactly to the normaliser.
      bf16x8 pb[2][4];
      float rs[2] = {0.f, 0.f};
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
      auto make_p = [&](int qb, int k2) {
        const int kb = k2 >> 1, b = 8 * (k2 & 1);
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = fast_exp2(fmaf(s[qb][kb][b + j], cm[qb], -m[qb]));
        pb[qb][k2] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        float r = rs[qb];
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 0, 1), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 2, 3), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 4, 5), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 6, 7), ones, r, false);
        rs[qb] = r;
      };
      // front half (does not touch O): scores, running max, P of keys 0-31; specialised for the
      // ragged last tile of a chunk so that the common tile has no masking branch inside
      auto front = [&](auto ragged) {
        scores(smem_k[buf], decltype(ragged)::value ? cur_nv : BN, s);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          cm[qb] = cq[qb] * ksc;  // > 0, so scaling commutes with the max
          mr[qb] = fmaxf(mr[qb], lane_max(s[qb], cm[qb]));
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          make_p(qb, 0);
          make_p(qb, 1);
        }
      };
      if (cur_nv < BN) front(std::integral_constant<bool, true>());
      else front(std::integral_constant<bool, false>());
      const uint16_t* sv = smem_v[buf];
      const int t = lane & 15, G = lane >> 4;
      // V^T operand of (d block cb, key step k2) through two transposed LDS reads
      auto v_op = [&](int cb, int k2) {
        const int row = 16 * k2 + 8 * hi + (t >> 2);
        const int col = 32 * cb + 16 * (G & 1) + 4 * (t & 3);
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(sv + lds_off<D>(row, col)));
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(sv + lds_off<D>(row + 4, col)));
        // whole-vector concatenation: element-wise 16-bit inserts are lowered wrongly by this
        // compiler (they reuse the first dword of each transposed read)
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 va[D / 32][2];
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        va[cb][0] = v_op(cb, 0);
        va[cb][1] = v_op(cb, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // P.V of keys 0-31 (k2 = 0, 1), each pair of MFMAs followed by a quarter of one query
      // block's P for keys 32-63
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          mfma_acc_agpr(o[0][cb], va[cb][k2], pb[0][k2]);
          mfma_acc_agpr(o[1][cb], va[cb][k2], pb[1][k2]);
          const int u = 2 * cb + k2;  // 0..7 for d = 128: (qb, k2') = (u / 4, 2 + (u / 2) % 2)
          if constexpr (D == 128) {
            if ((u & 1) == 0) make_p(u >> 2, 2 + ((u >> 1) & 1));
          } else {
            make_p(u >> 1, 2 + (u & 1));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P.V of keys 32-63
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const bf16x8 a2 = v_op(cb, 2), a3 = v_op(cb, 3);
        mfma_acc_agpr(o[0][cb], a2, pb[0][2]);
        mfma_acc_agpr(o[1][cb], a2, pb[1][2]);
        mfma_acc_agpr(o[0][cb], a3, pb[0][3]);
        mfma_acc_agpr(o[1][cb], a3, pb[1][3]);
      }
      l[0] += rs[0];
      l[1] += rs[1];
    }
    lds_fill_barrier();
    cur_row0 = nxt_row0;
    cur_nv = nxt_nv;
    nxt_row0 = n2_row0;
    nxt_nv = n2_nv;
  };

  // Pass 0 takes its reference from the first tile; pass 1 (rare) uses the true max of pass 0.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qb][cb][i] = 0.f;
        mfma_drain(o[qb][cb]);  // VALU writes before the first MFMA that reads them
      }
      l[qb] = 0.f;
    }
    cur_row0 = ld_const(tiles, 2 * kt0);
    cur_nv = ld_const(tiles, 2 * kt0 + 1);
    nxt_row0 = 0;
    nxt_nv = 0;
    if (kt0 + 1 < kt1) {
      nxt_row0 = ld_const(tiles, 2 * kt0 + 2);
      nxt_nv = ld_const(tiles, 2 * kt0 + 3);
    }
    Loader::issue(kbase, p.v, cur_row0, cur_nv, head, H, ska0, sva0);
    lds_fill_barrier();
    if (pass == 0 && wave_active) {
      // the reference: the max of the first tile (its scores are recomputed by the loop)
      float ksc = 1.f;
      if constexpr (FP8) ksc = ld_const(p.k_scale, (cur_row0 / 64) * H + head);
      f32x16 s[2][2];
      scores(smem_k[0], cur_nv, s);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        m[qb] = pair_max(lane_max(s[qb], cq[qb] * ksc));
        mr[qb] = m[qb];
      }
    }
    for (int kt = kt0; kt < kt1; ++kt) tile(kt, (kt - kt0) & 1);
    // Did any score exceed the reference by more than 2^64?  Decided for the whole workgroup, so
    // that every wave runs the same number of tiles (and barriers).
    bool redo = false;
    if (wave_active && pass == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        mr[qb] = pair_max(mr[qb]);
        redo = redo || (mr[qb] > m[qb] + 64.f);
      }
    }
    const bool wave_redo = __any(redo);
    if (lane == 0) redo_flags[wave] = wave_redo ? 1 : 0;
    __syncthreads();
    const bool any_redo = (redo_flags[0] | redo_flags[1] | redo_flags[2] | redo_flags[3]) != 0;
    __syncthreads();  // flags are rewritten by the next segment
    if (!any_redo) break;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) m[qb] = mr[qb];
  }

  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) mfma_drain(o[qb][cb]);
    const int r = 64 * wave + 32 * qb + l32;
    const float lt = pair_sum(l[qb]);
    const float inv = 1.f / lt;
    if (r >= q_rows) continue;
    // m is log2 of the reference exp(scale * s); lse = m * ln(2) + ln(l)
    const float lse_val = m[qb] * 0.6931471805599453f + logf(lt);
    if (slot < 0) {
      const size_t rowoff = ((size_t)(q_row0 + r) * H + head) * D;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * cb + 8 * g4 + 4 * hi;
          const float v0 = o[qb][cb][4 * g4] * inv, v1 = o[qb][cb][4 * g4 + 1] * inv;
          const float v2 = o[qb][cb][4 * g4 + 2] * inv, v3 = o[qb][cb][4 * g4 + 3] * inv;
          if constexpr (OUT_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + rowoff + d0) = make_float4(v0, v1, v2, v3);
          } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + rowoff + d0) =
                make_uint2(pack2_bf16(v0, v1), pack2_bf16(v2, v3));
          }
        }
      if (p.lse && hi == 0) p.lse[(size_t)head * p.lq + q_row0 + r] = lse_val;
    } else {
      float* po = p.part_o + ((size_t)slot * BM + r) * D;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * cb + 8 * g4 + 4 * hi;
          *reinterpret_cast<float4*>(po + d0) = make_float4(o[qb][cb][4 * g4] * inv, o[qb][cb][4 * g4 + 1] * inv,
                                                            o[qb][cb][4 * g4 + 2] * inv, o[qb][cb][4 * g4 + 3] * inv);
        }
      if (hi == 0) p.part_lse[(size_t)slot * BM + r] = lse_val;
    }
  }
}

// Persistent workgroup: runs the segments [ranges[2w], ranges[2w+1]) of the uploaded schedule.
template <int D, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(NTHR, 1) void attn_fwd_kernel(FwdParams p) {
  using Loader = TileLoader<D, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem_k[2][BN * Loader::KB];
  __shared__ __attribute__((aligned(16))) uint16_t smem_v[2][BN * D];
  __shared__ int redo_flags[NTHR / 64];
  const int32_t* hdr = p.blob;
  if (ld_const(hdr, H_NONCE_LO) != (int32_t)p.nonce_lo || ld_const(hdr, H_NONCE_HI) != (int32_t)p.nonce_hi) return;
  const int32_t* rg = p.blob + ld_const(hdr, H_OFF_RANGES);
  const int s0 = ld_const(rg, 2 * (int)blockIdx.x), s1 = ld_const(rg, 2 * (int)blockIdx.x + 1);
  const int32_t* segs = p.blob + ld_const(hdr, H_OFF_SEGS);
  const int32_t* items = p.blob + ld_const(hdr, H_OFF_ITEMS);
  const int32_t* tiles = p.blob + ld_const(hdr, H_OFF_TILES);
  for (int sg = s0; sg < s1; ++sg) {
    run_segment<D, FP8, OUT_F32>(p, items, ld_const(segs, sg * kSegInts), ld_const(segs, sg * kSegInts + 1),
                                 ld_const(segs, sg * kSegInts + 2), ld_const(segs, sg * kSegInts + 3), tiles, smem_k, smem_v, redo_flags);
  }
}

// Merge of split key ranges: out = sum_k exp(lse_k - lse) * O_k, lse = log sum_k exp(lse_k).  One
// thread per (row, 4 channels); a block covers 256 / (D/4) rows of one merge group.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
  constexpr int RPB = 256 / (D / 4);  // rows per block
  const int32_t* hdr = p.blob;
  if (ld_const(hdr, H_NONCE_LO) != (int32_t)p.nonce_lo || ld_const(hdr, H_NONCE_HI) != (int32_t)p.nonce_hi) return;
  const int grp = blockIdx.x / (BM / RPB), rblk = blockIdx.x % (BM / RPB);
  const int32_t* g = p.blob + ld_const(hdr, H_OFF_GROUPS) + (size_t)grp * kGroupInts;
  const int32_t* it = p.blob + ld_const(hdr, H_OFF_ITEMS) + (size_t)g[0] * kItemInts;
  const int head = it[0], q_row0 = it[1], rows = it[2], slot0 = g[1], parts = g[2];
  const int r = rblk * RPB + threadIdx.x / (D / 4), d4 = threadIdx.x % (D / 4);
  if (r >= rows) return;
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
  const unsigned blocks = (unsigned)groups * (BM / (256 / (head_dim / 4)));
  if (head_dim == 128) {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<128, false>), dim3(blocks), dim3(256), 0, s, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<64, false>), dim3(blocks), dim3(256), 0, s, p);
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
