// attn_fwd.hip -- block-causal chunk attention forward on gfx950 MFMA (bf16, or e4m3 for the
// scores), the merge of split key ranges, and the fp32 -> bf16 staging of fp32 I/O.
//
// What one workgroup computes: segments of work items, one item = (head, query tile of up to
// 256 rows of one query chunk, that chunk's visible key tiles).  The visible keys are the chunk's
// own tokens and every earlier, cleaner chunk's tokens (Wave Forcing project page, "01 - The
// design gap", directed frontier and "Key observation"); the planner has already reduced them to
// a list of 64-key tiles that never cross a page, so nothing here tests chunk visibility: masked
// tiles are simply not in the list.  Keys are read from the paged pool in place (project page,
// "03 - End-to-end KV transport", "Layout" panel).
//
// Data flow (4 waves, 64 query rows each, as two 32-row MFMA blocks):
//   K, V tiles [64 x d] : global -> LDS with global_load_lds_dwordx4, a ring of four buffers;
//                         each pair of key steps fills the two buffers the previous pair read
//   S^T = K . Q^T       : v_mfma_f32_32x32x16_bf16, K rows read from LDS in a bit-swapped order
//                         so each lane ends up owning 16 keys of one query
//   softmax             : P = exp2(S * c - m) in fp32 against a fixed per-row reference m
//   O^T += V^T . P^T    : P stays in registers as the B operand; V^T comes from LDS through
//                         ds_read_b64_tr_b16 transposed reads; O lives in AGPRs
//
// Kernel instances: head_dim 64 / 128 x {bf16 out, fp32 out, e4m3 scores, gated bf16 out, gated
// e4m3 scores}; a gated instance first checks, per item, the generation flags of the chunks it
// reads (gate_item).
//
// The key loop is software-pipelined in half tiles (32 keys).  One half step issues the score
// MFMAs of the next half and the P.V MFMAs of the previous half, one at a time, and between two
// MFMAs a few of the VALU operations that turn the current half's scores into P, so the matrix
// cores and the VALU work at the same time within the single wave of each SIMD.
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace wfattn {
namespace {

constexpr int BM = kBlockM;  // 256 query rows per workgroup
constexpr int BN = kBlockN;  // 64 keys per tile
constexpr int NTHR = 256;    // 4 waves of 64
constexpr int NBUF = 4;      // LDS ring depth (tiles)

// Row of the K tile that lane row r of the S^T A-operand reads: bits 2 and 3 swapped.  With it,
// accumulator register i of lane l holds key 16*(i/8) + 8*(l/32) + i%8 of the 32-key block.
__device__ __forceinline__ int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Calls f(integral_constant<int, i>) for i = B .. E-1, so that i is a constant expression.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// Global -> LDS staging of one key tile, K (bf16 rows of 2*D bytes, or e4m3 rows of D bytes) and
// V (bf16), with global_load_lds_dwordx4: lane i of a wave's load fills bytes [16i, 16i+16) of a
// contiguous 1 KB run of the tile, so the swizzle is applied on the global side (the lane that
// fills physical granule p of row r fetches logical granule p ^ f(r)).  The per-lane byte offsets
// relative to the tile's first pool row are fixed for a segment, so a fill is one scalar base
// address and one precomputed VGPR offset per load.  Rows past the tile's valid keys re-read the
// last valid row: finite data whose scores are masked to -inf and whose V rows then carry weight
// 0, so the pool's padding slots are never read.
//
// V8 (e4m3 V): a key tile's V is one contiguous block of the e4m3 V pool, [D channels][64 keys]
// of one head (the layout wfattn_quantize_v_fp8 writes, codes of keys past a chunk's end 0), so
// its fill is a plain copy of D*64 bytes with no ragged variant; rows of the LDS copy are channels.
template <int D, bool FP8, bool V8 = false>
struct TileLoader {
  static constexpr int KB = FP8 ? D : 2 * D;    // bytes per K row
  static constexpr int KG = KB / 16;            // 16-byte granules per K row
  static constexpr int VG = D / 8;              // 16-byte granules per V row
  static constexpr int VBYTES = V8 ? BN * D : BN * D * 2;  // bytes of one V tile
  static constexpr int KI = BN * KB / 1024 / 4; // 1 KB loads per wave for K
  static constexpr int VI = VBYTES / 1024 / 4;

  uint32_t koff[KI], voff[VI];
  int wave_u;  // wave index, uniform

  // Byte offset of granule g of K row r.  bf16: the same swizzle as V.  e4m3: rows are D bytes,
  // so 256/D rows share one 64-bank line; XOR with (r / (256/D)) spreads 16 rows of one granule
  // column over distinct banks.
  __device__ __forceinline__ static int kswz(int r, int g) {
    if constexpr (FP8) return g ^ ((r / (256 / D)) & (KG - 1));
    else return swz<D>(r, g);
  }
  __device__ __forceinline__ static int kswz_off(int r, int g) { return r * KB + kswz(r, g) * 16; }

  __device__ __forceinline__ static uint32_t k_src(int wave, int j, int lane, int nvalid, int head, int H) {
    const int chunk = (wave * KI + j) * 64 + lane;
    const int row = chunk / KG, g = kswz(row, chunk % KG);
    const int src = row < nvalid ? row : nvalid - 1;
    return (uint32_t)((src * H + head) * KB + g * 16);
  }
  __device__ __forceinline__ static uint32_t v_src(int wave, int j, int lane, int nvalid, int head, int H) {
    const int chunk = (wave * VI + j) * 64 + lane;
    if constexpr (V8) {  // row = channel, 4 granules of 16 keys; nvalid, head, H: see v_base
      const int c = chunk / 4;
      return (uint32_t)(c * 64 + v8swz(c, chunk % 4) * 16);
    } else {
      const int row = chunk / VG, g = swz<D>(row, chunk % VG);
      const int src = row < nvalid ? row : nvalid - 1;
      return (uint32_t)((src * H + head) * 2 * D + g * 16);
    }
  }
  // e4m3 V tile in LDS: row c (a channel) holds 64 key bytes as 4 granules, four rows per 256-byte
  // line of the 64 banks; physical granule p holds logical granule p ^ ((c / 4) mod 4), so the 16
  // lanes of one ds_read_b128 phase (channels c .. c+15, one logical granule) touch 16 distinct
  // 16-byte bank groups.
  __device__ __forceinline__ static int v8swz(int c, int g) { return g ^ ((c >> 2) & 3); }
  // first byte of the V tile whose first key is pool row row0
  __device__ __forceinline__ static const uint8_t* v_base(const uint8_t* vpool, int row0, int head, int H) {
    if constexpr (V8) return vpool + ((size_t)(row0 / 64) * H + head) * (size_t)(64 * D);
    else return vpool + (size_t)row0 * H * 2 * D;
  }

  __device__ __forceinline__ void init(int head, int H) {
    wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    set_k(BN, head, H);
    set_v(BN, head, H);
  }

  // koff / voff for a tile with nvalid valid keys (a chunk's last tile), in place; set_*(BN)
  // restores the full-tile offsets.
  __device__ __forceinline__ void set_k(int nvalid, int head, int H) {
#pragma unroll
    for (int j = 0; j < KI; ++j) koff[j] = k_src(wave_u, j, threadIdx.x & 63, nvalid, head, H);
  }
  __device__ __forceinline__ void set_v(int nvalid, int head, int H) {
#pragma unroll
    for (int j = 0; j < VI; ++j) voff[j] = v_src(wave_u, j, threadIdx.x & 63, nvalid, head, H);
  }

  // The fills are inline asm so that the compiler does not treat them as LDS stores: it would
  // otherwise wait for every in-flight fill before each LDS read.  Completion is awaited with
  // explicit vmcnt waits.  M0 carries the LDS destination of global_load_lds; nothing else in
  // these kernels uses M0.
  __device__ __forceinline__ static void dma16(uint32_t lds_addr, uint32_t off, const uint8_t* base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(off), "s"(base) : "memory");
  }
  // K of the tile whose first key is pool row row0, into the LDS buffer at byte address lds.
  __device__ __forceinline__ void fill_k(const uint8_t* kpool, int row0, int nvalid, int head, int H, uint32_t lds) const {
    const uint8_t* base = kpool + (size_t)row0 * H * KB;
    const int wave = wave_u;
    if (nvalid == BN) {
#pragma unroll
      for (int j = 0; j < KI; ++j) dma16(lds + (wave * KI + j) * 1024, koff[j], base);
    } else {
#pragma unroll
      for (int j = 0; j < KI; ++j)
        dma16(lds + (wave * KI + j) * 1024, k_src(wave, j, threadIdx.x & 63, nvalid, head, H), base);
    }
  }
  __device__ __forceinline__ void fill_v(const uint8_t* vpool, int row0, int nvalid, int head, int H, uint32_t lds) const {
    const uint8_t* base = v_base(vpool, row0, head, H);
    const int wave = wave_u;
    if (V8 || nvalid == BN) {
#pragma unroll
      for (int j = 0; j < VI; ++j) dma16(lds + (wave * VI + j) * 1024, voff[j], base);
    } else {
#pragma unroll
      for (int j = 0; j < VI; ++j)
        dma16(lds + (wave * VI + j) * 1024, v_src(wave, j, threadIdx.x & 63, nvalid, head, H), base);
    }
  }
};

// The VALU work that turns 32 scores per lane (2 query blocks x 16 keys) into bf16 P, as 80
// operations in a software-pipelined order: for element e, F(e) = fma(s, c, -m), X(e) = exp2, and
// per pair of elements C = convert to bf16x2.  Each operation depends only on operations at least
// two places earlier in the list, so any run of consecutive operations can be issued between two
// MFMAs without waiting on each other.  The row sums are taken separately, over the same
// bf16-rounded weights (so that the weights that multiply V sum exactly to the normaliser), with
// v_dot2 after the step's MFMAs: v_dot2 instructions do not issue while an MFMA is executing.
enum : int { OP_F = 0, OP_X = 1, OP_C = 2 };
constexpr int kValuOps = 80;
struct ValuProgram {
  int kind[kValuOps], idx[kValuOps];
  constexpr ValuProgram() : kind(), idx() {
    int n = 0;
    for (int s = 0; s < 36; ++s) {
      if (s < 32) { kind[n] = OP_F; idx[n] = s; ++n; }
      if (s >= 1 && s <= 32) { kind[n] = OP_X; idx[n] = s - 1; ++n; }
      if (s >= 3 && (s & 1) && (s - 3) / 2 < 16) { kind[n] = OP_C; idx[n] = (s - 3) / 2; ++n; }
    }
  }
};
constexpr ValuProgram kValu{};

// Order of the MFMAs inside a half step: NS score MFMAs spread evenly among NP P.V MFMAs.
__host__ __device__ constexpr bool region_is_s(int r, int ns, int np) {
  return ns > 0 && ((r + 1) * ns) / (ns + np) > (r * ns) / (ns + np);
}
__host__ __device__ constexpr int region_index(int r, int ns, int np) {  // index among its own kind
  int k = 0;
  for (int i = 0; i < r; ++i) k += region_is_s(i, ns, np) == region_is_s(r, ns, np);
  return k;
}
// VALU operations issued up to the start of region r, in proportion to the MFMA cycles of the
// regions before it (a score MFMA lasts ws times as long as a P.V MFMA: 2 for e4m3, 1 for bf16)
__host__ __device__ constexpr int valu_ops_before(int r, int ns, int np, int ws, int nops) {
  int w = 0, tot = 0;
  for (int i = 0; i < ns + np; ++i) {
    const int wi = region_is_s(i, ns, np) ? ws : 1;
    if (i < r) w += wi;
    tot += wi;
  }
  return (w * nops) / tot;
}
// first region that uses K operand ks (score MFMA 2*ks) or V operand t (P.V MFMA 2*t)
__host__ __device__ constexpr int k_first_use(int ks, int ns, int np) {
  for (int r = 0; r < ns + np; ++r)
    if (region_is_s(r, ns, np) && region_index(r, ns, np) == 2 * ks) return r;
  return 0;
}
__host__ __device__ constexpr int v_first_use(int t, int ns, int np) {
  for (int r = 0; r < ns + np; ++r)
    if (!region_is_s(r, ns, np) && region_index(r, ns, np) == 2 * t) return r;
  return 0;
}

// One segment: the key tiles [kt0, kt1) of one item (head, query tile of up to 256 rows).  Wave w
// owns query rows 64w .. 64w+63 as two 32-row blocks; every K and V^T operand read from LDS feeds
// one MFMA per block.  FP8: Q and K are e4m3 codes with one fp32 scale per (64-row block, head);
// the product of the two block scales and the softmax scale multiplies the fp32 accumulator
// once, and P.V stays bf16.
//
// Softmax reference.  P = exp2(s*c - m) against a per-row reference m in exp2 units, fixed from
// the first tile of the segment, so O is never rescaled inside the key loop and no running max is
// kept.  Any reference gives the exact softmax as long as no P overflows.  The row sum l bounds
// every P of the row; if some l reaches 2^64 (some score exceeded the first tile's max by more
// than 44 natural-log units) the segment is recomputed against the true row max, found by a
// score-only sweep, which no score exceeds.
//
// V8 (e4m3 K/V storage, with FP8): V tiles are e4m3 codes with one fp32 scale s_v per (64-key
// tile, head).  Each code converts exactly to bf16 and P.V stays a bf16 MFMA; the scale is folded
// into the weights instead, P' = exp2(s*c - (m - log2 s_v)) = s_v * P (one reference shift per
// tile and row), so sum_j P'_j code_j = sum_j P_j v_j, and the row sum adds each tile's sum of the
// rounded P' times 1/s_v, keeping l the sum of the weights that multiply V.
template <int D, bool FP8, bool OUT_F32, bool GATED, bool V8 = false>
__device__ __forceinline__ void run_segment(const FwdParams& p, const int32_t* items, int item, int kt0, int kt1,
                                            int slot, const int32_t* tiles,
                                            uint8_t (*smem_k)[BN * TileLoader<D, FP8, V8>::KB],
                                            uint8_t (*smem_v)[TileLoader<D, FP8, V8>::VBYTES], int* redo_flags) {
  static_assert(!V8 || (FP8 && !GATED && !OUT_F32), "e4m3 V comes with e4m3 scores, ungated, bf16 out");
  using Loader = TileLoader<D, FP8, V8>;
  constexpr int KI = Loader::KI, VI = Loader::VI;
  const int head = ld_const(items, item * kItemInts + 0), q_row0 = ld_const(items, item * kItemInts + 1);
  const int q_rows = ld_const(items, item * kItemInts + 2), qsb = ld_const(items, item * kItemInts + 3);
  const int H = p.H;
  // gated kernels: lane-dependent addressing is derived per segment (an opaque copy of the thread
  // index keeps the compiler from hoisting it out of the segment loop, where next to the gate's
  // registers it would spill)
  int tid = threadIdx.x;
  if constexpr (GATED) asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const bool wave_active = 64 * wave < q_rows;
  const int n = kt1 - kt0;

  Loader ld;
  ld.init(head, H);
  const uint8_t* kpool = FP8 ? p.k8 : reinterpret_cast<const uint8_t*>(p.k);
  const uint8_t* vpool = V8 ? p.v8 : reinterpret_cast<const uint8_t*>(p.v);
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
  // Q^T lives in AGPRs for the whole segment (read only by the score MFMAs)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < QREGS; ++ks) asm volatile("" : "+a"(qf[qb][ks]));

  // ---- operands ------------------------------------------------------------------------------
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type KVec;
  // K operand of score k-step ks for the 32 keys of half kb
  auto k_op = [&](const uint8_t* sk, int kb, int ks) -> KVec {
    const int krow = 32 * kb + sigma(l32);
    if constexpr (FP8) {
      const int g0 = 4 * ks + 2 * hi;
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(sk + Loader::kswz_off(krow, g0));
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(sk + Loader::kswz_off(krow, g0 + 1));
      return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *reinterpret_cast<const bf16x8*>(sk + Loader::kswz_off(krow, 2 * ks + hi));
    }
  };
  // V^T operand of (d block cb, 16-key step k2 of the tile) through two transposed LDS reads
  const int tq = lane & 15, G = lane >> 4;
  auto v_op = [&](const uint8_t* sv8, int cb, int k2) -> bf16x8 {
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(sv8);
    const int row = 16 * k2 + 8 * hi + (tq >> 2);
    const int col = 32 * cb + 16 * (G & 1) + 4 * (tq & 3);
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(sv + lds_off<D>(row, col)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(sv + lds_off<D>(row + 4, col)));
    // whole-vector concatenation: element-wise 16-bit inserts are lowered wrongly by this
    // compiler (they reuse the first dword of each transposed read)
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // e4m3 V^T operands of (d block cb, half h): one 16-byte read of channel 32cb + l32 holds the
  // keys of both 16-key steps of the half that this lane feeds (the V8 block stores each half's
  // 8-key groups in the order 0, 2, 1, 3): bytes 0-7 are keys 32h + 8hi + 0..7, bytes 8-15 keys
  // 32h + 16 + 8hi + 0..7.
  auto v8_raw = [&](const uint8_t* sv, int cb, int h) -> i32x4 {
    const int c = 32 * cb + l32;
    return *reinterpret_cast<const i32x4*>(sv + c * 64 + Loader::v8swz(c, 2 * h + hi) * 16);
  };
  // e4m3 codes -> bf16 (exact: 4 significant bits, exponents within bf16's range)
  auto v8_cvt = [&](const i32x4& r, bf16x8& a, bf16x8& b) {
    const bf16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[0], 1.f, false);
    const bf16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[0], 1.f, true);
    const bf16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[1], 1.f, false);
    const bf16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[1], 1.f, true);
    const bf16x2 w4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[2], 1.f, false);
    const bf16x2 w5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[2], 1.f, true);
    const bf16x2 w6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[3], 1.f, false);
    const bf16x2 w7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)r[3], 1.f, true);
    a = __builtin_shufflevector(__builtin_shufflevector(w0, w1, 0, 1, 2, 3), __builtin_shufflevector(w2, w3, 0, 1, 2, 3),
                                0, 1, 2, 3, 4, 5, 6, 7);
    b = __builtin_shufflevector(__builtin_shufflevector(w4, w5, 0, 1, 2, 3), __builtin_shufflevector(w6, w7, 0, 1, 2, 3),
                                0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Score MFMAs are inline asm so that Q^T can stay in AGPRs as their B operand (the builtins
  // would copy it into VGPRs, which the two score halves, P and the operands need).  The compiler
  // does not track their latency: every VALU read of a score follows score_drain() or enough
  // independent instructions (the pipelined loop reads a half's scores one half step later).
  auto s_mfma = [&](f32x16& acc, const KVec& a, int qb, int ks, auto firstc) {
    if constexpr (decltype(firstc)::value) {
      if constexpr (FP8) asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(qf[qb][ks]));
      else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(qf[qb][ks]));
    } else {
      if constexpr (FP8) asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(qf[qb][ks]));
      else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(qf[qb][ks]));
    }
  };
  // 24 wait states after the last score MFMA into s and before a VALU reads it (an 8-pass bf16
  // result needs 11, a 16-pass e4m3 one 19)
  auto score_drain = [&](f32x16 (&s)[2]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
  };

  // ---- softmax pieces ------------------------------------------------------------------------
  f32x16 o[2][D / 32];  // in AGPRs (see mfma_acc_agpr)
  float m[2], l[2];     // reference max (exp2 units) and this lane's half of the row sum
  auto clear_o = [&]() {
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
  };
  // keys of half kb at or past nvalid do not exist: their scores become -inf
  auto mask_half = [&](f32x16 (&s)[2], int kb, int nvalid) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + 16 * (i / 8) + 8 * hi + (i % 8) >= nvalid) s[qb][i] = -INFINITY;
  };
  // full score tile (both halves), used outside the pipelined loop
  auto scores_tile = [&](const uint8_t* sk, int nvalid, f32x16 (&s0)[2], f32x16 (&s1)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16(&s)[2] = kb ? s1 : s0;
      static_for<0, QREGS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        const KVec a = k_op(sk, kb, ks);
        s_mfma(s[0], a, 0, ks, std::integral_constant<bool, ks == 0>());
        s_mfma(s[1], a, 1, ks, std::integral_constant<bool, ks == 0>());
      });
    }
    score_drain(s0);
    score_drain(s1);
    if (nvalid < BN) {
      mask_half(s0, 0, nvalid);
      mask_half(s1, 1, nvalid);
    }
  };
  // max over this lane's 32 scores of one query block (two halves), times the score multiplier
  auto lane_max = [&](const f32x16& a, const f32x16& b, float mult) {
    float a0 = max3(a[0], a[1], a[2]), a1 = max3(a[3], a[4], a[5]);
    float a2 = max3(b[0], b[1], b[2]), a3 = max3(b[3], b[4], b[5]);
#pragma unroll
    for (int i = 6; i < 16; i += 2) {
      a0 = max3(a0, a[i], a[i + 1]);
      a2 = max3(a2, b[i], b[i + 1]);
    }
    return max3(a1, a3, fmaxf(a0, a2)) * mult;
  };

  // state of the VALU program for one half: exponent temporaries, packed pairs
  struct ValuState {
    float t[32];
    uint32_t pw[16];
  };
  // mo: the reference the exponent subtracts (m, or for e4m3 V the tile's shifted reference)
  auto valu_op = [&](auto kc, ValuState& st, const f32x16 (&s)[2], const float (&cm)[2], const float (&mo)[2]) {
    constexpr int k = decltype(kc)::value;
    constexpr int kind = kValu.kind[k], e = kValu.idx[k];
    if constexpr (kind == OP_F) {
      st.t[e] = fmaf(s[e >> 4][e & 15], cm[e >> 4], -mo[e >> 4]);
    } else if constexpr (kind == OP_X) {
      st.t[e] = fast_exp2(st.t[e]);
    } else {
      st.pw[e] = pack2_bf16(st.t[2 * e], st.t[2 * e + 1]);
    }
  };
  const bf16x2 ones2 = {(__bf16)1.f, (__bf16)1.f};
  // l += the sum of one half's bf16 weights (two v_dot2 chains per block: their latency).  Pairs
  // are taken with whole-vector shuffles: this compiler folds word extracts from a bit-cast
  // vector wrongly.
  auto row_sums = [&](const bf16x8 (&pb)[2][2], float isv) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 0, 1), ones2, a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 2, 3), ones2, a1, false);
        a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 4, 5), ones2, a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[qb][k2], pb[qb][k2], 6, 7), ones2, a1, false);
      }
      if constexpr (V8) l[qb] = fmaf(a0 + a1, isv, l[qb]);  // back from s_v * P to P
      else l[qb] += a0 + a1;
    }
  };
  auto anchor_l = [&]() { asm volatile("" ::"v"(l[0]), "v"(l[1])); };
  auto p_operands = [&](const ValuState& st, bf16x8 (&pb)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int b = 8 * qb + 4 * k2;
        const i32x4 w = {(int)st.pw[b], (int)st.pw[b + 1], (int)st.pw[b + 2], (int)st.pw[b + 3]};
        pb[qb][k2] = __builtin_bit_cast(bf16x8, w);
      }
  };
  // P for one half without interleaving (prologue)
  auto make_p_plain = [&](const f32x16 (&s)[2], const float (&cm)[2], const float (&mo)[2], float isv,
                          bf16x8 (&pb)[2][2]) {
    ValuState st;
    static_for<0, kValuOps>([&](auto kc) { valu_op(kc, st, s, cm, mo); });
    p_operands(st, pb);
    row_sums(pb, isv);
  };

  // One half step.  MFMAs: (if HAS_S) the scores of half kb_next from K buffer sk into s_next, and
  // the P.V of half `half` of the tile in V buffer sv with pb_in.  Between them, (if HAS_P) the VALU
  // program turning s_src into pb_out.
  constexpr int NS_FULL = 2 * QREGS;  // score MFMAs per half
  constexpr int NP = D / 8;           // P.V MFMAs per half: 2 blocks x D/32 x 2 k-steps
  constexpr int LA = 3;               // operand loads run this many MFMA regions ahead
  //
  // It also issues two groups of tile fills (global -> LDS, 1 KB per wave each; group g: ND_g loads,
  // offsets doff_g, LDS byte address dlds_g + 1024 j, global base dbase_g), spread evenly over its
  // MFMA regions so that the memory pipeline takes them in the background instead of stalling the
  // wave on a burst.
  auto half_step = [&](auto has_s, auto has_p, const uint8_t* sk, int kb_next, f32x16 (&s_next)[2],
                       const uint8_t* sv, int half, const bf16x8 (&pb_in)[2][2],
                       const f32x16 (&s_src)[2], const float (&cm)[2], const float (&mo)[2], bf16x8 (&pb_out)[2][2],
                       auto ndc, const uint32_t* doff, uint32_t dlds, const uint8_t* dbase,
                       auto ndc2, const uint32_t* doff2, uint32_t dlds2, const uint8_t* dbase2) {
    constexpr bool HS = decltype(has_s)::value, HP = decltype(has_p)::value;
    constexpr int ND1 = decltype(ndc)::value, ND = ND1 + decltype(ndc2)::value;
    constexpr int NS = HS ? NS_FULL : 0;
    constexpr int NR = NS + NP;
    constexpr int NKOP = HS ? QREGS : 0;  // K operands (each feeds both query blocks)
    constexpr int NVOP = NP / 2;          // V operands (each feeds both query blocks)
    KVec kop[QREGS];
    bf16x8 vop[NVOP];
    i32x4 vraw[NVOP / 2];  // e4m3 V: one read per d block feeds its two 16-key steps
    auto load_for = [&](auto rc) {  // operands whose first use is region r
      constexpr int r = decltype(rc)::value;
      static_for<0, NKOP>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (k_first_use(ks, NS, NP) == r) kop[ks] = k_op(sk, kb_next, ks);
      });
      static_for<0, NVOP>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (V8) {
          if constexpr ((t & 1) == 0 && v_first_use(t, NS, NP) == r) vraw[t >> 1] = v8_raw(sv, t >> 1, half);
        } else {
          if constexpr (v_first_use(t, NS, NP) == r) vop[t] = v_op(sv, t >> 1, 2 * half + (t & 1));
        }
      });
    };
    // e4m3 V: the conversion of the operands first used in region r, issued one region earlier
    // (the read went out LA regions earlier)
    auto conv_for = [&](auto rc) {
      constexpr int r = decltype(rc)::value;
      if constexpr (V8)
        static_for<0, NVOP>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          if constexpr ((t & 1) == 0 && v_first_use(t, NS, NP) == r) v8_cvt(vraw[t >> 1], vop[t], vop[t + 1]);
        });
    };
    ValuState st;
    static_for<0, LA>(load_for);
    conv_for(std::integral_constant<int, 0>());
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NR>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr int idx = region_index(r, NS, NP);
      if constexpr (region_is_s(r, NS, NP)) {
        constexpr int qb = idx & 1, ks = idx >> 1;
        s_mfma(s_next[qb], kop[ks], qb, ks, std::integral_constant<bool, ks == 0>());
      } else {
        constexpr int qb = idx & 1, t = idx >> 1;
        mfma_acc_agpr(o[qb][t >> 1], vop[t], pb_in[qb][t & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, ND>([&](auto dc) {
        constexpr int dj = decltype(dc)::value;
        if constexpr (((2 * dj + 1) * NR) / (2 * ND) == r) {
          if constexpr (dj < ND1) Loader::dma16(dlds + 1024 * dj, doff[dj], dbase);
          else Loader::dma16(dlds2 + 1024 * (dj - ND1), doff2[dj - ND1], dbase2);
        }
      });
      if constexpr (r + LA < NR) load_for(std::integral_constant<int, r + LA>());
      if constexpr (r + 1 < NR) conv_for(std::integral_constant<int, r + 1>());
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HP) {
        constexpr int WS = FP8 ? 2 : 1;
        static_for<valu_ops_before(r, NS, NP, WS, kValuOps), valu_ops_before(r + 1, NS, NP, WS, kValuOps)>(
            [&](auto kc) { valu_op(kc, st, s_src, cm, mo); });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (HP) {
      p_operands(st, pb_out);
      // Keep this step's VALU results in this step: without a use here the compiler may sink
      // them past a following branch into the next step, away from the MFMAs they overlap.
      asm volatile("" ::"v"(pb_out[0][0]), "v"(pb_out[0][1]), "v"(pb_out[1][0]), "v"(pb_out[1][1]));
      anchor_l();
    }
  };

  // ---- the key loop ------------------------------------------------------------------------
  // Ring: slot s (s >= -1) holds K of tile s+1 and V of tile s, in buffer (s+1) % 4.  Iteration j
  // reads slot j (scores of tile j+1, P.V of tile j).  Iterations come in pairs: the first of a
  // pair (j even) fills slots j+2 and j+3 into the two buffers the previous pair read; the second
  // waits for those loads and ends with the workgroup barrier, one per two key tiles.
  auto tix = [&](int j) { return 2 * (kt0 + j); };  // descriptor of the segment's j-th tile
  // Tile descriptors (first pool row, valid keys) are read with scalar loads one step before
  // they are needed, so no step waits on a scalar load.
  struct Desc {
    int row0, nv;
  };
  // Past the segment's end a descriptor repeats the segment's last tile: the constant-count fills
  // of the last steps then re-read keys this item is already reading, never a page of a chunk
  // outside its visible prefix (in gated kernels: never one whose flag it has not seen).
  auto load_desc = [&](int j) -> Desc {
    const int t = tix(j < n ? j : n - 1);
    return Desc{ld_const(tiles, t), ld_const(tiles, t + 1)};
  };
  // e4m3 key-block scale of the segment's tile j (one scale per 64-key tile and head: tiles
  // never cross a page and pages hold a multiple of 64 keys).  Ungated kernels read it through
  // the scalar cache, which is right for memory that no one writes during the launch.  In gated
  // kernels a producer may write the scales while the launch runs, so they are read like the
  // flags, with device-coherent vector loads: 64 tiles' scales at once, one per lane, each
  // 64-tile batch loaded when the walk first needs it, and picked out of the batch with a
  // readlane (a reload costs one vmcnt wait per 64 tiles).
  float sbatch = 1.f;
  int sb_cur = -1;
  auto coherent_scale = [&](int jt) -> float {
    const int row0 = tiles[tix(jt)];
    return __hip_atomic_load(p.k_scale + (size_t)(row0 / 64) * H + head, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto k_scale_of = [&](int j, const Desc& d) -> float {
    if constexpr (FP8 && GATED) {
      const int jt = j < n ? j : n - 1;
      const int b = jt >> 6;
      if (b != sb_cur) {
        const int jl = 64 * b + (threadIdx.x & 63);
        sbatch = jl < n ? coherent_scale(jl) : 1.f;
        sb_cur = b;
      }
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sbatch), jt & 63));
    } else if constexpr (FP8) {
      return ld_const(p.k_scale, (d.row0 / 64) * H + head);
    } else {
      return 1.f;
    }
  };
  // slot s: K of tile s+1 (descriptor dk) and V of tile s (descriptor dv), into buffer B
  auto fill_slot = [&](auto bufc, int s, const Desc& dk, const Desc& dv) {
    constexpr int B = decltype(bufc)::value;
    const uint32_t ka = (uint32_t)(uintptr_t)(WF_LDS void*)smem_k[B];
    const uint32_t va = (uint32_t)(uintptr_t)(WF_LDS void*)smem_v[B];
    if (s + 1 < n) ld.fill_k(kpool, dk.row0, dk.nv, head, H, ka);
    if (s >= 0 && s < n) ld.fill_v(vpool, dv.row0, dv.nv, head, H, va);
  };
  auto set_cm = [&](float ksc, float (&cm)[2]) {
    cm[0] = cq[0] * ksc;  // > 0, so scaling commutes with the max
    cm[1] = cq[1] * ksc;
  };
  // e4m3 V: the tile's V scale, the reference shifted by log2 of it, and its inverse
  auto v_scale_of = [&](const Desc& d) -> float {
    if constexpr (V8) return ld_const(p.v_scale, (d.row0 / 64) * H + head);
    else return 1.f;
  };
  auto set_mo = [&](float vsc, float (&mo)[2]) {
    const float lv = log2f(vsc);
    mo[0] = m[0] - lv;
    mo[1] = m[1] - lv;
  };

  bool fixed_m = false;  // pass 1: m already holds the true row max
  for (int pass = 0; pass < 2; ++pass) {
    clear_o();
    // prologue: slots -1, 0, 1 in flight; wait for slot -1 (K of tile 0)
    const Desc d0 = load_desc(0);
    Desc d1 = load_desc(1), d2 = load_desc(2), d3 = load_desc(3), d4 = load_desc(4);  // tiles j+1 .. j+4 of step j
    fill_slot(std::integral_constant<int, 0>(), -1, d0, d0);
    fill_slot(std::integral_constant<int, 1>(), 0, d1, d0);
    if (n > 1) fill_slot(std::integral_constant<int, 2>(), 1, d2, d1);
    {
      const bool k1 = n > 1, k2 = n > 2;  // loads issued after slot -1
      if (k2) wait_vmcnt<2 * KI + 2 * VI>();
      else if (k1) wait_vmcnt<KI + 2 * VI>();
      else wait_vmcnt<VI>();
    }
    __syncthreads();
    f32x16 s_a[2];      // scores of the current tile's second half
    bf16x8 p_a[2][2];   // P of the current tile's first half
    float cm_cur[2];
    set_cm(k_scale_of(0, d0), cm_cur);
    float ksc_nxt = k_scale_of(1, d1);
    float vsc_cur = v_scale_of(d0), vsc_nxt = v_scale_of(d1);
    float mo_cur[2];  // e4m3 V only
    int nv_cur = d0.nv;
    if (wave_active) {
      f32x16 s0[2];
      scores_tile(reinterpret_cast<const uint8_t*>(smem_k[0]), nv_cur, s0, s_a);
      if (!fixed_m) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) m[qb] = pair_max(lane_max(s0[qb], s_a[qb], cm_cur[qb]));
      }
      if constexpr (V8) set_mo(vsc_cur, mo_cur);
      make_p_plain(s0, cm_cur, V8 ? mo_cur : m, V8 ? 1.f / vsc_cur : 1.f, p_a);
    }
    wait_vmcnt<0>();  // slots 0 and 1: the first pair of iterations has no barrier between them
    __syncthreads();

    // iteration j reads slot j (buffer B = (j+1) % 4, a compile-time constant so that every LDS
    // address is a per-lane base plus an immediate offset).  FILL (j even): slot j+2 (K of tile
    // j+3, V of tile j+2) goes into buffer (B+2) % 4 during the first half step and slot j+3 (K of
    // tile j+4, V of tile j+3) into buffer (B+3) % 4 during the second.  Otherwise (j odd) the
    // iteration ends by waiting for those loads and with the barrier.  Past the segment's end the
    // descriptors repeat its last tile, so every pair issues the same number of (in-bounds) loads.
    auto step = [&](auto bufc, auto fillc, int j) {
      constexpr int B = decltype(bufc)::value;
      constexpr bool FILL = decltype(fillc)::value;
      // d4 was loaded during the previous step; using it only from here on keeps the compiler
      // from deriving values from it (and waiting for the load) right after the load.  The fill
      // descriptors are pinned to scalar registers here: the loop's four exits otherwise let the
      // compiler carry them around the loop in vector registers.
      auto pin = [](Desc& d) {
        d.row0 = __builtin_amdgcn_readfirstlane(d.row0);
        d.nv = __builtin_amdgcn_readfirstlane(d.nv);
        asm volatile("" : "+s"(d.row0), "+s"(d.nv));
      };
      pin(d2);
      pin(d3);
      pin(d4);
      constexpr int FB2 = (B + 2) % NBUF, FB3 = (B + 3) % NBUF;
      constexpr int NK = FILL ? KI : 0, NV = FILL ? VI : 0;
      const uint8_t* fkb2 = kpool + (size_t)d3.row0 * H * Loader::KB;
      const uint8_t* fvb2 = Loader::v_base(vpool, d2.row0, head, H);
      const uint8_t* fkb3 = kpool + (size_t)d4.row0 * H * Loader::KB;
      const uint8_t* fvb3 = Loader::v_base(vpool, d3.row0, head, H);
      const uint32_t fkl2 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_k[FB2] + ld.wave_u * KI * 1024;
      const uint32_t fvl2 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_v[FB2] + ld.wave_u * VI * 1024;
      const uint32_t fkl3 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_k[FB3] + ld.wave_u * KI * 1024;
      const uint32_t fvl3 = (uint32_t)(uintptr_t)(WF_LDS void*)smem_v[FB3] + ld.wave_u * VI * 1024;
      // rare: a chunk's last tile among those filled (an e4m3 V block is always whole: its tail
      // codes are 0); the fill offsets are patched for it and restored afterwards
      const int nk2 = d3.nv, nv2 = d2.nv, nk3 = d4.nv, nv3 = d3.nv;  // valid keys of the filled tiles
      bool k_ragged = false, v_ragged = false;
      auto patch = [&](int nk, int nv) {
        if (k_ragged) ld.set_k(BN, head, H);
        if (v_ragged) ld.set_v(BN, head, H);
        k_ragged = nk < BN;
        v_ragged = !V8 && nv < BN;
        if (k_ragged) ld.set_k(nk, head, H);
        if (v_ragged) ld.set_v(nv, head, H);
      };
      if constexpr (FILL) patch(nk2, nv2);
      // descriptors for the next step
      const Desc d5 = load_desc(j + 5);
      const float ksc_n2 = k_scale_of(j + 2, d2);
      const float vsc_n2 = v_scale_of(d2);
      const int nv_nxt = d1.nv;
      float cm_nxt[2], mo_nxt[2];
      set_cm(ksc_nxt, cm_nxt);
      if constexpr (V8) set_mo(vsc_nxt, mo_nxt);
      if (wave_active) {
        const uint8_t* sk = reinterpret_cast<const uint8_t*>(smem_k[B]);
        const uint8_t* sv = smem_v[B];
        if (nv_cur < BN) {  // tile j is a chunk's last, partial tile
          score_drain(s_a);
          mask_half(s_a, 1, nv_cur);
        }
        // A: scores of tile j+1 half 0; P.V of tile j half 0; P of tile j half 1
        f32x16 s_n0[2];
        bf16x8 p_1[2][2];
        half_step(std::true_type(), std::true_type(), sk, 0, s_n0, sv, 0, p_a, s_a, cm_cur, V8 ? mo_cur : m, p_1,
                  std::integral_constant<int, NK>(), ld.koff, fkl2, fkb2, std::integral_constant<int, NV>(), ld.voff,
                  fvl2, fvb2);
        if (nv_nxt < BN) {
          score_drain(s_n0);
          mask_half(s_n0, 0, nv_nxt);
        }
        if constexpr (FILL) patch(nk3, nv3);
        // B: scores of tile j+1 half 1; P.V of tile j half 1; P of tile j+1 half 0
        half_step(std::true_type(), std::true_type(), sk, 1, s_a, sv, 1, p_1, s_n0, cm_nxt, V8 ? mo_nxt : m, p_a,
                  std::integral_constant<int, NK>(), ld.koff, fkl3, fkb3, std::integral_constant<int, NV>(), ld.voff,
                  fvl3, fvb3);
        __builtin_amdgcn_sched_barrier(0);
        row_sums(p_1, V8 ? 1.f / vsc_cur : 1.f);
        row_sums(p_a, V8 ? 1.f / vsc_nxt : 1.f);
      } else if constexpr (FILL) {  // a wave without query rows still does its share of the fills
#pragma unroll
        for (int i = 0; i < KI; ++i) Loader::dma16(fkl2 + 1024 * i, ld.koff[i], fkb2);
#pragma unroll
        for (int i = 0; i < VI; ++i) Loader::dma16(fvl2 + 1024 * i, ld.voff[i], fvb2);
        patch(nk3, nv3);
#pragma unroll
        for (int i = 0; i < KI; ++i) Loader::dma16(fkl3 + 1024 * i, ld.koff[i], fkb3);
#pragma unroll
        for (int i = 0; i < VI; ++i) Loader::dma16(fvl3 + 1024 * i, ld.voff[i], fvb3);
      }
      if (k_ragged) ld.set_k(BN, head, H);
      if (v_ragged) ld.set_v(BN, head, H);
      cm_cur[0] = cm_nxt[0];
      cm_cur[1] = cm_nxt[1];
      if constexpr (V8) {
        mo_cur[0] = mo_nxt[0];
        mo_cur[1] = mo_nxt[1];
        vsc_cur = vsc_nxt;
        vsc_nxt = vsc_n2;
      }
      nv_cur = nv_nxt;
      d1 = d2;
      d2 = d3;
      d3 = d4;
      d4 = d5;
      ksc_nxt = ksc_n2;
      if constexpr (!FILL) {
        wait_vmcnt<0>();  // slots j+1 and j+2, filled by the previous iteration, have landed
        __syncthreads();
      }
    };
    // last tile (slot n-1, buffer n % 4): P.V only.  One instantiation with a runtime buffer, so
    // that O flows through a single path (a branch per buffer would make the register allocator
    // copy O between AGPRs, and such copies cannot be ordered after the asm MFMAs that write O).
    auto last = [&](int b) {
      if (wave_active) {
        const uint8_t* sv = smem_v[b];
        if (nv_cur < BN) {
          score_drain(s_a);
          mask_half(s_a, 1, nv_cur);
        }
        f32x16 dummy[2];
        bf16x8 p_1[2][2], p_unused[2][2];
        half_step(std::false_type(), std::true_type(), nullptr, 0, dummy, sv, 0, p_a, s_a, cm_cur, V8 ? mo_cur : m,
                  p_1, std::integral_constant<int, 0>(), nullptr, 0u, nullptr, std::integral_constant<int, 0>(), nullptr,
                  0u, nullptr);
        half_step(std::false_type(), std::false_type(), nullptr, 0, dummy, sv, 1, p_1, s_a, cm_cur, V8 ? mo_cur : m,
                  p_unused, std::integral_constant<int, 0>(), nullptr, 0u, nullptr, std::integral_constant<int, 0>(),
                  nullptr, 0u, nullptr);
        row_sums(p_1, V8 ? 1.f / vsc_cur : 1.f);
      }
    };
    // (a loop that ends after the first of a pair needs no barrier: the last tile's slot was
    // filled before the previous pair's barrier, and the pending loads go to other buffers)
    for (int j = 0;;) {
      if (j + 1 >= n) break;
      step(std::integral_constant<int, 1>(), std::true_type(), j++);
      if (j + 1 >= n) break;
      step(std::integral_constant<int, 2>(), std::false_type(), j++);
      if (j + 1 >= n) break;
      step(std::integral_constant<int, 3>(), std::true_type(), j++);
      if (j + 1 >= n) break;
      step(std::integral_constant<int, 0>(), std::false_type(), j++);
    }
    last(n % NBUF);
    wait_vmcnt<0>();  // the fills issued past the segment's end land before the ring is reused
    __syncthreads();  // the ring is refilled by the next pass or segment

    // Could some P have overflowed?  Decided for the whole workgroup, so that every wave runs the
    // same number of tiles (and barriers).
    bool redo = false;
    if (wave_active && !fixed_m) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) redo = redo || !(pair_sum(l[qb]) < 0x1p64f);
    }
    const bool wave_redo = __any(redo);
    if (lane == 0) redo_flags[wave] = wave_redo ? 1 : 0;
    __syncthreads();
    const bool any_redo = (redo_flags[0] | redo_flags[1] | redo_flags[2] | redo_flags[3]) != 0;
    __syncthreads();  // flags are rewritten by the next segment
    if (!any_redo) break;
    // score-only sweep for the true row max (rare path, one buffer, no overlap)
    float mr[2] = {-INFINITY, -INFINITY};
    for (int j = 0; j < n; ++j) {
      const Desc dj = load_desc(j);
      ld.fill_k(kpool, dj.row0, dj.nv, head, H, (uint32_t)(uintptr_t)(WF_LDS void*)smem_k[0]);
      wait_vmcnt<0>();
      __syncthreads();
      if (wave_active) {
        float cm[2];
        set_cm(k_scale_of(j, dj), cm);
        f32x16 s0[2], s1[2];
        scores_tile(reinterpret_cast<const uint8_t*>(smem_k[0]), dj.nv, s0, s1);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) mr[qb] = fmaxf(mr[qb], lane_max(s0[qb], s1[qb], cm[qb]));
      }
      __syncthreads();
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) m[qb] = pair_max(mr[qb]);
    fixed_m = true;
  }

  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) mfma_drain(o[qb][cb]);
    const int r = 64 * wave + 32 * qb + l32;
    const float lt = pair_sum(l[qb]);
    const float inv = 1.f / lt;
    // A split-K partial is stored as fp16 times 2^pexp, one exponent per row, chosen so that the
    // row's largest |value| lands in [2^14, 2^15): the full 11-bit significand for it, and no
    // overflow whatever the magnitude of V.
    int pexp = 0;
    if (slot >= 0) {
      float mx = 0.f;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(o[qb][cb][i]));
      mx = pair_max(mx) * inv;  // lanes l and l ^ 32 hold the two halves of one row
      if (mx > 0.f && mx < INFINITY) {
        int e;
        frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
        pexp = e - 15;
      }
    }
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
      uint16_t* po = p.part_o + ((size_t)slot * BM + r) * D;
      auto sc = [&](float x) { return ldexpf(x * inv, -pexp); };  // exact power-of-two step
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * cb + 8 * g4 + 4 * hi;
          *reinterpret_cast<uint2*>(po + d0) = make_uint2(pack2_f16(sc(o[qb][cb][4 * g4]), sc(o[qb][cb][4 * g4 + 1])),
                                                          pack2_f16(sc(o[qb][cb][4 * g4 + 2]), sc(o[qb][cb][4 * g4 + 3])));
        }
      if (hi == 0)
        *reinterpret_cast<float2*>(p.part_lse + 2 * ((size_t)slot * BM + r)) = make_float2(lse_val, __int_as_float(pexp));
    }
  }
}

// Gate of one work item: every chunk of rank 0 .. last (the item's visible chunks) must carry a
// generation flag at least the one the caller needs.  Wave 0 polls (at most gate_spin sleeps, so
// the wait always ends) and the decision is shared through LDS, so the whole workgroup takes the
// same branch.  A chunk that is not ready skips the item and sets bit 0 of the caller's status.
//
// Memory ordering.  The flags are read with device-coherent (agent-scope) relaxed atomic loads.
// No key or value of a chunk is read in this kernel before its flag is seen: every item of every
// workgroup passes this gate first, an item's tile fills (those past a segment's end included)
// only touch the tiles of its visible prefix, and the entry points require pools aligned to 256
// bytes, so with pages a multiple of 4 KB long no cache line holds bytes of two pages.  The
// caches hold nothing of this kernel's from before its start, so a chunk's pages cannot be stale
// in any cache once its flag is up.  The e4m3 key scales pack several pages' blocks into one
// line, so gated kernels read them with the same coherent loads as the flags (k_scale_of).  An
// agent-scope acquire would invalidate this XCD's L2 at every item and throw away the K/V reuse
// between the workgroups that share it; it is issued only after a poll that had to wait for a
// producer running alongside.
__device__ bool gate_item(const FwdParams& p, const int32_t* items, int item, int* decision) {
  const int32_t* byrank = p.blob + ld_const(p.blob, H_OFF_BYRANK);
  const int last = ld_const(items, item * kItemInts + 6);
  if (threadIdx.x < 64) {
    bool ready = false;
    int it = 0;
    for (;; ++it) {
      bool mine = true;
      for (int r = threadIdx.x; r <= last; r += 64) {
        const int c = byrank[r];
        const uint32_t f = __hip_atomic_load(p.gate_flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mine = mine && f >= p.gate_need[c];
      }
      ready = __all(mine);
      if (ready || it >= p.gate_spin) break;
      __builtin_amdgcn_s_sleep(63);
    }
    if (threadIdx.x == 0) {
      *decision = !ready ? 0 : (it == 0 ? 1 : 2);
      if (!ready) atomicOr(p.gate_status, 1u);
    }
  }
  __syncthreads();
  const int dec = *decision;
  __syncthreads();  // the decision word is rewritten by the next item's gate
  if (dec == 2) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return dec != 0;
}

// Persistent workgroup: runs the segments [ranges[2w], ranges[2w+1]) of the uploaded schedule.
// GATED: every item first passes gate_item.
template <int D, bool FP8, bool OUT_F32, bool GATED, bool V8 = false>
__global__ __launch_bounds__(NTHR, 1) void attn_fwd_kernel(FwdParams p) {
  using Loader = TileLoader<D, FP8, V8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem_k[NBUF][BN * Loader::KB];
  __shared__ __attribute__((aligned(16))) uint8_t smem_v[NBUF][Loader::VBYTES];
  __shared__ int redo_flags[NTHR / 64];
  const int32_t* hdr = p.blob;
  if (ld_const(hdr, H_NONCE_LO) != (int32_t)p.nonce_lo || ld_const(hdr, H_NONCE_HI) != (int32_t)p.nonce_hi) return;
  const int32_t* rg = p.blob + ld_const(hdr, H_OFF_RANGES);
  const int s0 = ld_const(rg, 2 * (int)blockIdx.x), s1 = ld_const(rg, 2 * (int)blockIdx.x + 1);
  const int32_t* segs = p.blob + ld_const(hdr, H_OFF_SEGS);
  const int32_t* items = p.blob + ld_const(hdr, H_OFF_ITEMS);
  const int32_t* tiles = p.blob + ld_const(hdr, H_OFF_TILES);
  __shared__ int gate_decision;
  for (int sg = s0; sg < s1; ++sg) {
    const int item = ld_const(segs, sg * kSegInts);
    if constexpr (GATED) {
      if (!gate_item(p, items, item, &gate_decision)) continue;
    }
    run_segment<D, FP8, OUT_F32, GATED, V8>(p, items, item, ld_const(segs, sg * kSegInts + 1),
                                 ld_const(segs, sg * kSegInts + 2), ld_const(segs, sg * kSegInts + 3), tiles, smem_k, smem_v, redo_flags);
  }
}

// Merge of split key ranges: out = sum_k exp(lse_k - lse) * O_k, lse = log sum_k exp(lse_k), where
// O_k is piece k's fp16 row times 2^(its row exponent), the power of two folded into the piece's
// weight.  One thread per (row, 8 channels); a block covers 256 / (D/8) rows of one merge group.  The pieces are
// taken in batches of kMergeBatch whose loads (lse and O alike) are all issued before any is used,
// so a batch costs one memory round trip; a later batch rescales what the earlier ones summed to
// its new running maximum.
constexpr int kMergeBatch = 4;
constexpr int kMergeTpr(int d) { return d / 8; }  // threads per row

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
  constexpr int TPR = kMergeTpr(D), RPB = 256 / TPR;  // rows per block
  const int32_t* hdr = p.blob;
  if (ld_const(hdr, H_NONCE_LO) != (int32_t)p.nonce_lo || ld_const(hdr, H_NONCE_HI) != (int32_t)p.nonce_hi) return;
  const int grp = blockIdx.x / (BM / RPB), rblk = blockIdx.x % (BM / RPB);
  const int32_t* g = p.blob + ld_const(hdr, H_OFF_GROUPS) + (size_t)grp * kGroupInts;
  const int32_t* it = p.blob + ld_const(hdr, H_OFF_ITEMS) + (size_t)g[0] * kItemInts;
  const int head = it[0], q_row0 = it[1], rows = it[2], slot0 = g[1], parts = g[2];
  const int r = rblk * RPB + threadIdx.x / TPR, d8 = threadIdx.x % TPR;
  if (r >= rows) return;
  float mx = -INFINITY, z = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < parts; k0 += kMergeBatch) {
    float lk[kMergeBatch];
    int ek[kMergeBatch];
    f16x8 ok[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      lk[j] = -INFINITY;
      ek[j] = 0;
      ok[j] = f16x8{};
      if (k0 + j < parts) {
        const size_t row = (size_t)(slot0 + k0 + j) * BM + r;
        const float2 le = *reinterpret_cast<const float2*>(p.part_lse + 2 * row);
        lk[j] = le.x;
        ek[j] = __float_as_int(le.y);
        ok[j] = *reinterpret_cast<const f16x8*>(p.part_o + row * D + 8 * d8);
      }
    }
    float mn = mx;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) mn = fmaxf(mn, lk[j]);
    // every batch holds at least one piece with a finite lse, so mn is finite; exp(-inf) = 0
    const float c = expf(mx - mn);
    z *= c;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= c;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float w = expf(lk[j] - mn);
      z += w;
      const float wo = ldexpf(w, ek[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wo * (float)ok[j][e];
    }
    mx = mn;
  }
  const float iz = 1.f / z;
  const size_t off = ((size_t)(q_row0 + r) * p.H + head) * D + 8 * d8;
  if constexpr (OUT_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.out) + off);
    dst[0] = make_float4(acc[0] * iz, acc[1] * iz, acc[2] * iz, acc[3] * iz);
    dst[1] = make_float4(acc[4] * iz, acc[5] * iz, acc[6] * iz, acc[7] * iz);
  } else {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + off) =
        make_uint4(pack2_bf16(acc[0] * iz, acc[1] * iz), pack2_bf16(acc[2] * iz, acc[3] * iz),
                   pack2_bf16(acc[4] * iz, acc[5] * iz), pack2_bf16(acc[6] * iz, acc[7] * iz));
  }
  if (p.lse && d8 == 0) p.lse[(size_t)head * p.lq + q_row0 + r] = mx + logf(z);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(in)[i];
    reinterpret_cast<uint2*>(out)[i] = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
  }
}

// fp32 -> bf16 staging of the pool rows some query can see: block i converts key tile i of the
// plan's tile list (its valid rows, row_elems = H * d values each); other rows are never read.
__global__ __launch_bounds__(256) void f32_tiles_to_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                                const int32_t* __restrict__ tiles, int64_t row_elems) {
  const int64_t base = (int64_t)tiles[2 * blockIdx.x] * row_elems;
  const int64_t n4 = (int64_t)tiles[2 * blockIdx.x + 1] * row_elems / 4;
  const float4* src = reinterpret_cast<const float4*>(in + base);
  uint2* dst = reinterpret_cast<uint2*>(out + base);
  for (int64_t i = threadIdx.x; i < n4; i += 256) {
    const float4 v = src[i];
    dst[i] = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
  }
}

}  // namespace

hipError_t launch_f32_tiles_to_bf16(const float* in, uint16_t* out, const int32_t* tiles, int n_tiles, int64_t row_elems,
                                    hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_tiles_to_bf16_kernel, dim3((unsigned)n_tiles), dim3(256), 0, s, in, out, tiles, row_elems);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const FwdParams& p, int head_dim, bool out_f32, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (p.gate_flags) hipLaunchKernelGGL((attn_fwd_kernel<128, false, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
    else if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<128, false, true, false>), dim3(grid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false, false, false>), dim3(grid), dim3(NTHR), 0, s, p);
  } else {
    if (p.gate_flags) hipLaunchKernelGGL((attn_fwd_kernel<64, false, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
    else if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<64, false, true, false>), dim3(grid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false, false, false>), dim3(grid), dim3(NTHR), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const FwdParams& p, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (p.gate_flags) hipLaunchKernelGGL((attn_fwd_kernel<128, true, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, true, false, false>), dim3(grid), dim3(NTHR), 0, s, p);
  } else {
    if (p.gate_flags) hipLaunchKernelGGL((attn_fwd_kernel<64, true, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, true, false, false>), dim3(grid), dim3(NTHR), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fp8kv(const FwdParams& p, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL((attn_fwd_kernel<128, true, false, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
  else hipLaunchKernelGGL((attn_fwd_kernel<64, true, false, false, true>), dim3(grid), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine(const FwdParams& p, int head_dim, bool out_f32, int groups, hipStream_t s) {
  if (groups <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)groups * (BM / (256 / kMergeTpr(head_dim)));
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
