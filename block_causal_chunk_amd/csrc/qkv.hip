// qkv.hip -- the producer's QKV projection with the pre-attention epilogue fused into it.
//
// A producer chunk publishes its K/V right after projecting them, at every layer (KipQuest paper
// page, "The deep dive"), and the conversion to the reduced-precision transport is not free
// (project page, "03 - End-to-end KV transport", "Precision" panel).  This kernel computes the
// projection qkv = x . W on the matrix cores and never writes it: each workgroup's output tile (256
// tokens x one head of q, k or v) goes straight through the epilogue of wfattn_rope_publish --
// rotation of q and k, bf16 rounding, e4m3 block quantization of q and/or k, page placement of k and
// v -- so the [tokens, 3, H, d] intermediate makes no round trip through HBM.
//
// GEMM.  Workgroup (row tile, role * H + head): rows t0 .. t0+255 of x [tokens, C] times the d
// columns of W [C, 3*H*d] that belong to (role, head).  4 waves; with d = 128 they form 2 x 2 (128
// tokens x 64 channels each), with d = 64 4 x 1 (64 tokens x 64 channels).  The reduction runs over
// C in steps of 64 through a 3-stage LDS ring that direct global -> LDS loads fill two steps
// ahead, so the loads of later steps are in flight while the matrix cores work on the current one
// (one barrier per step).  O[token][channel] += X[token][c] W[c][channel] on v_mfma_f32_32x32x16_bf16: the X operand
// is a plain 16-byte LDS read of a token row, the W operand a pair of transposed reads
// (ds_read_b64_tr_b16) of the row-major W slice, as the attention kernel reads V^T.
//
// Epilogue.  The fp32 accumulators are staged in LDS as the [256 tokens][d] tile; then wave w takes
// the 64-token tile w (one page-aligned 64-row block of the pool, one 64-row Q-scale block), one
// token row per lane: the lane reads its row and the token's angle row (cos, sin: contiguous, 16
// bytes at a time), rotates q and k pair by pair, rounds to bf16, and writes the bf16 row or
// quantizes the tile as one e4m3 block (the rule of wfattn_quantize_fp8, over the bf16 values).
#include "blockq.hpp"
#include "device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace wfattn {
namespace {

constexpr int QBM = 256;  // tokens per workgroup
constexpr int QBK = 64;   // reduction step
constexpr int NST = 3;    // LDS ring stages

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// One 16-byte global -> LDS load per lane (global_load_lds_dwordx4; M0 holds the LDS address of
// the wave's 1 KB run).  Inline asm, so that the compiler does not wait for it before LDS reads;
// completion is awaited with explicit vmcnt waits.  Nothing else in this kernel uses M0.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t off, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(off), "s"(base) : "memory");
}

template <int D>
struct QkvGeom {
  static constexpr int WC = D / 64;          // waves across the channels
  static constexpr int WR = 4 / WC;          // waves across the tokens
  static constexpr int TOKW = QBM / WR;      // tokens per wave
  static constexpr int TB = TOKW / 32;       // 32-token blocks per wave
  static constexpr int XG = QBM * QBK / 8 / 256;  // 16-byte granules of the x slice per thread
  static constexpr int WG = QBK * D / 8 / 256;    // of the W slice
  static constexpr int XBYTES = QBM * QBK * 2, WBYTES = QBK * D * 2;
};

// One element of a rotated channel pair (x0, x1) -> (x0 c - x1 s, x0 s + x1 c): own is this
// channel's value, other its partner's; every product and sum rounded to fp32 on its own (no
// fused multiply-add), as the rotation of wfattn_rope_publish.
__device__ __forceinline__ float rotate_one(float own, float other, float c, float s, int odd) {
#pragma clang fp contract(off)
  if (odd) {
    const float e = other * s, f = own * c;
    return e + f;
  }
  const float a = own * c, b = other * s;
  return a - b;
}

// x slice in LDS: row r (a token) is 128 bytes, two rows per 256-byte line of the 64 banks;
// granule g is stored at g ^ ((r / 2) mod 8), so the 16 lanes of one ds_read_b128 phase (rows
// r .. r+15, one granule) touch 16 distinct 16-byte bank groups
__device__ __forceinline__ int xswz(int r, int g) { return g ^ ((r >> 1) & 7); }
__device__ __forceinline__ int xoff(int r, int g) { return r * 128 + (xswz(r, g) << 4); }

template <int D>
__global__ __launch_bounds__(256, 1) void qkv_rope_publish_kernel(QkvParams p) {
  using G = QkvGeom<D>;
  const int32_t* hdr = p.blob;
  if (hdr[H_NONCE_LO] != (int32_t)p.nonce_lo || hdr[H_NONCE_HI] != (int32_t)p.nonce_hi) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * (G::XBYTES + G::WBYTES)];
  const int H = p.heads, C = p.hidden, n = p.tokens;
  // Workgroup -> (token tile tt, role-and-head column block rh).  The hardware hands consecutive
  // workgroups to the 8 XCDs in turn; workgroup w takes the next pair of XCD w % 8's contiguous
  // share of all pairs, and the pairs are ordered in blocks of 8 column blocks by token tile, so
  // the ~32 workgroups an XCD runs at once cover about 4 token tiles x 8 column blocks and share
  // their x and W slices in its L2.  (Any bijection is correct; this one only places the work.)
  constexpr int NX = 8, RB = 8;
  const int ntt = (n + QBM - 1) / QBM, nrh = 3 * H, nrb = (nrh + RB - 1) / RB;
  const int nwg = (int)gridDim.x, xcd = (int)blockIdx.x % NX, kx = (int)blockIdx.x / NX;
  const int pair = xcd * (nwg / NX) + (xcd < nwg % NX ? xcd : nwg % NX) + kx;
  const int rb = min(pair / (ntt * RB), nrb - 1);
  const int rem = pair - rb * ntt * RB, width = rb < nrb - 1 ? RB : nrh - rb * RB;
  const int tt = rem / width, rh = rb * RB + rem % width;
  const int t0 = tt * QBM;
  const int role = rh / H, head = rh % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wr = wave / G::WC, wc = wave % G::WC;
  const size_t ldw = (size_t)3 * H * D;
  const uint16_t* wcol = p.w + (size_t)(role * H + head) * D;

  // ---- GEMM ----------------------------------------------------------------------------------
  // Slices of x and W go global -> LDS with global_load_lds_dwordx4 into a ring of NST stages,
  // filled NST-1 steps ahead: lane i of a wave's load writes bytes [16i, 16i+16) of a 1 KB run of
  // the stage, so the swizzles are applied on the global side (the lane that fills physical
  // granule p of a row fetches its logical granule).  Per stage a thread issues XG + WG loads; the
  // wait before a step is a constant vmcnt.
  uint32_t xo_off[G::XG], wo_off[G::WG];  // per-lane byte offsets from the step's base addresses
#pragma unroll
  for (int i = 0; i < G::XG; ++i) {
    const int ch = (wave * G::XG + i) * 64 + lane, r = ch >> 3, pg = ch & 7;
    const int tok = t0 + r < n ? t0 + r : n - 1;  // rows past the chunk re-read its last token
    xo_off[i] = (uint32_t)((size_t)tok * C * 2 + 16 * xswz(r, pg));
  }
#pragma unroll
  for (int i = 0; i < G::WG; ++i) {
    const int ch = (wave * G::WG + i) * 64 + lane, kr = ch / (D / 8), pg = ch % (D / 8);
    wo_off[i] = (uint32_t)((size_t)kr * ldw * 2 + 16 * swz<D>(kr, pg));
  }
  auto stage_x = [&](int st) { return smem + st * (G::XBYTES + G::WBYTES); };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // uniform: the LDS address goes to M0
  auto fill = [&](int st, int k0) {
    const uint32_t xl = (uint32_t)(uintptr_t)(WF_LDS void*)stage_x(st) + wave_u * G::XG * 1024;
    const uint32_t wl = (uint32_t)(uintptr_t)(WF_LDS void*)(stage_x(st) + G::XBYTES) + wave_u * G::WG * 1024;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.x) + (size_t)k0 * 2;
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(wcol) + (size_t)k0 * ldw * 2;
#pragma unroll
    for (int i = 0; i < G::XG; ++i) dma16(xl + 1024 * i, xo_off[i], xb);
#pragma unroll
    for (int i = 0; i < G::WG; ++i) dma16(wl + 1024 * i, wo_off[i], wb);
  };
  const int tq = lane & 15, GG = lane >> 4;
  // W operand of channel block cb (32 channels) and reduction step ks (16 values of c)
  auto w_op = [&](const uint16_t* ws, int cb, int ks) -> bf16x8 {
    const int row = 16 * ks + 8 * hi + (tq >> 2);
    const int col = 64 * wc + 32 * cb + 16 * (GG & 1) + 4 * (tq & 3);
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(ws + lds_off<D>(row, col)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WF_LDS i16x4*)(ws + lds_off<D>(row + 4, col)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto x_op = [&](const uint8_t* xs, int tb, int ks) -> bf16x8 {
    const int r = G::TOKW * wr + 32 * tb + l32;
    return *reinterpret_cast<const bf16x8*>(xs + xoff(r, 2 * ks + hi));
  };
  f32x16 acc[G::TB][2];
#pragma unroll
  for (int tb = 0; tb < G::TB; ++tb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[tb][cb][j] = 0.f;
  const int nk = C / QBK;
  // prologue: steps 0 .. NST-2 in flight (a step past the end reloads the last one, so that every
  // step issues the same loads and the waits stay constant)
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0) fill(s0, (s0 < nk ? s0 : nk - 1) * QBK);
  for (int kb = 0; kb < nk; ++kb) {
    // step kb has landed once only the NST-2 younger stages' loads may be in flight
    wait_vmcnt<(NST - 2) * (G::XG + G::WG)>();
    __syncthreads();  // ... in every wave; and every wave is done with the stage refilled below
    const int nx = kb + NST - 1;
    fill(nx % NST, (nx < nk ? nx : nk - 1) * QBK);
    const uint8_t* xs = stage_x(kb % NST);
    const uint16_t* ws = reinterpret_cast<const uint16_t*>(xs + G::XBYTES);
#pragma unroll
    for (int ks = 0; ks < QBK / 16; ++ks) {
      bf16x8 wo[2], xo[G::TB];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) wo[cb] = w_op(ws, cb, ks);
#pragma unroll
      for (int tb = 0; tb < G::TB; ++tb) xo[tb] = x_op(xs, tb, ks);
#pragma unroll
      for (int tb = 0; tb < G::TB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[tb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xo[tb], wo[cb], acc[tb][cb], 0, 0, 0);
    }
  }
  wait_vmcnt<0>();  // the reloads issued past the end land before the LDS is reused
  __syncthreads();

  // ---- epilogue: stage the fp32 tile [256 tokens][D] in LDS (the GEMM's buffers are free now) -----
  // Row stride D+8 floats: the two halves of a wave store rows four apart, which the padding puts
  // 32 banks apart.
  constexpr int FS = D + 8;
  static_assert(QBM * FS * 4 <= NST * (G::XBYTES + G::WBYTES), "the fp32 tile fits in the GEMM's LDS");
  float* ftile = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int tb = 0; tb < G::TB; ++tb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int ch = 64 * wc + 32 * cb + l32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = G::TOKW * wr + 32 * tb + 8 * (j / 4) + 4 * hi + (j % 4);
        ftile[r * FS + ch] = acc[tb][cb][j];
      }
    }
  __syncthreads();

  // ---- epilogue: wave w takes the 64-token tile w (one page-aligned 64-row block of the pool, one
  // 64-row Q-scale block).  D/8 lanes share a token row, one 16-byte granule (8 channels, 4 rotary
  // pairs) each, so every read of the angles and every row write is a contiguous run per row;
  // a pass covers 64 / (D/8) rows.
  constexpr int GPR = D / 8, RPI = 64 / GPR, NIT = 64 / RPI;
  const int t = tt * (QBM / 64) + wave;  // tile of the chunk
  if (t * 64 >= n) return;
  const int32_t first_tile = p.blob[hdr[H_OFF_CHUNKS] + p.chunk * kChunkInts];
  const int32_t* td = p.blob + hdr[H_OFF_TILES] + (first_tile + t) * kTileInts;
  const int64_t row0 = td[0];
  const int nv = td[1];
  const int gi = lane % GPR, ri = lane / GPR;
  // q and k: each channel pair (2i, 2i+1) rotated by the token's angle i, every product and sum
  // rounded to fp32 on its own; then every value rounded to bf16
  uint4 val[NIT];
  auto tile_row = [&](int it) { return ftile + (64 * wave + RPI * it + ri) * FS + 8 * gi; };
  if (role < 2) {  // uniform: every angle load is issued before the first is used
    float4 cv[NIT], sn[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int row = RPI * it + ri;
      const int64_t tc = (int64_t)t * 64 + (row < nv ? row : 0);  // rows past the chunk: a valid angle row
      cv[it] = *reinterpret_cast<const float4*>(p.cos_t + tc * (D / 2) + 4 * gi);
      sn[it] = *reinterpret_cast<const float4*>(p.sin_t + tc * (D / 2) + 4 * gi);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float4 a = *reinterpret_cast<const float4*>(tile_row(it));
      const float4 b = *reinterpret_cast<const float4*>(tile_row(it) + 4);
      float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const float c[4] = {cv[it].x, cv[it].y, cv[it].z, cv[it].w};
      const float sv[4] = {sn[it].x, sn[it].y, sn[it].z, sn[it].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = y[2 * i], x1 = y[2 * i + 1];
        y[2 * i] = rotate_one(x0, x1, c[i], sv[i], 0);
        y[2 * i + 1] = rotate_one(x1, x0, c[i], sv[i], 1);
      }
      val[it] = make_uint4(pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3]), pack2_bf16(y[4], y[5]),
                           pack2_bf16(y[6], y[7]));
    }
  } else {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float4 a = *reinterpret_cast<const float4*>(tile_row(it));
      const float4 b = *reinterpret_cast<const float4*>(tile_row(it) + 4);
      val[it] = make_uint4(pack2_bf16(a.x, a.y), pack2_bf16(a.z, a.w), pack2_bf16(b.x, b.y), pack2_bf16(b.z, b.w));
    }
  }
  // destination row of tile row `row`: bf16 q, K (bf16 pool) or V
  auto bf16_row = [&](int row) -> uint16_t* {
    const int64_t tok = (int64_t)t * 64 + row;
    if (role == 0) return p.q_out ? p.q_out + (tok * H + head) * D : nullptr;
    if (role == 1) return p.k_pool ? p.k_pool + ((row0 + row) * H + head) * D : nullptr;
    return p.v_pool + ((row0 + row) * H + head) * D;
  };
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = RPI * it + ri;
    uint16_t* dst = bf16_row(row);
    if (dst && row < nv) reinterpret_cast<uint4*>(dst)[gi] = val[it];
  }
  // e4m3 rows: q8 (role 0) or the e4m3 K pool (role 1), the tile quantized as one block
  const bool q8 = role == 0 && p.q8, k8 = role == 1 && p.k8_pool;
  if (q8 || k8) {  // uniform across the wave
    float amax = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (RPI * it + ri < nv) {
        float v[8];
        unpack8(val[it], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = fabsf(v[e]);
          amax = (a > amax) ? a : amax;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o = __shfl_xor(amax, off);
      amax = (o > amax) ? o : amax;
    }
    float scale = 1.f, mult = 1.f;
    if (amax > 0.f) {
      scale = __fdiv_rn(amax, 448.f);
      mult = __fdiv_rn(448.f, amax);
    }
    if (lane == 0) {
      if (q8) p.q_scale[(size_t)t * H + head] = scale;
      else p.k_scale[(row0 / 64) * H + head] = scale;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int row = RPI * it + ri;
      if (row < nv) {
        float v[8];
        unpack8(val[it], v);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float q = __fmul_rn(v[e], mult);
          q = (q > 448.f) ? 448.f : q;
          q = (q < -448.f) ? -448.f : q;
          y[e] = q;
        }
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
        const int64_t tok = (int64_t)t * 64 + row;
        uint8_t* dst8 = q8 ? p.q8 + (tok * H + head) * D : p.k8_pool + ((row0 + row) * H + head) * D;
        reinterpret_cast<uint2*>(dst8)[gi] = make_uint2((uint32_t)w0, (uint32_t)w1);
      }
    }
  }
}

}  // namespace

hipError_t launch_qkv_rope_publish(const QkvParams& p, int32_t head_dim, hipStream_t s) {
  const unsigned nwg = (unsigned)((p.tokens + QBM - 1) / QBM) * (unsigned)(3 * p.heads);
  if (p.tokens > 0) {
    if (head_dim == 128) hipLaunchKernelGGL(qkv_rope_publish_kernel<128>, dim3(nwg), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(qkv_rope_publish_kernel<64>, dim3(nwg), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return p.flags ? launch_flag(p.flags, p.chunk, p.generation, s) : hipSuccess;
}

}  // namespace wfattn
