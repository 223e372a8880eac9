// api.hip -- the extern "C" entry points that touch the device: upload, forward, quantize.
// Every argument check runs before the first HIP call (see include/wfattn.h for the contract).
#include <cmath>
#include <mutex>

#include "kernels.hpp"
#include "plan.hpp"

using namespace wfattn;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

FwdParams base_params(const Plan* P, void* ws) {
  FwdParams fp{};
  char* w = static_cast<char*>(ws);
  fp.blob = reinterpret_cast<const int32_t*>(w + P->ws_blob);
  fp.part_o = reinterpret_cast<uint16_t*>(w + P->ws_part_o);
  fp.part_lse = reinterpret_cast<float*>(w + P->ws_part_lse);
  fp.H = P->num_heads;
  fp.lq = static_cast<int32_t>(P->lq);
  fp.scale = P->scale;
  fp.c = static_cast<float>(static_cast<double>(P->scale) * 1.4426950408889634);  // scale * log2(e)
  fp.nonce_lo = static_cast<uint32_t>(P->nonce & 0xffffffffu);
  fp.nonce_hi = static_cast<uint32_t>(P->nonce >> 32);
  return fp;
}

}  // namespace

extern "C" wfattn_status wfattn_plan_upload(const wfattn_plan_t* plan, void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return WFATTN_ERR_UNSUPPORTED;
  const Plan* P = as_plan(plan);
  if (ws_bytes < P->ws_base_bytes) return WFATTN_ERR_WORKSPACE;
  hipError_t e = hipMemcpyAsync(static_cast<char*>(ws) + P->ws_blob, P->blob.data(), P->blob.size() * sizeof(int32_t),
                                hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WFATTN_OK : WFATTN_ERR_DEVICE;
}

namespace {

struct Gate {
  const uint32_t* flags;
  const uint32_t* need;
  uint32_t* status;
  int32_t spin;
};

wfattn_status fwd_impl(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q, const void* k_pool,
                       const void* v_pool, void* out, float* lse, void* ws, size_t ws_bytes, void* stream,
                       const Gate* gate, hipEvent_t mark = nullptr) {
  if (!plan || !q || !k_pool || !v_pool || !out) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  if (dtype != WFATTN_BF16 && dtype != WFATTN_FP32) return WFATTN_ERR_UNSUPPORTED;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(ws, 256))
    return WFATTN_ERR_UNSUPPORTED;
  const Plan* P = as_plan(plan);
  const bool f32 = dtype == WFATTN_FP32;
  if (ws_bytes < (f32 ? P->ws_fp32_bytes : P->ws_base_bytes)) return WFATTN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FwdParams fp = base_params(P, ws);
  fp.out = out;
  fp.lse = lse;
  if (gate) {
    fp.gate_flags = gate->flags;
    fp.gate_need = gate->need;
    fp.gate_status = gate->status;
    fp.gate_spin = gate->spin;
  }
  if (f32) {
    char* w = static_cast<char*>(ws);
    uint16_t* sq = reinterpret_cast<uint16_t*>(w + P->stage_q_off);
    uint16_t* sk = reinterpret_cast<uint16_t*>(w + P->stage_k_off);
    uint16_t* sv = reinterpret_cast<uint16_t*>(w + P->stage_v_off);
    const int64_t qn = P->lq * P->num_heads * P->head_dim;
    const int64_t row_elems = static_cast<int64_t>(P->num_heads) * P->head_dim;
    const int32_t* tiles = fp.blob + P->off_tiles;  // the uploaded tile list; visible tiles first
    if (launch_f32_to_bf16(static_cast<const float*>(q), sq, qn, s) != hipSuccess ||
        launch_f32_tiles_to_bf16(static_cast<const float*>(k_pool), sk, tiles, P->n_vis_tiles, row_elems, s) !=
            hipSuccess ||
        launch_f32_tiles_to_bf16(static_cast<const float*>(v_pool), sv, tiles, P->n_vis_tiles, row_elems, s) !=
            hipSuccess)
      return WFATTN_ERR_DEVICE;
    fp.q = sq;
    fp.k = sk;
    fp.v = sv;
  } else {
    fp.q = static_cast<const uint16_t*>(q);
    fp.k = static_cast<const uint16_t*>(k_pool);
    fp.v = static_cast<const uint16_t*>(v_pool);
  }
  if (launch_attn_bf16(fp, P->head_dim, f32, P->n_wgs, s) != hipSuccess) return WFATTN_ERR_DEVICE;
  if (mark && hipEventRecord(mark, s) != hipSuccess) return WFATTN_ERR_DEVICE;
  if (launch_combine(fp, P->head_dim, f32, P->n_groups, s) != hipSuccess) return WFATTN_ERR_DEVICE;
  return WFATTN_OK;
}

// v_scale == nullptr: v_pool is the bf16 pool; else v_pool is the e4m3 V pool ([pool_rows / 64,
// H, d, 64] codes) with those scales
wfattn_status fwd8_impl(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale, const uint8_t* k8_pool,
                        const float* k_scale, const void* v_pool, const float* v_scale, void* out, float* lse,
                        void* ws, size_t ws_bytes, void* stream, const Gate* gate, hipEvent_t mark) {
  if (!plan || !q8 || !q_scale || !k8_pool || !k_scale || !v_pool || !out) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(q8, 16) || !aligned(k8_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) || !aligned(q_scale, 4) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(lse, 4) || !aligned(ws, 256))
    return WFATTN_ERR_UNSUPPORTED;
  const Plan* P = as_plan(plan);
  if (ws_bytes < P->ws_base_bytes) return WFATTN_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FwdParams fp = base_params(P, ws);
  fp.q8 = q8;
  fp.q_scale = q_scale;
  fp.k8 = k8_pool;
  fp.k_scale = k_scale;
  if (v_scale) {
    fp.v8 = static_cast<const uint8_t*>(v_pool);
    fp.v_scale = v_scale;
  } else {
    fp.v = static_cast<const uint16_t*>(v_pool);
  }
  fp.out = out;
  fp.lse = lse;
  if (gate) {
    fp.gate_flags = gate->flags;
    fp.gate_need = gate->need;
    fp.gate_status = gate->status;
    fp.gate_spin = gate->spin;
  }
  const hipError_t e = v_scale ? launch_attn_fp8kv(fp, P->head_dim, P->n_wgs, s) : launch_attn_fp8(fp, P->head_dim, P->n_wgs, s);
  if (e != hipSuccess) return WFATTN_ERR_DEVICE;
  if (mark && hipEventRecord(mark, s) != hipSuccess) return WFATTN_ERR_DEVICE;
  if (launch_combine(fp, P->head_dim, false, P->n_groups, s) != hipSuccess) return WFATTN_ERR_DEVICE;
  return WFATTN_OK;
}

}  // namespace

extern "C" wfattn_status wfattn_fwd(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q, const void* k_pool,
                                    const void* v_pool, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return fwd_impl(plan, dtype, q, k_pool, v_pool, out, lse, ws, ws_bytes, stream, nullptr);
}

extern "C" wfattn_status wfattn_fwd_gated(const wfattn_plan_t* plan, const void* q, const void* k_pool,
                                          const void* v_pool, void* out, float* lse, void* ws, size_t ws_bytes,
                                          const uint32_t* flags, const uint32_t* need, int32_t spin_limit,
                                          uint32_t* gate_status, void* stream) {
  if (!flags || !need || !gate_status) return WFATTN_ERR_NULL;
  if (spin_limit < 0 || spin_limit > WFATTN_GATE_SPIN_MAX) return WFATTN_ERR_RANGE;
  if (!aligned(flags, 4) || !aligned(need, 4) || !aligned(gate_status, 4)) return WFATTN_ERR_UNSUPPORTED;
  if (!aligned(k_pool, 256) || !aligned(v_pool, 256)) return WFATTN_ERR_UNSUPPORTED;  // no line spans two pages
  const Gate g{flags, need, gate_status, spin_limit};
  return fwd_impl(plan, WFATTN_BF16, q, k_pool, v_pool, out, lse, ws, ws_bytes, stream, &g);
}

extern "C" wfattn_status wfattn_publish_kv(const wfattn_plan_t* plan, int32_t chunk, const void* k_src,
                                           const void* v_src, void* k_pool, void* v_pool, uint32_t* flags,
                                           uint32_t generation, const void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !k_src || !v_src || !k_pool || !v_pool) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  const Plan* P = as_plan(plan);
  if (chunk < 0 || chunk >= P->num_chunks) return WFATTN_ERR_INVALID;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(flags, 4) || !aligned(ws, 256))
    return WFATTN_ERR_UNSUPPORTED;
  if (ws_bytes < P->ws_base_bytes) return WFATTN_ERR_WORKSPACE;
  PublishParams pp{};
  pp.k_src = static_cast<const uint16_t*>(k_src);
  pp.v_src = static_cast<const uint16_t*>(v_src);
  pp.k_pool = static_cast<uint16_t*>(k_pool);
  pp.v_pool = static_cast<uint16_t*>(v_pool);
  pp.blob = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + P->ws_blob);
  pp.chunk = chunk;
  pp.row_granules = P->num_heads * P->head_dim * 2 / 16;
  pp.nonce_lo = static_cast<uint32_t>(P->nonce & 0xffffffffu);
  pp.nonce_hi = static_cast<uint32_t>(P->nonce >> 32);
  pp.flags = flags;
  pp.generation = generation;
  const int64_t tokens = P->blob[P->off_chunks + static_cast<size_t>(chunk) * kChunkInts + 1];
  return launch_publish(pp, tokens, static_cast<hipStream_t>(stream)) == hipSuccess ? WFATTN_OK : WFATTN_ERR_DEVICE;
}

extern "C" wfattn_status wfattn_fwd_fp8(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                                        const uint8_t* k8_pool, const float* k_scale, const void* v_pool, void* out,
                                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  return fwd8_impl(plan, q8, q_scale, k8_pool, k_scale, v_pool, nullptr, out, lse, ws, ws_bytes, stream, nullptr,
                   nullptr);
}

extern "C" wfattn_status wfattn_fwd_fp8kv(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                                          const uint8_t* k8_pool, const float* k_scale, const uint8_t* v8_pool,
                                          const float* v_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                          void* stream) {
  if (!v_scale) return WFATTN_ERR_NULL;
  return fwd8_impl(plan, q8, q_scale, k8_pool, k_scale, v8_pool, v_scale, out, lse, ws, ws_bytes, stream, nullptr,
                   nullptr);
}

extern "C" wfattn_status wfattn_fwd_fp8kv_marked(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                                                 const uint8_t* k8_pool, const float* k_scale, const uint8_t* v8_pool,
                                                 const float* v_scale, void* out, float* lse, void* ws,
                                                 size_t ws_bytes, void* attn_done_event, void* stream) {
  if (!v_scale || !attn_done_event) return WFATTN_ERR_NULL;
  return fwd8_impl(plan, q8, q_scale, k8_pool, k_scale, v8_pool, v_scale, out, lse, ws, ws_bytes, stream, nullptr,
                   static_cast<hipEvent_t>(attn_done_event));
}

extern "C" wfattn_status wfattn_fwd_fp8_gated(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                                              const uint8_t* k8_pool, const float* k_scale, const void* v_pool,
                                              void* out, float* lse, void* ws, size_t ws_bytes,
                                              const uint32_t* flags, const uint32_t* need, int32_t spin_limit,
                                              uint32_t* gate_status, void* stream) {
  if (!flags || !need || !gate_status) return WFATTN_ERR_NULL;
  if (spin_limit < 0 || spin_limit > WFATTN_GATE_SPIN_MAX) return WFATTN_ERR_RANGE;
  if (!aligned(flags, 4) || !aligned(need, 4) || !aligned(gate_status, 4)) return WFATTN_ERR_UNSUPPORTED;
  if (!aligned(k8_pool, 256) || !aligned(v_pool, 256)) return WFATTN_ERR_UNSUPPORTED;  // no line spans two pages
  const Gate g{flags, need, gate_status, spin_limit};
  return fwd8_impl(plan, q8, q_scale, k8_pool, k_scale, v_pool, nullptr, out, lse, ws, ws_bytes, stream, &g, nullptr);
}

extern "C" wfattn_status wfattn_fwd_marked(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q,
                                           const void* k_pool, const void* v_pool, void* out, float* lse, void* ws,
                                           size_t ws_bytes, void* attn_done_event, void* stream) {
  if (!attn_done_event) return WFATTN_ERR_NULL;
  return fwd_impl(plan, dtype, q, k_pool, v_pool, out, lse, ws, ws_bytes, stream, nullptr,
                  static_cast<hipEvent_t>(attn_done_event));
}

extern "C" wfattn_status wfattn_fwd_fp8_marked(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                                               const uint8_t* k8_pool, const float* k_scale, const void* v_pool,
                                               void* out, float* lse, void* ws, size_t ws_bytes,
                                               void* attn_done_event, void* stream) {
  if (!attn_done_event) return WFATTN_ERR_NULL;
  return fwd8_impl(plan, q8, q_scale, k8_pool, k_scale, v_pool, nullptr, out, lse, ws, ws_bytes, stream, nullptr,
                   static_cast<hipEvent_t>(attn_done_event));
}

extern "C" wfattn_status wfattn_publish_kv_fp8(const wfattn_plan_t* plan, int32_t chunk, const void* k_src,
                                               const void* v_src, uint8_t* k8_pool, float* k_scale, void* v_pool,
                                               uint32_t* flags, uint32_t generation, const void* ws, size_t ws_bytes,
                                               void* stream) {
  if (!plan || !k_src || !v_src || !k8_pool || !k_scale || !v_pool) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  const Plan* P = as_plan(plan);
  if (chunk < 0 || chunk >= P->num_chunks) return WFATTN_ERR_INVALID;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k8_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(k_scale, 4) || !aligned(flags, 4) || !aligned(ws, 256))
    return WFATTN_ERR_UNSUPPORTED;
  if (ws_bytes < P->ws_base_bytes) return WFATTN_ERR_WORKSPACE;
  PublishFp8Params pp{};
  pp.k_src = static_cast<const uint16_t*>(k_src);
  pp.v_src = static_cast<const uint16_t*>(v_src);
  pp.k8_pool = k8_pool;
  pp.k_scale = k_scale;
  pp.v_pool = static_cast<uint16_t*>(v_pool);
  pp.blob = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + P->ws_blob);
  pp.chunk = chunk;
  pp.heads = P->num_heads;
  pp.nonce_lo = static_cast<uint32_t>(P->nonce & 0xffffffffu);
  pp.nonce_hi = static_cast<uint32_t>(P->nonce >> 32);
  pp.flags = flags;
  pp.generation = generation;
  const int64_t tokens = P->blob[P->off_chunks + static_cast<size_t>(chunk) * kChunkInts + 1];
  return launch_publish_fp8(pp, tokens, P->head_dim, static_cast<hipStream_t>(stream)) == hipSuccess
             ? WFATTN_OK
             : WFATTN_ERR_DEVICE;
}

extern "C" wfattn_status wfattn_rope_publish(const wfattn_plan_t* plan, int32_t chunk, const void* qkv,
                                             const float* cos_t, const float* sin_t, void* q_out, uint8_t* q8,
                                             float* q_scale, void* k_pool, uint8_t* k8_pool, float* k_scale,
                                             void* v_pool, uint32_t* flags, uint32_t generation, const void* ws,
                                             size_t ws_bytes, void* stream) {
  if (!plan || !qkv || !cos_t || !sin_t || !v_pool) return WFATTN_ERR_NULL;
  if (!k_pool == !k8_pool) return WFATTN_ERR_INVALID;  // exactly one form of K
  if ((k8_pool && !k_scale) || (q8 && !q_scale)) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  const Plan* P = as_plan(plan);
  if (chunk < 0 || chunk >= P->num_chunks) return WFATTN_ERR_INVALID;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(qkv, 16) || !aligned(cos_t, 16) || !aligned(sin_t, 16) || !aligned(q_out, 16) || !aligned(q8, 16) ||
      !aligned(q_scale, 4) || !aligned(k_pool, 16) || !aligned(k8_pool, 16) || !aligned(k_scale, 4) ||
      !aligned(v_pool, 16) || !aligned(flags, 4) || !aligned(ws, 256))
    return WFATTN_ERR_UNSUPPORTED;
  if (ws_bytes < P->ws_base_bytes) return WFATTN_ERR_WORKSPACE;
  RopeParams rp{};
  rp.qkv = static_cast<const uint16_t*>(qkv);
  rp.cos_t = cos_t;
  rp.sin_t = sin_t;
  rp.q_out = static_cast<uint16_t*>(q_out);
  rp.q8 = q8;
  rp.q_scale = q_scale;
  rp.k_pool = static_cast<uint16_t*>(k_pool);
  rp.k8_pool = k8_pool;
  rp.k_scale = k_scale;
  rp.v_pool = static_cast<uint16_t*>(v_pool);
  rp.blob = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + P->ws_blob);
  rp.chunk = chunk;
  rp.heads = P->num_heads;
  rp.nonce_lo = static_cast<uint32_t>(P->nonce & 0xffffffffu);
  rp.nonce_hi = static_cast<uint32_t>(P->nonce >> 32);
  rp.flags = flags;
  rp.generation = generation;
  const int64_t tokens = P->blob[P->off_chunks + static_cast<size_t>(chunk) * kChunkInts + 1];
  return launch_rope_publish(rp, tokens, P->head_dim, static_cast<hipStream_t>(stream)) == hipSuccess
             ? WFATTN_OK
             : WFATTN_ERR_DEVICE;
}

extern "C" wfattn_status wfattn_qkv_rope_publish(const wfattn_plan_t* plan, int32_t chunk, const void* x, const void* w,
                                                 int32_t hidden, const float* cos_t, const float* sin_t, void* q_out,
                                                 uint8_t* q8, float* q_scale, void* k_pool, uint8_t* k8_pool,
                                                 float* k_scale, void* v_pool, uint32_t* flags, uint32_t generation,
                                                 const void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !x || !w || !cos_t || !sin_t || !v_pool) return WFATTN_ERR_NULL;
  if (!k_pool == !k8_pool) return WFATTN_ERR_INVALID;  // exactly one form of K
  if ((k8_pool && !k_scale) || (q8 && !q_scale)) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  const Plan* P = as_plan(plan);
  if (chunk < 0 || chunk >= P->num_chunks) return WFATTN_ERR_INVALID;
  if (hidden < 64 || hidden % 64 != 0) return WFATTN_ERR_UNSUPPORTED;
  // the kernel addresses x with 32-bit byte offsets
  if (static_cast<int64_t>(P->blob[P->off_chunks + static_cast<size_t>(chunk) * kChunkInts + 1]) * hidden * 2 >
      INT32_MAX)
    return WFATTN_ERR_RANGE;
  if (!ws) return WFATTN_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(cos_t, 16) || !aligned(sin_t, 16) || !aligned(q_out, 16) ||
      !aligned(q8, 16) || !aligned(q_scale, 4) || !aligned(k_pool, 16) || !aligned(k8_pool, 16) ||
      !aligned(k_scale, 4) || !aligned(v_pool, 16) || !aligned(flags, 4) || !aligned(ws, 256))
    return WFATTN_ERR_UNSUPPORTED;
  if (ws_bytes < P->ws_base_bytes) return WFATTN_ERR_WORKSPACE;
  QkvParams qp{};
  qp.x = static_cast<const uint16_t*>(x);
  qp.w = static_cast<const uint16_t*>(w);
  qp.tokens = P->blob[P->off_chunks + static_cast<size_t>(chunk) * kChunkInts + 1];
  qp.hidden = hidden;
  qp.cos_t = cos_t;
  qp.sin_t = sin_t;
  qp.q_out = static_cast<uint16_t*>(q_out);
  qp.q8 = q8;
  qp.q_scale = q_scale;
  qp.k_pool = static_cast<uint16_t*>(k_pool);
  qp.k8_pool = k8_pool;
  qp.k_scale = k_scale;
  qp.v_pool = static_cast<uint16_t*>(v_pool);
  qp.blob = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + P->ws_blob);
  qp.chunk = chunk;
  qp.heads = P->num_heads;
  qp.nonce_lo = static_cast<uint32_t>(P->nonce & 0xffffffffu);
  qp.nonce_hi = static_cast<uint32_t>(P->nonce >> 32);
  qp.flags = flags;
  qp.generation = generation;
  return launch_qkv_rope_publish(qp, P->head_dim, static_cast<hipStream_t>(stream)) == hipSuccess ? WFATTN_OK
                                                                                                  : WFATTN_ERR_DEVICE;
}

extern "C" wfattn_status wfattn_device_geometry(int32_t device, int32_t* num_cus, int32_t* num_xcds) {
  if (!num_cus || !num_xcds) return WFATTN_ERR_NULL;
  int cus = 0, xcc = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
    return WFATTN_ERR_DEVICE;
  if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, device) != hipSuccess || xcc < 1 || cus % xcc != 0)
    xcc = 1;  // unknown: treat the device as one L2 domain
  *num_cus = cus;
  *num_xcds = xcc;
  return WFATTN_OK;
}

extern "C" wfattn_status wfattn_quantize_v_fp8(const void* v_bf16, int64_t rows, int32_t heads, int32_t head_dim,
                                               uint8_t* v8, float* scales, void* stream) {
  if (!v_bf16 || !v8 || !scales) return WFATTN_ERR_NULL;
  if (head_dim != 64 && head_dim != 128) return WFATTN_ERR_UNSUPPORTED;
  if (rows < 0 || rows % 64 != 0 || heads < 1) return WFATTN_ERR_RANGE;
  if (rows / 64 * static_cast<int64_t>(heads) > INT32_MAX) return WFATTN_ERR_RANGE;
  if (!aligned(v_bf16, 16) || !aligned(v8, 16) || !aligned(scales, 4)) return WFATTN_ERR_UNSUPPORTED;
  if (rows == 0) return WFATTN_OK;
  if (launch_quantize_v_fp8(static_cast<const uint16_t*>(v_bf16), rows, heads, head_dim, v8, scales,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return WFATTN_ERR_DEVICE;
  return WFATTN_OK;
}

extern "C" wfattn_status wfattn_quantize_fp8(const void* x_bf16, int64_t rows, int32_t heads, int32_t head_dim,
                                             uint8_t* x8, float* scales, void* stream) {
  if (!x_bf16 || !x8 || !scales) return WFATTN_ERR_NULL;
  if (head_dim != 64 && head_dim != 128) return WFATTN_ERR_UNSUPPORTED;
  if (rows < 0 || heads < 1) return WFATTN_ERR_RANGE;
  if ((rows + 63) / 64 * static_cast<int64_t>(heads) > INT32_MAX) return WFATTN_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(x8, 16) || !aligned(scales, 4)) return WFATTN_ERR_UNSUPPORTED;
  if (rows == 0) return WFATTN_OK;
  if (launch_quantize_fp8(static_cast<const uint16_t*>(x_bf16), rows, heads, head_dim, x8, scales,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return WFATTN_ERR_DEVICE;
  return WFATTN_OK;
}

// ---- forward without allocation ---------------------------------------------------------------
// The workspace of wfattn_fwd_noalloc is this file-scope device array: every GPU the library runs
// on holds one copy of it until the process ends.  Host code never passes `scratch` itself to a
// kernel or a copy (on the host that name is only a stand-in for the symbol); it uses the address
// hipGetSymbolAddress returns for the current device, looked up once per device.
namespace {

__device__ __align__(256) uint8_t scratch[WFATTN_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Address of the current device's copy of `scratch` (looked up on the first call per device).
wfattn_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WFATTN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return WFATTN_ERR_DEVICE;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return WFATTN_OK;
}

}  // namespace

extern "C" wfattn_status wfattn_fwd_noalloc(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q,
                                            const void* k_pool, const void* v_pool, void* out, float* lse,
                                            void* stream) {
  if (!plan || !q || !k_pool || !v_pool || !out) return WFATTN_ERR_NULL;
  if (!plan_ok(plan)) return WFATTN_ERR_INVALID;
  if (dtype != WFATTN_BF16 && dtype != WFATTN_FP32) return WFATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return WFATTN_ERR_UNSUPPORTED;
  const Plan* P = as_plan(plan);
  const size_t need = dtype == WFATTN_FP32 ? P->ws_fp32_bytes : P->ws_base_bytes;
  if (need > static_cast<size_t>(WFATTN_NOALLOC_MAX_BYTES)) return WFATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  const wfattn_status st = scratch_of_current_device(&ws);
  if (st != WFATTN_OK) return st;
  // this call's work list and page table replace whatever the previous call left in the array;
  // nothing else in it needs a starting value (split-K partials are written before they are read)
  if (hipMemcpyAsync(static_cast<char*>(ws) + P->ws_blob, P->blob.data(), P->blob.size() * sizeof(int32_t),
                     hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)) != hipSuccess)
    return WFATTN_ERR_DEVICE;
  return fwd_impl(plan, dtype, q, k_pool, v_pool, out, lse, ws, WFATTN_NOALLOC_MAX_BYTES, stream, nullptr);
}
