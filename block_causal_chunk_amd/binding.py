"""ctypes binding of libwfattn.so (include/wfattn.h).  Argument marshalling only: every step of
the attention runs in the library's HIP kernels.  torch supplies device memory and the stream.

Loading fails loudly when the library is missing; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwfattn.so")

WFATTN_OK, WFATTN_ERR_NULL, WFATTN_ERR_INVALID, WFATTN_ERR_RANGE = 0, 1, 2, 3
WFATTN_ERR_UNSUPPORTED, WFATTN_ERR_WORKSPACE, WFATTN_ERR_DEVICE, WFATTN_ERR_NOMEM = 4, 5, 6, 7
WFATTN_BF16, WFATTN_FP32 = 0, 1
WFATTN_WS_BF16, WFATTN_WS_FP32, WFATTN_WS_FP8 = 0, 1, 2

EXPORTED = ["wfattn_plan", "wfattn_plan_free", "wfattn_query_rows", "wfattn_workspace_bytes",
            "wfattn_plan_upload", "wfattn_plan_describe", "wfattn_fwd", "wfattn_fwd_fp8",
            "wfattn_quantize_fp8", "wfattn_status_str", "wfattn_abi_version", "wfattn_publish_kv",
            "wfattn_fwd_gated", "wfattn_publish_kv_fp8", "wfattn_rope_publish", "wfattn_fwd_marked",
            "wfattn_fwd_fp8_marked", "wfattn_fwd_fp8_gated", "wfattn_fwd_noalloc", "wfattn_quantize_v_fp8",
            "wfattn_fwd_fp8kv", "wfattn_fwd_fp8kv_marked", "wfattn_device_geometry", "wfattn_qkv_rope_publish"]
WFATTN_GATE_SPIN_MAX = 1 << 20
WFATTN_NOALLOC_MAX_BYTES = 64 << 20


class WfattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class ChunkTableC(ctypes.Structure):
    _fields_ = [("num_chunks", ctypes.c_int32), ("chunk_tokens", ctypes.POINTER(ctypes.c_int32)),
                ("chunk_order", ctypes.POINTER(ctypes.c_int32)),
                ("page_offsets", ctypes.POINTER(ctypes.c_int32)),
                ("page_ids", ctypes.POINTER(ctypes.c_int32)), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_query_chunks", ctypes.c_int32),
                ("query_chunks", ctypes.POINTER(ctypes.c_int32)), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class OptsC(ctypes.Structure):
    _fields_ = [("split_k", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("order_ties", ctypes.c_int32), ("num_cus", ctypes.c_int32), ("num_xcds", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.wfattn_plan.argtypes = [ctypes.POINTER(ChunkTableC), ctypes.POINTER(OptsC), ctypes.POINTER(vp)]
        L.wfattn_plan.restype = i32
        L.wfattn_plan_free.argtypes = [vp]
        L.wfattn_plan_free.restype = None
        L.wfattn_query_rows.argtypes = [vp]
        L.wfattn_query_rows.restype = i64
        L.wfattn_workspace_bytes.argtypes = [vp, i32]
        L.wfattn_workspace_bytes.restype = sz
        L.wfattn_plan_upload.argtypes = [vp, vp, sz, vp]
        L.wfattn_plan_upload.restype = i32
        L.wfattn_plan_describe.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int32), sz, ctypes.POINTER(sz)]
        L.wfattn_plan_describe.restype = i32
        L.wfattn_fwd.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.wfattn_fwd.restype = i32
        L.wfattn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.wfattn_fwd_fp8.restype = i32
        L.wfattn_fwd_marked.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.wfattn_fwd_marked.restype = i32
        L.wfattn_fwd_fp8_marked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.wfattn_fwd_fp8_marked.restype = i32
        L.wfattn_quantize_fp8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.wfattn_quantize_fp8.restype = i32
        L.wfattn_publish_kv.argtypes = [vp, i32, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, sz, vp]
        L.wfattn_publish_kv.restype = i32
        L.wfattn_fwd_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, i32, vp, vp]
        L.wfattn_fwd_gated.restype = i32
        L.wfattn_fwd_fp8_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, i32, vp, vp]
        L.wfattn_fwd_fp8_gated.restype = i32
        L.wfattn_publish_kv_fp8.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, sz, vp]
        L.wfattn_publish_kv_fp8.restype = i32
        L.wfattn_rope_publish.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, sz,
                                          vp]
        L.wfattn_rope_publish.restype = i32
        L.wfattn_qkv_rope_publish.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_uint32, vp, sz, vp]
        L.wfattn_qkv_rope_publish.restype = i32
        L.wfattn_device_geometry.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.wfattn_device_geometry.restype = i32
        L.wfattn_quantize_v_fp8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.wfattn_quantize_v_fp8.restype = i32
        L.wfattn_fwd_fp8kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.wfattn_fwd_fp8kv.restype = i32
        L.wfattn_fwd_fp8kv_marked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.wfattn_fwd_fp8kv_marked.restype = i32
        L.wfattn_fwd_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
        L.wfattn_fwd_noalloc.restype = i32
        L.wfattn_status_str.argtypes = [i32]
        L.wfattn_status_str.restype = ctypes.c_char_p
        L.wfattn_abi_version.argtypes = []
        L.wfattn_abi_version.restype = i32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().wfattn_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != WFATTN_OK:
        raise WfattnError(status, where)


def _ptr(t):
    """Device (or host) address of a torch tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns a wfattn_plan_t; the table arrays are copied by the library."""

    def __init__(self, handle: int):
        self.handle = ctypes.c_void_p(handle)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.wfattn_plan_free(self.handle)
            self.handle = None

    @property
    def query_rows(self) -> int:
        return int(lib().wfattn_query_rows(self.handle))

    def workspace_bytes(self, mode: int) -> int:
        return int(lib().wfattn_workspace_bytes(self.handle, int(mode)))

    def describe(self, what: int) -> np.ndarray:
        n = ctypes.c_size_t(0)
        _check(lib().wfattn_plan_describe(self.handle, int(what), None, 0, ctypes.byref(n)), "wfattn_plan_describe")
        buf = np.zeros(max(int(n.value), 1), np.int32)
        _check(lib().wfattn_plan_describe(self.handle, int(what), buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                          int(n.value), ctypes.byref(n)), "wfattn_plan_describe")
        return buf[: int(n.value)]


def make_table_c(table):
    """ChunkTableC view of a ChunkTable-like object; returns (struct, keep-alive arrays)."""
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (table.chunk_tokens, table.chunk_order,
                                                               table.page_offsets, table.page_ids,
                                                               table.query_chunks)]
    P = ctypes.POINTER(ctypes.c_int32)
    c = ChunkTableC(len(arrs[0]), arrs[0].ctypes.data_as(P), arrs[1].ctypes.data_as(P), arrs[2].ctypes.data_as(P),
                    arrs[3].ctypes.data_as(P), int(table.num_pages), int(table.page_size), len(arrs[4]),
                    arrs[4].ctypes.data_as(P), int(table.num_heads), int(table.head_dim),
                    float(table.softmax_scale))
    return c, arrs


def wfattn_plan(table, split_k: int = 0, xcd_remap: int = 0, order_ties: int = 0, num_cus: int = 0,
                num_xcds: int = 0) -> Plan:
    c, keep = make_table_c(table)
    o = OptsC(int(split_k), int(xcd_remap), int(order_ties), int(num_cus), int(num_xcds), 0, 0)
    h = ctypes.c_void_p()
    _check(lib().wfattn_plan(ctypes.byref(c), ctypes.byref(o), ctypes.byref(h)), "wfattn_plan")
    del keep
    return Plan(h.value)


_GEOMETRY = {}


def device_geometry(device: int):
    """(compute units, XCDs) of HIP device `device`, read once per device."""
    if device not in _GEOMETRY:
        cus, xcds = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().wfattn_device_geometry(int(device), ctypes.byref(cus), ctypes.byref(xcds)),
               "wfattn_device_geometry")
        _GEOMETRY[device] = (int(cus.value), int(xcds.value))
    return _GEOMETRY[device]


def wfattn_plan_upload(plan: Plan, ws, stream=None):
    _check(lib().wfattn_plan_upload(plan.handle, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "wfattn_plan_upload")


def wfattn_fwd(plan: Plan, dtype: int, q, k_pool, v_pool, out, lse, ws, stream=None):
    _check(lib().wfattn_fwd(plan.handle, int(dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "wfattn_fwd")


def wfattn_fwd_fp8(plan: Plan, q8, q_scale, k8_pool, k_scale, v_pool, out, lse, ws, stream=None):
    _check(lib().wfattn_fwd_fp8(plan.handle, _ptr(q8), _ptr(q_scale), _ptr(k8_pool), _ptr(k_scale), _ptr(v_pool),
                                _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "wfattn_fwd_fp8")


def wfattn_publish_kv(plan: Plan, chunk: int, k_src, v_src, k_pool, v_pool, flags, generation: int, ws, stream=None):
    _check(lib().wfattn_publish_kv(plan.handle, int(chunk), _ptr(k_src), _ptr(v_src), _ptr(k_pool), _ptr(v_pool),
                                   _ptr(flags), int(generation) & 0xffffffff, _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "wfattn_publish_kv")


def wfattn_publish_kv_fp8(plan: Plan, chunk: int, k_src, v_src, k8_pool, k_scale, v_pool, flags, generation: int,
                          ws, stream=None):
    _check(lib().wfattn_publish_kv_fp8(plan.handle, int(chunk), _ptr(k_src), _ptr(v_src), _ptr(k8_pool),
                                       _ptr(k_scale), _ptr(v_pool), _ptr(flags), int(generation) & 0xffffffff,
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "wfattn_publish_kv_fp8")


def wfattn_rope_publish(plan: Plan, chunk: int, qkv, cos_t, sin_t, q_out, q8, q_scale, k_pool, k8_pool, k_scale,
                        v_pool, flags, generation: int, ws, stream=None):
    _check(lib().wfattn_rope_publish(plan.handle, int(chunk), _ptr(qkv), _ptr(cos_t), _ptr(sin_t), _ptr(q_out),
                                     _ptr(q8), _ptr(q_scale), _ptr(k_pool), _ptr(k8_pool), _ptr(k_scale),
                                     _ptr(v_pool), _ptr(flags), int(generation) & 0xffffffff, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "wfattn_rope_publish")


def wfattn_qkv_rope_publish(plan: Plan, chunk: int, x, w, cos_t, sin_t, q_out, q8, q_scale, k_pool, k8_pool,
                            k_scale, v_pool, flags, generation: int, ws, stream=None):
    _check(lib().wfattn_qkv_rope_publish(plan.handle, int(chunk), _ptr(x), _ptr(w), int(x.shape[1]), _ptr(cos_t),
                                         _ptr(sin_t), _ptr(q_out), _ptr(q8), _ptr(q_scale), _ptr(k_pool),
                                         _ptr(k8_pool), _ptr(k_scale), _ptr(v_pool), _ptr(flags),
                                         int(generation) & 0xffffffff, _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "wfattn_qkv_rope_publish")


def wfattn_fwd_gated(plan: Plan, q, k_pool, v_pool, out, lse, ws, flags, need, spin_limit: int, gate_status,
                     stream=None):
    _check(lib().wfattn_fwd_gated(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(flags), _ptr(need), int(spin_limit),
                                  _ptr(gate_status), _stream(stream)), "wfattn_fwd_gated")


def wfattn_fwd_fp8_gated(plan: Plan, q8, q_scale, k8_pool, k_scale, v_pool, out, lse, ws, flags, need,
                         spin_limit: int, gate_status, stream=None):
    _check(lib().wfattn_fwd_fp8_gated(plan.handle, _ptr(q8), _ptr(q_scale), _ptr(k8_pool), _ptr(k_scale),
                                      _ptr(v_pool), _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                      _ptr(flags), _ptr(need), int(spin_limit), _ptr(gate_status), _stream(stream)),
           "wfattn_fwd_fp8_gated")


def wfattn_fwd_marked(plan: Plan, dtype: int, q, k_pool, v_pool, out, lse, ws, attn_done_event: int, stream=None):
    _check(lib().wfattn_fwd_marked(plan.handle, int(dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
                                   _ptr(ws), ws.numel() * ws.element_size(), attn_done_event, _stream(stream)),
           "wfattn_fwd_marked")


def wfattn_fwd_fp8_marked(plan: Plan, q8, q_scale, k8_pool, k_scale, v_pool, out, lse, ws, attn_done_event: int,
                          stream=None):
    _check(lib().wfattn_fwd_fp8_marked(plan.handle, _ptr(q8), _ptr(q_scale), _ptr(k8_pool), _ptr(k_scale),
                                       _ptr(v_pool), _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                       attn_done_event, _stream(stream)), "wfattn_fwd_fp8_marked")


def wfattn_fwd_noalloc(plan: Plan, dtype: int, q, k_pool, v_pool, out, lse, stream=None):
    _check(lib().wfattn_fwd_noalloc(plan.handle, int(dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out),
                                    _ptr(lse), _stream(stream)), "wfattn_fwd_noalloc")


def wfattn_quantize_v_fp8(v, rows: int, heads: int, head_dim: int, v8, scales, stream=None):
    _check(lib().wfattn_quantize_v_fp8(_ptr(v), int(rows), int(heads), int(head_dim), _ptr(v8), _ptr(scales),
                                       _stream(stream)), "wfattn_quantize_v_fp8")


def wfattn_fwd_fp8kv(plan: Plan, q8, q_scale, k8_pool, k_scale, v8_pool, v_scale, out, lse, ws, stream=None):
    _check(lib().wfattn_fwd_fp8kv(plan.handle, _ptr(q8), _ptr(q_scale), _ptr(k8_pool), _ptr(k_scale), _ptr(v8_pool),
                                  _ptr(v_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "wfattn_fwd_fp8kv")


def wfattn_fwd_fp8kv_marked(plan: Plan, q8, q_scale, k8_pool, k_scale, v8_pool, v_scale, out, lse, ws,
                            attn_done_event: int, stream=None):
    _check(lib().wfattn_fwd_fp8kv_marked(plan.handle, _ptr(q8), _ptr(q_scale), _ptr(k8_pool), _ptr(k_scale),
                                         _ptr(v8_pool), _ptr(v_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                         ws.numel() * ws.element_size(), attn_done_event, _stream(stream)),
           "wfattn_fwd_fp8kv_marked")


def wfattn_quantize_fp8(x, rows: int, heads: int, head_dim: int, x8, scales, stream=None):
    _check(lib().wfattn_quantize_fp8(_ptr(x), int(rows), int(heads), int(head_dim), _ptr(x8), _ptr(scales),
                                     _stream(stream)), "wfattn_quantize_fp8")


# ---------------------------------------------------------------------------------------------
# Convenience layer (allocation with torch, then the calls above).
# ---------------------------------------------------------------------------------------------
class Attention:
    """A plan plus its uploaded workspace on one device; call() runs one forward."""

    def __init__(self, table, device="cuda", mode: int = WFATTN_WS_BF16, split_k: int = 0, xcd_remap: int = 0,
                 stream=None, order_ties: int = 0):
        import torch
        self.table = table
        dev = torch.device(device)
        cus, xcds = device_geometry(dev.index if dev.index is not None else torch.cuda.current_device())
        self.plan = wfattn_plan(table, split_k=split_k, xcd_remap=xcd_remap, order_ties=order_ties, num_cus=cus,
                                num_xcds=xcds)
        self.mode = mode
        nbytes = self.plan.workspace_bytes(mode)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        wfattn_plan_upload(self.plan, self.ws, stream)
        self.lq = self.plan.query_rows

    def fwd(self, q, k_pool, v_pool, out=None, lse=None, want_lse=False, stream=None):
        import torch
        H, d = int(self.table.num_heads), int(self.table.head_dim)
        if out is None:
            out = torch.empty((self.lq, H, d), dtype=q.dtype, device=q.device)
        if lse is None and want_lse:
            lse = torch.empty((H, self.lq), dtype=torch.float32, device=q.device)
        dt = WFATTN_FP32 if q.dtype == torch.float32 else WFATTN_BF16
        wfattn_fwd(self.plan, dt, q, k_pool, v_pool, out, lse, self.ws, stream)
        return out, lse

    def fwd_fp8kv(self, q8, q_scale, k8_pool, k_scale, v8_pool, v_scale, out=None, lse=None, want_lse=False,
                  stream=None):
        import torch
        H, d = int(self.table.num_heads), int(self.table.head_dim)
        if out is None:
            out = torch.empty((self.lq, H, d), dtype=torch.bfloat16, device=v8_pool.device)
        if lse is None and want_lse:
            lse = torch.empty((H, self.lq), dtype=torch.float32, device=v8_pool.device)
        wfattn_fwd_fp8kv(self.plan, q8, q_scale, k8_pool, k_scale, v8_pool, v_scale, out, lse, self.ws, stream)
        return out, lse

    def fwd_fp8(self, q8, q_scale, k8_pool, k_scale, v_pool, out=None, lse=None, want_lse=False, stream=None):
        import torch
        H, d = int(self.table.num_heads), int(self.table.head_dim)
        if out is None:
            out = torch.empty((self.lq, H, d), dtype=torch.bfloat16, device=v_pool.device)
        if lse is None and want_lse:
            lse = torch.empty((H, self.lq), dtype=torch.float32, device=v_pool.device)
        wfattn_fwd_fp8(self.plan, q8, q_scale, k8_pool, k_scale, v_pool, out, lse, self.ws, stream)
        return out, lse


def quantize_v_fp8(v_pool, stream=None):
    """bf16 V pool [pages, page_size, H, d] -> (e4m3 V pool uint8 [pages*page_size/64, H, d, 64],
    scales f32 [pages*page_size/64, H]) in the layout of the e4m3 K/V forward."""
    import torch
    rows = v_pool.shape[0] * v_pool.shape[1]
    H, d = v_pool.shape[2], v_pool.shape[3]
    v8 = torch.empty((rows // 64, H, d, 64), dtype=torch.uint8, device=v_pool.device)
    sc = torch.empty((rows // 64, H), dtype=torch.float32, device=v_pool.device)
    wfattn_quantize_v_fp8(v_pool, rows, H, d, v8, sc, stream)
    return v8, sc


def quantize_fp8(x, stream=None):
    """x [rows, H, d] bf16 on the device -> (codes uint8 [rows, H, d], scales f32 [ceil(rows/64), H])."""
    import torch
    rows, H, d = x.shape
    x8 = torch.empty((rows, H, d), dtype=torch.uint8, device=x.device)
    sc = torch.empty(((rows + 63) // 64, H), dtype=torch.float32, device=x.device)
    wfattn_quantize_fp8(x, rows, H, d, x8, sc, stream)
    return x8, sc


def quantize_q_fp8(table, q, stream=None):
    """Q [Lq, H, d] bf16 -> codes and [nqb, H] scales with 64-row blocks restarting at each query chunk."""
    import torch
    H, d = int(table.num_heads), int(table.head_dim)
    toks = [int(table.chunk_tokens[c]) for c in table.query_chunks]
    nqb = sum((t + 63) // 64 for t in toks)
    x8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    sc = torch.empty((nqb, H), dtype=torch.float32, device=q.device)
    row, blk = 0, 0
    for t in toks:
        wfattn_quantize_fp8(q[row:row + t], t, H, d, x8[row:row + t], sc[blk:blk + (t + 63) // 64], stream)
        row += t
        blk += (t + 63) // 64
    return x8, sc
