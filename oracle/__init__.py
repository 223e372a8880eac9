"""CPU oracle for block-causal chunk attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its binding) never does.

Two independent statements of the same definition live here:
  * ``wf_oracle.c`` (fp64, OpenMP): walks the page table chunk by chunk, two-pass softmax;
  * ``dense.py`` (numpy fp64): gathers keys, builds an explicit block-lower-triangular mask.
plus an e4m3 codec and block quantizer written from the OCP 8-bit float definition, the
placement of a chunk's K/V into its pages (``publish_kv``) and the rotation of channel pairs
(``rotate_pairs``).
Every function is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwf_oracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = False) -> str:
    """Compile libwf_oracle.so with gcc (plain C, OpenMP)."""
    src = os.path.join(_HERE, "wf_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_attn_masked.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_double, _f64p, _f64p, _f64p, _u8p, _f64p,
                                         _f64p, ctypes.c_int32]
        L.oracle_attn_rows.argtypes = [ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_double, _f64p, _f64p, _f64p,
                                       ctypes.c_int64, _i64p, _f64p, _f64p, _f64p, ctypes.c_int32]
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_quantize_e4m3.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           _u8p, _f32p]
        L.oracle_dequantize_e4m3.argtypes = [_u8p, _f32p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, _f64p]
        L.oracle_merge_lse.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _f64p,
                                       _f64p, _f64p, _f64p]
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _f64(x):
    """Any array-like (numpy or torch, any float dtype) -> contiguous float64 numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def resolve_scale(table) -> float:
    """Softmax scale: the table's value if positive, else 1/sqrt(head_dim)."""
    s = float(table.softmax_scale)
    return s if s > 0 else 1.0 / math.sqrt(table.head_dim)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def attn_rows(table, q, k_pool, v_pool, rows=None, nthreads: int = 0, want_sumw2: bool = False):
    """Attention of the query rows ``rows`` (default: all) of ``table``: full inside a chunk,
    block-causal across chunks (Wave Forcing project page, "01 - The design gap", directed
    frontier and "Key observation"; KipQuest paper page, "The deep dive"), keys read from the
    pages in place ("03 - End-to-end KV transport", panel "03 - Layout").  ``wf_oracle.c`` states
    the rule and the two-pass softmax.

    q [Lq, H, d]; pools [num_pages, page_size, H, d]; any float dtype, widened to fp64 exactly.
    Returns (out [n, H, d], lse [n, H]) in fp64, natural log; with ``want_sumw2`` also
    sumw2 [n, H], the sum of the squared softmax weights of each row (no part of the attention:
    the tests size the LSE's rounding spread with it)."""
    H, d = int(table.num_heads), int(table.head_dim)
    qd, kd, vd = _f64(q), _f64(k_pool), _f64(v_pool)
    lq = int(sum(int(table.chunk_tokens[c]) for c in table.query_chunks))
    assert qd.shape == (lq, H, d), (qd.shape, lq, H, d)
    assert kd.shape == (table.num_pages, table.page_size, H, d) and vd.shape == kd.shape
    rows = np.arange(lq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.shape[0], H, d), np.float64)
    lse = np.empty((rows.shape[0], H), np.float64)
    w2 = np.empty((rows.shape[0], H), np.float64) if want_sumw2 else None
    ints = [np.ascontiguousarray(a, np.int32) for a in (table.chunk_tokens, table.chunk_order,
                                                        table.page_offsets, table.page_ids,
                                                        table.query_chunks)]
    rc = lib().oracle_attn_rows(len(ints[0]), _p(ints[0], _i32p), _p(ints[1], _i32p),
                                _p(ints[2], _i32p), _p(ints[3], _i32p), int(table.num_pages),
                                int(table.page_size), len(ints[4]), _p(ints[4], _i32p), H, d,
                                resolve_scale(table), _p(qd, _f64p), _p(kd, _f64p), _p(vd, _f64p),
                                rows.shape[0], _p(rows, _i64p), _p(out, _f64p), _p(lse, _f64p),
                                None if w2 is None else _p(w2, _f64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_rows failed with code %d" % rc)
    return (out, lse, w2) if want_sumw2 else (out, lse)


def publish_kv(table, chunk: int, k_src, v_src, k_pool, v_pool):
    """Place chunk ``chunk``'s keys and values, [tokens, H, d] in token order, into its pages:
    token u goes to physical page page_ids[page_offsets[chunk] + u // page_size], slot
    u % page_size (the producer writes into the consumer's fixed slots: Wave Forcing project
    page, "03 - End-to-end KV transport", panel "03 - Layout").  Returns new pools (numpy, the
    inputs' dtype); every other slot keeps its value."""
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    ks, vs = np.asarray(k_src), np.asarray(v_src)
    first = int(table.page_offsets[chunk])
    for u in range(int(table.chunk_tokens[chunk])):
        page = int(table.page_ids[first + u // int(table.page_size)])
        kp[page, u % int(table.page_size)] = ks[u]
        vp[page, u % int(table.page_size)] = vs[u]
    return kp, vp


def rotate_pairs(x, cos_t, sin_t):
    """Rotary embedding of x [tokens, H, d] (any float; widened exactly to float32) by per-token,
    per-pair angles given as cos_t, sin_t [tokens, d/2].  The pages take Q and K as already
    rotated and do not define the rotation; this is the usual rotary formula on adjacent channel
    pairs, the reading the fused pre-attention epilogue implements: channel pair (2i, 2i+1) becomes
    (x0 c - x1 s, x0 s + x1 c).  Each product and each sum is one float32 operation (numpy
    float32 arithmetic rounds every operation to nearest-even; nothing is fused), so the result is
    the float32 value of that formula.  Returns float32 [tokens, H, d]."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos_t, dtype=np.float32)[:, None, :]
    s = np.asarray(sin_t, dtype=np.float32)[:, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = (x0 * c) - (x1 * s)
    out[..., 1::2] = (x0 * s) + (x1 * c)
    return out


def qkv_project(x, w, heads: int, head_dim: int):
    """The QKV projection in fp64: x [tokens, hidden] times w [hidden, 3*H*d] (columns ordered
    (q|k|v, head, channel)), a plain matrix product, as [tokens, 3, H, d] float64.  The producer
    computes it right before publishing K/V (KipQuest paper page, "The deep dive")."""
    xd, wd = _f64(x), _f64(w)
    return (xd @ wd).reshape(xd.shape[0], 3, int(heads), int(head_dim))


def attn_masked(q, k, v, allowed, scale: float, nthreads: int = 0):
    """Softmax attention by its definition with an explicit 0/1 mask, one head: q [nq, d], k/v
    [nk, d], allowed [nq, nk] bool.  The pins feed it masks built independently of the chunk
    walk."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    al = np.ascontiguousarray(allowed, dtype=np.uint8)
    nq, d = qd.shape
    nk = kd.shape[0]
    out = np.empty((nq, d), np.float64)
    lse = np.empty((nq,), np.float64)
    rc = lib().oracle_attn_masked(nq, nk, d, float(scale), _p(qd, _f64p), _p(kd, _f64p),
                                  _p(vd, _f64p), _p(al, _u8p), _p(out, _f64p), _p(lse, _f64p),
                                  int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_masked failed with code %d" % rc)
    return out, lse


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 code (OCP 8-bit floating point, E4M3FN), in fp64."""
    c = np.asarray(codes, dtype=np.uint8).ravel()
    L = lib()
    return np.array([L.oracle_e4m3_decode(int(x)) for x in c], dtype=np.float64).reshape(np.shape(codes))


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each float32 value, ties to even, saturating to +-448, NaN kept."""
    a = np.asarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.oracle_e4m3_encode(float(v)) for v in a], dtype=np.uint8).reshape(np.shape(x))


def quantize_e4m3(x):
    """Block quantizer of the FP8 K/V transport (project page, "03 - End-to-end KV transport",
    "Precision" panel), one fp32 scale per (64 consecutive rows, head): amax/448, codes = e4m3 of
    x * (448/amax).  x [rows, H, d] (bf16 values; any float dtype) -> (x8 uint8 [rows,H,d],
    scales f32 [ceil(rows/64),H])."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    xf = np.ascontiguousarray(x, dtype=np.float32)
    rows, H, d = xf.shape
    x8 = np.empty(xf.shape, np.uint8)
    sc = np.empty(((rows + 63) // 64, H), np.float32)
    rc = lib().oracle_quantize_e4m3(_p(xf, _f32p), rows, H, d, _p(x8, _u8p), _p(sc, _f32p))
    if rc != 0:
        raise ValueError("oracle_quantize_e4m3 failed with code %d" % rc)
    return x8, sc


def dequantize_e4m3(x8, scales) -> np.ndarray:
    """decode(code) * scale of its (64-row block, head), in fp64: the values the e4m3 path means."""
    x8 = np.ascontiguousarray(x8, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    rows, H, d = x8.shape
    y = np.empty(x8.shape, np.float64)
    rc = lib().oracle_dequantize_e4m3(_p(x8, _u8p), _p(sc, _f32p), rows, H, d, _p(y, _f64p))
    if rc != 0:
        raise ValueError("oracle_dequantize_e4m3 failed with code %d" % rc)
    return y


# Slot of key k inside its 64-key block of the e4m3 V pool: within each 32-key half the 8-key
# groups are stored in the order 0, 2, 1, 3 (a layout choice of the e4m3 K/V storage, written out
# here from its statement, not derived from the GPU code).
_V8_GROUP_SLOT = (0, 2, 1, 3)


def v8_slot(key: int) -> int:
    half, grp, j = key // 32, (key // 8) % 4, key % 8
    return 32 * half + 8 * _V8_GROUP_SLOT[grp] + j


def quantize_v8(x):
    """e4m3 V pool of the e4m3 K/V storage (project page, "03 - End-to-end KV transport",
    "Precision" panel: FP8 K/V) from pool rows x [rows, H, d] (rows a multiple of 64; NaN marks
    padding slots): the block quantizer's codes and scales (``quantize_e4m3``: one scale per 64
    rows and head), a NaN value's code set to 0, then each (64-row block, head) laid out channel by
    channel with key k of the block at slot ``v8_slot(k)``.
    Returns (v8 uint8 [rows/64, H, d, 64], scales f32 [rows/64, H])."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    xf = np.ascontiguousarray(x, dtype=np.float32)
    rows, H, d = xf.shape
    if rows % 64:
        raise ValueError("rows must be a multiple of 64")
    x8, sc = quantize_e4m3(xf)
    x8[np.isnan(xf)] = 0
    blocks = x8.reshape(rows // 64, 64, H, d).transpose(0, 2, 3, 1)  # [block, H, d, key]
    out = np.empty(blocks.shape, np.uint8)
    for key in range(64):
        out[..., v8_slot(key)] = blocks[..., key]
    return out, sc


def dequantize_v8(v8, scales) -> np.ndarray:
    """Values of an e4m3 V pool in the layout of ``quantize_v8``, in pool row order [rows, H, d],
    fp64: decode(code) * scale of its (64-row block, head)."""
    v8 = np.asarray(v8, dtype=np.uint8)
    nb, H, d, _ = v8.shape
    lut = np.array([lib().oracle_e4m3_decode(c) for c in range(256)], np.float64)
    keys = np.empty((nb, H, d, 64), np.float64)
    for key in range(64):
        keys[..., key] = lut[v8[..., v8_slot(key)]]
    keys *= np.asarray(scales, np.float64)[:, :, None, None]
    return np.ascontiguousarray(keys.transpose(0, 3, 1, 2).reshape(nb * 64, H, d))


def merge_lse(o_parts, lse_parts):
    """Softmax over a union of disjoint key sets from the parts' normalised outputs and LSEs:
    out = sum_k exp(lse_k - lse) o_k, lse = log sum_k exp(lse_k) (an identity of the softmax; the
    pages print no formula).  o_parts [p, n, d], lse_parts [p, n] -> (out [n, d], lse [n])."""
    o = _f64(o_parts)
    l = _f64(lse_parts)
    p, n, d = o.shape
    out = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib().oracle_merge_lse(p, n, d, _p(o, _f64p), _p(l, _f64p), _p(out, _f64p), _p(lse, _f64p))
    if rc != 0:
        raise ValueError("oracle_merge_lse failed with code %d" % rc)
    return out, lse
