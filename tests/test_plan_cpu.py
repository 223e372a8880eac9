"""Host-side tests of libwfattn.so: exported symbols, every error a host can force, and the
schedule's coverage of the block-causal mask.  No compute call is made (no GPU here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_causal_chunk_amd.inputs import make_case, make_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from block_causal_chunk_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from block_causal_chunk_amd import build
        build.build()
    return binding


def test_exports_every_declared_symbol(B):
    hdr = open(os.path.join(ROOT, "include", "wfattn.h")).read()
    declared = set(re.findall(r"\b(wfattn_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(B.EXPORTED)
    L = B.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert L.wfattn_abi_version() == 3
    for s in range(8):
        assert B.status_str(s) and B.status_str(s) != "unknown status"


def test_probe_library_exports_and_rejects_bad_arguments(B):
    """The benchmark's exp-rate probe: every symbol wfprobe.h declares is exported, and bad
    arguments are refused before any HIP call."""
    from block_causal_chunk_amd import build
    path = build.PROBE_LIB
    if not os.path.exists(path):
        build.build()
    hdr = open(os.path.join(ROOT, "include", "wfprobe.h")).read()
    declared = set(re.findall(r"\b(wfprobe_[a-z0-9_]+)\s*\(", hdr))
    L = ctypes.CDLL(path)
    assert declared == {"wfprobe_exp_rate", "wfprobe_copy"}
    for name in declared:
        assert hasattr(L, name), name
    L.wfprobe_exp_rate.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.wfprobe_exp_rate.restype = ctypes.c_int64
    buf = (ctypes.c_float * 256)()
    assert L.wfprobe_exp_rate(None, 1, 1, None) == -1
    assert L.wfprobe_exp_rate(ctypes.addressof(buf), 0, 1, None) == -1
    assert L.wfprobe_exp_rate(ctypes.addressof(buf), 1, 0, None) == -1
    L.wfprobe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    L.wfprobe_copy.restype = ctypes.c_int32
    a = ctypes.addressof(buf)
    assert L.wfprobe_copy(None, a, 16, None) == -1
    assert L.wfprobe_copy(a, None, 16, None) == -1
    assert L.wfprobe_copy(a, a + 16 * 8, 0, None) == -1
    assert L.wfprobe_copy(a, a + 16 * 8, 24, None) == -1
    assert L.wfprobe_copy(a + 4, a + 16 * 8, 16, None) == -1


def _plan_status(B, t, **opts):
    c, keep = B.make_table_c(t)
    o = B.OptsC(opts.get("split_k", 0), opts.get("xcd_remap", 0), opts.get("order_ties", 0), opts.get("num_cus", 0),
                opts.get("num_xcds", 0), opts.get("block_m", 0), opts.get("block_n", 0))
    h = ctypes.c_void_p()
    st = B.lib().wfattn_plan(ctypes.byref(c), ctypes.byref(o), ctypes.byref(h))
    if st == 0:
        B.lib().wfattn_plan_free(h)
    return st


def _base():
    return make_table([100, 70, 130], [0, 1, 2], [1, 2], 64, 2, 128, shuffle_rng=np.random.default_rng(1), spare=2)


def test_plan_errors(B):
    assert _plan_status(B, _base()) == B.WFATTN_OK
    L = B.lib()
    h = ctypes.c_void_p()
    assert L.wfattn_plan(None, None, ctypes.byref(h)) == B.WFATTN_ERR_NULL
    c, keep = B.make_table_c(_base())
    assert L.wfattn_plan(ctypes.byref(c), None, None) == B.WFATTN_ERR_NULL
    c.page_ids = None
    assert L.wfattn_plan(ctypes.byref(c), None, ctypes.byref(h)) == B.WFATTN_ERR_NULL

    def mod(**kw):
        t = _base()
        for k, v in kw.items():
            setattr(t, k, v)
        return _plan_status(B, t)

    assert mod(chunk_tokens=np.array([100, 0, 130], np.int32)) == B.WFATTN_ERR_INVALID
    assert mod(chunk_order=np.array([0, 1, 1], np.int32)) == B.WFATTN_ERR_INVALID  # a tie
    assert mod(chunk_order=np.array([0, 1, 3], np.int32)) == B.WFATTN_ERR_INVALID
    t = _base()
    t.page_offsets = np.array([0, 2, 3, 6], np.int32)  # chunk 1 needs 2 pages, gets 1
    assert _plan_status(B, t) == B.WFATTN_ERR_INVALID
    assert mod(query_chunks=np.array([1, 1], np.int32)) == B.WFATTN_ERR_INVALID
    assert mod(query_chunks=np.array([3], np.int32)) == B.WFATTN_ERR_INVALID
    assert mod(query_chunks=np.array([], np.int32)) == B.WFATTN_ERR_INVALID  # no query chunk
    assert mod(num_heads=0) == B.WFATTN_ERR_INVALID
    assert mod(softmax_scale=float("nan")) == B.WFATTN_ERR_INVALID
    t = _base()
    t.page_ids = t.page_ids.copy()
    t.page_ids[3] = t.num_pages  # out of range
    assert _plan_status(B, t) == B.WFATTN_ERR_RANGE
    t.page_ids[3] = t.page_ids[0]  # reused
    assert _plan_status(B, t) == B.WFATTN_ERR_RANGE
    assert mod(head_dim=96) == B.WFATTN_ERR_UNSUPPORTED
    t = make_table([100, 70], [0, 1], [1], 32, 2, 128)  # page_size not a multiple of 64
    assert _plan_status(B, t) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), order_ties=2) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), order_ties=-1) == B.WFATTN_ERR_UNSUPPORTED
    # the kernels' tiles are fixed: block_m / block_n accept 0 or those values only
    assert _plan_status(B, _base(), block_m=256, block_n=64) == B.WFATTN_OK
    assert _plan_status(B, _base(), block_m=128) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), block_n=32) == B.WFATTN_ERR_UNSUPPORTED
    # device geometry: the XCD count must divide the CU count
    assert _plan_status(B, _base(), num_cus=84, num_xcds=8) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), num_cus=-1) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), num_cus=4097) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), num_cus=64, num_xcds=2) == B.WFATTN_OK
    # ties only where asked for; an order outside [0, num_chunks) stays invalid either way
    t = _base()
    t.chunk_order = np.array([0, 1, 1], np.int32)
    assert _plan_status(B, t, order_ties=1) == B.WFATTN_OK
    t.chunk_order = np.array([1, 1, 1], np.int32)
    assert _plan_status(B, t, order_ties=1) == B.WFATTN_OK
    t.chunk_order = np.array([0, 1, 3], np.int32)
    assert _plan_status(B, t, order_ties=1) == B.WFATTN_ERR_INVALID
    t.chunk_order = np.array([0, -1, 1], np.int32)
    assert _plan_status(B, t, order_ties=1) == B.WFATTN_ERR_INVALID
    assert _plan_status(B, _base(), split_k=-1) == B.WFATTN_ERR_UNSUPPORTED
    assert _plan_status(B, _base(), xcd_remap=2) == B.WFATTN_ERR_UNSUPPORTED
    t = make_table([100], [0], [0], 64, 2, 128)
    t.num_pages = 2 ** 26  # pool rows overflow int32
    assert _plan_status(B, t) == B.WFATTN_ERR_RANGE


def test_call_errors_before_any_hip_call(B):
    """Every check except DEVICE fires before the first HIP call, so fake addresses are safe."""
    plan = B.wfattn_plan(_base())
    L = B.lib()
    ws_need = plan.workspace_bytes(B.WFATTN_WS_BF16)
    assert ws_need > 0 and plan.workspace_bytes(B.WFATTN_WS_FP32) > ws_need
    assert plan.workspace_bytes(9) == 0
    A = 1 << 20  # a fake, aligned address that is never dereferenced
    h = plan.handle
    assert L.wfattn_fwd(h, 0, None, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd(None, 0, A, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd(h, 5, A, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd(h, 0, A + 8, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd(h, 0, A, A, A, A, A + 2, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd(h, 0, A, A, A, A, None, A + 16, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd(h, 0, A, A, A, A, None, None, ws_need, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_fwd(h, 0, A, A, A, A, None, A, ws_need - 1, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_fwd(h, 1, A, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_WORKSPACE  # fp32 needs staging
    bogus = ctypes.create_string_buffer(64)  # not a plan
    assert L.wfattn_fwd(ctypes.addressof(bogus), 0, A, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_INVALID
    assert L.wfattn_fwd_fp8(h, A, A, A, None, A, A, None, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd_fp8(h, A, A + 2, A, A, A, A, None, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd_fp8(h, A, A, A, A, A, A, None, A, 16, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_plan_upload(h, None, ws_need, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_plan_upload(h, A + 64, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_plan_upload(h, A, 8, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_plan_upload(None, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_quantize_fp8(None, 10, 2, 128, A, A, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_quantize_fp8(A, 10, 2, 96, A, A, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_quantize_fp8(A, -1, 2, 128, A, A, None) == B.WFATTN_ERR_RANGE
    assert L.wfattn_quantize_fp8(A, 10, 0, 128, A, A, None) == B.WFATTN_ERR_RANGE
    # publishing a chunk's K/V
    P = L.wfattn_publish_kv
    assert P(None, 1, A, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert P(h, 1, None, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert P(h, 1, A, A, A, None, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert P(ctypes.addressof(bogus), 1, A, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID
    assert P(h, 3, A, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID  # 3 chunks: ids 0..2
    assert P(h, -1, A, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID
    assert P(h, 1, A + 8, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert P(h, 1, A, A, A, A, A + 2, 3, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert P(h, 1, A, A, A, A, A, 3, None, ws_need, None) == B.WFATTN_ERR_WORKSPACE
    assert P(h, 1, A, A, A, A, A, 3, A, ws_need - 1, None) == B.WFATTN_ERR_WORKSPACE
    P8 = L.wfattn_publish_kv_fp8
    assert P8(h, 1, A, A, None, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert P8(h, 1, A, A, A, None, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert P8(h, 7, A, A, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID
    assert P8(h, 1, A, A, A, A + 2, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert P8(h, 1, A, A, A + 8, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert P8(h, 1, A, A, A, A, A, A, 3, None, ws_need, None) == B.WFATTN_ERR_WORKSPACE
    R = L.wfattn_rope_publish
    assert R(h, 1, None, A, A, A, A, A, A, None, None, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL
    assert R(h, 1, A, A, A, A, A, A, A, A, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID  # both K forms
    assert R(h, 1, A, A, A, A, A, A, None, None, A, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID  # neither
    assert R(h, 1, A, A, A, A, A, None, A, None, None, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL  # q8, no scale
    assert R(h, 1, A, A, A, A, None, None, None, A, None, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_NULL  # k8, no scale
    assert R(h, 9, A, A, A, A, None, None, A, None, None, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_INVALID
    assert R(h, 1, A, A + 8, A, A, None, None, A, None, None, A, A, 3, A, ws_need, None) == B.WFATTN_ERR_UNSUPPORTED
    assert R(h, 1, A, A, A, A, None, None, A, None, None, A, A, 3, A, 8, None) == B.WFATTN_ERR_WORKSPACE
    # the marked forwards (an event between the attention and the merge launches)
    assert L.wfattn_fwd_marked(h, 0, A, A, A, A, None, A, ws_need, None, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd_marked(h, 0, A + 8, A, A, A, None, A, ws_need, A, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd_fp8_marked(h, A, A, A, A, A, A, None, A, ws_need, None, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd_fp8_marked(h, A, A, A, A, A, A, None, A, 16, A, None) == B.WFATTN_ERR_WORKSPACE
    # the gated forward
    G = L.wfattn_fwd_gated
    assert G(h, A, A, A, A, None, A, ws_need, None, A, 0, A, None) == B.WFATTN_ERR_NULL
    assert G(h, A, A, A, A, None, A, ws_need, A, A, 0, None, None) == B.WFATTN_ERR_NULL
    assert G(h, A, A, A, A, None, A, ws_need, A, A, -1, A, None) == B.WFATTN_ERR_RANGE
    assert G(h, A, A, A, A, None, A, ws_need, A, A, B.WFATTN_GATE_SPIN_MAX + 1, A, None) == B.WFATTN_ERR_RANGE
    assert G(h, A, A, A, A, None, A, ws_need, A + 2, A, 0, A, None) == B.WFATTN_ERR_UNSUPPORTED
    assert G(h, None, A, A, A, None, A, ws_need, A, A, 0, A, None) == B.WFATTN_ERR_NULL
    assert G(h, A, A, A, A, None, A, ws_need - 1, A, A, 0, A, None) == B.WFATTN_ERR_WORKSPACE
    # the gated e4m3 forward
    G8 = L.wfattn_fwd_fp8_gated
    assert G8(h, A, A, A, A, A, A, None, A, ws_need, None, A, 0, A, None) == B.WFATTN_ERR_NULL
    assert G8(h, A, A, A, A, A, A, None, A, ws_need, A, A, 0, None, None) == B.WFATTN_ERR_NULL
    assert G8(h, A, A, A, A, A, A, None, A, ws_need, A, A, -1, A, None) == B.WFATTN_ERR_RANGE
    assert G8(h, A, A, A, A, A, A, None, A, ws_need, A, A, B.WFATTN_GATE_SPIN_MAX + 1, A, None) == B.WFATTN_ERR_RANGE
    assert G8(h, A, A, A, A, A, A, None, A, ws_need, A + 2, A, 0, A, None) == B.WFATTN_ERR_UNSUPPORTED
    assert G8(h, None, A, A, A, A, A, None, A, ws_need, A, A, 0, A, None) == B.WFATTN_ERR_NULL
    assert G8(h, A, A, A, A, A, A, None, A, 16, A, A, 0, A, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_quantize_fp8(A + 8, 10, 2, 128, A, A, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_quantize_fp8(A, 0, 2, 128, A, A, None) == B.WFATTN_OK  # nothing to do, no launch
    assert L.wfattn_query_rows(None) == -1
    assert L.wfattn_workspace_bytes(None, 0) == 0
    n = ctypes.c_size_t()
    assert L.wfattn_plan_describe(h, 7, None, 0, ctypes.byref(n)) == B.WFATTN_ERR_INVALID


def _owner_of_pool_row(t):
    """physical pool row -> (chunk, token) for every valid slot."""
    own = {}
    for b in range(t.num_chunks):
        for lp in range(int(t.page_offsets[b]), int(t.page_offsets[b + 1])):
            u0 = (lp - int(t.page_offsets[b])) * t.page_size
            for u in range(u0, min(u0 + t.page_size, int(t.chunk_tokens[b]))):
                own[int(t.page_ids[lp]) * t.page_size + u - u0] = (b, u)
    return own


def _check_tiles_vectorized(t, items, tiles, own, bm, bn):
    """Tile-level form of the exhaustive check for big tables: each key tile lies in one page of
    one chunk, the tiles of the clean -> noisy prefix of query chunk a cover exactly the tokens of
    the chunks visible to a, each once."""
    tile_chunk = np.empty(len(tiles), np.int64)
    for k, (row0, nv) in enumerate(tiles):
        b0, u0 = own[int(row0)]
        b1, u1 = own[int(row0) + int(nv) - 1]
        assert b0 == b1 and u1 == u0 + nv - 1
        tile_chunk[k] = b0
    for head, r0, rows, qsb, qi, nt, _, _ in items:
        a = int(t.query_chunks[qi])
        ch = tile_chunk[:nt]
        assert (t.chunk_order[ch] <= t.chunk_order[a]).all()
        vis = [b for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a]]
        assert int(tiles[:nt, 1].sum()) == sum(int(t.chunk_tokens[b]) for b in vis)
        assert set(ch.tolist()) == set(vis)


def _check_schedule(B, t, **kw):
    plan = B.wfattn_plan(t, **kw)
    summ = [int(x) for x in plan.describe(0)]
    n_items, n_tiles, n_groups, n_parts, bm, bn, max_parts, nqc, n_segs, n_wgs = summ
    items = plan.describe(1).reshape(-1, 8)
    tiles = plan.describe(2).reshape(-1, 2)
    groups = plan.describe(3).reshape(-1, 4)
    segs = plan.describe(4).reshape(-1, 4)
    ranges = plan.describe(5).reshape(-1, 2)
    assert items.shape[0] == n_items and tiles.shape[0] == n_tiles and groups.shape[0] == n_groups
    assert segs.shape[0] == n_segs and ranges.shape[0] == n_wgs and 1 <= n_wgs <= (kw.get("num_cus") or 256)
    # workgroup ranges partition the segment list in order
    assert ranges[0, 0] == 0 and ranges[-1, 1] == n_segs
    assert (ranges[1:, 0] == ranges[:-1, 1]).all() and (ranges[:, 1] >= ranges[:, 0]).all()
    own = _owner_of_pool_row(t)
    qstart = np.concatenate([[0], np.cumsum([int(t.chunk_tokens[a]) for a in t.query_chunks])])
    for head, r0, rows, qsb, qi, nt, _, _ in items:
        assert 0 <= head < t.num_heads and 1 <= rows <= bm and 1 <= nt <= n_tiles
        assert qstart[qi] <= r0 and r0 + rows <= qstart[qi + 1]  # a query tile never crosses a chunk
        assert (r0 - qstart[qi]) % bm == 0
    # the segments of each item cover its key tiles exactly once
    cover = [np.zeros(int(it[5]), np.int32) for it in items]
    slots = {}
    for item, k0, k1, slot in segs:
        assert 0 <= k0 < k1 <= items[item][5]
        cover[item][k0:k1] += 1
        if slot >= 0:
            assert slot not in slots
            slots[int(slot)] = int(item)
    assert all((c == 1).all() for c in cover)
    n_pairs = sum(int(it[5]) for it in items) * bn
    if n_pairs > 2_000_000:
        _check_tiles_vectorized(t, items, tiles, own, bm, bn)
        return plan, items, tiles
    seen = {}
    for i, (head, r0, rows, qsb, qi, nt, _, _) in enumerate(items):
        a = int(t.query_chunks[qi])
        for kt in range(nt):
            row0, nv = tiles[kt]
            assert 1 <= nv <= bn
            b0, u0 = own[int(row0)]
            for j in range(nv):
                b, u = own[int(row0) + j]
                assert b == b0 and u == u0 + j  # a key tile never crosses a page or a chunk
                assert t.chunk_order[b] <= t.chunk_order[a]  # no masked pair is ever enumerated
                key = (int(head), int(r0), b, u)
                assert key not in seen  # exactly once
                seen[key] = True
    expect = 0
    for qi, a in enumerate(t.query_chunks):
        vis = sum(int(t.chunk_tokens[b]) for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a])
        n_qt = -(-int(t.chunk_tokens[a]) // bm)
        expect += vis * n_qt * t.num_heads
    assert len(seen) == expect
    assert len(slots) == n_parts
    # merge groups: exactly the items with more than one segment, slots contiguous per item
    nseg = np.bincount(segs[:, 0], minlength=n_items)
    assert set(int(g[0]) for g in groups) == set(int(i) for i in np.nonzero(nseg > 1)[0])
    for item, s0, parts, _ in groups:
        assert parts == nseg[item] and parts <= max_parts
        assert all(slots[s] == item for s in range(s0, s0 + parts))
    return plan, items, tiles


@pytest.mark.parametrize("name", ["tiny_fp32", "wan13b_task", "wave_round", "long_rollout", "wan14b_fp8"])
def test_schedule_covers_mask_small(B, name):
    c = make_case(name, small=True)
    for split in (0, 1, 3):
        for x in (0, -1):
            _check_schedule(B, c.table, split_k=split, xcd_remap=x)


def test_schedule_random_tables(B):
    rng = np.random.default_rng(5)
    for _ in range(10):
        n = int(rng.integers(1, 7))
        tok = rng.integers(1, 400, size=n)
        t = make_table(tok, rng.permutation(n), rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False),
                       int(rng.choice([64, 128, 256])), int(rng.integers(1, 4)), int(rng.choice([64, 128])),
                       shuffle_rng=rng, spare=int(rng.integers(0, 4)))
        _check_schedule(B, t, split_k=int(rng.integers(0, 5)))


def test_schedule_random_tables_with_ties(B):
    """Equal orders (a bidirectional window): every query chunk of a tie group sees the whole group
    and every cleaner chunk, each key once, and never a noisier chunk."""
    rng = np.random.default_rng(6)
    for _ in range(10):
        n = int(rng.integers(1, 8))
        tok = rng.integers(1, 300, size=n)
        order = rng.integers(0, max(1, n // 2) + 1, size=n).clip(0, n - 1)
        t = make_table(tok, order, rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False),
                       int(rng.choice([64, 128])), int(rng.integers(1, 3)), int(rng.choice([64, 128])),
                       shuffle_rng=rng, spare=int(rng.integers(0, 3)))
        _check_schedule(B, t, split_k=int(rng.integers(0, 4)), order_ties=1)
    # a window of three tied chunks after a clean history: each window query tile gets the same prefix
    t = make_table([100, 64, 200, 130, 90, 70], [0, 1, 2, 2, 2, 3], [4, 2, 3], 64, 1, 128)
    plan, items, tiles = _check_schedule(B, t, order_ties=1)
    assert len(set(int(it[5]) for it in items)) == 1
    assert int(tiles[:int(items[0][5]), 1].sum()) == 100 + 64 + 200 + 130 + 90


def test_chunk_table_of_the_plan(B):
    """describe(6): per chunk its first key tile, tokens, rank in clean -> noisy order and the last
    rank it sees; with ties, every chunk of a tie group sees to the group's end.  Items carry the
    last rank their query chunk sees (the gate's range)."""
    t = make_table([100, 64, 200, 130, 90, 70], [0, 1, 2, 2, 2, 3], [4, 2, 5], 64, 1, 128)
    plan = B.wfattn_plan(t, order_ties=1)
    ch = plan.describe(6).reshape(-1, 4)
    tiles = plan.describe(2).reshape(-1, 2)
    items = plan.describe(1).reshape(-1, 8)
    assert ch[:, 1].tolist() == [100, 64, 200, 130, 90, 70]
    assert ch[:, 2].tolist() == [0, 1, 2, 3, 4, 5]  # ranks: by order, ties by chunk id
    assert ch[:, 3].tolist() == [0, 1, 4, 4, 4, 5]
    for c in range(6):  # a chunk's tiles start at its first tile and cover its tokens
        n = -(-int(t.chunk_tokens[c]) // 64)
        assert int(tiles[ch[c, 0]:ch[c, 0] + n, 1].sum()) == int(t.chunk_tokens[c])
    for it in items:
        a = int(t.query_chunks[it[4]])
        assert it[6] == ch[a, 3]


def test_schedule_full_size_tables_and_xcd_grouping(B):
    """The five workloads' tables (sizes only; no values are drawn): coverage, balance across
    the 256 workgroups and the 8 XCDs, and few heads per XCD."""
    from block_causal_chunk_amd.inputs import WORKLOADS
    for name, w in WORKLOADS.items():
        t = make_table(w["tokens"], list(range(len(w["tokens"]))), w["queries"], w["page"], w["H"], w["d"],
                       shuffle_rng=np.random.default_rng(0), spare=w["spare"])
        plan, items, tiles = _check_schedule(B, t)
        segs = plan.describe(4).reshape(-1, 4)
        ranges = plan.describe(5).reshape(-1, 2)
        load = np.array([sum(int(segs[s][2] - segs[s][1]) + 3 for s in range(a, b)) for a, b in ranges])
        if name != "tiny_fp32":
            assert load.max() <= 1.12 * load.mean() + 16, (name, load.max(), load.mean())
            xcd = np.zeros(8)
            heads = [set() for _ in range(8)]
            for wg, (a, b) in enumerate(ranges):
                for sidx in range(a, b):
                    xcd[wg % 8] += segs[sidx][2] - segs[sidx][1]
                    heads[wg % 8].add(int(items[segs[sidx][0]][0]))
            assert xcd.max() <= 1.15 * xcd.mean(), (name, xcd)
            assert max(len(h) for h in heads) <= -(-w["H"] // 8) + 2, (name, heads)
    t = make_table([4680] * 4, [0, 1, 2, 3], [3], 256, 12, 128)
    tiles = B.wfattn_plan(t, split_k=1).describe(2).reshape(-1, 2)
    assert tiles.shape[0] == 4 * (18 * 4 + 2) and tiles[:, 1].sum() == 4 * 4680


def test_noalloc_forward_checks_before_any_device_call(B):
    """wfattn_fwd_noalloc decides NULL, INVALID, UNSUPPORTED and WORKSPACE (a plan needing more than
    its 64 MiB device array) on the host, before its first HIP call."""
    from block_causal_chunk_amd.inputs import WORKLOADS
    L = B.lib()
    w = WORKLOADS["wan13b_task"]
    t = make_table(w["tokens"], list(range(len(w["tokens"]))), w["queries"], w["page"], w["H"], w["d"],
                   spare=w["spare"])
    plan = B.wfattn_plan(t)
    fake = 1 << 20  # aligned, never dereferenced
    assert plan.workspace_bytes(B.WFATTN_WS_BF16) <= B.WFATTN_NOALLOC_MAX_BYTES
    assert plan.workspace_bytes(B.WFATTN_WS_FP32) > B.WFATTN_NOALLOC_MAX_BYTES
    assert L.wfattn_fwd_noalloc(plan.handle, B.WFATTN_FP32, fake, fake, fake, fake, None, None) == B.WFATTN_ERR_WORKSPACE
    assert L.wfattn_fwd_noalloc(None, B.WFATTN_BF16, fake, fake, fake, fake, None, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd_noalloc(plan.handle, B.WFATTN_BF16, fake, None, fake, fake, None, None) == B.WFATTN_ERR_NULL
    assert L.wfattn_fwd_noalloc(plan.handle, 7, fake, fake, fake, fake, None, None) == B.WFATTN_ERR_UNSUPPORTED
    assert L.wfattn_fwd_noalloc(plan.handle, B.WFATTN_BF16, fake + 8, fake, fake, fake, None, None) == \
        B.WFATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("cus,xcds", [(32, 1), (128, 4), (80, 0), (304, 8)])
def test_schedule_on_a_partitioned_or_other_device(B, cus, xcds):
    """A device with another CU / XCD count (a compute partition of the chip, another part):
    every workgroup index stays below the CU count, the mask is still covered exactly once, and
    the work is balanced over those CUs."""
    from block_causal_chunk_amd.inputs import WORKLOADS
    w = WORKLOADS["wan13b_task"]
    t = make_table(w["tokens"], list(range(len(w["tokens"]))), w["queries"], w["page"], w["H"], w["d"],
                   shuffle_rng=np.random.default_rng(0), spare=w["spare"])
    plan, items, tiles = _check_schedule(B, t, num_cus=cus, num_xcds=xcds)
    segs = plan.describe(4).reshape(-1, 4)
    ranges = plan.describe(5).reshape(-1, 2)
    assert ranges.shape[0] <= cus
    load = np.array([sum(int(segs[s][2] - segs[s][1]) + 3 for s in range(a, b)) for a, b in ranges])
    assert load.max() <= 1.12 * load.mean() + 16, (load.max(), load.mean())
