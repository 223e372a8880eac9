"""Benchmark of block-causal chunk attention (libwfattn.so) on one MI355X.

One step = one wfattn_fwd call (every kernel of the hot path) over one DiT layer's attention of
one chunk-stage task, with inputs resident in HBM; the plan and its upload are built once per
round and timed separately.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--cold] [--no-configs]
                  [--no-cpu-baseline] [--no-extras]

Default workload: the Wan-1.3B chunk task (H=12, d=128, 4680 query tokens of one chunk against
18720 keys of the own chunk and three earlier ones, 256-token shuffled pages), bf16.  Before it,
the same run measures the other full-size workloads (the mixed-noise wave round, the long
rollout, the 14B-shaped e4m3 task) and the headline workload with a cold Infinity Cache; they go
into the line's "configs" object.  Every figure is a p50 over the timed calls (the pages report
p50 over steady ticks); the roofline prices the attention kernel's mean event-timed launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6  # TFLOP/s, dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8 = 5033.2
PEAK_MIXED = 3355.4  # e4m3 Q.K^T at the fp8 rate, P.V at the bf16 rate (equal FLOPs)


def effective_flops(table) -> float:
    """4 * d * H * sum over query chunks of tokens x visible keys (unmasked pairs only)."""
    t = table
    tot = 0
    for a in t.query_chunks:
        vis = sum(int(t.chunk_tokens[b]) for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a])
        tot += int(t.chunk_tokens[a]) * vis
    return 4.0 * t.head_dim * t.num_heads * tot


def gather_bytes(table, k_bytes: int, v_bytes: int = 2) -> tuple:
    """(K/V bytes staged into LDS per call, unique visible K/V bytes per call).  Every query tile of
    up to 256 rows of one head loads the 64-key tiles of its visible prefix (a tile never crosses a
    page), K at k_bytes and V at v_bytes per element."""
    t = table
    d, H = t.head_dim, t.num_heads
    tiles = []
    for c in range(t.num_chunks):
        tok = int(t.chunk_tokens[c])
        n = 0
        for p0 in range(0, tok, t.page_size):
            n += -(-min(t.page_size, tok - p0) // 64)
        tiles.append(n)
    staged = 0
    visible = set()
    for a in t.query_chunks:
        pre = [b for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a]]
        visible.update(pre)
        staged += H * -(-int(t.chunk_tokens[a]) // 256) * sum(tiles[b] for b in pre) * 64 * d * (k_bytes + v_bytes)
    unique = sum(int(t.chunk_tokens[b]) for b in visible) * H * d * (k_bytes + v_bytes)
    return staged, unique


def kernel_src_hash() -> str:
    h = hashlib.sha256()
    for f in ["attn_fwd.hip", "device.hpp", "kernels.hpp", "plan.cpp", "plan.hpp"]:
        h.update(open(os.path.join(ROOT, "block_causal_chunk_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str = ""):
    """Beyond-L2 bytes per call (attention + merge launches), or per launch of `kernel`, from the
    committed rocprofv3 counter summary, if it was taken with the current kernel sources; else
    None."""
    p = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("kernel_src_sha") != kernel_src_hash():
        return None
    if kernel:
        k = d.get("kernels", {}).get(kernel)
        return None if k is None else k["fetch_bytes"] + k["write_bytes"]
    return d.get("hbm_bytes_per_call")


def mfma_counters_from_profiles(workload: str):
    """MFMA busy fraction, VALU co-issue share and active clock of the attention kernel from the
    committed rocprofv3 counter summary, if it was taken with the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_mfma_util.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("kernel_src_sha") != kernel_src_hash():
        return None
    keys = ("mfma_busy_frac", "valu_coexec_frac_of_mfma_busy", "active_clock_ghz", "l2_hit_rate",
            "lds_bank_conflict_ratio")
    return {k: d[k] for k in keys if k in d}


def rope_publish(B, att, t, k_pool, k8_pool, k_scale, v, reps: int = 20):
    """Outside the timed steps: the fused pre-attention epilogue of the (first) query chunk, from a
    [tokens, 3, H, d] projection output: rotate Q and K, write Q (bf16, or e4m3 with block scales
    when k8_pool is given) and publish K (bf16 or e4m3) and V into the pages.  HBM-bound."""
    import torch
    H, d = t.num_heads, t.head_dim
    a = int(t.query_chunks[0])
    n = int(t.chunk_tokens[a])
    dev = v.device
    qkv = torch.randn((n, 3, H, d), device=dev).to(torch.bfloat16)
    th = torch.rand((n, d // 2), device=dev) * 6.283185307179586
    cos_t, sin_t = torch.cos(th), torch.sin(th)
    e4m3 = k8_pool is not None
    q_out = None if e4m3 else torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    q8 = torch.empty((n, H, d), dtype=torch.uint8, device=dev) if e4m3 else None
    qs = torch.empty(((n + 63) // 64, H), dtype=torch.float32, device=dev) if e4m3 else None
    kp = None if e4m3 else k_pool.clone()
    k8p = k8_pool.clone() if e4m3 else None
    ksp = k_scale.clone() if e4m3 else None
    vp = v.clone()

    def call():
        B.wfattn_rope_publish(att.plan, a, qkv, cos_t, sin_t, q_out, q8, qs, kp, k8p, ksp, vp, None, 0, att.ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    elems = n * H * d
    nbytes = 3 * elems * 2 + 2 * n * (d // 2) * 4 + elems * (1 if e4m3 else 2) + elems * (1 if e4m3 else 2) + elems * 2
    return {"rope_publish": {"chunk_tokens": n, "q_and_k": "e4m3" if e4m3 else "bf16", "ms": round(ms, 4),
                             "bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(nbytes / (ms * 1e-3) / 8e12, 4)}}


def qkv_fused(B, att, t, k_pool, v, reps: int = 20):
    """Outside the timed steps: the producer's QKV projection of the (first) query chunk with the
    pre-attention epilogue fused (wfattn_qkv_rope_publish: x [tokens, H*d] . W [H*d, 3*H*d] on the
    matrix cores, rotation, bf16 Q out, K and V into the pages), against the same work in two
    passes: torch's matmul (the vendor GEMM) writing the [tokens, 3, H, d] projection, then
    wfattn_rope_publish reading it back.  Both timed with HIP events, blocks alternated."""
    import numpy as np
    import torch
    H, d = t.num_heads, t.head_dim
    a = int(t.query_chunks[0])
    n = int(t.chunk_tokens[a])
    hid = H * d
    dev = v.device
    x = torch.randn((n, hid), device=dev).to(torch.bfloat16)
    w = (torch.randn((hid, 3 * hid), device=dev) / hid ** 0.5).to(torch.bfloat16)
    th = torch.rand((n, d // 2), device=dev) * 6.283185307179586
    cos_t, sin_t = torch.cos(th), torch.sin(th)
    q_out = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    kp, vp = k_pool.clone(), v.clone()
    qkv = torch.empty((n, 3 * hid), dtype=torch.bfloat16, device=dev)

    def fused():
        B.wfattn_qkv_rope_publish(att.plan, a, x, w, cos_t, sin_t, q_out, None, None, kp, None, None, vp, None, 0,
                                  att.ws)

    def two_pass():
        torch.matmul(x, w, out=qkv)
        B.wfattn_rope_publish(att.plan, a, qkv, cos_t, sin_t, q_out, None, None, kp, None, None, vp, None, 0, att.ws)

    def gemm_only():
        torch.matmul(x, w, out=qkv)

    for f in (fused, two_pass):
        for _ in range(5):
            f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = {"fused": [], "two_pass": [], "gemm_only": []}
    for _ in range(3):
        for name, f in (("fused", fused), ("two_pass", two_pass), ("gemm_only", gemm_only)):
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / reps)
    ms = {k: float(np.median(v)) for k, v in times.items()}
    flop = 2.0 * n * hid * 3 * hid
    inter = n * 3 * hid * 2  # the [tokens, 3, H, d] bf16 projection, written then read back
    return {"qkv_rope_publish": {"chunk_tokens": n, "hidden": hid, "fused_ms": round(ms["fused"], 4),
                                 "fused_tflops": round(flop / (ms["fused"] * 1e-3) / 1e12, 1),
                                 "fused_frac_of_bf16_peak": round(flop / (ms["fused"] * 1e-3) / 1e12 / PEAK_BF16, 4),
                                 "two_pass_ms": round(ms["two_pass"], 4),
                                 "vendor_gemm_alone_ms": round(ms["gemm_only"], 4),
                                 "intermediate_bytes_avoided": 2 * inter}}


def publish_fp8(B, att, t, q, k8, ks, v, reps: int = 20):
    """Outside the timed steps: wfattn_publish_kv_fp8 of the query chunk (K quantized to e4m3 per
    64-token block and head into the K8 pool, V copied), HBM-bound: 2 B read + 1 B written per K
    element, 2 + 2 B per V element, plus the scales."""
    import torch
    H, d = t.num_heads, t.head_dim
    a = int(t.query_chunks[0])
    n = int(t.chunk_tokens[a])
    sk = torch.randn((n, H, d), device=q.device).to(torch.bfloat16)
    sv = torch.randn((n, H, d), device=q.device).to(torch.bfloat16)
    k8p, ksp, vp = k8.clone(), ks.clone(), v.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        B.wfattn_publish_kv_fp8(att.plan, a, sk, sv, k8p, ksp, vp, None, 0, att.ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        B.wfattn_publish_kv_fp8(att.plan, a, sk, sv, k8p, ksp, vp, None, 0, att.ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = n * H * d * (2 + 1 + 2 + 2) + (-(-n // 64)) * H * 4
    return {"publish_kv_fp8": {"chunk_tokens": n, "ms": round(ms, 4), "bytes": nbytes,
                               "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                               "hbm_frac": round(nbytes / (ms * 1e-3) / 8e12, 4)}}


def publish_and_gate(B, att, t, q, k, v, reps: int = 20):
    """Outside the timed steps: (1) wfattn_publish_kv of the (first) query chunk's K/V from
    projection layout into its pages, an HBM-bound copy (read + write of K and V); (2) the gated
    forward with every flag ready, timed in alternating blocks with the plain forward so that both
    run at the same clock.  On the current stream, with HIP events."""
    import numpy as np
    import torch
    H, d = t.num_heads, t.head_dim
    a = int(t.query_chunks[0])
    n = int(t.chunk_tokens[a])
    sk = torch.randn((n, H, d), device=q.device).to(torch.bfloat16)
    sv = torch.randn((n, H, d), device=q.device).to(torch.bfloat16)
    kp, vp = k.clone(), v.clone()
    flags = torch.zeros(t.num_chunks, dtype=torch.int32, device=q.device)
    need = torch.ones(t.num_chunks, dtype=torch.int32, device=q.device)
    status = torch.zeros(1, dtype=torch.int32, device=q.device)
    out = torch.empty((t.lq, H, d), dtype=torch.bfloat16, device=q.device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        B.wfattn_publish_kv(att.plan, a, sk, sv, kp, vp, flags, 1, att.ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        B.wfattn_publish_kv(att.plan, a, sk, sv, kp, vp, flags, 1, att.ws)
    e1.record()
    torch.cuda.synchronize()
    pub_ms = e0.elapsed_time(e1) / reps
    pub_bytes = 2 * 2 * n * H * d * 2  # K and V, read and written, bf16
    # the same bytes through torch's device copy, as the reference for a copy of this size
    dk, dv = torch.empty_like(sk), torch.empty_like(sv)
    for _ in range(3):
        dk.copy_(sk)
        dv.copy_(sv)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dk.copy_(sk)
        dv.copy_(sv)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    flags.fill_(1)

    def gated():
        B.wfattn_fwd_gated(att.plan, q, k, v, out, None, att.ws, flags, need, 0, status)

    def plain():
        B.wfattn_fwd(att.plan, B.WFATTN_BF16, q, k, v, out, None, att.ws)

    # the clock ramps over ~30 calls: warm up, then alternate blocks so both see the same clock
    for _ in range(40):
        gated()
    times = {"gated": [], "plain": []}
    for _ in range(4):
        for name, f in (("gated", gated), ("plain", plain)):
            e0.record()
            for _ in range(reps // 2):
                f()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / (reps // 2))
    assert int(status.item()) == 0
    return {"publish_kv": {"chunk_tokens": n, "ms": round(pub_ms, 4), "bytes": pub_bytes,
                           "gbs": round(pub_bytes / (pub_ms * 1e-3) / 1e9, 1),
                           "hbm_frac": round(pub_bytes / (pub_ms * 1e-3) / 8e12, 4),
                           "torch_copy_same_bytes_gbs": round(pub_bytes / (copy_ms * 1e-3) / 1e9, 1)},
            "gated_fwd": {"ms": round(float(np.median(times["gated"])), 4),
                          "ungated_ms_same_run": round(float(np.median(times["plain"])), 4)}}


_PROBE = None


def probe_lib():
    """libwfprobe.so, the measurement probes built beside the attention library."""
    global _PROBE
    if _PROBE is None:
        import ctypes
        path = os.path.join(ROOT, "block_causal_chunk_amd", "libwfprobe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        L.wfprobe_exp_rate.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.wfprobe_exp_rate.restype = ctypes.c_int64
        L.wfprobe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.wfprobe_copy.restype = ctypes.c_int32
        _PROBE = L
    return _PROBE


def exp_peak_per_s(blocks: int = 2048, iters: int = 2048, reps: int = 5) -> float:
    """v_exp_f32 the chip retires per second with nothing else running, measured by the probe
    library built beside the attention library (8 workgroups of 256 lanes per CU, 8 independent
    chains per lane); the best of `reps` event-timed launches."""
    import torch
    L = probe_lib()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    n = L.wfprobe_exp_rate(out.data_ptr(), blocks, iters, stream)  # warm-up
    if n <= 0:
        raise RuntimeError("wfprobe_exp_rate failed")
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.wfprobe_exp_rate(out.data_ptr(), blocks, iters, stream)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, n / (e0.elapsed_time(e1) * 1e-3))
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("exp probe produced non-finite values")
    return best


def cpu_baseline(case, budget_s: float = 15.0, min_s: float = 10.0):
    """The oracle, as it stands, on a bounded sample of query rows of the same workload: the sample
    grows until one timed run takes at least min_s seconds (aiming at budget_s), or covers every
    row."""
    import numpy as np

    import oracle
    oracle.build()
    t = case.table
    q = case.q.double().numpy()
    k = case.k_pool.double().numpy()
    v = case.v_pool.double().numpy()
    lq = t.lq
    rng = np.random.default_rng(0)
    n = 16
    while True:
        rows = np.sort(rng.choice(lq, size=min(n, lq), replace=False))
        t0 = time.perf_counter()
        oracle.attn_rows(t, q, k, v, rows=rows)
        dt = time.perf_counter() - t0
        if dt >= min_s or n >= lq:
            break
        n = min(lq, int(n * min(8.0, max(1.2, budget_s / max(dt, 1e-3)))))
    # FLOPs of the sampled rows: each row sees the visible keys of its chunk
    qstart = np.concatenate([[0], np.cumsum([int(t.chunk_tokens[a]) for a in t.query_chunks])])
    vis = []
    for a in t.query_chunks:
        vis.append(sum(int(t.chunk_tokens[b]) for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a]))
    flops = sum(4.0 * t.head_dim * t.num_heads * vis[int(np.searchsorted(qstart, r, side="right") - 1)] for r in rows)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=oracle.max_threads(), kind="oracle",
                sample=f"{len(rows)} of {lq} query rows (all {t.num_heads} heads), fp64, {dt:.1f} s",
                seconds=dt, cpu=cpu_model())


def cpu_model() -> str:
    """Model name of the host CPU and the logical CPUs this process may use."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{name}, {len(os.sched_getaffinity(0))} logical CPUs available"


CONFIG_STEPS, CONFIG_WARMUP = 100, 30  # per workload of the "configs" object


def prepare(B, name, split_k=0, xcd_remap=0, dev="cuda:0"):
    """Build workload `name` on the device, plan it and upload the plan (quantize Q and the K pool
    for the e4m3 workload): everything a timed call needs, so that the calls of several workloads
    can then be timed back to back."""
    import torch

    from block_causal_chunk_amd.inputs import make_case

    case = make_case(name)
    t = case.table
    fp8 = name in ("wan14b_fp8", "wan14b_fp8kv")
    kv8 = name == "wan14b_fp8kv"  # V stored as e4m3 too
    f32 = case.io_dtype == torch.float32
    q, k, v = case.q.to(dev), case.k_pool.to(dev), case.v_pool.to(dev)
    H, d = t.num_heads, t.head_dim

    tp0 = time.perf_counter()
    mode = B.WFATTN_WS_FP8 if fp8 else (B.WFATTN_WS_FP32 if f32 else B.WFATTN_WS_BF16)
    att = B.Attention(t, device=dev, mode=mode, split_k=split_k, xcd_remap=xcd_remap)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - tp0) * 1e3
    summary = att.plan.describe(0)

    out = torch.empty((t.lq, H, d), dtype=torch.bfloat16 if not f32 else torch.float32, device=dev)
    quant_ms = None
    k8 = ks = None
    if fp8:
        rows = k.shape[0] * k.shape[1]
        kv = k.view(rows, H, d)
        k8 = torch.empty((rows, H, d), dtype=torch.uint8, device=dev)
        ks = torch.empty(((rows + 63) // 64, H), dtype=torch.float32, device=dev)
        q8, qs = B.quantize_q_fp8(t, q)
        B.wfattn_quantize_fp8(kv, rows, H, d, k8, ks)
        torch.cuda.synchronize()
        # quantization of the K pool timed on its own (it is HBM-bound and runs once per chunk)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            B.wfattn_quantize_fp8(kv, rows, H, d, k8, ks)
        e1.record()
        torch.cuda.synchronize()
        quant_ms = e0.elapsed_time(e1) / 10
        k8 = k8.view(k.shape)
        if kv8:
            v8, vs = B.quantize_v_fp8(v)

            def step():
                B.wfattn_fwd_fp8kv(att.plan, q8, qs, k8, ks, v8, vs, out, None, att.ws)

            def step_marked(ev):
                B.wfattn_fwd_fp8kv_marked(att.plan, q8, qs, k8, ks, v8, vs, out, None, att.ws, ev.cuda_event)
        else:
            def step():
                B.wfattn_fwd_fp8(att.plan, q8, qs, k8, ks, v, out, None, att.ws)

            def step_marked(ev):
                B.wfattn_fwd_fp8_marked(att.plan, q8, qs, k8, ks, v, out, None, att.ws, ev.cuda_event)
    else:
        dt = B.WFATTN_FP32 if f32 else B.WFATTN_BF16

        def step():
            B.wfattn_fwd(att.plan, dt, q, k, v, out, None, att.ws)

        def step_marked(ev):
            B.wfattn_fwd_marked(att.plan, dt, q, k, v, out, None, att.ws, ev.cuda_event)

    torch.cuda.synchronize()
    return dict(name=name, case=case, att=att, q=q, k=k, v=v, k8=k8, ks=ks, fp8=fp8, kv8=kv8, f32=f32, step=step,
                step_marked=step_marked, plan_ms=plan_ms, summary=summary, quant_ms=quant_ms)


def measure(prep, steps, warmup, cold=False, dev="cuda:0"):
    """Time `steps` calls of a prepared workload after `warmup` untimed ones, each bracketed by HIP
    events on the launch stream, plus an event the library records between the attention launch
    and the merge launch.  Returns the figures."""
    import numpy as np
    import torch
    name, case, step, step_marked = prep["name"], prep["case"], prep["step"], prep["step_marked"]
    t = case.table
    fp8, f32 = prep["fp8"], prep["f32"]
    H, d = t.num_heads, t.head_dim
    plan_ms, summary, quant_ms = prep["plan_ms"], prep["summary"], prep["quant_ms"]
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    # one more event per step, recorded by the library between the attention launch and the merge
    # launch (recorded once here so that it exists), to time the attention kernel on its own
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for ev in mids:
        ev.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            scratch.fill_(i & 0xFF)  # untimed 512 MB write evicts the Infinity Cache
        starts[i].record()
        step_marked(mids[i])
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del scratch
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms per call, stream events
    per_attn = np.array([s.elapsed_time(m) for s, m in zip(starts, mids)])  # the attention kernel alone
    p50 = float(np.median(per))
    attn_ms = float(per_attn.mean())
    flops = effective_flops(t)
    peak = PEAK_FP8 if fp8 else PEAK_BF16
    kflops = flops / (attn_ms * 1e-3) / 1e12
    r = {
        "workload": name, "cache": "cold" if cold else "warm", "steps": steps, "warmup": warmup,
        "heads": H, "head_dim": d, "query_tokens": t.lq, "key_tokens": int(sum(int(x) for x in t.chunk_tokens)),
        "query_chunks": len(t.query_chunks), "page_size": t.page_size,
        "dtype": ("e4m3 Q/K/V storage, e4m3 QK^T, bf16 PV" if prep["kv8"] else "e4m3 QK^T, bf16 PV") if fp8
        else ("bf16 (fp32 I/O)" if f32 else "bf16"),
        "p10_ms": round(float(np.percentile(per, 10)), 4), "p50_ms": round(p50, 4),
        "p90_ms": round(float(np.percentile(per, 90)), 4), "mean_ms": round(float(per.mean()), 4),
        "tflops": round(flops / (p50 * 1e-3) / 1e12, 2),
        "frac_of_peak": round(flops / (p50 * 1e-3) / 1e12 / peak, 4),
        "tasks_per_s": round(len(t.query_chunks) / (p50 * 1e-3), 1),
        "effective_gflop_per_step": round(flops / 1e9, 3),
        "plan_and_upload_ms": round(plan_ms, 3),
        "plan": {"items": int(summary[0]), "key_tiles": int(summary[1]), "merge_groups": int(summary[2]),
                 "splits": int(summary[6]), "block_m": int(summary[4]), "block_n": int(summary[5])},
        # the dominant kernel: effective FLOPs over the attention kernel's own mean event-timed launch
        "roofline": {"bound": "mfma", "achieved": round(kflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(kflops / peak, 4),
                     "traffic": traffic_from_profiles(name, "attn_fwd_kernel"),
                     "kernel": "attn_fwd_kernel", "kernel_ms": round(attn_ms, 4),
                     "kernel_p50_ms": round(float(np.median(per_attn)), 4),
                     "merge_ms": round(float(per.mean()) - attn_ms, 4)},
        "wall_s_timed": round(wall, 3),
    }
    if fp8:
        # e4m3 Q.K^T at the fp8 rate, P.V at the bf16 rate: the bound the workload's mix allows
        r["roofline"]["frac_of_mixed_bound"] = round(kflops / PEAK_MIXED, 4)
        r["roofline"]["mixed_bound"] = PEAK_MIXED
        r["quantize_k_pool_ms"] = round(quant_ms, 4)
    staged, unique = gather_bytes(t, 1 if fp8 else 2, 1 if prep["kv8"] else 2)
    traffic = traffic_from_profiles(name)
    sec = p50 * 1e-3
    r["gather"] = {"lds_staged_bytes": staged, "lds_staged_gbs": round(staged / sec / 1e9, 1),
                   "kv_unique_bytes": unique, "kv_unique_gbs": round(unique / sec / 1e9, 1),
                   "beyond_l2_gbs": None if traffic is None else round(traffic / sec / 1e9, 1),
                   "beyond_l2_bytes_per_call": traffic}
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="wan13b_task")
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=0)
    ap.add_argument("--cold", action="store_true", help="evict the 256 MB Infinity Cache between steps")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the headline workload (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the publish and gated-forward measurements (profiling runs)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds the oracle sample aims at (at least 10)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 256 MiB copy kernel (3 times) so that a "
                         "counter run can scale FETCH_SIZE/WRITE_SIZE against known bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on exactly one GPU (it has no collectives and no sharding); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_causal_chunk_amd import binding as B
    from block_causal_chunk_amd.inputs import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    dev = torch.device("cuda:0")

    # Every workload is built and planned first (host work, during which the GPU idles and its
    # clock falls back); then the calls run back to back: the other full-size workloads and the
    # headline workload with a cold cache (their figures go into "configs"), and the headline last,
    # so that its warm-up starts at the clock the chip holds under this load rather than from idle.
    names = [] if args.no_configs else [n for n in WORKLOADS if n not in (args.workload, "tiny_fp32")]
    preps = {}
    for name in names:
        print(f"bench: building {name}", file=sys.stderr, flush=True)
        preps[name] = prepare(B, name, dev=dev)
    print(f"bench: building {args.workload}", file=sys.stderr, flush=True)
    head = prepare(B, args.workload, split_k=args.split_k, xcd_remap=args.xcd_remap, dev=dev)
    configs = {}
    for name in names:
        print(f"bench: measuring {name}", file=sys.stderr, flush=True)
        configs[name] = measure(preps[name], CONFIG_STEPS, CONFIG_WARMUP, dev=dev)
    if names and not args.cold:
        print(f"bench: measuring {args.workload} (cold cache)", file=sys.stderr, flush=True)
        configs[args.workload + "_cold"] = measure(head, CONFIG_STEPS // 2, CONFIG_WARMUP, cold=True, dev=dev)
    print(f"bench: measuring {args.workload} (headline)", file=sys.stderr, flush=True)
    r = measure(head, args.steps, args.warmup, cold=args.cold, dev=dev)
    preps.clear()
    torch.cuda.empty_cache()
    case, att, t = head["case"], head["att"], head["case"].table
    q, k, v, k8, ks, fp8, f32 = (head[x] for x in ("q", "k", "v", "k8", "ks", "fp8", "f32"))
    H, d = t.num_heads, t.head_dim
    if args.copy_calibration:
        # the probe library's plain copy kernel, 256 MiB, so that a counter run can scale its
        # memory counters by what they read for known bytes
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            if probe_lib().wfprobe_copy(dst.data_ptr(), src.data_ptr(), src.numel(), stream) != 0:
                raise RuntimeError("wfprobe_copy failed")
        torch.cuda.synchronize()
        if not bool(torch.equal(src, dst)):
            raise RuntimeError("calibration copy is wrong")
        del src, dst
    extra = {}
    if not (f32 or args.no_extras):
        extra = publish_fp8(B, att, t, q, k8, ks, v) if fp8 else publish_and_gate(B, att, t, q, k, v)
        extra.update(rope_publish(B, att, t, None if fp8 else k, k8 if fp8 else None, ks if fp8 else None, v))
        if not fp8:
            extra.update(qkv_fused(B, att, t, k, v))
    exp_peak = exp_peak_per_s()
    p50 = r["p50_ms"]
    flops = effective_flops(t)
    tflops = flops / (p50 * 1e-3) / 1e12  # the whole call (attention + merge) at the p50 call
    exps = flops / (4.0 * d)  # one exponential per unmasked (query row, key, head)
    counters = mfma_counters_from_profiles(args.workload)
    peak = r["roofline"]["peak"]
    if counters is not None:
        # the roofline peak again at the clock the kernel actually ran at under load
        counters["peak_at_active_clock"] = round(peak * counters["active_clock_ghz"] / 2.4, 1)
        counters["frac_at_active_clock"] = round(r["roofline"]["achieved"] / counters["peak_at_active_clock"], 4)
    res = {
        "metric": "effective attention TFLOP/s + chunk-tasks/s, Wan-1.3B shape, % MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["p50_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic, seeded N(0,1) Q/K/V, shuffled 256-token pages",
        "config": {"workload": args.workload, "heads": H, "head_dim": d,
                   "query_tokens": t.lq, "key_tokens": r["key_tokens"],
                   "query_chunks": len(t.query_chunks), "page_size": t.page_size,
                   "cache": r["cache"]},
        "value_stat": "p50 of the timed calls",
        "frac_of_peak": r["frac_of_peak"],
        "tasks_per_s": r["tasks_per_s"],
        "p10_ms": r["p10_ms"], "p50_ms": r["p50_ms"], "p90_ms": r["p90_ms"], "mean_ms": r["mean_ms"],
        "effective_gflop_per_step": r["effective_gflop_per_step"],
        "plan_and_upload_ms": r["plan_and_upload_ms"],
        "plan": r["plan"],
        "roofline": r["roofline"],
        "mfma_counters": counters,
        "exps_per_s": round(exps / (p50 * 1e-3), 1),
        "exp_peak_per_s": round(exp_peak, 1),
        "exp_frac": round(exps / (p50 * 1e-3) / exp_peak, 4),
        "gather": r["gather"],
        "wall_s_timed": r["wall_s_timed"],
    }
    if fp8:
        res["quantize_k_pool_ms"] = r["quantize_k_pool_ms"]
    res.update(extra)
    if configs:
        res["configs"] = configs
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
        res["cpu_baseline"]["value"] = round(res["cpu_baseline"]["value"], 6)
        res["cpu_baseline"]["seconds"] = round(res["cpu_baseline"]["seconds"], 2)
        res["cpu_baseline"]["gpu_over_cpu"] = round(tflops / res["cpu_baseline"]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
