"""Host-side checks of bench.py: it refuses more than one GPU before touching a device, and its
profile lookups report counters only for the kernel sources they were taken with."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr and r.stdout == ""


def test_profile_lookups_follow_the_source_hash(tmp_path, monkeypatch):
    import bench
    w = "wan13b_task"
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{w}_hbm_traffic.json")
    d = json.load(open(path))
    if d["kernel_src_sha"] == bench.kernel_src_hash():
        k = d["kernels"]["attn_fwd_kernel"]
        assert bench.traffic_from_profiles(w, "attn_fwd_kernel") == k["fetch_bytes"] + k["write_bytes"]
        assert bench.traffic_from_profiles(w) == d["hbm_bytes_per_call"]
        assert bench.mfma_counters_from_profiles(w) is not None
    monkeypatch.setattr(bench, "kernel_src_hash", lambda: "0" * 16)
    assert bench.traffic_from_profiles(w) is None
    assert bench.traffic_from_profiles(w, "attn_fwd_kernel") is None


def test_effective_flops_of_the_chunk_task():
    """4 d H x query tokens x visible keys: 538.27 GFLOP for the Wan-1.3B chunk task."""
    import bench
    from block_causal_chunk_amd.inputs import make_case
    t = make_case("wan13b_task", small=False).table
    assert bench.effective_flops(t) == 4 * 128 * 12 * 4680 * 18720
