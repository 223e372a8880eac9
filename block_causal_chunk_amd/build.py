"""Build libwfattn.so (and the benchmark's probe, libwfprobe.so) in-tree with hipcc for gfx950
(runs on a host without a GPU)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwfattn.so")
SOURCES = ["plan.cpp", "api.hip", "attn_fwd.hip", "quant.hip", "publish.hip", "qkv.hip"]
PROBE_LIB = os.path.join(HERE, "libwfprobe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # never emit packed fp32 math (v_pk_fma_f32 & co.)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in VGPRs: with AGPR-form accumulators the allocator moves the
            # O tile between AGPRs and VGPRs around every MFMA group of the attention loop
            "-mllvm", "-amdgpu-mfma-vgpr-form=true",
            # keep the two specialisations of the attention tile's front half apart: sinking their
            # common tail into the join block would separate the exponentials from the MFMAs they
            # are meant to overlap
            "-mllvm", "-simplifycfg-sink-common=false",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n" + r.stdout)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libwfattn.so and libwfprobe.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
