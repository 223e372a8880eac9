"""Shared helpers for the GPU tests: device placement, oracle comparison and the tolerance gates.

Gates (applied to the whole compared tensor, in fp64, against the oracle):
  contract, bf16: max |err| <= 1e-2 and mean |err| <= 1e-3
  contract, fp8 : cosine >= 0.999 and max |err| <= 5e-2  (oracle on the unquantized inputs)
  self, bf16    : mean |err| <= 2e-3*rms, cosine >= 0.99999, and per element
                  |err| <= 2^-7*|ref| + 3e-2*rms, rms = RMS of the oracle output.  bf16 has an
                  8-bit significand, so rounding the output costs at most 2^-8*|ref|; rounding P
                  to bf16 (with the normaliser summed over the same rounded weights) moves each
                  weight by at most ~2^-7 relative, which stays within 2^-8*|ref| more when one
                  key dominates (peaky rows, e.g. outlier K channels); the absolute 3e-2*rms
                  term covers rows whose output cancels towards 0.  On N(0,1) inputs output
                  rounding alone gives a mean of about 1.1e-3*rms, so the mean gate leaves ~2x
                  headroom and still fails a kernel that drops one chunk's 72 tail keys
                  (mean ~4.6e-2*rms).
  lse           : |err| <= LSE_TOL = 4e-3 (natural log).  The row sum is taken over the
                  bf16-rounded P, each within a factor 1 +- 2^-8 of the exact weight, so the
                  sum -- and exp(lse) -- is within that factor: |err| <= ln(1 + 2^-8) ~ 3.9e-3.
"""
from __future__ import annotations

import numpy as np
import torch

LSE_TOL = 4e-3


def stats(out, ref):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(out - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    cos = float(np.sum(out * ref) / (np.linalg.norm(out) * np.linalg.norm(ref)))
    return dict(max=float(err.max()), mean=float(err.mean()), rms=rms, cos=cos,
                nmax=float(err.max()) / rms, nmean=float(err.mean()) / rms)


def check_bf16(out, ref, what=""):
    s = stats(out, ref)
    assert np.isfinite(out).all(), what
    assert s["max"] <= 1e-2 and s["mean"] <= 1e-3, (what, "contract", s)
    assert s["nmean"] <= 2e-3 and s["cos"] >= 0.99999, (what, "self", s)
    err = np.abs(np.asarray(out, np.float64) - np.asarray(ref, np.float64))
    bound = 2.0 ** -7 * np.abs(ref) + 3e-2 * s["rms"]
    worst = float((err / bound).max())
    assert worst <= 1.0, (what, "self per-element", worst, s)
    return s


def check_contract_bf16(out, ref, what=""):
    s = stats(out, ref)
    assert np.isfinite(out).all(), what
    assert s["max"] <= 1e-2 and s["mean"] <= 1e-3, (what, "contract", s)
    return s


def check_fp8_contract(out, ref, what=""):
    s = stats(out, ref)
    assert np.isfinite(out).all(), what
    assert s["cos"] >= 0.999 and s["max"] <= 5e-2, (what, "fp8 contract", s)
    return s


def to_dev(case):
    return (case.q.cuda(), case.k_pool.cuda(), case.v_pool.cuda())


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(lq, block_m=128, n=40, seed=0):
    """Rows spread over the query tiles, plus tile edges and the ragged tail."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, block_m - 1, block_m, lq - 1, lq - 2, (lq // block_m) * block_m, lq // 2]
    rows = set(int(r) for r in edge if 0 <= r < lq)
    rows.update(int(r) for r in rng.choice(lq, size=min(n, lq), replace=False))
    return np.array(sorted(rows), np.int64)
