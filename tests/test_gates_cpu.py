"""The LSE gate of the GPU tests (helpers.check_lse), checked on the CPU: an emulation of the
kernel's row sum (weights exp(s - m) against the first 64-key tile's max, each rounded to bf16,
summed in fp32) passes it, while the same emulation with one chunk's tail keys dropped -- a
shift that on average sits under the per-row worst-case cap -- fails it.  Here the table has 1,800 visible
keys, so dropping 6 of them matches the relative shift of dropping 72 of C2's 18,720."""
import numpy as np
import pytest
import torch

from block_causal_chunk_amd.inputs import fill_case, make_table
from helpers import LSE_CAP, check_lse


def _kernel_like_lse(t, q, k_pool, drop_tail=0):
    """lse per (row, head) the way the kernel forms it, from scores computed here in fp64."""
    H, d, P = t.num_heads, t.head_dim, t.page_size
    qd = q.double().numpy()
    kd = k_pool.double().numpy()
    keys = []
    a = int(t.query_chunks[0])
    vis = [b for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a]]
    for b in vis:
        n = int(t.chunk_tokens[b]) - (drop_tail if b == vis[0] else 0)
        for u in range(n):
            keys.append(kd[int(t.page_ids[int(t.page_offsets[b]) + u // P]), u % P])
    keys = np.stack(keys)  # [nk, H, d]
    s = np.einsum("qhd,khd->qhk", qd, keys) / np.sqrt(d)
    m = s[:, :, :64].max(-1, keepdims=True)
    p = torch.from_numpy(np.exp(s - m)).to(torch.float32).to(torch.bfloat16).to(torch.float32)
    l = p.sum(-1).numpy().astype(np.float64)
    return m[..., 0] + np.log(l)


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(5)
    t = make_table([600, 600, 600], [0, 1, 2], [2], 256, 2, 64, shuffle_rng=rng, spare=1)
    return fill_case("gate", t, rng, torch.bfloat16)


def test_rounding_emulation_passes(oracle_lib, case):
    t = case.table
    _, ref_lse, w2 = oracle_lib.attn_rows(t, case.q, case.k_pool, case.v_pool, want_sumw2=True)
    got = _kernel_like_lse(t, case.q, case.k_pool)
    mean, mx = check_lse(got, ref_lse, w2, "emulation")
    assert mean < 1.0 and mx < 5.0


def test_dropped_tail_keys_fail(oracle_lib, case):
    t = case.table
    _, ref_lse, w2 = oracle_lib.attn_rows(t, case.q, case.k_pool, case.v_pool, want_sumw2=True)
    got = _kernel_like_lse(t, case.q, case.k_pool, drop_tail=6)
    assert np.abs(got - ref_lse).mean() < LSE_CAP  # on average under the per-row cap
    with pytest.raises(AssertionError):
        check_lse(got, ref_lse, w2, "dropped tail")
