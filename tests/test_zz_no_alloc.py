"""wfattn_fwd_noalloc (the forward whose workspace is a device array inside the library) against
wfattn_fwd with a caller workspace: two calls in a row, the second with a smaller table, each
bit-identical to wfattn_fwd and within the oracle gates; a plan too large for the array is
refused before any device work."""
import numpy as np
import pytest
import torch

from block_causal_chunk_amd.inputs import fill_case, make_case, make_table
from helpers import check_bf16, check_lse, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_causal_chunk_amd import binding
    binding.lib()
    return binding


@pytest.fixture(scope="module")
def O():
    import oracle
    oracle.build()
    return oracle


def _medium(seed):
    rng = np.random.default_rng(seed)
    t = make_table([700, 650, 600, 500], [0, 1, 2, 3], [3, 2], 256, 3, 128, shuffle_rng=rng, spare=2)
    return fill_case("noalloc_medium", t, rng, torch.bfloat16)


def _noalloc(B, case, split_k=0):
    q, k, v = to_dev(case)
    t = case.table
    plan = B.wfattn_plan(t, split_k=split_k)
    out = torch.full((t.lq, t.num_heads, t.head_dim), float("nan"), dtype=q.dtype, device=q.device)
    lse = torch.full((t.num_heads, t.lq), float("nan"), dtype=torch.float32, device=q.device)
    dt = B.WFATTN_FP32 if q.dtype == torch.float32 else B.WFATTN_BF16
    B.wfattn_fwd_noalloc(plan, dt, q, k, v, out, lse)
    torch.cuda.synchronize()
    return out, lse, plan


def _with_workspace(B, case, split_k=0):
    q, k, v = to_dev(case)
    mode = B.WFATTN_WS_FP32 if q.dtype == torch.float32 else B.WFATTN_WS_BF16
    att = B.Attention(case.table, mode=mode, split_k=split_k)
    out, lse = att.fwd(q, k, v, want_lse=True)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_two_calls_second_smaller(B, O):
    big = _medium(5)                                   # 1,100 query rows, 3 heads, split-K merge
    small = make_case("tiny_fp32")                     # 192 rows, 2 heads, d 64, fp32 I/O
    for case, split in ((big, 3), (small, 0)):
        print(f"[case] noalloc {case.name} split_k={split}", flush=True)
        out, lse, _ = _noalloc(B, case, split)
        ref_out, ref_lse = _with_workspace(B, case, split)
        assert torch.equal(out.view(torch.int32) if out.dtype == torch.float32 else out.view(torch.int16),
                           ref_out.view(torch.int32) if ref_out.dtype == torch.float32 else ref_out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        if case.io_dtype == torch.float32:
            bq, bk, bv = (x.to(torch.bfloat16) for x in (case.q, case.k_pool, case.v_pool))
            ref, r_lse, r_w2 = O.attn_rows(case.table, bq, bk, bv, want_sumw2=True)
        else:
            ref, r_lse, r_w2 = O.attn_rows(case.table, case.q, case.k_pool, case.v_pool, want_sumw2=True)
        check_bf16(f64(out), ref, case.name)
        check_lse(f64(lse).T, r_lse, r_w2, case.name)


def test_noalloc_refuses_a_plan_beyond_the_array(B):
    c = make_case("wan13b_task", small=True)
    plan = B.wfattn_plan(c.table)
    need = plan.workspace_bytes(B.WFATTN_WS_FP32)
    assert need <= B.WFATTN_NOALLOC_MAX_BYTES
    # wave_round in fp32 I/O needs its bf16 staging copies (hundreds of MB): refused, nothing run
    from block_causal_chunk_amd.inputs import WORKLOADS
    w = WORKLOADS["wave_round"]
    t = make_table(w["tokens"], list(range(len(w["tokens"]))), w["queries"], w["page"], w["H"], w["d"],
                   spare=w["spare"])
    big = B.wfattn_plan(t)
    assert big.workspace_bytes(B.WFATTN_WS_FP32) > B.WFATTN_NOALLOC_MAX_BYTES
    fake = 1 << 20  # aligned, never dereferenced: the size check comes first
    st = B.lib().wfattn_fwd_noalloc(big.handle, B.WFATTN_FP32, fake, fake, fake, fake, None, None)
    assert st == B.WFATTN_ERR_WORKSPACE
