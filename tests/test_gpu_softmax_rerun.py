"""GPU parity of the softmax's overflow re-run.

The attention kernel takes each row's softmax reference m from the first key tile of a segment
and never rescales O; if a later tile scores far above that reference, the row sum reaches 2^64
(or P itself overflows to +inf) and the segment is computed again against the true row maxima.
These tests plant such keys: query row i is set to a sign vector u_i and a key in a late tile to
beta * u_i, so that the pair scores beta * sqrt(d) (scale 1/sqrt(d)) against N(0,1) scores
everywhere else.  Two levels:
  * ~50 nats above the rest: every P stays finite, but l >= 2^64 forces the re-run;
  * ~100 nats above: exp overflows fp32, so P = +inf (and O = inf or NaN) before the re-run.
Every element is compared with the fp64 oracle (the plain definition: project page, "01 - The
design gap", column C), for the bf16, fp32-I/O and e4m3 forwards, with split-K off, planner-chosen
and 3-way, and over a tied window.  The planted rows pass one key's V row through, so their
outputs are unit-scale: the relative self gates apply (helpers.check_bf16, contract=False), and
the planted rows themselves are checked against the oracle one by one.
"""
import numpy as np
import pytest
import torch

from block_causal_chunk_amd.inputs import fill_case, make_table
from helpers import check_bf16, check_lse, f64, to_dev

pytestmark = pytest.mark.gpu

LEVELS = {"l_over_2^64": 50.0, "p_inf": 100.0}  # planted score, in nats (the rest are ~N(0,1))


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


def _slot(t, chunk, u):
    """Pool (page, slot) of token u of `chunk`."""
    return int(t.page_ids[int(t.page_offsets[chunk]) + u // t.page_size]), u % t.page_size


def planted_case(level, seed, tied=False, d=128):
    """Three chunks of 320 tokens (five 64-key tiles each; 256-token pages, shuffled), H = 2.
    Strict order: chunk 2 is the query and sees chunks 0-2 (15 key tiles, so a 3-way split puts
    chunk 1's and chunk 2's tiles in later segments).  Tied: orders [0, 1, 1], queries [1, 2]; the
    window's chunks see each other both ways.  Planted pairs: (query row, key chunk, key token),
    keys late in their segment (never a segment's first tile)."""
    rng = np.random.default_rng(seed)
    tok, H = [320, 320, 320], 2
    order, queries = ([0, 1, 1], [1, 2]) if tied else ([0, 1, 2], [2])
    t = make_table(tok, order, queries, 256, H, d, shuffle_rng=rng, spare=2)
    c = fill_case(f"planted_{level}", t, rng, torch.bfloat16)
    beta = LEVELS[level] / np.sqrt(d)  # score = beta * |u|^2 / sqrt(d) = beta * sqrt(d)
    if tied:
        # rows of chunk 1 (rows 0..319) reach into chunk 2, the window partner; rows of chunk 2
        # (rows 320..639) into chunk 1
        plants = [(5, 2, 140), (200, 2, 300), (300, 2, 70), (330, 1, 200), (600, 1, 260)]
    else:
        plants = [(0, 2, 140), (63, 2, 200), (64, 2, 300), (255, 1, 230), (256, 2, 70), (319, 1, 100)]
    q = c.q.float()
    kp = c.k_pool.float()
    for i, (row, kc, u) in enumerate(plants):
        h = i % H
        sign = np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
        q[row, h] = torch.from_numpy(sign)
        page, slot = _slot(t, kc, u)
        kp[page, slot, h] = torch.from_numpy(beta * sign)
    c.q = q.to(torch.bfloat16)
    c.k_pool = kp.to(torch.bfloat16)
    return c, plants


def _dequantized(O, c):
    H, d = c.table.num_heads, c.table.head_dim
    rows = c.k_pool.shape[0] * c.k_pool.shape[1]
    k8, ks = O.quantize_e4m3(c.k_pool.reshape(rows, H, d))
    kdq = O.dequantize_e4m3(k8, ks).reshape(c.k_pool.shape)
    qdq, row = [], 0
    for a in c.table.query_chunks:
        n = int(c.table.chunk_tokens[a])
        x8, sc = O.quantize_e4m3(c.q[row:row + n])
        qdq.append(O.dequantize_e4m3(x8, sc))
        row += n
    return np.concatenate(qdq), kdq


def _check_planted_rows(got, ref, plants):
    """The planted rows are dominated by their key: the output is (almost) that key's V row."""
    for i, (row, _, _) in enumerate(plants):
        h = i % 2
        assert np.abs(got[row, h] - ref[row, h]).max() <= 2.0 ** -7 * np.abs(ref[row, h]).max() + 1e-3, (row, h)


@pytest.mark.parametrize("split_k", [1, 0, 3])
@pytest.mark.parametrize("level", list(LEVELS))
def test_rerun_bf16(B, O, level, split_k):
    c, plants = planted_case(level, 101)
    print(f"[case] softmax re-run bf16 level={level} split_k={split_k}", flush=True)
    ref, ref_lse, ref_w2 = O.attn_rows(c.table, c.q, c.k_pool, c.v_pool, want_sumw2=True)
    assert ref_lse.max() > LEVELS[level] - 5  # the plant took: some rows' lse sits near it
    q, k, v = to_dev(c)
    att = B.Attention(c.table, split_k=split_k)
    out, lse = att.fwd(q, k, v, want_lse=True)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.isfinite(got).all()
    check_bf16(got, ref, f"re-run bf16 {level}", contract=False)
    check_lse(f64(lse).T, ref_lse, ref_w2, f"re-run bf16 {level}")
    _check_planted_rows(got, ref, plants)


@pytest.mark.parametrize("split_k", [1, 0, 3])
@pytest.mark.parametrize("level", list(LEVELS))
def test_rerun_fp32_io(B, O, level, split_k):
    c, plants = planted_case(level, 103)
    c = type(c)(c.name, c.table, torch.float32, c.q.float(), c.k_pool.float(), c.v_pool.float())
    print(f"[case] softmax re-run fp32 I/O level={level} split_k={split_k}", flush=True)
    # the inputs are bf16 values, so the oracle on them is also the oracle on what the kernel uses
    ref, ref_lse, ref_w2 = O.attn_rows(c.table, c.q, c.k_pool, c.v_pool, want_sumw2=True)
    q, k, v = to_dev(c)
    att = B.Attention(c.table, mode=B.WFATTN_WS_FP32, split_k=split_k)
    out, lse = att.fwd(q, k, v, want_lse=True)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.isfinite(got).all()
    check_bf16(got, ref, f"re-run fp32 I/O {level}", contract=False)
    check_lse(f64(lse).T, ref_lse, ref_w2, f"re-run fp32 I/O {level}")
    _check_planted_rows(got, ref, plants)


@pytest.mark.parametrize("split_k", [1, 0, 3])
@pytest.mark.parametrize("level", list(LEVELS))
def test_rerun_e4m3(B, O, level, split_k):
    c, plants = planted_case(level, 107)
    t = c.table
    H, d = t.num_heads, t.head_dim
    print(f"[case] softmax re-run e4m3 level={level} split_k={split_k}", flush=True)
    qdq, kdq = _dequantized(O, c)
    ref, ref_lse, ref_w2 = O.attn_rows(t, qdq, kdq, c.v_pool, want_sumw2=True)
    q, k, v = to_dev(c)
    rows = k.shape[0] * k.shape[1]
    k8, ks = B.quantize_fp8(k.view(rows, H, d))
    q8, qs = B.quantize_q_fp8(t, q)
    att = B.Attention(t, mode=B.WFATTN_WS_FP8, split_k=split_k)
    out, lse = att.fwd_fp8(q8, qs, k8.view(k.shape), ks, v, want_lse=True)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.isfinite(got).all()
    check_bf16(got, ref, f"re-run e4m3 {level} (dequantized oracle)", contract=False)
    check_lse(f64(lse).T, ref_lse, ref_w2, f"re-run e4m3 {level}")
    _check_planted_rows(got, ref, plants)


@pytest.mark.parametrize("level", list(LEVELS))
def test_rerun_tied_window(B, O, level):
    c, plants = planted_case(level, 109, tied=True)
    t = c.table
    H, d = t.num_heads, t.head_dim
    ref, ref_lse, ref_w2 = O.attn_rows(t, c.q, c.k_pool, c.v_pool, want_sumw2=True)
    q, k, v = to_dev(c)
    for split in (1, 0, 3):
        print(f"[case] softmax re-run tied window bf16 level={level} split_k={split}", flush=True)
        att = B.Attention(t, split_k=split, order_ties=1)
        out, lse = att.fwd(q, k, v, want_lse=True)
        torch.cuda.synchronize()
        got = f64(out)
        assert np.isfinite(got).all()
        check_bf16(got, ref, f"re-run tied {level}", contract=False)
        check_lse(f64(lse).T, ref_lse, ref_w2, f"re-run tied {level}")
        _check_planted_rows(got, ref, plants)
    print(f"[case] softmax re-run tied window e4m3 level={level}", flush=True)
    qdq, kdq = _dequantized(O, c)
    ref8, ref8_lse, ref8_w2 = O.attn_rows(t, qdq, kdq, c.v_pool, want_sumw2=True)
    rows = k.shape[0] * k.shape[1]
    k8, ks = B.quantize_fp8(k.view(rows, H, d))
    q8, qs = B.quantize_q_fp8(t, q)
    att8 = B.Attention(t, mode=B.WFATTN_WS_FP8, order_ties=1)
    out8, lse8 = att8.fwd_fp8(q8, qs, k8.view(k.shape), ks, v, want_lse=True)
    torch.cuda.synchronize()
    got8 = f64(out8)
    assert np.isfinite(got8).all()
    check_bf16(got8, ref8, f"re-run tied e4m3 {level} (dequantized oracle)", contract=False)
    check_lse(f64(lse8).T, ref8_lse, ref8_w2, f"re-run tied e4m3 {level}")
    _check_planted_rows(got8, ref8, plants)
