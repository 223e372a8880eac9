"""Pins for the CPU oracle: each test ties it to something other than itself.

P1 dense explicit mask, P2 a library routine (torch SDPA in float64), P3 the single-chunk special
case, P4 closed forms, P5 permutation/page-shuffle invariance, P6 no reverse edge, P7
decomposition of a multi-chunk query set, P8 the e4m3 codec against the OCP definition and
torch's float8_e4m3fn, P9 merging key partitions through their LSEs, P10 ties in chunk order (full
attention when all tie, a tie group equals one merged chunk, SDPA), P11 placing a chunk's K/V
into its pages (round trip through the dense gather, rebuilding the input pool), P12 the rotary
embedding (special angles, complex multiplication), plus brute force on tiny
inputs, a hand-derived closed-form fixture, and checks that plausible mistakes would be caught.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_causal_chunk_amd.inputs import ChunkTable, fill_case, make_case, make_table

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

SMALL_NAMES = ["tiny_fp32", "wan13b_task", "wave_round", "long_rollout", "wan14b_fp8"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_table(rng, n, tokens_range=(5, 40), page_size=16, H=2, d=16, nq=None, spare=3):
    tokens = rng.integers(tokens_range[0], tokens_range[1] + 1, size=n)
    order = rng.permutation(n)
    nq = nq or rng.integers(1, n + 1)
    queries = rng.choice(n, size=nq, replace=False)
    return make_table(tokens, order, queries, page_size, H, d, shuffle_rng=rng, spare=spare)


def _contiguous_case(rng, tokens, order, queries, H, d):
    """One page per chunk of exactly its size is impossible for ragged sizes, so use page_size 1:
    then pool row p of an identity page table is token p of the chunk-by-chunk concatenation."""
    t = make_table(tokens, order, queries, 1, H, d, shuffle_rng=None, spare=0)
    return fill_case("contig", t, rng, torch.float32)


def _sdpa_mask(tokens, order, queries):
    owner = np.concatenate([np.full(t, b) for b, t in enumerate(tokens)])
    qc = np.concatenate([np.full(tokens[a], a) for a in queries])
    order = np.asarray(order)
    return torch.from_numpy(order[owner][None, :] <= order[qc][:, None])


# ---------------------------------------------------------------- P1: dense explicit mask
@pytest.mark.parametrize("name", SMALL_NAMES)
def test_p1_dense_mask_equals_chunked(oracle_lib, name):
    from oracle.dense import attn_dense
    c = make_case(name, small=True)
    o, l = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
    od, ld = attn_dense(c.table, c.q, c.k_pool, c.v_pool)
    assert np.abs(o - od).max() <= 1e-13
    assert np.abs(l - ld).max() <= 1e-13


def test_p1_dense_mask_random_tables(oracle_lib):
    from oracle.dense import attn_dense
    rng = np.random.default_rng(7)
    for _ in range(12):
        t = _random_table(rng, int(rng.integers(1, 6)))
        c = fill_case("rnd", t, rng, torch.float32)
        o, l = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
        od, ld = attn_dense(c.table, c.q, c.k_pool, c.v_pool)
        assert np.abs(o - od).max() <= 1e-13 and np.abs(l - ld).max() <= 1e-13


# ---------------------------------------------------------------- P2: library routine
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p2_sdpa_float64(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    n = 4
    tokens = list(rng.integers(8, 30, size=n))
    order = list(rng.permutation(n))
    queries = list(rng.choice(n, size=3, replace=False))
    H, d = 3, 32
    c = _contiguous_case(rng, tokens, order, queries, H, d)
    o, l = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
    keys = c.k_pool.double()[:, 0]  # page_size 1: [Lk, H, d]
    vals = c.v_pool.double()[:, 0]
    mask = _sdpa_mask(tokens, order, queries)
    q = c.q.double().transpose(0, 1)  # [H, Lq, d]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, keys.transpose(0, 1), vals.transpose(0, 1), attn_mask=mask)
    assert np.abs(o - ref.transpose(0, 1).numpy()).max() <= 1e-12
    # lse via torch.logsumexp of the masked scores
    s = (q @ keys.permute(1, 2, 0)) / math.sqrt(d)
    s = s.masked_fill(~mask, float("-inf"))
    assert np.abs(l - torch.logsumexp(s, dim=-1).T.numpy()).max() <= 1e-12


# ---------------------------------------------------------------- P10: ties in chunk order
# Chunks of equal order see each other both ways (the live bidirectional window of Rolling
# Forcing, Wave Forcing project page, "01 - The design gap", column "A - Live frontier"); the rule
# order[b] <= order[a] is unchanged.
def test_p10_all_tied_is_full_attention(oracle_lib):
    rng = np.random.default_rng(11)
    H, d, tokens = 2, 32, [9, 14, 6, 11]
    c = _contiguous_case(rng, tokens, [0, 0, 0, 0], [0, 1, 2, 3], H, d)
    o, l = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
    q = c.q.double().transpose(0, 1)
    k = c.k_pool.double()[:, 0].transpose(0, 1)
    v = c.v_pool.double()[:, 0].transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)  # no mask at all
    assert np.abs(o - ref.transpose(0, 1).numpy()).max() <= 1e-12
    s = (q @ k.transpose(1, 2)) / math.sqrt(d)
    assert np.abs(l - torch.logsumexp(s, dim=-1).T.numpy()).max() <= 1e-12


def test_p10_tie_group_equals_one_merged_chunk(oracle_lib):
    """Two tied chunks behave as one chunk holding both token sets: a table with the strict order
    the other pins cover gives the same outputs."""
    rng = np.random.default_rng(12)
    H, d = 2, 16
    tied = _contiguous_case(rng, [20, 17, 23, 11], [0, 1, 1, 2], [1, 2], H, d)
    merged = make_table([20, 40, 11], [0, 1, 2], [1], 1, H, d, shuffle_rng=None, spare=0)
    # page_size 1 and identity page tables: pool rows are the tokens chunk by chunk in both tables
    o_t, l_t = oracle_lib.attn_rows(tied.table, tied.q, tied.k_pool, tied.v_pool)
    o_m, l_m = oracle_lib.attn_rows(merged, tied.q, tied.k_pool, tied.v_pool)
    assert np.abs(o_t - o_m).max() <= 1e-13 and np.abs(l_t - l_m).max() <= 1e-13


@pytest.mark.parametrize("seed", [0, 1])
def test_p10_ties_sdpa_and_dense(oracle_lib, seed):
    from oracle.dense import attn_dense
    rng = np.random.default_rng(200 + seed)
    tokens = list(rng.integers(5, 25, size=6))
    order = [0, 1, 2, 2, 2, 3]
    queries = [4, 2, 5, 3]
    H, d = 2, 32
    c = _contiguous_case(rng, tokens, order, queries, H, d)
    o, l = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
    keys, vals = c.k_pool.double()[:, 0], c.v_pool.double()[:, 0]
    mask = _sdpa_mask(tokens, order, queries)
    q = c.q.double().transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, keys.transpose(0, 1), vals.transpose(0, 1), attn_mask=mask)
    assert np.abs(o - ref.transpose(0, 1).numpy()).max() <= 1e-12
    od, ld = attn_dense(c.table, c.q, c.k_pool, c.v_pool)
    assert np.abs(o - od).max() <= 1e-13 and np.abs(l - ld).max() <= 1e-13
    # the window really is two-way: the first query of chunk 4 sees chunk 2's keys, the first
    # query of chunk 2 (rows after chunk 4's) sees chunk 4's keys, and neither sees chunk 5
    m = mask.numpy()
    k2, k4, k5 = sum(tokens[:2]), sum(tokens[:4]), sum(tokens[:5])
    assert m[0, k2:k2 + tokens[2]].all() and m[tokens[4], k4:k4 + tokens[4]].all()
    assert not m[0, k5:].any() and not m[tokens[4], k5:].any()


# ---------------------------------------------------------------- P11: publishing K/V into pages
def test_p11_publish_round_trips_through_the_dense_gather(oracle_lib):
    """Publishing a chunk then reading the pool back with the dense form's gather gives the
    source rows; slots of other chunks and padding slots keep their values."""
    from oracle.dense import gather_keys
    rng = np.random.default_rng(21)
    t = make_table([70, 129, 64, 5], [1, 0, 3, 2], [0], 64, 2, 16, shuffle_rng=rng, spare=3)
    kp = rng.standard_normal((t.num_pages, t.page_size, 2, 16))
    vp = rng.standard_normal(kp.shape)
    c = 1
    ks = rng.standard_normal((int(t.chunk_tokens[c]), 2, 16))
    vs = rng.standard_normal(ks.shape)
    k2, v2 = oracle_lib.publish_kv(t, c, ks, vs, kp, vp)
    gk, owner = gather_keys(t, k2)
    gv, _ = gather_keys(t, v2)
    assert (gk[owner == c] == ks).all() and (gv[owner == c] == vs).all()
    gk0, _ = gather_keys(t, kp)
    assert (gk[owner != c] == gk0[owner != c]).all()
    changed = set((int(p), int(q)) for p, q in np.argwhere((k2 != kp).any(axis=(2, 3))))
    first = int(t.page_offsets[c])
    expect = set((int(t.page_ids[first + u // t.page_size]), u % t.page_size) for u in range(int(t.chunk_tokens[c])))
    assert changed == expect  # exactly the chunk's token slots


def test_p11_publishing_every_chunk_rebuilds_the_input_pool(oracle_lib):
    """The inputs module lays a case's draws into its pool independently; publishing each chunk's
    rows (read back by the dense gather) into an all-NaN pool rebuilds it exactly, padding too."""
    from oracle.dense import gather_keys
    c = make_case("wave_round", small=True)
    gk, owner = gather_keys(c.table, c.k_pool)
    gv, _ = gather_keys(c.table, c.v_pool)
    kp = np.full(c.k_pool.shape, np.nan)
    vp = np.full(c.v_pool.shape, np.nan)
    for b in range(c.table.num_chunks):
        kp, vp = oracle_lib.publish_kv(c.table, b, gk[owner == b], gv[owner == b], kp, vp)
    same = lambda a, b: ((a == b) | (np.isnan(a) & np.isnan(b))).all()
    assert same(kp, c.k_pool.double().numpy()) and same(vp, c.v_pool.double().numpy())


# ---------------------------------------------------------------- P12: rotary embedding
def _angles(rng, n, half):
    th = rng.uniform(-np.pi, np.pi, size=(n, half))
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32), th


def test_p12_rotation_special_angles(oracle_lib):
    rng = np.random.default_rng(71)
    x = rng.standard_normal((5, 3, 16)).astype(np.float32)
    one, zero = np.ones((5, 8), np.float32), np.zeros((5, 8), np.float32)
    assert np.array_equal(oracle_lib.rotate_pairs(x, one, zero), x)  # no rotation
    q = oracle_lib.rotate_pairs(x, zero, one)  # a quarter turn: (x0, x1) -> (-x1, x0)
    assert np.array_equal(q[..., 0::2], -x[..., 1::2]) and np.array_equal(q[..., 1::2], x[..., 0::2])


def test_p12_rotation_is_complex_multiplication(oracle_lib):
    """Against an independent statement: pair (x0, x1) as the complex number x0 + i x1, times
    exp(i theta), in complex128; the float32 formula stays within its rounding of it."""
    rng = np.random.default_rng(72)
    x = rng.standard_normal((40, 2, 32)).astype(np.float32)
    c, s_, th = _angles(rng, 40, 16)
    got = oracle_lib.rotate_pairs(x, c, s_).astype(np.float64)
    z = (x[..., 0::2].astype(np.float64) + 1j * x[..., 1::2]) * (c.astype(np.float64) + 1j * s_)[:, None, :]
    bound = 3 * 2.0 ** -24 * (np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])).astype(np.float64)
    assert (np.abs(got[..., 0::2] - z.real) <= bound).all() and (np.abs(got[..., 1::2] - z.imag) <= bound).all()
    # and by theta then -theta is the identity up to that rounding
    back = oracle_lib.rotate_pairs(oracle_lib.rotate_pairs(x, c, s_), c, -s_).astype(np.float64)
    assert np.abs(back - x).max() <= 1e-5 * np.abs(x).max()


# ---------------------------------------------------------------- P3: single chunk
def test_p3_single_chunk_is_full_attention(oracle_lib):
    rng = np.random.default_rng(3)
    H, d, T = 2, 64, 50
    c = _contiguous_case(rng, [T], [0], [0], H, d)
    o, _ = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
    q = c.q.double().transpose(0, 1)
    k = c.k_pool.double()[:, 0].transpose(0, 1)
    v = c.v_pool.double()[:, 0].transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)  # no mask
    assert np.abs(o - ref.transpose(0, 1).numpy()).max() <= 1e-12


# ---------------------------------------------------------------- P4: closed forms
def test_p4_constant_values_give_that_value(oracle_lib):
    c = make_case("wave_round", small=True)
    H, d = c.table.num_heads, c.table.head_dim
    vec = torch.randn(H, d, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    v = c.v_pool.clone()
    v[:] = vec  # every slot (padding too, which must never be read anyway)
    o, _ = oracle_lib.attn_rows(c.table, c.q, c.k_pool, v)
    assert np.abs(o - vec.double().numpy()[None]).max() <= 1e-13


@pytest.mark.parametrize("name", ["wave_round", "long_rollout", "tiny_fp32"])
def test_p4_zero_query_is_mean_of_visible_values(oracle_lib, name):
    c = make_case(name, small=True)
    t = c.table
    q = torch.zeros_like(c.q)
    o, l = oracle_lib.attn_rows(t, q, c.k_pool, c.v_pool)
    row = 0
    for a in t.query_chunks:
        vis = [b for b in range(t.num_chunks) if t.chunk_order[b] <= t.chunk_order[a]]
        vals, n = [], 0
        for b in vis:
            for u in range(int(t.chunk_tokens[b])):
                pg = int(t.page_ids[int(t.page_offsets[b]) + u // t.page_size])
                vals.append(c.v_pool[pg, u % t.page_size].double().numpy())
                n += 1
        mean = np.mean(vals, axis=0)
        rows = slice(row, row + int(t.chunk_tokens[a]))
        assert np.abs(o[rows] - mean[None]).max() <= 1e-13
        assert np.abs(l[rows] - math.log(n)).max() <= 1e-13  # all scores 0: lse = log(#visible)
        row += int(t.chunk_tokens[a])


def test_p4_rows_are_probability_vectors(oracle_lib):
    """V_j = e_j (one-hot): the output row is the softmax weight vector itself."""
    rng = np.random.default_rng(11)
    tokens, order, queries = [20, 16, 24], [1, 0, 2], [0, 1, 2]
    H, d = 1, 64
    c = _contiguous_case(rng, tokens, order, queries, H, d)
    lk = sum(tokens)
    v = torch.zeros_like(c.v_pool)
    for j in range(lk):
        v[j, 0, 0, j] = 1.0
    o, _ = oracle_lib.attn_rows(c.table, c.q, c.k_pool, v)
    w = o[:, 0, :lk]
    mask = _sdpa_mask(tokens, order, queries).numpy()
    assert np.abs(w.sum(axis=1) - 1).max() <= 1e-12
    assert (w[~mask] == 0).all() and (w[mask] > 0).all()
    assert np.abs(o[:, 0, lk:]).max() == 0


def test_p4_explicit_scale(oracle_lib):
    c = make_case("wan13b_task", small=True)
    t2 = c.table.copy()
    t2.softmax_scale = 0.25
    o1, _ = oracle_lib.attn_rows(c.table, c.q * 2, c.k_pool, c.v_pool)  # default 1/sqrt(128)
    q_scaled = c.q.double() * (0.25 * math.sqrt(128) * 2)
    t3 = c.table.copy()
    o2, _ = oracle_lib.attn_rows(t3, q_scaled, c.k_pool, c.v_pool)
    o3, _ = oracle_lib.attn_rows(t2, c.q.double() * 2, c.k_pool, c.v_pool)
    assert np.abs(o2 - o3).max() <= 1e-12
    assert np.abs(o1 - o3).max() > 1e-3


# ---------------------------------------------------------------- P5: permutations
def test_p5_page_shuffle_is_bitwise_invariant(oracle_lib):
    c = make_case("long_rollout", small=True)
    t = c.table
    rng = np.random.default_rng(99)
    newn = t.num_pages + 5
    perm = rng.permutation(newn).astype(np.int32)
    k2 = torch.full((newn,) + tuple(c.k_pool.shape[1:]), float("nan"), dtype=c.k_pool.dtype)
    v2 = k2.clone()
    t2 = t.copy()
    t2.num_pages = newn
    for lp in range(int(t.page_offsets[-1])):
        k2[perm[lp]] = c.k_pool[int(t.page_ids[lp])]
        v2[perm[lp]] = c.v_pool[int(t.page_ids[lp])]
        t2.page_ids[lp] = perm[lp]
    o1, l1 = oracle_lib.attn_rows(t, c.q, c.k_pool, c.v_pool)
    o2, l2 = oracle_lib.attn_rows(t2, c.q, k2, v2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_p5_chunk_relabel_is_invariant(oracle_lib):
    """Renumbering chunks (ids and their page runs) with the same orders permutes keys inside
    each visible set only."""
    c = make_case("wave_round", small=True)
    t = c.table
    n = t.num_chunks
    relabel = np.array([3, 6, 0, 5, 1, 4, 2])  # old id -> new id
    inv = np.argsort(relabel)
    tok = t.chunk_tokens[inv]
    order = t.chunk_order[inv]
    offs = np.zeros(n + 1, np.int32)
    ids = []
    for new in range(n):
        old = inv[new]
        pages = t.page_ids[t.page_offsets[old]: t.page_offsets[old + 1]]
        ids.extend(pages)
        offs[new + 1] = offs[new] + len(pages)
    t2 = ChunkTable(tok.astype(np.int32), order.astype(np.int32), offs, np.array(ids, np.int32),
                    t.num_pages, t.page_size, relabel[t.query_chunks].astype(np.int32),
                    t.num_heads, t.head_dim)
    o1, _ = oracle_lib.attn_rows(t, c.q, c.k_pool, c.v_pool)
    o2, _ = oracle_lib.attn_rows(t2, c.q, c.k_pool, c.v_pool)
    assert np.abs(o1 - o2).max() <= 1e-13


# ---------------------------------------------------------------- P6: no reverse edge
def test_p6_appending_later_chunks_changes_nothing(oracle_lib):
    rng = np.random.default_rng(21)
    base = make_table([40, 33, 50], [0, 1, 2], [1, 2], 16, 2, 32, shuffle_rng=rng, spare=2)
    c = fill_case("base", base, rng, torch.float32)
    # two later, noisier chunks appended; their K/V are huge so any leak would show
    t2 = make_table([40, 33, 50, 30, 20], [0, 1, 2, 3, 4], [1, 2], 16, 2, 32, shuffle_rng=None,
                    spare=0)
    extra_pages = int(t2.page_offsets[-1]) - int(base.page_offsets[-1])
    t2.num_pages = base.num_pages + extra_pages
    t2.page_ids = np.concatenate([base.page_ids, base.num_pages + np.arange(extra_pages)]).astype(np.int32)
    shape = (t2.num_pages,) + tuple(c.k_pool.shape[1:])
    k2 = torch.full(shape, 1e3)
    v2 = torch.full(shape, -1e3)
    k2[: base.num_pages] = c.k_pool
    v2[: base.num_pages] = c.v_pool
    o1, l1 = oracle_lib.attn_rows(base, c.q, c.k_pool, c.v_pool)
    o2, l2 = oracle_lib.attn_rows(t2, c.q, k2, v2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- P7: decomposition
def test_p7_multi_chunk_call_equals_single_chunk_calls(oracle_lib):
    c = make_case("wave_round", small=True)
    t = c.table
    o, l = oracle_lib.attn_rows(t, c.q, c.k_pool, c.v_pool)
    row = 0
    for a in t.query_chunks:
        n = int(t.chunk_tokens[a])
        t1 = t.copy()
        t1.query_chunks = np.array([a], np.int32)
        oa, la = oracle_lib.attn_rows(t1, c.q[row:row + n], c.k_pool, c.v_pool)
        assert np.array_equal(oa, o[row:row + n]) and np.array_equal(la, l[row:row + n])
        row += n


def test_rows_subset_matches_full(oracle_lib):
    c = make_case("wave_round", small=True)
    o, l = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool)
    rows = np.array([0, 5, 95, 96, 200, 479])
    os_, ls_ = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls_, l[rows])


# ---------------------------------------------------------------- P8: e4m3 codec
def test_p8_decode_all_codes_against_torch_and_spec(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle_lib.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(dec), nan) and np.array_equal(dec[~nan], ref[~nan])
    # points fixed by the format definition
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    assert dec[0x38] == 1.0 and dec[0xB8] == -1.0 and dec[0x07] == 7 * 2.0 ** -9
    assert np.all(np.diff(dec[:0x7F]) > 0)


def test_p8_encode_against_torch(oracle_lib):
    rng = np.random.default_rng(8)
    mags = oracle_lib.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2  # exact ties: must round to the even code
    x = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 4,
        rng.standard_normal(5000) * 1e-3, mids, -mids, mags, -mags]).astype(np.float32)
    enc = oracle_lib.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, ref)
    tie = oracle_lib.e4m3_encode(mids.astype(np.float32))
    assert np.all(tie % 2 == 0)
    # saturation (the reading: clamp to the largest finite magnitude)
    assert list(oracle_lib.e4m3_encode(np.array([449, 500, 1e30, -1e9], np.float32))) == [0x7E, 0x7E, 0x7E, 0xFE]


def test_p8_quantizer_properties(oracle_lib):
    rng = np.random.default_rng(12)
    rows, H, d = 150, 3, 128
    x = torch.from_numpy(rng.standard_normal((rows, H, d)).astype(np.float32)).to(torch.bfloat16)
    x[70:75, 1] *= 30  # a hot block
    x[128:, 2] = 0  # an all-zero block (rows 128..149 of head 2)
    x8, sc = oracle_lib.quantize_e4m3(x)
    assert sc.shape == (3, H)
    xf = x.float().numpy()
    for b in range(3):
        for h in range(H):
            blk = xf[64 * b: 64 * b + 64, h]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                assert sc[b, h] == 1.0 and (x8[64 * b: 64 * b + 64, h] == 0).all()
                continue
            assert sc[b, h] == np.float32(amax / np.float32(448))
            mult = np.float32(np.float32(448) / amax)
            # library routine for the rounding step: torch's float8_e4m3fn cast of the clamped product
            y = np.clip(blk * mult, -448, 448).astype(np.float32)
            ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(x8[64 * b: 64 * b + 64, h], ref)
            assert np.abs(oracle_lib.e4m3_decode(x8[64 * b: 64 * b + 64, h])).max() == 448.0
    deq = oracle_lib.dequantize_e4m3(x8, sc)
    # e4m3 relative spacing is 2^-3, so RNE error <= 2^-4 relative (normals) or half a subnormal step
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, np.repeat(sc, 64, axis=0)[:rows][:, :, None] * 2.0 ** -10)
    assert (err <= bound * (1 + 1e-6)).all()


# ---------------------------------------------------------------- P9: LSE combine
def test_p9_merging_key_partitions(oracle_lib):
    rng = np.random.default_rng(9)
    nq, nk, d = 17, 90, 64
    q, k, v = (rng.standard_normal(s) for s in [(nq, d), (nk, d), (nk, d)])
    allowed = rng.random((nq, nk)) < 0.7
    allowed[:, 0] = True
    full_o, full_l = oracle_lib.attn_masked(q, k, v, allowed, 0.125)
    cut = [0, 23, 60, nk]
    parts_o, parts_l = [], []
    for a, b in zip(cut[:-1], cut[1:]):
        m = np.zeros_like(allowed)
        m[:, a:b] = allowed[:, a:b]
        po, pl = oracle_lib.attn_masked(q, k, v, m, 0.125)
        po = np.nan_to_num(po)  # rows with no key in this part: weight exp(-inf) = 0
        parts_o.append(po)
        parts_l.append(pl)
    mo, ml = oracle_lib.merge_lse(np.stack(parts_o), np.stack(parts_l))
    assert np.abs(mo - full_o).max() <= 1e-13 and np.abs(ml - full_l).max() <= 1e-13


def test_p9_masked_form_against_sdpa_float64(oracle_lib):
    """The explicit-mask form the merge pin leans on, against torch's float64 SDPA and logsumexp
    with arbitrary boolean masks (not block-shaped), an explicit scale and the default 1/sqrt(d);
    a row with no visible key is NaN with lse -inf."""
    rng = np.random.default_rng(19)
    for nq, nk, d, scale in [(23, 61, 32, 0.2), (40, 17, 64, 1 / 8), (9, 130, 16, 0.25)]:
        q, k, v = (rng.standard_normal(s) for s in [(nq, d), (nk, d), (nk, d)])
        allowed = rng.random((nq, nk)) < 0.4
        allowed[np.arange(nq), rng.integers(0, nk, size=nq)] = True
        o, l = oracle_lib.attn_masked(q, k, v, allowed, scale)
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        m = torch.from_numpy(allowed)
        ref = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=m[None],
                                                               scale=scale)[0]
        assert np.abs(o - ref.numpy()).max() <= 1e-12
        sc = (qt @ kt.T * scale).masked_fill(~m, float("-inf"))
        assert np.abs(l - torch.logsumexp(sc, dim=-1).numpy()).max() <= 1e-12
    allowed = np.ones((3, 5), bool)
    allowed[1] = False
    q, k, v = (rng.standard_normal(s) for s in [(3, 8), (5, 8), (5, 8)])
    o, l = oracle_lib.attn_masked(q, k, v, allowed, 0.5)
    assert np.isnan(o[1]).all() and l[1] == -np.inf and np.isfinite(o[[0, 2]]).all()


def test_sum_of_squared_weights(oracle_lib):
    """The oracle's sum_j w_j^2 (used to size the LSE rounding gate): against torch's float64
    softmax of the masked scores; 1/N for a zero query (equal weights over N visible keys); 1 for
    a single visible key."""
    rng = np.random.default_rng(23)
    tokens, order, queries, H, d = [11, 7, 19], [1, 0, 2], [0, 2, 1], 2, 16
    c = _contiguous_case(rng, tokens, order, queries, H, d)
    _, _, w2 = oracle_lib.attn_rows(c.table, c.q, c.k_pool, c.v_pool, want_sumw2=True)
    keys = c.k_pool.double()[:, 0]
    mask = _sdpa_mask(tokens, order, queries)
    q = c.q.double().transpose(0, 1)
    s = (q @ keys.permute(1, 2, 0)) / math.sqrt(d)
    w = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
    assert np.abs(w2 - (w * w).sum(-1).T.numpy()).max() <= 1e-14
    q0 = torch.zeros_like(c.q)
    _, _, w2z = oracle_lib.attn_rows(c.table, q0, c.k_pool, c.v_pool, want_sumw2=True)
    nvis = mask.sum(-1).numpy().astype(np.float64)
    assert np.abs(w2z - (1.0 / nvis)[:, None]).max() <= 1e-15
    t1 = make_table([1], [0], [0], 64, 1, 16, shuffle_rng=None, spare=0)
    c1 = fill_case("one", t1, rng, torch.float32)
    _, _, w21 = oracle_lib.attn_rows(t1, c1.q, c1.k_pool, c1.v_pool, want_sumw2=True)
    assert w21[0, 0] == 1.0


# ---------------------------------------------------------------- brute force and golden
def test_brute_force_python_loops(oracle_lib):
    rng = np.random.default_rng(13)
    t = make_table([5, 7, 4], [2, 0, 1], [0, 2], 4, 2, 8, shuffle_rng=rng, spare=1)
    c = fill_case("bf", t, rng, torch.float32)
    o, l = oracle_lib.attn_rows(t, c.q, c.k_pool, c.v_pool)
    qs, kp, vp = c.q.double().tolist(), c.k_pool.double().tolist(), c.v_pool.double().tolist()
    row = 0
    for a in t.query_chunks:
        for _ in range(int(t.chunk_tokens[a])):
            for h in range(2):
                ss, vv = [], []
                for b in range(3):
                    if t.chunk_order[b] > t.chunk_order[a]:
                        continue
                    for u in range(int(t.chunk_tokens[b])):
                        pg = int(t.page_ids[int(t.page_offsets[b]) + u // 4])
                        kk = kp[pg][u % 4][h]
                        ss.append(sum(x * y for x, y in zip(qs[row][h], kk)) / math.sqrt(8))
                        vv.append(vp[pg][u % 4][h])
                m = max(ss)
                z = sum(math.exp(s - m) for s in ss)
                for ch in range(8):
                    ref = sum(math.exp(s - m) / z * v[ch] for s, v in zip(ss, vv))
                    assert abs(o[row, h, ch] - ref) <= 1e-12
                assert abs(l[row, h] - (m + math.log(z))) <= 1e-12
            row += 1


def _golden_value(x):
    if isinstance(x, (int, float)):
        return float(x)
    if x.startswith("ln"):
        return math.log(int(x[2:]))
    return float(Fraction(x))


def test_golden_two_chunk_closed_form(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "two_chunk_closed_form.json")))
    tb = g["table"]
    t = ChunkTable(*(np.array(tb[k], np.int32) for k in ["chunk_tokens", "chunk_order",
                                                          "page_offsets", "page_ids"]),
                   tb["num_pages"], tb["page_size"], np.array(tb["query_chunks"], np.int32),
                   tb["num_heads"], tb["head_dim"], tb["softmax_scale"])
    kp = np.full((2, 2, 1, 2), np.nan)
    vp = np.full((2, 2, 1, 2), np.nan)
    for b in range(2):
        pg = tb["page_ids"][tb["page_offsets"][b]]
        for u in range(2):
            kp[pg, u, 0] = [_golden_value(x) for x in g["keys_by_chunk"][b][u]]
            vp[pg, u, 0] = [_golden_value(x) for x in g["values_by_chunk"][b][u]]
    q = np.array(g["q"], np.float64)[:, None, :]
    o, l = oracle_lib.attn_rows(t, q, kp, vp)
    exp_o = np.array([[_golden_value(x) for x in r] for r in g["expected_out"]])
    exp_l = np.array([_golden_value(x) for x in g["expected_lse"]])
    assert np.abs(o[:, 0] - exp_o).max() <= 1e-15 * 8
    assert np.abs(l[:, 0] - exp_l).max() <= 1e-15 * 8


# ---------------------------------------------------------------- the pins catch mistakes
def test_pins_detect_plausible_mistakes(oracle_lib):
    """Feed the oracle a mistaken table (the kind of slip a kernel or planner could make) and
    check the dense pin sees the difference: reversed visibility, the physical page placement
    ignored, and a 1/d softmax scale instead of 1/sqrt(d)."""
    from oracle.dense import attn_dense
    c = make_case("wave_round", small=True)
    ref, _ = attn_dense(c.table, c.q, c.k_pool, c.v_pool)
    bad = c.table.copy()
    bad.chunk_order = (bad.num_chunks - 1 - bad.chunk_order).astype(np.int32)  # reversed edges
    o, _ = oracle_lib.attn_rows(bad, c.q, c.k_pool, c.v_pool)
    assert np.abs(o - ref).max() > 1e-2
    bad = c.table.copy()
    bad.page_ids = np.sort(bad.page_ids).astype(np.int32)  # physical placement ignored
    o = oracle_lib.attn_rows(bad, c.q, c.k_pool, c.v_pool)[0]
    assert not np.isfinite(o).all() or np.abs(o - ref).max() > 1e-2
    bad = c.table.copy()
    bad.softmax_scale = 1.0 / 128  # 1/d instead of 1/sqrt(d)
    o = oracle_lib.attn_rows(bad, c.q, c.k_pool, c.v_pool)[0]
    assert np.abs(o - ref).max() > 1e-3


# ---------------------------------------------------------------- e4m3 V pool (e4m3 K/V storage)
def test_v8_slot_order_is_the_stated_permutation(oracle_lib):
    """Keys 0-7 -> slots 0-7, 8-15 -> 16-23, 16-23 -> 8-15, 24-31 -> 24-31, the same in the upper
    half; a bijection on 0..63."""
    slots = [oracle_lib.v8_slot(k) for k in range(64)]
    assert slots[:8] == list(range(8)) and slots[8:16] == list(range(16, 24))
    assert slots[16:24] == list(range(8, 16)) and slots[24:32] == list(range(24, 32))
    assert slots[32:] == [32 + s for s in slots[:32]]
    assert sorted(slots) == list(range(64))


def test_v8_quantizer_against_the_row_quantizer(oracle_lib):
    """Every finite value's code and scale are those of the row-layout block quantizer (P8), placed
    at [block, head, channel, slot(key)]; NaN padding gets code 0; dequantizing gives back
    decode * scale in row order (0 at padding)."""
    rng = np.random.default_rng(29)
    rows, H, d = 192, 3, 16
    x = (rng.standard_normal((rows, H, d)) * rng.choice([0.1, 1.0, 30.0], size=(rows, 1, 1))).astype(np.float32)
    x[150:] = np.nan  # a chunk's last block, partly padding
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    v8, sc = oracle_lib.quantize_v8(x)
    x8, sc_rows = oracle_lib.quantize_e4m3(x)
    assert np.array_equal(sc, sc_rows)
    for r in range(rows):
        b, key = divmod(r, 64)
        for h in range(H):
            for c in range(d):
                want = 0 if np.isnan(x[r, h, c]) else x8[r, h, c]
                assert v8[b, h, c, oracle_lib.v8_slot(key)] == want
    y = oracle_lib.dequantize_v8(v8, sc)
    ref = np.nan_to_num(oracle_lib.dequantize_e4m3(x8, sc_rows), nan=0.0)
    assert np.array_equal(y, ref)


# ---------------------------------------------------------------- QKV projection
def test_qkv_projection_brute_force(oracle_lib):
    """qkv_project against the sum written out with Python loops, and its (role, head, channel)
    column order."""
    rng = np.random.default_rng(31)
    n, hid, H, d = 3, 5, 2, 4
    x = rng.standard_normal((n, hid))
    w = rng.standard_normal((hid, 3 * H * d))
    y = oracle_lib.qkv_project(x, w, H, d)
    for i in range(n):
        for r in range(3):
            for h in range(H):
                for c in range(d):
                    col = (r * H + h) * d + c
                    assert abs(y[i, r, h, c] - sum(x[i, k] * w[k, col] for k in range(hid))) <= 1e-12
