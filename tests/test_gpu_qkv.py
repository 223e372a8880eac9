"""GPU parity of the fused QKV projection + pre-attention epilogue (wfattn_qkv_rope_publish)
against the oracle: an fp64 matrix product (oracle.qkv_project), the rotation of channel pairs
(oracle.rotate_pairs), bf16 rounding, the block quantizer (oracle.quantize_e4m3) and the page
placement (oracle.publish_kv).

The kernel accumulates the product in fp32 on the matrix cores, in its own order, so its bf16
outputs are compared with the fp64 definition within bf16 rounding (2^-8 relative) plus the fp32
accumulation error of a hidden-size dot product (a small absolute floor), and with the oracle's
fp32 rotation of the fp32-rounded product mostly bit for bit.  The e4m3 outputs are then compared
bit for bit with the oracle's quantizer applied to the kernel's own bf16 values (the fused
epilogue quantizes exactly those), and every pool slot outside the chunk's pages is untouched.
"""
import numpy as np
import pytest
import torch

from block_causal_chunk_amd.inputs import make_table

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


def _setup(seed, tokens, chunk, H, d, hidden, page):
    rng = np.random.default_rng(seed)
    t = make_table(tokens, list(range(len(tokens))), [len(tokens) - 1], page, H, d, shuffle_rng=rng, spare=2)
    n = int(t.chunk_tokens[chunk])
    x = torch.from_numpy(rng.standard_normal((n, hidden), dtype=np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((hidden, 3 * H * d), dtype=np.float32) / np.sqrt(hidden)).to(torch.bfloat16)
    th = rng.random((n, d // 2)) * 2 * np.pi
    cos_t = torch.from_numpy(np.cos(th).astype(np.float32))
    sin_t = torch.from_numpy(np.sin(th).astype(np.float32))
    return t, n, x, w, cos_t, sin_t


def _reference(O, t, x, w, cos_t, sin_t):
    """(q, k, v) as float64 [n, H, d]: the exact product, its exact rotation; and the oracle's fp32
    rotation of the fp32-rounded product, rounded to bf16 (what an fp32 computation gives)."""
    H, d = t.num_heads, t.head_dim
    qkv = O.qkv_project(x, w, H, d)
    c, s = cos_t.double().numpy()[:, None, :], sin_t.double().numpy()[:, None, :]

    def exact_rot(a):
        out = np.empty_like(a)
        out[..., 0::2] = a[..., 0::2] * c - a[..., 1::2] * s
        out[..., 1::2] = a[..., 0::2] * s + a[..., 1::2] * c
        return out

    exact = [exact_rot(qkv[:, 0]), exact_rot(qkv[:, 1]), qkv[:, 2]]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    f32 = [bf(O.rotate_pairs(qkv[:, r].astype(np.float32), cos_t, sin_t)) for r in (0, 1)] + [bf(qkv[:, 2])]
    return exact, f32


def _close(got_bf16, exact, f32_bf16, what):
    g = got_bf16.double().numpy()
    err = np.abs(g - exact)
    bound = 1.01 * 2.0 ** -8 * np.abs(exact) + 5e-5
    assert (err <= bound).all(), (what, float((err / bound).max()))
    diff = (got_bf16.view(torch.int16) != f32_bf16.view(torch.int16)).float().mean().item()
    assert diff <= 0.01, (what, "share of elements differing from the fp32 computation", diff)


def _chunk_rows(t, chunk, pool):
    """The chunk's rows of a pool [pages, page, H, ...] in token order."""
    n = int(t.chunk_tokens[chunk])
    P = t.page_size
    rows = [pool[int(t.page_ids[int(t.page_offsets[chunk]) + u // P]), u % P] for u in range(n)]
    return torch.stack(rows)


def _run(B, t, chunk, x, w, cos_t, sin_t, e4m3):
    H, d = t.num_heads, t.head_dim
    n = int(t.chunk_tokens[chunk])
    att = B.Attention(t, mode=B.WFATTN_WS_FP8)
    shape = (t.num_pages, t.page_size, H, d)
    dev = "cuda"
    vp = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    flags = torch.zeros(t.num_chunks, dtype=torch.int32, device=dev)
    out = dict(v=vp, flags=flags)
    if e4m3:
        out["q8"] = torch.zeros((n, H, d), dtype=torch.uint8, device=dev)
        out["qs"] = torch.zeros(((n + 63) // 64, H), dtype=torch.float32, device=dev)
        out["k8"] = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
        out["ks"] = torch.full((t.num_pages * t.page_size // 64, H), -1.0, dtype=torch.float32, device=dev)
        out["q"] = torch.zeros((n, H, d), dtype=torch.bfloat16, device=dev)
        B.wfattn_qkv_rope_publish(att.plan, chunk, x.cuda(), w.cuda(), cos_t.cuda(), sin_t.cuda(), out["q"],
                                  out["q8"], out["qs"], None, out["k8"], out["ks"], vp, flags, 5, att.ws)
    else:
        out["q"] = torch.zeros((n, H, d), dtype=torch.bfloat16, device=dev)
        out["k"] = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
        B.wfattn_qkv_rope_publish(att.plan, chunk, x.cuda(), w.cuda(), cos_t.cuda(), sin_t.cuda(), out["q"], None,
                                  None, out["k"], None, None, vp, flags, 5, att.ws)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def _check_all(B, O, t, chunk, x, w, cos_t, sin_t):
    exact, f32 = _reference(O, t, x, w, cos_t, sin_t)
    H, d = t.num_heads, t.head_dim
    r = _run(B, t, chunk, x, w, cos_t, sin_t, e4m3=False)
    _close(r["q"], exact[0], f32[0], "q")
    k_rows = _chunk_rows(t, chunk, r["k"])
    _close(k_rows, exact[1], f32[1], "k")
    _close(_chunk_rows(t, chunk, r["v"]), exact[2], f32[2], "v")
    # every slot outside the chunk's pages, and the tail of its last page, untouched
    mark = torch.zeros(t.num_pages, t.page_size, dtype=torch.bool)
    for u in range(int(t.chunk_tokens[chunk])):
        mark[int(t.page_ids[int(t.page_offsets[chunk]) + u // t.page_size]), u % t.page_size] = True
    assert torch.isnan(r["k"][~mark]).all() and torch.isnan(r["v"][~mark]).all()
    assert [int(f) for f in r["flags"]] == [5 if b == chunk else 0 for b in range(t.num_chunks)]
    # e4m3: q8/q_scale from the kernel's own bf16 Q, the e4m3 K pool from its own bf16 K
    r8 = _run(B, t, chunk, x, w, cos_t, sin_t, e4m3=True)
    assert torch.equal(r8["q"].view(torch.int16), r["q"].view(torch.int16))  # the same bf16 Q both times
    q8_ref, qs_ref = O.quantize_e4m3(r["q"])
    assert np.array_equal(r8["q8"].numpy(), q8_ref) and np.array_equal(r8["qs"].numpy(), qs_ref)
    k8_ref, ks_ref = O.quantize_e4m3(k_rows)
    assert np.array_equal(_chunk_rows(t, chunk, r8["k8"]).numpy(), k8_ref)
    first = int(t.page_offsets[chunk])
    for blk in range(ks_ref.shape[0]):
        u = 64 * blk
        pr = int(t.page_ids[first + u // t.page_size]) * t.page_size + u % t.page_size
        assert np.array_equal(r8["ks"][pr // 64].numpy(), ks_ref[blk])
    assert (r8["k8"][~mark] == 0x7F).all()
    assert torch.equal(r8["v"].view(torch.int16)[mark], r["v"].view(torch.int16)[mark])


@pytest.mark.parametrize("d,hidden", [(128, 256), (64, 192)])
def test_qkv_rope_publish_small(B, O, d, hidden):
    """A 300-token chunk (two 256-row workgroups, the last 64-token tile ragged) on shuffled
    256-token pages, 2 heads."""
    t, n, x, w, c, s = _setup(71, [150, 300], 1, 2, d, hidden, 256)
    print(f"[case] fused qkv projection small d={d} hidden={hidden}", flush=True)
    _check_all(B, O, t, 1, x, w, c, s)


def test_qkv_rope_publish_wan13b_chunk(B, O):
    """One full Wan-1.3B chunk: 4,680 tokens, hidden 1536 = 12 heads x 128, 256-token pages."""
    t, n, x, w, c, s = _setup(73, [4680, 4680], 1, 12, 128, 1536, 256)
    print("[case] fused qkv projection, Wan-1.3B chunk", flush=True)
    _check_all(B, O, t, 1, x, w, c, s)
