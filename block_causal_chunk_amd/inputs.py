"""Seeded synthetic inputs for block-causal chunk attention.

This module only draws random numbers and lays them out; it contains none of the attention
arithmetic.  Both the GPU library's tests/benchmark and the CPU oracle consume what it builds,
so it is the one piece of code the two sides share.

Workload shapes (the pages give no activation statistics, so values are i.i.d. N(0, 1)):
  * a chunk is 3 latent frames (the GitHub README's quick start requires the latent frame count
    to be a multiple of three); at 832x480 one chunk is 3 x 30 x 52 = 4680 tokens;
  * the K/V of every chunk a query may read sit in a pool of fixed-size pages, one run of pages
    per producer chunk, read in place (project page, section 03, "Layout" panel);
  * chunk order 0 is the cleanest/oldest (anchor / sink), larger is later and noisier.

Recipe: numpy PCG64 ``default_rng(1000 + k)`` for workload k; per chunk in clean -> noisy order
draw Q (query chunks only), then K, then V as float32 ``[tokens, H, d]``; then (wave round only)
the outlier channels; then ``rng.permutation(num_pages)`` for the physical page ids.  Values are
rounded to bf16 with round-to-nearest-even (torch ``.to(bfloat16)``); unused slots of a chunk's
last page and the spare pages hold NaN so that any read of them shows in the output.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["ChunkTable", "Case", "WORKLOADS", "make_table", "make_case", "fill_case"]


@dataclass
class ChunkTable:
    """Host description of one call: chunks, their order, the page table and the query set."""

    chunk_tokens: np.ndarray  # int32 [n]
    chunk_order: np.ndarray  # int32 [n], a permutation of 0..n-1, 0 = cleanest
    page_offsets: np.ndarray  # int32 [n+1], CSR into page_ids
    page_ids: np.ndarray  # int32 [page_offsets[-1]], physical page of each logical page
    num_pages: int
    page_size: int
    query_chunks: np.ndarray  # int32, distinct chunk ids; Q rows are their tokens concatenated
    num_heads: int
    head_dim: int
    softmax_scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)

    @property
    def num_chunks(self) -> int:
        return int(self.chunk_tokens.shape[0])

    @property
    def lq(self) -> int:
        return int(sum(int(self.chunk_tokens[c]) for c in self.query_chunks))

    def copy(self) -> "ChunkTable":
        return ChunkTable(
            self.chunk_tokens.copy(), self.chunk_order.copy(), self.page_offsets.copy(),
            self.page_ids.copy(), self.num_pages, self.page_size, self.query_chunks.copy(),
            self.num_heads, self.head_dim, self.softmax_scale)


@dataclass
class Case:
    name: str
    table: ChunkTable
    io_dtype: torch.dtype  # torch.bfloat16 or torch.float32
    q: torch.Tensor  # [Lq, H, d] on the CPU
    k_pool: torch.Tensor  # [num_pages, page_size, H, d]
    v_pool: torch.Tensor
    meta: dict = field(default_factory=dict)


# Workloads: name -> parameters.  chunks are listed by chunk id; chunk id == order here.
WORKLOADS = {
    # 4 chunks x 48 tokens (3 frames x 16 tokens), every token a query, fp32 I/O
    "tiny_fp32": dict(k=1, H=2, d=64, tokens=[48] * 4, queries=[0, 1, 2, 3], page=64,
                      shuffle=False, spare=0, dtype="fp32"),
    # one Wan-1.3B chunk-stage task: own chunk + 3 earlier chunks
    "wan13b_task": dict(k=2, H=12, d=128, tokens=[4680] * 4, queries=[3], page=256,
                        shuffle=True, spare=8, dtype="bf16"),
    # a mixed-noise wave round: 2 clean prefix chunks + 5 active chunks, all 5 active are queries
    "wave_round": dict(k=3, H=12, d=128, tokens=[4680] * 7, queries=[2, 3, 4, 5, 6], page=256,
                       shuffle=True, spare=8, dtype="bf16", outlier_frac=0.05, outlier_mult=8.0),
    # long rollout: sink chunk + 8 rolling-window chunks + own chunk
    "long_rollout": dict(k=4, H=12, d=128, tokens=[4680] * 10, queries=[9], page=256,
                         shuffle=True, spare=8, dtype="bf16"),
    # 14B-shaped chunk task for the fp8 Q.K^T path
    "wan14b_fp8": dict(k=5, H=40, d=128, tokens=[4680] * 4, queries=[3], page=256,
                       shuffle=True, spare=8, dtype="bf16"),
    # the same task with K and V both stored as e4m3 (same seed, so the same values)
    "wan14b_fp8kv": dict(k=5, H=40, d=128, tokens=[4680] * 4, queries=[3], page=256,
                         shuffle=True, spare=8, dtype="bf16"),
}

# Scaled-down variants that the CPU oracle finishes in well under a second.
SMALL = dict(H=2, chunk_tokens=96, page=64)


def make_table(tokens, order, queries, page_size, H, d, *, shuffle_rng=None, spare=0,
               softmax_scale=0.0) -> ChunkTable:
    """Per-chunk pages (each chunk starts on a fresh page); physical ids are a permutation drawn
    from ``shuffle_rng`` (identity when None) over ``logical + spare`` pages."""
    tokens = np.asarray(tokens, dtype=np.int32)
    order = np.asarray(order, dtype=np.int32)
    npages = (tokens + page_size - 1) // page_size
    offs = np.zeros(len(tokens) + 1, dtype=np.int32)
    offs[1:] = np.cumsum(npages)
    n_logical = int(offs[-1])
    num_pages = n_logical + int(spare)
    if shuffle_rng is None:
        perm = np.arange(num_pages, dtype=np.int32)
    else:
        perm = shuffle_rng.permutation(num_pages).astype(np.int32)
    return ChunkTable(tokens, order, offs, perm[:n_logical].copy(), num_pages, int(page_size),
                      np.asarray(queries, dtype=np.int32), int(H), int(d), float(softmax_scale))


def _draw(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def fill_case(name, table: ChunkTable, rng, io_dtype=torch.bfloat16, outlier_frac=0.0,
              outlier_mult=1.0, meta=None) -> Case:
    """Draw Q/K/V for ``table`` with ``rng`` and lay them into a NaN-padded paged pool."""
    H, d, P = table.num_heads, table.head_dim, table.page_size
    n = table.num_chunks
    qset = set(int(c) for c in table.query_chunks)
    qs, ks, vs = {}, {}, {}
    for c in sorted(range(n), key=lambda c: int(table.chunk_order[c])):
        t = int(table.chunk_tokens[c])
        if c in qset:
            qs[c] = _draw(rng, (t, H, d))
        ks[c] = _draw(rng, (t, H, d))
        vs[c] = _draw(rng, (t, H, d))
    outliers = None
    if outlier_frac > 0:
        n_out = int(round(outlier_frac * d))
        outliers = np.stack([rng.choice(d, size=n_out, replace=False) for _ in range(H)])
        for c in range(n):
            for h in range(H):
                ks[c][:, h, outliers[h]] *= np.float32(outlier_mult)
    k_pool = np.full((table.num_pages, P, H, d), np.nan, dtype=np.float32)
    v_pool = np.full((table.num_pages, P, H, d), np.nan, dtype=np.float32)
    for c in range(n):
        t = int(table.chunk_tokens[c])
        for lp in range(int(table.page_offsets[c]), int(table.page_offsets[c + 1])):
            u0 = (lp - int(table.page_offsets[c])) * P
            u1 = min(u0 + P, t)
            pid = int(table.page_ids[lp])
            k_pool[pid, : u1 - u0] = ks[c][u0:u1]
            v_pool[pid, : u1 - u0] = vs[c][u0:u1]
    q = np.concatenate([qs[int(c)] for c in table.query_chunks], axis=0)
    m = dict(meta or {})
    if outliers is not None:
        m["outlier_channels"] = outliers
    return Case(name, table, io_dtype, torch.from_numpy(q).to(io_dtype),
                torch.from_numpy(k_pool).to(io_dtype), torch.from_numpy(v_pool).to(io_dtype), m)


def make_case(name: str, small: bool = False, seed: int | None = None) -> Case:
    """Build workload ``name`` (see WORKLOADS); ``small`` scales C2-C5 down to 2 heads,
    96-token chunks and 64-token pages (same chunk structure, same draw order)."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(1000 + w["k"] if seed is None else seed)
    H, d, page, tokens = w["H"], w["d"], w["page"], list(w["tokens"])
    if small and name != "tiny_fp32":
        H, page = SMALL["H"], SMALL["page"]
        tokens = [SMALL["chunk_tokens"]] * len(tokens)
    order = list(range(len(tokens)))
    io = torch.float32 if w["dtype"] == "fp32" else torch.bfloat16
    # Q/K/V are drawn first, the page permutation last (see the module docstring); the table is
    # built with an identity permutation and re-labelled after the draws.
    table = make_table(tokens, order, w["queries"], page, H, d, shuffle_rng=None,
                       spare=w["spare"])
    # draw values with the identity layout, then shuffle pages with the same rng
    case = fill_case(name + ("_small" if small else ""), table, rng, io,
                     w.get("outlier_frac", 0.0), w.get("outlier_mult", 1.0))
    if w["shuffle"]:
        perm = rng.permutation(table.num_pages).astype(np.int32)
        # logical page p moves from physical page table.page_ids[p] (== p) to perm[p]
        new_k = torch.full_like(case.k_pool, float("nan"))
        new_v = torch.full_like(case.v_pool, float("nan"))
        idx = torch.from_numpy(perm.astype(np.int64))
        new_k[idx] = case.k_pool
        new_v[idx] = case.v_pool
        case.k_pool, case.v_pool = new_k, new_v
        table.page_ids = perm[: int(table.page_offsets[-1])].copy()
    return case
