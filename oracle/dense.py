"""Dense-mask form of block-causal chunk attention (numpy fp64) -- TEST INFRASTRUCTURE.

A second, independent statement of the definition for small inputs: gather every key of every
chunk out of the paged pool into one contiguous array, build the explicit [Lq, Lk] visibility
matrix from chunk membership, and run an ordinary masked softmax over all keys (-inf where a key
is not visible).  Visibility (Wave Forcing project page, "01 - The design gap", the directed
frontier and its "Key observation"; KipQuest page, "The deep dive"): a query of chunk a sees
every token of chunk b iff b is not later/noisier than a, i.e. order[b] <= order[a]; this
includes b == a, where attention is full.
"""
from __future__ import annotations

import numpy as np

from . import _f64, resolve_scale


def gather_keys(table, pool):
    """All tokens of all chunks, chunk by chunk (by chunk id), token by token.
    Returns (keys [Lk, H, d] fp64, key_chunk [Lk] int)."""
    pool = _f64(pool)
    rows, owner = [], []
    for b in range(int(table.num_chunks)):
        first = int(table.page_offsets[b])
        for u in range(int(table.chunk_tokens[b])):
            page = int(table.page_ids[first + u // int(table.page_size)])
            rows.append(pool[page, u % int(table.page_size)])
            owner.append(b)
    return np.stack(rows), np.asarray(owner)


def query_chunk_of_rows(table):
    return np.concatenate([np.full(int(table.chunk_tokens[a]), int(a)) for a in table.query_chunks])


def visibility(table):
    """Explicit [Lq, Lk] boolean mask: block lower-triangular in clean -> noisy order."""
    _, owner = gather_keys_owner_only(table)
    qc = query_chunk_of_rows(table)
    order = np.asarray(table.chunk_order)
    return order[owner][None, :] <= order[qc][:, None]


def gather_keys_owner_only(table):
    owner = np.concatenate([np.full(int(table.chunk_tokens[b]), b) for b in range(int(table.num_chunks))])
    return None, owner


def attn_dense(table, q, k_pool, v_pool):
    """Returns (out [Lq, H, d], lse [Lq, H]) in fp64."""
    qd = _f64(q)
    K, owner = gather_keys(table, k_pool)
    V, _ = gather_keys(table, v_pool)
    mask = visibility(table)
    scale = resolve_scale(table)
    H = int(table.num_heads)
    out = np.empty_like(qd)
    lse = np.empty(qd.shape[:2])
    for h in range(H):
        s = scale * (qd[:, h, :] @ K[:, h, :].T)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        out[:, h, :] = (e / z) @ V[:, h, :]
        lse[:, h] = (m + np.log(z))[:, 0]
    return out, lse
