"""CPU oracle for the sparse attention that consumes the indexer's selection.

TEST INFRASTRUCTURE ONLY: the tests and ``bench.py``'s ``cpu_baseline`` leg
are the only callers; the GPU library and its binding never import it.

The page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
Streaming Top-k" (Abstract) describes the CSA pipeline as: the lightning
indexer scores the compressed entries, the top-k are kept per query, and a
sparse attention kernel reads only those entries.  The page states no
formula and no dimensions for that attention.  The reading taken here is the
plain softmax attention of one query row over its selected compressed
entries, in the shared-latent (multi-query) form: every one of the H query
heads attends over the same selected entries, each entry's latent vector is
the key (all D_K dims) and its first D_V dims are the value:

    out[i, h, :] = sum_{e in sel(i)} p_{h,e} kv[e, :D_V],
    p_{h,e} = softmax over e of (scale * q[i, h, :] . kv[e, :])

where sel(i) lists idx[i, :] without its -1 padding (an entry listed twice
counts twice) and a row with nothing selected gives zeros.  Everything is
computed in float64, one row at a time, with a max-shifted softmax.
"""
from __future__ import annotations

import numpy as np


def sparse_attention_row(q_row, kv, sel, d_v, scale):
    """One query row: q_row [H, D_K], sel the selected entry indices (no
    padding) -> [H, d_v] float64."""
    h = q_row.shape[0]
    if len(sel) == 0:
        return np.zeros((h, d_v), dtype=np.float64)
    lat = np.asarray(kv, dtype=np.float64)[np.asarray(sel, dtype=np.int64)]  # [n, D_K]
    logits = scale * (np.asarray(q_row, dtype=np.float64) @ lat.T)          # [H, n]
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ lat[:, :d_v]


def sparse_attention_with_magnitude(q, kv, idx, d_v, scale, rows=None):
    """As sparse_attention, plus mag[r, h, :] = sum_e p_{h,e} |kv[e, :d_v]|,
    the size of the terms each output element sums (what rounding errors of
    the weights scale with)."""
    q = np.asarray(q)
    idx = np.asarray(idx)
    rows = range(q.shape[0]) if rows is None else rows
    out = np.zeros((len(rows), q.shape[1], d_v), dtype=np.float64)
    mag = np.zeros_like(out)
    for r, i in enumerate(rows):
        sel = idx[i][idx[i] >= 0]
        if len(sel) == 0:
            continue
        lat = np.asarray(kv, dtype=np.float64)[sel.astype(np.int64)]
        logits = scale * (np.asarray(q[i], dtype=np.float64) @ lat.T)
        logits = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p = p / p.sum(axis=1, keepdims=True)
        out[r] = p @ lat[:, :d_v]
        mag[r] = p @ np.abs(lat[:, :d_v])
    return out, mag


def sparse_attention(q, kv, idx, d_v, scale, rows=None):
    """q [S, H, D_K], kv [T, D_K], idx [S, k] (int, -1 = none): out
    [len(rows), H, d_v] float64 for the given rows (default: all)."""
    q = np.asarray(q)
    idx = np.asarray(idx)
    rows = range(q.shape[0]) if rows is None else rows
    out = np.zeros((len(rows), q.shape[1], d_v), dtype=np.float64)
    for r, i in enumerate(rows):
        sel = idx[i][idx[i] >= 0]
        out[r] = sparse_attention_row(q[i], kv, sel, d_v, scale)
    return out
