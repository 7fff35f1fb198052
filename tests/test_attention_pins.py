"""CPU pins of the sparse-attention oracle (``oracle/attention.py``): values
worked by hand, closed forms, a reduction to a library attention routine, and
invariances, each checked to catch a plausible mistake in the oracle (planted
below in mutated copies)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import attention as att


# ------------------------------------------------------------ by hand ----

def test_worked_example_two_entries():
    # One head, D_K = D_V = 2, scale 1.  Entry 0 is (ln 3, 5), entry 1 is
    # (0, 1); q = (1, 0) gives logits ln 3 and 0, so the weights are 3/4 and
    # 1/4 and the output is (3/4 ln 3, 3/4*5 + 1/4*1) = (0.75 ln 3, 4).
    kv = np.array([[math.log(3.0), 5.0], [0.0, 1.0], [7.0, 7.0]])
    q = np.array([[[1.0, 0.0]]])
    idx = np.array([[0, 1, -1]])
    out = att.sparse_attention(q, kv, idx, 2, 1.0)
    assert np.allclose(out[0, 0], [0.75 * math.log(3.0), 4.0], rtol=0, atol=1e-15)


def test_worked_example_duplicates_and_scale():
    # Two heads, D_K = D_V = 1, scale 1/2, entries 2 and 4, selection
    # (1, 1, 0): entry 1 is listed twice and counts twice.
    #   head 0 (q = 0): uniform over three listed entries: (4 + 4 + 2)/3 = 10/3.
    #   head 1 (q = 1): logits 2, 2, 1, weights e^2, e^2, e:
    #     (4e^2 + 4e^2 + 2e) / (2e^2 + e) = (8e + 2) / (2e + 1).
    kv = np.array([[2.0], [4.0]])
    q = np.array([[[0.0], [1.0]]])
    idx = np.array([[1, 1, 0]])
    out = att.sparse_attention(q, kv, idx, 1, 0.5)
    e = math.e
    assert abs(out[0, 0, 0] - 10.0 / 3.0) < 1e-14
    assert abs(out[0, 1, 0] - (8 * e + 2) / (2 * e + 1)) < 1e-14


def test_empty_selection_gives_zeros():
    kv = np.ones((4, 8))
    q = np.ones((2, 3, 8))
    idx = np.array([[-1, -1], [2, -1]])
    out = att.sparse_attention(q, kv, idx, 4, 0.1)
    assert np.all(out[0] == 0.0)
    assert np.allclose(out[1], 1.0)


# ------------------------------------------------------- closed forms ----

def test_single_entry_returns_its_value():
    rng = np.random.default_rng(1)
    kv = rng.standard_normal((50, 24))
    q = rng.standard_normal((6, 4, 24))
    idx = np.full((6, 5), -1)
    idx[:, 2] = rng.integers(0, 50, 6)
    out = att.sparse_attention(q, kv, idx, 16, 0.3)
    for i in range(6):
        assert np.allclose(out[i], np.broadcast_to(kv[idx[i, 2], :16], (4, 16)), atol=1e-14)


def test_zero_query_averages_values():
    rng = np.random.default_rng(2)
    kv = rng.standard_normal((40, 12))
    q = np.zeros((3, 2, 12))
    idx = rng.integers(-1, 40, (3, 9))
    out = att.sparse_attention(q, kv, idx, 8, 1.7)
    for i in range(3):
        sel = idx[i][idx[i] >= 0]
        assert np.allclose(out[i], np.broadcast_to(kv[sel, :8].mean(axis=0), (2, 8)), atol=1e-14)


# --------------------------------------------------- library routine ----

def test_matches_library_attention_with_dense_mask():
    """Over distinct selected entries the sparse attention is dense softmax
    attention over all entries with the unselected ones masked out: torch's
    scaled_dot_product_attention (float64, CPU) with a boolean mask."""
    rng = np.random.default_rng(3)
    S, T, H, DK, DV, k = 12, 70, 5, 20, 12, 9
    kv = rng.standard_normal((T, DK))
    q = rng.standard_normal((S, H, DK))
    idx = np.full((S, k), -1)
    for i in range(S):
        n = int(rng.integers(1, k + 1))
        idx[i, :n] = rng.choice(T, n, replace=False)
        rng.shuffle(idx[i])
    scale = 0.37
    out = att.sparse_attention(q, kv, idx, DV, scale)
    mask = np.zeros((S, T), dtype=bool)
    for i in range(S):
        mask[i, idx[i][idx[i] >= 0]] = True
    Q = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(2)             # [H, S, 1, DK]
    K = torch.from_numpy(kv).expand(H, S, T, DK)                      # [H, S, T, DK]
    V = torch.from_numpy(kv[:, :DV]).expand(H, S, T, DV)
    M = torch.from_numpy(mask).unsqueeze(1).expand(S, 1, T).unsqueeze(0).expand(H, S, 1, T)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=M, scale=scale)
    ref = ref.squeeze(2).permute(1, 0, 2).numpy()                     # [S, H, DV]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------- invariance ----

def test_order_of_the_selection_does_not_matter():
    rng = np.random.default_rng(4)
    kv = rng.standard_normal((30, 16))
    q = rng.standard_normal((4, 3, 16))
    idx = rng.integers(-1, 30, (4, 11))
    out = att.sparse_attention(q, kv, idx, 8, 0.5)
    perm = idx[:, rng.permutation(11)]
    out2 = att.sparse_attention(q, kv, perm, 8, 0.5)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-13)


# ------------------------------------------------ planted mistakes ----

_ROW = att.sparse_attention_row


def _mutants():
    def no_scale(q_row, kv, sel, d_v, scale):
        return _ROW(q_row, kv, sel, d_v, 1.0)

    def softmax_over_heads(q_row, kv, sel, d_v, scale):
        if len(sel) == 0:
            return np.zeros((q_row.shape[0], d_v))
        lat = kv[np.asarray(sel)]
        lg = scale * (q_row @ lat.T)
        p = np.exp(lg - lg.max(axis=0, keepdims=True))
        p = p / p.sum(axis=0, keepdims=True)
        return p @ lat[:, :d_v]

    def values_from_tail(q_row, kv, sel, d_v, scale):
        if len(sel) == 0:
            return np.zeros((q_row.shape[0], d_v))
        lat = kv[np.asarray(sel)]
        lg = scale * (q_row @ lat.T)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        return p @ lat[:, -d_v:]

    def unnormalised(q_row, kv, sel, d_v, scale):
        if len(sel) == 0:
            return np.zeros((q_row.shape[0], d_v))
        lat = kv[np.asarray(sel)]
        lg = scale * (q_row @ lat.T)
        return np.exp(lg - lg.max(axis=1, keepdims=True)) @ lat[:, :d_v]

    def transposed_logits(q_row, kv, sel, d_v, scale):
        if len(sel) == 0:
            return np.zeros((q_row.shape[0], d_v))
        lat = kv[np.asarray(sel)]
        lg = scale * (q_row @ lat.T)
        lg = lg[::-1]
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        return p @ lat[:, :d_v]
    return [no_scale, softmax_over_heads, values_from_tail, unnormalised, transposed_logits]


def _pins_pass(row_fn):
    """All pins above, run against a row function; False when one fails."""
    saved = att.sparse_attention_row
    att.sparse_attention_row = row_fn
    try:
        for t in (test_worked_example_two_entries, test_worked_example_duplicates_and_scale,
                  test_single_entry_returns_its_value, test_zero_query_averages_values,
                  test_matches_library_attention_with_dense_mask):
            try:
                t()
            except AssertionError:
                return False
        return True
    finally:
        att.sparse_attention_row = saved


def test_pins_pass_on_the_oracle():
    assert _pins_pass(att.sparse_attention_row)


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutant):
    assert not _pins_pass(mutant)


def test_magnitude_variant_agrees_and_bounds():
    """The magnitude companion returns the same outputs, a sum of |values|
    that bounds them, and equals them when every value is nonnegative."""
    rng = np.random.default_rng(5)
    kv = rng.standard_normal((60, 20))
    q = rng.standard_normal((5, 4, 20))
    idx = rng.integers(-1, 60, (5, 13))
    out = att.sparse_attention(q, kv, idx, 12, 0.4)
    out2, mag = att.sparse_attention_with_magnitude(q, kv, idx, 12, 0.4)
    assert np.allclose(out, out2, rtol=1e-14, atol=1e-14)
    assert np.all(mag >= np.abs(out) - 1e-14)
    kvp = np.abs(kv)
    o3, m3 = att.sparse_attention_with_magnitude(q, kvp, idx, 12, 0.4)
    assert np.allclose(o3, m3, rtol=1e-14, atol=1e-14)
