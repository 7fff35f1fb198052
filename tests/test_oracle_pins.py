"""CPU tests of the oracle against what the definition and the mathematics fix.

Marked neither gpu nor slow: the whole module runs in well under a minute.
"""
from __future__ import annotations

import math
import os
import tempfile

import numpy as np
import pytest
import torch

import pins
from streaming_indexer_top_amd import inputs


def test_worked_examples(oracle_mod):
    assert pins.run_golden() == []


def test_brute_force_integer(oracle_mod):
    assert pins.run_brute_integer() == []


def test_brute_force_float(oracle_mod):
    assert pins.run_brute_float() == []


def test_fp32_error_bound_full_width(oracle_mod):
    assert pins.run_error_bound_wide() == []


def test_single_head_reduces_to_lexsort(oracle_mod):
    assert pins.run_single_head_lexsort() == []


def _invariants(idx, score, pos, T, m, k):
    for r in range(idx.shape[0]):
        n = min(T, (int(pos[r]) + 1) // m)
        cnt = min(k, n)
        row_i, row_s = idx[r], score[r]
        assert np.all(row_i[cnt:] == -1) and np.all(np.isneginf(row_s[cnt:]))
        valid = row_i[:cnt]
        assert len(set(valid.tolist())) == cnt
        assert np.all((valid >= 0) & (valid < n))
        vs = row_s[:cnt]
        assert np.all(np.isfinite(vs))
        # sorted by (score desc, idx asc)
        for t in range(cnt - 1):
            assert vs[t] > vs[t + 1] or (vs[t] == vs[t + 1] and valid[t] < valid[t + 1])
        assert not np.any((vs == 0) & np.signbit(vs))


def test_invariants_bf16_shaped(oracle_mod):
    S, T, H, D, m, k = 300, 70, 8, 32, 4, 24
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=11)
    idx, score = oracle_mod.topk(q.float().numpy(), w.float().numpy(), kc.float().numpy(), m, k)
    _invariants(idx, score, np.arange(S), T, m, k)


def test_maximality_integer(oracle_mod):
    """Every selected key scores at least as high as every unselected usable key."""
    S, T, H, D, m, k = 200, 48, 6, 16, 4, 10
    q, w, kc = pins.torch_seeded_integer(S, T, H, D, seed=21)
    idx, score = oracle_mod.topk(q, w, kc, m, k)
    for i in range(S):
        n = min(T, (i + 1) // m)
        full = oracle_mod.row_scores(q[i], w[i], kc, n)
        cnt = min(k, n)
        sel = set(idx[i, :cnt].tolist())
        if cnt and len(sel) < n:
            worst_sel = min(full[j] for j in sel)
            best_out = max(full[j] for j in range(n) if j not in sel)
            assert worst_sel >= best_out
        for t in range(cnt):
            assert score[i, t] == full[idx[i, t]]


def test_partition_merge_identity(oracle_mod):
    """Top-k of all keys equals the top-k of the union of per-chunk top-k
    lists, under the (score desc, index asc) order: the identity that the
    chunked partition-merge driver rests on."""
    rng = np.random.default_rng(7)
    T, H, D, k = 90, 5, 9, 12
    q = rng.integers(-3, 4, size=(4, H, D)).astype(np.float32)
    w = rng.choice(np.array([-2, -1, 1, 2], dtype=np.float32), size=(4, H))
    kc = rng.integers(-3, 4, size=(T, D)).astype(np.float32)
    far = np.full(4, 10 * T, dtype=np.int64)  # every key usable
    full_idx, full_sc = oracle_mod.topk(q, w, kc, 1, k, pos=far)
    for chunk in (7, 16, 31, 90):
        lists = []
        for c0 in range(0, T, chunk):
            ci, cs = oracle_mod.topk(q, w, kc[c0:c0 + chunk], 1, k, pos=far)
            lists.append((np.where(ci >= 0, ci + c0, -1), cs))
        for r in range(4):
            cand = [(float(cs[r, t]), int(ci[r, t])) for ci, cs in lists
                    for t in range(k) if ci[r, t] >= 0]
            cand.sort(key=lambda e: (-e[0], e[1]))
            assert [j for _, j in cand[:k]] == list(full_idx[r])
            assert [s for s, _ in cand[:k]] == [float(x) for x in full_sc[r]]


def test_integer_scores_exact_at_full_width(oracle_mod):
    """Integer inputs at H=64, D=128: |score| <= 9*128*2*64 < 2^24, so every
    fp32 partial sum is an exact integer and the oracle's scores equal exact
    int64 arithmetic (numpy), whatever the order."""
    S, T, H, D = 16, 40, 64, 128
    q, w, kc = pins.torch_seeded_integer(S, T, H, D, seed=5)
    qi, wi, ki = q.astype(np.int64), w.astype(np.int64), kc.astype(np.int64)
    for i in range(S):
        got = oracle_mod.row_scores(q[i], w[i], kc, T)
        dots = qi[i] @ ki.T  # [H, T]
        want = (wi[i][:, None] * np.maximum(dots, 0)).sum(axis=0)
        assert np.array_equal(got.astype(np.int64), want)
        assert np.all(got == want.astype(np.float32))


def test_pair_count_closed_form(oracle_mod):
    """P = sum_i n(i) = T*(m*(T-1)+2)/2 when S = m*T (rows i < m-1 see no key,
    then each key count holds for m rows, and the last count T for one row)."""
    for T, m in [(1, 1), (5, 1), (256, 4), (4096, 4), (16384, 4), (37, 3)]:
        S = m * T
        P = int(oracle_mod.n_valid(np.arange(S), T, m).sum())
        assert P == T * (m * (T - 1) + 2) // 2


def test_materialised_size_identity():
    """The page's 256 GB figure for the FP32 [B,S,H_I,T] score tensor at
    S=65,536, H_I=64, m=4 is exactly 2^38 bytes."""
    S, H, m = 65536, 64, 4
    T = S // m
    assert 1 * S * H * T * 4 == 2 ** 38 == 256 * 2 ** 30


def test_rows_independent_of_position_offset(oracle_mod):
    """Rows [a, b) computed alone with their absolute positions equal the
    same rows of the full run."""
    S, T, H, D, m, k = 120, 30, 4, 8, 4, 9
    q, w, kc = pins.torch_seeded_integer(S, T, H, D, seed=8)
    idx, sc = oracle_mod.topk(q, w, kc, m, k)
    a, b = 37, 91
    idx2, sc2 = oracle_mod.topk(q[a:b], w[a:b], kc, m, k, q_pos0=a)
    assert np.array_equal(idx[a:b], idx2) and np.array_equal(sc[a:b], sc2)


def test_rejects_nonfinite(oracle_mod):
    q = np.ones((2, 1, 2), dtype=np.float32)
    w = np.ones((2, 1), dtype=np.float32)
    kc = np.array([[1.0, np.nan]], dtype=np.float32)
    with pytest.raises(RuntimeError):
        oracle_mod.topk(q, w, kc, 1, 1)


def test_thread_count_does_not_change_result(oracle_mod):
    S, T, H, D, m, k = 64, 16, 3, 5, 2, 7
    q, w, kc = inputs.gaussian_fp32(S, T, H, D, seed=1)
    a = oracle_mod.topk(q.numpy(), w.numpy(), kc.numpy(), m, k, nthreads=1)
    b = oracle_mod.topk(q.numpy(), w.numpy(), kc.numpy(), m, k, nthreads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --- planted mistakes: each broken copy of the oracle must fail some pin ---

MUTANTS = {
    "no_relu": ("float r = (a > 0.0f) ? a : 0.0f;", "float r = a;"),
    "unweighted_heads": ("float t = w_row[h] * r;", "float t = r;"),
    "negated_weight": ("float t = w_row[h] * r;", "float t = -w_row[h] * r;"),
    "dropped_last_head": ("for (int32_t h = 0; h < H; ++h) {\n        const float *qh",
                          "for (int32_t h = 0; h < H - 1; ++h) {\n        const float *qh"),
    "q_transposed": ("float p = qh[d] * key[d];",
                     "float p = q_row[(int64_t)d * H + h] * key[d]; (void)qh;"),
    "causal_off_by_one": ("int64_t n = (pos + 1) / m;", "int64_t n = pos / m;"),
    "causal_one_extra": ("int64_t n = (pos + 1) / m;", "int64_t n = (pos + m) / m;"),
    "ties_index_desc": ("if (a->j < b->j) return -1;\n    if (a->j > b->j) return 1;",
                        "if (a->j < b->j) return 1;\n    if (a->j > b->j) return -1;"),
    "ascending_scores": ("if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
                         "if (a->s > b->s) return 1;\n    if (a->s < b->s) return -1;"),
    "pad_score_zero": ("score[t] = -INFINITY;", "score[t] = 0.0f;"),
    "pad_index_zero": ("idx[t] = -1;", "idx[t] = 0;"),
    "negative_zero_start": ("float s = 0.0f;\n    for (int32_t h", "float s = -0.0f;\n    for (int32_t h"),
    "first_head_weight_only": ("float t = w_row[h] * r;", "float t = w_row[0] * r;"),
    "relu_on_weighted_term": ("float t = w_row[h] * r;", "float t = w_row[h] * a; (void)r;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(oracle_mod, name):
    import oracle
    src_path = os.path.join(os.path.dirname(oracle.__file__), "csa_oracle.c")
    src = open(src_path).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "mut.c")
        with open(p, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.open_library(oracle.compile_source(p, os.path.join(d, "libmut.so")))
        caught = []
        for pin_name, pin in pins.ALL_PINS.items():
            if pin(lib):
                caught.append(pin_name)
                break
        assert caught, "no pin caught the planted mistake %s" % name
