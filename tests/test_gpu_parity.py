"""GPU parity: libcsa_indexer.so (through its C ABI) against the CPU oracle.

Integer-valued inputs are compared bit for bit (indices and score bits);
float inputs by the tolerance rules in ``checks.py`` (2e-3 relative scores,
threshold, min set recall 0.998).  Sizes run from tiny edge cases through
several tiles with ragged tails to the full workload shapes, where the oracle
checks a fixed sample of rows.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import checks
import oracle
import streaming_indexer_top_amd as csa
from streaming_indexer_top_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_topk(q, w, kc, m, k, **kw):
    idx, sc = csa.topk(q.to(DEV), w.to(DEV), kc.to(DEV), m, k, **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def oracle_topk(q, w, kc, m, k, rows=None, q_pos0=0):
    qf = q.float().cpu().numpy() if hasattr(q, "float") else q
    wf = w.float().cpu().numpy() if hasattr(w, "float") else w
    kf = kc.float().cpu().numpy() if hasattr(kc, "float") else kc
    if rows is None:
        return oracle.topk(qf, wf, kf, m, k, q_pos0=q_pos0)
    rows = np.asarray(rows, dtype=np.int64)
    return oracle.topk(qf[rows], wf[rows], kf, m, k, pos=rows + q_pos0)


def assert_no_fail(fails):
    assert not fails, "\n".join(fails[:10])


# ---------------------------------------------------------------- tiny ----

def test_tiny_fp32_gaussian():
    c = inputs.config(1)
    S, T, H, D, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    q, w, kc = inputs.gaussian_fp32(S, T, H, D, seed=1)
    say("tiny fp32 gaussian S=%d T=%d H=%d D=%d k=%d" % (S, T, H, D, k))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    fails, stats = checks.check_float(g_idx, g_sc, o_idx, o_sc, q.numpy(), w.numpy(),
                                      kc.numpy(), np.arange(S), T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("signed_w", [False, True])
def test_tiny_integer_bit_exact(dtype, signed_w):
    c = inputs.config(1)
    S, T, H, D, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=1, dtype=dtype, signed_w=signed_w)
    say("tiny integer %s signed_w=%s" % (dtype, signed_w))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))
    assert_no_fail(checks.check_structure(g_idx, g_sc, np.arange(S), T, m, k))


EDGE_CASES = [
    # S, T, H, D, m, k, q_pos0
    (1, 4, 4, 32, 4, 3, 0),       # one row, no usable key
    (7, 3, 4, 32, 1, 5, 0),       # ragged query block, k > T
    (37, 10, 5, 32, 1, 4, 0),     # m = 1
    (50, 9, 3, 64, 5, 6, 0),      # m = 5, D = 64
    (64, 16, 1, 32, 4, 2, 0),     # single head
    (64, 16, 33, 128, 4, 8, 0),   # heads spill into a second 32-head block
    (96, 200, 64, 128, 2, 20, 0),  # several key tiles, ragged tail
    (40, 30, 8, 32, 4, 7, 100),   # row offset: rows see all 30 keys
    (20, 0, 4, 32, 4, 5, 0),      # no keys at all
    (300, 300, 16, 64, 1, 2048, 0),  # k beyond every row's key count
]


@pytest.mark.parametrize("chunk", [0, 1280])
def test_fp32_long_rows_bit_exact(chunk):
    """fp32 integer inputs whose rows see about 3,250-3,300 keys (about a
    hundred 32-key tiles of the fp32 kernel, the last one ragged), with a
    ragged last query block (203 rows); with 1,280-key chunks the running
    lists are merged across three chunks."""
    S, T, H, D, m, k, q_pos0 = 203, 3500, 64, 128, 4, 300, 13000
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=77, dtype=torch.float32, signed_w=True)
    say("fp32 long rows chunk=%d" % chunk)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, chunk_keys=chunk)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


def test_fp32_gaussian_long_rows():
    """fp32 Gaussian inputs, 1,024 rows that see about 2,000-2,250 keys each,
    by the tolerance rules."""
    S, T, H, D, m, k, q_pos0 = 1024, 4096, 64, 128, 4, 512, 8000
    q, w, kc = inputs.gaussian_fp32(S, T, H, D, seed=5)
    say("fp32 gaussian long rows")
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    fails, stats = checks.check_float(g_idx, g_sc, o_idx, o_sc, q.numpy(), w.numpy(),
                                      kc.numpy(), np.arange(S) + q_pos0, T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", EDGE_CASES)
def test_edge_cases_bit_exact(dtype, case):
    S, T, H, D, m, k, q_pos0 = case
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=S + T, dtype=dtype, signed_w=True)
    say("edge case %s %s" % (case, dtype))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


def test_empty_query_set():
    q = torch.zeros((0, 4, 32), dtype=torch.bfloat16)
    w = torch.zeros((0, 4), dtype=torch.bfloat16)
    kc = torch.zeros((8, 32), dtype=torch.bfloat16)
    g_idx, g_sc = gpu_topk(q, w, kc, 4, 3)
    assert g_idx.shape == (0, 3) and g_sc.shape == (0, 3)


def test_crowded_threshold_bin_is_refined():
    """Every score lies in [1.0, 1.25), one bin of the score kernel's
    histogram, so the select kernel must split that bin by its next bits
    (more keys than its boundary buffer holds) and still return the exact
    top-k by the tolerance rules."""
    S, T, H, D, m, k, q_pos0 = 16, 8192, 1, 128, 1, 64, 10000
    g = torch.Generator().manual_seed(12)
    q = torch.full((S, H, D), 1.0 / 128, dtype=torch.bfloat16)
    w = torch.ones((S, H), dtype=torch.bfloat16)
    kc = (1.0 + 0.2 * torch.rand((T, D), generator=g)).to(torch.bfloat16)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    assert np.all((g_sc >= 1.0) & (g_sc < 1.25))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    fails, stats = checks.check_float(g_idx, g_sc, o_idx, o_sc, q.float().numpy(),
                                      w.float().numpy(), kc.float().numpy(),
                                      np.arange(S) + q_pos0, T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("k", [2048, 4096])
@pytest.mark.parametrize("values", ["all_zero", "two_values"])
def test_massively_tied_scores_bit_exact(dtype, k, values):
    """Rows of about 20,000 keys whose scores take one value (q = 0) or two
    (every third key scores 1, the rest 0): the boundary bin stays crowded
    after its refinement, so the select kernel falls back to its piecewise
    radix select, and the sort's buckets overflow into the bitonic sort.
    Ties go by index, so the result is unique; it must equal the oracle bit
    for bit with one chunk, with 4,096-key chunks and with key splits."""
    S, T, H, D, m = 16, 20000, 4, 32, 1
    q_pos0 = T - S  # rows see 19,985 .. 20,000 keys
    q = torch.zeros((S, H, D), dtype=dtype)
    w = torch.ones((S, H), dtype=dtype)
    kc = torch.zeros((T, D), dtype=dtype)
    if values == "two_values":
        q[:, :, 0] = 1.0
        kc[::3, 0] = 1.0
    say("tied scores %s k=%d %s" % (values, k, dtype))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    for kw in ({}, dict(chunk_keys=4096), dict(key_splits=4)):
        say("  %s" % kw)
        g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, **kw)
        assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nonfinite_inputs_stay_in_bounds(dtype):
    """NaN or Inf inputs give unspecified results (the library does not
    detect them), but the call completes in bounds: rows with finite inputs
    are still bit-exact, and every row returns min(k, n) distinct usable
    keys followed by padding."""
    S, T, H, D, m, k = 24, 6000, 8, 64, 1, 300
    q_pos0 = T - S
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=90, dtype=dtype, signed_w=True)
    q[0:4] = float("nan")            # every score NaN
    q[4:8, 0, 0] = float("inf")      # +-inf and NaN (inf * 0) logits in head 0
    w[8:12, 1] = float("-inf")       # an infinite head weight
    finite = np.arange(12, S)
    say("non-finite inputs %s" % dtype)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, rows=finite, q_pos0=q_pos0)
    assert_no_fail(checks.check_exact(g_idx[finite], g_sc[finite], o_idx, o_sc))
    n = oracle.n_valid(np.arange(S) + q_pos0, T, m)
    for r in range(S):
        c = int(min(k, n[r]))
        assert np.all(g_idx[r, :c] >= 0) and np.all(g_idx[r, :c] < n[r]), r
        assert len(np.unique(g_idx[r, :c])) == c, r
        assert np.all(g_idx[r, c:] == -1), r


def test_signed_zero_scores_are_positive():
    # Every head dot product is <= 0 and the weights are negative: every score
    # is zero and must come out as +0, with ties broken by index.
    S, T, H, D, m, k = 16, 4, 2, 32, 1, 3
    q = torch.zeros((S, H, D), dtype=torch.bfloat16)
    q[:, 0, 0] = -1.0
    q[:, 1, 1] = -1.0
    kc = torch.zeros((T, D), dtype=torch.bfloat16)
    kc[:, 0] = 1.0
    kc[:, 1] = 1.0
    w = -torch.ones((S, H), dtype=torch.bfloat16)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))
    assert not np.any(np.signbit(g_sc[g_idx >= 0]))


@pytest.mark.parametrize("sign", ["negative", "positive"])
@pytest.mark.parametrize("k", [256, 2048])
def test_one_sign_scores_bf16(sign, k):
    """All weights of one sign: every score has that sign (or is zero), so
    the sort's regions lie on one side of zero and are bucketed in the
    orderable integer; negative rows also put the best keys nearest zero.
    All rows checked by the tolerance rules."""
    S, T, H, D, m = 4096, 3000, 64, 128, 1
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=70 + k)
    w = w.abs() if sign == "positive" else -w.abs()
    say("one-sign scores %s k=%d" % (sign, k))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    fails, stats = checks.check_float(g_idx, g_sc, o_idx, o_sc, q.float().numpy(),
                                      w.float().numpy(), kc.float().numpy(), np.arange(S),
                                      T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


@pytest.mark.parametrize("chunk", [0, 1024])
def test_negative_weights_integer_bit_exact(chunk):
    """Integer inputs with negative weights only: scores <= 0, many exact
    ties (zero scores and repeated values), one chunk or several."""
    S, T, H, D, m, k = 2048, 3000, 8, 32, 1, 700
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=80, dtype=torch.bfloat16)
    w = -w
    say("negative integer weights chunk=%d" % chunk)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, chunk_keys=chunk)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


# -------------------------------------------------------------- medium ----

def test_medium_bf16_gaussian_full():
    S, T, H, D, m, k = 4096, 1024, 64, 128, 4, 256
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=2)
    say("medium bf16 gaussian S=%d T=%d k=%d" % (S, T, k))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    fails, stats = checks.check_float(g_idx, g_sc, o_idx, o_sc, q.float().numpy(),
                                      w.float().numpy(), kc.float().numpy(), np.arange(S),
                                      T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


def test_chunk_and_tile_grid_bit_identical():
    """Integer inputs, rows far longer than a chunk: every chunk x tile
    setting gives the same bits, equal to the oracle's."""
    S, T, H, D, m, k = 1024, 3000, 64, 128, 1, 512
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=4, dtype=torch.bfloat16, signed_w=True)
    q_pos0 = 2100  # rows see 2101..3000 keys
    say("chunk/tile grid S=%d T=%d k=%d" % (S, T, k))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    for chunk in (0, 256, 768, 2048):
        for tile in (64, 128, 192, 256):
            say("  chunk=%d tile=%d" % (chunk, tile))
            g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, chunk_keys=chunk, key_tile=tile)
            assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


def test_large_k_integer_bit_exact():
    """k up to 4096 (the larger select configuration): integer inputs bit for
    bit, with one chunk and with chunks much shorter than k (the running list
    holds more keys than a chunk has)."""
    S, T, H, D, m, k = 2048, 6000, 64, 128, 1, 4096
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=21, dtype=torch.bfloat16, signed_w=True)
    q_pos0 = 3000  # rows see 3001..5048 keys: below, at and above k
    say("large k integer S=%d T=%d k=%d" % (S, T, k))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    for chunk in (0, 1024, 2560):
        say("  chunk=%d" % chunk)
        g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, chunk_keys=chunk)
        assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


@pytest.mark.parametrize("k", [2049, 3000, 4096])
def test_large_k_bf16_gaussian(k):
    S, T, H, D, m = 4096, 6144, 64, 128, 1
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=22)
    q_pos0 = 2048  # rows see 2049..6144 keys
    say("large k bf16 S=%d T=%d k=%d" % (S, T, k))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    edge = np.array([k - q_pos0 - 2, k - q_pos0 - 1, k - q_pos0, S - 1])  # n(row) around k
    rows = np.unique(np.concatenate([np.arange(0, S, 16), np.clip(edge, 0, S - 1)]))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, rows=rows, q_pos0=q_pos0)
    fails, stats = checks.check_float(g_idx[rows], g_sc[rows], o_idx, o_sc,
                                      q.float().numpy()[rows], w.float().numpy()[rows],
                                      kc.float().numpy(), rows + q_pos0, T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


def test_large_k_beyond_keys_pads():
    S, T, H, D, m, k = 64, 1000, 8, 64, 1, 4096
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=23, dtype=torch.bfloat16, signed_w=True)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=900)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=900)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))
    assert (g_idx[:, 1000:] == -1).all()


def _stack(problems):
    return [torch.stack([p[i] for p in problems]).contiguous() for i in range(3)]


def test_batched_integer_bit_exact():
    """B problems with their own keys: each batch equals the oracle bit for
    bit, and equals the single call on its slices."""
    B, S, T, H, D, m, k = 3, 1500, 400, 64, 128, 4, 64
    probs = [inputs.integer_valued(S, T, H, D, seed=30 + b, dtype=torch.bfloat16, signed_w=True)
             for b in range(B)]
    q, w, kc = _stack(probs)
    say("batched integer B=%d S=%d T=%d k=%d" % (B, S, T, k))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k)
    assert g_idx.shape == (B, S, k)
    for b in range(B):
        o_idx, o_sc = oracle_topk(*probs[b], m, k)
        assert_no_fail(checks.check_exact(g_idx[b], g_sc[b], o_idx, o_sc))
        s_idx, s_sc = gpu_topk(*probs[b], m, k)
        assert np.array_equal(s_idx, g_idx[b])
        assert np.array_equal(s_sc.view(np.uint32), g_sc[b].view(np.uint32))


def test_batched_bf16_matches_single_calls_multi_pass():
    B, S, T, H, D, m, k = 2, 3000, 750, 64, 128, 4, 128
    probs = [inputs.bf16_gaussian(S, T, H, D, seed=40 + b) for b in range(B)]
    q, w, kc = _stack(probs)
    for budget, chunk in ((0, 0), (1, 256)):  # one pass; many passes and chunks
        say("batched bf16 budget=%d chunk=%d" % (budget, chunk))
        g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=100, workspace_budget=budget,
                               chunk_keys=chunk)
        for b in range(B):
            s_idx, s_sc = gpu_topk(*probs[b], m, k, q_pos0=100)
            assert np.array_equal(s_idx, g_idx[b])
            assert np.array_equal(s_sc.view(np.uint32), g_sc[b].view(np.uint32))


def test_batched_fp32_decode_with_key_splits():
    """Batched fp32 decode problems (12 rows against 9,000 keys each, so the
    plan splits the keys): each problem equals the oracle bit for bit and
    the single call on its slices."""
    B, S, T, H, D, m, k = 3, 12, 9000, 64, 128, 1, 700
    probs = [inputs.integer_valued(S, T, H, D, seed=60 + b, dtype=torch.float32, signed_w=True)
             for b in range(B)]
    q, w, kc = _stack(probs)
    q_pos0 = T - S
    say("batched fp32 decode B=%d S=%d T=%d k=%d" % (B, S, T, k))
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    for b in range(B):
        o_idx, o_sc = oracle_topk(*probs[b], m, k, q_pos0=q_pos0)
        assert_no_fail(checks.check_exact(g_idx[b], g_sc[b], o_idx, o_sc))
        s_idx, s_sc = gpu_topk(*probs[b], m, k, q_pos0=q_pos0)
        assert np.array_equal(s_idx, g_idx[b])
        assert np.array_equal(s_sc.view(np.uint32), g_sc[b].view(np.uint32))


@pytest.mark.parametrize("dtype, k", [(torch.bfloat16, 512), (torch.bfloat16, 4096),
                                      (torch.float32, 512)])
def test_key_splits_integer_bit_exact(dtype, k):
    """Few rows against many keys (decode shape): the keys are split, each
    split selects its own best k, the lists are merged in rounds.  Automatic
    and forced split counts, and several passes, all equal the oracle, for
    the bf16 and the fp32 score kernels."""
    S, T, H, D, m = 64, 20000, 64, 128, 1
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=50, dtype=dtype, signed_w=True)
    q_pos0 = T - 40  # rows see 19961..20000 keys (the last 24 rows all of them)
    say("key splits integer S=%d T=%d k=%d %s" % (S, T, k, dtype))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    for splits, budget in ((0, 0), (1, 0), (2, 0), (16, 0), (64, 0), (128, 0), (4, 1)):
        say("  key_splits=%d budget=%d" % (splits, budget))
        g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, key_splits=splits,
                               workspace_budget=budget)
        assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


def test_key_splits_bf16_decode():
    """32 new queries at the end of a 2^20-token sequence (262144 compressed
    keys): split plan against the oracle, and bit-identical to the unsplit
    (chunked) plan."""
    S, T, H, D, m, k = 32, 262144, 64, 128, 4, 2048
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=51)
    q_pos0 = 4 * T - S
    say("decode bf16 S=%d T=%d k=%d" % (S, T, k))
    a_idx, a_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0)
    b_idx, b_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, key_splits=1)
    assert np.array_equal(a_idx, b_idx)
    assert np.array_equal(a_sc.view(np.uint32), b_sc.view(np.uint32))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    fails, stats = checks.check_float(a_idx, a_sc, o_idx, o_sc, q.float().numpy(),
                                      w.float().numpy(), kc.float().numpy(),
                                      np.arange(S) + q_pos0, T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


@pytest.mark.parametrize("chunk", [0, 256])
def test_k1_bit_exact(chunk):
    """k = 1: the single best key often lies in the boundary bin alone."""
    S, T, H, D, m, k = 1121, 2447, 17, 128, 8, 1
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=60, dtype=torch.bfloat16, signed_w=True)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=1168, chunk_keys=chunk)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=1168)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


def _random_config(rng):
    dt = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    D = int(rng.choice([32, 64, 128]))
    H = int(rng.choice([1, 3, 17, 32, 33, 64]))
    m = int(rng.integers(1, 9))
    S = int(rng.integers(1, 1500))
    T = int(rng.integers(0, 4000))
    q_pos0 = int(rng.integers(0, 3000)) if rng.random() < 0.5 else 0
    k = int(rng.choice([1, 7, 64, 300, 2048, 2049, 4096]))
    opts = dict(chunk_keys=int(rng.choice([0, 0, 256, 1024])),
                key_tile=int(rng.choice([0, 64, 128, 192, 256])),
                key_splits=int(rng.choice([0, 0, 1, 2, 8])),
                workspace_budget=int(rng.choice([0, 0, 1, 1 << 20])))
    return dt, S, T, H, D, m, k, q_pos0, opts


@pytest.mark.parametrize("case", range(30))
def test_random_configs_integer_bit_exact(case):
    """Seeded random shapes, causal offsets, k, dtypes and options (chunks,
    tiles, key splits, tiny workspaces): integer inputs equal the oracle bit
    for bit."""
    rng = np.random.default_rng(1000 + case)
    dt, S, T, H, D, m, k, q_pos0, opts = _random_config(rng)
    say("random case %d: %s S=%d T=%d H=%d D=%d m=%d k=%d q_pos0=%d %s"
        % (case, dt, S, T, H, D, m, k, q_pos0, opts))
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=2000 + case, dtype=dt, signed_w=True)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, **opts)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


@pytest.mark.parametrize("case", range(20))
def test_random_configs_bf16_gaussian(case):
    """Seeded random V4-shaped bf16 problems with long rows (up to 30000
    keys: boundary refinement, running lists, key splits), checked by the
    tolerance rules on up to 64 sampled rows."""
    rng = np.random.default_rng(3000 + case)
    S = int(rng.integers(1, 4000))
    T = int(rng.integers(1, 30000))
    m = int(rng.choice([1, 2, 4, 8]))
    q_pos0 = int(rng.integers(0, 20000)) if rng.random() < 0.5 else 0
    k = int(rng.choice([1, 16, 500, 2048, 3000, 4096]))
    opts = dict(chunk_keys=int(rng.choice([0, 0, 4096, 16384])),
                key_tile=int(rng.choice([0, 64, 128, 192, 256])),
                key_splits=int(rng.choice([0, 0, 1, 4, 16])),
                workspace_budget=int(rng.choice([0, 0, 1 << 24])))
    say("gaussian case %d: S=%d T=%d m=%d k=%d q_pos0=%d %s" % (case, S, T, m, k, q_pos0, opts))
    q, w, kc = inputs.bf16_gaussian(S, T, 64, 128, seed=4000 + case)
    g_idx, g_sc = gpu_topk(q, w, kc, m, k, q_pos0=q_pos0, **opts)
    rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 62)]))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, rows=rows, q_pos0=q_pos0)
    fails, stats = checks.check_float(g_idx[rows], g_sc[rows], o_idx, o_sc,
                                      q.float().numpy()[rows], w.float().numpy()[rows],
                                      kc.float().numpy(), rows + q_pos0, T, m, k)
    say("stats %s" % stats)
    assert_no_fail(fails)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", ["chunks", "key_splits"])
def test_hip_graph_replays_match_eager(shape, dtype):
    """The call enqueues only kernel launches on the caller's stream (no
    allocation, no memset), so it can be captured in a HIP graph.  Every
    replay, with eager work in between, equals the eager result, for the
    bf16 and the fp32 score kernels."""
    if shape == "chunks":
        S, T, H, D, m, k, q_pos0, kw = 3000, 2500, 64, 128, 4, 512, 0, dict(chunk_keys=256)
    else:
        S, T, H, D, m, k, q_pos0, kw = 16, 60000, 64, 128, 1, 2048, 59984, {}
    gen = inputs.bf16_gaussian if dtype == "bf16" else inputs.gaussian_fp32
    q, w, kc = [t.to(DEV) for t in gen(S, T, H, D, seed=70)]
    say("graph %s %s" % (shape, dtype))
    ws_bytes = csa.workspace_size(S, T, H, D, m, k, q_pos0=q_pos0, dtype=q.dtype, **kw)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=DEV)
    idx = torch.empty((S, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((S, k), dtype=torch.float32, device=DEV)
    e_idx, e_sc = csa.topk(q, w, kc, m, k, q_pos0=q_pos0, **kw)  # eager (also warms up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        csa.topk(q, w, kc, m, k, q_pos0=q_pos0, workspace=ws, out=(idx, sc), **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        csa.topk(q, w, kc, m, k, q_pos0=q_pos0, workspace=ws, out=(idx, sc), **kw)
    for rep in range(3):
        idx.fill_(7)
        sc.zero_()
        ws.fill_(0xAB)  # the replay must not depend on the workspace's contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, e_idx), "replay %d" % rep
        assert torch.equal(sc.view(torch.int32), e_sc.view(torch.int32)), "replay %d" % rep
        _ = (q.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()


def test_small_workspace_many_passes():
    S, T, H, D, m, k = 2000, 500, 8, 64, 4, 64
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=6, dtype=torch.bfloat16, signed_w=True)
    o_idx, o_sc = oracle_topk(q, w, kc, m, k)
    for budget, chunk in ((1, 0), (300 * 1024, 256), (5 << 20, 0)):
        say("workspace budget %d chunk %d" % (budget, chunk))
        g_idx, g_sc = gpu_topk(q, w, kc, m, k, workspace_budget=budget, chunk_keys=chunk)
        assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))


def test_row_range_matches_full_run():
    S, T, H, D, m, k = 3000, 750, 64, 128, 4, 128
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=8)
    full = gpu_topk(q, w, kc, m, k)
    a, b = 1111, 2345
    part = gpu_topk(q[a:b].contiguous(), w[a:b].contiguous(), kc, m, k, q_pos0=a)
    assert np.array_equal(full[0][a:b], part[0])
    assert np.array_equal(full[1][a:b].view(np.uint32), part[1].view(np.uint32))


def test_scaling_keys_by_two_doubles_scores_exactly():
    S, T, H, D, m, k = 2048, 512, 64, 128, 4, 64
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=9)
    a_idx, a_sc = gpu_topk(q, w, kc, m, k)
    b_idx, b_sc = gpu_topk(q, w, (kc.float() * 2).to(torch.bfloat16), m, k)
    assert np.array_equal(a_idx, b_idx)
    assert np.array_equal(a_sc * 2, b_sc)


def test_repeat_runs_bit_identical():
    S, T, H, D, m, k = 4096, 1024, 64, 128, 4, 512
    q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=10)
    a = gpu_topk(q, w, kc, m, k)
    b = gpu_topk(q, w, kc, m, k)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


# ------------------------------------------------- full workload shapes ----

def _full_shape_check(cfg_n, kc_kind="gaussian", sample=None, integer=False, seed=None,
                      shard_tail=0):
    c = inputs.config(cfg_n)
    S, T, H, D, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    seed = cfg_n if seed is None else seed
    say("config %d S=%d T=%d %s%s sample=%s" % (cfg_n, S, T, "integer " if integer else "",
                                                kc_kind, sample))
    gen_dev = DEV if S >= 65536 else "cpu"
    if integer:
        q, w, kc = inputs.integer_valued(S, T, H, D, seed=seed, dtype=torch.bfloat16,
                                         signed_w=True, device=gen_dev)
    elif kc_kind == "mixture":
        q, w, kc = inputs.bf16_mixture(S, T, H, D, seed=seed, device=gen_dev)
    else:
        q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=seed, device=gen_dev)
    q, w, kc = q.to(DEV), w.to(DEV), kc.to(DEV)
    idx, sc = csa.topk(q, w, kc, m, k)
    torch.cuda.synchronize()
    if shard_tail:
        # The last rows on their own (the heaviest shard of a row-sharded
        # run): q_pos0 places them, and the outputs must equal the full run's.
        R = shard_tail
        s_idx, s_sc = csa.topk(q[S - R:], w[S - R:], kc, m, k, q_pos0=S - R)
        torch.cuda.synchronize()
        assert torch.equal(s_idx, idx[S - R:])
        assert torch.equal(s_sc.view(torch.int32), sc[S - R:].view(torch.int32))
        say("  tail shard of %d rows with q_pos0=%d identical to the full run" % (R, S - R))
        del s_idx, s_sc
    rows = np.arange(S) if sample is None else np.array(inputs.sample_rows(S, m, k, sample, seed))
    rows_t = torch.from_numpy(rows).to(DEV)
    g_idx = idx[rows_t].cpu().numpy()
    g_sc = sc[rows_t].cpu().numpy()
    qf = q[rows_t].float().cpu().numpy()
    wf = w[rows_t].float().cpu().numpy()
    kf = kc.float().cpu().numpy()
    del idx, sc, q, w
    torch.cuda.empty_cache()
    say("  gpu done, oracle on %d rows" % len(rows))
    o_idx, o_sc = oracle.topk(qf, wf, kf, m, k, pos=rows)
    if integer:
        assert_no_fail(checks.check_exact(g_idx, g_sc, o_idx, o_sc))
        return
    fails, stats = checks.check_float(g_idx, g_sc, o_idx, o_sc, qf, wf, kf, rows, T, m, k)
    say("  stats %s" % stats)
    assert_no_fail(fails)


def test_cfg2_integer_bit_exact():
    _full_shape_check(2, integer=True)


def test_cfg2_bf16_all_rows():
    _full_shape_check(2)


def test_cfg3_bf16_sampled():
    _full_shape_check(3, sample=4096)


def test_cfg3_integer_sampled():
    _full_shape_check(3, sample=1024, integer=True)


@pytest.mark.slow
def test_cfg4_mixture_sampled():
    _full_shape_check(4, kc_kind="mixture", sample=1024)


@pytest.mark.slow
def test_cfg5_sampled():
    _full_shape_check(5, sample=256, shard_tail=8192)


@pytest.mark.slow
def test_cfg5_integer_sampled():
    """The long-context shape (S = 2^20, T = 262,144) with signed integer
    inputs through the default plan (four 65,536-key chunks per long row,
    running lists merged after every chunk, many passes): 256 sampled rows,
    boundary rows included, bit for bit against the oracle.  Integer scores
    tie densely (about 15 keys share each value near the k-th), so the
    (score desc, index asc) order is exercised across chunk boundaries."""
    _full_shape_check(5, sample=256, integer=True)


def test_full_size_chunk_and_tile_grid_integer_bit_exact():
    """Rows that see all 262,144 keys of the long-context key table, signed
    integer inputs: every chunk size of the page's sweep (4,096 .. 65,536
    keys, i.e. 64 .. 4 chunks merged into the running lists) times every key
    tile (64, 128, 256), plus the automatic plan (key splits) and forced
    split counts, equals the oracle bit for bit."""
    S, T, H, D, m, k = 128, 262144, 64, 128, 4, 2048
    q_pos0 = m * T - S  # rows see T-31 .. T keys
    q, w, kc = inputs.integer_valued(S, T, H, D, seed=90, dtype=torch.bfloat16, signed_w=True)
    say("full-size chunk/tile grid S=%d T=%d k=%d q_pos0=%d" % (S, T, k, q_pos0))
    o_idx, o_sc = oracle_topk(q, w, kc, m, k, q_pos0=q_pos0)
    qd, wd, kd = q.to(DEV), w.to(DEV), kc.to(DEV)
    settings = [dict(chunk_keys=c, key_tile=t) for c in (4096, 8192, 16384, 32768, 65536)
                for t in (64, 128, 256)]
    settings += [dict(chunk_keys=c, key_tile=192) for c in (4096, 65536)]
    settings += [dict(), dict(key_splits=1), dict(key_splits=4), dict(key_splits=64)]
    for kw in settings:
        say("  %s" % kw)
        idx, sc = csa.topk(qd, wd, kd, m, k, q_pos0=q_pos0, **kw)
        torch.cuda.synchronize()
        assert_no_fail(checks.check_exact(idx.cpu().numpy(), sc.cpu().numpy(), o_idx, o_sc))


def test_host_or_strided_caller_buffers_are_refused():
    """Outputs or a workspace in host memory, or a stride-0 workspace, are
    refused by the binding before any library call."""
    say("caller buffers on the host")
    q, w, kc = inputs.integer_valued(64, 16, 4, 32, seed=3, dtype=torch.bfloat16)
    q, w, kc = q.to(DEV), w.to(DEV), kc.to(DEV)
    host_out = (torch.empty((64, 8), dtype=torch.int32), torch.empty((64, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="must be on"):
        csa.topk(q, w, kc, 4, 8, out=host_out)
    with pytest.raises(ValueError, match="must be on"):
        csa.topk_noalloc(q, w, kc, 4, 8, out=host_out)
    with pytest.raises(ValueError, match="must be on"):
        csa.topk(q, w, kc, 4, 8, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous"):
        csa.topk(q, w, kc, 4, 8,
                 workspace=torch.zeros(1, dtype=torch.uint8, device=DEV).expand(1 << 24))
    qa = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((16, 128), dtype=torch.bfloat16, device=DEV)
    ia = torch.zeros((4, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="must be on"):
        csa.sparse_attention(qa, kv, ia, 128, out=torch.empty((4, 64, 128), dtype=torch.bfloat16))
    torch.cuda.synchronize()


def test_concurrent_calls_from_host_threads():
    """Calls from several host threads at once, each on its own stream with
    its own workspace and outputs (the library's shared state is only
    synchronised bookkeeping), give the results of serial calls bit for
    bit."""
    import threading
    say("concurrent host threads")
    probs = []
    for t in range(4):
        dt = torch.bfloat16 if t % 2 == 0 else torch.float32
        q, w, kc = [x.to(DEV) for x in inputs.integer_valued(500 + 100 * t, 3000, 64, 128,
                                                             seed=120 + t, dtype=dt,
                                                             signed_w=True)]
        probs.append((q, w, kc, 4, 256 + 64 * t))
    serial = []
    for q, w, kc, m, k in probs:
        serial.append(csa.topk(q, w, kc, m, k))
    torch.cuda.synchronize()
    results = [None] * len(probs)
    errors = []

    def work(i):
        try:
            q, w, kc, m, k = probs[i]
            st = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(st):
                out = None
                for _ in range(3):
                    out = csa.topk(q, w, kc, m, k)
                st.synchronize()
            results[i] = out
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(probs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (a, b) in enumerate(zip(serial, results)):
        assert torch.equal(a[0], b[0]), i
        assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), i

