"""GPU parity of the sparse attention (``csa_sparse_attention`` through the C
ABI) against the float64 oracle in ``oracle/attention.py``.

Tolerance, from the arithmetic: logits are fp32 sums of exact bf16 products;
the softmax weights are fp32 and rounded to bf16 (relative error <= 2^-9
each) for the weighted sum, which accumulates in fp32, while the normaliser
sums the unrounded weights; the output is rounded to bf16 (<= 2^-9 of it).
So every element obeys

    |out - ref| <= 2^-8 * (|ref| + sum_e p_e |v_e|) + 1e-6

with sum_e p_e |v_e| from the oracle, leaving room for the fp32 logit error.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import streaming_indexer_top_amd as csa
from oracle import attention as att
from streaming_indexer_top_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_and_check(q, kv, idx, d_v, scale, rows=None):
    out = csa.sparse_attention(q.to(DEV), kv.to(DEV), idx.to(DEV), d_v, scale=scale)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    rows = list(range(q.shape[0])) if rows is None else list(rows)
    ref, mag = att.sparse_attention_with_magnitude(q.float().numpy(), kv.float().numpy(),
                                                   idx.numpy(), d_v, scale, rows=rows)
    g = g[rows]
    err = np.abs(g - ref)
    bound = 2.0 ** -8 * (np.abs(ref) + mag) + 1e-6
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "first failures (row, head, dim): %s; err %s bound %s" % (
        bad[:5].tolist(), err[tuple(bad[0])], bound[tuple(bad[0])])
    return g, ref


def random_selection(rng, S, T, k, pad_frac=0.2):
    idx = rng.integers(0, T, (S, k)).astype(np.int32)
    for i in range(S):
        n = int(rng.integers(0, k + 1)) if rng.random() < pad_frac else k
        idx[i, n:] = -1
    return torch.from_numpy(idx)


@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("dims", [(576, 512), (128, 128)])
@pytest.mark.parametrize("k", [1, 31, 32, 33, 65, 96, 100, 130, 192, 2048])
def test_random_selections(H, dims, k):
    """Tile counts 1..7 and 64 cover every exit point of the tile loop
    (unrolled by three) and ragged last tiles."""
    DK, DV = dims
    S, T = 37, 3000
    say("attention H=%d dk=%d dv=%d k=%d" % (H, DK, DV, k))
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=100 + k + H + DK)
    rng = np.random.default_rng(k * 7 + H)
    idx = random_selection(rng, S, T, k)
    idx[0, :] = -1                      # a row with nothing selected
    if k >= 4:
        idx[1, : k // 2] = idx[1, 0]    # a row with repeated entries
    g, _ = run_and_check(q, kv, idx, DV, 1.0 / DK ** 0.5)
    assert np.all(g[0] == 0.0)


@pytest.mark.parametrize("H", [32, 64])
def test_no_entries_at_all(H):
    S, T, DK, DV = 5, 10, 576, 512
    say("attention k=0 H=%d" % H)
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=7)
    idx = torch.empty((S, 0), dtype=torch.int32)
    out = csa.sparse_attention(q.to(DEV), kv.to(DEV), idx.to(DEV), DV)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("S, T, k", [(1, 1, 1), (1, 1, 40), (3, 2, 33)])
def test_smallest_tables(H, S, T, k):
    """A one- or two-row latent table, one query row or three, with k above
    T (entries repeat): every selected entry is one of the few rows, some
    rows padded."""
    DK, DV = 576, 512
    say("attention smallest S=%d T=%d k=%d H=%d" % (S, T, k, H))
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=300 + S + T + k + H)
    idx = random_selection(np.random.default_rng(S + T + k), S, T, k, pad_frac=0.5)
    run_and_check(q, kv, idx, DV, 1.0 / DK ** 0.5)


def test_no_query_rows():
    """S = 0: an empty output and no launch."""
    q = torch.empty((0, 64, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((10, 576), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((0, 8), dtype=torch.int32, device=DEV)
    out = csa.sparse_attention(q, kv, idx, 512)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 64, 512)


def test_nonfinite_queries_stay_in_bounds():
    """NaN or Inf in some query rows gives those rows unspecified outputs
    (not detected), but the launch completes and every other row still
    matches the oracle."""
    S, T, H, DK, DV, k = 12, 700, 64, 576, 512, 90
    say("attention non-finite q")
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=55)
    q[0] = float("nan")
    q[1, 3, 5] = float("inf")
    q[2, :, 0] = float("-inf")
    idx = random_selection(np.random.default_rng(55), S, T, k)
    run_and_check(q, kv, idx, DV, 1.0 / DK ** 0.5, rows=range(3, S))


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_growing_logits_move_the_reference_max(sign):
    """Entries ordered so that the scaled logit rises (by logit for a
    positive scale, against it for a negative one) and a large scale: each
    tile's max rises by far more than the lazy-rescale threshold, so the
    accumulators are rescaled again and again; a single dominant entry at
    the end must win."""
    S, T, H, DK, DV, k = 8, 4096, 64, 576, 512, 512
    say("attention growing logits, scale sign %+g" % sign)
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=9)
    rng = np.random.default_rng(9)
    idx = np.zeros((S, k), dtype=np.int32)
    qf, kf = q.float().numpy(), kv.float().numpy()
    for i in range(S):
        sel = rng.choice(T, k, replace=False)
        score = sign * (qf[i, 0] @ kf[sel].T)   # head 0's scaled logits, up to 0.5
        idx[i] = sel[np.argsort(score)]         # ascending: maxima keep rising
    run_and_check(q, kv, torch.from_numpy(idx), DV, 0.5 * sign)


@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("dims", [(576, 512), (128, 128)])
@pytest.mark.parametrize("scale_mul", [-1.0, -0.0, 0.0])
def test_negative_and_zero_scale(H, dims, scale_mul):
    """Any finite scale is legal.  A negative one favours the smallest
    logits (the 8-wave kernel moves its sign into q, an exact flip); a zero
    one gives every selected entry the same weight, so a row's output is the
    mean of its values.  Both against the oracle, with padding, a row with
    nothing selected and ragged tiles."""
    DK, DV = dims
    S, T, k = 23, 1500, 130
    say("attention H=%d dk=%d scale x %r" % (H, DK, scale_mul))
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=41 + H + DK)
    idx = random_selection(np.random.default_rng(41 + H), S, T, k)
    idx[0, :] = -1
    scale = scale_mul * 2.0 / DK ** 0.5
    g, _ = run_and_check(q, kv, idx, DV, scale)
    assert np.all(g[0] == 0.0)


def test_indexer_selection_feeds_attention():
    """The composition the page runs: the indexer's top-k (causal padding
    with -1 included) drives the attention; checked on every row."""
    S, T, Hi, Di, m, k = 256, 64, 64, 128, 4, 40
    qi, wi, kc = inputs.bf16_gaussian(S, T, Hi, Di, seed=12)
    idx, _ = csa.topk(qi.to(DEV), wi.to(DEV), kc.to(DEV), m, k)
    torch.cuda.synchronize()
    q, kv = inputs.attention_gaussian(S, T, 64, 576, seed=13)
    run_and_check(q, kv, idx.cpu(), 512, 1.0 / 576 ** 0.5)


def test_bench_shape_sampled_rows():
    """The measured shape (64 heads, 576/512, k = 2048) at S = 8192 against
    a 65,536-entry latent table, 48 rows checked."""
    S, T, H, DK, DV, k = 8192, 65536, 64, 576, 512, 2048
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=21)
    rng = np.random.default_rng(21)
    idx = torch.from_numpy(rng.integers(0, T, (S, k)).astype(np.int32))
    rows = sorted(set([0, 1, S - 1] + rng.integers(0, S, 45).tolist()))
    run_and_check(q, kv, idx, DV, 1.0 / DK ** 0.5, rows=rows)


def test_full_composed_shape_sampled_rows():
    """The page's composed shape for the attention (S = 262,144 query rows,
    65,536 latent entries, 64 heads, 576/512, k = 2048), in the launch the
    bench times: one call over every row.  Selections are uniform over the
    table, with every 97th row padded after 1,500 entries; 24 rows (the
    first, the last, padded ones and seeded draws) against the oracle.  q
    (19 GB) and the output (17 GB) are generated and kept on the GPU."""
    S, T, H, DK, DV, k = 262144, 65536, 64, 576, 512, 2048
    say("attention full composed shape S=%d T=%d" % (S, T))
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    q = torch.empty((S, H, DK), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, S, 16384):  # fp32 draws in slices, so the temporary stays small
        q[r0:r0 + 16384] = torch.randn((16384, H, DK), generator=g, device=DEV).bfloat16()
    kv = torch.randn((T, DK), generator=g, device=DEV).bfloat16()
    idx = torch.randint(0, T, (S, k), generator=g, device=DEV, dtype=torch.int32)
    idx[::97, 1500:] = -1
    out = csa.sparse_attention(q, kv, idx, DV)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    rows = sorted(set([0, 97, 970, S - 1] + rng.integers(0, S, 20).tolist()))
    sel = torch.tensor(rows, device=DEV)
    g_rows = out[sel].float().cpu().numpy()
    ref, mag = att.sparse_attention_with_magnitude(q[sel].float().cpu().numpy(), kv.float().cpu().numpy(),
                                                   idx[sel].cpu().numpy(), DV, 1.0 / DK ** 0.5)
    del q, out
    torch.cuda.empty_cache()
    err = np.abs(g_rows - ref)
    bound = 2.0 ** -8 * (np.abs(ref) + mag) + 1e-6
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "first failures (sample, head, dim): %s" % bad[:5].tolist()


def test_repeat_runs_bit_identical():
    S, T, H, DK, DV, k = 64, 2000, 64, 576, 512, 300
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=31)
    idx = random_selection(np.random.default_rng(31), S, T, k).to(DEV)
    q, kv = q.to(DEV), kv.to(DEV)
    a = csa.sparse_attention(q, kv, idx, DV)
    b = csa.sparse_attention(q, kv, idx, DV)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_out_of_range_indices_count_as_padding():
    """Indices outside [0, T) (other than -1) are treated like -1: the
    output equals, bit for bit, that of the same selection with those
    entries set to -1, which in turn matches the oracle."""
    S, T, H, DK, DV, k = 9, 500, 64, 576, 512, 70
    say("attention out-of-range indices")
    q, kv = inputs.attention_gaussian(S, T, H, DK, seed=31)
    rng = np.random.default_rng(31)
    idx = rng.integers(0, T, (S, k)).astype(np.int32)
    bad = rng.random((S, k)) < 0.2
    junk = rng.choice(np.array([-7, -2**31, T, T + 1, 2**31 - 1], dtype=np.int64), size=(S, k))
    idx_bad = np.where(bad, junk, idx).astype(np.int32)
    idx_pad = np.where(bad, -1, idx).astype(np.int32)
    o_bad = csa.sparse_attention(q.to(DEV), kv.to(DEV), torch.from_numpy(idx_bad).to(DEV), DV)
    o_pad = csa.sparse_attention(q.to(DEV), kv.to(DEV), torch.from_numpy(idx_pad).to(DEV), DV)
    torch.cuda.synchronize()
    assert torch.equal(o_bad.cpu(), o_pad.cpu())
    run_and_check(q, kv, torch.from_numpy(idx_pad), DV, 1.0 / DK ** 0.5)


def test_composed_step_hip_graph_replays_match_eager():
    """Both calls enqueue only kernel launches on the caller's stream (no
    allocation, no memset), so the composed step, indexer then attention,
    can be captured in one HIP graph.  Every replay, with eager work in
    between and the outputs and workspace scribbled over first, equals the
    eager result bit for bit."""
    S, T, Hi, Di, m, k = 512, 256, 64, 128, 4, 96
    H, DK, DV = 64, 576, 512
    say("attention composed step in a HIP graph")
    qi, wi, kc = [t.to(DEV) for t in inputs.bf16_gaussian(S, T, Hi, Di, seed=41)]
    q, kv = [t.to(DEV) for t in inputs.attention_gaussian(S, T, H, DK, seed=42)]
    ws = torch.empty((max(csa.workspace_size(S, T, Hi, Di, m, k), 1),), dtype=torch.uint8, device=DEV)
    idx = torch.empty((S, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((S, k), dtype=torch.float32, device=DEV)
    out = torch.empty((S, H, DV), dtype=torch.bfloat16, device=DEV)
    e_idx, _ = csa.topk(qi, wi, kc, m, k)
    e_out = csa.sparse_attention(q, kv, e_idx, DV)
    torch.cuda.synchronize()

    def step():
        csa.topk(qi, wi, kc, m, k, workspace=ws, out=(idx, sc))
        csa.sparse_attention(q, kv, idx, DV, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        idx.fill_(-1)
        out.fill_(7.0)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, e_idx), "replay %d" % rep
        assert torch.equal(out.view(torch.int16), e_out.view(torch.int16)), "replay %d" % rep
        _ = (q.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
