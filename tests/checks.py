"""Comparison of GPU outputs with the CPU oracle.

Integer-valued inputs have exactly one correct output (every score is an
exact integer in fp32 under any summation order), so those are compared bit
for bit.  Float inputs are compared by the tolerance rules of the indexer
top-k:

* score agreement: for every returned key j,
  |s_gpu(j) - s_orc(j)| <= rel * max(|s_orc(j)|, |s_kth|), where s_kth is the
  oracle's score at rank min(k, n) of the row (a plain relative test would
  reject correct results where cancellation leaves a score near zero); the
  stats count the keys that pass only through the |s_kth| floor;
* threshold: every returned key has s_orc(j) >= s_kth - rel * |s_kth|;
* set recall: |gpu set & oracle set| / min(k, n) >= min_recall, the minimum
  over the checked rows;
* structure: the valid entries come first, are distinct usable keys, sorted by
  the returned score descending then index ascending, padding -1 / -inf, and
  no score is -0.
"""
from __future__ import annotations

import numpy as np

import oracle


def as_np(t):
    if hasattr(t, "detach"):
        t = t.detach()
        if t.dtype.is_floating_point and t.dtype != __import__("torch").float32:
            t = t.float()
        return t.cpu().numpy()
    return np.asarray(t)


def check_structure(idx, score, pos, T, m, k):
    """Invariants that hold for any correct output; returns failure strings."""
    fails = []
    n = oracle.n_valid(pos, T, m)
    cnt = np.minimum(n, k)
    cols = np.arange(k)[None, :]
    valid = cols < cnt[:, None]
    if np.any(idx[~valid] != -1) or np.any(~np.isneginf(score[~valid])):
        fails.append("padding is not idx -1 / score -inf after the valid entries")
    if np.any((idx < 0) & valid) or np.any((idx >= n[:, None]) & valid):
        fails.append("returned key outside [0, n)")
    if np.any(~np.isfinite(score[valid])):
        fails.append("non-finite score in a valid slot")
    if np.any((score == 0) & np.signbit(score)):
        fails.append("-0 in the output")
    # sorted: s[t] > s[t+1] or (== and idx[t] < idx[t+1]) among valid pairs
    both = valid[:, :-1] & valid[:, 1:]
    s0, s1 = score[:, :-1], score[:, 1:]
    i0, i1 = idx[:, :-1], idx[:, 1:]
    ok = (s0 > s1) | ((s0 == s1) & (i0 < i1))
    if np.any(both & ~ok):
        r = int(np.argwhere(both & ~ok)[0][0])
        fails.append("row %d not sorted by (score desc, idx asc)" % r)
    for r in range(idx.shape[0]):
        c = int(cnt[r])
        if c and len(np.unique(idx[r, :c])) != c:
            fails.append("row %d has duplicate keys" % r)
            break
    return fails


def check_exact(g_idx, g_score, o_idx, o_score):
    fails = []
    if not np.array_equal(g_idx, o_idx):
        bad = np.argwhere(g_idx != o_idx)
        r, c = bad[0]
        fails.append("idx differs at %d places, first row %d col %d: gpu %d oracle %d"
                     % (len(bad), r, c, g_idx[r, c], o_idx[r, c]))
    if not np.array_equal(g_score.view(np.uint32), o_score.view(np.uint32)):
        bad = np.argwhere(g_score.view(np.uint32) != o_score.view(np.uint32))
        r, c = bad[0]
        fails.append("score bits differ at %d places, first row %d col %d: gpu %r oracle %r"
                     % (len(bad), r, c, g_score[r, c], o_score[r, c]))
    return fails


def check_float(g_idx, g_score, o_idx, o_score, q_rows, w_rows, kc, pos, T, m, k,
                rel=2e-3, min_recall=0.998):
    """Tolerance comparison of sampled rows.  q_rows/w_rows are the fp32
    (exactly upcast) inputs of the checked rows; kc all keys.  Returns
    (failures, stats)."""
    fails = check_structure(g_idx, g_score, pos, T, m, k)
    n = oracle.n_valid(pos, T, m)
    recalls = []
    relaxed = 0
    max_err = 0.0
    worst_thr = 0.0
    for r in range(g_idx.shape[0]):
        c = int(min(n[r], k))
        if c == 0:
            recalls.append(1.0)
            continue
        gi = g_idx[r, :c]
        oi = o_idx[r, :c]
        s_kth = float(o_score[r, c - 1])
        scale_kth = abs(s_kth)
        o_map = dict(zip(oi.tolist(), o_score[r, :c].tolist()))
        missing = [int(j) for j in gi if int(j) not in o_map]
        if missing:
            extra = oracle.row_scores(q_rows[r], w_rows[r], kc[np.array(missing)], len(missing))
            o_map.update(zip(missing, extra.tolist()))
        s_orc = np.array([o_map[int(j)] for j in gi], dtype=np.float64)
        s_gpu = g_score[r, :c].astype(np.float64)
        tol = rel * np.maximum(np.abs(s_orc), scale_kth)
        err = np.abs(s_gpu - s_orc)
        # Keys that pass only through the k-th-score floor of the bound (a
        # plain relative test would reject them): cancellation near zero.
        relaxed += int(np.count_nonzero((err > rel * np.abs(s_orc)) & (err <= tol)))
        if np.any(err > tol):
            t = int(np.argmax(err - tol))
            fails.append("row %d key %d: gpu score %r vs oracle %r beyond %g relative"
                         % (r, gi[t], s_gpu[t], s_orc[t], rel))
        denom = np.maximum(np.abs(s_orc), max(scale_kth, 1e-30))
        max_err = max(max_err, float(np.max(err / denom)))
        low = s_orc < s_kth - rel * scale_kth
        if np.any(low):
            t = int(np.argmax(low))
            fails.append("row %d key %d: oracle score %r below the k-th %r minus tolerance"
                         % (r, gi[t], s_orc[t], s_kth))
        if scale_kth > 0:
            worst_thr = max(worst_thr, float(np.max((s_kth - s_orc) / scale_kth)))
        recalls.append(len(np.intersect1d(gi, oi, assume_unique=True)) / c)
    recalls = np.array(recalls) if recalls else np.ones(1)
    if recalls.min() < min_recall:
        r = int(np.argmin(recalls))
        fails.append("row %d recall %.5f below %.4f" % (r, recalls[r], min_recall))
    stats = {"recall_min": float(recalls.min()), "recall_mean": float(recalls.mean()),
             "max_rel_score_err": max_err, "worst_below_kth": worst_thr,
             "keys_within_kth_floor_only": relaxed, "rows": int(g_idx.shape[0])}
    return fails, stats
