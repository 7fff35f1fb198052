"""Brute-force checker for tiny inputs, independent of the oracle.

Scores are exact rationals (``fractions.Fraction``) of the given float
inputs, so there is no rounding at all.  The usable keys of a row are counted
one by one from the causal rule ((j+1)*m <= i+1) rather than by a formula, and
selection is by rank counting rather than by sorting:

    rank(j) = #{j' usable : s(j') > s(j)} + #{j' < j usable : s(j') == s(j)}

Key j is returned at output position rank(j) when rank(j) < k.  This is the
definition of "top-k ordered by score descending, then index ascending" with
no algorithm in between.  Only for a handful of rows and keys.
"""
from __future__ import annotations

from fractions import Fraction


def exact_scores(q_row, w_row, kc, n):
    """Exact score of keys 0..n-1 for one row: sum_h w_h * max(q_h . kc_j, 0)."""
    out = []
    for j in range(n):
        total = Fraction(0)
        for h in range(len(q_row)):
            dot = Fraction(0)
            for d in range(len(q_row[h])):
                dot += Fraction(float(q_row[h][d])) * Fraction(float(kc[j][d]))
            if dot > 0:
                total += Fraction(float(w_row[h])) * dot
        out.append(total)
    return out


def usable(pos, T, m):
    return sum(1 for j in range(T) if (j + 1) * m <= pos + 1)


def brute_topk(q, w, kc, m, k, pos):
    """Returns (idx rows, exact score rows) as Python lists; padding -1 / None."""
    T = len(kc)
    idx_rows, score_rows = [], []
    for r, p in enumerate(pos):
        n = usable(int(p), T, m)
        s = exact_scores(q[r], w[r], kc, n)
        idx = [-1] * k
        sc = [None] * k
        for j in range(n):
            rank = sum(1 for jj in range(n) if s[jj] > s[j]) + \
                sum(1 for jj in range(j) if s[jj] == s[j])
            if rank < k:
                idx[rank] = j
                sc[rank] = s[j]
        idx_rows.append(idx)
        score_rows.append(sc)
    return idx_rows, score_rows
