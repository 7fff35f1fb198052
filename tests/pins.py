"""Pins of the CPU oracle: checks that tie it to something other than itself.

Each ``run_*`` function runs one kind of pin against an oracle library handle
(``None`` = the built oracle) and returns a list of failure messages, so the
same pins can be run against deliberately broken copies of the oracle to show
that they would catch such mistakes.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

import brute
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.txt")

U32 = Fraction(1, 1 << 24)  # unit roundoff of fp32, round to nearest


def gamma(n: int) -> Fraction:
    return n * U32 / (1 - n * U32)


def _num(tok: str) -> float:
    if tok == "-inf":
        return -math.inf
    if tok == "inf":
        return math.inf
    return float(tok)


def parse_golden(path: str = GOLDEN):
    """Sections of the worked-example file as dicts."""
    sections = []
    cur = None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = {"name": line[1:-1], "expect": [], "sign": []}
                sections.append(cur)
                continue
            if line.startswith("expect "):
                head, rest = line[len("expect "):].split(":", 1)
                idx_s, sc_s = rest.split("|")
                cur["expect"].append((int(head), [int(t) for t in idx_s.split()],
                                      [_num(t) for t in sc_s.split()]))
                continue
            if line.startswith("sign "):
                _, row, col, sgn = line.split()
                cur["sign"].append((int(row), int(col), sgn))
                continue
            key, val = [t.strip() for t in line.split("=", 1)]
            if key in ("kc", "q"):
                cur[key] = [[float(t) for t in part.split()] for part in val.split(";")]
            elif key == "w":
                cur[key] = [float(t) for t in val.split()]
            else:
                cur[key] = int(val)
    return sections


def run_golden(lib=None):
    fails = []
    for ex in parse_golden():
        rows, m, k = ex["rows"], ex["m"], ex["k"]
        kc = np.array(ex["kc"], dtype=np.float32)
        qh = np.array(ex["q"], dtype=np.float32)  # [H, D]
        q = np.broadcast_to(qh, (rows, *qh.shape)).copy()
        w = np.broadcast_to(np.array(ex["w"], dtype=np.float32), (rows, qh.shape[0])).copy()
        try:
            idx, score = oracle.topk(q, w, kc, m, k, nthreads=2, lib=lib)
        except Exception as e:  # a broken oracle may fail outright
            fails.append("%s: oracle raised %r" % (ex["name"], e))
            continue
        for row, e_idx, e_sc in ex["expect"]:
            if list(idx[row]) != e_idx:
                fails.append("%s row %d: idx %s != %s" % (ex["name"], row, list(idx[row]), e_idx))
            got = [float(x) for x in score[row]]
            if got != e_sc:
                fails.append("%s row %d: score %s != %s" % (ex["name"], row, got, e_sc))
        for row, col, sgn in ex["sign"]:
            neg = math.copysign(1.0, float(score[row, col])) < 0
            if neg != (sgn == "-"):
                fails.append("%s row %d col %d: sign bit wrong" % (ex["name"], row, col))
    return fails


def _tiny_case(rng, integer: bool):
    S = int(rng.integers(1, 30))
    m = int(rng.integers(1, 6))
    T = int(rng.integers(0, 12))
    H = int(rng.integers(1, 5))
    D = int(rng.integers(1, 6))
    k = int(rng.integers(1, 14))
    q_pos0 = int(rng.choice([0, 0, int(rng.integers(0, 40))]))
    if integer:
        q = rng.integers(-3, 4, size=(S, H, D)).astype(np.float32)
        kc = rng.integers(-3, 4, size=(T, D)).astype(np.float32)
        w = rng.choice(np.array([-2, -1, 1, 2], dtype=np.float32), size=(S, H))
    else:
        q = rng.standard_normal((S, H, D)).astype(np.float32)
        kc = rng.standard_normal((T, D)).astype(np.float32)
        w = rng.standard_normal((S, H)).astype(np.float32)
    pos = np.arange(S, dtype=np.int64) + q_pos0
    return q, w, kc, m, k, pos


def run_brute_integer(lib=None, cases: int = 60, seed: int = 1234):
    """Integer-valued tiny cases: every score is an exact integer in fp32, so
    the oracle must match the exact brute force bit for bit."""
    fails = []
    rng = np.random.default_rng(seed)
    for c in range(cases):
        q, w, kc, m, k, pos = _tiny_case(rng, integer=True)
        try:
            idx, score = oracle.topk(q, w, kc, m, k, pos=pos, nthreads=3, lib=lib)
        except Exception as e:
            fails.append("case %d: oracle raised %r" % (c, e))
            continue
        b_idx, b_sc = brute.brute_topk(q, w, kc, m, k, pos)
        for r in range(len(pos)):
            if list(idx[r]) != b_idx[r]:
                fails.append("case %d row %d: idx %s != brute %s" % (c, r, list(idx[r]), b_idx[r]))
                break
            want = [float(s) if s is not None else -math.inf for s in b_sc[r]]
            if [float(x) for x in score[r]] != want:
                fails.append("case %d row %d: score %s != brute %s" % (c, r, list(score[r]), want))
                break
            if any(float(x) == 0.0 and math.copysign(1.0, float(x)) < 0 for x in score[r]):
                fails.append("case %d row %d: -0 in output" % (c, r))
                break
    return fails


def score_bound(q_row, w_row, key) -> tuple[Fraction, Fraction]:
    """(exact score, error bound of an fp32 evaluation in the oracle's order).

    The inner dot of length D has error at most gamma_D * sum_d |q k|
    (recursive summation, Higham, Accuracy and Stability of Numerical
    Algorithms, ch. 3); the ReLU does not enlarge it; the outer weighted sum
    of H terms adds gamma_H * sum_h |w_h| * |relu_h| with relu_h within that
    inner error of its exact value."""
    H, D = len(q_row), len(key)
    g_d, g_h = gamma(D), gamma(H)
    exact = Fraction(0)
    bound = Fraction(0)
    for h in range(H):
        dot = Fraction(0)
        absdot = Fraction(0)
        for d in range(D):
            p = Fraction(float(q_row[h][d])) * Fraction(float(key[d]))
            dot += p
            absdot += abs(p)
        r = dot if dot > 0 else Fraction(0)
        wh = Fraction(float(w_row[h]))
        e_h = g_d * absdot
        exact += wh * r
        bound += g_h * abs(wh) * (r + e_h) + abs(wh) * e_h
    return exact, bound


def run_brute_float(lib=None, cases: int = 40, seed: int = 99):
    """Gaussian tiny cases: oracle scores within the fp32 error bound of the
    exact value; the order may differ from the exact order only between keys
    whose exact scores lie within their combined bounds."""
    fails = []
    rng = np.random.default_rng(seed)
    for c in range(cases):
        q, w, kc, m, k, pos = _tiny_case(rng, integer=False)
        try:
            idx, score = oracle.topk(q, w, kc, m, k, pos=pos, nthreads=2, lib=lib)
        except Exception as e:
            fails.append("case %d: oracle raised %r" % (c, e))
            continue
        T = len(kc)
        for r in range(len(pos)):
            n = brute.usable(int(pos[r]), T, m)
            ex = [score_bound(q[r], w[r], kc[j]) for j in range(n)]
            b_idx, _ = brute.brute_topk(q[r:r + 1], w[r:r + 1], kc, m, k, pos[r:r + 1])
            b_idx = b_idx[0]
            cnt = min(k, n)
            got = list(idx[r])
            if got[cnt:] != [-1] * (k - cnt) or any(x != -math.inf for x in score[r, cnt:]):
                fails.append("case %d row %d: padding wrong" % (c, r))
                break
            if sorted(got[:cnt]) != sorted(set(got[:cnt])) or any(not (0 <= j < n) for j in got[:cnt]):
                fails.append("case %d row %d: invalid indices %s" % (c, r, got))
                break
            bad = False
            for t in range(cnt):
                j = got[t]
                s_ex, bnd = ex[j]
                if abs(Fraction(float(score[r, t])) - s_ex) > bnd:
                    fails.append("case %d row %d key %d: score outside fp32 bound" % (c, r, j))
                    bad = True
                    break
                jb = b_idx[t]
                if jb != j:
                    s_b, bnd_b = ex[jb]
                    if abs(s_ex - s_b) > bnd + bnd_b:
                        fails.append("case %d row %d pos %d: key %d where exact order has %d"
                                     % (c, r, t, j, jb))
                        bad = True
                        break
            if bad:
                break
    return fails


def run_error_bound_wide(lib=None, seed: int = 5, keys: int = 12):
    """fp32 row scores at the full head count and head width (H=64, D=128)
    stay within the recursive-summation bound of the exact value."""
    fails = []
    rng = np.random.default_rng(seed)
    H, D = 64, 128
    q = (rng.standard_normal((H, D)) / math.sqrt(D)).astype(np.float32)
    w = (rng.standard_normal(H) / math.sqrt(H)).astype(np.float32)
    kc = (rng.standard_normal((keys, D)) / math.sqrt(D)).astype(np.float32)
    try:
        got = oracle.row_scores(q, w, kc, keys, lib=lib)
    except Exception as e:
        return ["oracle raised %r" % (e,)]
    for j in range(keys):
        s_ex, bnd = score_bound(q, w, kc[j])
        if abs(Fraction(float(got[j])) - s_ex) > bnd:
            fails.append("key %d: |%r - exact| above bound %g" % (j, float(got[j]), float(bnd)))
    return fails


def run_single_head_lexsort(lib=None, seed: int = 3):
    """H=1 and w=1 with integer inputs: the score is the ReLU of an exact
    integer dot product (numpy int64 matmul) and the selection is numpy's
    lexsort on (-score, index)."""
    fails = []
    rng = np.random.default_rng(seed)
    S, T, D, m, k = 96, 20, 7, 4, 6
    qi = rng.integers(-3, 4, size=(S, 1, D))
    ki = rng.integers(-3, 4, size=(T, D))
    w = np.ones((S, 1), dtype=np.float32)
    try:
        idx, score = oracle.topk(qi.astype(np.float32), w, ki.astype(np.float32), m, k,
                                 nthreads=2, lib=lib)
    except Exception as e:
        return ["oracle raised %r" % (e,)]
    dots = qi[:, 0, :].astype(np.int64) @ ki.T.astype(np.int64)
    s = np.maximum(dots, 0)
    for i in range(S):
        n = min(T, (i + 1) // m)
        j = np.arange(n)
        order = np.lexsort((j, -s[i, :n]))[:k]
        want_idx = list(order) + [-1] * (k - len(order))
        if list(idx[i]) != want_idx:
            fails.append("row %d: %s != lexsort %s" % (i, list(idx[i]), want_idx))
            break
        want_sc = [float(s[i, t]) for t in order] + [-math.inf] * (k - len(order))
        if [float(x) for x in score[i]] != want_sc:
            fails.append("row %d: scores differ" % i)
            break
    return fails


ALL_PINS = {
    "golden": run_golden,
    "brute_integer": run_brute_integer,
    "brute_float": run_brute_float,
    "error_bound_wide": run_error_bound_wide,
    "single_head_lexsort": run_single_head_lexsort,
}


def torch_seeded_integer(S, T, H, D, seed):
    """Convenience: integer inputs from the shared generator as numpy."""
    from streaming_indexer_top_amd import inputs
    q, w, kc = inputs.integer_valued(S, T, H, D, seed, dtype=torch.float32, signed_w=True)
    return q.numpy(), w.numpy(), kc.numpy()
