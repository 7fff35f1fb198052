"""GPU test of the allocation-free entry point (csa_indexer_topk_noalloc):
through the C ABI, its outputs equal csa_indexer_topk's bit for bit on the
same inputs, for two calls in a row on one stream, the second smaller than
the first (the scratch keeps the first call's contents, which the second
must not depend on), and for plans that need many passes of the fixed
scratch and that use key splits."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import streaming_indexer_top_amd as csa
from streaming_indexer_top_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same(a, b):
    return torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def _case(kind, S, T, m, k, seed, q_pos0=0):
    if kind == "integer":
        q, w, kc = inputs.integer_valued(S, T, 64, 128, seed=seed, dtype=torch.bfloat16,
                                         signed_w=True, device=DEV)
    else:
        q, w, kc = inputs.bf16_gaussian(S, T, 64, 128, seed=seed, device=DEV)
    return q, w, kc, m, k, q_pos0


def test_noalloc_matches_workspace_call_twice_in_a_row():
    # First the bench shape (65,536 rows: 3 passes with the default 2 GiB
    # workspace, 32 passes of the 256 MiB scratch), then a smaller problem.
    cases = [("gaussian", 65536, 16384, 4, 2048, 3, 0),
             ("integer", 3000, 2500, 4, 512, 11, 0)]
    for kind, S, T, m, k, seed, q0 in cases:
        q, w, kc, m, k, q0 = _case(kind, S, T, m, k, seed, q0)
        say("noalloc %s S=%d T=%d k=%d" % (kind, S, T, k))
        ref = csa.topk(q, w, kc, m, k, q_pos0=q0)
        idx = torch.full((S, k), 7, dtype=torch.int32, device=DEV)
        sc = torch.zeros((S, k), dtype=torch.float32, device=DEV)
        got = csa.topk_noalloc(q, w, kc, m, k, q_pos0=q0, out=(idx, sc))
        torch.cuda.synchronize()
        assert got[0] is idx and got[1] is sc
        assert _same(ref, got), "%s S=%d differs from the workspace call" % (kind, S)
        del q, w, kc, ref, got, idx, sc
        torch.cuda.empty_cache()


def test_noalloc_key_splits_and_chunks():
    # Decode shape (automatic key splits inside the scratch), then a long
    # chunked row set with a caller-fixed chunk size, each against the
    # workspace call.
    for S, T, m, k, q0, kw in ((16, 200000, 1, 2048, 199984, {}),
                               (512, 70000, 1, 1000, 69488, dict(chunk_keys=8192))):
        q, w, kc, m, k, q0 = _case("gaussian", S, T, m, k, 21, q0)
        say("noalloc decode/chunks S=%d T=%d %s" % (S, T, kw))
        ref = csa.topk(q, w, kc, m, k, q_pos0=q0, **kw)
        got = csa.topk_noalloc(q, w, kc, m, k, q_pos0=q0, **kw)
        torch.cuda.synchronize()
        assert _same(ref, got)


def test_noalloc_fp32_inputs():
    # fp32 inputs (the fp32 score kernel), a decode shape with automatic key
    # splits and then a multi-chunk row set, each against the workspace call.
    for S, T, m, k, q0, kw in ((16, 60000, 1, 2048, 59984, {}),
                               (300, 9000, 1, 700, 8700, dict(chunk_keys=2048))):
        q, w, kc = inputs.gaussian_fp32(S, T, 64, 128, seed=31, device=DEV)
        say("noalloc fp32 S=%d T=%d %s" % (S, T, kw))
        ref = csa.topk(q, w, kc, m, k, q_pos0=q0, **kw)
        got = csa.topk_noalloc(q, w, kc, m, k, q_pos0=q0, **kw)
        torch.cuda.synchronize()
        assert _same(ref, got)

