"""CPU tests of the C ABI: the library loads, exports every symbol its header
declares, and rejects bad arguments before touching the GPU.  No call here
reaches a kernel launch."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import streaming_indexer_top_amd as csa
from streaming_indexer_top_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa_indexer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(csa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = csa.load_library()
    assert lib.csa_abi_version() == 4
    for st in range(0, 11):
        assert lib.csa_status_str(st)


def _ws(S, T, H=64, D=128, m=4, k=2048, **kw):
    return csa.workspace_size(S, T, H, D, m, k, **kw)


def test_workspace_bounded_independent_of_sequence_length():
    # The score tensor [S, H, T] at S = 2^20 would be 64 TiB; the workspace
    # stays within the default 2 GiB budget at every size.
    for S in (1 << 14, 1 << 16, 1 << 18, 1 << 20):
        b = _ws(S, S // 4)
        assert 0 < b <= (2 << 30)
    assert _ws(1 << 20, 1 << 18, workspace_budget=256 << 20) <= 256 << 20


def test_workspace_zero_without_usable_keys():
    assert _ws(3, 100, m=4) == 0           # rows 0..2 see no key
    assert _ws(100, 0) == 0                 # no keys
    assert _ws(0, 100) == 0                 # no rows


def test_workspace_single_chunk_when_small():
    # 1024 rows, last row sees 256 keys: one chunk of 256 keys, no lists.
    assert _ws(1024, 256, H=4, D=32, k=16) == 1024 * 256 * 4 + 1024 * 16


def test_key_splits_for_few_rows():
    # 64 decode rows against 262144 keys: one chunk of all keys cut into
    # splits, each with its own list -> scores + 64 splits x 64 rows x (16 B
    # summary + k*8 B list + 16 B state), within the default budget.
    b = _ws(64, 1 << 18, q_pos0=(1 << 20) - 64)
    per_split_row = 16 + 2048 * 8 + 16
    assert b >= 64 * (1 << 18) * 4 + 64 * 64 * per_split_row
    # Splits off: one 65536-key chunk at a time with one running list per row.
    b1 = _ws(64, 1 << 18, q_pos0=(1 << 20) - 64, key_splits=1)
    assert b1 == 64 * 65536 * 4 + 1024 + 64 * 2048 * 8 + 1024
    # Many rows: no splits (same as key_splits=1).
    assert _ws(1 << 14, 1 << 12) == _ws(1 << 14, 1 << 12, key_splits=1)
    # fp32 plans exactly as bf16 (its kernel writes the same chunk summaries).
    assert _ws(64, 1 << 18, q_pos0=(1 << 20) - 64, dtype=torch.float32) == b
    assert _ws(64, 1 << 18, q_pos0=(1 << 20) - 64, dtype=torch.float32, key_splits=1) == b1


def test_workspace_tiny_budget_still_fits_one_block():
    b = _ws(1 << 16, 1 << 14, workspace_budget=1)
    assert b > 0
    assert b <= 8 * (1 << 14) * 4 + 8 * 2048 * 8 + 1024


def _call(lib, q=1, w=1, kc=1, dtype=1, S=8, T=8, H=4, D=32, m=4, k=2, q_pos0=0,
          idx=1, score=1, ws=None, ws_bytes=0, opts=None):
    P = ctypes.c_void_p
    al = 4096  # a fake, suitably aligned address: every call here fails a check first
    conv = lambda v: P(al * v if isinstance(v, int) and v in (0, 1) else v)
    return lib.csa_indexer_topk(conv(q), conv(w), conv(kc), dtype, S, T, H, D, m, k, q_pos0,
                                conv(idx), conv(score), P(ws), ws_bytes,
                                ctypes.byref(opts) if opts is not None else None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 3),
    (dict(S=-1), 2),
    (dict(T=-1), 2),
    (dict(H=0), 2),
    (dict(H=65), 2),
    (dict(D=48), 2),
    (dict(m=0), 2),
    (dict(k=0), 2),
    (dict(q_pos0=-3), 2),
    (dict(k=4097), 6),
    (dict(q=0), 1),
    (dict(w=0), 1),
    (dict(idx=0), 1),
    (dict(score=0), 1),
    (dict(kc=0), 1),
    (dict(q=4096 + 8), 4),
    (dict(kc=4096 + 4), 4),
    (dict(score=4096 + 2), 4),
    (dict(ws=None, ws_bytes=0), 1),  # keys exist, so a workspace is required
])
def test_argument_checks_fail_before_any_device_work(kw, status):
    lib = csa.load_library()
    assert _call(lib, **kw) == status


def _call_batched(lib, B=2, q=1, ws=None, ws_bytes=0, S=8, T=8, k=2):
    P = ctypes.c_void_p
    al = 4096
    conv = lambda v: P(al * v if isinstance(v, int) and v in (0, 1) else v)
    return lib.csa_indexer_topk_batched(conv(q), conv(1), conv(1), 1, B, S, T, 4, 32, 4, k, 0,
                                        conv(1), conv(1), P(ws), ws_bytes, None, None)


def test_batched_argument_checks():
    lib = csa.load_library()
    assert _call_batched(lib, B=-1) == 2
    assert _call_batched(lib, B=3, q=0) == 1
    assert _call_batched(lib, B=3, k=5000) == 6
    assert _call_batched(lib, B=3) == 1  # keys exist, so a workspace is required
    assert _call_batched(lib, B=0, S=0) == 0  # no problem: nothing to do


def test_workspace_too_small():
    lib = csa.load_library()
    assert _call(lib, ws=4096 * 16, ws_bytes=64, S=4096, T=1024) == 5


def test_bad_options():
    lib = csa.load_library()
    for field, val in (("chunk_keys", 100), ("chunk_keys", (1 << 24) + 256), ("key_tile", 96),
                       ("workspace_budget", -1),
                       ("key_splits", 3), ("key_splits", 256), ("key_splits", -2)):
        o = binding.csa_opts()
        setattr(o, field, val)
        assert _call(lib, opts=o) == 8, field
    o = binding.csa_opts()
    o.reserved[2] = 1
    assert _call(lib, opts=o) == 8


def test_python_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros((4, 2, 32), dtype=torch.bfloat16)
    w = torch.zeros((4, 2), dtype=torch.bfloat16)
    kc = torch.zeros((3, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # CPU tensors: no silent CPU path
        csa.topk(q, w, kc, 4, 2)
    with pytest.raises(TypeError):
        csa.topk(q, w.float(), kc, 4, 2)
    with pytest.raises(ValueError):
        csa.topk(q, w[:3], kc, 4, 2)


def test_caller_buffers_must_be_contiguous_and_on_the_inputs_device():
    # Outputs and workspace that the caller passes in reach the library only
    # as an address and a size, so the binding checks where they live.
    cpu = torch.device("cpu")
    binding._caller_buffer(torch.zeros(4), cpu, "out")
    with pytest.raises(ValueError, match="must be on"):
        binding._caller_buffer(torch.zeros(4), torch.device("cuda", 0), "out")
    with pytest.raises(ValueError, match="contiguous"):
        binding._caller_buffer(torch.zeros(4, 4).t(), cpu, "out")
    # A stride-0 view reports far more bytes than it holds.
    with pytest.raises(ValueError, match="contiguous"):
        binding._caller_buffer(torch.zeros(1, dtype=torch.uint8).expand(1 << 20), cpu, "workspace")


@pytest.mark.parametrize("args, status", [
    # (S, T, H, D_K, D_V, k, dtype, scale)
    ((-1, 10, 64, 576, 512, 8, binding.CSA_BF16, 0.1), 2),
    ((4, 10, 64, 576, 512, -1, binding.CSA_BF16, 0.1), 2),
    ((4, 10, 0, 576, 512, 8, binding.CSA_BF16, 0.1), 2),
    ((4, 10, 64, 576, 512, 8, binding.CSA_BF16, float("nan")), 2),
    ((4, 10, 64, 576, 512, 8, binding.CSA_BF16, float("inf")), 2),
    ((4, 10, 64, 576, 512, 8, binding.CSA_BF16, 3.0e38), 2),   # scale * log2(e) overflows fp32
    ((4, 10, 64, 576, 512, 8, binding.CSA_BF16, -3.0e38), 2),
    ((4, 10, 64, 576, 512, 8, 7, 0.1), 3),
    ((4, 10, 64, 576, 512, 8, binding.CSA_F32, 0.1), 6),
    ((4, 10, 48, 576, 512, 8, binding.CSA_BF16, 0.1), 6),
    ((4, 10, 64, 256, 256, 8, binding.CSA_BF16, 0.1), 6),
    ((4, 10, 64, 576, 512, (1 << 20) + 1, binding.CSA_BF16, 0.1), 6),
    ((4, 1 << 21, 64, 576, 512, 8, binding.CSA_BF16, 0.1), 6),
    ((4, 1864136, 64, 576, 512, 8, binding.CSA_BF16, 0.1), 6),   # first T with T * 576 * 2 >= 2^31
    ((4, 1 << 62, 64, 576, 512, 8, binding.CSA_BF16, 0.1), 6),   # T * D_K * 2 would overflow int64
    ((1 << 31, 10, 64, 576, 512, 8, binding.CSA_BF16, 0.1), 6),
])
def test_sparse_attention_argument_checks(args, status):
    """Bad shapes, dtypes, scales and unsupported sizes are refused before
    any HIP call (dummy pointers: nothing is dereferenced)."""
    S, T, H, DK, DV, k, dt, scale = args
    lib = csa.load_library()
    p = ctypes.c_void_p(256)
    assert lib.csa_sparse_attention(p, p, p, p, dt, S, T, H, DK, DV, k, scale, None) == status


def test_sparse_attention_null_and_alignment_checks():
    lib = csa.load_library()
    p, z = ctypes.c_void_p(256), ctypes.c_void_p(0)
    a = (binding.CSA_BF16, 4, 10, 64, 576, 512, 8, 0.1, None)
    assert lib.csa_sparse_attention(z, p, p, p, *a) == 1
    assert lib.csa_sparse_attention(p, z, p, p, *a) == 1
    assert lib.csa_sparse_attention(p, p, z, p, *a) == 1
    assert lib.csa_sparse_attention(p, p, p, z, *a) == 1
    assert lib.csa_sparse_attention(ctypes.c_void_p(264), p, p, p, *a) == 4
    assert lib.csa_sparse_attention(p, p, ctypes.c_void_p(258), p, *a) == 4
    # No rows: nothing to do, nothing touched.
    assert lib.csa_sparse_attention(z, z, z, z, binding.CSA_BF16, 0, 10, 64, 576, 512, 8,
                                    0.1, None) == 0


def test_noalloc_rejects_beyond_scratch_before_any_hip_call():
    """The allocation-free entry point checks everything before any HIP call
    (dummy device pointers: nothing is dereferenced).  One query block of 8
    rows against a caller-fixed 2^24-key chunk needs 512 MiB of scores, above
    the 256 MiB scratch: CSA_ERR_SCRATCH_TOO_SMALL.  Bad arguments give the
    same codes as csa_indexer_topk."""
    lib = csa.load_library()
    p = ctypes.c_void_p(256)
    T = 1 << 24
    big = binding._opts(chunk_keys=1 << 24)
    assert lib.csa_indexer_topk_noalloc(p, p, p, binding.CSA_BF16, 8, T, 64, 128, 1, 16, T,
                                        p, p, ctypes.byref(big), None) == 9
    assert b"256 MiB" in lib.csa_status_str(9)
    # Same shapes with a chunk that fits: no error before the HIP part, so
    # only argument errors are probed here.
    assert lib.csa_indexer_topk_noalloc(p, p, p, 7, 8, 100, 64, 128, 1, 16, 0, p, p, None,
                                        None) == 3
    assert lib.csa_indexer_topk_noalloc(p, p, p, 1, 8, 100, 64, 128, 0, 16, 0, p, p, None,
                                        None) == 2
    assert lib.csa_indexer_topk_noalloc(ctypes.c_void_p(0), p, p, 1, 8, 100, 64, 128, 1, 16, 0,
                                        p, p, None, None) == 1
    assert lib.csa_indexer_topk_noalloc(p, p, p, 1, 8, 100, 64, 128, 1, 5000, 0, p, p, None,
                                        None) == 6
    neg = binding._opts(workspace_budget=-1)
    assert lib.csa_indexer_topk_noalloc(p, p, p, 1, 8, 100, 64, 128, 1, 16, 0, p, p,
                                        ctypes.byref(neg), None) == 8
    # No rows: nothing to do, no scratch needed, nothing touched.
    z = ctypes.c_void_p(0)
    assert lib.csa_indexer_topk_noalloc(z, z, z, 1, 0, 100, 64, 128, 1, 16, 0, z, z, None,
                                        None) == 0
