"""Python binding of libcsa_indexer.so (argument marshalling only).

Every step of the indexer runs in the library's HIP kernels; this module
only checks tensor metadata, allocates outputs and workspace with PyTorch on
the inputs' device, and passes raw pointers and torch's current HIP stream
through ctypes.  If the library is missing or fails to load, every call
raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcsa_indexer.so")

CSA_F32 = 0
CSA_BF16 = 1
CSA_KERNEL_SCORE = 0
CSA_KERNEL_SELECT = 1
CSA_KERNEL_MERGE = 2
CSA_KERNEL_ATTENTION = 3
CSA_KERNEL_KINDS = 4
KERNEL_NAMES = ("score", "select", "merge", "attention")

EXPORTS = ("csa_abi_version", "csa_status_str", "csa_indexer_topk_workspace_size",
           "csa_indexer_topk", "csa_indexer_topk_batched", "csa_profile_enable",
           "csa_profile_collect", "csa_sparse_attention", "csa_indexer_topk_noalloc")


class CsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("csa_indexer status %d: %s" % (status, msg))
        self.status = status


class csa_opts(ctypes.Structure):
    _fields_ = [("chunk_keys", ctypes.c_int64),
                ("key_tile", ctypes.c_int32),
                ("key_splits", ctypes.c_int32),
                ("workspace_budget", ctypes.c_int64),
                ("reserved", ctypes.c_int64 * 4)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load (once) and declare the C ABI."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libcsa_indexer.so not built at %s: run "
                           "python -m streaming_indexer_top_amd.build" % p)
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.csa_abi_version.argtypes = []
    lib.csa_abi_version.restype = ctypes.c_int
    lib.csa_status_str.argtypes = [ctypes.c_int]
    lib.csa_status_str.restype = ctypes.c_char_p
    lib.csa_indexer_topk_workspace_size.argtypes = [i64, i64, i32, i32, i32, i64, i64, i32,
                                                    ctypes.POINTER(csa_opts),
                                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.csa_indexer_topk_workspace_size.restype = ctypes.c_int
    lib.csa_indexer_topk.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i64, i64,
                                     vp, vp, vp, ctypes.c_size_t, ctypes.POINTER(csa_opts), vp]
    lib.csa_indexer_topk.restype = ctypes.c_int
    lib.csa_indexer_topk_batched.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, i32, i64,
                                             i64, vp, vp, vp, ctypes.c_size_t,
                                             ctypes.POINTER(csa_opts), vp]
    lib.csa_indexer_topk_batched.restype = ctypes.c_int
    lib.csa_indexer_topk_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i64, i64,
                                             vp, vp, ctypes.POINTER(csa_opts), vp]
    lib.csa_indexer_topk_noalloc.restype = ctypes.c_int
    lib.csa_profile_enable.argtypes = [ctypes.c_int]
    lib.csa_profile_enable.restype = ctypes.c_int
    lib.csa_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), i32]
    lib.csa_profile_collect.restype = ctypes.c_int
    lib.csa_sparse_attention.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i64,
                                         ctypes.c_float, vp]
    lib.csa_sparse_attention.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().csa_status_str(status).decode()
        raise CsaError(status, msg)


def abi_version() -> int:
    return load_library().csa_abi_version()


def _opts(chunk_keys=0, key_tile=0, workspace_budget=0, key_splits=0):
    o = csa_opts()
    o.chunk_keys = int(chunk_keys or 0)
    o.key_tile = int(key_tile or 0)
    o.workspace_budget = int(workspace_budget or 0)
    o.key_splits = int(key_splits or 0)
    return o


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return CSA_BF16
    if t == torch.float32:
        return CSA_F32
    raise TypeError("q, w, kc must be bfloat16 or float32, got %s" % t)


def _caller_buffer(t: torch.Tensor, dev: torch.device, name: str) -> None:
    """A buffer the caller passes in (outputs, workspace) must be contiguous
    and on the inputs' GPU: the library gets only its address and size."""
    if t.device != dev:
        raise ValueError("%s must be on %s, not %s" % (name, dev, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_size(S, T, H, D, m, k, *, q_pos0=0, dtype=torch.bfloat16, chunk_keys=0,
                   key_tile=0, workspace_budget=0, key_splits=0) -> int:
    out = ctypes.c_size_t(0)
    o = _opts(chunk_keys, key_tile, workspace_budget, key_splits)
    _check(load_library().csa_indexer_topk_workspace_size(
        int(S), int(T), int(H), int(D), int(m), int(k), int(q_pos0), _dtype_code(dtype),
        ctypes.byref(o), ctypes.byref(out)))
    return int(out.value)


def topk(q: torch.Tensor, w: torch.Tensor, kc: torch.Tensor, m: int, k: int, *,
         q_pos0: int = 0, chunk_keys: int = 0, key_tile: int = 0, workspace_budget: int = 0,
         key_splits: int = 0, workspace: torch.Tensor | None = None, out: tuple | None = None):
    """CSA lightning-indexer top-k on the GPU.

    q [S, H, D], w [S, H], kc [T, D]: contiguous device tensors, all bfloat16
    or all float32.  Returns (idx [S, k] int32, score [S, k] float32), rows
    ordered by score descending then key index ascending, padded with -1 /
    -inf.  Runs on torch's current stream; does not synchronise.

    Batched form: q [B, S, H, D], w [B, S, H], kc [B, T, D] (B independent
    problems, each with its own keys) gives idx, score [B, S, k]; the
    workspace is sized for one problem and reused.
    """
    batched = q.dim() == 4
    if batched:
        if w.dim() != 3 or kc.dim() != 3:
            raise ValueError("batched: q must be [B,S,H,D], w [B,S,H], kc [B,T,D]")
        B, S, H, D = q.shape
        T = kc.shape[1]
        if tuple(w.shape) != (B, S, H) or kc.shape[0] != B or kc.shape[2] != D:
            raise ValueError("shape mismatch: q %s, w %s, kc %s"
                             % (tuple(q.shape), tuple(w.shape), tuple(kc.shape)))
        oshape = (B, S, k)
    else:
        if q.dim() != 3 or w.dim() != 2 or kc.dim() != 2:
            raise ValueError("q must be [S,H,D], w [S,H], kc [T,D]")
        S, H, D = q.shape
        T = kc.shape[0]
        if tuple(w.shape) != (S, H) or (kc.shape[1] != D):
            raise ValueError("shape mismatch: q %s, w %s, kc %s"
                             % (tuple(q.shape), tuple(w.shape), tuple(kc.shape)))
        oshape = (S, k)
    if not (q.dtype == w.dtype == kc.dtype):
        raise TypeError("q, w, kc must share one dtype")
    dev = q.device
    if dev.type != "cuda" or w.device != dev or kc.device != dev:
        raise ValueError("q, w, kc must be on one GPU device")
    for name, t in (("q", q), ("w", w), ("kc", kc)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    dt = _dtype_code(q.dtype)
    lib = load_library()
    o = _opts(chunk_keys, key_tile, workspace_budget, key_splits)
    if out is None:
        idx = torch.empty(oshape, dtype=torch.int32, device=dev)
        score = torch.empty(oshape, dtype=torch.float32, device=dev)
    else:
        idx, score = out
        if tuple(idx.shape) != oshape or tuple(score.shape) != oshape \
                or idx.dtype != torch.int32 or score.dtype != torch.float32:
            raise ValueError("out must be contiguous int32/float32 tensors of shape %s"
                             % (oshape,))
        _caller_buffer(idx, dev, "out idx")
        _caller_buffer(score, dev, "out score")
    if workspace is None:
        nbytes = workspace_size(S, T, H, D, m, k, q_pos0=q_pos0, dtype=q.dtype,
                                chunk_keys=chunk_keys, key_tile=key_tile,
                                workspace_budget=workspace_budget, key_splits=key_splits)
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    else:
        _caller_buffer(workspace, dev, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        if batched:
            _check(lib.csa_indexer_topk_batched(
                ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                ctypes.c_void_p(kc.data_ptr()), dt, B, S, T, H, D, int(m), int(k), int(q_pos0),
                ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(score.data_ptr()),
                ctypes.c_void_p(workspace.data_ptr()), nbytes, ctypes.byref(o),
                ctypes.c_void_p(stream)))
        else:
            _check(lib.csa_indexer_topk(
                ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                ctypes.c_void_p(kc.data_ptr()), dt, S, T, H, D, int(m), int(k), int(q_pos0),
                ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(score.data_ptr()),
                ctypes.c_void_p(workspace.data_ptr()), nbytes, ctypes.byref(o),
                ctypes.c_void_p(stream)))
    return idx, score


def topk_noalloc(q: torch.Tensor, w: torch.Tensor, kc: torch.Tensor, m: int, k: int, *,
                 q_pos0: int = 0, chunk_keys: int = 0, key_tile: int = 0,
                 workspace_budget: int = 0, key_splits: int = 0, out: tuple | None = None):
    """``topk`` through the library's allocation-free entry point: no
    workspace (the library's fixed per-GPU scratch serves instead).  Pass
    ``out`` = (idx, score) to allocate nothing at all.  Calls that overlap
    on one GPU share that scratch and race; calls ordered on one stream do
    not."""
    if q.dim() != 3 or w.dim() != 2 or kc.dim() != 2:
        raise ValueError("q must be [S,H,D], w [S,H], kc [T,D]")
    S, H, D = q.shape
    T = kc.shape[0]
    if tuple(w.shape) != (S, H) or kc.shape[1] != D:
        raise ValueError("shape mismatch: q %s, w %s, kc %s"
                         % (tuple(q.shape), tuple(w.shape), tuple(kc.shape)))
    if not (q.dtype == w.dtype == kc.dtype):
        raise TypeError("q, w, kc must share one dtype")
    dev = q.device
    if dev.type != "cuda" or w.device != dev or kc.device != dev:
        raise ValueError("q, w, kc must be on one GPU device")
    for name, t in (("q", q), ("w", w), ("kc", kc)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if out is None:
        idx = torch.empty((S, k), dtype=torch.int32, device=dev)
        score = torch.empty((S, k), dtype=torch.float32, device=dev)
    else:
        idx, score = out
        if tuple(idx.shape) != (S, k) or tuple(score.shape) != (S, k) \
                or idx.dtype != torch.int32 or score.dtype != torch.float32:
            raise ValueError("out must be contiguous int32/float32 tensors of shape %s"
                             % ((S, k),))
        _caller_buffer(idx, dev, "out idx")
        _caller_buffer(score, dev, "out score")
    o = _opts(chunk_keys, key_tile, workspace_budget, key_splits)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        _check(load_library().csa_indexer_topk_noalloc(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(w.data_ptr()),
            ctypes.c_void_p(kc.data_ptr()), _dtype_code(q.dtype), S, T, H, D, int(m), int(k),
            int(q_pos0), ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(score.data_ptr()),
            ctypes.byref(o), ctypes.c_void_p(stream)))
    return idx, score


def sparse_attention(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor, d_v: int, *,
                     scale: float | None = None, out: torch.Tensor | None = None):
    """Sparse attention of each query row over its selected entries (the CSA
    consumer of ``topk``'s idx), shared-latent form: all heads attend over
    the same entries, kv[e, :] is an entry's key and kv[e, :d_v] its value.

    q [S, H, D_K], kv [T, D_K] bfloat16, idx [S, k] int32 (-1 = none), all
    contiguous on one GPU.  scale defaults to 1/sqrt(D_K).  Returns out
    [S, H, d_v] bfloat16.  Runs on torch's current stream.
    """
    if q.dim() != 3 or kv.dim() != 2 or idx.dim() != 2:
        raise ValueError("q must be [S,H,D_K], kv [T,D_K], idx [S,k]")
    S, H, DK = q.shape
    T = kv.shape[0]
    if kv.shape[1] != DK or idx.shape[0] != S:
        raise ValueError("shape mismatch: q %s, kv %s, idx %s"
                         % (tuple(q.shape), tuple(kv.shape), tuple(idx.shape)))
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16 or idx.dtype != torch.int32:
        raise TypeError("q and kv must be bfloat16, idx int32")
    dev = q.device
    if dev.type != "cuda" or kv.device != dev or idx.device != dev:
        raise ValueError("q, kv, idx must be on one GPU device")
    for name, t in (("q", q), ("kv", kv), ("idx", idx)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    k = idx.shape[1]
    if scale is None:
        scale = 1.0 / float(DK) ** 0.5
    oshape = (S, H, int(d_v))
    if out is None:
        out = torch.empty(oshape, dtype=torch.bfloat16, device=dev)
    else:
        if tuple(out.shape) != oshape or out.dtype != torch.bfloat16:
            raise ValueError("out must be a contiguous bfloat16 tensor of shape %s" % (oshape,))
        _caller_buffer(out, dev, "out")
    lib = load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        _check(lib.csa_sparse_attention(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv.data_ptr()),
            ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(out.data_ptr()), CSA_BF16,
            S, T, H, DK, int(d_v), k, float(scale), ctypes.c_void_p(stream)))
    return out


def profile_enable(on: bool = True):
    _check(load_library().csa_profile_enable(1 if on else 0))


def profile_collect():
    """{kernel name: (total ms, launches)} since the last collect; waits for
    the recorded events."""
    ms = (ctypes.c_double * CSA_KERNEL_KINDS)()
    n = (ctypes.c_int64 * CSA_KERNEL_KINDS)()
    _check(load_library().csa_profile_collect(ms, n, CSA_KERNEL_KINDS))
    return {KERNEL_NAMES[i]: (ms[i], n[i]) for i in range(CSA_KERNEL_KINDS)}
