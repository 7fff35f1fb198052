"""Seeded synthetic inputs for the CSA lightning-indexer top-k.

This module only draws random tensors; it holds none of the indexer's
arithmetic, so both the GPU path and the CPU oracle can take their inputs from
it.  The page ("StreamIndex: Memory-Bounded Compressed Sparse Attention via
Streaming Top-k", Abstract) measures on synthetic V4-shaped inputs; the shapes
and distributions here follow that: H_I=64 indexer heads, head dimension 128,
compression ratio m=4, k=2048 at the large sizes.

Every generator draws with a ``torch.Generator`` seeded by ``seed`` in the
fixed order q, w, kc (mixture keys: centres, assignments, noise), in float32,
then rounds to the requested dtype (round to nearest even for bfloat16).  Large
tensors are drawn in fixed slices so the stream of draws never depends on free
memory.
"""
from __future__ import annotations

import math

import torch

# Rows drawn per slice for the large device-side generators.
_SLICE_ELEMS = 1 << 28


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_sliced(shape, g, device, scale, out_dtype):
    """N(0,1)*scale drawn row-slice by row-slice, stored as ``out_dtype``."""
    out = torch.empty(shape, dtype=out_dtype, device=device)
    if out.numel() == 0:
        return out
    row_elems = max(1, out[0].numel())
    step = max(1, _SLICE_ELEMS // row_elems)
    for r0 in range(0, shape[0], step):
        r1 = min(shape[0], r0 + step)
        x = torch.randn((r1 - r0, *shape[1:]), generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out[r0:r1].copy_(x)
        del x
    return out


def gaussian_fp32(S: int, T: int, H: int, D: int, seed: int, device="cpu"):
    """Tiny-indexer distribution: q, kc ~ N(0,1) and w ~ U(0,1)/H, all fp32."""
    g = _gen(seed, device)
    q = torch.randn((S, H, D), generator=g, device=device, dtype=torch.float32)
    w = torch.rand((S, H), generator=g, device=device, dtype=torch.float32) / H
    kc = torch.randn((T, D), generator=g, device=device, dtype=torch.float32)
    return q, w, kc


def _randint_sliced(lo, hi, shape, g, device, out_dtype):
    """Uniform integers on [lo, hi) drawn row-slice by row-slice (the int64
    draws of a whole large tensor would need 4x its bf16 size), stored as
    ``out_dtype``."""
    out = torch.empty(shape, dtype=out_dtype, device=device)
    if out.numel() == 0:
        return out
    row_elems = max(1, out[0].numel())
    step = max(1, _SLICE_ELEMS // row_elems)
    for r0 in range(0, shape[0], step):
        r1 = min(shape[0], r0 + step)
        out[r0:r1].copy_(torch.randint(lo, hi, (r1 - r0, *shape[1:]), generator=g, device=device))
    return out


def integer_valued(S: int, T: int, H: int, D: int, seed: int, dtype=torch.float32,
                   signed_w: bool = False, device="cpu"):
    """Integer-valued inputs, exact in fp32 and bf16: q, kc uniform on
    {-3..3}; w uniform on {1, 2}, or on {-2, -1, 1, 2} when ``signed_w``.
    A q of more than 2^28 elements is drawn in row slices."""
    g = _gen(seed, device)
    if S * H * D > _SLICE_ELEMS:
        q = _randint_sliced(-3, 4, (S, H, D), g, device, dtype)
    else:
        q = torch.randint(-3, 4, (S, H, D), generator=g, device=device).to(dtype)
    if signed_w:
        wi = torch.randint(0, 4, (S, H), generator=g, device=device)
        table = torch.tensor([-2, -1, 1, 2], device=device)
        w = table[wi].to(dtype)
    else:
        w = torch.randint(1, 3, (S, H), generator=g, device=device).to(dtype)
    kc = torch.randint(-3, 4, (T, D), generator=g, device=device).to(dtype)
    return q, w, kc


def bf16_gaussian(S: int, T: int, H: int, D: int, seed: int, device="cpu"):
    """V4-shaped bf16 inputs: q, kc ~ N(0,1)/sqrt(D) and w ~ N(0,1)/sqrt(H)
    (signed), drawn in fp32 and rounded to bf16."""
    g = _gen(seed, device)
    q = _randn_sliced((S, H, D), g, device, 1.0 / math.sqrt(D), torch.bfloat16)
    w = _randn_sliced((S, H), g, device, 1.0 / math.sqrt(H), torch.bfloat16)
    kc = _randn_sliced((T, D), g, device, 1.0 / math.sqrt(D), torch.bfloat16)
    return q, w, kc


def bf16_mixture(S: int, T: int, H: int, D: int, seed: int, device="cpu",
                 components: int = 64, spread: float = 0.3):
    """q and w as ``bf16_gaussian``; keys from a Gaussian mixture: centres
    ~ N(0, I), each key picks a centre uniformly and adds N(0, spread^2)
    noise.  Many keys then score almost alike, which stresses tie handling
    in the top-k merge."""
    g = _gen(seed, device)
    q = _randn_sliced((S, H, D), g, device, 1.0 / math.sqrt(D), torch.bfloat16)
    w = _randn_sliced((S, H), g, device, 1.0 / math.sqrt(H), torch.bfloat16)
    centres = torch.randn((components, D), generator=g, device=device, dtype=torch.float32)
    assign = torch.randint(0, components, (T,), generator=g, device=device)
    noise = torch.randn((T, D), generator=g, device=device, dtype=torch.float32)
    kc = (centres[assign] + spread * noise).to(torch.bfloat16)
    return q, w, kc


def attention_gaussian(S: int, T: int, H: int, DK: int, seed: int, device="cpu"):
    """Inputs of the sparse attention: q [S, H, DK] and the latent rows kv
    [T, DK], entries N(0, 1) drawn in fp32 and rounded to bf16."""
    g = _gen(seed, device)
    q = _randn_sliced((S, H, DK), g, device, 1.0, torch.bfloat16)
    kv = _randn_sliced((T, DK), g, device, 1.0, torch.bfloat16)
    return q, kv


def sample_rows(S: int, m: int, k: int, count: int, seed: int):
    """A fixed set of query rows to check at sizes where the oracle cannot
    take every row: the boundary rows (first rows, the first row with a key,
    the rows where the number of usable keys crosses k, the last rows), then
    seeded uniform draws without replacement up to ``count``.  Sorted."""
    fixed = [0, 1, m - 1, m, m * k - 2, m * k - 1, m * k, m * k + 1, S - m - 1, S - 2, S - 1]
    chosen = sorted({r for r in fixed if 0 <= r < S})
    if count <= len(chosen) or count >= S:
        return chosen[:count] if count < S else list(range(S))
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    taken = set(chosen)
    perm = torch.randperm(S, generator=g).tolist()
    for r in perm:
        if len(taken) >= count:
            break
        taken.add(r)
    return sorted(taken)


def config(n: int):
    """The five workloads, by number, as keyword dicts (S, T, H, D, m, k)."""
    table = {
        1: dict(S=1024, T=256, H=4, D=32, m=4, k=16),
        2: dict(S=16384, T=4096, H=64, D=128, m=4, k=2048),
        3: dict(S=65536, T=16384, H=64, D=128, m=4, k=2048),
        4: dict(S=262144, T=65536, H=64, D=128, m=4, k=2048),
        5: dict(S=1048576, T=262144, H=64, D=128, m=4, k=2048),
    }
    return dict(table[n])
