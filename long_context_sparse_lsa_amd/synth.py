"""Seeded synthetic inputs for the LSA workloads.

This module only draws random numbers: int8 indexer queries/keys uniform in a
closed range, integer per-head weights, and bf16 attention q/k/v drawn from
N(0, 1) in float32 and rounded to bfloat16 by torch's round-to-nearest-even
cast. It holds none of the method's arithmetic, so both the HIP path and the
oracle can consume the same tensors.

Every tensor has its own seed, derived from (workload name, tensor name,
layer, base seed), so any tensor can be regenerated on its own.
"""
import hashlib

import numpy as np
import torch

BASE_SEED = 20260630


def seed_of(*parts) -> int:
    h = hashlib.blake2b(repr(parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def int8_uniform(shape, lo: int, hi: int, seed: int, device="cpu") -> torch.Tensor:
    """int8 values uniform on the closed range [lo, hi]."""
    assert -128 <= lo <= hi <= 127
    g = _gen(seed, device)
    return torch.randint(lo, hi + 1, tuple(shape), dtype=torch.int8,
                         generator=g, device=device)


def bf16_normal(shape, seed: int, device="cpu", chunk_elems=1 << 28) -> torch.Tensor:
    """N(0,1) drawn in float32, rounded to bfloat16 (nearest-even)."""
    shape = tuple(shape)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    g = _gen(seed, device)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=g, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def int_weights(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-head integer weights uniform on [lo, hi] (host array)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def indexer_inputs(wl, device="cpu", base=BASE_SEED, L=None, B=None):
    """Indexer tensors of a workload.

    prefill:  q_idx [B, L, H_I, d_I], k_idx [B, L, d_I]
    decode:   q_idx [B, H_I, d_I] (the target row), k_idx [B, N, d_I]
    w:        [H_I] int32 host array
    """
    L = wl.L if L is None else L
    B = wl.B if B is None else B
    w = int_weights(wl.H_I, wl.w_lo, wl.w_hi, seed_of(wl.name, "w", base))
    if wl.kind == "prefill":
        qshape = (B, L, wl.H_I, wl.d_I)
    else:
        qshape = (B, wl.H_I, wl.d_I)
    q_idx = int8_uniform(qshape, wl.qk_lo, wl.qk_hi, seed_of(wl.name, "q_idx", base), device)
    k_idx = int8_uniform((B, L, wl.d_I), wl.qk_lo, wl.qk_hi,
                         seed_of(wl.name, "k_idx", base), device)
    return q_idx, k_idx, w


def attention_inputs(wl, layer=0, device="cpu", base=BASE_SEED, L=None, B=None):
    """Attention tensors of one layer.

    prefill:  q [B, L, H, D], k/v [B, L, D]
    decode:   q [B, n_q, H, D], k/v caches [B, N, D]
    """
    L = wl.L if L is None else L
    B = wl.B if B is None else B
    if wl.kind == "prefill":
        qshape = (B, L, wl.H, wl.D)
    else:
        qshape = (B, wl.n_q, wl.H, wl.D)
    q = bf16_normal(qshape, seed_of(wl.name, "q", layer, base), device)
    k = bf16_normal((B, L, wl.D), seed_of(wl.name, "k", layer, base), device)
    v = bf16_normal((B, L, wl.D), seed_of(wl.name, "v", layer, base), device)
    return q, k, v
