"""The no-alloc split-KV decode entry point against the workspace one.

lsa_sparse_attn_decode_noalloc runs the same kernels as
lsa_sparse_attn_decode with the partials in the library's fixed scratch
array; both must give bit-identical o and lse, on two calls in a row (the
second with a smaller batch, so the array holds the first call's partials
when the second starts), and agree with the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_lsa_amd import _lib as L
from long_context_sparse_lsa_amd import synth
from tests._util import AttnErrors, f64, need_gpu, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, n_q, H, n_k, K_tot, seed):
    g = np.random.default_rng(seed)
    idx = np.full((B, 1, K_tot), -1, dtype=np.int32)
    n_sel = np.zeros((B, 1), dtype=np.int32)
    for b in range(B):
        n = int(g.integers(1, K_tot + 1))
        idx[b, 0, :n] = np.sort(g.choice(n_k, n, replace=False))
        n_sel[b, 0] = n
    q = synth.bf16_normal((B, n_q, H, 128), synth.seed_of("noalloc-q", seed), DEV)
    k = synth.bf16_normal((B, n_k, 128), synth.seed_of("noalloc-k", seed), DEV)
    v = synth.bf16_normal((B, n_k, 128), synth.seed_of("noalloc-v", seed), DEV)
    return q, k, v, torch.tensor(idx, device=DEV), torch.tensor(n_sel, device=DEV)


def test_noalloc_decode_matches_workspace_decode():
    need_gpu()
    L.load()
    cases = [(16, 4, 64, 20000, 2564, 8, 1), (3, 2, 32, 5000, 700, 5, 2)]  # second call: smaller
    for B, n_q, H, n_k, K_tot, n_split, seed in cases:
        say(f"noalloc decode B={B} n_q={n_q} H={H} n_k={n_k} K_tot={K_tot} n_split={n_split}")
        q, k, v, idx, n_sel = _case(B, n_q, H, n_k, K_tot, seed)
        o_ref, l_ref = L.lsa_sparse_attn_decode(q, k, v, idx, n_sel, n_split=n_split, want_lse=True)
        o, lse = L.lsa_sparse_attn_decode_noalloc(q, k, v, idx, n_sel, n_split=n_split, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "no-alloc decode differs from the workspace call"
        In, Nn = np_(idx), np_(n_sel)
        qf, kf, vf, of = f64(q), f64(k), f64(v), f64(o)
        err = AttnErrors(f"noalloc B={B}")
        for b in range(min(B, 4)):
            ref, _ = O.attend(qf[b].reshape(-1, 128), kf[b], vf[b], In[b, 0, : Nn[b, 0]], 128 ** -0.5)
            err.add(of[b].reshape(-1, 128), ref)
        err.check()


def test_noalloc_rejects_sizes_beyond_the_scratch():
    need_gpu()
    lib = L.load()
    cap = lib.lsa_noalloc_scratch_bytes()
    B = cap // (8 * 4 * 128 * 264) + 1   # more partial rows than the array holds
    P = ctypes.c_void_p
    F = P(0x7F0000000000)
    s = lib.lsa_sparse_attn_decode_noalloc(F, F, F, F, F, 1, B, 4, 1000, 128, 128, 64, 8, 0.088, F, None, None)
    assert s == L.LSA_SCRATCH_LIMIT
