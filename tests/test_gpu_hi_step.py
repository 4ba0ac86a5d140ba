"""GPU parity of the fused HI decode step (lsa_hier_decode_step).

The fused step must equal lsa_hier_select followed by lsa_sparse_attn_decode
bit for bit (idx, n_sel, o, lse: the same device code in one persistent
launch), its lists must equal the oracle's HI selection, its outputs must be
within the attention tolerance of the oracle, repeated calls must be
bit-identical, and no wait may have hit its bound (workspace word 1).
"""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_lsa_amd import _lib as L
from long_context_sparse_lsa_amd import configs, synth
from tests._util import AttnErrors, f64, need_gpu, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    L.load()


def run_case(B, n_k, blk, rec, ns, W, kd, n_split, seed, check_rows=None):
    g = lambda shape, *s: synth.int8_uniform(shape, -16, 15, synth.seed_of("hi-step", seed, *s), DEV)  # noqa: E731
    q_idx, k_idx = g((B, 64, 128), "q"), g((B, n_k, 128), "k")
    w = synth.int_weights(64, 1, 8, seed)
    q = synth.bf16_normal((B, 1, 64, 128), synth.seed_of("hi-step", seed, "aq"), DEV)
    kc = synth.bf16_normal((B, n_k, 128), synth.seed_of("hi-step", seed, "ak"), DEV)
    vc = synth.bf16_normal((B, n_k, 128), synth.seed_of("hi-step", seed, "av"), DEV)
    kblk = L.lsa_block_summary(k_idx, blk)
    idx, n_sel, o, lse = L.lsa_hier_decode_step(q_idx, k_idx, kblk, w, q, kc, vc, blk, rec, ns, W, kd,
                                                n_split=n_split, want_lse=True)
    idx2, n_sel2, o2, lse2 = L.lsa_hier_decode_step(q_idx, k_idx, kblk, w, q, kc, vc, blk, rec, ns, W, kd,
                                                    n_split=n_split, want_lse=True)
    ridx, rn = L.lsa_hier_select(q_idx, k_idx, kblk, w, blk, rec, ns, W, kd)
    ro, rl = L.lsa_sparse_attn_decode(q, kc, vc, ridx[:, None].contiguous(), rn[:, None].contiguous(),
                                      n_split=n_split, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2) and torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(idx, ridx) and torch.equal(n_sel, rn), "fused lists differ from lsa_hier_select"
    assert torch.equal(o, ro) and torch.equal(lse, rl), "fused attention differs from lsa_sparse_attn_decode"
    err = AttnErrors(f"hi step n_k={n_k} blk={blk} rec={rec}")
    In, Nn = np_(idx), np_(n_sel)
    for b in (check_rows if check_rows is not None else range(B)):
        kn = np_(k_idx[b])
        ref = O.hier_select(np_(q_idx[b]), kn, O.block_summary(kn, blk), w, blk, rec, ns, W, kd)
        assert np.array_equal(In[b, : Nn[b]], ref), f"b{b}: idx differs from the oracle"
        assert np.all(In[b, Nn[b]:] == -1)
        t = torch.as_tensor(ref, dtype=torch.long, device=DEV)
        ref_o, ref_l = O.attend(f64(q[b, 0]), f64(kc[b][t]), f64(vc[b][t]), np.arange(len(ref)), 128 ** -0.5)
        err.add(f64(o[b, 0]), ref_o)
        assert np.abs(np_(lse[b, 0]) - ref_l).max() < 1e-3
    say("  ", err.check())


@pytest.mark.parametrize("B,n_k,blk,rec,ns,W,kd,n_split", [
    (4, 40000, 64, 256, 4, 512, 2048, 8),    # C4's selection shape on a shorter cache
    (3, 30001, 128, 64, 4, 300, 1000, 5),    # a partial last block, 5 parts
    (2, 9000, 64, 3, 4, 512, 2048, 8),       # fewer candidates than k_dyn: n_sel shrinks
    (5, 16384, 32, 500, 0, 0, 700, 1),       # no sinks or window, one part
])
def test_hi_step_matches_separate_calls_and_oracle(B, n_k, blk, rec, ns, W, kd, n_split):
    say(f"hi step B={B} n_k={n_k} blk={blk} rec={rec} K={ns}+{W}+{kd} parts={n_split}")
    run_case(B, n_k, blk, rec, ns, W, kd, n_split, seed=n_k + blk)


def test_hi_step_c4_full_size():
    """The C4 workload (B = 4, 1M keys, block 64, recall 256, 4 + 512 + 2048,
    8 parts) as bench.py --fused runs it."""
    wl = configs.C4
    say("hi step at C4")
    q_idx, k_idx, w = synth.indexer_inputs(wl, DEV)
    q, kc, vc = synth.attention_inputs(wl, 0, DEV)
    kblk = L.lsa_block_summary(k_idx, wl.blk)
    idx, n_sel, o = L.lsa_hier_decode_step(q_idx, k_idx, kblk, w, q, kc, vc, wl.blk, wl.n_blk_recall, wl.n_sink,
                                           wl.n_window, wl.k_dyn, n_split=wl.n_split)
    ridx, rn = L.lsa_hier_select(q_idx, k_idx, kblk, w, wl.blk, wl.n_blk_recall, wl.n_sink, wl.n_window, wl.k_dyn)
    ro = L.lsa_sparse_attn_decode(q, kc, vc, ridx[:, None].contiguous(), rn[:, None].contiguous(),
                                  n_split=wl.n_split)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx) and torch.equal(n_sel, rn) and torch.equal(o, ro)
    b = 1
    kn = np_(k_idx[b])
    ref = O.hier_select(np_(q_idx[b]), kn, O.block_summary(kn, wl.blk), w, wl.blk, wl.n_blk_recall, wl.n_sink,
                        wl.n_window, wl.k_dyn)
    assert np.array_equal(np_(idx[b, : n_sel[b]]), ref)


def test_hi_step_reports_no_exceeded_wait():
    B, n_k = 2, 20000
    g = lambda shape, s: synth.int8_uniform(shape, -16, 15, synth.seed_of("hi-step-w", s), DEV)  # noqa: E731
    q_idx, k_idx = g((B, 64, 128), 1), g((B, n_k, 128), 2)
    q = synth.bf16_normal((B, 1, 64, 128), 3, DEV)
    kc, vc = synth.bf16_normal((B, n_k, 128), 4, DEV), synth.bf16_normal((B, n_k, 128), 5, DEV)
    kblk = L.lsa_block_summary(k_idx, 64)
    ws = torch.full((1 << 24,), 255, dtype=torch.uint8, device=DEV)   # garbage counters: the call clears them
    L.lsa_hier_decode_step(q_idx, k_idx, kblk, np.ones(64, np.int32), q, kc, vc, 64, 32, 4, 128, 512, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:256].view(torch.int32)[1]) == 0
