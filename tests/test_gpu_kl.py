"""GPU parity of the LSA warm-up KL operator (lsa_kl_warmup).

Checked row by row against oracle.kl_warmup_row (float64, its own softmax
normalisers). Bound, from the arithmetic: the kernel's probabilities are
exp2(S sl2 - lse2) with S an fp32 MFMA sum of exact bf16 products and lse the
forward's fp32 log-sum-exp (error a few 1e-7 in the natural log, measured),
so each p_j carries a relative error below 1e-5; log-softmax of the fp32
logits adds a few fp32 ulps. Hence |dlogits_gpu - dlogits| <= 1e-5 (p + q) +
1e-7 and |kl_gpu - kl| <= 1e-5 (1 + sum_j p_j |log p_j - log q_j|) + 1e-5 sum
over the n log terms' fp32 rounding (bounded by 1e-6 n). Every call runs twice
and must be bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_lsa_amd import _lib as L
from long_context_sparse_lsa_amd import synth
from tests._util import f64, need_gpu, np_, say
from tests.test_gpu_backward import random_lists

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    L.load()


def bf(shape, *seed):
    return synth.bf16_normal(shape, synth.seed_of("kl", *seed), DEV)


def run_kl(B, Lq, H, n_k, idx, n_sel, seed, what, logits=None):
    q, k, v = bf((B, Lq, H, 128), "q", seed), bf((B, n_k, 128), "k", seed), bf((B, n_k, 128), "v", seed)
    _, lse = L.lsa_sparse_attn_prefill(q, k, v, idx, n_sel, want_lse=True)
    if logits is None:
        g = torch.Generator(device=DEV)
        g.manual_seed(synth.seed_of("kl-logits", seed))
        logits = 2.0 * torch.randn(idx.shape, generator=g, device=DEV, dtype=torch.float32)
    kl, dl = L.lsa_kl_warmup(q, k, idx, n_sel, lse, logits)
    kl2, dl2 = L.lsa_kl_warmup(q, k, idx, n_sel, lse, logits)
    torch.cuda.synchronize()
    assert torch.equal(kl, kl2) and torch.equal(dl, dl2), f"{what}: not deterministic"
    In, Nn, lg = np_(idx), np_(n_sel), np_(logits).astype(np.float64)
    qf, kf = f64(q), f64(k)
    klg, dlg = np_(kl), np_(dl)
    worst_kl = worst_dl = 0.0
    for b in range(B):
        for t in range(Lq):
            n = int(Nn[b, t])
            assert np.all(dlg[b, t, n:] == 0), f"{what}: padding of row {t}"
            if n == 0:
                assert klg[b, t] == 0, f"{what}: empty row {t}"
                continue
            sel = In[b, t, :n]
            ref_kl, ref_g = O.kl_warmup_row(qf[b, t], kf[b], sel, 128 ** -0.5, lg[b, t, :n])
            # q and p of the row, for the bound (p = softmax(logits) - gradient)
            m = lg[b, t, :n].max()
            qd = np.exp(lg[b, t, :n] - m)
            qd /= qd.sum()
            p = qd - ref_g
            bound_g = 1e-5 * (np.abs(p) + qd) + 1e-7
            e_g = np.abs(dlg[b, t, :n] - ref_g)
            assert np.all(e_g <= bound_g), f"{what}: row {t} gradient error {e_g.max():.3g}"
            pos = p > 0
            spread = float(np.sum(p[pos] * np.abs(np.log(p[pos]) - np.log(qd[pos]))))
            bound_kl = 1e-5 * (1 + spread) + 1e-6 * n
            e_kl = abs(float(klg[b, t]) - ref_kl)
            assert e_kl <= bound_kl, f"{what}: row {t} KL {klg[b, t]} vs {ref_kl}"
            worst_kl, worst_dl = max(worst_kl, e_kl), max(worst_dl, float(e_g.max()))
    say(f"  {what}: max-abs kl {worst_kl:.3g}, dlogits {worst_dl:.3g}")


@pytest.mark.parametrize("H", [32, 64, 128])
def test_kl_random_lists(H):
    B, Lq, K_tot = 2, 300, 200
    say(f"kl random lists H={H}")
    idx, n_sel = random_lists(B, Lq, K_tot, Lq, 60 + H, empty_rows=(3, 250))
    run_kl(B, Lq, H, Lq, idx, n_sel, H, f"random H={H}")


def test_kl_dense_warmup_lists():
    # the dense warm-up: every row's list is all of 0..t
    B, Lq, H = 1, 160, 64
    idx, n_sel = random_lists(B, Lq, 256, Lq, 9)
    run_kl(B, Lq, H, Lq, idx, n_sel, 9, "dense")


def test_kl_on_selected_lists_with_indexer_logits():
    """Sparse-stage KL on the lists the fused selector picks, with the
    indexer's own scores (scaled) as logits."""
    B, Lq, H, H_I, d_I = 1, 1200, 64, 64, 128
    q_idx = synth.int8_uniform((B, Lq, H_I, d_I), -16, 15, synth.seed_of("kl-i", 1), DEV)
    k_idx = synth.int8_uniform((B, Lq, d_I), -16, 15, synth.seed_of("kl-i", 2), DEV)
    w = synth.int_weights(H_I, 1, 8, 3)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, 4, 64, 188, q_off=0)
    scores = L.lsa_index_score(q_idx, k_idx, w, q_off=0)
    # the indexer scores of each row's listed keys as logits, scaled to O(1)
    logits = torch.gather(scores.float(), 2, idx.clamp(min=0).long()) * (1.0 / 65536.0)
    logits = torch.where(idx >= 0, logits, torch.zeros_like(logits)).contiguous()
    run_kl(B, Lq, H, Lq, idx, n_sel, 5, "selected lists", logits=logits)
