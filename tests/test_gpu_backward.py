"""GPU parity of the deterministic sparse attention backward.

lsa_sparse_attn_backward is checked against the float64 oracle
(oracle.sparse_attn_backward) element by element, with a bound derived from
the arithmetic of the kernel:
  - each gradient element is a sum of terms of which one factor was rounded
    to bf16 once (P for dv, dS for dq and dk: relative error 2^-9), and dq is
    written in bf16 (another 2^-9 of |dq|);
  - dS = P (dP - Delta) carries the error of Delta = sum_d dO . o computed
    from the forward's bf16 output o, whose own error is at most 2^-8 of
    sum_s P_s |v_s| per element (the bf16 P of its PV product and the bf16
    rounding of o), so |dDelta| <= e = 2^-8 sum_d |dO_d| sum_s P_s |v_s,d|;
  - the fp32 sums, exp2 and the 2^-32 fixed-point rounding add far less.
With R the sum of |term| an element adds up and E the sum of the terms'
Delta errors (P e |k| for dq and dk), |gpu - oracle| <= 2^-7 R + 2 E + 1e-5:
twice each error source. Every call runs twice and must be bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_lsa_amd import _lib as L
from long_context_sparse_lsa_amd import synth
from tests._util import f64, need_gpu, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL = 2.0 ** -7
ATOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    L.load()


def bf(shape, *seed):
    return synth.bf16_normal(shape, synth.seed_of("bwd", *seed), DEV)


def grad_bounds(q, k, v, lists, scale, do):
    """Error bound of each gradient element (see the module docstring)."""
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for t, sel in enumerate(lists):
        if len(sel) == 0:
            continue
        Ks, Vs = k[sel], v[sel]
        z = q[t] @ Ks.T * scale
        P = np.exp(z - z.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        ot = P @ Vs
        ds = P * (do[t] @ Vs.T - (do[t] * ot).sum(axis=1, keepdims=True))
        e = 2.0 ** -8 * (np.abs(do[t]) * (P @ np.abs(Vs))).sum(axis=1, keepdims=True)   # [H, 1]
        bq[t] = scale * (REL * np.abs(ds) + 2 * P * e) @ np.abs(Ks)
        bk[sel] += scale * (REL * np.abs(ds) + 2 * P * e).T @ np.abs(q[t])
        bv[sel] += REL * P.T @ np.abs(do[t])
    return bq + ATOL, bk + ATOL, bv + ATOL


def check_grads(got, ref, bounds, what):
    for g, r, bd, n in zip(got, ref, bounds, ("dq", "dk", "dv")):
        err = np.abs(g - r)
        worst = float((err / bd).max())
        assert worst <= 1.0, f"{what} {n}: error {err.max():.3g}, {worst:.3g} of its bound"
    return [float(np.abs(g - r).max()) for g, r in zip(got, ref)]


def run_case(B, Lq, H, n_k, idx, n_sel, seed, what):
    q, do = bf((B, Lq, H, 128), "q", seed), bf((B, Lq, H, 128), "do", seed)
    k, v = bf((B, n_k, 128), "k", seed), bf((B, n_k, 128), "v", seed)
    o, lse = L.lsa_sparse_attn_prefill(q, k, v, idx, n_sel, want_lse=True)
    dq, dk, dv = L.lsa_sparse_attn_backward(q, k, v, idx, n_sel, o, lse, do)
    dq2, dk2, dv2 = L.lsa_sparse_attn_backward(q, k, v, idx, n_sel, o, lse, do)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), f"{what}: not deterministic"
    In, Nn = np_(idx), np_(n_sel)
    qf, kf, vf, dof = f64(q), f64(k), f64(v), f64(do)
    gq, gk, gv = f64(dq), f64(dk), f64(dv)
    errs = []
    for b in range(B):
        lists = [In[b, t, : Nn[b, t]] for t in range(Lq)]
        ref = O.sparse_attn_backward(qf[b], kf[b], vf[b], lists, 128 ** -0.5, dof[b])
        bounds = grad_bounds(qf[b], kf[b], vf[b], lists, 128 ** -0.5, dof[b])
        errs.append(check_grads((gq[b], gk[b], gv[b]), ref, bounds, f"{what} b{b}"))
    say(f"  {what}: max-abs dq/dk/dv {np.max(errs, axis=0)}")


def random_lists(B, Lq, K_tot, n_k, seed, empty_rows=()):
    rng = np.random.default_rng(seed)
    idx = np.full((B, Lq, K_tot), -1, dtype=np.int32)
    n_sel = np.zeros((B, Lq), dtype=np.int32)
    for b in range(B):
        for t in range(Lq):
            if t in empty_rows:
                continue
            n = min(t + 1, K_tot, n_k)
            idx[b, t, :n] = np.sort(rng.choice(min(t + 1, n_k), n, replace=False))
            n_sel[b, t] = n
    return torch.tensor(idx, device=DEV), torch.tensor(n_sel, device=DEV)


@pytest.mark.parametrize("H", [32, 64, 128])
def test_backward_random_lists(H):
    B, Lq, K_tot = 2, 257, 150
    say(f"backward random lists H={H}")
    idx, n_sel = random_lists(B, Lq, K_tot, Lq, 40 + H, empty_rows=(7, 100))
    run_case(B, Lq, H, Lq, idx, n_sel, H, f"random H={H}")


def test_backward_dense_causal_budget():
    # K_tot >= L: every row attends to all of 0..t
    B, Lq, H = 1, 200, 64
    idx, n_sel = random_lists(B, Lq, 256, Lq, 5)
    run_case(B, Lq, H, Lq, idx, n_sel, 7, "dense causal")


def test_backward_on_selected_lists_with_window():
    """A training step of the whole path on a small prefill: fused indexer +
    top-k selection (sinks, window, top-k), forward with lse, backward."""
    B, Lq, H, H_I, d_I = 1, 1500, 64, 64, 128
    g = lambda *s: synth.int8_uniform(*s[:3], synth.seed_of("bwd-i", s[3]), DEV)  # noqa: E731
    q_idx, k_idx = g((B, Lq, H_I, d_I), -16, 15, 1), g((B, Lq, d_I), -16, 15, 2)
    w = synth.int_weights(H_I, 1, 8, 3)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, 4, 64, 188, q_off=0)
    run_case(B, Lq, H, Lq, idx, n_sel, 11, "selected lists")
