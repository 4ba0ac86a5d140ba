"""GPU parity of the thresholded prefill selection (lsa_select_topk, fused).

Rows with at least 16384 candidates take a threshold from an exactly scored
sample of their candidates (every 64th position), and the full scoring pass
keeps only the (score, position) pairs at or above it; the top-k of those
survivors is the row's top-k whenever they number at least k_dyn. Rows where
that cannot be shown (too few survivors, a full segment) are redone by the
dense path. Either way the lists must equal the dense selection over the full
score matrix bit for bit, on every row, and the oracle's on sampled rows.

Cases: random rows (the threshold holds), keys planted at the sampled
positions that defeat the threshold on chosen rows (those rows are redone),
identical keys (every score ties, every segment overflows, all rows redone),
a block of rows that all lie past the threshold boundary (q_off > 0), and
H_I = 32, d_I = 64.
"""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_lsa_amd import _lib as L
from long_context_sparse_lsa_amd import synth
from tests._util import need_gpu, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
NS, W, KD = 4, 512, 1020


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    L.load()


def i8(shape, lo, hi, *seed):
    return synth.int8_uniform(shape, lo, hi, synth.seed_of("filter", *seed), DEV)


def check_rows_against_dense(q_idx, k_idx, w, q_off, what, oracle_rows=(), cfg=(NS, W, KD)):
    """Fused (thresholded) lists == dense lists from the full score matrix."""
    ns, win, kd = cfg
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, ns, win, kd, q_off=q_off)
    idx2, n_sel2 = L.lsa_select_topk(q_idx, k_idx, w, ns, win, kd, q_off=q_off)
    S = L.lsa_index_score(q_idx, k_idx, w, q_off=q_off)
    ref, ref_n = L.lsa_select_topk(scores=S, n_sink=ns, n_window=win, k_dyn=kd, q_off=q_off)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2), f"{what}: not deterministic"
    bad = (idx != ref).any(dim=-1) | (n_sel != ref_n)
    assert not bool(bad.any()), f"{what}: {int(bad.sum())} rows differ from the dense selection, first " \
                                f"{np.argwhere(np_(bad))[:4].tolist()}"
    del S
    B = q_idx.shape[0]
    for b, i in oracle_rows:
        t = q_off + i
        qn, kn = np_(q_idx[b, i:i + 1]), np_(k_idx[b, : t + 1])
        s_t = O.index_scores(qn, kn, w, q_off=t)[0]
        exp = O.select_flat(s_t, t, ns, win, kd)
        assert int(n_sel[b, i]) == len(exp) and np.array_equal(np_(idx[b, i, : len(exp)]), exp), \
            f"{what}: b{b} t{t} differs from the oracle"
    say(f"  {what}: {B}x{q_idx.shape[1]} rows equal the dense selection")
    return idx, n_sel


def test_filter_random_rows_two_sequences():
    B, Lq = 2, 20480
    say(f"filter random B={B} L={Lq}")
    q = i8((B, Lq, 64, 128), -16, 15, "q")
    k = i8((B, Lq, 128), -16, 15, "k")
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 1))
    rows = [(0, 16898), (0, 16899), (1, 16900), (0, 18000), (1, 20479), (0, 20479), (1, 100)]
    check_rows_against_dense(q, k, w, 0, "random", rows)


def test_filter_planted_sample_keys_force_redo():
    """Keys at every multiple of 32 (a superset of the sampled positions) are
    made to dominate the scores of every third row: their samples then set a
    threshold that only a few times j* keys reach, fewer than k_dyn, and
    those rows are redone."""
    Lq = 20480
    say(f"filter planted L={Lq}")
    q = i8((1, Lq, 64, 128), -16, 15, "pq")
    k = i8((1, Lq, 128), -16, 15, "pk")
    k[0, ::32, :64] = 15
    hit = torch.arange(Lq, device=DEV) % 3 == 0
    q[0, hit, :, :64] = 15
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 2))
    rows = [(0, 17001), (0, 17002), (0, 19998), (0, 20001)]
    check_rows_against_dense(q, k, w, 0, "planted", rows)


def test_filter_all_ties_overflow():
    """Every key equal: every candidate ties, the threshold keeps them all,
    segments overflow and each row is redone (its list: the k lowest positions)."""
    Lq = 18432
    say(f"filter ties L={Lq}")
    q = i8((1, Lq, 64, 128), -16, 15, "tq")
    k = i8((1, 1, 128), -16, 15, "tk").expand(1, Lq, 128).contiguous()
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 3))
    idx, n_sel = check_rows_against_dense(q, k, w, 0, "ties", [(0, 18000)])
    t = Lq - 1
    exp = np.concatenate([np.arange(NS), np.arange(NS, NS + KD), np.arange(t - W + 1, t + 1)])
    assert np.array_equal(np_(idx[0, t, : int(n_sel[0, t])]), exp)


def test_filter_rows_past_boundary_with_offset():
    """A chunk of rows at the end of a longer cache: every row is past the
    16384-candidate boundary, so the pass has no dense part."""
    n_k, n_q = 24000, 5000
    say(f"filter q_off n_k={n_k} n_q={n_q}")
    q = i8((1, n_q, 64, 128), -16, 15, "oq")
    k = i8((1, n_k, 128), -16, 15, "ok")
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 4))
    check_rows_against_dense(q, k, w, n_k - n_q, "offset", [(0, 0), (0, 4999)])


def test_filter_h32_d64():
    Lq = 19000
    say(f"filter H_I=32 d_I=64 L={Lq}")
    q = i8((1, Lq, 32, 64), -128, 127, "hq")
    k = i8((1, Lq, 64), -128, 127, "hk")
    wmax = ((1 << 31) - 1) // (64 * 16384 * 32)
    w = synth.int_weights(32, -wmax, wmax, synth.seed_of("filter-w", 5))
    check_rows_against_dense(q, k, w, 0, "h32d64", [(0, 18999), (0, 17500)])


@pytest.mark.parametrize("ns,win,kd", [(0, 0, 1020), (4, 64, 4096), (1, 1, 300)])
def test_filter_budgets(ns, win, kd):
    """No sinks and no window; a large k_dyn (the widest survivor kernel); a
    small k_dyn whose sample threshold keeps several times k."""
    Lq = 20480
    say(f"filter budgets ns={ns} W={win} k={kd}")
    q = i8((1, Lq, 64, 128), -16, 15, "bq", kd)
    k = i8((1, Lq, 128), -16, 15, "bk", kd)
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 6, kd))
    rows = [(0, 16384 + win + ns), (0, Lq - 1)]
    check_rows_against_dense(q, k, w, 0, f"budget {ns}+{win}+{kd}", rows, cfg=(ns, win, kd))


def test_filter_multi_pass_rows():
    """A sequence of several dense passes (10922 rows each at 48K keys): the
    thresholded rows go in passes of two dense passes' rows where four would
    overflow the segment buffer, then of the remaining rows at once; every
    list equals the dense selection."""
    Lq = 49152
    say(f"filter multi-pass L={Lq}")
    q = i8((1, Lq, 64, 128), -16, 15, "mq")
    k = i8((1, Lq, 128), -16, 15, "mk")
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 7))
    rows = [(0, 17500), (0, 21843), (0, 32765), (0, 32766), (0, 49151)]
    check_rows_against_dense(q, k, w, 0, "multi-pass", rows)


def test_filter_multi_pass_redo():
    """Planted sample keys defeat the threshold of every third row of a
    multi-pass sequence: the failed rows of a long thresholded pass are redone
    in dense-pass pieces, each with its own part of the fail flags."""
    Lq = 49152
    say(f"filter multi-pass planted L={Lq}")
    q = i8((1, Lq, 64, 128), -16, 15, "mpq")
    k = i8((1, Lq, 128), -16, 15, "mpk")
    k[0, ::32, :64] = 15
    hit = torch.arange(Lq, device=DEV) % 3 == 0
    q[0, hit, :, :64] = 15
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 8))
    rows = [(0, 21843), (0, 21844), (0, 43689), (0, 49149)]
    check_rows_against_dense(q, k, w, 0, "multi-pass planted", rows)


def test_filter_multi_pass_two_sequences():
    """Two sequences of several dense passes each, with a chunk of rows at
    the end of a longer cache (q_off > 0): the thresholded passes of the
    second sequence start from its own rows, keys and outputs."""
    n_k, n_q = 49152, 40000
    say(f"filter multi-pass B=2 n_k={n_k} n_q={n_q}")
    q = i8((2, n_q, 64, 128), -16, 15, "m2q")
    k = i8((2, n_k, 128), -16, 15, "m2k")
    w = synth.int_weights(64, 1, 8, synth.seed_of("filter-w", 9))
    rows = [(0, 0), (1, 0), (1, 12000), (0, 25000), (1, 39999)]
    check_rows_against_dense(q, k, w, n_k - n_q, "multi-pass B=2", rows)
