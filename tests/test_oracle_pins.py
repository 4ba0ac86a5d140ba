"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something it does not compute itself: a
hand-worked example, a closed form, a library routine (full sort, heapq,
Fraction rounding, numpy rint, torch SDPA), brute force on tiny inputs, or an
invariant that holds for any input. The cases are built so that a plausible
slip (a dropped ReLU, a wrong sign or head weight, a transposed operand, an
off-by-one at the window or sink boundary, a reversed tie-break) fails one.
"""
import heapq
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------- O1
def test_scores_hand_worked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_worked_indexer.json")))
    q = np.array(g["q_row"])[None]
    k = np.array(g["k"])
    S = O.index_scores(q, k, np.array(g["w"]))[0]
    assert S.tolist() == g["scores_t7"]
    # the same row placed at position 3: keys 4..7 masked
    S3 = O.index_scores(q, k, np.array(g["w"]), q_off=3)[0]
    assert S3.tolist()[:4] == g["scores_t7"][:4]
    assert all(x == O.INT32_MIN for x in S3.tolist()[4:])


def test_scores_brute_force_tiny():
    for trial in range(20):
        n_q, H, d, n_k = RNG.integers(1, 5), RNG.integers(1, 4), RNG.integers(1, 9), RNG.integers(1, 12)
        q = RNG.integers(-128, 128, (n_q, H, d))
        k = RNG.integers(-128, 128, (n_k, d))
        w = RNG.integers(-5, 9, H)
        off = int(RNG.integers(0, n_k))
        S = O.index_scores(q, k, w, q_off=off)
        for i in range(n_q):
            for s in range(n_k):
                if s > off + i:
                    exp = O.INT32_MIN
                else:
                    exp = 0
                    for h in range(H):
                        dot = sum(int(q[i, h, j]) * int(k[s, j]) for j in range(d))
                        exp += int(w[h]) * max(0, dot)
                assert S[i, s] == exp


def test_scores_closed_form_constant():
    # constant q = a, k = b: S = sum_h w_h * max(0, d*a*b)
    for a, b in [(3, 5), (-3, 5), (-16, -16), (7, 0)]:
        H, d = 6, 128
        w = np.arange(1, H + 1)
        q = np.full((2, H, d), a)
        k = np.full((5, d), b)
        S = O.index_scores(q, k, w)
        assert np.all(S == w.sum() * max(0, d * a * b))


def test_scores_extreme_bound():
    # worst case of the 64-head, d=128 workloads: all -16, w = 8
    q = np.full((1, 64, 128), -16)
    k = np.full((3, 128), -16)
    S = O.index_scores(q, k, np.full(64, 8))
    assert np.all(S == 16_777_216)


def test_scores_relu_sign_and_head_weights():
    # q = -k on a single head scores 0 (ReLU), q = k scores w*|k|^2
    k = RNG.integers(-16, 16, (4, 32))
    assert np.all(O.index_scores(-k[:1][None], k[:1], [7]) == 0)
    assert O.index_scores(k[:1][None], k[:1], [7])[0, 0] == 7 * int((k[0] ** 2).sum())
    # planted heads: head h has one non-zero q dim d_h; key s has one non-zero
    # dim; distinct weights expose a wrong head->weight mapping or transpose
    H, d = 3, 5
    w = np.array([1, 10, 100])
    q = np.zeros((1, H, d), dtype=np.int64)
    q[0, 0, 1] = 2
    q[0, 1, 3] = -3
    q[0, 2, 4] = 5
    k = np.zeros((4, d), dtype=np.int64)
    k[0, 1] = 4        # head0: 8
    k[1, 3] = -1       # head1: 3*10 = 30
    k[2, 4] = -2       # head2: -10 -> relu 0
    k[3, 1] = 1
    k[3, 4] = 1        # head0: 2, head2: 5*100
    S = O.index_scores(q, k, w)[0]
    assert S.tolist() == [8, 30, 0, 2 + 500]


def test_scores_single_head_is_relu_of_dot():
    q = RNG.integers(-16, 16, (3, 1, 128))
    k = RNG.integers(-16, 16, (50, 128))
    S = O.index_scores(q, k, [1])
    ref = np.maximum(np.einsum("id,sd->is", q[:, 0].astype(np.int64), k.astype(np.int64)), 0)
    assert np.array_equal(S, ref)
    assert np.array_equal(S[0], np.maximum([int(np.dot(q[0, 0], k[s])) for s in range(50)], 0))


# ----------------------------------------------------------------------------- O2
def test_select_hand_worked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_worked_indexer.json")))
    q = np.array(g["q_row"])[None]
    k = np.array(g["k"])
    for c in g["select"]:
        S = O.index_scores(q, k, np.array(g["w"]), q_off=c["t"])[0]
        sel = O.select_flat(S, c["t"], c["n_sink"], c["n_window"], c["k_dyn"])
        assert sel.tolist() == c["idx"]


def _ref_select_sorted(S, t, n_sink, W, k):
    if t + 1 <= n_sink + W + k:
        return list(range(t + 1))
    cand = list(range(n_sink, t - W + 1))
    best = sorted(cand, key=lambda s: (-int(S[s]), s))[:k]
    return sorted(list(range(n_sink)) + best + list(range(t - W + 1, t + 1)))


def _ref_select_heap(S, t, n_sink, W, k):
    if t + 1 <= n_sink + W + k:
        return list(range(t + 1))
    cand = range(n_sink, t - W + 1)
    best = [s for (_, s) in heapq.nsmallest(k, ((-int(S[s]), s) for s in cand))]
    return sorted(list(range(n_sink)) + best + list(range(t - W + 1, t + 1)))


@pytest.mark.parametrize("trial", range(30))
def test_select_matches_full_sort_and_heap(trial):
    rng = np.random.default_rng(trial)
    n = int(rng.integers(1, 80))
    S = rng.integers(0, 6, n)  # small range: many ties
    t = n - 1
    n_sink, W, k = int(rng.integers(0, 4)), int(rng.integers(0, 6)), int(rng.integers(0, 12))
    sel = O.select_flat(S, t, n_sink, W, k).tolist()
    assert sel == _ref_select_sorted(S, t, n_sink, W, k)
    assert sel == _ref_select_heap(S, t, n_sink, W, k)


def test_select_closed_forms():
    n_sink, W, k, t = 4, 16, 10, 99
    # all scores equal: the lowest candidate positions win
    sel = O.select_flat(np.zeros(100, dtype=np.int64), t, n_sink, W, k)
    assert sel.tolist() == list(range(4)) + list(range(4, 14)) + list(range(84, 100))
    # increasing scores: the candidates closest to the window win
    sel = O.select_flat(np.arange(100), t, n_sink, W, k)
    assert sel.tolist() == list(range(4)) + list(range(74, 84)) + list(range(84, 100))
    # decreasing scores: the first candidates win
    sel = O.select_flat(-np.arange(100), t, n_sink, W, k)
    assert sel.tolist() == list(range(14)) + list(range(84, 100))
    # short rows keep every key
    for t in range(0, n_sink + W + k):
        assert O.select_flat(np.arange(100), t, n_sink, W, k).tolist() == list(range(t + 1))
    # first row past the short regime: exactly one candidate is dropped
    t = n_sink + W + k
    sel = O.select_flat(np.arange(100), t, n_sink, W, k)
    assert len(sel) == n_sink + W + k and n_sink not in sel.tolist()


def test_select_invariants_random():
    for trial in range(20):
        rng = np.random.default_rng(100 + trial)
        n = int(rng.integers(50, 400))
        n_sink, W, k = 4, int(rng.integers(0, 40)), int(rng.integers(1, 60))
        q = rng.integers(-8, 8, (1, 4, 16))
        kk = rng.integers(-8, 8, (n, 16))
        S = O.index_scores(q, kk, rng.integers(1, 5, 4), q_off=n - 1)[0]
        t = n - 1
        sel = O.select_flat(S, t, n_sink, W, k)
        K_tot = n_sink + W + k
        assert len(sel) == min(t + 1, K_tot)
        assert np.all(np.diff(sel) > 0) and sel.max() <= t and sel.min() >= 0
        if t + 1 > K_tot:
            assert set(range(n_sink)) <= set(sel.tolist())
            assert set(range(t - W + 1, t + 1)) <= set(sel.tolist())
            chosen = set(sel.tolist()) - set(range(n_sink)) - set(range(t - W + 1, t + 1))
            rest = set(range(n_sink, t - W + 1)) - chosen
            key = lambda s: (int(S[s]), -s)  # noqa: E731
            if rest:
                assert min(key(s) for s in chosen) > max(key(s) for s in rest)


# ----------------------------------------------------------------------------- O3
def test_block_summary_hand_worked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_worked_block_summary.json")))
    for c in g["cases"]:
        kb = O.block_summary(np.array(c["keys"])[:, None], g["blk"])
        assert kb.shape == (1, 1) and kb[0, 0] == c["mean"], c


def test_block_summary_library_rounding():
    rng = np.random.default_rng(7)
    k = rng.integers(-128, 128, (64 * 9 + 13, 24))
    kb = O.block_summary(k, 64)
    assert kb.shape == (10, 24)
    for b in range(10):
        rows = k[b * 64: (b + 1) * 64]
        for d in range(24):
            s, c = int(rows[:, d].sum()), rows.shape[0]
            assert kb[b, d] == max(-128, min(127, round(Fraction(s, c))))  # half-even
        if rows.shape[0] == 64:  # S/64 exact in fp64, rint is half-even
            assert np.array_equal(kb[b], np.rint(rows.sum(0) / 64.0).astype(np.int64))


# ----------------------------------------------------------------------------- O4
def test_hier_all_blocks_equals_flat():
    rng = np.random.default_rng(11)
    for trial in range(6):
        n, blk = int(rng.integers(300, 700)), 16
        q = rng.integers(-16, 16, (4, 32))
        k = rng.integers(-16, 16, (n, 32))
        w = rng.integers(1, 9, 4)
        kbar = O.block_summary(k, blk)
        n_sink, W, kd = 4, int(rng.integers(0, 50)), int(rng.integers(1, 80))
        flat = O.decode_select(q, k, w, n_sink, W, kd)
        hier = O.hier_select(q, k, kbar, w, blk, 10_000, n_sink, W, kd)
        assert np.array_equal(flat, hier)


def test_hier_planted_block_recalled_first():
    rng = np.random.default_rng(12)
    n, blk, d = 1024, 32, 16
    k = rng.integers(-2, 3, (n, d))
    q = np.ones((2, d), dtype=np.int64)
    k[10 * blk: 11 * blk] = 15          # block 10's keys align with q
    kbar = O.block_summary(k, blk)
    sel = O.hier_select(q, k, kbar, [1, 1], blk, 1, 4, 8, 16)
    fine = sel[4:-8]
    assert len(fine) == 16 and np.all((fine >= 10 * blk) & (fine < 11 * blk))
    # recalling one block yields only that block's candidates (fewer than k_dyn)
    sel = O.hier_select(q, k, kbar, [1, 1], blk, 1, 4, 8, 100)
    fine = sel[4:-8]
    assert len(fine) == blk and fine.tolist() == list(range(10 * blk, 11 * blk))


def _py_score(q_row, key, w):
    """One indexer score in Python ints (brute force)."""
    return sum(int(wh) * max(0, sum(int(a) * int(b) for a, b in zip(qh, key))) for wh, qh in zip(w, q_row))


def _hier_brute(q, k, kbar, w, blk, rec, n_sink, W, kd):
    """HI selection by enumeration: the blocks that hold at least one
    candidate position n_sink..t-W, ranked by a full sort on (-score, block);
    the candidates of the recalled blocks ranked by (-score, position)."""
    t = len(k) - 1
    if t + 1 <= n_sink + W + kd:
        return list(range(t + 1))
    cand = set(range(n_sink, t - W + 1))
    elig = sorted({s // blk for s in cand})
    ranked = sorted(elig, key=lambda b: (-_py_score(q, kbar[b], w), b))
    recalled = set(ranked[:rec])
    fine = [s for s in sorted(cand) if s // blk in recalled]
    fine = sorted(sorted(fine, key=lambda s: (-_py_score(q, k[s], w), s))[:kd])
    return list(range(n_sink)) + fine + list(range(t - W + 1, t + 1))


def test_hier_window_only_blocks_never_recalled():
    # W >= 2 * blk, so the last blocks hold window positions only; the block
    # with the best summary score is one of them and must not take a recall
    # slot (R12: only blocks that meet the candidate range compete)
    rng = np.random.default_rng(13)
    blk, d, n_sink = 16, 8, 4
    for trial in range(4):
        W = int(rng.integers(2 * blk, 4 * blk))
        n = int(rng.integers(12 * blk, 20 * blk))
        k = rng.integers(-3, 4, (n, d))
        q = rng.integers(1, 4, (2, d))
        t = n - 1
        wo = (t - W) // blk + 1 + int(rng.integers(0, (t // blk) - (t - W) // blk))  # a window-only block
        assert wo * blk > t - W and wo <= t // blk
        k[wo * blk: min(n, (wo + 1) * blk)] = 12     # aligned with q: highest summary score
        k[3 * blk: 4 * blk] = 6                      # a candidate block, second highest
        kbar = O.block_summary(k, blk)
        w = [1, 2]
        for rec, kd in ((1, 5), (1, 40), (3, 20)):
            got = O.hier_select(q, k, kbar, w, blk, rec, n_sink, W, kd)
            ref = _hier_brute(q, k, kbar, w, blk, rec, n_sink, W, kd)
            assert got.tolist() == ref, (trial, rec, kd)
            fine = got[n_sink: len(got) - W]
            assert len(fine) == min(kd, rec * blk) and np.all((fine >= n_sink) & (fine <= t - W))
            if rec == 1:   # the one recalled block is the candidate block 3
                assert np.all(fine // blk == 3)


def test_hier_random_against_enumeration():
    rng = np.random.default_rng(14)
    for trial in range(8):
        blk = int(rng.choice([8, 16]))
        n_sink, W, kd = int(rng.integers(0, 6)), int(rng.integers(0, 3 * blk)), int(rng.integers(1, 30))
        n = int(rng.integers(n_sink + W + kd + 2, 300))
        k = rng.integers(-8, 8, (n, 6))
        q = rng.integers(-8, 8, (3, 6))
        w = rng.integers(1, 5, 3)
        kbar = O.block_summary(k, blk)
        rec = int(rng.integers(1, 6))
        got = O.hier_select(q, k, kbar, w, blk, rec, n_sink, W, kd)
        assert got.tolist() == _hier_brute(q, k, kbar, w, blk, rec, n_sink, W, kd), trial


def test_hier_short_context_keeps_every_key():
    # t + 1 <= K_tot: every position 0..t, whatever the scores (R7); one more
    # key than K_tot selects again
    rng = np.random.default_rng(15)
    n_sink, W, kd, blk = 4, 20, 12, 8
    K_tot = n_sink + W + kd
    for n in (1, 2, 17, K_tot - 1, K_tot):
        k = rng.integers(-8, 8, (n, 6))
        q = rng.integers(-8, 8, (2, 6))
        got = O.hier_select(q, k, O.block_summary(k, blk), [1, 3], blk, 1, n_sink, W, kd)
        assert got.tolist() == list(range(n))
    k = rng.integers(-8, 8, (K_tot + 1, 6))
    q = rng.integers(-8, 8, (2, 6))
    got = O.hier_select(q, k, O.block_summary(k, blk), [1, 3], blk, 1, n_sink, W, kd)
    assert len(got) < K_tot + 1
    assert got.tolist() == _hier_brute(q, k, O.block_summary(k, blk), [1, 3], blk, 1, n_sink, W, kd)


# ----------------------------------------------------------------------------- O6
def _bf16_round(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def test_attention_full_budget_equals_dense_causal_sdpa():
    rng = np.random.default_rng(21)
    L, H, D = 40, 4, 16
    q = _bf16_round(rng.standard_normal((L, H, D)))
    k = _bf16_round(rng.standard_normal((L, D)))
    v = _bf16_round(rng.standard_normal((L, D)))
    scale = 1 / math.sqrt(D)
    n_sink, W, kd = 2, 5, 50    # K_tot >= L: every row keeps 0..t
    o = np.zeros((L, H, D))
    for t in range(L):
        sel = O.select_flat(np.zeros(L, dtype=np.int64), t, n_sink, W, kd)
        o[t], _ = O.attend(q[t], k, v, sel, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                # [1,H,L,D]
    kt = torch.from_numpy(k)[None, None].expand(1, H, L, D)
    vt = torch.from_numpy(v)[None, None].expand(1, H, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    assert np.allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


def test_attention_closed_forms():
    rng = np.random.default_rng(22)
    N, D = 30, 8
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    sel = np.array([0, 3, 7, 8, 20])
    # q = 0: uniform weights -> mean of the selected v, lse = log(n)
    o, lse = O.attend(np.zeros((2, D)), k, v, sel, 0.3)
    assert np.allclose(o, v[sel].mean(0)) and np.allclose(lse, math.log(len(sel)))
    # constant v -> o = v
    vc = np.tile(rng.standard_normal(D), (N, 1))
    o, _ = O.attend(rng.standard_normal((3, D)), k, vc, sel, 0.3)
    assert np.allclose(o, vc[0])
    # single key -> o = v_s, lse = scale * q.k_s
    qq = rng.standard_normal((1, D))
    o, lse = O.attend(qq, k, v, np.array([7]), 0.5)
    assert np.allclose(o[0], v[7]) and np.isclose(lse[0], 0.5 * qq[0] @ k[7])
    # two keys: closed-form softmax
    o, lse = O.attend(qq, k, v, np.array([1, 2]), 0.5)
    z1, z2 = 0.5 * qq[0] @ k[1], 0.5 * qq[0] @ k[2]
    p1 = 1 / (1 + math.exp(z2 - z1))
    assert np.allclose(o[0], p1 * v[1] + (1 - p1) * v[2])
    assert np.isclose(lse[0], math.log(math.exp(z1) + math.exp(z2)))


# ----------------------------------------------------------------------------- O7
def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(23)
    N, D, R = 200, 16, 6
    k, v = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    q = rng.standard_normal((R, D)) * 2
    sel = np.sort(rng.choice(N, 77, replace=False))
    o_ref, lse_ref = O.attend(q, k, v, sel, 0.25)
    for n_split in (1, 2, 3, 8, 77, 100):
        parts = [O.attend_partial(q, k, v, sel[a:b], 0.25) for a, b in O.split_ranges(len(sel), n_split)]
        o, lse = O.merge_partials(parts)
        assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref, atol=1e-13)
    # arbitrary uneven partitions
    cuts = sorted(rng.choice(np.arange(1, 77), 5, replace=False).tolist())
    bounds = [0] + cuts + [77]
    parts = [O.attend_partial(q, k, v, sel[a:b], 0.25) for a, b in zip(bounds[:-1], bounds[1:])]
    o, lse = O.merge_partials(parts)
    assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref, atol=1e-13)


def test_split_ranges_cover():
    for n, s in itertools.product([0, 1, 5, 2564, 2048], [1, 3, 8]):
        r = O.split_ranges(n, s)
        assert len(r) == s and r[0][0] == 0 and r[-1][1] == n
        assert all(a <= b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(s - 1))


# ---------------------------------------------------------------- KVP sharding
def test_kvp_sharded_topk_merge_is_exact():
    """Sharding the cache by position, keeping each shard's local top-k and
    merging the candidates reproduces the flat top-k exactly (the multi-GPU
    decode design); partial attention per shard + LSE merge equals unsharded."""
    rng = np.random.default_rng(31)
    n, d, H = 3000, 32, 4
    q = rng.integers(-16, 16, (H, d))
    k = rng.integers(-16, 16, (n, d))
    w = rng.integers(1, 9, H)
    n_sink, W, kd = 4, 64, 200
    t = n - 1
    S = O.index_scores(q[None], k, w, q_off=t)[0]
    flat = O.select_flat(S, t, n_sink, W, kd)
    lo, hi = n_sink, t - W
    for R in (2, 3, 8):
        edges = np.linspace(lo, hi + 1, R + 1).astype(int)
        cands = []
        for r in range(R):
            pos = np.arange(edges[r], edges[r + 1])
            cands.append(O.topk_by_score_then_pos(pos, S[pos], kd))
        c = np.concatenate(cands)
        merged = O.topk_by_score_then_pos(c, S[c], kd)
        got = np.concatenate([np.arange(n_sink), merged, np.arange(t - W + 1, t + 1)])
        assert np.array_equal(got, flat)
    qa = rng.standard_normal((8, 16))
    ka, va = rng.standard_normal((n, 16)), rng.standard_normal((n, 16))
    o_ref, lse_ref = O.attend(qa, ka, va, flat, 0.25)
    shards = np.array_split(flat, 4)
    o, lse = O.merge_partials([O.attend_partial(qa, ka, va, s, 0.25) for s in shards])
    assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref, atol=1e-13)


def test_bf16_bits_exact():
    x = torch.randn(1000).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f64(bits), x.double().numpy())


def test_mtp_row_lists_causal_tails():
    """Hand case and invariants: row j ends in the j positions after the
    target, keeps the target's list in front, stays strictly ascending, and
    its last position is its own (tgt + j); row 0 is the target's list."""
    rows = O.mtp_row_lists([0, 3, 9, 10], 10, 4)
    assert [r.tolist() for r in rows] == [[0, 3, 9, 10], [0, 3, 9, 10, 11], [0, 3, 9, 10, 11, 12],
                                          [0, 3, 9, 10, 11, 12, 13]]
    rng = np.random.default_rng(3)
    for _ in range(20):
        tgt = int(rng.integers(5, 500))
        sel = np.sort(rng.choice(tgt + 1, int(rng.integers(1, tgt + 1)), replace=False))
        n_q = int(rng.integers(1, 6))
        for j, r in enumerate(O.mtp_row_lists(sel, tgt, n_q)):
            assert len(r) == len(sel) + j and np.all(np.diff(r) > 0)
            assert np.array_equal(r[: len(sel)], sel)
            assert j == 0 or r[-1] == tgt + j


# ----------------------------------------------------------------------------- backward
def _loss(q, k, v, lists, scale, do):
    """sum(dO * o) through the oracle's forward (itself pinned to SDPA)."""
    tot = 0.0
    for t, sel in enumerate(lists):
        o, _ = O.attend(q[t], k, v, np.asarray(sel), scale)
        tot += float((do[t] * o).sum())
    return tot


def _rand_lists(rng, L, N, max_len):
    return [np.sort(rng.choice(N, int(rng.integers(1, max_len + 1)), replace=False)) for _ in range(L)]


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(21)
    L, H, D, N, scale = 5, 2, 4, 7, 0.7
    q, do = rng.standard_normal((L, H, D)), rng.standard_normal((L, H, D))
    k, v = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    lists = _rand_lists(rng, L, N, 5)
    dq, dk, dv = O.sparse_attn_backward(q, k, v, lists, scale, do)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for ix in np.ndindex(x.shape):
            x0 = x[ix]
            x[ix] = x0 + eps
            up = _loss(q, k, v, lists, scale, do)
            x[ix] = x0 - eps
            dn = _loss(q, k, v, lists, scale, do)
            x[ix] = x0
            num[ix] = (up - dn) / (2 * eps)
        assert np.abs(num - g).max() < 1e-7 * max(1.0, np.abs(g).max()), name


def _torch_grads(q, k, v, mask, scale, do):
    """float64 autograd of torch SDPA with a boolean keep-mask [L, N]; the one
    KV head is expanded over the query heads, so its gradients sum over them."""
    qt = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)        # [H, L, D]
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    H = q.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.expand(H, -1, -1), vt.expand(H, -1, -1), attn_mask=torch.tensor(mask), scale=scale)
    o.backward(torch.tensor(do.transpose(1, 0, 2)))
    return qt.grad.numpy().transpose(1, 0, 2), kt.grad.numpy(), vt.grad.numpy()


def test_backward_dense_budget_equals_torch_autograd():
    # every key 0..t selected (K_tot >= L): the sparse backward is the dense
    # causal one
    rng = np.random.default_rng(22)
    L, H, D = 40, 3, 16
    q, do = rng.standard_normal((L, H, D)), rng.standard_normal((L, H, D))
    k, v = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    lists = [np.arange(t + 1) for t in range(L)]
    got = O.sparse_attn_backward(q, k, v, lists, D ** -0.5, do)
    ref = _torch_grads(q, k, v, np.tril(np.ones((L, L), dtype=bool)), D ** -0.5, do)
    for g, r, n in zip(got, ref, "qkv"):
        assert np.abs(g - r).max() < 1e-12, n


def test_backward_sparse_lists_equal_masked_torch_autograd():
    rng = np.random.default_rng(23)
    L, H, D, N = 24, 4, 8, 50
    q, do = rng.standard_normal((L, H, D)), rng.standard_normal((L, H, D))
    k, v = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    lists = _rand_lists(rng, L, N, 12)
    mask = np.zeros((L, N), dtype=bool)
    for t, sel in enumerate(lists):
        mask[t, sel] = True
    got = O.sparse_attn_backward(q, k, v, lists, 0.3, do)
    ref = _torch_grads(q, k, v, mask, 0.3, do)
    for g, r, n in zip(got, ref, "qkv"):
        assert np.abs(g - r).max() < 1e-12, n


def test_backward_closed_forms():
    rng = np.random.default_rng(24)
    L, H, D, N = 6, 2, 8, 10
    q, do = rng.standard_normal((L, H, D)), rng.standard_normal((L, H, D))
    k, v = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    # one key per row: p = 1, so dS = 0 (dq = 0, dk = 0) and dv[s] sums dO
    lists = [np.array([t % 3]) for t in range(L)]
    dq, dk, dv = O.sparse_attn_backward(q, k, v, lists, 0.5, do)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    for s in range(3):
        rows = [t for t in range(L) if t % 3 == s]
        assert np.allclose(dv[s], do[rows].sum(axis=(0, 1)), atol=1e-12)
    assert np.all(dv[3:] == 0)
    # all keys equal: the softmax gradient rows sum to zero, so dq = 0
    kc = np.tile(rng.standard_normal(D), (N, 1))
    lists = _rand_lists(rng, L, N, N)
    dq, _, _ = O.sparse_attn_backward(q, kc, v, lists, 0.5, do)
    assert np.abs(dq).max() < 1e-12


# ----------------------------------------------------------------------------- KL operator
def _head_avg_p(q_row, k, sel, scale):
    """Target distribution from torch's softmax (a library routine)."""
    z = torch.tensor(q_row) @ torch.tensor(k[sel]).T * scale
    return torch.softmax(z, dim=-1).mean(dim=0).numpy()


def test_kl_matches_scipy_and_softmax():
    from scipy.special import rel_entr, softmax
    rng = np.random.default_rng(31)
    for trial in range(6):
        H, D, N = int(rng.integers(1, 5)), 16, 60
        k = rng.standard_normal((N, D))
        q = rng.standard_normal((H, D))
        sel = np.sort(rng.choice(N, int(rng.integers(1, 40)), replace=False))
        lg = 3 * rng.standard_normal(len(sel))
        kl, g = O.kl_warmup_row(q, k, sel, 0.25, lg)
        p = _head_avg_p(q, k, sel, 0.25)
        qd = softmax(lg)
        assert abs(kl - rel_entr(p, qd).sum()) < 1e-12
        assert np.abs(g - (qd - p)).max() < 1e-14
        assert kl >= 0 and abs(g.sum()) < 1e-12


def test_kl_closed_forms_and_finite_differences():
    from scipy.stats import entropy
    rng = np.random.default_rng(32)
    H, D, N = 3, 8, 30
    k, q = rng.standard_normal((N, D)), rng.standard_normal((H, D))
    sel = np.arange(5, 25)
    p = _head_avg_p(q, k, sel, 0.4)
    # logits = log p (+ any constant): KL = 0, gradient 0
    kl, g = O.kl_warmup_row(q, k, sel, 0.4, np.log(p) + 7.0)
    assert abs(kl) < 1e-12 and np.abs(g).max() < 1e-12
    # uniform indexer: KL = log n - entropy(p)
    kl, _ = O.kl_warmup_row(q, k, sel, 0.4, np.zeros(len(sel)))
    assert abs(kl - (np.log(len(sel)) - entropy(p))) < 1e-12
    # gradient by central differences
    lg = rng.standard_normal(len(sel))
    _, g = O.kl_warmup_row(q, k, sel, 0.4, lg)
    eps = 1e-6
    for i in range(len(sel)):
        a, b = lg.copy(), lg.copy()
        a[i] += eps
        b[i] -= eps
        num = (O.kl_warmup_row(q, k, sel, 0.4, a)[0] - O.kl_warmup_row(q, k, sel, 0.4, b)[0]) / (2 * eps)
        assert abs(num - g[i]) < 1e-8
