"""GPU parity of every C-ABI entry point against the CPU oracle.

Shapes span several MFMA / selection tiles with ragged tails. Indices must
match bit-exactly; attention outputs must be within max-abs 1e-2 and
mean-abs 1e-3 of the float64 oracle. Every call also runs twice and must be
bit-identical (determinism).
"""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_lsa_amd import _lib as L
from long_context_sparse_lsa_amd import configs, synth
from tests._util import AttnErrors, assert_attn_close, f64, need_gpu, np_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    L.load()


def i8(shape, lo, hi, *seed):
    return synth.int8_uniform(shape, lo, hi, synth.seed_of("parity", *seed), DEV)


def bf(shape, *seed):
    return synth.bf16_normal(shape, synth.seed_of("parity", *seed), DEV)


def weights(H_I, d_I, seed, lo=None, hi=None):
    wmax = max(1, ((1 << 31) - 1) // (d_I * 16384 * H_I))
    lo = -wmax if lo is None else lo
    hi = wmax if hi is None else hi
    return synth.int_weights(H_I, lo, hi, synth.seed_of("parity-w", seed))


def check_idx(idx_row, n_sel, ref, K_tot, what):
    got = np.asarray(idx_row)
    assert n_sel == len(ref), f"{what}: n_sel {n_sel} != {len(ref)}"
    assert np.array_equal(got[:n_sel], ref), f"{what}: idx differs"
    assert np.all(got[n_sel:K_tot] == -1), f"{what}: padding"


# ------------------------------------------------------------------ indexer
@pytest.mark.parametrize("H_I,d_I", [(4, 64), (8, 128), (16, 64), (32, 128), (64, 128), (64, 64), (128, 128)])
def test_index_score_exact(H_I, d_I):
    B, n_q, n_k = 2, 37, 333
    say(f"index_score H_I={H_I} d_I={d_I}")
    q = i8((B, n_q, H_I, d_I), -128, 127, "q", H_I, d_I)
    k = i8((B, n_k, d_I), -128, 127, "k", H_I, d_I)
    w = weights(H_I, d_I, (H_I, d_I))
    S = L.lsa_index_score(q, k, w, q_off=n_k - n_q)
    S2 = L.lsa_index_score(q, k, w, q_off=n_k - n_q)
    torch.cuda.synchronize()
    assert torch.equal(S, S2)
    for b in range(B):
        ref = O.index_scores(np_(q[b]), np_(k[b]), w, q_off=n_k - n_q)
        assert np.array_equal(np_(S[b]), ref)


@pytest.mark.parametrize("H_I,d_I", [(64, 128), (32, 64)])
def test_index_score_mixed_fold(H_I, d_I):
    """Positive weights with small q fold into the int8 operand; rows with a
    large q value cannot, and take the weighted epilogue. Both must be exact."""
    say(f"index_score mixed fold H_I={H_I} d_I={d_I}")
    B, n_q, n_k = 2, 45, 700
    q = i8((B, n_q, H_I, d_I), -16, 15, "mq", H_I, d_I)
    q[0, 3, 5, 7] = 100          # this wave cannot fold (8 * 100 > 127)
    q[1, 40, 0, 0] = -128
    k = i8((B, n_k, d_I), -128, 127, "mk", H_I, d_I)
    w = synth.int_weights(H_I, 1, 8, 13)
    S = L.lsa_index_score(q, k, w, q_off=n_k - n_q)
    torch.cuda.synchronize()
    for b in range(B):
        assert np.array_equal(np_(S[b]), O.index_scores(np_(q[b]), np_(k[b]), w, q_off=n_k - n_q))


def test_index_score_decode_and_full_causal():
    say("index_score decode / causal")
    B, H_I, d_I, n_k = 3, 64, 128, 5000
    q = i8((B, 1, H_I, d_I), -16, 15, "qd")
    k = i8((B, n_k, d_I), -16, 15, "kd")
    w = synth.int_weights(H_I, 1, 8, 5)
    S = L.lsa_index_score(q, k, w, q_off=n_k - 1)
    for b in range(B):
        assert np.array_equal(np_(S[b]), O.index_scores(np_(q[b]), np_(k[b]), w, q_off=n_k - 1))
    # full causal square from position 0 (upper triangle masked)
    q = i8((1, 200, 8, 64), -128, 127, "qc")
    k = i8((1, 200, 64), -128, 127, "kc")
    w = weights(8, 64, "c")
    S = L.lsa_index_score(q, k, w, q_off=0)
    assert np.array_equal(np_(S[0]), O.index_scores(np_(q[0]), np_(k[0]), w, q_off=0))


# ------------------------------------------------------------------ selection
@pytest.mark.parametrize("n_k,hi", [(20000, 50), (70000, 50), (70000, 1 << 24)])
@pytest.mark.parametrize("cfg", [(4, 64, 300), (0, 0, 50), (4, 0, 1000), (1, 16, 0), (4, 512, 9000),
                                 (4, 512, 1532)])
def test_select_given_scores_ties_and_chunks(cfg, n_k, hi):
    """20000 candidates fit one chunk; 70000 take the two-stage path. Scores
    drawn from [0, 50) tie heavily; from [0, 2^24) they need several digits."""
    n_sink, W, kd = cfg
    say(f"select scores-given cfg={cfg} n_k={n_k} hi={hi}")
    B, n_q = 2, 3
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    scores = torch.randint(0, hi, (B, n_q, n_k), dtype=torch.int32, generator=g, device=DEV)
    q_off = n_k - n_q
    idx, n_sel = L.lsa_select_topk(scores=scores, n_sink=n_sink, n_window=W, k_dyn=kd, q_off=q_off)
    idx2, n_sel2 = L.lsa_select_topk(scores=scores, n_sink=n_sink, n_window=W, k_dyn=kd, q_off=q_off)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2)
    Sn, In, Nn = np_(scores), np_(idx), np_(n_sel)
    K_tot = n_sink + W + kd
    for b in range(B):
        for i in range(n_q):
            ref = O.select_flat(Sn[b, i], q_off + i, n_sink, W, kd)
            check_idx(In[b, i], Nn[b, i], ref, K_tot, f"b{b} i{i}")


@pytest.mark.parametrize("n_k,kd,hi", [(600000, 2048, 1 << 24), (1 << 20, 2048, 50), (1 << 20, 2048, 1 << 24),
                                       (290000, 9000, 1 << 24)])
def test_select_three_levels(n_k, kd, hi):
    """Rows whose chunk survivors exceed one reduction pass (more than 16
    chunks of 32768 keys at k_dyn = 2048) go through the middle stage: given
    scores at up to 1M candidates, with heavy ties, against the oracle."""
    say(f"select three levels n_k={n_k} k_dyn={kd} hi={hi}")
    B, n_q, n_sink, W = 1, 2, 4, 512
    g = torch.Generator(device=DEV)
    g.manual_seed(n_k + kd)
    scores = torch.randint(0, hi, (B, n_q, n_k), dtype=torch.int32, generator=g, device=DEV)
    q_off = n_k - n_q
    idx, n_sel = L.lsa_select_topk(scores=scores, n_sink=n_sink, n_window=W, k_dyn=kd, q_off=q_off)
    idx2, n_sel2 = L.lsa_select_topk(scores=scores, n_sink=n_sink, n_window=W, k_dyn=kd, q_off=q_off)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2)
    Sn, In, Nn = np_(scores), np_(idx), np_(n_sel)
    for i in range(n_q):
        ref = O.select_flat(Sn[0, i], q_off + i, n_sink, W, kd)
        check_idx(In[0, i], Nn[0, i], ref, n_sink + W + kd, f"row {i}")


def test_fused_select_decode_1m_flat():
    """Flat decode selection (scored and selected by one call) over a 1M-key
    cache: the middle stage in the fused path, against the oracle."""
    B, n_k, H_I, d_I = 2, 1 << 20, 64, 128
    say("fused flat decode selection at 1M keys")
    q_idx = i8((B, 1, H_I, d_I), -16, 15, "m1q")
    k_idx = i8((B, n_k, d_I), -16, 15, "m1k")
    w = synth.int_weights(H_I, 1, 8, 91)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, 4, 512, 2048, q_off=n_k - 1)
    torch.cuda.synchronize()
    for b in range(B):
        ref = O.decode_select(np_(q_idx[b, 0]), np_(k_idx[b]), w, 4, 512, 2048)
        check_idx(np_(idx[b, 0]), int(n_sel[b, 0]), ref, 4 + 512 + 2048, f"b{b}")


@pytest.mark.parametrize("n_q,n_k", [(720, 41000), (2100, 10000)])
@pytest.mark.parametrize("hi", [50, 1 << 24])
def test_select_many_long_rows_half_chunks(hi, n_q, n_k):
    """Launches with many rows that take the 512-thread chunk geometry: rows
    longer than one 1024-thread chunk (two-stage), and rows of at most 16384
    candidates (one chunk). Sampled rows against the oracle, including the
    first and last rows and rows with heavy ties."""
    say(f"select many long rows hi={hi} n_q={n_q} n_k={n_k}")
    n_sink, W, kd = 4, 1024, 1020
    g = torch.Generator(device=DEV)
    g.manual_seed(83)
    scores = torch.randint(0, hi, (1, n_q, n_k), dtype=torch.int32, generator=g, device=DEV)
    q_off = n_k - n_q
    idx, n_sel = L.lsa_select_topk(scores=scores, n_sink=n_sink, n_window=W, k_dyn=kd, q_off=q_off)
    torch.cuda.synchronize()
    Sn, In, Nn = np_(scores), np_(idx), np_(n_sel)
    K_tot = n_sink + W + kd
    rng = np.random.default_rng(7)
    for i in sorted({0, 1, n_q - 1, *rng.integers(0, n_q, 10).tolist()}):
        ref = O.select_flat(Sn[0, i], q_off + i, n_sink, W, kd)
        check_idx(In[0, i], Nn[0, i], ref, K_tot, f"row {i}")


@pytest.mark.parametrize("n_k", [20000, 70000])
def test_select_structured_rows(n_k):
    """Structured rows: every 8th candidate scores low (or only those score
    high), and a row whose threshold value is shared by thousands of ties.
    Selection must stay exact on one chunk and across chunks."""
    say(f"select structured rows n_k={n_k}")
    n_sink, W, kd = 4, 512, 1532
    n_q = 3
    g = torch.Generator(device=DEV)
    g.manual_seed(79)
    pos = torch.arange(n_k, device=DEV)
    high = torch.randint(1 << 20, 1 << 24, (n_k,), dtype=torch.int32, generator=g, device=DEV)
    low = torch.randint(0, 1000, (n_k,), dtype=torch.int32, generator=g, device=DEV)
    # row 0: every candidate whose offset from the first one is a multiple of 8 scores low
    r0 = torch.where((pos - n_sink) % 8 == 0, low, high)
    # row 1: kd - 10 large scores, then 6000 ties at one value, the rest low
    r1 = low.clone()
    r1[torch.randperm(n_k - W - n_sink, generator=g, device=DEV)[:kd - 10] + n_sink] = 1 << 23
    tie = torch.randperm(n_k - W - n_sink, generator=g, device=DEV)[:6000] + n_sink
    r1[tie] = torch.where(r1[tie] == (1 << 23), r1[tie], torch.full_like(r1[tie], 5000))
    # row 2: only the sampled candidates score high
    r2 = torch.where((pos - n_sink) % 8 == 0, high, low)
    scores = torch.stack([r0, r1, r2])[None].contiguous()
    q_off = n_k - n_q
    idx, n_sel = L.lsa_select_topk(scores=scores, n_sink=n_sink, n_window=W, k_dyn=kd, q_off=q_off)
    Sn, In, Nn = np_(scores), np_(idx), np_(n_sel)
    for i in range(n_q):
        ref = O.select_flat(Sn[0, i], q_off + i, n_sink, W, kd)
        check_idx(In[0, i], Nn[0, i], ref, n_sink + W + kd, f"row {i}")


def test_select_given_scores_short_rows():
    say("select short rows")
    n = 300
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    scores = torch.randint(-1000, 1000, (1, n, n), dtype=torch.int32, generator=g, device=DEV)
    idx, n_sel = L.lsa_select_topk(scores=scores, n_sink=4, n_window=64, k_dyn=188, q_off=0)
    Sn, In, Nn = np_(scores), np_(idx), np_(n_sel)
    for t in range(n):
        check_idx(In[0, t], Nn[0, t], O.select_flat(Sn[0, t], t, 4, 64, 188), 256, f"t{t}")


def test_fused_select_c1_full():
    wl = configs.C1
    say("fused select C1 full")
    q_idx, k_idx, w = synth.indexer_inputs(wl, DEV)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
    idx2, _ = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    qn, kn, In, Nn = np_(q_idx[0]), np_(k_idx[0]), np_(idx[0]), np_(n_sel[0])
    for r0 in range(0, wl.L, 512):
        S = O.index_scores(qn[r0:r0 + 512], kn, w, q_off=r0)
        for i in range(S.shape[0]):
            t = r0 + i
            check_idx(In[t], Nn[t], O.select_flat(S[i], t, wl.n_sink, wl.n_window, wl.k_dyn), wl.K_tot, f"t{t}")


def test_fused_select_multichunk_matches_unfused_and_oracle():
    say("fused select 9000 x H_I 64")
    wl = configs.C2
    Lq = 9000
    q_idx, k_idx, w = synth.indexer_inputs(wl, DEV, L=Lq)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
    S = L.lsa_index_score(q_idx, k_idx, w, q_off=0)
    idx_u, n_sel_u = L.lsa_select_topk(scores=S, n_sink=wl.n_sink, n_window=wl.n_window, k_dyn=wl.k_dyn, q_off=0)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_u) and torch.equal(n_sel, n_sel_u)
    del S
    qn, kn, In, Nn = np_(q_idx[0]), np_(k_idx[0]), np_(idx[0]), np_(n_sel[0])
    rows = [0, 1, 2046, 2047, 2048, 2049, 5000, 8700, 8707, 8708, 8709, 8998, 8999]
    for t in rows:
        S_t = O.index_scores(qn[t:t + 1], kn[: t + 1], w, q_off=t)[0]
        check_idx(In[t], Nn[t], O.select_flat(S_t, t, wl.n_sink, wl.n_window, wl.k_dyn), wl.K_tot, f"t{t}")


@pytest.mark.parametrize("B,n_q", [(5, 1), (3, 4)])
def test_fused_select_decode_batch(B, n_q):
    """Several short sequences scored and selected in one pass (decode)."""
    say(f"fused select decode B={B} n_q={n_q}")
    n_k, H_I, d_I = 12000, 64, 128
    q = i8((B, n_q, H_I, d_I), -16, 15, "fdq", B, n_q)
    k = i8((B, n_k, d_I), -16, 15, "fdk", B, n_q)
    w = synth.int_weights(H_I, 1, 8, 11)
    q_off = n_k - n_q
    idx, n_sel = L.lsa_select_topk(q, k, w, 4, 512, 2048, q_off=q_off)
    torch.cuda.synchronize()
    In, Nn = np_(idx), np_(n_sel)
    for b in range(B):
        S = O.index_scores(np_(q[b]), np_(k[b]), w, q_off=q_off)
        for i in range(n_q):
            ref = O.select_flat(S[i], q_off + i, 4, 512, 2048)
            check_idx(In[b, i], Nn[b, i], ref, 4 + 512 + 2048, f"b{b} i{i}")


@pytest.mark.parametrize("n_q,H_I", [(1, 64), (4, 64), (2, 32), (1, 128)])
def test_fused_select_ragged_batch(n_q, H_I):
    """A decode batch whose sequences hold different numbers of keys: every row
    matches the oracle at its own position, and the batch equals one
    lsa_select_topk call per sequence on that sequence's keys alone. Lengths
    cover rows that keep every key, a length of 0 and one past the capacity
    (both clamped)."""
    say(f"fused select ragged n_q={n_q} H_I={H_I}")
    n_k, d_I = 9000, 128
    ns, W, kd = 4, 64, 500
    K_tot = ns + W + kd
    lens = [0, 300, K_tot, K_tot + 1, 2000, 5123, n_k, n_k + 77]
    B = len(lens)
    q = i8((B, n_q, H_I, d_I), -16, 15, "rgq", n_q, H_I)
    k = i8((B, n_k, d_I), -16, 15, "rgk", n_q, H_I)
    w = synth.int_weights(H_I, 1, 8, 13)
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx, n_sel = L.lsa_select_topk_ragged(q, k, w, ctx, ns, W, kd)
    idx2, n_sel2 = L.lsa_select_topk_ragged(q, k, w, ctx, ns, W, kd)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2)
    In, Nn = np_(idx), np_(n_sel)
    for b, ln in enumerate(lens):
        Lb = min(max(ln, n_q), n_k)
        kb = k[b:b + 1, :Lb].contiguous()
        ref_i, ref_n = L.lsa_select_topk(q[b:b + 1].contiguous(), kb, w, ns, W, kd, q_off=Lb - n_q)
        assert torch.equal(ref_i[0], idx[b]) and torch.equal(ref_n[0], n_sel[b]), f"b{b} len {ln}"
        S = O.index_scores(np_(q[b]), np_(kb[0]), w, q_off=Lb - n_q)
        for i in range(n_q):
            ref = O.select_flat(S[i], Lb - n_q + i, ns, W, kd)
            check_idx(In[b, i], Nn[b, i], ref, K_tot, f"b{b} i{i}")


# ------------------------------------------------------------------ HI
@pytest.mark.parametrize("blk,d_I", [(32, 128), (64, 128), (128, 128), (256, 128), (300, 128), (1024, 128),
                                     (64, 64), (96, 64)])
def test_block_summary(blk, d_I):
    """Blocks of up to 256 rows take the 16-bit packed sums, longer ones the
    plain sums; full blocks of a power-of-two size round by shifts, partial
    tails and other sizes by division."""
    say(f"block summary blk={blk} d_I={d_I}")
    n_k = blk * 37 + 13
    k = i8((2, n_k, d_I), -128, 127, "bs", blk, d_I)
    kb = L.lsa_block_summary(k, blk)
    for b in range(2):
        assert np.array_equal(np_(kb[b]).astype(np.int64), O.block_summary(np_(k[b]), blk))
    for v in (-128, 127, -1):
        k = torch.full((1, 64 * 3, 64), v, dtype=torch.int8, device=DEV)
        assert torch.all(L.lsa_block_summary(k, 64) == v)


@pytest.mark.parametrize("blk", [64, 96])
def test_block_summary_append(blk):
    """Summaries kept current while keys are appended: after every append the
    summaries of the keys so far equal the oracle's (partial tail blocks use
    their own count) and a full lsa_block_summary of those keys; rows past the
    last block are untouched."""
    say(f"block summary append blk={blk}")
    B, n_cap, d_I = 3, 1000, 128
    k = i8((B, n_cap, d_I), -128, 127, "bsa", blk)
    nbr = -(-n_cap // blk)
    kb = torch.full((B, nbr, d_I), 77, dtype=torch.int8, device=DEV)
    n = 0
    for n_new in (1, 5, blk - 1, blk, blk + 1, 3 * blk, 3 * blk, 3 * blk + 7, 999, 1000):
        L.lsa_block_summary_append(k, kb, n, n_new, blk)
        n = n_new
        nb = -(-n // blk)
        full = L.lsa_block_summary(k[:, :n].contiguous(), blk)
        assert torch.equal(kb[:, :nb], full), f"after {n} keys"
        for b in range(B):
            assert np.array_equal(np_(kb[b, :nb]).astype(np.int64), O.block_summary(np_(k[b, :n]), blk))
        assert torch.all(kb[:, nb:] == 77)


@pytest.mark.parametrize("rec,ns,W,kd", [(32, 4, 512, 300), (8, 4, 64, 1000), (1000, 4, 128, 500), (3, 0, 0, 64)])
def test_hier_select_matches_oracle(rec, ns, W, kd):
    say(f"hier select rec={rec} ns={ns} W={W} kd={kd}")
    B, n_k, H_I, d_I, blk = 2, 20000, 64, 128, 64
    q = i8((B, H_I, d_I), -16, 15, "hq")
    k = i8((B, n_k, d_I), -16, 15, "hk")
    w = synth.int_weights(H_I, 1, 8, 9)
    kb = L.lsa_block_summary(k, blk)
    idx, n_sel = L.lsa_hier_select(q, k, kb, w, blk, rec, ns, W, kd)
    idx2, _ = L.lsa_hier_select(q, k, kb, w, blk, rec, ns, W, kd)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    In, Nn = np_(idx), np_(n_sel)
    for b in range(B):
        kn = np_(k[b])
        ref = O.hier_select(np_(q[b]), kn, O.block_summary(kn, blk), w, blk, rec, ns, W, kd)
        check_idx(In[b], Nn[b], ref, ns + W + kd, f"b{b}")
    if rec >= n_k // blk:   # every eligible block recalled: HI equals flat selection
        flat, nf = L.lsa_select_topk(q[:, None].contiguous(), k, w, ns, W, kd, q_off=n_k - 1)
        assert torch.equal(flat[:, 0], idx) and torch.equal(nf[:, 0], n_sel)


@pytest.mark.parametrize("rec", [6, 24])
def test_hier_select_ragged_batch(rec):
    """HI selection for a ragged batch: every sequence matches the oracle's HI
    selection on its own keys (query at its last key, summaries of those keys),
    and equals lsa_hier_select run on that sequence alone. Summary rows past a
    sequence's keys hold noise, which must not be read. Lengths cover sequences
    that keep every key, a length of 0 and one past the capacity (both
    clamped), and a partial last block; rec = 6 recalls fewer candidates than
    k_dyn, so lists come out short."""
    say(f"hier select ragged rec={rec}")
    n_k, d_I, H_I, blk = 12000, 128, 64, 64
    ns, W, kd = 4, 64, 500
    K_tot = ns + W + kd
    lens = [0, 300, K_tot, K_tot + 1, 2000, blk * 60 + 17, n_k, n_k + 77]
    B = len(lens)
    q = i8((B, H_I, d_I), -16, 15, "hrq", rec)
    k = i8((B, n_k, d_I), -16, 15, "hrk", rec)
    w = synth.int_weights(H_I, 1, 8, 21)
    nbk = (n_k + blk - 1) // blk
    kb = i8((B, nbk, d_I), -128, 127, "hrn", rec)
    Ls = [min(max(ln, 1), n_k) for ln in lens]
    for b, Lb in enumerate(Ls):
        kb[b, :(Lb + blk - 1) // blk] = L.lsa_block_summary(k[b:b + 1, :Lb].contiguous(), blk)[0]
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx, n_sel = L.lsa_hier_select_ragged(q, k, kb, w, ctx, blk, rec, ns, W, kd)
    idx2, n_sel2 = L.lsa_hier_select_ragged(q, k, kb, w, ctx, blk, rec, ns, W, kd)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(n_sel, n_sel2)
    In, Nn = np_(idx), np_(n_sel)
    for b, Lb in enumerate(Ls):
        kn = np_(k[b, :Lb])
        ref = O.hier_select(np_(q[b]), kn, O.block_summary(kn, blk), w, blk, rec, ns, W, kd)
        check_idx(In[b], Nn[b], ref, K_tot, f"b{b} len {lens[b]}")
        kbb = kb[b:b + 1, :(Lb + blk - 1) // blk].contiguous()
        one, n_one = L.lsa_hier_select(q[b:b + 1].contiguous(), k[b:b + 1, :Lb].contiguous(), kbb, w, blk, rec,
                                       ns, W, kd)
        assert torch.equal(one[0], idx[b]) and torch.equal(n_one[0], n_sel[b]), f"b{b} len {lens[b]}"


def test_hier_planted_block():
    say("hier planted block")
    n_k, blk = 8192, 64
    k = i8((1, n_k, 128), -2, 2, "pk")
    k[0, 40 * blk:41 * blk] = 15
    q = torch.ones((1, 8, 128), dtype=torch.int8, device=DEV)
    kb = L.lsa_block_summary(k, blk)
    idx, n_sel = L.lsa_hier_select(q, k, kb, [1] * 8, blk, 1, 4, 8, 16)
    fine = np_(idx[0])[4:4 + 16]
    assert int(n_sel[0]) == 28 and np.all((fine >= 40 * blk) & (fine < 41 * blk))


def test_hier_index_reused_by_two_layers():
    """HI and CLI together: one HI selection per step, consumed unchanged by
    the decode attention of two layers (independent q, K, V per layer, 4 MTP
    rows sharing the index); the index matches the oracle and every layer's
    output matches the oracle's attention over that index; reuse equals
    recomputing the index for the second layer."""
    say("hier + CLI two layers")
    B, n_k, H_I, d_I, blk, H, n_q = 2, 12000, 64, 128, 64, 64, 4
    ns, W, kd, rec = 4, 256, 700, 24
    q_idx = i8((B, H_I, d_I), -16, 15, "hcq")
    k_idx = i8((B, n_k, d_I), -16, 15, "hck")
    w = synth.int_weights(H_I, 1, 8, 17)
    kb = L.lsa_block_summary(k_idx, blk)
    idx, n_sel = L.lsa_hier_select(q_idx, k_idx, kb, w, blk, rec, ns, W, kd)
    outs = []
    for layer in range(2):
        q = bf((B, n_q, H, 128), "hcl", layer)
        kc, vc = bf((B, n_k, 128), "hck", layer), bf((B, n_k, 128), "hcv", layer)
        outs.append((L.lsa_sparse_attn_decode(q, kc, vc, idx[:, None], n_sel[:, None], n_split=8), q, kc, vc))
    idx_re, n_sel_re = L.lsa_hier_select(q_idx, k_idx, kb, w, blk, rec, ns, W, kd)
    q, kc, vc = outs[1][1:]
    o_re = L.lsa_sparse_attn_decode(q, kc, vc, idx_re[:, None], n_sel_re[:, None], n_split=8)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_re) and torch.equal(outs[1][0], o_re)
    In, Nn = np_(idx), np_(n_sel)
    for b in range(B):
        kn = np_(k_idx[b])
        ref = O.hier_select(np_(q_idx[b]), kn, O.block_summary(kn, blk), w, blk, rec, ns, W, kd)
        check_idx(In[b], Nn[b], ref, ns + W + kd, f"b{b}")
    for layer, (o, q, kc, vc) in enumerate(outs):
        qf, kf, vf, of = f64(q), f64(kc), f64(vc), f64(o)
        err = AttnErrors(f"HI+CLI layer {layer}")
        for b in range(B):
            sel = In[b, : Nn[b]]
            for r in range(n_q):
                ref_o, _ = O.attend(qf[b, r], kf[b], vf[b], sel, 128 ** -0.5)
                err.add(of[b, r], ref_o)
        err.check()


@pytest.mark.parametrize("n_q,n_split", [(4, 8), (2, 3)])
def test_mtp_rows_with_causal_tails(n_q, n_split):
    """MTP step whose draft rows also see the drafts before them: the target's
    flat selection, extended per row by lsa_mtp_row_index, equals the oracle's
    row lists exactly; decode attention with one index per row matches the
    oracle's attention over those lists."""
    say(f"mtp rows n_q={n_q} n_split={n_split}")
    B, n_k, H_I, d_I, H = 3, 6000, 64, 128, 64
    ns, W, kd = 4, 128, 500
    n_c = n_k + n_q - 1                      # cache with the drafts' keys appended
    q_idx = i8((B, 1, H_I, d_I), -16, 15, "mq", n_q)
    k_idx = i8((B, n_k, d_I), -16, 15, "mk", n_q)
    w = synth.int_weights(H_I, 1, 8, 19)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, ns, W, kd, q_off=n_k - 1)
    tgt = torch.full((B,), n_k - 1, dtype=torch.int32, device=DEV)
    rows, n_rows = L.lsa_mtp_row_index(idx[:, 0].contiguous(), n_sel[:, 0].contiguous(), tgt, n_q)
    q = bf((B, n_q, H, 128), "mtq", n_q)
    kc, vc = bf((B, n_c, 128), "mtk", n_q), bf((B, n_c, 128), "mtv", n_q)
    o = L.lsa_sparse_attn_decode(q, kc, vc, rows, n_rows, n_split=n_split)
    # the same rows without per-row lists: the shared list plus each row's tail
    o2, lse2 = L.lsa_sparse_attn_decode_mtp(q, kc, vc, idx, n_sel, tgt, n_split=n_split, want_lse=True)
    o3, lse3 = L.lsa_sparse_attn_decode_mtp(q, kc, vc, idx, n_sel, tgt, n_split=n_split, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(lse2, lse3)
    Rn, Nn, In, Sn = np_(rows), np_(n_rows), np_(idx), np_(n_sel)
    qf, kf, vf, of, of2, lf2 = f64(q), f64(kc), f64(vc), f64(o), f64(o2), np_(lse2)
    err = AttnErrors(f"mtp rows n_q={n_q}")
    err2 = AttnErrors(f"mtp shared list n_q={n_q}")
    for b in range(B):
        ref_sel = O.decode_select(np_(q_idx[b, 0]), np_(k_idx[b]), w, ns, W, kd)
        assert np.array_equal(In[b, 0, : Sn[b, 0]], ref_sel)
        for j, ref in enumerate(O.mtp_row_lists(ref_sel, n_k - 1, n_q)):
            check_idx(Rn[b, j], Nn[b, j], ref, ns + W + kd + n_q - 1, f"b{b} row {j}")
            ref_o, ref_l = O.attend(qf[b, j], kf[b], vf[b], ref, 128 ** -0.5)
            err.add(of[b, j], ref_o)
            err2.add(of2[b, j], ref_o)
            assert np.abs(lf2[b, j] - ref_l).max() < 1e-3
    err.check()
    err2.check()


@pytest.mark.parametrize("n_split", [8, 3])
def test_mtp_short_lists(n_split):
    """MTP rows with causal tails on lists shorter than the split count (empty
    parts), including an empty target list: the target row then attends to
    nothing (o = 0, lse = -inf) and draft row j to the j drafts alone."""
    B, n_q, H, n_k = 4, 4, 64, 400
    lens, tgts = [0, 5, 49, 1], [10, 30, 200, 0]
    K_tot = 64
    rng = np.random.default_rng(77)
    idx = np.full((B, 1, K_tot), -1, dtype=np.int32)
    for b in range(B):
        idx[b, 0, : lens[b]] = np.sort(rng.choice(tgts[b] + 1, lens[b], replace=False))
    idx_d = torch.tensor(idx, device=DEV)
    n_sel = torch.tensor(np.array(lens, dtype=np.int32)[:, None], device=DEV)
    tgt = torch.tensor(np.array(tgts, dtype=np.int32), device=DEV)
    say(f"mtp short lists n_split={n_split} lens={lens}")
    q = bf((B, n_q, H, 128), "msq", n_split)
    kc, vc = bf((B, n_k, 128), "msk", n_split), bf((B, n_k, 128), "msv", n_split)
    o, lse = L.lsa_sparse_attn_decode_mtp(q, kc, vc, idx_d, n_sel, tgt, n_split=n_split, want_lse=True)
    o2, lse2 = L.lsa_sparse_attn_decode_mtp(q, kc, vc, idx_d, n_sel, tgt, n_split=n_split, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    qf, kf, vf, of, lf = f64(q), f64(kc), f64(vc), f64(o), np_(lse)
    assert np.all(np.isfinite(of)), "non-finite output"
    err = AttnErrors(f"mtp short lists n_split={n_split}")
    for b in range(B):
        for j, ref in enumerate(O.mtp_row_lists(idx[b, 0, : lens[b]], tgts[b], n_q)):
            if len(ref) == 0:
                assert np.all(of[b, j] == 0) and np.all(np.isneginf(lf[b, j])), f"b{b} row {j}"
                continue
            ref_o, ref_l = O.attend(qf[b, j], kf[b], vf[b], ref, 128 ** -0.5)
            err.add(of[b, j], ref_o)
            assert np.abs(lf[b, j] - ref_l).max() < 1e-3, f"b{b} row {j} lse"
    err.check()


# ------------------------------------------------------------------ attention
def random_index(B, rows, K_tot, t_of_row, n_k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((B, rows, K_tot), -1, dtype=np.int32)
    n_sel = np.zeros((B, rows), dtype=np.int32)
    for b in range(B):
        for r in range(rows):
            t = t_of_row(r)
            n = min(t + 1, K_tot)
            sel = np.sort(rng.choice(t + 1, n, replace=False))
            idx[b, r, :n] = sel
            n_sel[b, r] = n
    return idx, n_sel


@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_prefill_attention(H):
    say(f"prefill attention H={H}")
    B, Lq, K_tot = 2, 333, 96
    q = bf((B, Lq, H, 128), "pq", H)
    k = bf((B, Lq, 128), "pk", H)
    v = bf((B, Lq, 128), "pv", H)
    idx, n_sel = random_index(B, Lq, K_tot, lambda r: r, Lq, H)
    idx[1, 200, 7] = Lq + 5          # out-of-range entry: skipped by the kernel
    idx_t, ns_t = torch.from_numpy(idx).to(DEV), torch.from_numpy(n_sel).to(DEV)
    o, lse = L.lsa_sparse_attn_prefill(q, k, v, idx_t, ns_t, want_lse=True)
    o2, lse2 = L.lsa_sparse_attn_prefill(q, k, v, idx_t, ns_t, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    qf, kf, vf, of, lf = f64(q), f64(k), f64(v), f64(o), np_(lse)
    scale = 128 ** -0.5
    for b in range(B):
        ref_o = np.zeros((Lq, H, 128))
        ref_l = np.zeros((Lq, H))
        for t in range(Lq):
            sel = idx[b, t, : n_sel[b, t]]
            sel = sel[(sel >= 0) & (sel < Lq)]
            ref_o[t], ref_l[t] = O.attend(qf[b, t], kf[b], vf[b], sel, scale)
        assert_attn_close(of[b], ref_o, f"o b{b}")
        assert np.abs(lf[b] - ref_l).max() < 1e-3


@pytest.mark.parametrize("H,Lq", [(64, 300), (128, 300), (64, 301)])
def test_prefill_attention_windows(H, Lq):
    """Lists that end in runs of consecutive positions (SI windows) of many
    lengths, where neighbouring rows' runs are shifted by one position, equal,
    far apart, shorter than two blocks, or not a whole number of blocks; the
    two rows of a workgroup attend a shared run once. Every row against the
    oracle, and bit-identical repeats."""
    say(f"prefill attention windows H={H} Lq={Lq}")
    B, n_k, K_tot = 2, 5000, 700
    q = bf((B, Lq, H, 128), "wq", H)
    k = bf((B, n_k, 128), "wk", H)
    v = bf((B, n_k, 128), "wv", H)
    rng = np.random.default_rng(H + 1)
    idx = np.full((B, Lq, K_tot), -1, dtype=np.int32)
    n_sel = np.zeros((B, Lq), dtype=np.int32)
    for b in range(B):
        for t in range(Lq):
            kind = (t // 2) % 6
            W = [512, 300, 96, 64, 40, 600][kind]
            end = 3000 + t + (0 if kind != 2 else 700 * (t % 2))   # kind 2: the two rows' runs far apart
            if kind == 5 and t % 2:
                end -= 1                                          # equal runs in both rows
            win = np.arange(end - W + 1, end + 1)
            n_pre = int(rng.integers(0, K_tot - W + 1))
            pre = np.sort(rng.choice(end - W - 1, n_pre, replace=False)) if n_pre else np.zeros(0, np.int64)
            sel = np.concatenate([pre, win])
            idx[b, t, : len(sel)] = sel
            n_sel[b, t] = len(sel)
    n_sel[0, 17] = 0                      # rows with nothing selected
    idx[0, 17] = -1
    n_sel[1, Lq - 1] = 0
    idx[1, Lq - 1] = -1
    idx_t, ns_t = torch.from_numpy(idx).to(DEV), torch.from_numpy(n_sel).to(DEV)
    o, lse = L.lsa_sparse_attn_prefill(q, k, v, idx_t, ns_t, want_lse=True)
    o2, lse2 = L.lsa_sparse_attn_prefill(q, k, v, idx_t, ns_t, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    qf, kf, vf, of, lf = f64(q), f64(k), f64(v), f64(o), np_(lse)
    for b in range(B):
        ref_o = np.zeros((Lq, H, 128))
        ref_l = np.full((Lq, H), -np.inf)
        for t in range(Lq):
            if n_sel[b, t] > 0:
                ref_o[t], ref_l[t] = O.attend(qf[b, t], kf[b], vf[b], idx[b, t, : n_sel[b, t]], 128 ** -0.5)
        assert_attn_close(of[b], ref_o, f"o b{b}")
        empty = n_sel[b] == 0
        assert np.all(np.isneginf(lf[b][empty])) and np.all(of[b][empty] == 0)
        assert np.abs(lf[b][~empty] - ref_l[~empty]).max() < 1e-3


@pytest.mark.parametrize("H,n_q,n_idx,n_split", [(64, 4, 1, 8), (64, 4, 4, 3), (16, 2, 1, 5), (128, 1, 1, 1),
                                                 (64, 1, 1, 64), (32, 4, 1, 2), (32, 1, 1, 8), (128, 2, 2, 16),
                                                 (64, 3, 1, 4), (16, 8, 8, 1)])
def test_decode_attention(H, n_q, n_idx, n_split):
    say(f"decode attention H={H} n_q={n_q} n_idx={n_idx} n_split={n_split}")
    B, n_k, K_tot = 3, 5000, 700
    q = bf((B, n_q, H, 128), "dq", H, n_q)
    kc = bf((B, n_k, 128), "dk", H)
    vc = bf((B, n_k, 128), "dv", H)
    rng = np.random.default_rng(n_split)
    idx = np.full((B, n_idx, K_tot), -1, dtype=np.int32)
    n_sel = np.zeros((B, n_idx), dtype=np.int32)
    for b in range(B):
        for r in range(n_idx):
            n = [700, 650, 5][b]   # the last has fewer keys than splits
            idx[b, r, :n] = np.sort(rng.choice(n_k, n, replace=False))
            n_sel[b, r] = n
    idx_t, ns_t = torch.from_numpy(idx).to(DEV), torch.from_numpy(n_sel).to(DEV)
    o, lse = L.lsa_sparse_attn_decode(q, kc, vc, idx_t, ns_t, n_split=n_split, want_lse=True)
    o2, lse2 = L.lsa_sparse_attn_decode(q, kc, vc, idx_t, ns_t, n_split=n_split, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    qf, kf, vf, of, lf = f64(q), f64(kc), f64(vc), f64(o), np_(lse)
    scale = 128 ** -0.5
    err = AttnErrors(f"decode n_split={n_split}")
    refs = {}
    for b in range(B):
        for r in range(n_q):
            sel = idx[b, 0 if n_idx == 1 else r, : n_sel[b, 0 if n_idx == 1 else r]]
            ref_o, ref_l = O.attend(qf[b, r], kf[b], vf[b], sel, scale)
            refs[b, r] = ref_o
            err.add(of[b, r], ref_o)
            assert np.abs(lf[b, r] - ref_l).max() < 1e-3
    err.check()
    if n_split > 1:   # the split count changes rounding only: n_split = 1 is in tolerance too
        o1 = f64(L.lsa_sparse_attn_decode(q, kc, vc, idx_t, ns_t, n_split=1))
        err1 = AttnErrors("decode n_split=1")
        for (b, r), ref_o in refs.items():
            err1.add(o1[b, r], ref_o)
        err1.check()


# ------------------------------------------------------------------ whole path
def test_c1_end_to_end_and_cli_reuse():
    wl = configs.C1
    say("C1 end to end")
    q_idx, k_idx, w = synth.indexer_inputs(wl, DEV)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
    outs = []
    for layer in range(2):   # two layers reuse the layer-1 index (CLI)
        q, k, v = synth.attention_inputs(wl, layer, DEV)
        outs.append((L.lsa_sparse_attn_prefill(q, k, v, idx, n_sel), q, k, v))
    # reuse equals recomputing the index
    idx_re, n_sel_re = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
    q, k, v = outs[1][1:]
    o_re = L.lsa_sparse_attn_prefill(q, k, v, idx_re, n_sel_re)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_re) and torch.equal(outs[1][0], o_re)
    In, Nn = np_(idx[0]), np_(n_sel[0])
    qn, kn = np_(q_idx[0]), np_(k_idx[0])
    rows = list(range(0, 8)) + list(range(250, 262)) + list(range(4090, 4096)) + list(range(1000, 4000, 97))
    for layer, (o, q, k, v) in enumerate(outs):
        qf, kf, vf, of = f64(q[0]), f64(k[0]), f64(v[0]), f64(o[0])
        err = AttnErrors(f"C1 layer {layer}")
        for t in rows:
            S = O.index_scores(qn[t:t + 1], kn[: t + 1], w, q_off=t)[0]
            sel = O.select_flat(S, t, wl.n_sink, wl.n_window, wl.k_dyn)
            assert np.array_equal(In[t, : Nn[t]], sel)
            ref, _ = O.attend(qf[t], kf, vf, sel, wl.scale)
            err.add(of[t], ref)
        err.check()


def test_kernel_timing_records_launches():
    """The event timing aid counts each kernel launch and reports positive
    durations; switching it off clears the records."""
    wl = configs.C1
    q_idx, k_idx, w = synth.indexer_inputs(wl, DEV)
    q, k, v = synth.attention_inputs(wl, 0, DEV)
    L.lsa_kernel_timing(True)
    try:
        idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
        for _ in range(3):
            L.lsa_sparse_attn_prefill(q, k, v, idx, n_sel)
        ms, n = L.lsa_kernel_time("attn_prefill_kernel")
        assert n == 3 and ms > 0.0
        ms, n = L.lsa_kernel_time("select_stage_a")
        assert n >= 1 and ms > 0.0
        assert L.lsa_kernel_time("no_such_kernel") == (0.0, 0)
    finally:
        L.lsa_kernel_timing(False)
    assert L.lsa_kernel_time("attn_prefill_kernel")[1] == 0


def test_decode_step_graph_replays_match_eager():
    """A decode step (selection + split-KV attention) captured as a HIP
    graph gives the eager result on every replay, with eager work and
    synchronisations of the program between the replays."""
    wl = configs.C3.scaled(B=3, L=20000)
    q_idx, k_idx, w = synth.indexer_inputs(wl, DEV)
    q, kc, vc = synth.attention_inputs(wl, 0, DEV)
    q1 = q_idx[:, None].contiguous()

    def step():
        idx, n_sel = L.lsa_select_topk(q1, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=wl.L - 1)
        return idx, L.lsa_sparse_attn_decode(q, kc, vc, idx, n_sel, n_split=wl.n_split)

    idx_e, o_e = step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        idx_g, o_g = step()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx_e), f"replay {rep}: idx"
        assert torch.equal(o_g, o_e), f"replay {rep}: o"
        step()   # eager work between replays
        torch.cuda.synchronize()
