"""Plain CPU oracle of the LongCat Sparse Attention (LSA) hot path.

TEST INFRASTRUCTURE ONLY. This module exists so that tests, the smoke check
and the benchmark's CPU-baseline leg can check the HIP kernels against an
obviously correct, slow implementation. The product path (the C-ABI library
and its Python binding) never imports, calls or falls back to it, and it
shares no code with the HIP path.

Precision: integers are exact (int64); floating point is float64.

Sources (page title, section):
  [LSA]  LongCat-2.0 release article (techsir.com, "美团大模型LongCat-2.0 正式发布"),
         section "LongCat 稀疏注意力": the indexer picks keys per query; SI mixes a
         hardware-aligned contiguous read with dynamic selection; CLI reuses
         one index across consecutive layers and across the 3 MTP draft steps;
         HI scores blocks coarsely, then tokens inside the recalled blocks.
  [SINK] "如何在 5 万张国产芯片训练出 1.6T 万亿参数模型？" (xiaored5.github.io),
         section "架构拆解 ① LSA": each query reads the top-k keys plus a few
         fixed sink tokens.
  [KVP]  same page, section "③ KVP 解码切分示意": each rank attends over its
         shard of the KV cache and the partial results are merged.

The pages leave the indexer arithmetic open. The reading used throughout:
  S[t, s] = sum_h w_h * max(0, q_I[t, h, :] . k_I[s, :])
with int8 q_I, k_I, integer per-head weights w, exact int32 result, and top-k
ties broken by score descending, then position ascending.
"""
import numpy as np

INT32_MIN = -(1 << 31)
NO_MASK = None


# ----------------------------------------------------------------------------
# a1/a2  Indexer score  ([LSA]: the lightweight indexer scores every cached key)
# ----------------------------------------------------------------------------
def index_scores(q_idx, k_idx, w, q_off=NO_MASK):
    """Indexer scores of n_q query rows against n_k keys.

    q_idx: [n_q, H_I, d_I] integers (int8 range), k_idx: [n_k, d_I], w: [H_I].
    Row i sits at position q_off + i; keys s > q_off + i are not visible and
    get INT32_MIN. q_off=None means no causal mask.

    The dot products are taken as float64 BLAS products: every product and
    every partial sum is an integer of magnitude <= d_I * 128 * 128 < 2**53,
    so any summation order is exact. ReLU, weighting and the head sum are
    then done in int64.
    """
    q = np.asarray(q_idx)
    k = np.asarray(k_idx)
    w = np.asarray(w, dtype=np.int64)
    n_q, H_I, d_I = q.shape
    n_k = k.shape[0]
    dots = q.reshape(n_q * H_I, d_I).astype(np.float64) @ k.astype(np.float64).T
    dots = np.rint(dots).astype(np.int64).reshape(n_q, H_I, n_k)
    relu = np.maximum(dots, 0)
    S = np.einsum("h,ihs->is", w, relu)
    assert np.all(np.abs(S) < (1 << 31)), "score leaves the int32 range"
    if q_off is not None:
        pos = q_off + np.arange(n_q)[:, None]
        S = np.where(np.arange(n_k)[None, :] <= pos, S, INT32_MIN)
    return S


# ----------------------------------------------------------------------------
# a3  Flat selection: sinks + SI window + dynamic top-k ([LSA] SI, [SINK])
# ----------------------------------------------------------------------------
def candidate_range(t, n_sink, n_window):
    """Positions open to the dynamic top-k for a query at t: [n_sink, t - W]."""
    return n_sink, t - n_window


def topk_by_score_then_pos(positions, scores, k):
    """The k entries with the largest score; equal scores: lower position first."""
    positions = np.asarray(positions, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.int64)
    order = np.lexsort((positions, -scores))
    return np.sort(positions[order[:k]])


def select_flat(score_row, t, n_sink, n_window, k_dyn):
    """Selected key positions of the query at position t, ascending.

    If t + 1 <= K_tot every key 0..t is kept. Otherwise: the sinks 0..n_sink-1,
    the window t-W+1..t, and the k_dyn best of the candidates n_sink..t-W.
    """
    K_tot = n_sink + n_window + k_dyn
    if t + 1 <= K_tot:
        return np.arange(t + 1, dtype=np.int64)
    lo, hi = candidate_range(t, n_sink, n_window)
    cand = np.arange(lo, hi + 1, dtype=np.int64)
    top = topk_by_score_then_pos(cand, np.asarray(score_row)[cand], k_dyn)
    return np.concatenate([np.arange(n_sink, dtype=np.int64), top,
                           np.arange(t - n_window + 1, t + 1, dtype=np.int64)])


def pad_idx(sel, K_tot):
    out = np.full(K_tot, -1, dtype=np.int64)
    out[: len(sel)] = sel
    return out


# ----------------------------------------------------------------------------
# a4  HI block summary (rule: round-half-even mean of the block's int8 keys)
# ----------------------------------------------------------------------------
def round_half_even_div(S, c):
    """Integer S / c rounded to nearest, ties to even (c > 0)."""
    S = np.asarray(S, dtype=np.int64)
    q = np.floor_divide(S, c)
    r = S - q * c
    up = (2 * r > c) | ((2 * r == c) & (q % 2 == 1))
    return q + up.astype(np.int64)


def block_summary(k_idx, blk):
    """kbar[b, :] = clamp(RNE(mean of k_idx rows b*blk .. b*blk+c-1), -128, 127)."""
    k = np.asarray(k_idx, dtype=np.int64)
    n_k, d = k.shape
    nb = -(-n_k // blk)
    out = np.empty((nb, d), dtype=np.int64)
    for b in range(nb):
        rows = k[b * blk: min(n_k, (b + 1) * blk)]
        out[b] = round_half_even_div(rows.sum(axis=0), rows.shape[0])
    return np.clip(out, -128, 127)


# ----------------------------------------------------------------------------
# a5/a6  HI: coarse block recall, then fine token top-k ([LSA] HI)
# ----------------------------------------------------------------------------
def hier_select(q_row, k_idx, kbar, w, blk, n_blk_recall, n_sink, n_window, k_dyn, t=None):
    """Selected key positions of one decode query (at t = n_k - 1 by default).

    Coarse: blocks that intersect the candidate range are scored with the
    indexer formula against their summary key; the n_blk_recall best (score
    descending, block ascending) are recalled. Fine: the candidate positions
    inside the recalled blocks are scored per token, and the best
    min(k_dyn, #candidates) are kept. Sinks and window are added as in the flat
    selection.
    """
    k_idx = np.asarray(k_idx)
    n_k = k_idx.shape[0]
    t = n_k - 1 if t is None else t
    K_tot = n_sink + n_window + k_dyn
    if t + 1 <= K_tot:
        return np.arange(t + 1, dtype=np.int64)
    lo, hi = candidate_range(t, n_sink, n_window)
    blocks = np.arange(lo // blk, hi // blk + 1, dtype=np.int64)
    bscore = index_scores(np.asarray(q_row)[None], np.asarray(kbar)[blocks], w)[0]
    recalled = topk_by_score_then_pos(blocks, bscore, n_blk_recall)
    cand = np.concatenate([np.arange(b * blk, (b + 1) * blk) for b in recalled])
    cand = cand[(cand >= lo) & (cand <= hi)]
    tscore = index_scores(np.asarray(q_row)[None], k_idx[cand], w)[0]
    fine = topk_by_score_then_pos(cand, tscore, min(k_dyn, len(cand)))
    return np.concatenate([np.arange(n_sink, dtype=np.int64), fine,
                           np.arange(t - n_window + 1, t + 1, dtype=np.int64)])


# ----------------------------------------------------------------------------
# a8/a9  Sparse attention over the gathered keys ([SINK]: attend only to the
#        selected keys), plus the split / merge of [KVP]
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def attend(q_rows, k, v, sel, scale):
    """Softmax attention of query rows over one selected key set.

    q_rows: [R, D] float64 (all rows attend over the same `sel`),
    k, v: [N, D] float64, sel: selected positions.
    Returns o [R, D] and the natural-log log-sum-exp [R].
    """
    Ks = k[sel]
    Vs = v[sel]
    z = (q_rows @ Ks.T) * scale
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ Vs) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def attend_partial(q_rows, k, v, sel, scale):
    """One split of the selected keys: (m, l, o) with o normalised by l.

    An empty split yields m = -inf, l = 0, o = 0.
    """
    R, D = q_rows.shape
    if len(sel) == 0:
        return np.full(R, -np.inf), np.zeros(R), np.zeros((R, D))
    z = (q_rows @ k[sel].T) * scale
    m = z.max(axis=1)
    p = np.exp(z - m[:, None])
    l = p.sum(axis=1)
    o = (p @ v[sel]) / l[:, None]
    return m, l, o


def merge_partials(parts):
    """Log-sum-exp merge of split partials [(m, l, o), ...].

    M = max_j m_j, Lam = sum_j l_j exp(m_j - M), o = sum_j l_j exp(m_j - M) o_j / Lam,
    lse = M + log(Lam).
    """
    m = np.stack([p[0] for p in parts])          # [J, R]
    l = np.stack([p[1] for p in parts])
    o = np.stack([p[2] for p in parts])          # [J, R, D]
    M = m.max(axis=0)
    a = np.where(l > 0, l * np.exp(m - M[None]), 0.0)
    Lam = a.sum(axis=0)
    out = (a[:, :, None] * o).sum(axis=0) / Lam[:, None]
    return out, M + np.log(Lam)


def split_ranges(n_sel, n_split):
    """Contiguous parts of ceil(n_sel / n_split) entries of the selected list."""
    cs = -(-n_sel // n_split)
    return [(min(n_sel, j * cs), min(n_sel, (j + 1) * cs)) for j in range(n_split)]


# ----------------------------------------------------------------------------
# Whole-path helpers for sampled rows
# ----------------------------------------------------------------------------
def prefill_rows(q_idx, k_idx, w, rows, n_sink, n_window, k_dyn):
    """Selections of the given prefill rows (row t sits at position t)."""
    out = {}
    for t in rows:
        S = index_scores(np.asarray(q_idx[t])[None], np.asarray(k_idx[: t + 1]), w, q_off=t)[0]
        out[int(t)] = select_flat(S, t, n_sink, n_window, k_dyn)
    return out


def decode_select(q_row, k_idx, w, n_sink, n_window, k_dyn):
    """Flat decode selection for the target query at t = n_k - 1."""
    n_k = np.asarray(k_idx).shape[0]
    S = index_scores(np.asarray(q_row)[None], k_idx, w, q_off=n_k - 1)[0]
    return select_flat(S, n_k - 1, n_sink, n_window, k_dyn)


def mtp_row_lists(sel, tgt, n_q):
    """Per-row key lists of an MTP step whose draft rows see the drafts before
    them (the causal variant of the index reuse across the MTP draft steps in
    [LSA]'s CLI paragraph): the target row, at position tgt, keeps the
    target's selection `sel` (positions <= tgt); draft row j (1 <= j < n_q),
    at tgt + j, adds the positions tgt + 1 .. tgt + j, whose keys the drafts
    appended to the cache."""
    sel = np.asarray(sel, dtype=np.int64)
    return [np.concatenate([sel, np.arange(tgt + 1, tgt + j + 1, dtype=np.int64)]) for j in range(n_q)]


# ----------------------------------------------------------------------------
# Sparse attention backward (the deterministic attention operators of the
# training write-ups: "如何在 5 万张国产芯片训练出 1.6T 万亿参数模型？", section
# "④ 痛点③", which pairs the LSA operator with deterministic attention; the
# haoling.cc article, section 三, on a deterministic attention backward)
# ----------------------------------------------------------------------------
def attend_backward(q_rows, k, v, sel, scale, do_rows):
    """Gradients of the loss sum(dO * o) for query rows attending over one
    selected key set (the chain rule through o = softmax(scale q k^T) v).

    q_rows, do_rows: [R, D]; k, v: [N, D]; sel: selected positions (unique).
    Returns dq [R, D] and the gradients of the selected rows of k and v,
    dk_sel, dv_sel [len(sel), D] (rows in the order of `sel`).
    """
    Ks = k[sel]
    Vs = v[sel]
    z = (q_rows @ Ks.T) * scale
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)          # softmax over the selected keys
    o = p @ Vs
    dp = do_rows @ Vs.T                            # d loss / d p
    delta = (do_rows * o).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)                          # d loss / d z (softmax Jacobian)
    dq = (ds @ Ks) * scale
    dk_sel = (ds.T @ q_rows) * scale
    dv_sel = p.T @ do_rows
    return dq, dk_sel, dv_sel


def sparse_attn_backward(q, k, v, lists, scale, do):
    """Backward of sparse prefill attention over one sequence.

    q, do: [L, H, D]; k, v: [N, D] (one KV head shared by the H heads);
    lists[t]: the positions row t attends to (unique). Every head of row t
    uses row t's list. Returns dq [L, H, D], dk [N, D], dv [N, D]: a key's
    gradient is the sum of the contributions of every row that selected it.
    """
    L = q.shape[0]
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for t in range(L):
        sel = np.asarray(lists[t], dtype=np.int64)
        if len(sel) == 0:
            continue
        dq[t], dks, dvs = attend_backward(q[t], k, v, sel, scale, do[t])
        dk[sel] += dks
        dv[sel] += dvs
    return dq, dk, dv


# ----------------------------------------------------------------------------
# LSA warm-up KL operator ([LSA training] release article, section
# "长上下文训练 — LSA 算子与前向优化": a KL loss operator that gives loss and
# gradient from one forward pass)
# ----------------------------------------------------------------------------
def kl_warmup_row(q_row, k, sel, scale, logits):
    """KL(p || softmax(logits)) over one row's key list and its gradient.

    q_row: [H, D] attention queries of the row; k: [N, D]; sel: the row's key
    positions; logits: [len(sel)] indexer logits of those keys. The target p
    is the attention distribution averaged over the H heads,
    p_s = (1/H) sum_h softmax_s(scale q_h . k_s). Returns (KL, d KL / d logits),
    the gradient being softmax(logits) - p.
    """
    z = (q_row @ k[sel].T) * scale                          # [H, n]
    a = np.exp(z - z.max(axis=1, keepdims=True))
    a = a / a.sum(axis=1, keepdims=True)
    p = a.mean(axis=0)
    lg = np.asarray(logits, dtype=np.float64)
    log_q = lg - (lg.max() + np.log(np.exp(lg - lg.max()).sum()))
    qd = np.exp(log_q)
    nz = p > 0
    kl = float(np.sum(p[nz] * (np.log(p[nz]) - log_q[nz])))
    return kl, qd - p
