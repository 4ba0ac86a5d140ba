"""ctypes binding of liblsa.so (include/lsa.h).

Argument marshalling only: each function takes torch device tensors, checks
dtypes and shapes, allocates outputs and workspace with torch, and calls the
C entry point of the same name on the current torch stream. There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsa.so")

LSA_OK, LSA_INVALID_ARG, LSA_UNSUPPORTED, LSA_WORKSPACE, LSA_RANGE, LSA_HIP, LSA_SCRATCH_LIMIT = range(7)


class LSAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class LSAUnavailable(RuntimeError):
    pass


class SelectCfg(ctypes.Structure):
    _fields_ = [("n_sink", ctypes.c_int32), ("n_window", ctypes.c_int32), ("k_dyn", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_Z = ctypes.c_size_t
_ZP = ctypes.POINTER(ctypes.c_size_t)

SIGNATURES = {
    "lsa_status_string": (ctypes.c_char_p, [_I]),
    "lsa_index_score": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "lsa_select_topk": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, SelectCfg, _P, _P, _P, _Z, _ZP, _P]),
    "lsa_select_topk_ragged": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, SelectCfg, _P, _P, _P, _Z, _ZP, _P]),
    "lsa_block_summary": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "lsa_mtp_row_index": (_I, [_P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "lsa_block_summary_append": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "lsa_hier_select": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, SelectCfg, _P, _P, _P, _Z, _ZP, _P]),
    "lsa_hier_select_ragged": (_I, [_P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, SelectCfg, _P, _P, _P, _Z, _ZP,
                                    _P]),
    "lsa_sparse_attn_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "lsa_sparse_attn_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _Z, _ZP, _P]),
    "lsa_sparse_attn_decode_mtp": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _Z, _ZP,
                                        _P]),
    "lsa_kernel_timing": (_I, [_I]),
    "lsa_kernel_time": (_I, [ctypes.c_char_p, ctypes.POINTER(_F), ctypes.POINTER(_I)]),
    "lsa_probe_mfma": (_I, [_I, _I, _I, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "lsa_probe_mfma_data": (_I, [_I, _I, _I, _P, ctypes.c_int64, _P, ctypes.c_int64, _P,
                                 ctypes.POINTER(ctypes.c_double), _P]),
    "lsa_sparse_attn_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "lsa_noalloc_scratch_bytes": (_Z, []),
    "lsa_sparse_attn_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _Z,
                                      _ZP, _P]),
    "lsa_kl_warmup": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "lsa_hier_decode_step": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, SelectCfg, _I, _I, _I, _F, _P,
                                  _P, _P, _P, _P, _Z, _ZP, _P]),
}

_lib = None


def load(path=LIB_PATH):
    """Load liblsa.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LSAUnavailable(f"{path} is missing: build it with python -m long_context_sparse_lsa_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def status_string(s):
    return load().lsa_status_string(int(s)).decode()


def _check(fn, s):
    if s != LSA_OK:
        raise LSAError(fn, s, status_string(s))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _weights(w, H_I):
    w = np.ascontiguousarray(np.asarray(w, dtype=np.int32).reshape(-1))
    if w.shape[0] != H_I:
        raise ValueError(f"w has {w.shape[0]} entries, H_I = {H_I}")
    return w, w.ctypes.data_as(ctypes.c_void_p)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
def lsa_index_score(q_idx, k_idx, w, q_off=None, out=None):
    """q_idx [B, n_q, H_I, d_I] int8, k_idx [B, n_k, d_I] int8, w [H_I] host ints.
    Returns scores [B, n_q, n_k] int32 (INT32_MIN where s > q_off + i).
    q_off defaults to n_k - n_q (the rows are the last n_q positions)."""
    lib = load()
    _dev(q_idx, torch.int8, "q_idx")
    _dev(k_idx, torch.int8, "k_idx")
    B, n_q, H_I, d_I = q_idx.shape
    n_k = k_idx.shape[1]
    if k_idx.shape != (B, n_k, d_I):
        raise ValueError("k_idx shape mismatch")
    q_off = n_k - n_q if q_off is None else int(q_off)
    wh, wp = _weights(w, H_I)
    if out is None:
        out = torch.empty((B, n_q, n_k), dtype=torch.int32, device=q_idx.device)
    _check("lsa_index_score", lib.lsa_index_score(_ptr(q_idx), _ptr(k_idx), wp, B, n_q, n_k, H_I, d_I,
                                                  q_off, _ptr(out), _stream()))
    return out


def lsa_select_topk(q_idx=None, k_idx=None, w=None, n_sink=4, n_window=0, k_dyn=0, q_off=None,
                    scores=None, n_k=None, out=None):
    """Flat selection. Either scores [B, n_q, n_k] int32 or (q_idx, k_idx, w)
    for the fused path. Returns (idx [B, n_q, K_tot] int32, n_sel [B, n_q] int32)."""
    lib = load()
    K_tot = n_sink + n_window + k_dyn
    cfg = SelectCfg(n_sink, n_window, k_dyn)
    if scores is not None:
        _dev(scores, torch.int32, "scores")
        B, n_q, n_k = scores.shape
        H_I = d_I = 0
        wp = None
        dev = scores.device
    else:
        _dev(q_idx, torch.int8, "q_idx")
        _dev(k_idx, torch.int8, "k_idx")
        B, n_q, H_I, d_I = q_idx.shape
        n_k = k_idx.shape[1]
        if k_idx.shape != (B, n_k, d_I):
            raise ValueError("k_idx shape mismatch")
        wh, wp = _weights(w, H_I)
        dev = q_idx.device
    q_off = n_k - n_q if q_off is None else int(q_off)
    need = ctypes.c_size_t(0)
    args = (_ptr(scores), _ptr(q_idx) if scores is None else None, _ptr(k_idx) if scores is None else None,
            wp, B, n_q, n_k, H_I, d_I, q_off, cfg)
    _check("lsa_select_topk", lib.lsa_select_topk(*args, None, None, None, 0, ctypes.byref(need), None))
    ws = _workspace(need.value, dev)
    if out is None:
        idx = torch.empty((B, n_q, K_tot), dtype=torch.int32, device=dev)
        n_sel = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    else:
        idx, n_sel = out
    _check("lsa_select_topk", lib.lsa_select_topk(*args, _ptr(idx), _ptr(n_sel), _ptr(ws), ws.numel(),
                                                  None, _stream()))
    return idx, n_sel


def lsa_select_topk_ragged(q_idx, k_idx, w, ctx_len, n_sink=4, n_window=0, k_dyn=0, out=None):
    """Flat selection for a ragged decode batch: sequence b holds
    clamp(ctx_len[b], n_q, n_k) keys of its cache k_idx [B, n_k, d_I], and its
    n_q rows are its last n_q positions. ctx_len [B] int32 on the device.
    Returns (idx [B, n_q, K_tot] int32, n_sel [B, n_q] int32)."""
    lib = load()
    _dev(q_idx, torch.int8, "q_idx")
    _dev(k_idx, torch.int8, "k_idx")
    _dev(ctx_len, torch.int32, "ctx_len")
    B, n_q, H_I, d_I = q_idx.shape
    n_k = k_idx.shape[1]
    if k_idx.shape != (B, n_k, d_I) or tuple(ctx_len.shape) != (B,):
        raise ValueError("k_idx / ctx_len shape mismatch")
    wh, wp = _weights(w, H_I)
    cfg = SelectCfg(n_sink, n_window, k_dyn)
    K_tot = n_sink + n_window + k_dyn
    need = ctypes.c_size_t(0)
    args = (_ptr(q_idx), _ptr(k_idx), wp, B, n_q, n_k, H_I, d_I, _ptr(ctx_len), cfg)
    _check("lsa_select_topk_ragged",
           lib.lsa_select_topk_ragged(*args, None, None, None, 0, ctypes.byref(need), None))
    ws = _workspace(need.value, q_idx.device)
    if out is None:
        idx = torch.empty((B, n_q, K_tot), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B, n_q), dtype=torch.int32, device=q_idx.device)
    else:
        idx, n_sel = out
    _check("lsa_select_topk_ragged", lib.lsa_select_topk_ragged(*args, _ptr(idx), _ptr(n_sel), _ptr(ws),
                                                                ws.numel(), None, _stream()))
    return idx, n_sel


def lsa_mtp_row_index(idx, n_sel, tgt_pos, n_q):
    """Rows of an MTP step whose drafts see the drafts before them: idx [B, K_tot],
    n_sel [B] (the target's selection), tgt_pos [B] int32 on the device.
    Returns (idx_rows [B, n_q, K_tot + n_q - 1], n_sel_rows [B, n_q]) for
    lsa_sparse_attn_decode with one index per row."""
    lib = load()
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    _dev(tgt_pos, torch.int32, "tgt_pos")
    B, K_tot = idx.shape
    idx_rows = torch.empty((B, n_q, K_tot + n_q - 1), dtype=torch.int32, device=idx.device)
    n_sel_rows = torch.empty((B, n_q), dtype=torch.int32, device=idx.device)
    _check("lsa_mtp_row_index", lib.lsa_mtp_row_index(_ptr(idx), _ptr(n_sel), B, K_tot, n_q, _ptr(tgt_pos),
                                                      _ptr(idx_rows), _ptr(n_sel_rows), _stream()))
    return idx_rows, n_sel_rows


def lsa_block_summary(k_idx, blk):
    """k_idx [B, n_k, d_I] int8 -> k_blk [B, ceil(n_k/blk), d_I] int8."""
    lib = load()
    _dev(k_idx, torch.int8, "k_idx")
    B, n_k, d_I = k_idx.shape
    nb = -(-n_k // blk)
    out = torch.empty((B, nb, d_I), dtype=torch.int8, device=k_idx.device)
    _check("lsa_block_summary", lib.lsa_block_summary(_ptr(k_idx), B, n_k, d_I, blk, _ptr(out), _stream()))
    return out


def lsa_block_summary_append(k_cache, k_blk, n_old, n_new, blk):
    """Update k_blk [B, ceil(n_cap/blk), d_I] in place after keys n_old..n_new-1
    were written to k_cache [B, n_cap, d_I]. Returns k_blk."""
    lib = load()
    _dev(k_cache, torch.int8, "k_cache")
    _dev(k_blk, torch.int8, "k_blk")
    B, n_cap, d_I = k_cache.shape
    if k_blk.shape != (B, -(-n_cap // blk), d_I):
        raise ValueError("k_blk shape mismatch")
    _check("lsa_block_summary_append", lib.lsa_block_summary_append(_ptr(k_cache), B, n_cap, int(n_old), int(n_new),
                                                                    d_I, blk, _ptr(k_blk), _stream()))
    return k_blk


def _hier(name, q_idx, k_idx, k_blk, w, ctx_len, blk, n_blk_recall, n_sink, n_window, k_dyn):
    lib = load()
    _dev(q_idx, torch.int8, "q_idx")
    _dev(k_idx, torch.int8, "k_idx")
    _dev(k_blk, torch.int8, "k_blk")
    B, H_I, d_I = q_idx.shape
    n_k = k_idx.shape[1]
    wh, wp = _weights(w, H_I)
    cfg = SelectCfg(n_sink, n_window, k_dyn)
    K_tot = n_sink + n_window + k_dyn
    need = ctypes.c_size_t(0)
    if ctx_len is None:
        args = (_ptr(q_idx), _ptr(k_idx), _ptr(k_blk), wp, B, n_k, H_I, d_I, blk, n_blk_recall, cfg)
    else:
        _dev(ctx_len, torch.int32, "ctx_len")
        if tuple(ctx_len.shape) != (B,):
            raise ValueError("ctx_len shape mismatch")
        args = (_ptr(q_idx), _ptr(k_idx), _ptr(k_blk), wp, B, n_k, _ptr(ctx_len), H_I, d_I, blk, n_blk_recall,
                cfg)
    fn = getattr(lib, name)
    _check(name, fn(*args, None, None, None, 0, ctypes.byref(need), None))
    ws = _workspace(need.value, q_idx.device)
    idx = torch.empty((B, K_tot), dtype=torch.int32, device=q_idx.device)
    n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
    _check(name, fn(*args, _ptr(idx), _ptr(n_sel), _ptr(ws), ws.numel(), None, _stream()))
    return idx, n_sel


def lsa_hier_select(q_idx, k_idx, k_blk, w, blk, n_blk_recall, n_sink, n_window, k_dyn):
    """HI decode selection for the query at n_k - 1.
    q_idx [B, H_I, d_I] int8. Returns (idx [B, K_tot], n_sel [B])."""
    return _hier("lsa_hier_select", q_idx, k_idx, k_blk, w, None, blk, n_blk_recall, n_sink, n_window, k_dyn)


def lsa_hier_select_ragged(q_idx, k_idx, k_blk, w, ctx_len, blk, n_blk_recall, n_sink, n_window, k_dyn):
    """HI decode selection for a ragged batch: sequence b holds
    clamp(ctx_len[b], 1, n_k) keys of k_idx [B, n_k, d_I] and its query sits
    at the last of them; k_blk holds each sequence's summaries of those keys.
    ctx_len [B] int32 on the device. Returns (idx [B, K_tot], n_sel [B])."""
    return _hier("lsa_hier_select_ragged", q_idx, k_idx, k_blk, w, ctx_len, blk, n_blk_recall, n_sink, n_window,
                 k_dyn)


def lsa_hier_decode_step(q_idx, k_idx, k_blk, w, q, k_cache, v_cache, blk, n_blk_recall, n_sink, n_window, k_dyn,
                         n_split=8, scale=None, want_lse=False, ws=None):
    """Fused HI decode step: q_idx [B, H_I, d_I] int8, k_idx [B, n_k, d_I],
    k_blk from lsa_block_summary, w [H_I] host ints, q [B, 1, H, D] bf16,
    caches [B, n_k, D] bf16. Returns (idx [B, K_tot], n_sel [B], o [B, 1, H, D]
    bf16[, lse [B, 1, H]]). ws: optional uint8 workspace (its first 256 bytes
    hold the step's counters; int32 word 1 flags an exceeded wait)."""
    lib = load()
    for t, n in ((q_idx, "q_idx"), (k_idx, "k_idx"), (k_blk, "k_blk")):
        _dev(t, torch.int8, n)
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, n)
    B, H_I, d_I = q_idx.shape
    n_k = k_idx.shape[1]
    _, n_q, H, D = q.shape
    if n_q != 1 or q.shape[0] != B or k_cache.shape != (B, n_k, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    wh, wp = _weights(w, H_I)
    cfg = SelectCfg(n_sink, n_window, k_dyn)
    K_tot = n_sink + n_window + k_dyn
    scale = D ** -0.5 if scale is None else float(scale)
    need = ctypes.c_size_t(0)
    args = (_ptr(q_idx), _ptr(k_idx), _ptr(k_blk), wp, _ptr(q), _ptr(k_cache), _ptr(v_cache), B, n_k, H_I, d_I, blk,
            n_blk_recall, cfg, H, D, n_split, scale)
    _check("lsa_hier_decode_step", lib.lsa_hier_decode_step(*args, None, None, None, None, None, 0,
                                                            ctypes.byref(need), None))
    if ws is None or ws.numel() < need.value:
        ws = _workspace(need.value, q.device)
    idx = torch.empty((B, K_tot), dtype=torch.int32, device=q.device)
    n_sel = torch.empty((B,), dtype=torch.int32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, 1, H), dtype=torch.float32, device=q.device) if want_lse else None
    _check("lsa_hier_decode_step", lib.lsa_hier_decode_step(*args, _ptr(idx), _ptr(n_sel), _ptr(o), _ptr(lse),
                                                            _ptr(ws), ws.numel(), None, _stream()))
    return (idx, n_sel, o, lse) if want_lse else (idx, n_sel, o)


def lsa_sparse_attn_prefill(q, k, v, idx, n_sel, scale=None, want_lse=False, out=None):
    """q [B, L, H, D] bf16, k/v [B, n_k, D] bf16, idx [B, L, K_tot] int32, n_sel [B, L].
    Returns o [B, L, H, D] bf16 (and lse [B, L, H] fp32 if want_lse)."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    B, L, H, D = q.shape
    n_k = k.shape[1]
    K_tot = idx.shape[-1]
    if idx.shape != (B, L, K_tot) or n_sel.shape != (B, L) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, L, H), dtype=torch.float32, device=q.device) if want_lse else None
    _check("lsa_sparse_attn_prefill", lib.lsa_sparse_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(n_sel), B, L, n_k, H, D, K_tot, scale,
        _ptr(o), _ptr(lse), _stream()))
    return (o, lse) if want_lse else o


def lsa_sparse_attn_decode(q, k_cache, v_cache, idx, n_sel, n_split=8, scale=None, want_lse=False, ws=None):
    """q [B, n_q, H, D] bf16; caches [B, n_k, D]; idx [B, n_idx, K_tot] (n_idx 1 or n_q).
    Returns o [B, n_q, H, D] bf16 (and lse [B, n_q, H] if want_lse)."""
    lib = load()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, n)
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    B, n_q, H, D = q.shape
    n_k = k_cache.shape[1]
    n_idx, K_tot = idx.shape[1], idx.shape[2]
    if idx.shape[0] != B or n_sel.shape != (B, n_idx):
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else float(scale)
    need = ctypes.c_size_t(0)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), _ptr(n_sel), n_idx, B, n_q, n_k, H, D, K_tot,
            n_split, scale)
    _check("lsa_sparse_attn_decode", lib.lsa_sparse_attn_decode(*args, None, None, None, 0, ctypes.byref(need),
                                                                None))
    if ws is None or ws.numel() < need.value:
        ws = _workspace(need.value, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device) if want_lse else None
    _check("lsa_sparse_attn_decode", lib.lsa_sparse_attn_decode(*args, _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                                                None, _stream()))
    return (o, lse) if want_lse else o


def lsa_sparse_attn_backward(q, k, v, idx, n_sel, o, lse, d_o, scale=None, ws=None):
    """Deterministic backward of lsa_sparse_attn_prefill: q, o, d_o [B, L, H, D]
    bf16, lse [B, L, H] fp32 (the forward's), k/v [B, n_k, D] bf16, idx
    [B, L, K_tot], n_sel [B, L]. Returns (dq bf16 like q, dk fp32, dv fp32)."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _dev(t, torch.bfloat16, n)
    _dev(lse, torch.float32, "lse")
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    B, L, H, D = q.shape
    n_k = k.shape[1]
    K_tot = idx.shape[-1]
    if (idx.shape != (B, L, K_tot) or n_sel.shape != (B, L) or v.shape != k.shape or o.shape != q.shape
            or d_o.shape != q.shape or lse.shape != (B, L, H)):
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else float(scale)
    need = ctypes.c_size_t(0)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(n_sel), _ptr(o), _ptr(lse), _ptr(d_o), B, L, n_k, H, D,
            K_tot, scale)
    _check("lsa_sparse_attn_backward", lib.lsa_sparse_attn_backward(*args, None, None, None, None, 0,
                                                                    ctypes.byref(need), None))
    if ws is None or ws.numel() < need.value:
        ws = _workspace(need.value, q.device)
    dq = torch.empty_like(q)
    dk = torch.empty((B, n_k, D), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    _check("lsa_sparse_attn_backward", lib.lsa_sparse_attn_backward(*args, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                                                    ws.numel(), None, _stream()))
    return dq, dk, dv


def lsa_kl_warmup(q, k, idx, n_sel, lse, logits, scale=None):
    """Warm-up KL of each row's head-averaged attention distribution against
    the softmax of its indexer logits: q [B, L, H, D] bf16, k [B, n_k, D] bf16,
    idx [B, L, K_tot], n_sel [B, L], lse [B, L, H] fp32 (the forward's), logits
    [B, L, K_tot] fp32. Returns (kl [B, L] fp32, dlogits [B, L, K_tot] fp32)."""
    lib = load()
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k")
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    _dev(lse, torch.float32, "lse")
    _dev(logits, torch.float32, "logits")
    B, Lq, H, D = q.shape
    n_k = k.shape[1]
    K_tot = idx.shape[-1]
    if idx.shape != (B, Lq, K_tot) or n_sel.shape != (B, Lq) or lse.shape != (B, Lq, H) or logits.shape != idx.shape:
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else float(scale)
    kl = torch.empty((B, Lq), dtype=torch.float32, device=q.device)
    dlog = torch.empty((B, Lq, K_tot), dtype=torch.float32, device=q.device)
    _check("lsa_kl_warmup", lib.lsa_kl_warmup(_ptr(q), _ptr(k), _ptr(idx), _ptr(n_sel), _ptr(lse), _ptr(logits), B,
                                              Lq, n_k, H, D, K_tot, scale, _ptr(kl), _ptr(dlog), _stream()))
    return kl, dlog


def lsa_sparse_attn_decode_noalloc(q, k_cache, v_cache, idx, n_sel, n_split=8, scale=None, want_lse=False):
    """lsa_sparse_attn_decode with the partials in the library's fixed scratch
    array (no workspace). Returns o [B, n_q, H, D] bf16 (and lse)."""
    lib = load()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, n)
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    B, n_q, H, D = q.shape
    n_k = k_cache.shape[1]
    n_idx, K_tot = idx.shape[1], idx.shape[2]
    if idx.shape[0] != B or n_sel.shape != (B, n_idx):
        raise ValueError("shape mismatch")
    scale = D ** -0.5 if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device) if want_lse else None
    _check("lsa_sparse_attn_decode_noalloc", lib.lsa_sparse_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), _ptr(n_sel), n_idx, B, n_q, n_k, H, D, K_tot, n_split,
        scale, _ptr(o), _ptr(lse), _stream()))
    return (o, lse) if want_lse else o


def lsa_sparse_attn_decode_mtp(q, k_cache, v_cache, idx, n_sel, tgt_pos, n_split=8, scale=None, want_lse=False,
                               ws=None):
    """Decode for MTP rows with causal tails: idx [B, 1, K_tot] (the target's
    list, shared), tgt_pos [B] int32 on the device; row j also attends to
    tgt_pos + 1 .. tgt_pos + j. Returns o [B, n_q, H, D] (and lse)."""
    lib = load()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, n)
    _dev(idx, torch.int32, "idx")
    _dev(n_sel, torch.int32, "n_sel")
    _dev(tgt_pos, torch.int32, "tgt_pos")
    B, n_q, H, D = q.shape
    n_k = k_cache.shape[1]
    if idx.shape[:2] != (B, 1) or n_sel.shape != (B, 1) or tuple(tgt_pos.shape) != (B,):
        raise ValueError("shape mismatch")
    K_tot = idx.shape[2]
    scale = D ** -0.5 if scale is None else float(scale)
    need = ctypes.c_size_t(0)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), _ptr(n_sel), _ptr(tgt_pos), B, n_q, n_k, H, D, K_tot,
            n_split, scale)
    _check("lsa_sparse_attn_decode_mtp",
           lib.lsa_sparse_attn_decode_mtp(*args, None, None, None, 0, ctypes.byref(need), None))
    if ws is None or ws.numel() < need.value:
        ws = _workspace(need.value, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device) if want_lse else None
    _check("lsa_sparse_attn_decode_mtp", lib.lsa_sparse_attn_decode_mtp(*args, _ptr(o), _ptr(lse), _ptr(ws),
                                                                        ws.numel(), None, _stream()))
    return (o, lse) if want_lse else o


def lsa_kernel_timing(on):
    """Start (True) or stop (False) per-launch HIP event timing in the
    library; either way the earlier records are cleared."""
    _check("lsa_kernel_timing", load().lsa_kernel_timing(1 if on else 0))


def lsa_kernel_time(name):
    """(mean ms, launches) of kernel `name` since timing was switched on."""
    ms, n = _F(), _I()
    _check("lsa_kernel_time", load().lsa_kernel_time(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def lsa_probe_mfma(kind, n_wg, iters, sink):
    """Enqueue the matrix-core peak probe (kind 0 int8, 1 bf16) on the
    current stream; sink is an int32 device tensor of n_wg entries. Returns
    the operations one launch performs (time the launch with events)."""
    _dev(sink, torch.int32, "sink")
    if sink.numel() < n_wg:
        raise ValueError("sink needs n_wg entries")
    ops = ctypes.c_double(0.0)
    _check("lsa_probe_mfma", load().lsa_probe_mfma(int(kind), int(n_wg), int(iters), _ptr(sink), ctypes.byref(ops),
                                                   _stream()))
    return float(ops.value)


def lsa_probe_mfma_data(kind, n_wg, iters, a, b, sink):
    """The probe with operands drawn from device tensors a and b (any dtype,
    contiguous, 16-byte aligned, at least 16 bytes): kind 0 reads them as
    int8 fragments, kind 1 as bf16. Returns the operations one launch
    performs."""
    _dev(sink, torch.int32, "sink")
    if sink.numel() < n_wg:
        raise ValueError("sink needs n_wg entries")
    for t, nm in ((a, "a"), (b, "b")):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{nm} must be a contiguous device tensor")
    ops = ctypes.c_double(0.0)
    _check("lsa_probe_mfma_data",
           load().lsa_probe_mfma_data(int(kind), int(n_wg), int(iters), _ptr(a), a.numel() * a.element_size(), _ptr(b),
                                      b.numel() * b.element_size(), _ptr(sink), ctypes.byref(ops), _stream()))
    return float(ops.value)
