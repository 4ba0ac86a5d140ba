"""The C ABI on a machine without a GPU: the library loads, exports every
symbol that include/lsa.h declares, and rejects bad arguments synchronously,
before any HIP call (every call below returns before a launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

from long_context_sparse_lsa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="liblsa.so not built")

FAKE = 0x7F0000000000  # 256-aligned, never dereferenced: every call fails its checks first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = L.load()
    names = declared_functions()
    assert set(names) == set(L.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(7):
        msg = L.status_string(s)
        assert msg.startswith("LSA_")
    assert "UNKNOWN" in L.status_string(99)


def _w(vals):
    a = np.asarray(vals, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


P = ctypes.c_void_p


def test_index_score_argument_checks():
    lib = L.load()
    w, wp = _w([1, 2, 3, 4])
    ok = dict(q=P(FAKE), k=P(FAKE), B=1, n_q=4, n_k=8, H_I=4, d_I=64, off=4, s=P(FAKE))

    def call(**kw):
        a = dict(ok, **kw)
        return lib.lsa_index_score(a["q"], a["k"], kw.get("wp", wp), a["B"], a["n_q"], a["n_k"], a["H_I"],
                                   a["d_I"], a["off"], a["s"], None)

    assert call(q=None) == L.LSA_INVALID_ARG
    assert call(k=P(FAKE + 8)) == L.LSA_INVALID_ARG        # misaligned
    assert call(s=P(FAKE + 2)) == L.LSA_INVALID_ARG
    assert call(B=0) == L.LSA_INVALID_ARG
    assert call(n_q=-1) == L.LSA_INVALID_ARG
    assert call(off=-1) == L.LSA_INVALID_ARG
    assert call(d_I=96) == L.LSA_UNSUPPORTED
    assert call(H_I=12) == L.LSA_UNSUPPORTED
    assert call(wp=None) == L.LSA_INVALID_ARG
    big, bigp = _w([1 << 20, 1, 1, 1])
    assert call(wp=bigp) == L.LSA_RANGE
    # bound: sum|w| * d_I * 2^14 < 2^31  -> for d_I=64: sum|w| < 2048
    edge, edgep = _w([2047, 0, 0, 0])
    over, overp = _w([2047, 0, 0, -1])
    assert call(wp=overp) == L.LSA_RANGE
    del edge, edgep


def test_select_topk_checks_and_workspace_query():
    lib = L.load()
    need = ctypes.c_size_t(0)
    cfg = L.SelectCfg(4, 512, 1532)
    w, wp = _w([1] * 64)
    # size query: ws = NULL with ws_needed set returns the size, launches nothing
    s = lib.lsa_select_topk(None, P(FAKE), P(FAKE), wp, 1, 32768, 32768, 64, 128, 0, cfg,
                            None, None, None, 0, ctypes.byref(need), None)
    assert s == L.LSA_OK and need.value > 0 and need.value % 256 == 0
    fused_need = need.value
    s = lib.lsa_select_topk(P(FAKE), None, None, None, 1, 32768, 32768, 0, 0, 0, cfg,
                            None, None, None, 0, ctypes.byref(need), None)
    assert s == L.LSA_OK and 0 < need.value < fused_need
    # too small a workspace
    s = lib.lsa_select_topk(P(FAKE), None, None, None, 1, 32768, 32768, 0, 0, 0, cfg,
                            P(FAKE), P(FAKE), P(FAKE), need.value - 256, None, None)
    assert s == L.LSA_WORKSPACE
    # inconsistent sizes
    assert lib.lsa_select_topk(P(FAKE), None, None, None, 1, 10, 5, 0, 0, 0, cfg,
                               P(FAKE), P(FAKE), P(FAKE), 1 << 30, None, None) == L.LSA_INVALID_ARG
    bad = L.SelectCfg(-1, 4, 4)
    assert lib.lsa_select_topk(P(FAKE), None, None, None, 1, 10, 10, 0, 0, 0, bad,
                               P(FAKE), P(FAKE), P(FAKE), 1 << 30, None, None) == L.LSA_INVALID_ARG
    zero = L.SelectCfg(0, 0, 0)
    assert lib.lsa_select_topk(P(FAKE), None, None, None, 1, 10, 10, 0, 0, 0, zero,
                               P(FAKE), P(FAKE), P(FAKE), 1 << 30, None, None) == L.LSA_INVALID_ARG
    # fused path needs supported indexer shapes and in-range weights
    assert lib.lsa_select_topk(None, P(FAKE), P(FAKE), wp, 1, 10, 10, 64, 96, 0, cfg,
                               P(FAKE), P(FAKE), P(FAKE), 1 << 30, None, None) == L.LSA_UNSUPPORTED
    big, bigp = _w([1 << 16] * 64)
    assert lib.lsa_select_topk(None, P(FAKE), P(FAKE), bigp, 1, 10, 10, 64, 128, 0, cfg,
                               P(FAKE), P(FAKE), P(FAKE), 1 << 30, None, None) == L.LSA_RANGE


def test_select_topk_candidate_limit():
    """Flat selection holds up to (32768 / k_cap)^2 chunks of 32768 keys per row
    (a middle reduction stage past 16 chunks at k_dyn = 2048): 8388608
    candidates; one more is unsupported. A 1M-key cache is supported."""
    lib = L.load()
    need = ctypes.c_size_t(0)
    cfg = L.SelectCfg(4, 512, 2048)
    for n_k, want in ((1 << 20, L.LSA_OK), (8388608 + 516, L.LSA_OK), (8388608 + 517, L.LSA_UNSUPPORTED)):
        s = lib.lsa_select_topk(P(FAKE), None, None, None, 1, 1, n_k, 0, 0, n_k - 1, cfg,
                                None, None, None, 0, ctypes.byref(need), None)
        assert s == want, (n_k, s)
    w, wp = _w([1] * 64)
    s = lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), wp, 4, 1, 1 << 20, 64, 128, P(FAKE), cfg,
                                   None, None, None, 0, ctypes.byref(need), None)
    assert s == L.LSA_OK


def test_select_topk_ragged_checks():
    lib = L.load()
    need = ctypes.c_size_t(0)
    cfg = L.SelectCfg(4, 512, 2048)
    w, wp = _w([1] * 64)
    # sized for full-length sequences: the same workspace as the fused path at q_off = n_k - n_q
    s = lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), wp, 64, 1, 131072, 64, 128, P(FAKE), cfg,
                                   None, None, None, 0, ctypes.byref(need), None)
    assert s == L.LSA_OK and need.value > 0
    ragged_need = need.value
    s = lib.lsa_select_topk(None, P(FAKE), P(FAKE), wp, 64, 1, 131072, 64, 128, 131071, cfg,
                            None, None, None, 0, ctypes.byref(need), None)
    assert s == L.LSA_OK and need.value == ragged_need
    # the length array is required
    assert lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), wp, 64, 1, 131072, 64, 128, None, cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_INVALID_ARG
    # more query rows than cache slots, unsupported indexer shape, weights out of range, small workspace
    assert lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), wp, 2, 8, 4, 64, 128, P(FAKE), cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_INVALID_ARG
    assert lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), wp, 2, 1, 4096, 64, 96, P(FAKE), cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_UNSUPPORTED
    big, bigp = _w([1 << 16] * 64)
    assert lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), bigp, 2, 1, 4096, 64, 128, P(FAKE), cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_RANGE
    assert lib.lsa_select_topk_ragged(P(FAKE), P(FAKE), wp, 64, 1, 131072, 64, 128, P(FAKE), cfg,
                                      P(FAKE), P(FAKE), P(FAKE), ragged_need - 256, None, None) == L.LSA_WORKSPACE


def test_hier_select_ragged_checks():
    lib = L.load()
    need = ctypes.c_size_t(0)
    cfg = L.SelectCfg(4, 512, 2048)
    w, wp = _w([1] * 64)
    f = P(FAKE)
    # sized for full-length sequences: the same workspace as the uniform call
    assert lib.lsa_hier_select(f, f, f, wp, 4, 1 << 20, 64, 128, 64, 256, cfg,
                               None, None, None, 0, ctypes.byref(need), None) == L.LSA_OK
    uniform_need = need.value
    assert lib.lsa_hier_select_ragged(f, f, f, wp, 4, 1 << 20, f, 64, 128, 64, 256, cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_OK
    assert need.value == uniform_need > 0
    # the length array is required; block size and workspace checks as the uniform call
    assert lib.lsa_hier_select_ragged(f, f, f, wp, 4, 1 << 20, None, 64, 128, 64, 256, cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_INVALID_ARG
    assert lib.lsa_hier_select_ragged(f, f, f, wp, 4, 1 << 20, f, 64, 128, 48, 256, cfg,
                                      None, None, None, 0, ctypes.byref(need), None) == L.LSA_UNSUPPORTED
    assert lib.lsa_hier_select_ragged(f, f, f, wp, 4, 1 << 20, f, 64, 128, 64, 256, cfg,
                                      f, f, f, uniform_need - 256, None, None) == L.LSA_WORKSPACE


def test_mtp_row_index_checks():
    lib = L.load()
    f = P(FAKE)
    need = ctypes.c_size_t(0)
    dargs = [f, f, f, f, f, f, 64, 4, 131072, 64, 128, 2564, 8, 0.088]
    assert lib.lsa_sparse_attn_decode_mtp(*dargs, f, None, None, 0, ctypes.byref(need), None) == L.LSA_OK
    bad = list(dargs)
    bad[5] = None       # tgt_pos
    assert lib.lsa_sparse_attn_decode_mtp(*bad, f, None, None, 0, ctypes.byref(need), None) == L.LSA_INVALID_ARG
    bad = list(dargs)
    bad[7] = 33         # n_q: the drafts' keys must fit one block
    assert lib.lsa_sparse_attn_decode_mtp(*bad, f, None, None, 0, ctypes.byref(need), None) == L.LSA_UNSUPPORTED
    assert lib.lsa_mtp_row_index(None, f, 2, 100, 4, f, f, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_mtp_row_index(f, f, 2, 100, 4, None, f, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_mtp_row_index(f, f, 0, 100, 4, f, f, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_mtp_row_index(f, f, 2, 0, 4, f, f, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_mtp_row_index(f, f, 2, 100, 0, f, f, f, None) == L.LSA_INVALID_ARG


def test_hier_and_summary_checks():
    lib = L.load()
    # appending to a cache: order and bounds of the key counts
    f = P(FAKE)
    assert lib.lsa_block_summary_append(f, 1, 1000, 10, 5, 128, 64, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_block_summary_append(f, 1, 1000, 10, 1001, 128, 64, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_block_summary_append(f, 1, 1000, -1, 5, 128, 64, f, None) == L.LSA_INVALID_ARG
    assert lib.lsa_block_summary_append(f, 1, 1000, 10, 20, 100, 64, f, None) == L.LSA_UNSUPPORTED
    assert lib.lsa_block_summary_append(f, 1, 1000, 10, 10, 128, 64, f, None) == L.LSA_OK  # nothing new
    need = ctypes.c_size_t(0)
    cfg = L.SelectCfg(4, 512, 2048)
    w, wp = _w([1] * 64)
    s = lib.lsa_hier_select(P(FAKE), P(FAKE), P(FAKE), wp, 4, 1 << 20, 64, 128, 64, 256, cfg,
                            None, None, None, 0, ctypes.byref(need), None)
    assert s == L.LSA_OK and need.value > 0
    assert lib.lsa_hier_select(P(FAKE), P(FAKE), P(FAKE), wp, 4, 1 << 20, 64, 128, 48, 256, cfg,
                               None, None, None, 0, ctypes.byref(need), None) == L.LSA_UNSUPPORTED
    assert lib.lsa_hier_select(P(FAKE), P(FAKE), P(FAKE), wp, 4, 1 << 20, 64, 128, 64, 0, cfg,
                               None, None, None, 0, ctypes.byref(need), None) == L.LSA_INVALID_ARG
    assert lib.lsa_block_summary(None, 1, 64, 128, 64, P(FAKE), None) == L.LSA_INVALID_ARG
    assert lib.lsa_block_summary(P(FAKE), 1, 64, 100, 64, P(FAKE), None) == L.LSA_UNSUPPORTED
    assert lib.lsa_block_summary(P(FAKE), 1, 64, 128, 0, P(FAKE), None) == L.LSA_INVALID_ARG


def test_attention_checks():
    lib = L.load()
    f = P(FAKE)
    args = [f, f, f, f, f, 1, 16, 16, 64, 128, 256, 0.088]   # valid: never called as is
    bad_d = list(args)
    bad_d[9] = 64
    assert lib.lsa_sparse_attn_prefill(*bad_d, f, None, None) == L.LSA_UNSUPPORTED
    bad_h = list(args)
    bad_h[8] = 48
    assert lib.lsa_sparse_attn_prefill(*bad_h, f, None, None) == L.LSA_UNSUPPORTED
    big = list(args)
    big[7] = 1 << 24    # n_k past the 32-bit byte offsets of the cache gathers
    assert lib.lsa_sparse_attn_prefill(*big, f, None, None) == L.LSA_UNSUPPORTED
    bad_s = list(args)
    bad_s[11] = float("nan")
    assert lib.lsa_sparse_attn_prefill(*bad_s, f, None, None) == L.LSA_INVALID_ARG
    assert lib.lsa_sparse_attn_prefill(None, *args[1:], f, None, None) == L.LSA_INVALID_ARG
    need = ctypes.c_size_t(0)
    dargs = [f, f, f, f, f, 1, 64, 4, 131072, 64, 128, 2564, 8, 0.088]
    assert lib.lsa_sparse_attn_decode(*dargs, f, None, None, 0, ctypes.byref(need), None) == L.LSA_OK
    # partials per (sequence, part, row, head): m and l in fp32, 128 fp16 outputs
    assert need.value >= 64 * 4 * 64 * 8 * (2 * 4 + 128 * 2)
    bad = list(dargs)
    bad[5] = 3          # n_idx neither 1 nor n_q
    assert lib.lsa_sparse_attn_decode(*bad, f, None, None, 0, ctypes.byref(need), None) == L.LSA_INVALID_ARG
    bad = list(dargs)
    bad[8] = 1 << 24    # n_k
    assert lib.lsa_sparse_attn_decode(*bad, f, None, None, 0, ctypes.byref(need), None) == L.LSA_UNSUPPORTED
    bad = list(dargs)
    bad[12] = 65        # n_split
    assert lib.lsa_sparse_attn_decode(*bad, f, None, None, 0, ctypes.byref(need), None) == L.LSA_UNSUPPORTED
    assert lib.lsa_sparse_attn_decode(*dargs, f, None, f, 100, None, None) == L.LSA_WORKSPACE


def test_kernel_timing_without_launches():
    """Timing on/off and reads touch no GPU while nothing was recorded."""
    lib = L.load()
    ms, n = ctypes.c_float(1.0), ctypes.c_int32(7)
    assert lib.lsa_kernel_time(None, ctypes.byref(ms), ctypes.byref(n)) == L.LSA_INVALID_ARG
    assert lib.lsa_kernel_time(b"attn_prefill_kernel", None, ctypes.byref(n)) == L.LSA_INVALID_ARG
    assert lib.lsa_kernel_timing(0) == L.LSA_OK
    assert lib.lsa_kernel_time(b"attn_prefill_kernel", ctypes.byref(ms), ctypes.byref(n)) == L.LSA_OK
    assert n.value == 0 and ms.value == 0.0
    assert lib.lsa_kernel_timing(0) == L.LSA_OK


def test_probe_argument_checks():
    """Both matrix-core probes reject bad arguments before any launch."""
    lib = L.load()
    f, ops = P(FAKE), ctypes.c_double(0.0)
    assert lib.lsa_probe_mfma(0, 8, 4, None, ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    assert lib.lsa_probe_mfma(0, 8, 4, P(FAKE + 2), ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    assert lib.lsa_probe_mfma(0, 0, 4, f, ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    assert lib.lsa_probe_mfma(2, 8, 4, f, ctypes.byref(ops), None) == L.LSA_UNSUPPORTED
    ok = [0, 8, 4, f, 64, f, 64, f]
    bad = list(ok); bad[3] = None
    assert lib.lsa_probe_mfma_data(*bad, ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    bad = list(ok); bad[5] = P(FAKE + 8)      # b not 16-byte aligned
    assert lib.lsa_probe_mfma_data(*bad, ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    bad = list(ok); bad[4] = 15               # fewer than one 16-byte fragment
    assert lib.lsa_probe_mfma_data(*bad, ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    bad = list(ok); bad[2] = 0
    assert lib.lsa_probe_mfma_data(*bad, ctypes.byref(ops), None) == L.LSA_INVALID_ARG
    bad = list(ok); bad[0] = 3
    assert lib.lsa_probe_mfma_data(*bad, ctypes.byref(ops), None) == L.LSA_UNSUPPORTED
