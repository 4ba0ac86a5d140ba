// C ABI of the LSA hot path: argument checks, workspace sizing, launches.
//
// Every check that the host can make runs before the first launch, so an
// argument error never leaves half of the work enqueued. The library
// allocates nothing at run time: workspace comes from the caller, except for
// the no-alloc decode entry at the end of this file, whose fixed scratch array
// is part of the loaded code (its per-device address is the only state kept).
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "lsa.h"
#include "lsa_internal.h"

using namespace lsa;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool al16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }
bool hi_ok(int h) { return h == 4 || h == 8 || h == 16 || h == 32 || h == 64 || h == 128; }
bool di_ok(int d) { return d == 64 || d == 128; }
bool heads_ok(int h) { return h == 16 || h == 32 || h == 64 || h == 128; }

int32_t load_weights(const int32_t* w, int H_I, int d_I, WArgs& wa) {
  if (w == nullptr) return LSA_INVALID_ARG;
  int64_t s = 0;
  for (int h = 0; h < 128; ++h) wa.w[h] = 0;
  for (int h = 0; h < H_I; ++h) {
    wa.w[h] = w[h];
    s += w[h] < 0 ? -(int64_t)w[h] : (int64_t)w[h];
  }
  // every |q.k| <= d_I * 128 * 128, so |S| <= sum|w| * d_I * 2^14
  if (s * d_I * 16384 >= ((int64_t)1 << 31)) return LSA_RANGE;
  return LSA_OK;
}

int32_t cfg_ok(const lsa_select_cfg& c) {
  if (c.n_sink < 0 || c.n_window < 0 || c.k_dyn < 0) return LSA_INVALID_ARG;
  if ((int64_t)c.n_sink + c.n_window + c.k_dyn < 1) return LSA_INVALID_ARG;
  if ((int64_t)c.n_sink + c.n_window + c.k_dyn > (1 << 20)) return LSA_UNSUPPORTED;
  return LSA_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_HIP; }

int k_cap_of(int k) { return std::max(4, (k + 3) / 4 * 4); }

int chunks_of(int64_t nc, int k_cap) { return select_chunks(nc, k_cap); }

// Stage two of a multi-chunk selection holds every chunk's survivors at once.
bool survivors_ok(int64_t max_nc, int k_cap) { return select_fits(max_nc, k_cap); }

// Rows per pass of the fused (score + select) prefill path: the score buffer
// of one pass is at most kFusedScoreBytes.
constexpr size_t kFusedScoreBytes = (size_t)2048 << 20;
// Returns the rows of one query range (R) and the sequences per pass (nb):
// a long prefill is cut into row ranges of one sequence (nb = 1), a short
// decode batch puts many whole sequences into one pass.
void fused_pass(int B, int n_q, int n_k, int& R, int& nb) {
  int64_t r = (int64_t)(kFusedScoreBytes / sizeof(int32_t)) / n_k;
  r = std::max<int64_t>(4, r / 4 * 4);
  if (r <= n_q) {
    R = (int)r;
    nb = 1;
  } else {
    R = n_q;
    nb = (int)std::min<int64_t>(B, r / n_q);
  }
}

}  // namespace

extern "C" const char* lsa_status_string(int32_t s) {
  switch (s) {
    case LSA_OK: return "LSA_OK";
    case LSA_INVALID_ARG: return "LSA_INVALID_ARG: null, misaligned, non-positive or inconsistent argument";
    case LSA_UNSUPPORTED: return "LSA_UNSUPPORTED: shape outside the supported set";
    case LSA_WORKSPACE: return "LSA_WORKSPACE: workspace too small";
    case LSA_RANGE: return "LSA_RANGE: sum|w| * d_I * 128^2 >= 2^31, scores would not be exact int32";
    case LSA_HIP: return "LSA_HIP: a HIP launch failed";
    case LSA_SCRATCH_LIMIT:
      return "LSA_SCRATCH_LIMIT: the sizes need more than the library's fixed scratch array";
    default: return "LSA_UNKNOWN_STATUS";
  }
}

extern "C" int32_t lsa_index_score(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                                   int32_t B, int32_t n_q, int32_t n_k, int32_t H_I, int32_t d_I,
                                   int32_t q_off, int32_t* scores, void* stream) {
  if (!al16(q_idx) || !al16(k_idx) || !al4(scores)) return LSA_INVALID_ARG;
  if (B <= 0 || n_q <= 0 || n_k <= 0 || q_off < 0) return LSA_INVALID_ARG;
  if (!hi_ok(H_I) || !di_ok(d_I)) return LSA_UNSUPPORTED;
  ScoreArgs a{};
  int32_t s = load_weights(w, H_I, d_I, a.w);
  if (s != LSA_OK) return s;
  a.q = q_idx;
  a.k = k_idx;
  a.B = B;
  a.n_q = n_q;
  a.n_k = n_k;
  a.H_I = H_I;
  a.d_I = d_I;
  a.q_bstride = (int64_t)n_q * H_I * d_I;
  a.k_bstride = (int64_t)n_k * d_I;
  a.s_bstride = (int64_t)n_q * n_k;
  a.ld = n_k;
  a.n_keys = n_k;
  a.mask_off = q_off;
  a.pos_lo = 0;
  a.blocks = nullptr;
  a.fill_masked = 1;
  a.scores = scores;
  return hip_status(launch_index_score(a, (hipStream_t)stream));
}

// Thresholded selection (FilterArgs): rows with at least kFilterMinCand
// candidates, in passes of one sequence (prefill), score a sample of every
// kSampM-th position first; the sample's threshold lets the full scoring pass
// keep about (lam + 6 sqrt(lam) + 10) * kSampM pairs per row (lam = k / kSampM)
// instead of writing every score, and the survivors' top-k is exact whenever
// they number at least k; other rows are redone by the dense path.
constexpr int kSampM = 64;
constexpr int kFilterMinCand = 16384;
// Thresholded rows go in passes of up to this many dense passes' rows (the
// segments are far smaller than dense scores), which halves or quarters the
// launches per row and the part of each launch spent draining its last round.
constexpr int kFiltPassMul = 4;

struct FilterPlan {
  bool on = false;
  int64_t surv = 0;  // expected survivors of a row, at most
  int max_surv = 0;  // survivors the survivor selection holds (twice surv)
};

FilterPlan filter_plan(const lsa_select_cfg& cfg, int H_I, int d_I) {
  FilterPlan p;
  const int k = cfg.k_dyn;
  if (k < 64 || (H_I != 32 && H_I != 64) || (d_I != 64 && d_I != 128)) return p;
  // the sample of a row holds at most nc / m + 1 of its nc >= kFilterMinCand candidates
  const double lam = (double)k / kSampM + (double)k / kFilterMinCand;
  const double jstar = std::ceil(lam + 6.0 * std::sqrt(lam) + 10.0);
  p.surv = (int64_t)std::ceil(jstar * (kSampM + 1));
  p.on = 2 * p.surv <= filter_select_capacity();
  p.max_surv = (int)(2 * p.surv);
  return p;
}

// Pairs one (row, chunk) segment holds: survivors of a chunk of ck keys in a
// row of at least nc_min candidates number about mu = surv * min(1, ck /
// nc_min); the capacity leaves room for the threshold's spread.
int seg_cap_of(const FilterPlan& p, int ck, int64_t nc_min) {
  const double mu = (double)p.surv * std::min(1.0, (double)ck / (double)nc_min);
  const int64_t cap = (int64_t)std::ceil(1.6 * mu + 8.0 * std::sqrt(mu) + 64.0);
  return (int)std::min<int64_t>(ck, (cap + 63) / 64 * 64);
}

// Workspace of the fused path for passes of `rows` rows: the dense score
// buffer (which the filtered rows' segments share), the selection's chunk
// workspace, then the sample scores, thresholds, fail flags and segment counts
// (these four for thresholded passes of up to kFiltPassMul * rows rows).
struct FusedWs {
  size_t sbuf, sel, samp, tau, fail, cnt, total;
  int64_t samp_ld;
  int max_segs;
};
FusedWs fused_ws(int64_t rows, int n_k, int64_t max_nc, int k_cap, bool filter) {
  FusedWs w{};
  w.sbuf = align_up((size_t)rows * n_k * sizeof(int32_t));
  w.sel = align_up(select_ws_bytes((int)rows, chunks_of(max_nc, k_cap), k_cap));
  if (filter) {
    const int64_t fr = rows * kFiltPassMul;
    w.samp_ld = ((int64_t)n_k / kSampM + 1 + 3) / 4 * 4;
    w.max_segs = (n_k + 4095) / 4096;
    w.samp = align_up((size_t)fr * w.samp_ld * sizeof(int32_t));
    w.tau = align_up((size_t)fr * sizeof(int32_t));
    w.fail = w.tau;
    w.cnt = align_up((size_t)fr * w.max_segs * sizeof(int32_t));
  }
  w.total = w.sbuf + w.sel + w.samp + w.tau + w.fail + w.cnt;
  return w;
}

// Fused path of the flat selection: score a pass of rows (candidates only)
// into the workspace, then select. A pass covers nb sequences times one range
// of Rr query rows. ctx_len (device, per sequence, or null): ragged lengths,
// row i of sequence b at position clamp(ctx_len[b], n_q, n_k) - n_q + i
// (q_off is then n_k - n_q). Passes of one sequence without ctx_len take the
// thresholded selection for their rows of at least kFilterMinCand candidates.
static int32_t fused_select(const int8_t* q_idx, const int8_t* k_idx, const WArgs& wa, int B, int n_q, int n_k,
                            int H_I, int d_I, int q_off, const lsa_select_cfg& cfg, int R, int nb_pass,
                            const int32_t* ctx_len, int32_t* idx, int32_t* n_sel, void* ws, hipStream_t st) {
  const int K_tot = cfg.n_sink + cfg.n_window + cfg.k_dyn;
  const int k_cap = k_cap_of(cfg.k_dyn);
  const FilterPlan fp = ctx_len == nullptr && nb_pass == 1 ? filter_plan(cfg, H_I, d_I) : FilterPlan{};
  const int64_t max_nc = (int64_t)q_off + n_q - cfg.n_window - cfg.n_sink;
  const FusedWs wl = fused_ws((int64_t)R * nb_pass, n_k, max_nc, k_cap, fp.on);
  int32_t* sbuf = (int32_t*)ws;
  void* sel_ws = (char*)ws + wl.sbuf;
  int32_t* samp = (int32_t*)((char*)sel_ws + wl.sel);
  int32_t* tau = (int32_t*)((char*)samp + wl.samp);
  int32_t* fail = (int32_t*)((char*)tau + wl.tau);
  int32_t* seg_cnt = (int32_t*)((char*)fail + wl.fail);

  SelectArgs sa{};
  sa.mode = SEL_FLAT;
  sa.n_sink = cfg.n_sink;
  sa.n_window = cfg.n_window;
  sa.k_dyn = cfg.k_dyn;
  sa.out_ld = K_tot;
  sa.k_cap = k_cap;

  // the indexer launch over rows [r0, r0 + Rr) of sequences b0 .. b0 + nb - 1
  auto score_args = [&](int b0, int nb, int r0, int Rr) {
    const int t_last = q_off + r0 + Rr - 1;
    ScoreArgs a{};
    a.w = wa;
    a.q = q_idx + ((int64_t)b0 * n_q + r0) * H_I * d_I;
    a.k = k_idx + (int64_t)b0 * n_k * d_I;
    a.B = nb;
    a.n_q = Rr;
    a.n_k = n_k;
    a.H_I = H_I;
    a.d_I = d_I;
    a.q_bstride = (int64_t)n_q * H_I * d_I;
    a.k_bstride = (int64_t)n_k * d_I;
    a.s_bstride = (int64_t)Rr * n_k;
    a.ld = n_k;
    a.n_keys = (int)std::min<int64_t>(n_k, (int64_t)t_last - cfg.n_window + 1);
    a.mask_off = q_off + r0 - cfg.n_window;
    a.pos_lo = cfg.n_sink;
    a.fill_masked = 0;
    a.scores = sbuf;
    a.shift = SeqShift{ctx_len ? ctx_len + b0 : nullptr, n_q, n_k};
    return a;
  };

  // dense: every candidate score of the rows, then the chunked selection
  // (only the rows flagged in `flags`, when given)
  auto dense_rows = [&](int b0, int nb, int r0, int Rr, const int32_t* flags) -> int32_t {
    const int t_last = q_off + r0 + Rr - 1;
    const int64_t nc_last = (int64_t)t_last - cfg.n_window - cfg.n_sink + 1;
    if (nc_last > 0 && t_last + 1 > K_tot) {
      ScoreArgs a = score_args(b0, nb, r0, Rr);
      a.row_flags = flags;
      if (a.n_keys > 0) {
        const int32_t s = hip_status(launch_index_score(a, st));
        if (s != LSA_OK) return s;
      }
    }
    // rows of the pass: sequence b0 + j, query r0 + i at row j * Rr + i
    SelectArgs d = sa;
    d.scores = sbuf;
    d.ld = n_k;
    d.n_rows = nb * Rr;
    d.n_q = Rr;
    d.q_off = q_off + r0;
    d.row0 = 0;
    d.shift = SeqShift{ctx_len ? ctx_len + b0 : nullptr, n_q, n_k};
    d.row_flags = flags;
    select_plan(d, nc_last);
    select_bind_ws(d, sel_ws, nb * Rr);
    // nb > 1 only when Rr == n_q (r0 == 0), so the pass's output rows are
    // contiguous in idx / n_sel
    d.idx = idx + ((int64_t)b0 * n_q + r0) * K_tot;
    d.n_sel = n_sel + (int64_t)b0 * n_q + r0;
    return hip_status(launch_select(d, st));
  };

  // thresholded: rows [r0, r0 + Rr) of sequence b0 (Rr <= kFiltPassMul * R),
  // every one non-trivial with at least kFilterMinCand candidates. Returns
  // LSA_UNSUPPORTED (before any launch) when its segments do not fit the
  // dense score buffer.
  auto filtered_rows = [&](int b0, int r0, int Rr) -> int32_t {
    const int t_first = q_off + r0, t_last = q_off + r0 + Rr - 1;
    const int64_t nc_first = (int64_t)t_first - cfg.n_window - cfg.n_sink + 1;
    ScoreArgs a = score_args(b0, 1, r0, Rr);
    const int ck = index_prefill_auto_chunk(a);
    const int nsg = (a.n_keys + ck - 1) / ck;
    const int cap = seg_cap_of(fp, ck, nc_first);
    const int J = (t_last - cfg.n_window) / kSampM + 1;  // sampled positions 0, m, .., (J - 1) m
    if (Rr > kFiltPassMul * R || nsg > wl.max_segs || nsg > 256 ||
        (size_t)Rr * nsg * cap * 8 > std::min<size_t>(wl.sbuf, (size_t)1 << 31) || J > 32768 ||
        (int64_t)J > wl.samp_ld)
      return LSA_UNSUPPORTED;
    // 1. the sample: every row against positions j * m, j < J (no mask; the
    //    threshold kernel takes each row's own candidates)
    ScoreArgs sm = a;
    sm.kstride = kSampM;
    sm.n_keys = J;
    sm.mask_off = J;
    sm.pos_lo = 0;
    sm.scores = samp;
    sm.ld = wl.samp_ld;
    sm.s_bstride = (int64_t)Rr * wl.samp_ld;
    {
      const int64_t n_qt = (Rr + 15) / 16;
      int cks = 1024;
      while (cks < 16384 && (int64_t)((J + 2 * cks - 1) / (2 * cks)) * n_qt >= 1024) cks *= 2;
      sm.chunk_keys = cks;
    }
    int32_t s = hip_status(launch_index_score(sm, st));
    if (s != LSA_OK) return s;
    // 2. thresholds
    FilterArgs f{};
    f.sel = sa;
    f.sel.n_rows = Rr;
    f.sel.n_q = Rr;
    f.sel.q_off = t_first;
    f.sel.row0 = 0;
    f.sel.idx = idx + ((int64_t)b0 * n_q + r0) * K_tot;
    f.sel.n_sel = n_sel + (int64_t)b0 * n_q + r0;
    f.samp = samp;
    f.samp_ld = wl.samp_ld;
    f.samp_m = kSampM;
    f.tau = tau;
    f.seg = sbuf;
    f.seg_cnt = seg_cnt;
    f.seg_chunks = nsg;
    f.seg_cap = cap;
    f.fail = fail;
    s = hip_status(launch_filter_threshold(f, J, st));
    if (s != LSA_OK) return s;
    // 3. the full scoring pass, keeping the pairs at or above the thresholds
    a.chunk_keys = ck;
    a.tau = tau;
    a.seg = sbuf;
    a.seg_cnt = seg_cnt;
    a.seg_chunks = nsg;
    a.seg_cap = cap;
    s = hip_status(launch_index_score(a, st));
    if (s != LSA_OK) return s;
    // 4. top-k of the survivors; 5. the dense path for the rows that failed,
    //    in passes of at most R rows (the dense buffer's size)
    s = hip_status(launch_filter_select(f, fp.max_surv, st));
    if (s != LSA_OK) return s;
    for (int x = 0; x < Rr; x += R) {
      s = dense_rows(b0, 1, r0 + x, std::min(R, Rr - x), fail + x);
      if (s != LSA_OK) return s;
    }
    return LSA_OK;
  };

  for (int b0 = 0; b0 < B; b0 += nb_pass) {
    const int nb = std::min(nb_pass, B - b0);
    for (int r0 = 0; r0 < n_q;) {
      const int Rr = std::min(R, n_q - r0);
      // first row of the pass with kFilterMinCand candidates
      int rf = Rr;
      if (fp.on && nb == 1) {
        const int64_t t_f = (int64_t)kFilterMinCand + cfg.n_window + cfg.n_sink - 1;
        rf = (int)std::min<int64_t>(Rr, std::max<int64_t>(0, t_f - (q_off + r0)));
        if (Rr - rf < 16 || (int64_t)q_off + r0 + rf + 1 <= K_tot) rf = Rr;
      }
      int32_t s = LSA_OK;
      int r_next = r0 + Rr;
      if (rf < Rr) {
        // the thresholded rows from r0 + rf on, through the next passes' rows
        // while their segments fit (the longest of kFiltPassMul, 2, 1 passes)
        s = LSA_UNSUPPORTED;
        for (int m = kFiltPassMul; m >= 1 && s == LSA_UNSUPPORTED; m /= 2) {
          const int f_end = (int)std::min<int64_t>(n_q, (int64_t)r0 + (int64_t)m * R);
          if (m > 1 && f_end <= r0 + Rr) continue;
          s = filtered_rows(b0, r0 + rf, f_end - (r0 + rf));
          if (s == LSA_OK) r_next = f_end;
        }
        if (s == LSA_UNSUPPORTED) rf = Rr;  // nothing launched: the whole pass goes dense
        else if (s != LSA_OK) return s;
      }
      if (rf > 0) {
        s = dense_rows(b0, nb, r0, rf, nullptr);
        if (s != LSA_OK) return s;
      }
      r0 = r_next;
    }
  }
  return LSA_OK;
}

extern "C" int32_t lsa_select_topk(const int32_t* scores, const int8_t* q_idx, const int8_t* k_idx,
                                   const int32_t* w, int32_t B, int32_t n_q, int32_t n_k,
                                   int32_t H_I, int32_t d_I, int32_t q_off, lsa_select_cfg cfg,
                                   int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes,
                                   size_t* ws_needed, void* stream) {
  int32_t s = cfg_ok(cfg);
  if (s != LSA_OK) return s;
  if (B <= 0 || n_q <= 0 || n_k <= 0 || q_off < 0 || (int64_t)q_off + n_q > n_k) return LSA_INVALID_ARG;
  const int K_tot = cfg.n_sink + cfg.n_window + cfg.k_dyn;
  const int k_cap = k_cap_of(cfg.k_dyn);
  const int64_t max_nc = (int64_t)q_off + n_q - cfg.n_window - cfg.n_sink;  // last row's candidates
  if (!survivors_ok(max_nc, k_cap)) return LSA_UNSUPPORTED;
  WArgs wa{};
  if (scores == nullptr) {
    if (!al16(q_idx) || !al16(k_idx)) return LSA_INVALID_ARG;
    if (!hi_ok(H_I) || !di_ok(d_I)) return LSA_UNSUPPORTED;
    s = load_weights(w, H_I, d_I, wa);
    if (s != LSA_OK) return s;
  } else if (!al4(scores)) {
    return LSA_INVALID_ARG;
  }

  // workspace
  size_t need;
  int R = 0, nb_pass = 1;
  int rows_pass = B * n_q;
  if (scores != nullptr) {
    const size_t per_row = select_ws_bytes(1, chunks_of(max_nc, k_cap), k_cap);
    if (per_row > 0)
      rows_pass = (int)std::max<size_t>(1, std::min<size_t>(rows_pass, kFusedScoreBytes / per_row));
    need = select_ws_bytes(rows_pass, chunks_of(max_nc, k_cap), k_cap);
  } else {
    fused_pass(B, n_q, n_k, R, nb_pass);
    need = fused_ws((int64_t)R * nb_pass, n_k, max_nc, k_cap, nb_pass == 1 && filter_plan(cfg, H_I, d_I).on).total;
  }
  need = align_up(std::max<size_t>(need, 1));
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al4(idx) || !al4(n_sel) || !al16(ws)) return LSA_INVALID_ARG;
  if (ws_bytes < need) return LSA_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;

  SelectArgs sa{};
  sa.mode = SEL_FLAT;
  sa.n_sink = cfg.n_sink;
  sa.n_window = cfg.n_window;
  sa.k_dyn = cfg.k_dyn;
  sa.out_ld = K_tot;
  sa.k_cap = k_cap;
  if (scores != nullptr) {
    // passes of rows_pass rows (b, i) in flattened order; a pass never mixes
    // the row -> position mapping because position = q_off + (row % n_q)
    for (int64_t r0 = 0; r0 < (int64_t)B * n_q; r0 += rows_pass) {
      const int Rr = (int)std::min<int64_t>(rows_pass, (int64_t)B * n_q - r0);
      sa.scores = scores + r0 * n_k;
      sa.ld = n_k;
      sa.n_rows = Rr;
      sa.n_q = n_q;
      sa.q_off = q_off;
      sa.row0 = (int)(r0 % n_q);
      sa.idx = idx + r0 * K_tot;
      sa.n_sel = n_sel + r0;
      select_plan(sa, max_nc);
      select_bind_ws(sa, ws, Rr);
      s = hip_status(launch_select(sa, st));
      if (s != LSA_OK) return s;
    }
    return LSA_OK;
  }

  return fused_select(q_idx, k_idx, wa, B, n_q, n_k, H_I, d_I, q_off, cfg, R, nb_pass, nullptr, idx, n_sel, ws,
                      st);
}

extern "C" int32_t lsa_select_topk_ragged(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                                          int32_t B, int32_t n_q, int32_t n_k, int32_t H_I, int32_t d_I,
                                          const int32_t* ctx_len, lsa_select_cfg cfg, int32_t* idx,
                                          int32_t* n_sel, void* ws, size_t ws_bytes, size_t* ws_needed,
                                          void* stream) {
  int32_t s = cfg_ok(cfg);
  if (s != LSA_OK) return s;
  if (B <= 0 || n_q <= 0 || n_k <= 0 || n_q > n_k) return LSA_INVALID_ARG;
  if (!al16(q_idx) || !al16(k_idx) || !al4(ctx_len)) return LSA_INVALID_ARG;
  if (!hi_ok(H_I) || !di_ok(d_I)) return LSA_UNSUPPORTED;
  const int k_cap = k_cap_of(cfg.k_dyn);
  const int64_t max_nc = (int64_t)n_k - cfg.n_window - cfg.n_sink;  // candidates of a full-length row
  if (!survivors_ok(max_nc, k_cap)) return LSA_UNSUPPORTED;
  WArgs wa{};
  s = load_weights(w, H_I, d_I, wa);
  if (s != LSA_OK) return s;
  int R = 0, nb_pass = 1;
  fused_pass(B, n_q, n_k, R, nb_pass);
  size_t need = fused_ws((int64_t)R * nb_pass, n_k, max_nc, k_cap, false).total;
  need = align_up(std::max<size_t>(need, 1));
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al4(idx) || !al4(n_sel) || !al16(ws)) return LSA_INVALID_ARG;
  if (ws_bytes < need) return LSA_WORKSPACE;
  return fused_select(q_idx, k_idx, wa, B, n_q, n_k, H_I, d_I, n_k - n_q, cfg, R, nb_pass, ctx_len, idx, n_sel,
                      ws, (hipStream_t)stream);
}

extern "C" int32_t lsa_mtp_row_index(const int32_t* idx, const int32_t* n_sel, int32_t B, int32_t K_tot,
                                     int32_t n_q, const int32_t* tgt_pos, int32_t* idx_rows,
                                     int32_t* n_sel_rows, void* stream) {
  if (!al4(idx) || !al4(n_sel) || !al4(tgt_pos) || !al4(idx_rows) || !al4(n_sel_rows)) return LSA_INVALID_ARG;
  if (B <= 0 || K_tot <= 0 || n_q <= 0 || (int64_t)K_tot + n_q - 1 > (1 << 20)) return LSA_INVALID_ARG;
  if (n_q > 65535) return LSA_UNSUPPORTED;
  return hip_status(
      launch_mtp_index(idx, n_sel, B, K_tot, n_q, tgt_pos, idx_rows, n_sel_rows, (hipStream_t)stream));
}

extern "C" int32_t lsa_block_summary(const int8_t* k_idx, int32_t B, int32_t n_k, int32_t d_I,
                                     int32_t blk, int8_t* k_blk, void* stream) {
  if (!al16(k_idx) || !al16(k_blk)) return LSA_INVALID_ARG;
  if (B <= 0 || n_k <= 0 || blk <= 0) return LSA_INVALID_ARG;
  if (!di_ok(d_I) || blk > 1024) return LSA_UNSUPPORTED;
  const int nb = (int)(((int64_t)n_k + blk - 1) / blk);
  return hip_status(launch_block_summary(k_idx, B, n_k, n_k, d_I, blk, 0, nb, k_blk, (hipStream_t)stream));
}

extern "C" int32_t lsa_block_summary_append(const int8_t* k_idx, int32_t B, int32_t n_cap, int32_t n_old,
                                            int32_t n_new, int32_t d_I, int32_t blk, int8_t* k_blk,
                                            void* stream) {
  if (!al16(k_idx) || !al16(k_blk)) return LSA_INVALID_ARG;
  if (B <= 0 || n_cap <= 0 || blk <= 0 || n_old < 0 || n_old > n_new || n_new > n_cap) return LSA_INVALID_ARG;
  if (!di_ok(d_I) || blk > 1024) return LSA_UNSUPPORTED;
  if (n_new == n_old) return LSA_OK;
  const int j0 = n_old / blk, j1 = (n_new - 1) / blk;  // blocks holding the new keys
  return hip_status(launch_block_summary(k_idx, B, n_cap, n_new, d_I, blk, j0, j1 - j0 + 1, k_blk,
                                         (hipStream_t)stream));
}

// HI selection; with ctx_len set, sequence b holds clamp(ctx_len[b], 1, n_k)
// keys and its query sits at the last of them (every range below is the
// full-length one, narrowed per sequence on the GPU).
static int32_t hier_select(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk, const int32_t* w,
                           int32_t B, int32_t n_k, const int32_t* ctx_len, int32_t H_I, int32_t d_I, int32_t blk,
                           int32_t n_blk_recall, lsa_select_cfg cfg, int32_t* idx, int32_t* n_sel, void* ws,
                           size_t ws_bytes, size_t* ws_needed, void* stream) {
  int32_t s = cfg_ok(cfg);
  if (s != LSA_OK) return s;
  if (B <= 0 || n_k <= 0 || blk <= 0 || n_blk_recall <= 0) return LSA_INVALID_ARG;
  if (!hi_ok(H_I) || !di_ok(d_I) || blk % 32 != 0 || blk > 1024) return LSA_UNSUPPORTED;
  if ((int64_t)n_blk_recall * blk > (1 << 30)) return LSA_UNSUPPORTED;
  WArgs wa{};
  const int K_tot = cfg.n_sink + cfg.n_window + cfg.k_dyn;
  const int t = n_k - 1;
  const bool trivial = t + 1 <= K_tot;
  const int lo = cfg.n_sink, hi = t - cfg.n_window;
  const int nblocks = (n_k + blk - 1) / blk;
  const int b_lo = trivial ? 0 : lo / blk, b_hi = trivial ? 0 : hi / blk;
  const int n_elig = trivial ? 0 : b_hi - b_lo + 1;
  const int n_virt = n_blk_recall * blk;
  const int kc_coarse = k_cap_of(n_blk_recall), kc_fine = k_cap_of(cfg.k_dyn);
  if (!survivors_ok(n_elig, kc_coarse) || !survivors_ok(n_virt, kc_fine)) return LSA_UNSUPPORTED;

  const size_t sz_coarse = align_up((size_t)B * nblocks * sizeof(int32_t));
  const size_t sz_blocks = align_up((size_t)B * n_blk_recall * sizeof(int32_t));
  const size_t sz_nblk = align_up((size_t)B * sizeof(int32_t));
  const size_t sz_fine = align_up((size_t)B * n_virt * sizeof(int32_t));
  const size_t sz_sel = align_up(std::max(select_ws_bytes(B, chunks_of(n_elig, kc_coarse), kc_coarse),
                                          select_ws_bytes(B, chunks_of(n_virt, kc_fine), kc_fine)));
  const size_t need = trivial ? kAlign : sz_coarse + sz_blocks + sz_nblk + sz_fine + sz_sel;
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al16(q_idx) || !al16(k_idx) || !al16(k_blk) || !al4(idx) || !al4(n_sel) || !al16(ws))
    return LSA_INVALID_ARG;
  s = load_weights(w, H_I, d_I, wa);
  if (s != LSA_OK) return s;
  if (ws_bytes < need) return LSA_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const SeqShift shift{ctx_len, 1, n_k};

  if (trivial) {
    SelectArgs sa{};
    sa.mode = SEL_FLAT;
    sa.n_rows = B;
    sa.n_q = 1;
    sa.q_off = t;
    sa.shift = shift;
    sa.n_sink = cfg.n_sink;
    sa.n_window = cfg.n_window;
    sa.k_dyn = cfg.k_dyn;
    sa.idx = idx;
    sa.n_sel = n_sel;
    sa.out_ld = K_tot;
    sa.k_cap = kc_fine;
    select_plan(sa, 1);
    return hip_status(launch_select(sa, st));
  }

  char* p = (char*)ws;
  int32_t* coarse = (int32_t*)p;
  p += sz_coarse;
  int32_t* blocks = (int32_t*)p;
  p += sz_blocks;
  int32_t* nblk = (int32_t*)p;
  p += sz_nblk;
  int32_t* fine = (int32_t*)p;
  p += sz_fine;
  void* sel_ws = p;

  // coarse scores of the eligible blocks
  ScoreArgs a{};
  a.w = wa;
  a.q = q_idx;
  a.k = k_blk;
  a.B = B;
  a.n_q = 1;
  a.n_k = nblocks;
  a.H_I = H_I;
  a.d_I = d_I;
  a.q_bstride = (int64_t)H_I * d_I;
  a.k_bstride = (int64_t)nblocks * d_I;
  a.s_bstride = nblocks;
  a.ld = nblocks;
  a.n_keys = b_hi + 1;
  a.mask_off = b_hi;
  a.pos_lo = b_lo;
  a.blocks = nullptr;
  a.fill_masked = 0;
  a.scores = coarse;
  s = hip_status(launch_index_score(a, st));
  if (s != LSA_OK) return s;

  // recall the best blocks (ascending ids, -1 padded)
  SelectArgs sc{};
  sc.mode = SEL_RAW;
  sc.scores = coarse;
  sc.ld = nblocks;
  sc.n_rows = B;
  sc.raw_lo = b_lo;
  sc.raw_hi = b_hi;
  sc.raw_k = n_blk_recall;
  sc.raw_hi_pos = hi;
  sc.raw_div = blk;
  sc.shift = shift;
  sc.idx = blocks;
  sc.n_sel = nblk;
  sc.out_ld = n_blk_recall;
  sc.k_cap = kc_coarse;
  select_plan(sc, n_elig);
  select_bind_ws(sc, sel_ws, B);
  s = hip_status(launch_select(sc, st));
  if (s != LSA_OK) return s;

  // fine scores of the candidate tokens inside the recalled blocks
  ScoreArgs f = a;
  f.k = k_idx;
  f.n_k = n_k;
  f.k_bstride = (int64_t)n_k * d_I;
  f.s_bstride = n_virt;
  f.ld = n_virt;
  f.n_keys = n_virt;
  f.mask_off = hi;
  f.pos_lo = lo;
  f.blocks = blocks;
  f.blk = blk;
  f.nbr = n_blk_recall;
  f.fill_masked = 1;
  f.scores = fine;
  f.shift = shift;
  s = hip_status(launch_index_score(f, st));
  if (s != LSA_OK) return s;

  SelectArgs sf{};
  sf.mode = SEL_INDIRECT;
  sf.scores = fine;
  sf.ld = n_virt;
  sf.n_rows = B;
  sf.n_sink = cfg.n_sink;
  sf.n_window = cfg.n_window;
  sf.k_dyn = cfg.k_dyn;
  sf.blocks = blocks;
  sf.blk = blk;
  sf.nbr = n_blk_recall;
  sf.n_virt = n_virt;
  sf.t_fixed = t;
  sf.shift = shift;
  sf.idx = idx;
  sf.n_sel = n_sel;
  sf.out_ld = K_tot;
  sf.k_cap = kc_fine;
  select_plan(sf, n_virt);
  select_bind_ws(sf, sel_ws, B);
  return hip_status(launch_select(sf, st));
}

extern "C" int32_t lsa_hier_select(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk,
                                   const int32_t* w, int32_t B, int32_t n_k, int32_t H_I,
                                   int32_t d_I, int32_t blk, int32_t n_blk_recall,
                                   lsa_select_cfg cfg, int32_t* idx, int32_t* n_sel, void* ws,
                                   size_t ws_bytes, size_t* ws_needed, void* stream) {
  return hier_select(q_idx, k_idx, k_blk, w, B, n_k, nullptr, H_I, d_I, blk, n_blk_recall, cfg, idx, n_sel, ws,
                     ws_bytes, ws_needed, stream);
}

extern "C" int32_t lsa_hier_select_ragged(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk,
                                          const int32_t* w, int32_t B, int32_t n_k, const int32_t* ctx_len,
                                          int32_t H_I, int32_t d_I, int32_t blk, int32_t n_blk_recall,
                                          lsa_select_cfg cfg, int32_t* idx, int32_t* n_sel, void* ws,
                                          size_t ws_bytes, size_t* ws_needed, void* stream) {
  if (!al4(ctx_len)) return LSA_INVALID_ARG;
  return hier_select(q_idx, k_idx, k_blk, w, B, n_k, ctx_len, H_I, d_I, blk, n_blk_recall, cfg, idx, n_sel, ws,
                     ws_bytes, ws_needed, stream);
}

extern "C" int32_t lsa_sparse_attn_prefill(const lsa_bf16* q, const lsa_bf16* k, const lsa_bf16* v,
                                           const int32_t* idx, const int32_t* n_sel, int32_t B,
                                           int32_t L, int32_t n_k, int32_t H, int32_t D,
                                           int32_t K_tot, float scale, lsa_bf16* o, float* lse,
                                           void* stream) {
  if (!al16(q) || !al16(k) || !al16(v) || !al4(idx) || !al4(n_sel) || !al16(o)) return LSA_INVALID_ARG;
  if (lse != nullptr && !al4(lse)) return LSA_INVALID_ARG;
  if (B <= 0 || L <= 0 || n_k <= 0 || K_tot <= 0 || !(scale > 0.f) || !isfinite(scale)) return LSA_INVALID_ARG;
  if (D != 128 || !heads_ok(H) || n_k > kMaxCacheKeys) return LSA_UNSUPPORTED;
  PrefillArgs a{q, k, v, idx, n_sel, B, L, n_k, H, K_tot, scale * 1.4426950408889634f, o, lse};
  return hip_status(launch_attn_prefill(a, (hipStream_t)stream));
}

static int32_t attn_decode(const lsa_bf16* q, const lsa_bf16* k_cache, const lsa_bf16* v_cache,
                           const int32_t* idx, const int32_t* n_sel, const int32_t* tgt_pos, int32_t n_idx,
                           int32_t B, int32_t n_q, int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                           int32_t n_split, float scale, lsa_bf16* o, float* lse, void* ws, size_t ws_bytes,
                           size_t* ws_needed, void* stream) {
  if (B <= 0 || n_q <= 0 || n_k <= 0 || K_tot <= 0 || !(scale > 0.f) || !isfinite(scale)) return LSA_INVALID_ARG;
  if (n_idx != 1 && n_idx != n_q) return LSA_INVALID_ARG;
  if (D != 128 || !heads_ok(H) || n_split < 1 || n_split > 64 || n_k > kMaxCacheKeys) return LSA_UNSUPPORTED;
  const size_t need = align_up(decode_ws_bytes(B, n_q, H, n_split));
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al16(q) || !al16(k_cache) || !al16(v_cache) || !al4(idx) || !al4(n_sel) || !al16(o) ||
      !al16(ws))
    return LSA_INVALID_ARG;
  if (lse != nullptr && !al4(lse)) return LSA_INVALID_ARG;
  if (ws_bytes < need) return LSA_WORKSPACE;
  const size_t rows = (size_t)B * n_split * n_q * H;
  DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.idx = idx;
  a.n_sel = n_sel;
  a.n_idx = n_idx;
  a.B = B;
  a.n_q = n_q;
  a.n_k = n_k;
  a.H = H;
  a.K_tot = K_tot;
  a.n_split = n_split;
  a.sl2 = scale * 1.4426950408889634f;
  a.o = o;
  a.lse = lse;
  a.ws_m = (float*)ws;
  a.ws_l = a.ws_m + rows;
  a.ws_o = (_Float16*)((char*)ws + align_up(rows * 2 * sizeof(float)));
  a.tgt_pos = tgt_pos;
  return hip_status(launch_attn_decode(a, (hipStream_t)stream));
}

extern "C" int32_t lsa_sparse_attn_decode(const lsa_bf16* q, const lsa_bf16* k_cache,
                                          const lsa_bf16* v_cache, const int32_t* idx,
                                          const int32_t* n_sel, int32_t n_idx, int32_t B,
                                          int32_t n_q, int32_t n_k, int32_t H, int32_t D,
                                          int32_t K_tot, int32_t n_split, float scale, lsa_bf16* o,
                                          float* lse, void* ws, size_t ws_bytes, size_t* ws_needed,
                                          void* stream) {
  return attn_decode(q, k_cache, v_cache, idx, n_sel, nullptr, n_idx, B, n_q, n_k, H, D, K_tot, n_split, scale, o,
                     lse, ws, ws_bytes, ws_needed, stream);
}

extern "C" int32_t lsa_sparse_attn_decode_mtp(const lsa_bf16* q, const lsa_bf16* k_cache,
                                              const lsa_bf16* v_cache, const int32_t* idx,
                                              const int32_t* n_sel, const int32_t* tgt_pos, int32_t B,
                                              int32_t n_q, int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                                              int32_t n_split, float scale, lsa_bf16* o, float* lse, void* ws,
                                              size_t ws_bytes, size_t* ws_needed, void* stream) {
  if (!al4(tgt_pos)) return LSA_INVALID_ARG;
  if (n_q > 32) return LSA_UNSUPPORTED;  // the drafts' keys fit one 32-key block
  return attn_decode(q, k_cache, v_cache, idx, n_sel, tgt_pos, 1, B, n_q, n_k, H, D, K_tot, n_split, scale, o,
                     lse, ws, ws_bytes, ws_needed, stream);
}

// ------------------------------------------------------------------ no-alloc
// Split-KV decode for callers that cannot allocate (code under graph capture,
// tight serving loops): the partials live in a fixed file-scope device array
// instead of a caller workspace. Each GPU the library runs on holds its own
// copy of the array until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address is looked up once per device, with that device
// current, and that address is what the launches get.
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, or null on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t lsa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int32_t lsa_sparse_attn_decode_noalloc(const lsa_bf16* q, const lsa_bf16* k_cache,
                                                  const lsa_bf16* v_cache, const int32_t* idx,
                                                  const int32_t* n_sel, int32_t n_idx, int32_t B, int32_t n_q,
                                                  int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                                                  int32_t n_split, float scale, lsa_bf16* o, float* lse,
                                                  void* stream) {
  // size checks first (no device call yet): the partials must fit the array
  size_t need = 0;
  const int32_t s = attn_decode(q, k_cache, v_cache, idx, n_sel, nullptr, n_idx, B, n_q, n_k, H, D, K_tot,
                                n_split, scale, o, lse, nullptr, 0, &need, stream);
  if (s != LSA_OK) return s;
  if (need > kNoAllocScratchBytes) return LSA_SCRATCH_LIMIT;
  void* ws = scratch_ptr();
  if (ws == nullptr) return LSA_HIP;
  return attn_decode(q, k_cache, v_cache, idx, n_sel, nullptr, n_idx, B, n_q, n_k, H, D, K_tot, n_split, scale,
                     o, lse, ws, kNoAllocScratchBytes, nullptr, stream);
}
