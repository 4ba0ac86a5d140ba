// Host-side launch interfaces shared between the LSA translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa.h"

namespace lsa {

// Per-head indexer weights travel in the kernel arguments.
struct WArgs {
  int32_t w[128];
};

// Indexer score launch. Row i of sequence b scores the virtual keys
// [0, n_keys); virtual key v sits at position v, or, when `blocks` is given, at
// blocks[b * nbr + v / blk] * blk + v % blk (a negative block id is invalid).
// A key at position p is visible to row i iff pos_lo <= p <= mask_off + i
// (+ the sequence's shift, below). Visible scores go to
// scores[b * s_bstride + i * ld + v]; invisible ones get INT32_MIN when
// fill_masked, else are left untouched.
// Ragged batches: with ctx_len set (device, one entry per sequence of the
// launch), sequence b holds L_b = clamp(ctx_len[b], ctx_rows, ctx_cap) keys
// and every visibility limit of its rows moves by L_b - ctx_cap.
struct SeqShift {
  const int32_t* ctx_len;
  int ctx_rows, ctx_cap;
};
__host__ __device__ inline int seq_shift(const SeqShift& s, int b) {
  if (s.ctx_len == nullptr) return 0;
  const int L = s.ctx_len[b] < s.ctx_rows ? s.ctx_rows : s.ctx_len[b];
  return (L < s.ctx_cap ? L : s.ctx_cap) - s.ctx_cap;
}
struct ScoreArgs {
  const int8_t* q;
  const int8_t* k;
  WArgs w;
  int B, n_q, n_k, H_I, d_I;
  int64_t q_bstride, k_bstride, s_bstride, ld;
  int n_keys;
  int mask_off, pos_lo;
  const int32_t* blocks;
  int blk, nbr;
  int fill_masked;
  int32_t* scores;
  SeqShift shift;
  // Many-row variant only (index_prefill below):
  // virtual key v is row v * kstride of k (0 or 1: row v);
  int kstride;
  // keys per workgroup (a multiple of 256; 0: the launch chooses);
  int chunk_keys;
  // non-null: only query tiles holding a row i with row_flags[i] != 0 run;
  const int32_t* row_flags;
  // non-null: filtered output. Instead of dense scores, row i keeps the
  // (score, position) pairs of its visible keys with score >= tau[i], in key
  // order, in the segment of its key chunk c = v / chunk_keys:
  // seg[2 * ((i * seg_chunks + c) * seg_cap + n)] for n < seg_cap, and
  // seg_cnt[i * seg_chunks + c] counts all of them (it may exceed seg_cap).
  // Needs B == 1 and chunk_keys set.
  const int32_t* tau;
  int32_t* seg;
  int32_t* seg_cnt;
  int seg_chunks, seg_cap;
};
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t st);
// Many-row variant (LDS-shared key tiles); covers direct keys (no blocks),
// H_I in {32, 64}, n_q >= 16, no ragged shift.
bool index_prefill_supported(const ScoreArgs& a);
hipError_t launch_index_prefill(const ScoreArgs& a, hipStream_t st);
// The keys per workgroup a launch of a with chunk_keys == 0 would take.
int index_prefill_auto_chunk(const ScoreArgs& a);
// Few-row variant (long per-wave key ranges streamed through registers);
// direct keys or a block table with blk >= 32, H_I in {32, 64, 128}.
bool index_decode_supported(const ScoreArgs& a);
hipError_t launch_index_decode(const ScoreArgs& a, hipStream_t st);

// Selection launch.
enum SelMode { SEL_FLAT = 0, SEL_RAW = 1, SEL_INDIRECT = 2 };
struct SelectArgs {
  int mode;
  const int32_t* scores;  // row r's scores at scores + r * ld, indexed by virtual key
  int64_t ld;
  int n_rows;
  // FLAT: row r is query r % n_q at t = q_off + r % n_q (+ the shift of its
  // sequence r / n_q when shift.ctx_len is set); candidates are the
  // positions [n_sink, t - n_window]; virtual key == position.
  // (row0 offsets the row count when a launch covers a slice of the rows.)
  int n_q, q_off, row0, n_sink, n_window, k_dyn;
  // RAW: candidates [raw_lo, raw_hi] (virtual == position), keep raw_k.
  // With shift.ctx_len set, row r (sequence row0 + r) stops at
  // min(raw_hi, floor((raw_hi_pos + its shift) / raw_div)) instead.
  int raw_lo, raw_hi, raw_k, raw_hi_pos, raw_div;
  SeqShift shift;
  // INDIRECT: candidates are virtual keys [0, n_virt) of row r, at positions
  // blocks[r * nbr + v / blk] * blk + v % blk, valid iff score != INT32_MIN;
  // the query sits at t_fixed (+ the shift of sequence row0 + r, whose row
  // keeps every position 0 .. t when t + 1 <= K_tot); keep k_dyn; sinks and
  // window as in FLAT.
  const int32_t* blocks;
  int blk, nbr, n_virt, t_fixed;
  // outputs: FLAT / INDIRECT write the assembled list (sinks, top-k, window),
  // RAW writes only the kept positions; both ascending, -1 padded to out_ld.
  int32_t* idx;
  int32_t* n_sel;
  int out_ld;
  // multi-chunk rows: per-chunk candidates in workspace
  int32_t* ws_score;
  int32_t* ws_pos;
  int32_t* ws_cnt;
  int max_chunks;  // chunks of the longest row (select_plan)
  // rows whose chunk survivors exceed one stage-B pass first reduce groups of
  // `group` chunks to k_cap survivors each into ws2 (0: no middle stage)
  int group;
  int32_t* ws2_score;
  int32_t* ws2_pos;
  int chunk_e;     // candidates per thread of a chunk (select_plan)
  int chunk_nt;    // threads of a stage-A workgroup (select_plan)
  int k_cap;
  // non-null: rows r with row_flags[r] == 0 are skipped
  const int32_t* row_flags;
};
// Chunk geometry for rows of at most max_nc candidates keeping k_cap each:
// the largest chunk count a plan can pick for such rows (workspace sizing),
// whether the stage-two input of such rows fits kSelMaxSurvivors, and a plan
// (from max_nc, a.n_rows and a.k_cap) that sets max_chunks, chunk_e and
// chunk_nt together.
int select_chunks(int64_t max_nc, int k_cap);
bool select_fits(int64_t max_nc, int k_cap);
void select_plan(SelectArgs& a, int64_t max_nc);
// Largest input of one reduction pass over chunk survivors; with the middle
// stage a row may have up to (kSelMaxSurvivors / k_cap)^2 chunks.
constexpr int64_t kSelMaxSurvivors = 32 * 1024;
size_t select_ws_bytes(int n_rows, int max_chunks, int k_cap);
void select_bind_ws(SelectArgs& a, void* ws, int n_rows);
hipError_t launch_select(const SelectArgs& a, hipStream_t st);

// Thresholded selection of long FLAT rows (B == 1, no ragged shift). A sample
// of every row's candidates (positions j * samp_m, scored exactly into
// samp[r * samp_ld + j]) gives a per-row score threshold tau[r] (a high-rank
// sample order statistic, INT32_MIN when the sample is too small); the full
// scoring pass then keeps only the pairs at or above it (ScoreArgs::tau), and
// the top-k of the row is the top-k of those survivors whenever they number
// at least k (and no segment overflowed): the selection is then exact. Rows
// where that fails get fail[r] = 1 and are redone by the dense path
// (row_flags of the score and select launches); the others get 0.
struct FilterArgs {
  SelectArgs sel;  // FLAT geometry and outputs of the rows (row0 == 0, no shift)
  const int32_t* samp;
  int64_t samp_ld;
  int samp_m;
  int32_t* tau;
  const int32_t* seg;
  const int32_t* seg_cnt;
  int seg_chunks, seg_cap;
  int32_t* fail;
};
// The sampled candidates of the rows number at most max_ns (<= 32768).
hipError_t launch_filter_threshold(const FilterArgs& f, int max_ns, hipStream_t st);
// Rows with more than max_surv survivors (<= filter_select_capacity()) are
// redone; seg_chunks <= 256.
int filter_select_capacity();
hipError_t launch_filter_select(const FilterArgs& f, int max_surv, hipStream_t st);

// Sparse attention launches (bf16 bit patterns as uint16_t; sl2 is
// scale * log2(e): softmax runs in base 2). K/V rows of one sequence are
// gathered with 32-bit byte offsets, which bounds n_k.
constexpr int32_t kMaxCacheKeys = (1 << 24) - 1;
struct PrefillArgs {
  const uint16_t *q, *k, *v;
  const int32_t *idx, *n_sel;
  int B, L, n_k, H, K_tot;
  float sl2;
  uint16_t* o;
  float* lse;
};
hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t st);

// Sparse attention backward, in row chunks. Row t of sequence b attends over
// idx[b, t, :n_sel] (distinct positions); o and lse are the forward's outputs
// for the same rows, d_o the gradient of the loss with respect to o. Phase 1
// (launch_attn_bwd) writes dq (bf16) of the chunk's rows [r0, r1) of the
// B * L rows and, for every (row, list slot) pair, the pair's contribution to
// the key's gradients: contrib[(row - r0) * K_tot + slot] holds 256 bf16, dk
// (scaled) then dv. Phase 2 (launch_bwd_scatter) lists the pairs of each key
// (counts, exclusive scan, fill) and sums each key's contributions as int64
// fixed point (value * 2^32) into dk_acc / dv_acc [B * n_k, 128], which start
// at zero before the first chunk; launch_attn_bwd_finish converts them.
struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *d_o;
  const float* lse;
  const int32_t *idx, *n_sel;
  int B, L, n_k, H, K_tot;
  float sl2;  // scale * log2(e)
  float scale;
  uint16_t* dq;
  int64_t r0, r1;
  uint16_t* contrib;
};
struct ScatterArgs {
  const int32_t *idx, *n_sel;
  int L, n_k, K_tot;
  int64_t r0, r1;
  int n_keys;               // B * n_k
  int32_t *cnt, *cur, *tot;  // [n_keys], [n_keys], [ceil(n_keys / 4096)]
  int32_t *lkey, *lpair;    // [(r1 - r0) * K_tot]
  const uint16_t* contrib;
  int64_t *dk_acc, *dv_acc;
};
constexpr int kScanBlock = 4096;
constexpr int kMaxScanKeys = kScanBlock * kScanBlock;
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_scatter(const ScatterArgs& a, hipStream_t st);
hipError_t launch_attn_bwd_finish(const int64_t* acc, float* out, size_t n, hipStream_t st);

// Warm-up KL operator: per row, KL(head-averaged attention distribution over
// the row's list || softmax of the row's logits) and its logit gradient.
struct KlArgs {
  const uint16_t *q, *k;
  const float* lse;
  const int32_t *idx, *n_sel;
  const float* logits;
  int B, L, n_k, H, K_tot;
  float sl2;  // scale * log2(e)
  float* kl;
  float* dlogits;
};
hipError_t launch_kl_warmup(const KlArgs& a, hipStream_t st);

struct DecodeArgs {
  const uint16_t *q, *k, *v;
  const int32_t *idx, *n_sel;
  int n_idx, B, n_q, n_k, H, K_tot, n_split;
  float sl2;
  uint16_t* o;
  float* lse;
  float *ws_m, *ws_l;
  _Float16* ws_o;
  const int32_t* tgt_pos;  // MTP causal tails (n_idx == 1), or null
};
size_t decode_ws_bytes(int B, int n_q, int H, int n_split);
hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t st);

// HI block summary launch: blocks [j0, j0 + nbj) of k [B, n_cap, d_I] with
// n_len keys present, into kb [B, ceil(n_cap / blk), d_I].
hipError_t launch_block_summary(const int8_t* k, int B, int n_cap, int n_len, int d_I, int blk, int j0,
                                int nbj, int8_t* kb, hipStream_t st);

// MTP draft rows' lists: the target's list plus the drafts up to each row.
hipError_t launch_mtp_index(const int32_t* idx, const int32_t* n_sel, int B, int K_tot, int n_q,
                            const int32_t* tgt_pos, int32_t* idx_rows, int32_t* n_sel_rows, hipStream_t st);

// Brackets one kernel launch with HIP events on its stream while kernel
// timing (lsa_kernel_timing) is on; name is the kernel's base name.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t st);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  void* a_;
};

}  // namespace lsa
