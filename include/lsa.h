/*
 * lsa.h — C ABI of the LongCat Sparse Attention (LSA) hot path on MI355X (gfx950).
 *
 * What the calls compute (page title, section):
 *   LongCat-2.0 release article (techsir.com), section "LongCat 稀疏注意力":
 *     a lightweight indexer scores the cached keys for each query; the
 *     streaming-aware indexing (SI) paragraph mixes a contiguous, hardware-
 *     aligned read with dynamically chosen keys; the cross-layer indexing (CLI)
 *     paragraph reuses one index across consecutive layers and across the
 *     three MTP draft steps; the hierarchical indexing (HI) paragraph scores
 *     blocks coarsely and then tokens inside the recalled blocks.
 *   "如何在 5 万张国产芯片训练出 1.6T 万亿参数模型？", section "架构拆解 ① LSA":
 *     each query reads only the top-k keys plus a few fixed sink tokens.
 *   same page, section "③ KVP 解码切分示意": partial attention over parts of
 *     the KV cache, merged afterwards (here: split-KV with a log-sum-exp merge).
 *
 * Indexer arithmetic (the pages leave it open; this library fixes it):
 *   S[t, s] = sum_h w[h] * max(0, sum_d q_idx[t, h, d] * k_idx[s, d])
 * with int8 q_idx / k_idx, int32 weights and an exact int32 result. Selection
 * keeps sinks 0..n_sink-1, the window t-n_window+1..t and the k_dyn best of the
 * candidates n_sink..t-n_window by (score descending, position ascending); a
 * query with t+1 <= K_tot keeps every key 0..t. Output lists are ascending,
 * padded with -1 past n_sel.
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned, contiguous, row-major DEVICE buffers, 16-byte
 *     aligned, except `w`, which is a short HOST array (copied into the kernel
 *     arguments at the call). The library never allocates or frees memory.
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream) and the call returns after enqueueing.
 *   - Argument errors are returned synchronously before anything is launched;
 *     a kernel fault surfaces at the caller's next synchronisation.
 *   - Position lists (`idx`) given to the attention calls are trusted to be
 *     < n_k; entries outside [0, n_k) are skipped rather than read.
 *   - Workspace: pass ws = NULL to get the byte count in *ws_needed; then pass
 *     a device buffer of at least that size. Workspace content is scratch.
 *   - Results are deterministic: repeated calls give bit-identical outputs
 *     (no floating-point atomics; fixed reduction and merge orders).
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t lsa_bf16; /* bfloat16 bit pattern */

/* Selection budget: K_tot = n_sink + n_window + k_dyn. n_window = 0 turns the
 * SI window off; k_dyn = 0 keeps only sinks and window. */
typedef struct {
  int32_t n_sink;
  int32_t n_window;
  int32_t k_dyn;
} lsa_select_cfg;

enum {
  LSA_OK = 0,
  LSA_INVALID_ARG = 1, /* NULL, misaligned, non-positive or inconsistent sizes */
  LSA_UNSUPPORTED = 2, /* shape outside the tuned set (see each call)         */
  LSA_WORKSPACE = 3,   /* workspace too small                                 */
  LSA_RANGE = 4,       /* sum_h |w[h]| * d_I * 128 * 128 >= 2^31: int32 not exact */
  LSA_HIP = 5,         /* a HIP launch reported an error                       */
  LSA_SCRATCH_LIMIT = 6 /* sizes exceed the fixed scratch of a no-alloc call    */
};

/* Human-readable name of a status code (static storage). */
const char* lsa_status_string(int32_t status);

/* Indexer scores (step "index first" of the LSA section).
 *   q_idx  [B, n_q, H_I, d_I] int8 ; query row i of each sequence sits at
 *                                    position q_off + i
 *   k_idx  [B, n_k, d_I] int8
 *   w      [H_I] int32, HOST array
 *   scores [B, n_q, n_k] int32 out: S for s <= q_off + i, INT32_MIN otherwise
 * Supported: d_I in {64, 128}; H_I in {4, 8, 16, 32, 64, 128}. */
int32_t lsa_index_score(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                        int32_t B, int32_t n_q, int32_t n_k, int32_t H_I, int32_t d_I,
                        int32_t q_off, int32_t* scores, void* stream);

/* Flat selection: sinks + SI window + dynamic top-k (SI paragraph; sinks).
 *   scores  [B, n_q, n_k] int32 as written by lsa_index_score, or NULL: then
 *           the call scores q_idx / k_idx / w itself (fused indexer + top-k)
 *   idx     [B, n_q, K_tot] int32 out, ascending, -1 padded
 *   n_sel   [B, n_q] int32 out, min(q_off + i + 1, K_tot)
 * Requires q_off + n_q <= n_k. A row's candidates are selected in chunks of
 * 32768 whose survivors (k_dyn each, rounded up to a multiple of 4: k_cap)
 * are reduced in at most two further passes of 32768 entries: rows of up to
 * (32768 / k_cap)^2 chunks are supported (8388608 candidates at k_dyn =
 * 2048), longer ones return LSA_UNSUPPORTED. The limit is checked against the
 * longest row the call can see (for lsa_select_topk_ragged: the cache
 * capacity n_k).
 * Fused path, one sequence per pass (prefill): rows with at least 16384
 * candidates first score every 64th candidate; a high order statistic of that
 * sample is a per-row threshold, the full scoring pass keeps only the
 * (score, position) pairs at or above it, and the row's top-k is taken from
 * those survivors when they number at least k_dyn (then exactly the same
 * list). Rows where that does not hold are scored and selected again in
 * full within the same call, so the result never depends on the sample. */
int32_t lsa_select_topk(const int32_t* scores, const int8_t* q_idx, const int8_t* k_idx,
                        const int32_t* w, int32_t B, int32_t n_q, int32_t n_k, int32_t H_I,
                        int32_t d_I, int32_t q_off, lsa_select_cfg cfg, int32_t* idx,
                        int32_t* n_sel, void* ws, size_t ws_bytes, size_t* ws_needed,
                        void* stream);

/* Flat selection for a decode batch whose sequences hold different numbers of
 * cached keys (a ragged batch); the same selection as lsa_select_topk (SI
 * paragraph; sinks), fused with the scoring.
 *   ctx_len [B] int32, DEVICE: keys held by each sequence, read on the GPU
 *           and clamped to [n_q, n_k] (so a bad length cannot read past the
 *           cache); L_b = clamp(ctx_len[b], n_q, n_k)
 *   q_idx [B, n_q, H_I, d_I] int8; k_idx [B, n_k, d_I] int8, n_k the cache
 *           capacity; only keys 0 .. L_b - 1 of sequence b are ever visible
 *   query row i of sequence b sits at position t = L_b - n_q + i (the last
 *   n_q positions of the sequence)
 *   idx [B, n_q, K_tot] int32 out, ascending, -1 padded; n_sel [B, n_q] out,
 *   min(t + 1, K_tot)
 * The workspace is sized for full-length sequences (L_b = n_k). Errors as
 * lsa_select_topk; ctx_len NULL or misaligned is LSA_INVALID_ARG. */
int32_t lsa_select_topk_ragged(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                               int32_t B, int32_t n_q, int32_t n_k, int32_t H_I, int32_t d_I,
                               const int32_t* ctx_len, lsa_select_cfg cfg, int32_t* idx,
                               int32_t* n_sel, void* ws, size_t ws_bytes, size_t* ws_needed,
                               void* stream);

/* HI block summary: k_blk[b, j, :] = clamp(round-half-even(mean of the keys of
 * block j), -128, 127); a tail block of c < blk keys uses its own mean.
 *   k_idx [B, n_k, d_I] int8 -> k_blk [B, ceil(n_k / blk), d_I] int8
 * Supported: blk in [1, 1024]; d_I in {64, 128}. */
int32_t lsa_block_summary(const int8_t* k_idx, int32_t B, int32_t n_k, int32_t d_I,
                          int32_t blk, int8_t* k_blk, void* stream);

/* HI block summaries kept current while keys are appended to a cache (same
 * summary as lsa_block_summary; HI paragraph). k_idx [B, n_cap, d_I] holds
 * n_new keys per sequence, of which keys n_old .. n_new-1 are new; k_blk
 * [B, ceil(n_cap / blk), d_I] holds the summaries of the first n_old keys.
 * Recomputes only the blocks the new keys fall in (block n_old / blk, which
 * may have been a partial tail, up to block (n_new - 1) / blk); afterwards
 * rows 0 .. ceil(n_new / blk) - 1 of k_blk equal lsa_block_summary of the
 * first n_new keys. Rows past that are not touched.
 * Requires 0 <= n_old <= n_new <= n_cap (n_old == n_new does nothing).
 * Supported: blk in [1, 1024]; d_I in {64, 128}. */
int32_t lsa_block_summary_append(const int8_t* k_idx, int32_t B, int32_t n_cap, int32_t n_old,
                                 int32_t n_new, int32_t d_I, int32_t blk, int8_t* k_blk,
                                 void* stream);

/* HI decode selection for the query at position n_k - 1 (HI paragraph).
 * Coarse: blocks intersecting the candidate range are scored with the indexer
 * formula against k_blk; the n_blk_recall best (score desc, block asc) are
 * recalled. Fine: candidate tokens inside them are scored and the best
 * min(k_dyn, #candidates) kept; sinks and window added as in the flat case.
 *   q_idx [B, H_I, d_I] int8, k_idx [B, n_k, d_I], k_blk from lsa_block_summary
 *   idx [B, K_tot] int32 out (ascending, -1 padded), n_sel [B] int32 out
 * Supported: blk a multiple of 32 in [32, 1024]. */
int32_t lsa_hier_select(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk,
                        const int32_t* w, int32_t B, int32_t n_k, int32_t H_I, int32_t d_I,
                        int32_t blk, int32_t n_blk_recall, lsa_select_cfg cfg, int32_t* idx,
                        int32_t* n_sel, void* ws, size_t ws_bytes, size_t* ws_needed,
                        void* stream);

/* HI decode selection for a ragged batch (HI paragraph; as lsa_hier_select,
 * per sequence). Sequence b holds L_b = clamp(ctx_len[b], 1, n_k) keys of its
 * cache and its query sits at L_b - 1; only those keys are ever candidates.
 *   ctx_len [B] int32, DEVICE, read on the GPU
 *   k_idx [B, n_k, d_I], n_k the cache capacity; k_blk [B, ceil(n_k / blk),
 *   d_I] whose first ceil(L_b / blk) rows of sequence b summarize its first
 *   L_b keys (lsa_block_summary / lsa_block_summary_append per sequence)
 *   idx [B, K_tot] out, ascending, -1 padded; n_sel [B] out, min(L_b, K_tot)
 *     when all candidates fit the recalled blocks
 * The workspace is sized for full-length sequences. Errors as
 * lsa_hier_select; ctx_len NULL or misaligned is LSA_INVALID_ARG. */
int32_t lsa_hier_select_ragged(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk,
                               const int32_t* w, int32_t B, int32_t n_k, const int32_t* ctx_len,
                               int32_t H_I, int32_t d_I, int32_t blk, int32_t n_blk_recall,
                               lsa_select_cfg cfg, int32_t* idx, int32_t* n_sel, void* ws,
                               size_t ws_bytes, size_t* ws_needed, void* stream);

/* Fused HI decode step (a "super kernel": LongCat-2.0 release article, section
 * "面向国产算力芯片的优化" on fusing small operators into one kernel; the 1.6T
 * write-up, section "② 设备层"): the block recall, token selection and split-KV
 * attention of one decode step, with the query at position n_k - 1 of each
 * sequence, in two launches (a tiny counter fill and one persistent kernel
 * whose workgroups take the step's work items in dependency order). The
 * results equal lsa_hier_select followed by lsa_sparse_attn_decode (n_q = 1,
 * n_idx = 1) bit for bit; idx / n_sel are written as lsa_hier_select writes
 * them, so later layers can reuse them (CLI).
 *   q_idx [B, H_I, d_I] int8, k_idx [B, n_k, d_I], k_blk [B, ceil(n_k / blk),
 *   d_I] (lsa_block_summary), w [H_I] host; q [B, 1, H, D] bf16, k_cache /
 *   v_cache [B, n_k, D] bf16
 *   idx [B, K_tot], n_sel [B] out; o [B, 1, H, D] bf16 out; lse [B, 1, H] or NULL
 * Supported: H_I = 64, d_I = 128, H = 64, D = 128, one query row per
 * sequence, n_split in [1, 8], blk a multiple of 32 in [32, 1024], at most
 * 16384 eligible blocks and n_blk_recall * blk <= 16384, n_k > K_tot (shorter
 * contexts: lsa_hier_select); LSA_UNSUPPORTED otherwise. The workspace's first
 * 256 bytes hold the step's counters; word 1 is set if a wait ever exceeded
 * its bound (never in a correct run: the bound only keeps a fault from
 * hanging the GPU). Errors otherwise as lsa_hier_select. */
int32_t lsa_hier_decode_step(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk, const int32_t* w,
                             const lsa_bf16* q, const lsa_bf16* k_cache, const lsa_bf16* v_cache, int32_t B,
                             int32_t n_k, int32_t H_I, int32_t d_I, int32_t blk, int32_t n_blk_recall,
                             lsa_select_cfg cfg, int32_t H, int32_t D, int32_t n_split, float scale,
                             int32_t* idx, int32_t* n_sel, lsa_bf16* o, float* lse, void* ws, size_t ws_bytes,
                             size_t* ws_needed, void* stream);

/* MTP draft rows that also see the drafts before them (a causal variant of the
 * index reuse across the MTP draft steps, CLI paragraph). The target row of
 * sequence b sits at tgt_pos[b]; draft row j (1 <= j < n_q) sits at
 * tgt_pos[b] + j, its key and value already appended to the cache. Row j's
 * list is the target's list followed by tgt_pos[b] + 1 .. tgt_pos[b] + j;
 * row 0's is the target's list.
 *   idx [B, K_tot], n_sel [B]: the target's selection (positions <= tgt_pos)
 *   tgt_pos [B] int32, DEVICE
 *   idx_rows [B, n_q, K_tot + n_q - 1] int32 out, ascending, -1 padded;
 *   n_sel_rows [B, n_q] int32 out (n_sel + j)
 * Pass them to lsa_sparse_attn_decode with n_idx = n_q and K_tot + n_q - 1.
 * Errors: LSA_INVALID_ARG for NULL/misaligned pointers or non-positive sizes. */
int32_t lsa_mtp_row_index(const int32_t* idx, const int32_t* n_sel, int32_t B, int32_t K_tot,
                          int32_t n_q, const int32_t* tgt_pos, int32_t* idx_rows, int32_t* n_sel_rows,
                          void* stream);

/* Sparse attention, prefill: query row t of sequence b attends over the keys
 * idx[b, t, 0 .. n_sel[b, t]-1] of its sequence (one KV head shared by H query
 * heads); softmax(scale * q.k) in fp32, output bf16. Passing the same idx to
 * consecutive layers is cross-layer index reuse (CLI paragraph). Each row's
 * list must be strictly ascending with no duplicates, as the selection writes
 * it: two neighbouring rows whose lists end in runs of consecutive positions
 * (their SI windows) attend those runs through one shared gather, and a run is
 * recognised from its first and last entries.
 *   q [B, L, H, D] bf16, k / v [B, n_k, D] bf16, idx [B, L, K_tot], n_sel [B, L]
 *   o [B, L, H, D] bf16 out; lse [B, L, H] fp32 out (natural log) or NULL
 * Supported: D = 128; H in {16, 32, 64, 128}; n_k <= 16777215 (cache rows are
 * addressed with 32-bit byte offsets). */
int32_t lsa_sparse_attn_prefill(const lsa_bf16* q, const lsa_bf16* k, const lsa_bf16* v,
                                const int32_t* idx, const int32_t* n_sel, int32_t B,
                                int32_t L, int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                                float scale, lsa_bf16* o, float* lse, void* stream);

/* Sparse attention, decode with split-KV and a log-sum-exp merge (KVP section,
 * one-GPU form). The selected list of each index row is cut into n_split
 * contiguous parts of ceil(n_sel / n_split) entries; each part yields
 * (max, sum, output) partials, merged over parts in a fixed binary tree.
 * The partials live in the workspace: max and sum in fp32, each part's output
 * normalised by its own sum in fp16 (rounded to nearest).
 *   q [B, n_q, H, D] bf16; k_cache / v_cache [B, n_k, D] bf16
 *   idx [B, n_idx, K_tot], n_sel [B, n_idx]; n_idx = 1: every query row of a
 *   sequence uses the one index (MTP draft reuse), else n_idx = n_q
 *   o [B, n_q, H, D] bf16 out; lse [B, n_q, H] fp32 out or NULL
 * Supported: D = 128; H in {16, 32, 64, 128}; n_split in [1, 64];
 * n_k <= 16777215. */
int32_t lsa_sparse_attn_decode(const lsa_bf16* q, const lsa_bf16* k_cache,
                               const lsa_bf16* v_cache, const int32_t* idx,
                               const int32_t* n_sel, int32_t n_idx, int32_t B, int32_t n_q,
                               int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                               int32_t n_split, float scale, lsa_bf16* o, float* lse,
                               void* ws, size_t ws_bytes, size_t* ws_needed, void* stream);

/* Sparse attention backward, deterministic (training; "如何在 5 万张国产芯片训练出
 * 1.6T 万亿参数模型？", section "④ 痛点③：长上下文训练三招": the LSA operator comes with
 * deterministic attention operators; haoling.cc article, section 三: a
 * deterministic attention backward and deterministic scatter operators).
 * Gradients of a loss L through o = lsa_sparse_attn_prefill(q, k, v, idx,
 * n_sel), given d_o = dL/do:
 *   dq[t, h] = scale sum_s dS[t,h,s] k[s],  dk[s] = scale sum_{t,h} dS[t,h,s] q[t,h],
 *   dv[s] = sum_{t,h} P[t,h,s] d_o[t,h],     dS = P (d_o . v_s - sum_d d_o . o)
 * over the keys s of each row's list; a key's gradient sums the contributions
 * of every row that selected it. P is recomputed from lse.
 *   q, d_o, o [B, L, H, D] bf16 (o: the forward's output); lse [B, L, H] fp32
 *   (the forward's natural-log lse); k, v [B, n_k, D] bf16; idx [B, L, K_tot],
 *   n_sel [B, L]: each row's list of distinct positions (as the selection
 *   writes them)
 *   dq [B, L, H, D] bf16 out; dk, dv [B, n_k, D] fp32 out (keys no row
 *   selected get 0)
 * Each (row, key) pair's contribution to dk and dv (a sum over the H heads)
 * is stored once in bf16; the pairs of each key are listed, and each key's
 * contributions are summed as int64 fixed point (value * 2^32, exact for
 * values at or above 2^-24 in magnitude). Integer sums do not depend on the
 * order of their terms, so repeated calls are bit-identical; the rounding
 * beyond fp32 arithmetic is the bf16 of each contribution. Every partial sum
 * of one element must stay below 2^31 in magnitude (the int64 range).
 * Rows are processed in chunks whose contributions fit 8 GiB.
 *   ws: query with ws = NULL (about 2 * B * n_k * 1 KiB of accumulators plus
 *   up to 8 GiB of contributions and 8 bytes per (row, slot) of a chunk)
 * Supported: D = 128; H in {32, 64, 128}; n_k <= 16777215; B * n_k <= 2^24.
 * Errors: LSA_INVALID_ARG for NULL/misaligned pointers or bad sizes,
 * LSA_UNSUPPORTED for other shapes, LSA_WORKSPACE, LSA_HIP. */
int32_t lsa_sparse_attn_backward(const lsa_bf16* q, const lsa_bf16* k, const lsa_bf16* v,
                                 const int32_t* idx, const int32_t* n_sel, const lsa_bf16* o,
                                 const float* lse, const lsa_bf16* d_o, int32_t B, int32_t L,
                                 int32_t n_k, int32_t H, int32_t D, int32_t K_tot, float scale,
                                 lsa_bf16* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                 size_t* ws_needed, void* stream);

/* LSA warm-up KL operator (LongCat-2.0 release article, section "长上下文训练",
 * paragraph "LSA 算子与前向优化": a KL-loss operator whose single forward pass
 * gives both the loss and its gradient). For query row t of sequence b with
 * key list idx[b, t, :n] (n = n_sel[b, t]; the selected keys, or every key
 * 0..t for a dense warm-up) and indexer logits logits[b, t, :n] of those keys:
 *   p_j  = (1/H) sum_h exp(scale q[t,h] . k[idx_j] - lse[t,h])   (the row's
 *          attention distribution averaged over its H heads; lse is the
 *          forward's, lsa_sparse_attn_prefill over the same lists)
 *   kl[b, t] = sum_j p_j (log p_j - log softmax(logits)_j)
 *   dlogits[b, t, j] = softmax(logits)_j - p_j  (d kl / d logits; 0 for j >= n)
 * No gradient flows into the attention (warm-up trains the indexer alone).
 *   q [B, L, H, D] bf16, k [B, n_k, D] bf16, lse [B, L, H] fp32, idx / n_sel as
 *   for lsa_sparse_attn_prefill (distinct positions), logits [B, L, K_tot] fp32
 *   kl [B, L] fp32 out (a row with n = 0 gets 0), dlogits [B, L, K_tot] fp32 out
 * Deterministic: the head and key sums run in a fixed order.
 * Supported: D = 128; H in {32, 64, 128}; n_k <= 16777215.
 * Errors: LSA_INVALID_ARG for NULL/misaligned pointers or bad sizes,
 * LSA_UNSUPPORTED for other shapes, LSA_HIP. */
int32_t lsa_kl_warmup(const lsa_bf16* q, const lsa_bf16* k, const int32_t* idx, const int32_t* n_sel,
                      const float* lse, const float* logits, int32_t B, int32_t L, int32_t n_k, int32_t H,
                      int32_t D, int32_t K_tot, float scale, float* kl, float* dlogits, void* stream);

/* lsa_sparse_attn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the split-KV partials in
 * a fixed scratch array inside the library instead of a caller workspace. The
 * array holds lsa_noalloc_scratch_bytes() bytes (40 MiB; C3's batch of 64
 * sequences x 8 parts x 4 rows x 64 heads needs 35 MB) per GPU, allocated
 * with the library's code on each device and held until the process ends.
 * The call allocates nothing and issues no memset: every partial is written
 * before it is read. Calls that overlap on one GPU (several streams or host
 * threads) share that array and race; serialize them.
 *   arguments as lsa_sparse_attn_decode, without ws / ws_bytes / ws_needed
 * Errors: as lsa_sparse_attn_decode; LSA_SCRATCH_LIMIT when the partials
 * (B * n_split * n_q * H rows of 264 bytes) exceed the array; LSA_HIP when the
 * array's device address cannot be found. */
int32_t lsa_sparse_attn_decode_noalloc(const lsa_bf16* q, const lsa_bf16* k_cache,
                                       const lsa_bf16* v_cache, const int32_t* idx,
                                       const int32_t* n_sel, int32_t n_idx, int32_t B, int32_t n_q,
                                       int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                                       int32_t n_split, float scale, lsa_bf16* o, float* lse,
                                       void* stream);
size_t lsa_noalloc_scratch_bytes(void);

/* The same split-KV decode for MTP rows with causal tails, without building
 * per-row lists: all n_q rows of a sequence share the target's list idx
 * (n_idx = 1), and row j (1 <= j < n_q, at position tgt_pos[b] + j)
 * additionally attends to tgt_pos[b] + 1 .. tgt_pos[b] + j, the drafts' keys
 * already in the cache; row 0 attends to the list alone. Equal, up to the
 * order of float accumulation, to lsa_sparse_attn_decode over the lists of
 * lsa_mtp_row_index. The drafts' keys join the last of the n_split parts.
 *   idx [B, 1, K_tot], n_sel [B, 1]; tgt_pos [B] int32, DEVICE; the rest as
 *   lsa_sparse_attn_decode (same workspace size)
 * Supported: as lsa_sparse_attn_decode, and n_q <= 32. */
int32_t lsa_sparse_attn_decode_mtp(const lsa_bf16* q, const lsa_bf16* k_cache,
                                   const lsa_bf16* v_cache, const int32_t* idx,
                                   const int32_t* n_sel, const int32_t* tgt_pos, int32_t B,
                                   int32_t n_q, int32_t n_k, int32_t H, int32_t D, int32_t K_tot,
                                   int32_t n_split, float scale, lsa_bf16* o, float* lse,
                                   void* ws, size_t ws_bytes, size_t* ws_needed, void* stream);

/* Kernel timing, a measurement aid (not part of the method). While on, every
 * kernel launch of the library is bracketed by two HIP events recorded on
 * the launch stream; a launch costs two event records more.
 *   lsa_kernel_timing(on): waits for the events still pending, clears all
 *     records, then starts (on != 0) or stops (on == 0) recording.
 *   lsa_kernel_time(name, ms_mean, launches): mean duration in ms and count
 *     of the recorded launches of kernel `name` (waits for their events).
 *     Names: "index_prefill_kernel", "index_decode_kernel",
 *     "index_score_kernel", "select_stage_a", "select_stage_m",
 *     "select_stage_b", "filter_threshold_kernel", "filter_select_kernel",
 *     "attn_prefill_kernel", "attn_decode_partial", "attn_decode_merge",
 *     "block_summary_kernel", "mtp_index_kernel", "hi_step_kernel",
 *     "attn_bwd_kernel", "bwd_count_kernel", "bwd_scan_kernel",
 *     "bwd_fill_kernel", "bwd_reduce_kernel", "attn_bwd_finish_kernel",
 *     "kl_warmup_kernel", "fill_zero_kernel". An unknown name reports 0
 *     launches. While timing is off (the default) no event is created and
 *     a launch pays one relaxed load.
 * Errors: LSA_INVALID_ARG for NULL pointers, LSA_HIP for a failed event call.
 * Not for concurrent use from several host threads while launches run. */
int32_t lsa_kernel_timing(int32_t on);
int32_t lsa_kernel_time(const char* name, float* ms_mean, int32_t* launches);

/* Matrix-core peak probe, a measurement aid (not part of the method): enqueues
 * n_wg workgroups of 4 waves, each wave issuing `iters` rounds of 8
 * independent MFMA instructions on register operands (no memory traffic),
 * so that the caller's event timing of the launch gives the rate the chip
 * sustains at its current clock.
 *   kind 0: v_mfma_i32_32x32x32_i8 (65536 int8 ops each); kind 1:
 *   v_mfma_f32_32x32x16_bf16 (32768 flop each)
 *   sink [n_wg] int32, DEVICE: one value per workgroup (keeps results live)
 *   *ops (may be NULL): the operations one launch performs
 * Errors: LSA_INVALID_ARG for a NULL or misaligned sink or non-positive
 * sizes, LSA_UNSUPPORTED for another kind, LSA_HIP for a launch error. */
int32_t lsa_probe_mfma(int32_t kind, int32_t n_wg, int32_t iters, int32_t* sink, double* ops, void* stream);

/* The same probe with operands from caller data: every lane loads 8 A and 8
 * B fragments of 16 bytes (lane t of the grid reads 16-byte units
 * 8t .. 8t + 7 of a and 8t + 3 .. 8t + 10 of b, each index taken modulo the
 * array's unit count) and chain j multiplies A fragment j by B fragment
 * j + 1, so consecutive instructions see different operands. Passing arrays
 * of the kernel's own operands (the indexer's folded query bytes and key
 * bytes; bf16 keys and queries) gives the rate the matrix cores sustain on
 * that data: their power draw grows with the number of operand bits that
 * switch between instructions, and the clock the chip holds falls with it.
 *   kind, n_wg, iters, sink, ops, stream: as lsa_probe_mfma
 *   a, b: DEVICE, 16-byte aligned, read only; a_bytes, b_bytes >= 16 (a
 *     trailing part shorter than 16 bytes is not read)
 * Errors: LSA_INVALID_ARG for NULL or misaligned pointers, sizes below 16 or
 * non-positive counts, LSA_UNSUPPORTED for another kind, LSA_HIP for a
 * launch error. */
int32_t lsa_probe_mfma_data(int32_t kind, int32_t n_wg, int32_t iters, const void* a, int64_t a_bytes, const void* b,
                            int64_t b_bytes, int32_t* sink, double* ops, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
