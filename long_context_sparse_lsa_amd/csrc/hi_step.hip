// Fused HI decode step: block recall, token selection and split-KV sparse
// attention of one decode step in one persistent launch (a "super kernel").
//
// The LongCat-2.0 release article (section "面向国产算力芯片的优化", Super Kernel)
// and the 1.6T write-up (section "② 设备层", ① Super Kernel) fuse the small
// operators of a decode step into one kernel to cut launch overhead. Here the
// HI path (the release article's "LongCat 稀疏注意力" HI paragraph) runs as a
// queue of work items taken in order by a fixed grid of workgroups:
//   1. coarse: indexer scores of the eligible blocks' summary keys, in tiles
//   2. recall: per sequence, the n_blk_recall best blocks (score desc, block asc)
//   3. fine:   indexer scores of the candidate tokens in the recalled blocks
//   4. select: per sequence, the k_dyn best tokens; sinks and window added
//   5. attend: per sequence and part of the list, split-KV partials
//   6. merge:  per sequence, the log-sum-exp merge of the parts
// The same device code as the separate kernels does each item (score_dev.h,
// select_dev.h, attn_dev.h), so the results are those of lsa_hier_select
// followed by lsa_sparse_attn_decode, bit for bit.
//
// A workgroup takes a ticket from a counter; ticket order is the phase order
// above, so an item only ever waits for items with smaller tickets, which are
// held by workgroups already running: the queue always drains. An item waits
// on per-sequence completion counters (an agent-scope acquire after its
// producers' agent-scope release), so sequence b's recall starts as soon as
// b's coarse tiles are done. Every wait is bounded: past kSpinLimit polls it
// sets the error word and goes on, so a fault cannot become a hang.
#include <math.h>

#include <algorithm>

#include "attn_dev.h"
#include "lsa_device.h"
#include "lsa_internal.h"
#include "score_dev.h"
#include "select_dev.h"

namespace lsa {

namespace {

constexpr int kStepThreads = 512;  // 8 waves: the attention part's 2 head groups x 4 key subranges
constexpr int kSelE = 32;          // selection keys per thread: 16384 per sequence and stage
constexpr int kTileKeys = 512;     // keys scored per scoring item (64 per wave)
constexpr int kSpinLimit = 1 << 22;
using StepCfg = DecodeCfg<2, 4>;
constexpr int kUnion = std::max<int>(std::max<int>(StepCfg::kBytes, (int)sizeof(SelShared<kStepThreads>)),
                                     8 * kMaxBlkIds * 4);

// sync words: 0 ticket, 1 error, then per sequence: coarse tiles done,
// recall done, fine tiles done, selection done, parts done
constexpr int kSyncPerSeq = 5;
enum { kCoarse = 0, kRecall = 1, kFine = 2, kSel = 3, kAttn = 4 };

// Everything the items read. The kernel copies it to LDS once, so that the
// items reload fields after each barrier instead of holding ~100 uniform
// values live in scalar registers across the item loop.
struct HiStepArgs {
  const int8_t *q_idx, *k_blk, *k_idx;
  const int32_t* blocks_ro;  // the recalled blocks, as the fine scorer reads them
  int fold_ok;
  int B, n_k, blk, n_rec, b_lo, b_hi, n_virt, t, lo, hi, n_sink, n_window, k_dyn, K_tot;
  int32_t* coarse_sc;  // [B, nblocks]
  int32_t* blocks;     // [B, n_rec]
  int32_t* fine_sc;    // [B, n_virt]
  int32_t* idx;        // [B, K_tot]
  int32_t* n_sel;      // [B]
  int nblocks;
  int tiles_c, tiles_f;
  int32_t* sync;
  DecodeArgs att;
};
static_assert(kUnion + 512 + 16 + (int)sizeof(HiStepArgs) <= 160 * 1024, "LDS");

__device__ __forceinline__ int* seq_word(const HiStepArgs& a, int b, int k) { return a.sync + 2 + kSyncPerSeq * b + k; }

__device__ __forceinline__ void wait_count(const HiStepArgs& a, int* w, int target) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(a.sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ void signal_done(int* w) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // every wave's stores of the item
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Top k of n int32 scores (INT32_MIN: not a candidate) by (score desc, index
// asc); emit(o, i) for the kept indices i in ascending order. Returns the count.
template <class Emit>
__device__ __forceinline__ int select_top(const int32_t* row, int n, int k, SelShared<kStepThreads>& sh, Emit emit) {
  uint32_t u[kSelE];
  load_keys<kSelE>(row, 0, n, u);
  int n_valid;
  uint32_t kmin, kmax, T;
  int shift, r_eq;
  chunk_stats<kSelE, kStepThreads>(u, sh, n_valid, kmin, kmax);
  if (!plan_trivial(k, n_valid, T, shift, r_eq))
    radix_select<kSelE, kStepThreads>(u, kmin, kmax, k, sh, T, shift, r_eq);
  const int i0 = threadIdx.x * kSelE;
  return compact<kSelE, kStepThreads>(u, T, shift, r_eq, sh, [&](int o, int e) { emit(o, i0 + e); });
}

// One scoring item: keys [tile * kTileKeys, + kTileKeys) of sequence b; the
// 8 waves run as two 4-wave scoring groups of 64 keys per wave. Coarse:
// virtual key = block id, summaries k_blk; fine: virtual key v is position
// blocks[v / blk] * blk + v % blk, visible iff lo <= position <= hi.
template <bool FINE>
__device__ __forceinline__ void score_item(const HiStepArgs& a, int b, int tile, const int* wl, int* bl) {
  ScoreArgs s;
  s.B = 1;
  s.n_q = 1;
  s.H_I = 64;
  s.d_I = 128;
  s.q = a.q_idx + (int64_t)b * 64 * 128;
  s.q_bstride = 64 * 128;
  s.shift = SeqShift{nullptr, 1, 1};
  if constexpr (!FINE) {
    s.k = a.k_blk + (int64_t)b * a.nblocks * 128;
    s.n_k = a.nblocks;
    s.k_bstride = (int64_t)a.nblocks * 128;
    s.s_bstride = s.ld = a.nblocks;
    s.n_keys = a.b_hi + 1;
    s.mask_off = a.b_hi;
    s.pos_lo = a.b_lo;
    s.blocks = nullptr;
    s.blk = 1;
    s.nbr = 0;
    s.fill_masked = 0;
    s.scores = a.coarse_sc + (int64_t)b * a.nblocks;
  } else {
    s.k = a.k_idx + (int64_t)b * a.n_k * 128;
    s.n_k = a.n_k;
    s.k_bstride = (int64_t)a.n_k * 128;
    s.s_bstride = s.ld = a.n_virt;
    s.n_keys = a.n_virt;
    s.mask_off = a.hi;
    s.pos_lo = a.lo;
    s.blocks = a.blocks_ro + (int64_t)b * a.n_rec;
    s.blk = a.blk;
    s.nbr = a.n_rec;
    s.fill_masked = 1;
    s.scores = a.fine_sc + (int64_t)b * a.n_virt;
  }
  const int wv = wave_id();
  // each 4-wave group has its own block-table slices in LDS
  decode_score_body<64, 128, kDepthShort>(s, kTileKeys / 8, a.fold_ok, 0, 2 * tile + (wv >> 2), 0, wv & 3, wl,
                                          bl + (wv >> 2) * kWaves * kMaxBlkIds);
}

// The items of the step.
__device__ __forceinline__ void item_coarse(const HiStepArgs& a, int b, int tile, const int* wl, char* lds) {
  score_item<false>(a, b, tile, wl, (int*)lds);
  signal_done(seq_word(a, b, kCoarse));
}

__device__ __forceinline__ void item_recall(const HiStepArgs& a, int b, char* lds) {
  wait_count(a, seq_word(a, b, kCoarse), a.tiles_c);
  SelShared<kStepThreads>& sh = *(SelShared<kStepThreads>*)lds;
  int32_t* out = a.blocks + (int64_t)b * a.n_rec;
  const int b_lo = a.b_lo;
  const int cnt = select_top(a.coarse_sc + (int64_t)b * a.nblocks + b_lo, a.b_hi - b_lo + 1, a.n_rec, sh,
                             [&](int o, int i) { out[o] = b_lo + i; });
  for (int i = cnt + threadIdx.x; i < a.n_rec; i += kStepThreads) out[i] = -1;
  signal_done(seq_word(a, b, kRecall));
}

__device__ __forceinline__ void item_fine(const HiStepArgs& a, int b, int tile, const int* wl, char* lds) {
  wait_count(a, seq_word(a, b, kRecall), 1);
  score_item<true>(a, b, tile, wl, (int*)lds);
  signal_done(seq_word(a, b, kFine));
}

__device__ __forceinline__ void item_select(const HiStepArgs& a, int b, char* lds) {
  wait_count(a, seq_word(a, b, kFine), a.tiles_f);
  SelShared<kStepThreads>& sh = *(SelShared<kStepThreads>*)lds;
  const int32_t* bl = a.blocks + (int64_t)b * a.n_rec;
  const int n_sink = a.n_sink, blk = a.blk, K_tot = a.K_tot;
  int32_t* out = a.idx + (int64_t)b * K_tot;
  const int cnt = select_top(a.fine_sc + (int64_t)b * a.n_virt, a.n_virt, a.k_dyn, sh,
                             [&](int o, int v) { out[n_sink + o] = bl[v / blk] * blk + v % blk; });
  for (int i = threadIdx.x; i < n_sink; i += kStepThreads) out[i] = i;
  const int w0 = n_sink + cnt, W = a.n_window, t = a.t;
  for (int i = threadIdx.x; i < W; i += kStepThreads) out[w0 + i] = t - W + 1 + i;
  for (int i = w0 + W + threadIdx.x; i < K_tot; i += kStepThreads) out[i] = -1;
  if (threadIdx.x == 0) a.n_sel[b] = w0 + W;
  signal_done(seq_word(a, b, kSel));
}

__device__ __forceinline__ void item_attend(const HiStepArgs& a, int b, int split, char* lds) {
  wait_count(a, seq_word(a, b, kSel), 1);
  decode_partial_body<2, 4>(a.att, 0, split, b, lds);
  signal_done(seq_word(a, b, kAttn));
}

__device__ __forceinline__ void item_merge(const HiStepArgs& a, int b) {
  wait_count(a, seq_word(a, b, kAttn), a.att.n_split);
  const int R = a.att.n_q * a.att.H;
  for (int u = threadIdx.x; u < R * 16; u += kStepThreads)
    decode_merge_row<8>(a.att, (int64_t)b * R + u / 16, 8 * (u % 16));
}

__global__ __launch_bounds__(kStepThreads) void hi_step_kernel(HiStepArgs ka, WArgs w) {
  __shared__ __attribute__((aligned(16))) char lds_u[kUnion];
  __shared__ __attribute__((aligned(16))) int wl[128];
  __shared__ __attribute__((aligned(16))) HiStepArgs a;
  __shared__ int item_sh;
  for (int h = threadIdx.x; h < 128; h += kStepThreads) wl[h] = h < 64 ? w.w[h] : 0;
  if (threadIdx.x == 0) a = ka;
  for (;;) {
    __syncthreads();  // the previous item is done with item_sh and the LDS union
    if (threadIdx.x == 0) item_sh = __hip_atomic_fetch_add(a.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = item_sh;
    const int tc = a.tiles_c, tf = a.tiles_f, ns = a.att.n_split, B = a.B;
    const int n1 = B * tc, n2 = n1 + B, n3 = n2 + B * tf, n4 = n3 + B, n5 = n4 + B * ns, n6 = n5 + B;
    if (it >= n6) break;
    if (it < n1) item_coarse(a, it / tc, it % tc, wl, lds_u);
    else if (it < n2) item_recall(a, it - n1, lds_u);
    else if (it < n3) item_fine(a, (it - n2) / tf, (it - n2) % tf, wl, lds_u);
    else if (it < n4) item_select(a, it - n3, lds_u);
    else if (it < n5) item_attend(a, (it - n4) / ns, (it - n4) % ns, lds_u);
    else item_merge(a, it - n5);
  }
}

}  // namespace

}  // namespace lsa

using namespace lsa;

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool al16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }
}  // namespace

extern "C" int32_t lsa_hier_decode_step(const int8_t* q_idx, const int8_t* k_idx, const int8_t* k_blk,
                                        const int32_t* w, const lsa_bf16* q, const lsa_bf16* k_cache,
                                        const lsa_bf16* v_cache, int32_t B, int32_t n_k, int32_t H_I, int32_t d_I,
                                        int32_t blk, int32_t n_blk_recall, lsa_select_cfg cfg, int32_t H,
                                        int32_t D, int32_t n_split, float scale, int32_t* idx, int32_t* n_sel,
                                        lsa_bf16* o, float* lse, void* ws, size_t ws_bytes, size_t* ws_needed,
                                        void* stream) {
  if (B <= 0 || n_k <= 0 || blk <= 0 || n_blk_recall <= 0 || !(scale > 0.f) || !isfinite(scale))
    return LSA_INVALID_ARG;
  if (cfg.n_sink < 0 || cfg.n_window < 0 || cfg.k_dyn < 0) return LSA_INVALID_ARG;
  const int64_t K_tot64 = (int64_t)cfg.n_sink + cfg.n_window + cfg.k_dyn;
  if (K_tot64 < 1 || K_tot64 > (1 << 20)) return LSA_INVALID_ARG;
  const int K_tot = (int)K_tot64;
  if (H_I != 64 || d_I != 128 || H != 64 || D != 128 || n_split < 1 || n_split > 8) return LSA_UNSUPPORTED;
  if (blk % 32 != 0 || blk > 1024 || n_k > kMaxCacheKeys) return LSA_UNSUPPORTED;
  const int t = n_k - 1;
  const int lo = cfg.n_sink, hi = t - cfg.n_window;
  if (t + 1 <= K_tot || hi < lo) return LSA_UNSUPPORTED;  // short contexts: lsa_hier_select
  const int b_lo = lo / blk, b_hi = hi / blk;
  const int64_t n_virt = (int64_t)n_blk_recall * blk;
  const int cap = kStepThreads * kSelE;
  if (b_hi - b_lo + 1 > cap || n_virt > cap || n_blk_recall > cap) return LSA_UNSUPPORTED;
  const int nblocks = (n_k + blk - 1) / blk;
  const int tiles_c = (b_hi + 1 + kTileKeys - 1) / kTileKeys;
  const int tiles_f = (int)((n_virt + kTileKeys - 1) / kTileKeys);
  const size_t sz_sync = align_up((2 + (size_t)kSyncPerSeq * B) * sizeof(int32_t));
  const size_t sz_coarse = align_up((size_t)B * nblocks * sizeof(int32_t));
  const size_t sz_blocks = align_up((size_t)B * n_blk_recall * sizeof(int32_t));
  const size_t sz_fine = align_up((size_t)B * n_virt * sizeof(int32_t));
  const size_t rows = (size_t)B * n_split * H;
  const size_t sz_part = align_up(decode_ws_bytes(B, 1, H, n_split));
  const size_t need = sz_sync + sz_coarse + sz_blocks + sz_fine + sz_part;
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al16(q_idx) || !al16(k_idx) || !al16(k_blk) || !al16(q) || !al16(k_cache) || !al16(v_cache) ||
      !al4(idx) || !al4(n_sel) || !al16(o) || !al16(ws) || w == nullptr)
    return LSA_INVALID_ARG;
  if (lse != nullptr && !al4(lse)) return LSA_INVALID_ARG;
  if (ws_bytes < need) return LSA_WORKSPACE;
  int64_t wsum = 0;
  int fold_ok = 1;
  WArgs wa{};
  for (int h = 0; h < 64; ++h) {
    wa.w[h] = w[h];
    wsum += w[h] < 0 ? -(int64_t)w[h] : (int64_t)w[h];
    fold_ok &= w[h] >= 0;
  }
  if (wsum * d_I * 16384 >= ((int64_t)1 << 31)) return LSA_RANGE;

  char* p = (char*)ws;
  HiStepArgs a{};
  a.sync = (int32_t*)p;
  p += sz_sync;
  a.coarse_sc = (int32_t*)p;
  p += sz_coarse;
  a.blocks = (int32_t*)p;
  a.blocks_ro = a.blocks;
  p += sz_blocks;
  a.fine_sc = (int32_t*)p;
  p += sz_fine;
  char* part = p;
  a.q_idx = q_idx;
  a.k_blk = k_blk;
  a.k_idx = k_idx;
  a.fold_ok = fold_ok;
  a.B = B;
  a.n_k = n_k;
  a.blk = blk;
  a.n_rec = n_blk_recall;
  a.b_lo = b_lo;
  a.b_hi = b_hi;
  a.n_virt = (int)n_virt;
  a.t = t;
  a.lo = lo;
  a.hi = hi;
  a.n_sink = cfg.n_sink;
  a.n_window = cfg.n_window;
  a.k_dyn = cfg.k_dyn;
  a.K_tot = K_tot;
  a.idx = idx;
  a.n_sel = n_sel;
  a.nblocks = nblocks;
  a.tiles_c = tiles_c;
  a.tiles_f = tiles_f;
  // attention over the selected lists (one query row per sequence)
  DecodeArgs& d = a.att;
  d.q = q;
  d.k = k_cache;
  d.v = v_cache;
  d.idx = idx;
  d.n_sel = n_sel;
  d.n_idx = 1;
  d.B = B;
  d.n_q = 1;
  d.n_k = n_k;
  d.H = H;
  d.K_tot = K_tot;
  d.n_split = n_split;
  d.sl2 = scale * 1.4426950408889634f;
  d.o = o;
  d.lse = lse;
  d.ws_m = (float*)part;
  d.ws_l = d.ws_m + rows;
  d.ws_o = (_Float16*)(part + align_up(rows * 2 * sizeof(float)));
  d.tgt_pos = nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (launch_fill_zero(a.sync, sz_sync, st) != hipSuccess) return LSA_HIP;
  {
    KernelTimer kt("hi_step_kernel", st);
    hipLaunchKernelGGL(hi_step_kernel, dim3(256), dim3(kStepThreads), 0, st, a, wa);
  }
  return hipGetLastError() == hipSuccess ? LSA_OK : LSA_HIP;
}
