// Top-k selection over exact int32 indexer scores (gfx950).
//
// Keeps, for each query row, the k candidates with the largest score; equal
// scores go to the lower position. (LongCat-2.0 release article, section
// "LongCat 稀疏注意力": the indexer picks the top-k keys per query; the SI
// paragraph pairs them with a contiguous window, and the sinks of the
// "架构拆解 ① LSA" section of the 1.6T training write-up are always kept.)
//
// One workgroup of 1024 threads takes a chunk of up to 1024 * E candidates of
// one row and holds them in registers, E consecutive candidates per thread
// (blocked layout, so thread order is candidate order). Scores map to
// order-preserving uint32 keys (INT32_MIN, the "not a candidate" mark, maps to
// 0). A radix select finds the exact k-th largest key T: the first digit
// starts at the highest bit in which the chunk's smallest and largest keys
// differ, so a chunk whose scores span 2^18 values needs two or three 8-bit
// passes, each an LDS histogram of the keys that still match the prefix
// (integer counts: independent of arrival order). A stable compaction (two
// block-wide prefix sums in thread order) then keeps every key above T and
// the first r keys equal to T, i.e. the lowest positions among the ties, and
// writes them in ascending position order. The result is bit-exact.
//
// Rows longer than one chunk run in two stages: stage A keeps the chunk-local
// top min(k, valid) of every chunk (a superset of the row's top-k inside that
// chunk), stage B selects the row's top-k from the concatenated survivors,
// which are still in ascending position order.
#include <algorithm>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "select_dev.h"
#include "select_geom.h"

namespace lsa {

namespace {

constexpr int SEL_NT = 1024;  // threads of a stage-B workgroup (and the widest stage A)

template <int NT>
__device__ void write_trivial(const SelectArgs& a, int r, int t) {
  int32_t* out = a.idx + (int64_t)r * a.out_ld;
  for (int i = threadIdx.x; i < a.out_ld; i += NT) out[i] = i <= t ? i : -1;
  if (threadIdx.x == 0) a.n_sel[r] = t + 1;
}

// Sinks, window and padding around `count` kept positions already written.
template <int NT>
__device__ void finalize(const SelectArgs& a, int r, const RowGeom& gm, int count) {
  int32_t* out = a.idx + (int64_t)r * a.out_ld;
  if (a.mode == SEL_RAW) {
    for (int i = count + threadIdx.x; i < a.out_ld; i += NT) out[i] = -1;
    if (threadIdx.x == 0) a.n_sel[r] = count;
    return;
  }
  const int ns = a.n_sink, W = a.n_window;
  for (int i = threadIdx.x; i < ns; i += NT) out[i] = i;
  const int w0 = ns + count;
  for (int i = threadIdx.x; i < W; i += NT) out[w0 + i] = gm.t - W + 1 + i;
  for (int i = w0 + W + threadIdx.x; i < a.out_ld; i += NT) out[i] = -1;
  if (threadIdx.x == 0) a.n_sel[r] = w0 + W;
}

// Chunk statistics: number of nonzero keys, their min and max. Also clears
// the radix counts and the list (published by the same barrier).
template <int E, int NT, int MINW>
__global__ __launch_bounds__(NT, MINW) void select_stage_a(SelectArgs a) {
  __shared__ SelShared<NT> sh;
  constexpr int CH = NT * E;
  const int r = blockIdx.x, j = blockIdx.y;
  if (a.row_flags != nullptr && a.row_flags[r] == 0) return;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) {
    if (j == 0) write_trivial<NT>(a, r, gm.t);
    return;
  }
  const int n_chunks = max(1, (gm.nc + CH - 1) / CH);
  if (j >= n_chunks) return;
  const int v0 = gm.c_lo + j * CH;
  const int n = max(0, min(CH, gm.nc - j * CH));
  const int32_t* row = a.scores + (int64_t)r * a.ld;
  uint32_t u[E];
  load_keys<E>(row, v0, n, u);
  int n_valid;
  uint32_t kmin, kmax, T;
  chunk_stats<E, NT>(u, sh, n_valid, kmin, kmax);
  int shift, r_eq;
  if (!plan_trivial(gm.k, n_valid, T, shift, r_eq)) radix_select<E, NT>(u, kmin, kmax, gm.k, sh, T, shift, r_eq);
  const int i0 = threadIdx.x * E;
  if (n_chunks == 1) {
    int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
    const int cnt =
        compact<E, NT>(u, T, shift, r_eq, sh, [&](int o, int e) { out[o] = pos_of(a, r, v0 + i0 + e); });
    finalize<NT>(a, r, gm, cnt);
  } else {
    const int64_t base = ((int64_t)r * a.max_chunks + j) * a.k_cap;
    int32_t* ws_s = a.ws_score + base;
    int32_t* ws_p = a.ws_pos + base;
    const int cnt = compact<E, NT>(u, T, shift, r_eq, sh, [&](int o, int e) {
      ws_s[o] = row[v0 + i0 + e];  // the score itself (still in cache)
      ws_p[o] = pos_of(a, r, v0 + i0 + e);
    });
    for (int i = cnt + threadIdx.x; i < a.k_cap; i += NT) ws_s[i] = kMasked;
  }
}

// Chunk groups of the middle stage in the longest row.
__host__ __device__ inline int mid_groups(const SelectArgs& a) { return (a.max_chunks + a.group - 1) / a.group; }

// Middle stage (rows with more chunk survivors than one pass holds): group g
// of row r reduces the survivors of chunks [g * group, (g + 1) * group) to
// their top k, kept as (score, position) pairs in ws2 and padded with
// INT32_MIN. The survivors are in ascending position order and so are the
// kept pairs, so ties still go to the lower position.
template <int E>
__global__ __launch_bounds__(SEL_NT) void select_stage_m(SelectArgs a, int CH) {
  __shared__ SelShared<SEL_NT> sh;
  const int r = blockIdx.x, g = blockIdx.y;
  if (a.row_flags != nullptr && a.row_flags[r] == 0) return;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) return;
  const int n_chunks = (gm.nc + CH - 1) / CH;
  const int c0 = g * a.group, c1 = min(n_chunks, c0 + a.group);
  if (n_chunks <= 1 || c0 >= c1) return;
  const int n = (c1 - c0) * a.k_cap;
  const int64_t base = ((int64_t)r * a.max_chunks + c0) * a.k_cap;
  const int32_t* ws_s = a.ws_score + base;
  const int32_t* ws_p = a.ws_pos + base;
  uint32_t u[E];
  load_keys<E>(ws_s, 0, n, u);
  int n_valid;
  uint32_t kmin, kmax, T;
  chunk_stats<E, SEL_NT>(u, sh, n_valid, kmin, kmax);
  int shift, r_eq;
  if (!plan_trivial(gm.k, n_valid, T, shift, r_eq))
    radix_select<E, SEL_NT>(u, kmin, kmax, gm.k, sh, T, shift, r_eq);
  const int i0 = threadIdx.x * E;
  const int64_t ob = ((int64_t)r * mid_groups(a) + g) * a.k_cap;
  int32_t* os = a.ws2_score + ob;
  int32_t* op = a.ws2_pos + ob;
  const int cnt = compact<E, SEL_NT>(u, T, shift, r_eq, sh, [&](int o, int e) {
    os[o] = ws_s[i0 + e];
    op[o] = ws_p[i0 + e];
  });
  for (int i = cnt + threadIdx.x; i < a.k_cap; i += SEL_NT) os[i] = kMasked;
}

// Stage B: top-k of the concatenated chunk survivors (n_chunks * k_cap
// entries, padded with INT32_MIN) of one row, or, after the middle stage, of
// the row's group survivors.
template <int E>
__global__ __launch_bounds__(SEL_NT) void select_stage_b(SelectArgs a, int CH) {
  __shared__ SelShared<SEL_NT> sh;
  const int r = blockIdx.x;
  if (a.row_flags != nullptr && a.row_flags[r] == 0) return;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) return;
  const int n_chunks = (gm.nc + CH - 1) / CH;
  if (n_chunks <= 1) return;
  const bool mid = a.group > 0;
  const int n = mid ? (n_chunks + a.group - 1) / a.group * a.k_cap : n_chunks * a.k_cap;
  const int64_t base = (int64_t)r * (mid ? mid_groups(a) : a.max_chunks) * a.k_cap;
  const int32_t* ws_s = (mid ? a.ws2_score : a.ws_score) + base;
  const int32_t* ws_p = (mid ? a.ws2_pos : a.ws_pos) + base;
  uint32_t u[E];
  load_keys<E>(ws_s, 0, n, u);
  int n_valid;
  uint32_t kmin, kmax, T;
  chunk_stats<E, SEL_NT>(u, sh, n_valid, kmin, kmax);
  int shift, r_eq;
  if (!plan_trivial(gm.k, n_valid, T, shift, r_eq))
    radix_select<E, SEL_NT>(u, kmin, kmax, gm.k, sh, T, shift, r_eq);
  const int i0 = threadIdx.x * E;
  int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
  const int cnt = compact<E, SEL_NT>(u, T, shift, r_eq, sh, [&](int o, int e) { out[o] = ws_p[i0 + e]; });
  finalize<SEL_NT>(a, r, gm, cnt);
}

// Threshold of a row's sampled candidates: the j*-th largest sampled score,
// j* = ceil(lam + 6 sqrt(lam) + 10) with lam = k * n_s / nc the expected
// number of the row's top k among its n_s sampled candidates (of nc). Fewer
// than j* of the top k fall in the sample except with odds far below 1e-9
// for a sample that behaves like a random one, and then at least k
// candidates score at or above the threshold; about j* * nc / n_s do. When
// the sample holds j* or fewer scores, every candidate is kept.
template <int E, int NT>
__global__ __launch_bounds__(NT) void filter_threshold_kernel(FilterArgs f) {
  __shared__ SelShared<NT> sh;
  const SelectArgs& a = f.sel;
  const int r = blockIdx.x;
  const RowGeom gm = row_geom(a, r);
  const int m = f.samp_m;
  int32_t tau = INT32_MIN;
  const int j_lo = (gm.c_lo + m - 1) / m;
  const int j_hi = gm.trivial ? -1 : (gm.c_lo + gm.nc - 1) / m;
  const int n_s = max(0, j_hi - j_lo + 1);
  if (n_s > 0) {
    uint32_t u[E];
    load_keys<E>(f.samp + (int64_t)r * f.samp_ld, j_lo, n_s, u);
    int n_valid;
    uint32_t kmin, kmax;
    chunk_stats<E, NT>(u, sh, n_valid, kmin, kmax);
    const float lam = (float)gm.k * (float)n_s / (float)gm.nc;
    const int jstar = (int)ceilf(lam + 6.0f * sqrtf(lam) + 10.0f);
    if (jstar < n_valid) {
      uint32_t T;
      int shift, r_eq;
      radix_select<E, NT>(u, kmin, kmax, jstar, sh, T, shift, r_eq);
      // T has zeros below `shift`: every sampled key >= T is among the kept
      tau = (int32_t)(T ^ 0x80000000u);
    }
  }
  if (threadIdx.x == 0) f.tau[r] = tau;
}

// Top-k of a row's survivors: segments (row, chunk) of (score, position)
// pairs in ascending position order, concatenated in chunk order. Thread t
// takes the ee = ceil(total / NT) consecutive entries from t * ee (blocked:
// thread order is position order, every thread holding some); their
// addresses come first, then all loads issue back to back. The row fails
// (fail = 1, outputs left to the redo) when a segment overflowed, the
// survivors do not fit or are fewer than k.
template <int E, int NT>
__global__ __launch_bounds__(NT) void filter_select_kernel(FilterArgs f) {
  __shared__ SelShared<NT> sh;
  __shared__ int pref[NT + 1];
  const SelectArgs& a = f.sel;
  const int r = blockIdx.x, tid = threadIdx.x;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) {
    write_trivial<NT>(a, r, gm.t);
    if (tid == 0) f.fail[r] = 0;
    return;
  }
  const int nsg = f.seg_chunks;
  const int cnt = tid < nsg ? f.seg_cnt[(int64_t)r * nsg + tid] : 0;
  uint32_t total;
  const uint32_t off = block_excl_scan<NT>((uint32_t)min(cnt, f.seg_cap + 1), sh, &total);
  if (tid < nsg) pref[tid] = (int)off;
  if (tid == 0) pref[nsg] = (int)total;
  const int over = __syncthreads_or(cnt > f.seg_cap);
  if (over || (int)total < gm.k || total > (uint32_t)(NT * E)) {
    if (tid == 0) f.fail[r] = 1;
    return;
  }
  const int n = (int)total;
  const int ee = (n + NT - 1) / NT;  // entries per thread (<= E)
  const int i0 = tid * ee;
  // segment of entry i0, then the entry offsets of [i0, i0 + ee) (clamped to
  // the last entry: loads past it read a valid pair and are masked below)
  int sg = 0;
  for (int lo = 0, hi = nsg - 1; lo <= hi;) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid] <= min(i0, n - 1)) {
      sg = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  int eoff[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = min(i0 + min(e, ee - 1), n - 1);
    while (pref[sg + 1] <= i) ++sg;
    eoff[e] = (sg * f.seg_cap + (i - pref[sg])) * 2;
  }
  const int32_t* seg_r = f.seg + (int64_t)r * nsg * f.seg_cap * 2;
  v2u x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = *(const v2u*)(seg_r + eoff[e]);
  uint32_t u[E];
#pragma unroll
  for (int e = 0; e < E; ++e) u[e] = e < ee && i0 + e < n ? score_key((int32_t)x[e][0]) : 0u;
  int n_valid;
  uint32_t kmin, kmax, T;
  chunk_stats<E, NT>(u, sh, n_valid, kmin, kmax);
  int shift, r_eq;
  if (!plan_trivial(gm.k, n_valid, T, shift, r_eq)) radix_select<E, NT>(u, kmin, kmax, gm.k, sh, T, shift, r_eq);
  int32_t* out = a.idx + (int64_t)r * a.out_ld + a.n_sink;
  const int kept = compact<E, NT, true>(u, T, shift, r_eq, sh, [&](int o, int e) { out[o] = (int)x[e][1]; });
  finalize<NT>(a, r, gm, kept);
  if (tid == 0) f.fail[r] = 0;
}

// Chunk geometry: E candidates per thread of a workgroup of NT threads.
struct SelGeo {
  int e, chunks, nt;
};

SelGeo sel_geo(int64_t max_nc) {
  const int e = max_nc <= (int64_t)SEL_NT * 4 ? 4 : max_nc <= (int64_t)SEL_NT * 16 ? 16 : 32;
  const int64_t ch = (int64_t)SEL_NT * e;
  return SelGeo{e, (int)(max_nc <= ch ? 1 : (max_nc + ch - 1) / ch), SEL_NT};
}

// Rows longer than one 1024-thread chunk, in launches with enough chunks to
// hold four 512-thread workgroups per CU twice over, take half-size chunks:
// four workgroups per CU overlap one another's loads and barriers better
// (C5 rows: stage A -10%, stage B +15% of a smaller time). With few rows
// (decode batches) the longer stage B costs more than stage A saves. The
// same workgroup size serves large launches of rows that fit one chunk of
// 16384 keys.
constexpr int kHalfChunkLaunch = 2 * 256 * 4;

SelGeo sel_geo_half(int64_t max_nc) {
  constexpr int64_t ch = 512 * 32;
  return SelGeo{32, (int)((max_nc + ch - 1) / ch), 512};
}

bool half_fits(int64_t max_nc, int k_cap) {
  return max_nc > (int64_t)SEL_NT * 32 && (int64_t)sel_geo_half(max_nc).chunks * k_cap <= kSelMaxSurvivors;
}

// Stage A runs two workgroups per CU (registers capped at 64 per lane) when
// there are enough chunks to fill the GPU twice over, so that one
// workgroup's load latency and barriers overlap the other's work; with fewer
// chunks it keeps the full register budget, one workgroup per CU.
constexpr int kTwoPerCuChunks = 2 * 256 * 2;

template <int E, int NT>
hipError_t launch_e(const SelectArgs& a, hipStream_t st) {
  constexpr int CH = NT * E;
  dim3 ga(a.n_rows, max(a.max_chunks, 1));
  {
    KernelTimer kt("select_stage_a", st);
    if ((int64_t)a.n_rows * max(a.max_chunks, 1) >= kTwoPerCuChunks * (SEL_NT / NT))
      hipLaunchKernelGGL((select_stage_a<E, NT, 8>), ga, dim3(NT), 0, st, a);
    else
      hipLaunchKernelGGL((select_stage_a<E, NT, 1>), ga, dim3(NT), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  if (a.group > 0) {
    const int64_t nm = (int64_t)a.group * a.k_cap;  // input of one group
    const dim3 gm(a.n_rows, mid_groups(a));
    KernelTimer kt("select_stage_m", st);
    if (nm <= SEL_NT * 4) hipLaunchKernelGGL((select_stage_m<4>), gm, dim3(SEL_NT), 0, st, a, CH);
    else if (nm <= SEL_NT * 8) hipLaunchKernelGGL((select_stage_m<8>), gm, dim3(SEL_NT), 0, st, a, CH);
    else if (nm <= SEL_NT * 16) hipLaunchKernelGGL((select_stage_m<16>), gm, dim3(SEL_NT), 0, st, a, CH);
    else hipLaunchKernelGGL((select_stage_m<32>), gm, dim3(SEL_NT), 0, st, a, CH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // survivors of one row: max_chunks * k_cap, or its groups' k_cap each
  const int64_t nb = (int64_t)(a.group > 0 ? mid_groups(a) : a.max_chunks) * a.k_cap;
  KernelTimer kt("select_stage_b", st);
  if (nb <= SEL_NT * 4) hipLaunchKernelGGL((select_stage_b<4>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  else if (nb <= SEL_NT * 8) hipLaunchKernelGGL((select_stage_b<8>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  else if (nb <= SEL_NT * 16) hipLaunchKernelGGL((select_stage_b<16>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  else hipLaunchKernelGGL((select_stage_b<32>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  return hipGetLastError();
}

}  // namespace

int select_chunks(int64_t max_nc, int k_cap) {
  return half_fits(max_nc, k_cap) ? sel_geo_half(max_nc).chunks : sel_geo(max_nc).chunks;
}

// Chunks per middle-stage group for c chunks of k_cap survivors (0: none).
static int mid_group(int c, int k_cap) {
  if (c <= 1 || (int64_t)c * k_cap <= kSelMaxSurvivors) return 0;
  return (int)(kSelMaxSurvivors / k_cap);
}

bool select_fits(int64_t max_nc, int k_cap) {
  const int c = sel_geo(max_nc).chunks;
  if (c <= 1 || (int64_t)c * k_cap <= kSelMaxSurvivors) return true;
  const int G = mid_group(c, k_cap);
  return G >= 1 && (int64_t)((c + G - 1) / G) * k_cap <= kSelMaxSurvivors;
}

void select_plan(SelectArgs& a, int64_t max_nc) {
  SelGeo g = sel_geo(max_nc);
  if (half_fits(max_nc, a.k_cap) && (int64_t)a.n_rows * sel_geo_half(max_nc).chunks >= kHalfChunkLaunch)
    g = sel_geo_half(max_nc);
  // rows of at most 16384 candidates in a large launch: one 512-thread chunk
  // of 32 keys per thread instead of a 1024-thread one of 16 (C2's first pass:
  // stage A 0.40 -> 0.30 ms)
  if (g.e == 16 && a.n_rows >= kHalfChunkLaunch) g = SelGeo{32, 1, 512};
  a.chunk_e = g.e;
  a.chunk_nt = g.nt;
  a.max_chunks = g.chunks;
  a.group = mid_group(g.chunks, a.k_cap);
}

size_t select_ws_bytes(int n_rows, int max_chunks, int k_cap) {
  if (max_chunks <= 1) return 0;
  size_t b = (size_t)2 * n_rows * max_chunks * k_cap * sizeof(int32_t);
  const int G = mid_group(max_chunks, k_cap);
  if (G > 0) b += (size_t)2 * n_rows * ((max_chunks + G - 1) / G) * k_cap * sizeof(int32_t);
  return b;
}

void select_bind_ws(SelectArgs& a, void* ws, int n_rows) {
  if (a.max_chunks <= 1 || ws == nullptr) {
    a.ws_score = a.ws_pos = a.ws2_score = a.ws2_pos = nullptr;
    return;
  }
  a.ws_score = (int32_t*)ws;
  a.ws_pos = a.ws_score + (size_t)n_rows * a.max_chunks * a.k_cap;
  if (a.group > 0) {
    a.ws2_score = a.ws_pos + (size_t)n_rows * a.max_chunks * a.k_cap;
    a.ws2_pos = a.ws2_score + (size_t)n_rows * mid_groups(a) * a.k_cap;
  } else {
    a.ws2_score = a.ws2_pos = nullptr;
  }
}

hipError_t launch_filter_threshold(const FilterArgs& f, int max_ns, hipStream_t st) {
  if (f.sel.n_rows <= 0) return hipSuccess;
  const dim3 grid(f.sel.n_rows);
  KernelTimer kt("filter_threshold_kernel", st);
  if (max_ns <= 256 * 16) hipLaunchKernelGGL((filter_threshold_kernel<16, 256>), grid, dim3(256), 0, st, f);
  else if (max_ns <= 256 * 32) hipLaunchKernelGGL((filter_threshold_kernel<32, 256>), grid, dim3(256), 0, st, f);
  else if (max_ns <= SEL_NT * 32) hipLaunchKernelGGL((filter_threshold_kernel<32, SEL_NT>), grid, dim3(SEL_NT), 0, st, f);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Survivor capacity of the survivor selection: 256 threads (several rows per
// CU at once) up to 8192 survivors, then wider workgroups.
int filter_select_capacity() { return 32 * SEL_NT; }

hipError_t launch_filter_select(const FilterArgs& f, int max_surv, hipStream_t st) {
  if (f.sel.n_rows <= 0) return hipSuccess;
  if (f.seg_chunks < 1 || f.seg_chunks > 256) return hipErrorInvalidValue;
  const dim3 grid(f.sel.n_rows);
  KernelTimer kt("filter_select_kernel", st);
  if (max_surv <= 256 * 8) hipLaunchKernelGGL((filter_select_kernel<8, 256>), grid, dim3(256), 0, st, f);
  else if (max_surv <= 256 * 16) hipLaunchKernelGGL((filter_select_kernel<16, 256>), grid, dim3(256), 0, st, f);
  else if (max_surv <= 256 * 32) hipLaunchKernelGGL((filter_select_kernel<32, 256>), grid, dim3(256), 0, st, f);
  else if (max_surv <= 512 * 32) hipLaunchKernelGGL((filter_select_kernel<32, 512>), grid, dim3(512), 0, st, f);
  else if (max_surv <= SEL_NT * 32) hipLaunchKernelGGL((filter_select_kernel<32, SEL_NT>), grid, dim3(SEL_NT), 0, st, f);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// The geometry must come from select_plan (k_cap set first); one reduction
// pass over survivors holds at most kSelMaxSurvivors entries.
hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.max_chunks > 1 && (int64_t)a.max_chunks * a.k_cap > kSelMaxSurvivors &&
      (a.group <= 0 || (int64_t)mid_groups(a) * a.k_cap > kSelMaxSurvivors))
    return hipErrorInvalidValue;
  if (a.chunk_e == 4) return launch_e<4, SEL_NT>(a, st);
  if (a.chunk_e == 16) return launch_e<16, SEL_NT>(a, st);
  if (a.chunk_nt == 512) return launch_e<32, 512>(a, st);
  return launch_e<32, SEL_NT>(a, st);
}

}  // namespace lsa
