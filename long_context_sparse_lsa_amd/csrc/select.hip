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

namespace lsa {

namespace {

constexpr int SEL_NT = 1024;  // threads of a stage-B workgroup (and the widest stage A)

constexpr int kBins1 = 256;   // first radix digit: 8 bits
constexpr int kList = 4096;   // keys of the first pass's threshold bin kept in LDS

template <int NT>
struct SelShared {
  static constexpr int NW = NT / 64;
  alignas(16) uint32_t hist1[kBins1];  // first pass
  alignas(16) uint32_t hist[3][256];   // later pass p counts into hist[p % 3]
  uint32_t list[kList];
  int list_n;
  uint32_t scan_w[NW];   // per-wave totals of the compaction scan
  uint32_t st_w[3][NW];  // per-wave count, min, max of the chunk
};

struct RowGeom {
  int trivial;
  int t;
  int c_lo, nc;
  int k;
};

__device__ __forceinline__ RowGeom row_geom(const SelectArgs& a, int r) {
  RowGeom gm{0, 0, 0, 0, 0};
  if (a.mode == SEL_FLAT) {
    const int t = a.q_off + (a.row0 + r) % a.n_q + seq_shift(a.shift, (a.row0 + r) / a.n_q);
    gm.t = t;
    if (t + 1 <= a.n_sink + a.n_window + a.k_dyn) {
      gm.trivial = 1;
      return gm;
    }
    gm.c_lo = a.n_sink;
    gm.nc = t - a.n_window - a.n_sink + 1;
    gm.k = a.k_dyn;
  } else if (a.mode == SEL_RAW) {
    int hi = a.raw_hi;
    if (a.shift.ctx_len != nullptr) {
      const int hp = a.raw_hi_pos + seq_shift(a.shift, a.row0 + r);
      hi = min(hp >= 0 ? hp / a.raw_div : -1, a.raw_hi);
    }
    gm.c_lo = a.raw_lo;
    gm.nc = max(0, hi - a.raw_lo + 1);
    gm.k = a.raw_k;
  } else {
    gm.t = a.t_fixed;
    gm.c_lo = 0;
    gm.nc = a.n_virt;
    gm.k = a.k_dyn;
    if (a.shift.ctx_len != nullptr) {
      gm.t += seq_shift(a.shift, a.row0 + r);
      gm.trivial = gm.t + 1 <= a.n_sink + a.n_window + a.k_dyn;
    }
  }
  return gm;
}

__device__ __forceinline__ int pos_of(const SelectArgs& a, int r, int v) {
  if (a.mode != SEL_INDIRECT) return v;
  const int bi = a.blocks[(int64_t)r * a.nbr + v / a.blk];
  return bi * a.blk + v % a.blk;
}

// Exclusive prefix sum over the block in thread order (mod 2^32); *total
// gets the sum. One barrier: sh.scan_w is written once per workgroup.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SelShared<NT>& sh, uint32_t* total) {
  const uint32_t incl = (uint32_t)wave_incl_scan((int)v);
  if (lane_id() == 63) sh.scan_w[wave_id()] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SelShared<NT>::NW; ++w) {
    const uint32_t x = sh.scan_w[w];
    off += (w < wave_id()) ? x : 0u;
    tot += x;
  }
  *total = tot;
  return off + incl - v;
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d, 64));
  return v;
}

// The bin of the k_rem-th largest key from per-bin counts, found by every
// wave on its own (no broadcast barrier): lane l owns B / 64 consecutive
// bins, a suffix sum over lanes gives the keys above each lane's bins, and
// the one lane whose bins hold the k_rem-th largest scans them. Returns the
// bin, the keys in bins above it and the keys in it, wave-uniform.
template <int B>
__device__ __forceinline__ void find_bin(const uint32_t* hist, int k_rem, uint32_t& d, int& above, int& eq) {
  constexpr int PL = B / 64;  // bins per lane
  const int l = lane_id();
  const v4i* hp = (const v4i*)(hist + PL * l);
  int sl = 0;
#pragma unroll
  for (int i = 0; i < PL / 4; ++i) {
    const v4i h4 = hp[i];
    sl += h4[0] + h4[1] + h4[2] + h4[3];
  }
  int v = sl;  // inclusive suffix sum over lanes
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) {
    const int t = __shfl_down(v, dd, 64);
    if (l + dd < 64) v += t;
  }
  int cum = v - sl;  // keys in bins above this lane's bins
  int my_bin = 0, my_above = 0, my_eq = 0;
  const bool mine = cum < k_rem && k_rem <= cum + sl;
  if (mine) {
    for (int i = PL - 1; i >= 0; --i) {
      const int h = (int)hist[PL * l + i];
      if (cum < k_rem && k_rem <= cum + h) {
        my_bin = PL * l + i;
        my_above = cum;
        my_eq = h;
        break;
      }
      cum += h;
    }
  }
  const uint64_t who = __ballot(mine);
  const int src = __ffsll((unsigned long long)who) - 1;
  d = (uint32_t)__shfl(my_bin, src, 64);
  above = __shfl(my_above, src, 64);
  eq = __shfl(my_eq, src, 64);
}

// Threshold of the k-th largest nonzero key of the chunk (0 < k < #nonzero).
// On return an entry u is kept iff (u >> shift) > (T >> shift), or
// (u >> shift) == (T >> shift) and it is among the first r_eq such entries.
// The first pass counts every key by an 8-bit digit starting at the highest
// bit in which the chunk's keys differ (an 11-bit digit leaves fewer keys in
// the threshold bin but costs more to search: measured slower at every chunk
// size here). The keys of the bin that holds the threshold are then copied
// to an LDS list
// when they fit, and further 8-bit passes count only those. Later pass p
// counts into hist[p % 3] (hist[0] and hist[1] start cleared); after its
// barrier every wave finds the digit itself and clears hist[(p + 2) % 3],
// which no wave reads any more and none writes before the next barrier.
template <int E, int NT>
__device__ void radix_select(const uint32_t (&u)[E], uint32_t kmin, uint32_t kmax, int k,
                             SelShared<NT>& sh, uint32_t& T, int& shift_out, int& r_eq) {
  if (kmin == kmax) {  // every candidate has the same key: take the first k
    T = kmax;
    shift_out = 0;
    r_eq = k;
    return;
  }
  const int tid = threadIdx.x;
  int hb = 31 - __clz(kmin ^ kmax);  // highest differing bit
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmax & mask;
  int k_rem = k;
  // pass 1 over all keys (all nonzero keys share the bits above hb); small
  // chunks take an 8-bit digit, whose counts are cheaper to search
  constexpr int B1 = kBins1;
  int lo = max(0, hb - 7);
  uint32_t dmask = (2u << (hb - lo)) - 1u;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (u[e] != 0u) atomicAdd(&sh.hist1[(u[e] >> lo) & dmask], 1u);
  __syncthreads();
  uint32_t d;
  int above, eq;
  find_bin<B1>(sh.hist1, k_rem, d, above, eq);
  k_rem -= above;
  prefix |= d << lo;
  mask |= dmask << lo;
  if (eq == k_rem || lo == 0) {
    T = prefix;
    shift_out = lo;
    r_eq = k_rem;
    return;
  }
  const bool listed = eq <= kList;
  if (listed) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (u[e] != 0u && (u[e] & mask) == prefix) sh.list[atomicAdd(&sh.list_n, 1)] = u[e];
    __syncthreads();
  }
  hb = lo - 1;
  for (int p = 0;; ++p) {
    uint32_t* hist = sh.hist[p % 3];
    lo = max(0, hb - 7);
    dmask = (2u << (hb - lo)) - 1u;
    if (listed) {
      for (int i = tid; i < eq; i += NT) {
        const uint32_t x = sh.list[i];
        if ((x & mask) == prefix) atomicAdd(&hist[(x >> lo) & dmask], 1u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (u[e] != 0u && (u[e] & mask) == prefix) atomicAdd(&hist[(u[e] >> lo) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 256) sh.hist[(p + 2) % 3][tid] = 0u;
    int above2, eq2;
    find_bin<256>(hist, k_rem, d, above2, eq2);
    k_rem -= above2;
    prefix |= d << lo;
    mask |= dmask << lo;
    if (eq2 == k_rem || lo == 0) {
      T = prefix;
      shift_out = lo;
      r_eq = k_rem;
      return;
    }
    hb = lo - 1;
  }
}

// Stable compaction over the chunk; emit(out_pos, e) for each kept entry e
// of this thread, in candidate order. Returns the number kept. Each thread
// builds bit masks of its entries above and equal to the threshold; one
// scan of the packed counts (above << 16 | equal; each at most 32768) gives
// both prefixes, and an entry equal to the threshold is kept while fewer
// than r_eq equal entries precede it. Only the kept entries are visited.
template <int E, int NT, class Emit>
__device__ int compact(const uint32_t (&u)[E], uint32_t T, int shift, int r_eq, SelShared<NT>& sh, Emit emit) {
  static_assert(E <= 32, "one mask bit per entry");
  const uint32_t Ts = T >> shift;
  uint32_t gt = 0u, em = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t us = u[e] >> shift;
    const bool valid = u[e] != 0u;
    gt |= (uint32_t)(valid && us > Ts) << e;
    em |= (uint32_t)(valid && us == Ts) << e;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<NT>(((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(em), sh, &tot);
  const int eq_before = (int)(ex & 0xffffu);
  int o = (int)(ex >> 16) + min(eq_before, r_eq);
  uint32_t keep = gt;
  for (int take = r_eq - eq_before; take > 0 && em != 0u; --take) {
    keep |= em & (0u - em);  // lowest remaining equal entry
    em &= em - 1u;
  }
  while (keep != 0u) {
    const int e = __ffs(keep) - 1;
    keep &= keep - 1u;
    emit(o++, e);
  }
  return (int)(tot >> 16) + min((int)(tot & 0xffffu), r_eq);
}

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
template <int E, int NT>
__device__ void chunk_stats(const uint32_t (&u)[E], SelShared<NT>& sh, int& n_valid, uint32_t& kmin,
                            uint32_t& kmax) {
  int cnt = 0;
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cnt += u[e] != 0u;
    if (u[e] != 0u) {
      mn = min(mn, u[e]);
      mx = max(mx, u[e]);
    }
  }
  cnt = wave_sum(cnt);
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  if (lane_id() == 0) {
    sh.st_w[0][wave_id()] = (uint32_t)cnt;
    sh.st_w[1][wave_id()] = mn;
    sh.st_w[2][wave_id()] = mx;
  }
  for (int i = threadIdx.x; i < kBins1; i += NT) sh.hist1[i] = 0u;
  if (threadIdx.x < 256) {
    sh.hist[0][threadIdx.x] = 0u;
    sh.hist[1][threadIdx.x] = 0u;
  }
  if (threadIdx.x == 0) sh.list_n = 0;
  __syncthreads();
  int tot = 0;
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < SelShared<NT>::NW; ++w) {
    tot += (int)sh.st_w[0][w];
    mn = min(mn, sh.st_w[1][w]);
    mx = max(mx, sh.st_w[2][w]);
  }
  n_valid = tot;
  kmin = mn;
  kmax = mx;
}

// Keys of candidates [v0, v0 + n) of a score row, E per thread (blocked).
template <int E>
__device__ void load_keys(const int32_t* row, int v0, int n, uint32_t (&u)[E]) {
  const int i0 = threadIdx.x * E;
  const int32_t* src = row + v0 + i0;
  const bool vec = (((uintptr_t)src & 15u) == 0) && i0 + E <= n;
  if (vec) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const v4i x = *(const v4i*)(src + e);
#pragma unroll
      for (int j = 0; j < 4; ++j) u[e + j] = score_key(x[j]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) u[e] = i0 + e < n ? score_key(src[e]) : 0u;
  }
}

// Keep count for "k of n_valid" that needs no radix pass, or -1.
__device__ __forceinline__ bool plan_trivial(int k, int n_valid, uint32_t& T, int& shift, int& r_eq) {
  if (k <= 0) {
    T = 0xffffffffu;  // nothing above, no ties taken
    shift = 0;
    r_eq = 0;
    return true;
  }
  if (k >= n_valid) {
    T = 0u;  // every nonzero key is above 0
    shift = 0;
    r_eq = 0;
    return true;
  }
  return false;
}

template <int E, int NT, int MINW>
__global__ __launch_bounds__(NT, MINW) void select_stage_a(SelectArgs a) {
  __shared__ SelShared<NT> sh;
  constexpr int CH = NT * E;
  const int r = blockIdx.x, j = blockIdx.y;
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

// Stage B: top-k of the concatenated chunk survivors (n_chunks * k_cap
// entries, padded with INT32_MIN) of one row.
template <int E>
__global__ __launch_bounds__(SEL_NT) void select_stage_b(SelectArgs a, int CH) {
  __shared__ SelShared<SEL_NT> sh;
  const int r = blockIdx.x;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) return;
  const int n_chunks = (gm.nc + CH - 1) / CH;
  if (n_chunks <= 1) return;
  const int n = n_chunks * a.k_cap;
  const int64_t base = (int64_t)r * a.max_chunks * a.k_cap;
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
  int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
  const int cnt = compact<E, SEL_NT>(u, T, shift, r_eq, sh, [&](int o, int e) { out[o] = ws_p[i0 + e]; });
  finalize<SEL_NT>(a, r, gm, cnt);
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
  // survivors of one row: max_chunks * k_cap
  const int64_t nb = (int64_t)a.max_chunks * a.k_cap;
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

bool select_fits(int64_t max_nc, int k_cap) {
  const int c = sel_geo(max_nc).chunks;
  return c <= 1 || (int64_t)c * k_cap <= kSelMaxSurvivors;
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
}

size_t select_ws_bytes(int n_rows, int max_chunks, int k_cap) {
  if (max_chunks <= 1) return 0;
  return (size_t)2 * n_rows * max_chunks * k_cap * sizeof(int32_t);
}

void select_bind_ws(SelectArgs& a, void* ws, int n_rows) {
  if (a.max_chunks <= 1 || ws == nullptr) {
    a.ws_score = a.ws_pos = nullptr;
    return;
  }
  a.ws_score = (int32_t*)ws;
  a.ws_pos = a.ws_score + (size_t)n_rows * a.max_chunks * a.k_cap;
}

// The geometry must come from select_plan (k_cap set first), and the stage-B
// survivor count max_chunks * k_cap must fit 32 * 1024 entries.
hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.max_chunks > 1 && (int64_t)a.max_chunks * a.k_cap > kSelMaxSurvivors) return hipErrorInvalidValue;
  if (a.chunk_e == 4) return launch_e<4, SEL_NT>(a, st);
  if (a.chunk_e == 16) return launch_e<16, SEL_NT>(a, st);
  if (a.chunk_nt == 512) return launch_e<32, 512>(a, st);
  return launch_e<32, SEL_NT>(a, st);
}

}  // namespace lsa
