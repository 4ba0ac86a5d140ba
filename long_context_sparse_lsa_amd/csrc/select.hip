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
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int SEL_NT = 1024;
constexpr int SEL_NW = SEL_NT / 64;

struct SelShared {
  uint32_t hist[256];
  int scan_w[SEL_NW];
  uint32_t red_w[2][SEL_NW];
  int bcast[4];
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
    const int t = a.q_off + (a.row0 + r) % a.n_q;
    gm.t = t;
    if (t + 1 <= a.n_sink + a.n_window + a.k_dyn) {
      gm.trivial = 1;
      return gm;
    }
    gm.c_lo = a.n_sink;
    gm.nc = t - a.n_window - a.n_sink + 1;
    gm.k = a.k_dyn;
  } else if (a.mode == SEL_RAW) {
    gm.c_lo = a.raw_lo;
    gm.nc = max(0, a.raw_hi - a.raw_lo + 1);
    gm.k = a.raw_k;
  } else {
    gm.t = a.t_fixed;
    gm.c_lo = 0;
    gm.nc = a.n_virt;
    gm.k = a.k_dyn;
  }
  return gm;
}

__device__ __forceinline__ int pos_of(const SelectArgs& a, int r, int v) {
  if (a.mode != SEL_INDIRECT) return v;
  const int bi = a.blocks[(int64_t)r * a.nbr + v / a.blk];
  return bi * a.blk + v % a.blk;
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, SelShared& sh, int* total) {
  const int incl = wave_incl_scan(v);
  if (lane_id() == 63) sh.scan_w[wave_id()] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_NW; ++w) {
    const int x = sh.scan_w[w];
    off += (w < wave_id()) ? x : 0;
    tot += x;
  }
  __syncthreads();
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

// Threshold of the k-th largest nonzero key of the chunk (0 < k < #nonzero).
// On return an entry u is kept iff (u >> shift) > (T >> shift), or
// (u >> shift) == (T >> shift) and it is among the first r_eq such entries.
template <int E>
__device__ void radix_select(const uint32_t (&u)[E], uint32_t kmin, uint32_t kmax, int k,
                             SelShared& sh, uint32_t& T, int& shift_out, int& r_eq) {
  if (kmin == kmax) {  // every candidate has the same key: take the first k
    T = kmax;
    shift_out = 0;
    r_eq = k;
    return;
  }
  int hb = 31 - __clz(kmin ^ kmax);  // highest differing bit
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmax & mask;
  int k_rem = k;
  const int tid = threadIdx.x;
  while (true) {
    const int lo = max(0, hb - 7);
    const uint32_t dmask = (2u << (hb - lo)) - 1u;  // digit of hb - lo + 1 bits
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (u[e] != 0u && (u[e] & mask) == prefix) atomicAdd(&sh.hist[(u[e] >> lo) & dmask], 1u);
    __syncthreads();
    if (wave_id() == 0) {
      // lane l owns bins 4l .. 4l+3; find the bin holding the k_rem-th largest
      const int l = lane_id();
      int h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (int)sh.hist[4 * l + e];
      const int s = h[0] + h[1] + h[2] + h[3];
      int v = s;  // inclusive suffix sum over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_down(v, d, 64);
        if (l + d < 64) v += t;
      }
      int cum = v - s;  // keys in bins above this lane's bins
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (cum < k_rem && k_rem <= cum + h[e]) {
          sh.bcast[0] = 4 * l + e;
          sh.bcast[1] = cum;
          sh.bcast[2] = h[e];
        }
        cum += h[e];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sh.bcast[0];
    const int above = sh.bcast[1], eq = sh.bcast[2];
    __syncthreads();  // bcast / hist are rewritten by the next pass
    k_rem -= above;
    prefix |= d << lo;
    mask |= dmask << lo;
    if (eq == k_rem || lo == 0) {
      T = prefix;
      shift_out = lo;
      r_eq = k_rem;
      return;
    }
    hb = lo - 1;
  }
}

// Stable compaction over the chunk; emit(out_pos, e) for each kept entry e
// of this thread, in candidate order. Returns the number kept.
template <int E, class Emit>
__device__ int compact(const uint32_t (&u)[E], uint32_t T, int shift, int r_eq, SelShared& sh, Emit emit) {
  const uint32_t Ts = T >> shift;
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) n_eq += (u[e] != 0u && (u[e] >> shift) == Ts);
  int eq_tot;
  int eq_rank = block_excl_scan(n_eq, sh, &eq_tot);
  uint32_t keep = 0;  // bit e: entry e kept (E <= 32)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool valid = u[e] != 0u;
    const uint32_t us = u[e] >> shift;
    const bool eq = valid && us == Ts;
    const bool sel = (valid && us > Ts) || (eq && eq_rank < r_eq);
    eq_rank += eq;
    keep |= (uint32_t)sel << e;
  }
  int tot;
  int o = block_excl_scan(__popc(keep), sh, &tot);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((keep >> e) & 1u) emit(o++, e);
  return tot;
}

__device__ void write_trivial(const SelectArgs& a, int r, int t) {
  int32_t* out = a.idx + (int64_t)r * a.out_ld;
  for (int i = threadIdx.x; i < a.out_ld; i += SEL_NT) out[i] = i <= t ? i : -1;
  if (threadIdx.x == 0) a.n_sel[r] = t + 1;
}

// Sinks, window and padding around `count` kept positions already written.
__device__ void finalize(const SelectArgs& a, int r, const RowGeom& gm, int count) {
  int32_t* out = a.idx + (int64_t)r * a.out_ld;
  if (a.mode == SEL_RAW) {
    for (int i = count + threadIdx.x; i < a.out_ld; i += SEL_NT) out[i] = -1;
    if (threadIdx.x == 0) a.n_sel[r] = count;
    return;
  }
  const int ns = a.n_sink, W = a.n_window;
  for (int i = threadIdx.x; i < ns; i += SEL_NT) out[i] = i;
  const int w0 = ns + count;
  for (int i = threadIdx.x; i < W; i += SEL_NT) out[w0 + i] = gm.t - W + 1 + i;
  for (int i = w0 + W + threadIdx.x; i < a.out_ld; i += SEL_NT) out[i] = -1;
  if (threadIdx.x == 0) a.n_sel[r] = w0 + W;
}

// Chunk statistics: number of nonzero keys, their min and max.
template <int E>
__device__ void chunk_stats(const uint32_t (&u)[E], SelShared& sh, int& n_valid, uint32_t& kmin,
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
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  if (lane_id() == 0) {
    sh.red_w[0][wave_id()] = mn;
    sh.red_w[1][wave_id()] = mx;
  }
  int tot;
  block_excl_scan(cnt, sh, &tot);  // its barriers also publish red_w
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < SEL_NW; ++w) {
    mn = min(mn, sh.red_w[0][w]);
    mx = max(mx, sh.red_w[1][w]);
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

template <int E>
__global__ __launch_bounds__(SEL_NT) void select_stage_a(SelectArgs a) {
  __shared__ SelShared sh;
  constexpr int CH = SEL_NT * E;
  const int r = blockIdx.x, j = blockIdx.y;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) {
    if (j == 0) write_trivial(a, r, gm.t);
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
  chunk_stats<E>(u, sh, n_valid, kmin, kmax);
  int shift, r_eq;
  if (!plan_trivial(gm.k, n_valid, T, shift, r_eq)) radix_select<E>(u, kmin, kmax, gm.k, sh, T, shift, r_eq);
  const int i0 = threadIdx.x * E;
  if (n_chunks == 1) {
    int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
    const int cnt = compact<E>(u, T, shift, r_eq, sh, [&](int o, int e) { out[o] = pos_of(a, r, v0 + i0 + e); });
    finalize(a, r, gm, cnt);
  } else {
    const int64_t base = ((int64_t)r * a.max_chunks + j) * a.k_cap;
    int32_t* ws_s = a.ws_score + base;
    int32_t* ws_p = a.ws_pos + base;
    const int cnt = compact<E>(u, T, shift, r_eq, sh, [&](int o, int e) {
      ws_s[o] = (int32_t)(u[e] ^ 0x80000000u);
      ws_p[o] = pos_of(a, r, v0 + i0 + e);
    });
    for (int i = cnt + threadIdx.x; i < a.k_cap; i += SEL_NT) ws_s[i] = kMasked;
  }
}

// Stage B: top-k of the concatenated chunk survivors (n_chunks * k_cap
// entries, padded with INT32_MIN) of one row.
template <int E>
__global__ __launch_bounds__(SEL_NT) void select_stage_b(SelectArgs a, int CH) {
  __shared__ SelShared sh;
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
  chunk_stats<E>(u, sh, n_valid, kmin, kmax);
  int shift, r_eq;
  if (!plan_trivial(gm.k, n_valid, T, shift, r_eq)) radix_select<E>(u, kmin, kmax, gm.k, sh, T, shift, r_eq);
  const int i0 = threadIdx.x * E;
  int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
  const int cnt = compact<E>(u, T, shift, r_eq, sh, [&](int o, int e) { out[o] = ws_p[i0 + e]; });
  finalize(a, r, gm, cnt);
}

int chunk_e(int64_t max_nc) {
  if (max_nc <= SEL_NT * 4) return 4;
  if (max_nc <= SEL_NT * 16) return 16;
  return 32;
}

template <int E>
hipError_t launch_e(const SelectArgs& a, hipStream_t st) {
  constexpr int CH = SEL_NT * E;
  dim3 ga(a.n_rows, max(a.max_chunks, 1));
  hipLaunchKernelGGL((select_stage_a<E>), ga, dim3(SEL_NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  // survivors of one row: max_chunks * k_cap
  const int64_t nb = (int64_t)a.max_chunks * a.k_cap;
  if (nb <= SEL_NT * 4) hipLaunchKernelGGL((select_stage_b<4>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  else if (nb <= SEL_NT * 16) hipLaunchKernelGGL((select_stage_b<16>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  else hipLaunchKernelGGL((select_stage_b<32>), dim3(a.n_rows), dim3(SEL_NT), 0, st, a, CH);
  return hipGetLastError();
}

}  // namespace

int select_chunks(int64_t max_nc) {
  const int64_t ch = (int64_t)SEL_NT * chunk_e(max_nc);
  return (int)(max_nc <= ch ? 1 : (max_nc + ch - 1) / ch);
}

void select_plan(SelectArgs& a, int64_t max_nc) {
  a.chunk_e = chunk_e(max_nc);
  a.max_chunks = select_chunks(max_nc);
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

// max_chunks must equal select_chunks(max candidates per row) and the stage-B
// survivor count max_chunks * k_cap must fit 32 * 1024 entries.
hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.max_chunks > 1 && (int64_t)a.max_chunks * a.k_cap > kSelMaxSurvivors) return hipErrorInvalidValue;
  const int E = a.chunk_e;
  if (E == 4) return launch_e<4>(a, st);
  if (E == 16) return launch_e<16>(a, st);
  return launch_e<32>(a, st);
}

}  // namespace lsa
