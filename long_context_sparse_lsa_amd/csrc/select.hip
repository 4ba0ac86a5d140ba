// Top-k selection over exact int32 indexer scores (gfx950).
//
// Keeps, for each query row, the k candidates with the largest score; equal
// scores go to the lower position. (LongCat-2.0 release article, section
// "LongCat 稀疏注意力": the indexer picks the top-k keys per query; the SI
// paragraph pairs them with a contiguous window, and the sinks of the
// "架构拆解 ① LSA" section of the 1.6T training write-up are always kept.)
//
// Method: radix select on the order-preserving uint32 image of the score,
// 8 bits per pass, with LDS histograms (integer atomics: counts do not depend
// on arrival order). It yields the exact k-th largest score T and how many of
// the entries equal to T are taken; a stable, order-preserving compaction then
// keeps every entry above T and the first r entries equal to T. Candidates are
// laid out in ascending position, so the output is ascending and bit-exact.
//
// Rows with more than kSelChunk candidates run in two stages: stage A keeps
// min(k, chunk) per chunk (a superset of the row's top-k within that chunk),
// stage B selects the row's top-k from the concatenated chunk survivors.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

constexpr int SEL_NT = 512;
constexpr int SEL_NW = SEL_NT / 64;
constexpr int SEL_EPT = 4;

struct SelShared {
  uint32_t hist[256];
  int scan_tmp[SEL_NW];
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

__device__ __forceinline__ int block_excl_scan(int v, SelShared& sh, int* total) {
  const int incl = wave_incl_scan(v);
  if (lane_id() == 63) sh.scan_tmp[wave_id()] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_NW; ++w) {
    const int x = sh.scan_tmp[w];
    off += (w < wave_id()) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

__device__ __forceinline__ int block_sum(int v, SelShared& sh) {
  int tot;
  block_excl_scan(v, sh, &tot);
  return tot;
}

// Threshold of the k-th largest key among get(0..n-1) (0 < k <= #nonzero keys).
// Entry u is kept iff (u >> shift) > (T >> shift), or (u >> shift) == (T >> shift)
// and it is among the first r_eq such entries in index order.
template <class Get>
__device__ void radix_select(Get get, int n, int k, SelShared& sh, uint32_t& T, int& shift_out,
                             int& r_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int k_rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += SEL_NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += SEL_NT) {
      const uint32_t u = get(i);
      if ((u & mask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave_id() == 0) {
      const int l = lane_id();
      int h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (int)sh.hist[4 * l + e];
      const int s = h[0] + h[1] + h[2] + h[3];
      int v = s;
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
    k_rem -= above;
    prefix |= d << shift;
    mask |= 255u << shift;
    if (eq == k_rem || shift == 0) {
      T = prefix;
      shift_out = shift;
      r_eq = k_rem;
      return;
    }
  }
}

// Stable compaction: calls emit(out_pos, i, u) for every kept entry, in index
// order; returns the number kept (uniform over the block).
template <class Get, class Emit>
__device__ int compact(Get get, int n, uint32_t T, int shift, int r_eq, SelShared& sh, Emit emit) {
  const uint32_t Ts = T >> shift;
  int eq_before = 0, sel_before = 0;
  for (int base = 0; base < n; base += SEL_NT * SEL_EPT) {
    const int i0 = base + threadIdx.x * SEL_EPT;
    uint32_t u[SEL_EPT];
    int gt[SEL_EPT], eq[SEL_EPT];
    int n_eq = 0;
#pragma unroll
    for (int e = 0; e < SEL_EPT; ++e) {
      const bool in = i0 + e < n;
      u[e] = in ? get(i0 + e) : 0u;
      const uint32_t us = u[e] >> shift;
      gt[e] = in && us > Ts;
      eq[e] = in && us == Ts;
      n_eq += eq[e];
    }
    int eq_tot;
    int eq_rank = eq_before + block_excl_scan(n_eq, sh, &eq_tot);
    int sel[SEL_EPT], n_sel = 0;
#pragma unroll
    for (int e = 0; e < SEL_EPT; ++e) {
      sel[e] = gt[e] || (eq[e] && eq_rank < r_eq);
      eq_rank += eq[e];
      n_sel += sel[e];
    }
    int sel_tot;
    int opos = sel_before + block_excl_scan(n_sel, sh, &sel_tot);
#pragma unroll
    for (int e = 0; e < SEL_EPT; ++e)
      if (sel[e]) emit(opos++, i0 + e, u[e]);
    eq_before += eq_tot;
    sel_before += sel_tot;
  }
  return sel_before;
}

// Selection parameters for "keep k of the valid entries".
__device__ __forceinline__ void plan(int k, int n_valid, uint32_t& T, int& shift, int& r_eq,
                                     bool& need_radix) {
  need_radix = false;
  if (k <= 0) {
    T = 0xffffffffu;
    shift = 0;
    r_eq = 0;  // nothing exceeds T; ties not taken
  } else if (k >= n_valid) {
    T = 0u;
    shift = 0;
    r_eq = 0;  // every nonzero key exceeds 0
  } else {
    need_radix = true;
  }
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

__global__ __launch_bounds__(SEL_NT) void select_stage_a(SelectArgs a) {
  __shared__ uint32_t keys[kSelChunk];
  __shared__ SelShared sh;
  const int r = blockIdx.x, j = blockIdx.y;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) {
    if (j == 0) write_trivial(a, r, gm.t);
    return;
  }
  const int n_chunks = (gm.nc + kSelChunk - 1) / kSelChunk;
  if (j >= max(n_chunks, 1)) return;
  const int v0 = gm.c_lo + j * kSelChunk;
  const int n = min(kSelChunk, gm.nc - j * kSelChunk);
  const int32_t* row = a.scores + (int64_t)r * a.ld;
  int valid = 0;
  for (int i = threadIdx.x; i < n; i += SEL_NT) {
    const uint32_t u = score_key(row[v0 + i]);
    keys[i] = u;
    valid += u != 0u;
  }
  const int n_valid = block_sum(valid, sh);  // includes a barrier: keys[] complete
  uint32_t T;
  int shift, r_eq;
  bool need;
  plan(gm.k, n_valid, T, shift, r_eq, need);
  auto get = [&](int i) -> uint32_t { return keys[i]; };
  if (need) radix_select(get, n, gm.k, sh, T, shift, r_eq);
  if (n_chunks <= 1) {
    int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
    const int cnt = compact(get, n, T, shift, r_eq, sh,
                            [&](int o, int i, uint32_t) { out[o] = pos_of(a, r, v0 + i); });
    finalize(a, r, gm, cnt);
  } else {
    const int64_t base = ((int64_t)r * a.max_chunks + j) * a.k_cap;
    int32_t* ws_s = a.ws_score + base;
    int32_t* ws_p = a.ws_pos + base;
    const int cnt = compact(get, n, T, shift, r_eq, sh, [&](int o, int i, uint32_t u) {
      ws_s[o] = (int32_t)(u ^ 0x80000000u);
      ws_p[o] = pos_of(a, r, v0 + i);
    });
    for (int i = cnt + threadIdx.x; i < a.k_cap; i += SEL_NT) ws_s[i] = kMasked;
  }
}

__global__ __launch_bounds__(SEL_NT) void select_stage_b(SelectArgs a) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  const RowGeom gm = row_geom(a, r);
  if (gm.trivial) return;
  const int n_chunks = (gm.nc + kSelChunk - 1) / kSelChunk;
  if (n_chunks <= 1) return;
  const int n = n_chunks * a.k_cap;
  const int64_t base = (int64_t)r * a.max_chunks * a.k_cap;
  const int32_t* ws_s = a.ws_score + base;
  const int32_t* ws_p = a.ws_pos + base;
  int valid = 0;
  for (int i = threadIdx.x; i < n; i += SEL_NT) valid += ws_s[i] != kMasked;
  const int n_valid = block_sum(valid, sh);
  uint32_t T;
  int shift, r_eq;
  bool need;
  plan(gm.k, n_valid, T, shift, r_eq, need);
  auto get = [&](int i) -> uint32_t { return score_key(ws_s[i]); };
  if (need) radix_select(get, n, gm.k, sh, T, shift, r_eq);
  int32_t* out = a.idx + (int64_t)r * a.out_ld + (a.mode == SEL_RAW ? 0 : a.n_sink);
  const int cnt =
      compact(get, n, T, shift, r_eq, sh, [&](int o, int i, uint32_t) { out[o] = ws_p[i]; });
  finalize(a, r, gm, cnt);
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

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  dim3 ga(a.n_rows, max(a.max_chunks, 1));
  hipLaunchKernelGGL(select_stage_a, ga, dim3(SEL_NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  hipLaunchKernelGGL(select_stage_b, dim3(a.n_rows), dim3(SEL_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
