// Radix-select building blocks shared by the selection kernels and the fused
// HI decode step: exact top-k of order-preserving uint32 keys held in
// registers (E per thread, blocked), an LDS histogram per 8-bit digit, and a
// stable compaction in thread (candidate) order. See select.hip for the
// method and its measured variants.
#pragma once
#include "lsa_device.h"

namespace lsa {

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
// than r_eq equal entries precede it. Only the kept entries are visited
// (STATIC: every e in turn, so that emit may index a register array by e
// without a per-lane index).
template <int E, int NT, bool STATIC = false, class Emit>
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
  if constexpr (STATIC) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((keep >> e) & 1u) emit(o++, e);
  } else {
    while (keep != 0u) {
      const int e = __ffs(keep) - 1;
      keep &= keep - 1u;
      emit(o++, e);
    }
  }
  return (int)(tot >> 16) + min((int)(tot & 0xffffu), r_eq);
}

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


}  // namespace lsa
