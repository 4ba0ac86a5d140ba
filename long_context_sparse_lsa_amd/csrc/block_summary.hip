// HI block summary keys (gfx950).
//
// kbar[b, j, d] = clamp(round-half-even(sum of the block's keys / count), -128, 127).
// (LongCat-2.0 release article, section "LongCat 稀疏注意力", HI paragraph:
// a block-level approximate score drives the coarse recall; the summary key of
// a block is the rounded mean of its int8 indexer keys.)
//
// A wave takes blocks in turn (block w, w + waves, ...: consecutive waves
// read consecutive blocks at the same time). Each 16-byte load of the wave
// covers 64 / (d_I / 16) whole consecutive key rows (1 KiB, coalesced), lane l
// taking dims 16 (l % (d_I / 16)) .. + 15 of row l / (d_I / 16) of each
// group, and eight such loads are in flight together (sixteen when a block
// fits one round of loads: the wave's next block loads while the current
// one is reduced; measured 124 -> 108 us at four 1M-key caches, 4.97 TB/s,
// against 5.8-5.95 TB/s for a plain streaming read). Blocks of at most 256
// rows are summed as biased bytes (value + 128, at most 65280 per dim) in
// 16-bit fields, two dims per register (one byte permute and one add per two
// bytes), so the per-dim sums take 8 registers instead of 16; the sums are
// then added across the lanes that hold the same dims (lane-xor steps) and
// one lane per 16 dims writes the rounded means, with shifts when the row
// count is a power of two. Integer sums are exact, so the result does not
// depend on order. A launch covers blocks [j0, j0 + nbj) of every sequence,
// so appending keys to a cache recomputes only the blocks the new keys fall
// in.
#include <algorithm>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

__device__ __forceinline__ int rne_div(int s, int c) {
  int q = s / c;
  if (s % c != 0 && s < 0) q -= 1;  // floor
  const int r = s - q * c;          // 0 <= r < c
  q += (2 * r > c) || (2 * r == c && (q & 1));
  return min(127, max(-128, q));
}

// The same for c = 2^sh.
__device__ __forceinline__ int rne_shift(int s, int sh) {
  int q = s >> sh;                // floor
  const int r = s - (q << sh);    // 0 <= r < c
  const int c = 1 << sh;
  q += (2 * r > c) || (2 * r == c && (q & 1));
  return min(127, max(-128, q));
}

constexpr int kLoads = 8;  // 16-byte loads in flight per lane

// Writes the rounded means of a block (sum[e]: dims 16 ci + e over c rows).
__device__ __forceinline__ void put_means(const int (&sum)[16], int c, int8_t* dst) {
  const bool pow2 = (c & (c - 1)) == 0;
  const int sh = 31 - __clz(c);
  v4i out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t u = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = pow2 ? rne_shift(sum[4 * w + e], sh) : rne_div(sum[4 * w + e], c);
      u |= ((uint32_t)m & 0xffu) << (8 * e);
    }
    out[w] = (int)u;
  }
  *(v4i*)dst = out;
}

// A missing row loads as bytes of -128, which the bias turns into zeros.
constexpr int kAbsent = (int)0x80808080u;

// Biased 16-bit sums of one lane's loaded rows into acc (see above).
__device__ __forceinline__ void add_packed(const v4i (&x)[kLoads], uint32_t (&acc)[8]) {
#pragma unroll
  for (int u = 0; u < kLoads; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t y = (uint32_t)x[u][w] ^ 0x80808080u;
      acc[2 * w] += __builtin_amdgcn_perm(0u, y, 0x0c020c00u);
      acc[2 * w + 1] += __builtin_amdgcn_perm(0u, y, 0x0c030c01u);
    }
}

// Lane sums over the lanes holding the same dims, then the means of block
// (b, j) of c rows.
__device__ __forceinline__ void finish_packed(uint32_t (&acc)[8], int cpr, int rl, int c, int8_t* dst) {
  for (int m = cpr; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (uint32_t)shfl_xor_i((int)acc[e], m);
  if (rl != 0) return;
  int sum[16];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sum[4 * w + 0] = (int)(acc[2 * w] & 0xffffu) - 128 * c;
    sum[4 * w + 2] = (int)(acc[2 * w] >> 16) - 128 * c;
    sum[4 * w + 1] = (int)(acc[2 * w + 1] & 0xffffu) - 128 * c;
    sum[4 * w + 3] = (int)(acc[2 * w + 1] >> 16) - 128 * c;
  }
  put_means(sum, c, dst);
}

// k: [B, n_cap, d_I] (n_len keys present per sequence); kb: [B, kb_rows, d_I].
// PACK: blocks of at most 256 rows (16-bit biased sums). Blocks that one
// round of loads covers (blk <= 8 * rows per load) are double-buffered: the
// wave's next block is loaded while the current one is reduced.
template <bool PACK>
__global__ __launch_bounds__(256) void block_summary_kernel(const int8_t* __restrict__ k, int B, int n_cap,
                                                            int n_len, int d_I, int blk, int j0, int nbj,
                                                            int kb_rows, int8_t* __restrict__ kb) {
  const int l = lane_id();
  const int cpr = d_I / 16, rpl = 64 / cpr;  // 16-byte chunks per row, rows per wave load
  const int ci = l % cpr, rl = l / cpr;
  const int64_t n_tasks = (int64_t)B * nbj;
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  const int64_t first = (int64_t)blockIdx.x * 4 + wave_id();
  // task -> (rows present c, first key byte of this lane, summary row)
  auto geom = [&](int64_t task, int& c, const int8_t*& src, int8_t*& dst) {
    const int j = j0 + (int)(task % nbj);
    const int b = (int)(task / nbj);
    const int r0 = j * blk;
    c = min(blk, n_len - r0);
    src = k + ((int64_t)b * n_cap + r0) * d_I + ci * 16;
    dst = kb + ((int64_t)b * kb_rows + j) * d_I + ci * 16;
  };
  // rows past c: bytes of -128 (zeros after the bias of the packed sums;
  // the plain sums take them away again below)
  auto load = [&](const int8_t* src, int c, v4i (&x)[kLoads]) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int rr = rl + u * rpl;
      x[u] = rr < c ? *(const v4i*)(src + (int64_t)rr * d_I) : v4i{kAbsent, kAbsent, kAbsent, kAbsent};
    }
  };
  if constexpr (PACK) {
    if (blk <= kLoads * rpl) {
      int c0, c1;
      const int8_t *s0, *s1;
      int8_t *d0, *d1;
      v4i x0[kLoads], x1[kLoads];
      int64_t task = first;
      if (task < n_tasks) {
        geom(task, c0, s0, d0);
        load(s0, c0, x0);
      }
      while (task < n_tasks) {
        const int64_t t1 = task + n_waves;
        if (t1 < n_tasks) {
          geom(t1, c1, s1, d1);
          load(s1, c1, x1);
        }
        uint32_t acc[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        add_packed(x0, acc);
        finish_packed(acc, cpr, rl, c0, d0);
        if (t1 >= n_tasks) break;
        const int64_t t2 = t1 + n_waves;
        if (t2 < n_tasks) {
          geom(t2, c0, s0, d0);
          load(s0, c0, x0);
        }
        uint32_t acc1[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        add_packed(x1, acc1);
        finish_packed(acc1, cpr, rl, c1, d1);
        task = t2;
      }
      return;
    }
  }
  for (int64_t task = first; task < n_tasks; task += n_waves) {
    int c;
    const int8_t* src;
    int8_t* dst;
    geom(task, c, src, dst);
    if constexpr (PACK) {
      uint32_t acc[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      for (int r = 0; r < c; r += kLoads * rpl) {
        v4i x[kLoads];
        load(src + (int64_t)r * d_I, c - r, x);
        add_packed(x, acc);
      }
      finish_packed(acc, cpr, rl, c, dst);
    } else {
      int sum[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[e] = 0;
      for (int r = 0; r < c; r += kLoads * rpl) {
        v4i x[kLoads];
        load(src + (int64_t)r * d_I, c - r, x);
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[4 * w + e] += (int)(int8_t)((uint32_t)x[u][w] >> (8 * e));
      }
      // this lane's missing rows added -128 each to its 16 dims
      int missing = 0;
      for (int r = 0; r < c; r += kLoads * rpl)
#pragma unroll
        for (int u = 0; u < kLoads; ++u) missing += rl + u * rpl >= c - r;
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[e] += 128 * missing;
      for (int m = cpr; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[e] += shfl_xor_i(sum[e], m);
      if (rl == 0) put_means(sum, c, dst);
    }
  }
}

hipError_t launch_block_summary(const int8_t* k, int B, int n_cap, int n_len, int d_I, int blk, int j0,
                                int nbj, int8_t* kb, hipStream_t st) {
  if (nbj <= 0) return hipSuccess;
  const int kb_rows = (int)(((int64_t)n_cap + blk - 1) / blk);
  // two resident waves per SIMD (the double-buffered form holds two blocks'
  // loads in 175 VGPRs), each taking blocks in turn
  const int64_t waves = std::min<int64_t>((int64_t)B * nbj, 256 * 4 * 2);
  KernelTimer kt("block_summary_kernel", st);
  if (blk <= 256)
    hipLaunchKernelGGL(block_summary_kernel<true>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, k, B, n_cap,
                       n_len, d_I, blk, j0, nbj, kb_rows, kb);
  else
    hipLaunchKernelGGL(block_summary_kernel<false>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, k, B,
                       n_cap, n_len, d_I, blk, j0, nbj, kb_rows, kb);
  return hipGetLastError();
}

}  // namespace lsa
