// HI block summary keys (gfx950).
//
// kbar[b, j, d] = clamp(round-half-even(sum of the block's keys / count), -128, 127).
// (LongCat-2.0 release article, section "LongCat 稀疏注意力", HI paragraph:
// a block-level approximate score drives the coarse recall; the summary key of
// a block is the rounded mean of its int8 indexer keys.)
//
// One wave owns one block: each 16-byte load of the wave covers 64 / (d_I /
// 16) whole consecutive key rows (1 KiB, coalesced), lane l taking dims
// 16 (l % (d_I / 16)) .. + 15 of row l / (d_I / 16) of each group; the 16
// per-dim sums are then added across the lanes that hold the same dims
// (lane-xor steps) and one lane per 16 dims writes the rounded means. Integer
// sums are exact, so the result does not depend on order. A launch covers
// blocks [j0, j0 + nbj) of every sequence, so appending keys to a cache
// recomputes only the blocks the new keys fall in.
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

// k: [B, n_cap, d_I] (n_len keys present per sequence); kb: [B, kb_rows, d_I].
__global__ __launch_bounds__(256) void block_summary_kernel(const int8_t* __restrict__ k, int B, int n_cap,
                                                            int n_len, int d_I, int blk, int j0, int nbj,
                                                            int kb_rows, int8_t* __restrict__ kb) {
  const int l = lane_id();
  const int64_t task = (int64_t)blockIdx.x * 4 + wave_id();
  if (task >= (int64_t)B * nbj) return;
  const int j = j0 + (int)(task % nbj);
  const int b = (int)(task / nbj);
  const int cpr = d_I / 16, rpl = 64 / cpr;  // 16-byte chunks per row, rows per wave load
  const int ci = l % cpr, rl = l / cpr;
  const int r0 = j * blk;
  const int c = min(blk, n_len - r0);
  int sum[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) sum[e] = 0;
  const int8_t* src = k + ((int64_t)b * n_cap + r0) * d_I + ci * 16;
  // four loads in flight per lane; rows past c read as zeros
  for (int r = rl; r < c; r += 4 * rpl) {
    v4i x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = r + u * rpl;
      x[u] = rr < c ? *(const v4i*)(src + (int64_t)rr * d_I) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[4 * w + e] += (int)(int8_t)((uint32_t)x[u][w] >> (8 * e));
  }
  for (int m = cpr; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[e] += shfl_xor_i(sum[e], m);
  if (rl != 0) return;
  v4i out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t u = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) u |= ((uint32_t)rne_div(sum[4 * w + e], c) & 0xffu) << (8 * e);
    out[w] = (int)u;
  }
  *(v4i*)(kb + ((int64_t)b * kb_rows + j) * d_I + ci * 16) = out;
}

hipError_t launch_block_summary(const int8_t* k, int B, int n_cap, int n_len, int d_I, int blk, int j0,
                                int nbj, int8_t* kb, hipStream_t st) {
  if (nbj <= 0) return hipSuccess;
  const int kb_rows = (int)(((int64_t)n_cap + blk - 1) / blk);
  const int64_t waves = (int64_t)B * nbj;  // one wave per block
  KernelTimer kt("block_summary_kernel", st);
  hipLaunchKernelGGL(block_summary_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     st, k, B, n_cap, n_len, d_I, blk, j0, nbj, kb_rows, kb);
  return hipGetLastError();
}

}  // namespace lsa
