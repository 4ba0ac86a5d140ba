// HI block summary keys (gfx950).
//
// kbar[b, j, d] = clamp(round-half-even(sum of the block's keys / count), -128, 127).
// (LongCat-2.0 release article, section "LongCat 稀疏注意力", HI paragraph:
// a block-level approximate score drives the coarse recall; the summary key of
// a block is the rounded mean of its int8 indexer keys.)
//
// One thread owns 16 dims of one block and walks the block's rows with 16-byte
// loads; integer sums are exact, so the result does not depend on order. A
// launch covers blocks [j0, j0 + nbj) of every sequence, so appending keys to
// a cache recomputes only the blocks the new keys fall in.
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
  const int cpr = d_I / 16;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)B * nbj * cpr) return;
  const int ci = (int)(t % cpr);
  const int j = j0 + (int)((t / cpr) % nbj);
  const int b = (int)(t / ((int64_t)cpr * nbj));
  const int r0 = j * blk;
  const int c = min(blk, n_len - r0);
  int sum[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) sum[e] = 0;
  const int8_t* src = k + ((int64_t)b * n_cap + r0) * d_I + ci * 16;
  for (int r = 0; r < c; ++r) {
    const v4i x = *(const v4i*)(src + (int64_t)r * d_I);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[4 * w + e] += (int)(int8_t)((uint32_t)x[w] >> (8 * e));
  }
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
  const int64_t threads = (int64_t)B * nbj * (d_I / 16);
  KernelTimer kt("block_summary_kernel", st);
  hipLaunchKernelGGL(block_summary_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, k, B, n_cap, n_len, d_I, blk, j0, nbj, kb_rows, kb);
  return hipGetLastError();
}

}  // namespace lsa
