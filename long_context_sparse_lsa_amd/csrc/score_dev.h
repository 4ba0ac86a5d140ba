// Decode / HI indexer scoring device code, shared by index_decode_kernel and
// the fused HI decode step. The design is described in index_decode.hip.
#pragma once
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {


constexpr int kWaves = 4;
constexpr int kDepthLong = 4;      // key tiles in flight per wave, long scans
constexpr int kDepthShort = 2;     // and in launches of at most 4 tiles per wave
constexpr int kMaxBlkIds = 136;    // block-table entries per wave in LDS
constexpr int kMaxKeysPerWave = 4096;

template <int MB, int KS>
__device__ __forceinline__ void tile_mfma(const v4i (&A)[MB][KS], const v4i (&Bk)[KS], v16i (&acc)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v16i{};
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_i8_32x32x32(A[mb][j], Bk[j], acc[mb]);
}

// Lane-partial score of query qi (its M-blocks [qi * MQ, (qi + 1) * MQ)).
template <int MB, int MQ, bool FOLD>
__device__ __forceinline__ int query_sum(const v16i (&acc)[MB], int qi, const int* wl) {
  int s = 0;
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    const int mb = qi * MQ + m;
    if constexpr (FOLD) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) s = s + max(acc[mb][i], 0) + max(acc[mb][i + 1], 0);
    } else {
      const int g = lane_id() >> 5;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v4i w4 = *(const v4i*)(wl + 32 * mb + 8 * i4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) s += __mul24(max(acc[mb][4 * i4 + e], 0), w4[e]);
      }
    }
  }
  return s;
}

template <int HI, int DI, int DEPTH, bool FOLD>
__device__ __forceinline__ void scan_keys(const ScoreArgs& a, const v4i (&A)[HI >= 64 ? HI / 32 : 2][DI / 32],
                                          const int* wl, const int* blw, int bfirst, int b, int q0, int v0,
                                          int v1) {
  constexpr int MB = HI >= 64 ? HI / 32 : 2;
  constexpr int NQ = 32 * MB / HI;  // query rows per wave: 1 or 2
  const int mask_off = a.mask_off + seq_shift(a.shift, b);
  constexpr int MQ = MB / NQ;       // M-blocks per query
  constexpr int KS = DI / 32;
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const bool direct = a.blocks == nullptr;
  const int8_t* kb = a.k + (int64_t)b * a.k_bstride;
  int32_t* sc = a.scores + (int64_t)b * a.s_bstride;

  auto pos_of = [&](int v) -> int {
    if (direct) return v;
    const int bi = blw[v / a.blk - bfirst];
    return bi < 0 ? -1 : bi * a.blk + v % a.blk;
  };
  auto load = [&](int t, v4i (&Bt)[KS]) {
    const int p = pos_of(min(v0 + 32 * t + c, v1 - 1));
    const int pp = (unsigned)p < (unsigned)a.n_k ? p : 0;
    const v4i* src = (const v4i*)(kb + (int64_t)pp * DI + g * (DI / 2));
#pragma unroll
    for (int j = 0; j < KS; ++j) Bt[j] = src[j];
  };
  auto store = [&](int qi, int v, int p, int val) {
    const int gq = q0 + qi;
    if (gq >= a.n_q || v >= v1) return;
    const bool vis = p >= a.pos_lo && p <= mask_off + gq;
    if (vis) sc[(int64_t)gq * a.ld + v] = val;
    else if (a.fill_masked) sc[(int64_t)gq * a.ld + v] = kMasked;
  };

  const int T = (v1 - v0 + 31) / 32;
  v4i ring[DEPTH][KS];
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) load(u, ring[u]);
  for (int t0 = 0; t0 < T; t0 += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int t = t0 + u;
      if (t < T) {
        v16i acc[MB];
        tile_mfma<MB, KS>(A, ring[u], acc);
        const int v = v0 + 32 * t + c;
        const int p = v < v1 ? pos_of(v) : -1;
        if constexpr (NQ == 1) {
          const int s = xor32_sum(query_sum<MB, MQ, FOLD>(acc, 0, wl));
          if (g == 0) store(0, v, p, s);
        } else {
          const int s0 = query_sum<MB, MQ, FOLD>(acc, 0, wl);
          const int s1 = query_sum<MB, MQ, FOLD>(acc, 1, wl);
          // lane half g finishes query g
          store(g, v, p, pair_sum32(s0, s1));
        }
      }
      load(t + DEPTH, ring[u]);
    }
  }
}

// The scan of wave wv (of kWaves) in workgroup (bq, by, b) of the decode
// scoring grid: query tile bq, keys [(by * kWaves + wv) * kpw, + kpw). wl: the
// weights in LDS (128 entries); bl: kWaves * kMaxBlkIds ints of LDS.
template <int HI, int DI, int DEPTH>
__device__ __forceinline__ void decode_score_body(const ScoreArgs& a, int kpw, int fold_ok, int bq, int by, int b,
                                                  int wv, const int* wl, int* bl) {
  constexpr int MB = HI >= 64 ? HI / 32 : 2;
  constexpr int NQ = 32 * MB / HI;
  constexpr int KS = DI / 32;
  const int l = lane_id(), c = l & 31, g = l >> 5;
  const int q0 = bq * NQ;
  const int nq_tile = min(NQ, a.n_q - q0);
  const int v0 = (by * kWaves + wv) * kpw;
  const int v1 = min(v0 + kpw, a.n_keys);
  if (v0 >= v1) return;
  const bool direct = a.blocks == nullptr;
  const int mask_off = a.mask_off + seq_shift(a.shift, b);
  if (direct && (v0 > mask_off + q0 + nq_tile - 1 || v1 <= a.pos_lo)) {
    // nothing in this range is visible to any row of the tile
    if (a.fill_masked) {
      int32_t* sc = a.scores + (int64_t)b * a.s_bstride;
      for (int qi = 0; qi < nq_tile; ++qi)
        for (int v = v0 + l; v < v1; v += 64) sc[(int64_t)(q0 + qi) * a.ld + v] = kMasked;
    }
    return;
  }
  // this wave's slice of the block table (HI fine stage)
  int* blw = bl + wv * kMaxBlkIds;
  const int bfirst = direct ? 0 : v0 / a.blk;
  if (!direct) {
    const int nb = (v1 - 1) / a.blk - bfirst + 1;
    for (int i = l; i < nb; i += 64) blw[i] = a.blocks[(int64_t)b * a.nbr + bfirst + i];
  }

  // A operand: this wave's query rows, MB M-blocks x KS 16-byte pieces
  v4i A[MB][KS];
  const int8_t* qb = a.q + (int64_t)b * a.q_bstride;
  bool ok = fold_ok != 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = 32 * mb + c;
    const int gq = q0 + r / HI, h = r % HI;
    const v4i* src = (const v4i*)(qb + ((int64_t)gq * HI + h) * DI + g * (DI / 2));
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      A[mb][j] = gq < a.n_q ? src[j] : v4i{0, 0, 0, 0};
      ok = ok && bytes_scale_fit(A[mb][j], wl[h]);
    }
  }
  if (__all(ok)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < KS; ++j) A[mb][j] = scale_bytes(A[mb][j], wl[(32 * mb + c) % HI]);
    scan_keys<HI, DI, DEPTH, true>(a, A, wl, blw, bfirst, b, q0, v0, v1);
  } else {
    scan_keys<HI, DI, DEPTH, false>(a, A, wl, blw, bfirst, b, q0, v0, v1);
  }
}

}  // namespace lsa
