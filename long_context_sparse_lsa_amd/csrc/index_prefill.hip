// Indexer scoring for many query rows at once (prefill), int8 MFMA on gfx950.
//
// S[t, s] = sum_h w[h] * max(0, q_I[t, h, :] . k_I[s, :]), exact in int32.
// (LongCat-2.0 release article, section "LongCat 稀疏注意力": the lightweight
// indexer scores the keys for each query; the arithmetic -- int8 q/k, integer
// head weights, int32 result -- is fixed by this library.)
//
// GEMM view: M = (query, head) rows, N = keys, K = d_I. A workgroup of 4 waves
// owns 4 * QW queries and walks a chunk of keys in tiles of 128 keys that are
// staged once in LDS and read by all four waves (each key byte feeds
// 4 * QW * H_I multiply-adds). A wave keeps its QW queries (QW * H_I rows) in
// registers as the A operand for the whole chunk.
//
// Weight folding: w[h] * max(0, x) == max(0, w[h] * x) for w[h] >= 0, and
// (w[h] q) . k == w[h] (q . k). When every weight is >= 0 and every product
// w[h] * q[t, h, d] of a wave's rows fits int8, the wave multiplies the
// weights into its A operand once, and the epilogue is a plain sum of ReLUs
// (max + three-input add). Otherwise the wave keeps q as is and applies the
// weights in the epilogue (max + 24-bit multiply-add). Both are exact, so the
// choice never changes a score.
//
// Output layout of the 32x32x32 int8 MFMA: lane l holds key column l % 32 and
// rows 8 * (i / 4) + 4 * (l / 32) + i % 4 of register i. A query owns H_I
// consecutive rows, i.e. H_I / 32 whole M-blocks, so its head sum is a
// per-lane sum over those blocks plus one exchange between lane halves.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int kTileKeys = 128;  // keys per LDS tile
constexpr int kQW = 2;          // queries per wave
constexpr int kWaves = 4;
constexpr int kQT = kQW * kWaves;  // queries per workgroup

template <int DI>
struct TileGeom {
  static constexpr int kRow = DI + 16;                 // padded LDS row: conflict-free b128 reads
  static constexpr int kBytes = kTileKeys * kRow;      // one stage
  static constexpr int kChunks = kTileKeys * DI / 16;  // 16-byte pieces per tile
  static constexpr int kPerThread = kChunks / (64 * kWaves);
};

// True iff w times each of the 16 int8 values of v stays in [-128, 127].
__device__ __forceinline__ bool bytes_scale_fit(v4i v, int w) {
  bool ok = true;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int x = (int)(int8_t)((uint32_t)v[e] >> (8 * b)) * w;
      ok = ok && x >= -128 && x <= 127;
    }
  return ok;
}

// The 16 int8 values of v times w (each product known to fit int8).
__device__ __forceinline__ v4i scale_bytes(v4i v, int w) {
  v4i r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t o = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int x = (int)(int8_t)((uint32_t)v[e] >> (8 * b)) * w;
      o |= ((uint32_t)x & 0xffu) << (8 * b);
    }
    r[e] = (int)o;
  }
  return r;
}

template <int HI, int DI, bool FOLD>
__device__ __forceinline__ void score_chunk(const ScoreArgs& a, const v4i (&A)[kQW][HI / 32][DI / 32],
                                            const int* wl, const int8_t* kb, char* lds, int v_begin,
                                            int v_end, int row0, int32_t* sc) {
  using G = TileGeom<DI>;
  constexpr int MB = HI / 32, KS = DI / 32;
  const int tid = threadIdx.x;
  const int l = lane_id(), g = l >> 5, c = l & 31;
  // per-register head weights (rows 8*(i/4) + 4*g + i%4 of block mb); only
  // the unfolded epilogue needs them
  int W[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) W[mb][i] = FOLD ? 0 : wl[32 * mb + 8 * (i / 4) + 4 * g + (i % 4)];
  // The two queries of this wave sit at rows row0 and row0 + 1; lane half g
  // stores row row0 + g.
  const int my_row = row0 + g;
  const int vis_hi_row = a.mask_off + my_row;                 // last visible key of my row
  const int vis_hi_wave = a.mask_off + min(row0 + kQW - 1, a.n_q - 1);

  // global -> register prefetch of one tile
  v4i pf[G::kPerThread];
  auto fetch = [&](int v0) {
#pragma unroll
    for (int u = 0; u < G::kPerThread; ++u) {
      const int id = tid + u * 64 * kWaves;
      const int key = id / (DI / 16), part = id % (DI / 16);
      const int v = v0 + key;
      pf[u] = v < v_end ? *(const v4i*)(kb + (int64_t)v * DI + part * 16) : v4i{0, 0, 0, 0};
    }
  };
  auto stash = [&](char* stage) {
#pragma unroll
    for (int u = 0; u < G::kPerThread; ++u) {
      const int id = tid + u * 64 * kWaves;
      const int key = id / (DI / 16), part = id % (DI / 16);
      *(v4i*)(stage + key * G::kRow + part * 16) = pf[u];
    }
  };

  fetch(v_begin);
  stash(lds);
  __syncthreads();
  int stage = 0;
  for (int v0 = v_begin; v0 < v_end; v0 += kTileKeys) {
    const bool more = v0 + kTileKeys < v_end;
    if (more) fetch(v0 + kTileKeys);
    const char* tile = lds + stage * G::kBytes;
#pragma unroll 1
    for (int nb = 0; nb < kTileKeys / 32; ++nb) {
      const int p0 = v0 + 32 * nb;  // first key of the block
      if (p0 >= v_end) break;
      const int v = p0 + c;
      const bool blk_vis = p0 <= vis_hi_wave && p0 + 31 >= a.pos_lo;
      if (!blk_vis) {
        if (a.fill_masked && my_row < a.n_q && v < v_end) sc[(int64_t)my_row * a.ld + v] = kMasked;
        continue;
      }
      v4i Bk[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) Bk[j] = *(const v4i*)(tile + (32 * nb + c) * G::kRow + g * (DI / 2) + 16 * j);
      int part[kQW];
#pragma unroll
      for (int q = 0; q < kQW; ++q) {
        v16i acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = v16i{};
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_i8_32x32x32(A[q][mb][j], Bk[j], acc[mb]);
        int s = 0;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            if constexpr (FOLD) {
              s = s + max(acc[mb][i], 0) + max(acc[mb][i + 1], 0);
            } else {
              s += __mul24(max(acc[mb][i], 0), W[mb][i]) + __mul24(max(acc[mb][i + 1], 0), W[mb][i + 1]);
            }
          }
        part[q] = s;
      }
      // lane half g finishes query g: it keeps its own part of query g and
      // receives the other half's part of query g
      const int send = g ? part[0] : part[1];
      const int recv = shfl_xor_i(send, 32);
      const int full = (g ? part[1] : part[0]) + recv;
      if (my_row < a.n_q && v < v_end) {
        if (v >= a.pos_lo && v <= vis_hi_row) sc[(int64_t)my_row * a.ld + v] = full;
        else if (a.fill_masked) sc[(int64_t)my_row * a.ld + v] = kMasked;
      }
    }
    if (more) {
      stash(lds + (stage ^ 1) * G::kBytes);
      stage ^= 1;
    }
    __syncthreads();
  }
}

template <int HI, int DI>
__global__ __launch_bounds__(256, 2) void index_prefill_kernel(ScoreArgs a, int KC, int fold_ok) {
  using G = TileGeom<DI>;
  constexpr int MB = HI / 32, KS = DI / 32;
  __shared__ __attribute__((aligned(16))) char lds[2 * G::kBytes];
  __shared__ int wl[HI];
  const int chunk = blockIdx.x, qt = blockIdx.y, b = blockIdx.z;
  const int q0 = qt * kQT;
  const int v_begin = chunk * KC;
  const int v_end = min(v_begin + KC, a.n_keys);
  const int last_row = min(q0 + kQT, a.n_q) - 1;
  int32_t* sc = a.scores + (int64_t)b * a.s_bstride;
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int wv = wave_id();

  // whole chunk invisible to every row of the tile
  if (v_begin > a.mask_off + last_row || v_end <= a.pos_lo) {
    if (a.fill_masked) {
      for (int r = q0; r <= last_row; ++r)
        for (int v = v_begin + threadIdx.x; v < v_end; v += 256) sc[(int64_t)r * a.ld + v] = kMasked;
    }
    return;
  }
  if (threadIdx.x < HI) wl[threadIdx.x] = a.w.w[threadIdx.x];
  __syncthreads();

  const int row0 = q0 + wv * kQW;
  v4i A[kQW][MB][KS];
  const int8_t* qb = a.q + (int64_t)b * a.q_bstride;
#pragma unroll
  for (int q = 0; q < kQW; ++q)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = row0 + q, h = 32 * mb + c;
      const v4i* src = (const v4i*)(qb + ((int64_t)row * HI + h) * DI + g * (DI / 2));
#pragma unroll
      for (int j = 0; j < KS; ++j) A[q][mb][j] = row < a.n_q ? src[j] : v4i{0, 0, 0, 0};
    }
  // fold the weights into A when that is exact for every row of the wave
  bool ok = fold_ok != 0;
#pragma unroll
  for (int q = 0; q < kQW; ++q)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int wh = wl[32 * mb + c];
#pragma unroll
      for (int j = 0; j < KS; ++j) ok = ok && bytes_scale_fit(A[q][mb][j], wh);
    }
  const bool fold = __all(ok);
  const int8_t* kb = a.k + (int64_t)b * a.k_bstride;
  if (fold) {
#pragma unroll
    for (int q = 0; q < kQW; ++q)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int wh = wl[32 * mb + c];
#pragma unroll
        for (int j = 0; j < KS; ++j) A[q][mb][j] = scale_bytes(A[q][mb][j], wh);
      }
    score_chunk<HI, DI, true>(a, A, wl, kb, lds, v_begin, v_end, row0, sc);
  } else {
    score_chunk<HI, DI, false>(a, A, wl, kb, lds, v_begin, v_end, row0, sc);
  }
}

template <int HI, int DI>
hipError_t launch_t(const ScoreArgs& a, int fold_ok, hipStream_t st) {
  // keys per workgroup: long enough to amortise the A load, short enough to
  // give the chip many workgroups
  const int KC = 1024;
  dim3 grid((a.n_keys + KC - 1) / KC, (a.n_q + kQT - 1) / kQT, a.B);
  hipLaunchKernelGGL((index_prefill_kernel<HI, DI>), grid, dim3(256), 0, st, a, KC, fold_ok);
  return hipGetLastError();
}

}  // namespace

bool index_prefill_supported(const ScoreArgs& a) {
  return a.blocks == nullptr && (a.H_I == 32 || a.H_I == 64) &&
         (a.d_I == 64 || a.d_I == 128) && a.n_q >= kQT;
}

hipError_t launch_index_prefill(const ScoreArgs& a, hipStream_t st) {
  int fold_ok = 1;
  for (int h = 0; h < a.H_I; ++h) fold_ok &= a.w.w[h] >= 0;
#define LSA_CASE(h, d) \
  if (a.H_I == h && a.d_I == d) return launch_t<h, d>(a, fold_ok, st);
  LSA_CASE(32, 64) LSA_CASE(32, 128) LSA_CASE(64, 64) LSA_CASE(64, 128)
#undef LSA_CASE
  return hipErrorInvalidValue;
}

}  // namespace lsa
