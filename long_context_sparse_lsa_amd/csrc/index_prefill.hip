// Indexer scoring for many query rows at once (prefill), int8 MFMA on gfx950.
//
// S[t, s] = sum_h w[h] * max(0, q_I[t, h, :] . k_I[s, :]), exact in int32.
// (LongCat-2.0 release article, section "LongCat 稀疏注意力": the lightweight
// indexer scores the keys for each query; the arithmetic -- int8 q/k, integer
// head weights, int32 result -- is fixed by this library.)
//
// GEMM view: M = (query, head) rows, N = keys, K = d_I. A workgroup of 4 waves
// (one per SIMD) owns 8 consecutive queries, 2 per wave, and walks a chunk
// of 4096 to 16384 keys in tiles of 128 keys that are staged once in LDS
// (double-buffered) and read by all four waves. A wave keeps its 2 queries'
// rows (2 * H_I rows) in registers as the A operand for the whole chunk, so
// every 16-byte LDS read of the key operand feeds 2 * H_I / 32 MFMAs, and the
// A operand is loaded once per chunk (the longest chunk that still leaves
// several rounds of workgroups).
//
// Per 32-key block a wave runs, for each of its 2 queries, H_I/32 * d_I/32
// MFMAs and a ReLU / head-sum epilogue on the VALU. The MFMA pipe and the
// VALU overlap across waves, not within one: three workgroups share a CU (at
// most 168 registers per lane, 33 KB of LDS each), so each SIMD holds three
// waves and their epilogues run under one another's MFMAs (2.3% faster at
// the 128K prefill than two waves of 4 queries with 256-key tiles).
//
// Weight folding: w[h] * max(0, x) == max(0, w[h] * x) for w[h] >= 0, and
// (w[h] q) . k == w[h] (q . k). When every weight is >= 0 and every product
// w[h] * q[t, h, d] of the wave's queries fits int8, the wave multiplies the
// weights into its A operand once, and the epilogue is a plain sum of ReLUs
// (max + three-input add). Otherwise the wave keeps q as is and applies the
// weights in the epilogue (max + 24-bit multiply-add, weights read from LDS).
// Both are exact, so the choice never changes a score.
//
// Filtered output: with a per-row threshold tau, a pair of queries' 32
// scores (one per lane half) is kept where score >= tau of the lane's query.
// A ballot gives the kept lanes, their rank within the half (mbcnt) their
// place after the row's running count, and one 8-byte buffer store per lane
// writes (score, position) (dropped lanes store out of range, so there is no
// branch); each row's keys are visited by one wave in key order, so each
// (row, chunk) segment is in ascending position order.
//
// Output layout of the 32x32x32 int8 MFMA: lane l holds key column l % 32 and
// rows 8 * (i / 4) + 4 * (l / 32) + i % 4 of register i. A query owns H_I
// consecutive rows (H_I / 32 whole M-blocks), so its head sum is a per-lane
// sum plus one exchange between lane halves. Queries are finished in pairs:
// lane half g ends up with query 2p + g's sums, and one 64-lane store writes
// both queries' 32 scores.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int kTileKeys = 128;  // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kQW = 2;                   // queries per wave
constexpr int kQT = kWaves * kQW;        // queries per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMinChunkKeys = 4096;      // keys per workgroup: 4096, 8192 or 16384
constexpr int kMaxChunkKeys = 16384;
constexpr int kFullGrid = 2048;           // workgroups of about three rounds over the chip
constexpr int kBlocks = kTileKeys / 32;  // 32-key blocks per tile

// A key tile in LDS: rows of DI bytes, unpadded, written by direct
// global -> LDS loads (each 64-lane load fills 1 KB, lane i at byte 16 i).
// Within a row the 16-byte parts are permuted so that the same part of 8
// consecutive keys lands in 8 distinct 16-byte bank groups: the key-operand
// reads (lane c reads key c) are then free of bank conflicts.
template <int DI>
struct TileGeom {
  static constexpr int kParts = DI / 16;                   // 16-byte parts of a row
  static constexpr int kRowsPerLine = 8 / kParts;          // rows per 128 bytes
  static constexpr int kBytes = kTileKeys * DI;            // one stage
  static constexpr int kPerWave = kTileKeys * DI / 1024 / kWaves;  // 1 KB loads per wave
};

template <int DI>
__device__ __forceinline__ int tile_off(int key, int part) {
  using G = TileGeom<DI>;
  return key * DI + 16 * (part ^ ((key / G::kRowsPerLine) & (G::kParts - 1)));
}

// Lane-partial head sum of one 32-key block (this lane's rows, key l % 32).
// Unfolded, the weights of this lane's rows come from LDS (wl holds w[h];
// rows 8*(i/4) + 4*g + i%4 of block mb are four consecutive heads).
template <int MB, bool FOLD>
__device__ __forceinline__ int head_sum(const v16i (&acc)[MB], const int* wl) {
  int s = 0;
  if constexpr (FOLD) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) s = s + max(acc[mb][i], 0) + max(acc[mb][i + 1], 0);
  } else {
    const int g = lane_id() >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v4i w4 = *(const v4i*)(wl + 32 * mb + 8 * i4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) s += __mul24(max(acc[mb][4 * i4 + e], 0), w4[e]);
      }
  }
  return s;
}

template <int MB, int KS>
__device__ __forceinline__ void block_mfma(const v4i (&A)[MB][KS], const v4i (&Bk)[KS], v16i (&acc)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v16i{};
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_i8_32x32x32(A[mb][j], Bk[j], acc[mb]);
}

template <int DI, int KS>
__device__ __forceinline__ void read_b(const char* tile, int nb, v4i (&Bk)[KS]) {
  using G = TileGeom<DI>;
  const int l = lane_id(), g = l >> 5, c = l & 31;
#pragma unroll
  for (int j = 0; j < KS; ++j) Bk[j] = *(const v4i*)(tile + tile_off<DI>(32 * nb + c, g * (G::kParts / 2) + j));
}

// Filtered-output state of a wave: for query pair p (queries 2p, 2p + 1 of
// the wave), lane half g holds query 2p + g's threshold and the byte offset
// of its segment; cnt0 / cnt1 are the two queries' running counts
// (wave-uniform). Stores go through a buffer resource over the segment
// array, so a lane that keeps nothing stores to an offset past its end,
// which the hardware drops: the epilogue has no branch.
struct FiltState {
  int tau[kQW / 2];
  uint32_t segoff[kQW / 2];
  int cnt0[kQW / 2], cnt1[kQW / 2];
};
constexpr uint32_t kDropOffset = 0x80000000u;  // segment arrays are at most 2 GiB

// Keeps this lane's score s of key v (query 2p + g of the wave) when it is
// visible and at least the query's threshold.
__device__ __forceinline__ void filt_put(const ScoreArgs& a, FiltState& fs, int p, int s, int v, bool vis) {
  const int g = lane_id() >> 5;
  const bool keep = vis && s >= fs.tau[p];
  const uint64_t m = __ballot(keep);
  const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
  const int n_lo = __popc(lo);
  // rank among the kept lanes of the whole wave; half 1 discounts half 0's
  const int rank = (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
  const int off = rank + (g ? fs.cnt1[p] - n_lo : fs.cnt0[p]);
  const uint32_t voff = keep && off < a.seg_cap ? fs.segoff[p] + 8u * (uint32_t)off : kDropOffset;
  const __amdgpu_buffer_rsrc_t res =
      uniform_rsrc(a.seg, (uint32_t)((int64_t)a.n_q * a.seg_chunks * a.seg_cap * 8));
  __builtin_amdgcn_raw_buffer_store_b64(v2u{(uint32_t)s, (uint32_t)v}, res, voff, 0, 0);
  fs.cnt0[p] += n_lo;
  fs.cnt1[p] += __popc(hi);
}

// Scores of this wave's queries row0 .. row0+3 against keys [v_begin, v_end).
template <int HI, int DI, bool FOLD, bool FILT>
__device__ __forceinline__ void score_chunk(const ScoreArgs& a, const v4i (&A)[kQW][HI / 32][DI / 32],
                                            const int* wl, const int8_t* kb, char* lds0, char* lds1,
                                            int v_begin, int v_end, int row0, int32_t* sc, FiltState& fs) {
  using G = TileGeom<DI>;
  constexpr int MB = HI / 32, KS = DI / 32;
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int vis_lo_wave = a.mask_off + row0;  // last key visible to every query of the wave
  const bool rows_ok = row0 + kQW <= a.n_q;
  const int ks = a.kstride > 1 ? a.kstride : 1;

  // direct global -> LDS loads of one tile into a stage: load u of wave w
  // fills rows [8 (w * kPerWave + u), +8) (DI = 128) of the stage
  // Buffer loads: lane offsets are fixed (the part permutation of a lane does
  // not depend on the load, every load starting at a multiple of 8 rows), the
  // tile position goes in the scalar offset, and rows past the batch's keys
  // read as zero (range-checked by the buffer; such keys are never stored).
  // (with a key stride, virtual key v is row v * ks: the same LDS layout,
  // each lane's row and the tile position scaled by ks)
  const int wbase = __builtin_amdgcn_readfirstlane(wave_id() * G::kPerWave);
  const int lane_key = l / G::kParts;
  const int lane_off =
      lane_key * ks * DI + 16 * ((l % G::kParts) ^ ((lane_key / G::kRowsPerLine) & (G::kParts - 1)));
  const __amdgpu_buffer_rsrc_t kres =
      __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, (int)((int64_t)a.n_k * DI), 0x00020000);
  auto fetch = [&](int v0, char* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < G::kPerWave; ++u) {
      const int n = wbase + u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (__attribute__((address_space(3))) void*)(stage + n * 1024), 16,
                                               lane_off, (v0 + n * (64 / G::kParts)) * ks * DI, 0, 0);
    }
  };

  // One tile from stage `tile` while the next one loads into `next`. The two
  // stages are separate LDS arrays, and the loop below names each one
  // explicitly, so the compiler can tell the next tile's loads apart from
  // this tile's reads and does not wait for them before reading.
  auto step = [&](int v0, const char* tile, char* next) __attribute__((always_inline)) {
    const bool more = v0 + kTileKeys < v_end;
    if (more) fetch(v0 + kTileKeys, next);
    // per block: each query's MFMAs and epilogue in turn, one 64-lane store
    // per pair of queries; the other wave on the SIMD fills the MFMA pipe
    auto fast_block = [&](int nb) __attribute__((always_inline)) {
      v4i Bk[KS];
      read_b<DI, KS>(tile, nb, Bk);
#pragma unroll
      for (int qp = 0; qp < kQW; qp += 2) {
        // both queries' MFMAs first: the first epilogue then runs while
        // the second query's products finish. The epilogue runs at a
        // raised wave priority: the SIMD's other wave, issuing products,
        // needs an issue slot only once per MFMA, and the VALU work is no
        // longer held back by it (measured: about 3% faster)
        v16i acc0[MB], acc1[MB];
        __builtin_amdgcn_s_setprio(0);
        block_mfma<MB, KS>(A[qp], Bk, acc0);
        block_mfma<MB, KS>(A[qp + 1], Bk, acc1);
        __builtin_amdgcn_s_setprio(2);
        const int s0 = head_sum<MB, FOLD>(acc0, wl);
        const int s1 = head_sum<MB, FOLD>(acc1, wl);
        // lane half g ends with query qp + g's full sum
        if constexpr (FILT)
          filt_put(a, fs, qp / 2, pair_sum32(s0, s1), v0 + 32 * nb + c, true);
        else
          sc[(int64_t)(row0 + qp + g) * a.ld + v0 + 32 * nb + c] = pair_sum32(s0, s1);
      }
    };
    // every key of the tile visible to every query of the wave
    const bool fast = rows_ok && v0 >= a.pos_lo && v0 + kTileKeys <= v_end && v0 + kTileKeys - 1 <= vis_lo_wave;
    if (fast) {
#pragma unroll
      for (int nb = 0; nb < kBlocks; ++nb) fast_block(nb);
    } else {
#pragma unroll 1
      for (int nb = 0; nb < kBlocks; ++nb) {
        const int p0 = v0 + 32 * nb;  // first key of the block
        if (p0 >= v_end) break;
        // a block of the tile that every query of the wave sees whole (the
        // blocks before the diagonal) takes the fast form
        if (rows_ok && p0 >= a.pos_lo && p0 + 32 <= v_end && p0 + 31 <= vis_lo_wave) {
          fast_block(nb);
          continue;
        }
        const int v = p0 + c;
        v4i Bk[KS];
        read_b<DI, KS>(tile, nb, Bk);
#pragma unroll
        for (int qp = 0; qp < kQW; qp += 2) {
          // the two queries of this pair; lane half g stores row0 + qp + g
          const int rowA = row0 + qp, row = rowA + g;
          const bool vis_any = rowA < a.n_q && p0 <= a.mask_off + rowA + 1 && p0 + 31 >= a.pos_lo;
          int full = kMasked;
          if (vis_any) {
            v16i acc[MB];
            block_mfma<MB, KS>(A[qp], Bk, acc);
            const int s0 = head_sum<MB, FOLD>(acc, wl);
            block_mfma<MB, KS>(A[qp + 1], Bk, acc);
            const int s1 = head_sum<MB, FOLD>(acc, wl);
            full = pair_sum32(s0, s1);
          }
          if constexpr (FILT) {
            filt_put(a, fs, qp / 2, full, v, row < a.n_q && v < v_end && v >= a.pos_lo && v <= a.mask_off + row);
          } else if (row < a.n_q && v < v_end) {
            int32_t* dst = sc + (int64_t)row * a.ld + v;
            if (v >= a.pos_lo && v <= a.mask_off + row) *dst = full;
            else if (a.fill_masked) *dst = kMasked;
          }
        }
      }
    }
    // this wave's loads of the next tile have landed; the barrier publishes
    // every wave's and frees the current stage for the tile after
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  fetch(v_begin, lds0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int v0 = v_begin; v0 < v_end; v0 += 2 * kTileKeys) {
    step(v0, lds0, lds1);
    if (v0 + kTileKeys < v_end) step(v0 + kTileKeys, lds1, lds0);
  }
}

// Grid: gridDim.x * gridDim.y = chunks * query tiles, walked chunk-major:
// consecutive workgroups (which the dispatcher deals to the 8 XCDs in turn)
// take consecutive query tiles of one key chunk, so every XCD gets the same
// mix of chunks and the chunk's keys are shared in each XCD's L2.
template <int HI, int DI, bool FILT>
__global__ __launch_bounds__(kThreads, 3) void index_prefill_kernel(ScoreArgs a, int fold_ok, int chunk_keys) {
  using G = TileGeom<DI>;
  constexpr int MB = HI / 32, KS = DI / 32;
  __shared__ __attribute__((aligned(16))) char lds0[G::kBytes];
  __shared__ __attribute__((aligned(16))) char lds1[G::kBytes];
  __shared__ __attribute__((aligned(16))) int wl[HI];
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int n_qt = (a.n_q + kQT - 1) / kQT;
  // query tiles in descending order: under a causal mask the later rows
  // have the most visible keys, and the longest workgroups start first
  const int chunk = lin / n_qt, qt = n_qt - 1 - lin % n_qt, b = blockIdx.z;
  const int q0 = qt * kQT;
  const int v_begin = chunk * chunk_keys;
  const int last_row = min(q0 + kQT, a.n_q) - 1;
  // without masked fill, keys past the last one visible to the workgroup's
  // rows are never stored and are not scored
  const int v_end = min(min(v_begin + chunk_keys, a.n_keys),
                        a.fill_masked ? a.n_keys : a.mask_off + last_row + 1);
  int32_t* sc = a.scores + (int64_t)b * a.s_bstride;
  const int l = lane_id(), g = l >> 5, c = l & 31;

  // only tiles with a flagged row run (a redo of some rows)
  if (a.row_flags != nullptr) {
    const int r = q0 + (int)threadIdx.x;
    const int f = threadIdx.x < kQT && r <= last_row ? a.row_flags[r] : 0;
    if (!__syncthreads_or(f)) return;
  }
  // whole chunk invisible to every row of the workgroup
  if (v_begin > a.mask_off + last_row || v_end <= a.pos_lo) {
    if constexpr (FILT) {
      const int r = q0 + (int)threadIdx.x;
      if (threadIdx.x < kQT && r <= last_row) a.seg_cnt[(int64_t)r * a.seg_chunks + chunk] = 0;
    } else if (a.fill_masked) {
      for (int r = q0; r <= last_row; ++r)
        for (int v = v_begin + threadIdx.x; v < v_end; v += kThreads) sc[(int64_t)r * a.ld + v] = kMasked;
    }
    return;
  }
  if (threadIdx.x < HI) wl[threadIdx.x] = a.w.w[threadIdx.x];
  __syncthreads();

  const int row0 = q0 + kQW * wave_id();
  v4i A[kQW][MB][KS];
  const int8_t* qb = a.q + (int64_t)b * a.q_bstride;
#pragma unroll
  for (int q = 0; q < kQW; ++q) {
    const int qrow = min(row0 + q, a.n_q - 1);  // rows past n_q compute on a valid row, store nothing
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const v4i* src = (const v4i*)(qb + ((int64_t)qrow * HI + 32 * mb + c) * DI + g * (DI / 2));
#pragma unroll
      for (int j = 0; j < KS; ++j) A[q][mb][j] = src[j];
    }
  }
  // fold the weights into A when that is exact for every row of the wave
  bool ok = fold_ok != 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int wh = wl[32 * mb + c];
#pragma unroll
    for (int q = 0; q < kQW; ++q)
#pragma unroll
      for (int j = 0; j < KS; ++j) ok = ok && bytes_scale_fit(A[q][mb][j], wh);
  }
  const bool fold = __all(ok);
  const int8_t* kb = a.k + (int64_t)b * a.k_bstride;
  FiltState fs;
  if constexpr (FILT) {
#pragma unroll
    for (int p = 0; p < kQW / 2; ++p) {
      const int r = min(row0 + 2 * p + g, a.n_q - 1);
      fs.tau[p] = a.tau[r];
      fs.segoff[p] = (uint32_t)(((int64_t)r * a.seg_chunks + chunk) * a.seg_cap * 8);
      fs.cnt0[p] = fs.cnt1[p] = 0;
    }
  }
  if (fold) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int wh = wl[32 * mb + c];
#pragma unroll
      for (int q = 0; q < kQW; ++q)
#pragma unroll
        for (int j = 0; j < KS; ++j) A[q][mb][j] = scale_bytes(A[q][mb][j], wh);
    }
    score_chunk<HI, DI, true, FILT>(a, A, wl, kb, lds0, lds1, v_begin, v_end, row0, sc, fs);
  } else {
    score_chunk<HI, DI, false, FILT>(a, A, wl, kb, lds0, lds1, v_begin, v_end, row0, sc, fs);
  }
  if constexpr (FILT) {
    // lane 0 of each half: the count of its query (rows past n_q store nothing)
#pragma unroll
    for (int p = 0; p < kQW / 2; ++p) {
      const int r = row0 + 2 * p + g;
      if (c == 0 && r < a.n_q) a.seg_cnt[(int64_t)r * a.seg_chunks + chunk] = g ? fs.cnt1[p] : fs.cnt0[p];
    }
  }
}

template <int HI, int DI>
hipError_t launch_t(const ScoreArgs& a, int fold_ok, hipStream_t st) {
  const int64_t n_qt = (a.n_q + kQT - 1) / kQT;
  const int ck = a.chunk_keys > 0 ? a.chunk_keys : index_prefill_auto_chunk(a);
  const int64_t n_chunks = (a.n_keys + ck - 1) / ck;
  if (n_chunks * n_qt > INT32_MAX) return hipErrorInvalidValue;
  if (a.tau != nullptr && (a.B != 1 || a.seg_chunks != n_chunks)) return hipErrorInvalidValue;
  dim3 grid((unsigned)n_chunks, (unsigned)n_qt, a.B);
  KernelTimer kt("index_prefill_kernel", st);
  if (a.tau != nullptr)
    hipLaunchKernelGGL((index_prefill_kernel<HI, DI, true>), grid, dim3(kThreads), 0, st, a, fold_ok, ck);
  else
    hipLaunchKernelGGL((index_prefill_kernel<HI, DI, false>), grid, dim3(kThreads), 0, st, a, fold_ok, ck);
  return hipGetLastError();
}

}  // namespace

// Longer chunks load each query's A operand fewer times; they are taken
// while the grid still fills the chip for several rounds.
int index_prefill_auto_chunk(const ScoreArgs& a) {
  const int64_t n_qt = (a.n_q + kQT - 1) / kQT;
  int ck = kMinChunkKeys;
  while (ck < kMaxChunkKeys && (int64_t)((a.n_keys + 2 * ck - 1) / (2 * ck)) * n_qt * a.B >= kFullGrid) ck *= 2;
  return ck;
}

bool index_prefill_supported(const ScoreArgs& a) {
  return a.blocks == nullptr && a.shift.ctx_len == nullptr && (a.H_I == 32 || a.H_I == 64) &&
         (a.d_I == 64 || a.d_I == 128) && a.n_q >= kQT && (a.chunk_keys <= 0 || a.chunk_keys % kTileKeys == 0) &&
         (int64_t)(a.n_keys - 1) * (a.kstride > 1 ? a.kstride : 1) < a.n_k;
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
