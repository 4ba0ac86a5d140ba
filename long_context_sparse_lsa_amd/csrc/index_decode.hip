// Indexer scoring for a few query rows per sequence (decode and the two HI
// stages) on int8 MFMA (gfx950).
//
// S[t, s] = sum_h w[h] * max(0, q_I[t, h, :] . k_I[s, :]), exact in int32
// (LongCat-2.0 release article, section "LongCat 稀疏注意力"; the arithmetic
// is fixed by this library as int8 q/k, integer head weights, int32 result).
//
// With one query row per sequence the scan reads every key once and does
// little arithmetic per byte, so it is bound by HBM streaming. Each wave owns
// a long contiguous key range, loads its query rows (the MFMA A operand) once,
// and streams 32-key tiles straight into registers through a ring of DEPTH
// tiles: the loads of tile t + DEPTH are issued as soon as tile t has gone
// through the MFMAs, so DEPTH tiles are in flight per wave at all times.
// Long scans use a ring of 4 (a deeper or shallower ring, or twice the
// waves, was no faster at C3); launches whose waves get at most four tiles
// each (the HI stages) use a ring of 2 and twice the waves, which shortens
// their latency-bound run (C4: -2 us per launch).
// No load is conditional: keys past the range re-read the range's last key,
// which only touches lines already in cache. In the HI fine stage (keys
// addressed through a block table) the wave first copies its slice of the
// table to LDS, so key addresses never wait on a global load.
//
// Layout of the 32x32x32 int8 MFMA: lane l supplies row / key l % 32 and
// half l / 32 of the d_I bytes (A and B use the same byte-to-slot map, so
// the product is exact); the accumulator gives lane l key column l % 32 and
// rows 8 * (i / 4) + 4 * (l / 32) + i % 4 of register i. A query owns H_I
// consecutive rows, so its head sum is a per-lane sum plus one exchange
// between lane halves. Weights are folded into A when that is exact (every
// weight >= 0 and every product w[h] * q fits int8, checked per wave), else
// applied in the epilogue from LDS; both give the same integers.
#include <algorithm>

#include "lsa_device.h"
#include "lsa_internal.h"

#include "score_dev.h"

namespace lsa {

namespace {

template <int HI, int DI, int DEPTH>
__global__ __launch_bounds__(64 * kWaves) void index_decode_kernel(ScoreArgs a, int kpw, int fold_ok) {
  __shared__ __attribute__((aligned(16))) int wl[128];
  __shared__ int bl[kWaves * kMaxBlkIds];
  for (int h = threadIdx.x; h < 128; h += 64 * kWaves) wl[h] = h < HI ? a.w.w[h] : 0;
  __syncthreads();
  decode_score_body<HI, DI, DEPTH>(a, kpw, fold_ok, blockIdx.x, blockIdx.y, blockIdx.z, wave_id(), wl, bl);
}

template <int HI, int DI>
hipError_t launch_t(const ScoreArgs& a, hipStream_t st) {
  constexpr int MB = HI >= 64 ? HI / 32 : 2;
  constexpr int NQ = 32 * MB / HI;
  const int qtiles = (a.n_q + NQ - 1) / NQ;
  // one wave per wave slot of the GPU (256 CUs x 2 waves per SIMD x 4), so
  // that every wave streams from start to end without a second round; each
  // wave takes a multiple of 32 * DEPTH keys
  const int64_t total = (int64_t)a.B * qtiles * a.n_keys;
  int64_t kpw = (total + 2047) / 2048;
  const bool short_scan = kpw <= 32 * kDepthLong;
  const int depth = short_scan ? kDepthShort : kDepthLong;
  kpw = (kpw + 32 * depth - 1) / (32 * depth) * (32 * depth);
  kpw = std::min<int64_t>(std::max<int64_t>(kpw, 32 * depth), kMaxKeysPerWave);
  const int64_t per_wg = kpw * kWaves;
  dim3 grid((unsigned)qtiles, (unsigned)((a.n_keys + per_wg - 1) / per_wg), (unsigned)a.B);
  int fold_ok = 1;
  for (int h = 0; h < a.H_I; ++h) fold_ok &= a.w.w[h] >= 0;
  KernelTimer kt("index_decode_kernel", st);
  if (short_scan)
    hipLaunchKernelGGL((index_decode_kernel<HI, DI, kDepthShort>), grid, dim3(64 * kWaves), 0, st, a, (int)kpw,
                       fold_ok);
  else
    hipLaunchKernelGGL((index_decode_kernel<HI, DI, kDepthLong>), grid, dim3(64 * kWaves), 0, st, a, (int)kpw,
                       fold_ok);
  return hipGetLastError();
}

}  // namespace

bool index_decode_supported(const ScoreArgs& a) {
  // a wave's keys span at most kMaxKeysPerWave / blk + 2 table entries
  const bool table_ok = a.blocks == nullptr || (a.blk >= 32 && kMaxKeysPerWave / a.blk + 2 <= kMaxBlkIds);
  return (a.H_I == 32 || a.H_I == 64 || a.H_I == 128) && (a.d_I == 64 || a.d_I == 128) && table_ok;
}

hipError_t launch_index_decode(const ScoreArgs& a, hipStream_t st) {
#define LSA_CASE(h, d) \
  if (a.H_I == h && a.d_I == d) return launch_t<h, d>(a, st);
  LSA_CASE(32, 64) LSA_CASE(32, 128) LSA_CASE(64, 64) LSA_CASE(64, 128) LSA_CASE(128, 64) LSA_CASE(128, 128)
#undef LSA_CASE
  return hipErrorInvalidValue;
}

}  // namespace lsa
