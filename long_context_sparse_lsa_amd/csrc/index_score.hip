// Indexer scoring on int8 MFMA (gfx950).
//
// S[t, s] = sum_h w[h] * max(0, q_I[t, h, :] . k_I[s, :]), exact in int32.
// (LongCat-2.0 release article, section "LongCat 稀疏注意力": a lightweight
// indexer scores the keys for each query; its arithmetic is fixed by this
// library as int8 q/k, integer head weights and an int32 result.)
//
// GEMM view: M = (query, head) rows, N = keys, K = d_I. A wave owns a tile of
// R = 32*MB rows (MB >= 2 M-blocks of 32) and walks 32-key tiles. Each lane
// keeps its query rows in registers (A operand) for the whole kernel and loads
// the key tile straight from memory: lane l takes key l%32 and one half of
// its d_I bytes (lanes 0-31 the first half, 32-63 the second). A and B are
// loaded with the same byte-to-contraction-slot assignment, so the product
// is exact whatever slot order the hardware uses internally.
//
// Epilogue: the 32x32 accumulator gives lane l the column (key) l%32 and rows
// 8*(i/4) + 4*(l/32) + i%4 of each M-block; queries own H_I consecutive rows,
// so the head sum is a per-lane sum over whole groups of 4 registers plus, for
// H_I >= 8, one exchange with lane l^32. ReLU and the weight are max + 24-bit
// multiply-add (|dot| <= 2^21 and |w| < 2^11 under the range check).
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

template <int HI, int DI>
__global__ __launch_bounds__(256) void index_score_kernel(ScoreArgs a, int QT, int KC) {
  constexpr int MB = HI > 64 ? HI / 32 : 2;
  constexpr int R = 32 * MB;
  constexpr int KS = DI / 32;
  constexpr int NQ = R / HI;
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int wv = wave_id();
  const int KT = 4 / QT;
  const int tile = blockIdx.x * QT + (wv % QT);
  const int ksub = wv / QT;
  const int b = blockIdx.z;
  const int q0 = tile * NQ;
  if (q0 >= a.n_q) return;
  const int nq_tile = min(NQ, a.n_q - q0);
  const int sub = KC / KT;
  const int v_begin = blockIdx.y * KC + ksub * sub;
  const int v_end = min(v_begin + sub, a.n_keys);
  if (v_begin >= v_end) return;

  int32_t* sc = a.scores + (int64_t)b * a.s_bstride;
  const bool direct = a.blocks == nullptr;
  const int mask_off = a.mask_off + seq_shift(a.shift, b);
  const int vis_hi = mask_off + q0 + nq_tile - 1;
  if (direct && (v_begin > vis_hi || v_end <= a.pos_lo)) {
    // nothing visible in this range for any row of the tile
    if (a.fill_masked) {
      for (int qi = 0; qi < nq_tile; ++qi)
        for (int v = v_begin + l; v < v_end; v += 64) sc[(int64_t)(q0 + qi) * a.ld + v] = kMasked;
    }
    return;
  }

  // A operand: MB M-blocks x KS k-steps of 16 bytes.
  v4i A[MB][KS];
  const int8_t* qb = a.q + (int64_t)b * a.q_bstride;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = 32 * mb + c;
    const int qi = r / HI, h = r % HI;
    const int gq = q0 + qi;
    const v4i* src = (const v4i*)(qb + ((int64_t)gq * HI + h) * DI + g * (DI / 2));
#pragma unroll
    for (int j = 0; j < KS; ++j) A[mb][j] = (gq < a.n_q) ? src[j] : v4i{0, 0, 0, 0};
  }
  // Per-register head weights of this lane.
  int W[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) W[mb][i] = a.w.w[(32 * mb + 8 * (i / 4) + 4 * g + (i % 4)) % HI];

  const int8_t* kb = a.k + (int64_t)b * a.k_bstride;
  const int32_t* blk_row = direct ? nullptr : a.blocks + (int64_t)b * a.nbr;

  auto key_pos = [&](int v) -> int {
    if (direct) return v;
    const int bi = blk_row[v / a.blk];
    return bi < 0 ? -1 : bi * a.blk + v % a.blk;
  };
  auto load_b = [&](int v, v4i* Bt) {
    const int p = (v < v_end) ? key_pos(v) : -1;
    if (p >= 0 && p < a.n_k) {
      const v4i* src = (const v4i*)(kb + (int64_t)p * DI + g * (DI / 2));
#pragma unroll
      for (int j = 0; j < KS; ++j) Bt[j] = src[j];
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) Bt[j] = v4i{0, 0, 0, 0};
    }
    return p;
  };

  v4i Bc[KS], Bn[KS];
  int pc = load_b(v_begin + c, Bc);
  for (int s0 = v_begin; s0 < v_end; s0 += 32) {
    const int v = s0 + c;
    const int pn = (s0 + 32 < v_end) ? load_b(s0 + 32 + c, Bn) : -1;
    v16i acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = v16i{};
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_i8_32x32x32(A[mb][j], Bc[j], acc[mb]);

    int part[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        int s = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) s += __mul24(max(acc[mb][4 * i4 + e], 0), W[mb][4 * i4 + e]);
        part[mb][i4] = s;
      }

    auto store = [&](int qi, int val) {
      const int gq = q0 + qi;
      if (gq >= a.n_q || v >= v_end) return;
      const bool vis = pc >= a.pos_lo && pc <= mask_off + gq;
      if (vis) sc[(int64_t)gq * a.ld + v] = val;
      else if (a.fill_masked) sc[(int64_t)gq * a.ld + v] = kMasked;
    };
    if constexpr (HI == 4) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) store(8 * mb + 2 * i4 + g, part[mb][i4]);
    } else {
      constexpr int SPQ = HI / 8;
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        int s = 0;
#pragma unroll
        for (int e = 0; e < SPQ; ++e) {
          const int slot = qi * SPQ + e;
          s += part[slot / 4][slot % 4];
        }
        s += shfl_xor_i(s, 32);
        if ((NQ == 1 && g == 0) || (NQ > 1 && (qi & 1) == g)) store(qi, s);
      }
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) Bc[j] = Bn[j];
    pc = pn;
  }
}

template <int HI, int DI>
static hipError_t launch_t(const ScoreArgs& a, hipStream_t st) {
  constexpr int MB = HI > 64 ? HI / 32 : 2;
  constexpr int NQ = 32 * MB / HI;
  const int n_tiles = (a.n_q + NQ - 1) / NQ;
  const int QT = n_tiles >= 16 ? 4 : 1;
  const int KC = QT == 4 ? 256 : 512;
  dim3 grid((n_tiles + QT - 1) / QT, (a.n_keys + KC - 1) / KC, a.B);
  KernelTimer kt("index_score_kernel", st);
  hipLaunchKernelGGL((index_score_kernel<HI, DI>), grid, dim3(256), 0, st, a, QT, KC);
  return hipGetLastError();
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t st) {
  if (index_prefill_supported(a)) return launch_index_prefill(a, st);
  // key strides, row flags and filtered output exist only in the many-row variant
  if (a.kstride > 1 || a.row_flags != nullptr || a.tau != nullptr || a.chunk_keys > 0) return hipErrorInvalidValue;
  if (index_decode_supported(a)) return launch_index_decode(a, st);
#define LSA_CASE(h, d) \
  if (a.H_I == h && a.d_I == d) return launch_t<h, d>(a, st);
  LSA_CASE(4, 64) LSA_CASE(4, 128) LSA_CASE(8, 64) LSA_CASE(8, 128)
  LSA_CASE(16, 64) LSA_CASE(16, 128) LSA_CASE(32, 64) LSA_CASE(32, 128)
  LSA_CASE(64, 64) LSA_CASE(64, 128) LSA_CASE(128, 64) LSA_CASE(128, 128)
#undef LSA_CASE
  return hipErrorInvalidValue;
}

}  // namespace lsa
