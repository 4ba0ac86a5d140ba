// Sparse attention over gathered keys on bf16 MFMA (gfx950).
//
// Each query row attends only to its selected keys (the top-k keys plus the
// sink tokens: "架构拆解 ① LSA" section of the 1.6T training write-up; the
// LongCat-2.0 release article, section "LongCat 稀疏注意力", for SI / CLI).
// All query heads share one KV head, so a wave computes every head of a query
// (or of a group of decode rows) against one gathered key tile at a time.
//
// Wave tile (32 keys x 32*NB heads), transposed products so that no
// register shuffles are needed between the two GEMMs:
//   S^T = K * Q^T  : A = gathered K rows (lane = key), B = Q^T (lane = head)
//   O^T += V^T * P^T: A = V^T from LDS (lane = dim),   B = P^T (lane = head)
// The S^T accumulator gives lane l the head l%32 and 16 keys; those are
// exactly the keys the P^T operand of the second product needs in that lane,
// so softmax probabilities go from accumulator to operand in place. K and V
// rows of a block are staged row-major in LDS; the V^T operand comes from
// transposing LDS reads. Online softmax runs in fp32 in base 2.
//
// Prefill gives each wave one query row and 64 heads. Decode gives each
// wave 32 heads of one query row so that two waves fit on a SIMD, and the
// waves that read the same index share one gather of each K/V block.
//
// Decode splits the selected list into n_split contiguous parts (the one-GPU
// form of the KV-cache parallel decode of the "③ KVP 解码切分示意" section) and
// merges the (max, sum, output) partials with a fixed-shape binary tree.
#include <math.h>

#include "attn_dev.h"
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {


// ------------------------------------------------------------------ prefill
template <int NB>
__global__ __launch_bounds__(256) void attn_prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_all[4 * kWaveLds];
  const int wv = wave_id();
  const int HB = (a.H + 32 * NB - 1) / (32 * NB);
  // Workgroups go to the 8 XCDs round-robin; remap so that each XCD walks a
  // contiguous range of query rows. Rows that run together on one XCD then
  // share their SI windows and sinks in that XCD's L2.
  // (The grid is a multiple of 8 workgroups; the map is a bijection on it.)
  const int64_t per = gridDim.x / 8, bx = blockIdx.x;
  const int64_t tile = (bx % 8) * per + bx / 8;
  const int64_t gi = tile * 4 + wv;
  if (gi >= (int64_t)a.B * a.L * HB) return;
  const int64_t gq = gi / HB;
  const int hb = (int)(gi % HB);
  const int b = (int)(gq / a.L);
  const int l = lane_id(), g = l >> 5, c = l & 31;
  v8bf Q[NB][8];
  load_q<NB>(a.q + gq * a.H * kD, hb * 32 * NB, a.H, Q);
  AttnState<NB> st;
  attn_init(st);
  const int n = min(max(a.n_sel[gq], 0), a.K_tot);
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const uint16_t* V = a.v + (int64_t)b * a.n_k * kD;
  constexpr int kR = 2;
  const int trips = ((n + 31) / 32 + kR - 1) / kR * kR;
  attn_keys<NB, 1, kR, false>(Q, true, K, V, a.idx + gq * a.K_tot, 0, n, trips, a.n_k, a.sl2, 0, st,
                             lds_all + wv * kWaveLds);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.l[nb] += shfl_xor_f(st.l[nb], 32);  // both key halves

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int h = hb * 32 * NB + 32 * nb + c;
    if (h >= a.H) continue;
    const float inv = st.l[nb] > 0.f ? 1.f / st.l[nb] : 0.f;
    uint16_t* orow = a.o + (gq * a.H + h) * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v16f& O = st.o[mb][nb];
        const uint32_t w0 = pack_bf16x2(O[4 * i4] * inv, O[4 * i4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(O[4 * i4 + 2] * inv, O[4 * i4 + 3] * inv);
        *(v2u*)(orow + 32 * mb + 8 * i4 + 4 * g) = v2u{w0, w1};
      }
    if (a.lse && g == 0)
      a.lse[gq * a.H + h] = st.l[nb] > 0.f ? (st.m[nb] + log2f(st.l[nb])) * 0.69314718055994531f : -INFINITY;
  }
}

// Length of the longest run of consecutive positions that ends a row's list,
// in whole blocks of 32: the largest T = 32 m <= n with
// ids[n - 1] - ids[n - T] == T - 1 (the list is strictly ascending, so the T
// entries are then exactly the positions ids[n - T] .. ids[n - 1]). Lane l
// tests T = 32 (l + 1); the lanes that pass form a prefix. Returns the same
// value in every lane; 0 when no block-long run ends the list.
__device__ __forceinline__ int contiguous_tail(const int32_t* ids, int n) {
  const int T = 32 * (lane_id() + 1);
  bool ok = false;
  if (T <= n) ok = ids[n - T] == ids[n - 1] - (T - 1);
  const uint64_t m = (uint64_t)__ballot(ok);
  return m ? 32 * (64 - __clzll((long long)m)) : 0;
}

// Keys at the consecutive cache positions [u0, u1], 32 per block, gathered
// once by all TW waves of the workgroup into one pair of LDS buffers (the
// rows' SI windows, which overlap almost entirely). A wave attends only to
// the positions [lo, hi] of its own row: the others enter its block as
// invalid keys. trips: steps, a multiple of R covering the range.
template <int TW, int R>
__device__ void attn_keys_range(const v8bf (&Q)[1][8], const uint16_t* K, const uint16_t* V, int u0, int u1,
                                int lo, int hi, int trips, int n_k, float sl2, int gw, AttnState<1>& st,
                                char* lds) {
  static_assert(R % 2 == 0, "block parity selects the LDS buffer");
  const int l = lane_id(), c = l & 31;
  const int G = l >> 4, jj = l & 15;
  const int vt_off = kVOff + (4 * (G >> 1) + (jj >> 2)) * kVRow + (16 * (G & 1) + 4 * (jj & 3)) * 2;
  const __amdgpu_buffer_rsrc_t kr = cache_rsrc(K, n_k), vr = cache_rsrc(V, n_k);
  auto gpos = [&](int bi) {
    const int p = u0 + 32 * bi + c;
    return p <= u1 ? p : -1;
  };
  auto rpos = [&](int bi) {
    const int p = u0 + 32 * bi + c;
    return p >= lo && p <= hi ? p : -1;
  };
  const int nblk = (u1 - u0 + 32) / 32;
  KVStage<TW> stg[R];
#pragma unroll
  for (int j = 0; j < R; ++j) gather_kv<TW>(kr, vr, gpos(j), gw, stg[j]);
  store_kv<TW>(stg[0], lds, gw);
  for (int it = 0; it < trips; it += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int bi = it + u;
      __syncthreads();  // block bi in its buffer for all; the other buffer free
      gather_kv<TW>(kr, vr, gpos(bi + R), gw, stg[u]);
      if (bi < nblk) attn_block<1>(Q, lds + (u & 1) * kBlkLds, rpos(bi), n_k, sl2, vt_off, st);
      store_kv<TW>(stg[(u + 1) % R], lds + ((u + 1) & 1) * kBlkLds, gw);
    }
  }
}

// Prefill with 32 heads per wave (two waves per SIMD): the TW waves of a
// query row (H = 32 * TW) share one gather of each K/V block in LDS, and a
// workgroup of 4 waves takes 4 / TW rows. Barriers run over the whole
// workgroup, so its rows step through max(n_sel) blocks together.
template <int TW>
__global__ __launch_bounds__(256) void attn_prefill_shared(PrefillArgs a) {
  constexpr int RW = 4 / TW;
  __shared__ __attribute__((aligned(16))) char lds_all[RW * 2 * kBlkLds];
  const int wv = wave_id(), gw = wv % TW, sr = wv / TW;
  const int64_t per = gridDim.x / 8, bx = blockIdx.x;
  const int64_t tile = (bx % 8) * per + bx / 8;
  const int64_t rows = (int64_t)a.B * a.L;
  const int64_t gq0 = tile * RW;
  if (gq0 >= rows) return;  // the same for every wave of the workgroup
  const bool active = gq0 + sr < rows;
  const int64_t gq = active ? gq0 + sr : rows - 1;  // a missing row repeats the last, stores nothing
  const int b = (int)(gq / a.L);
  const int l = lane_id(), g = l >> 5, c = l & 31;
  v8bf Q[1][8];
  load_q<1>(a.q + gq * a.H * kD, gw * 32, a.H, Q);
  AttnState<1> st;
  attn_init(st);
  const int n = min(max(a.n_sel[gq], 0), a.K_tot);
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const uint16_t* V = a.v + (int64_t)b * a.n_k * kD;
  constexpr int kR = 2;
  // Two rows of one sequence whose lists both end in long runs of
  // consecutive positions (their SI windows) that nearly coincide: the runs
  // are left out of the per-row pass and attended in a second pass over
  // their union, gathered once for both rows. Every wave derives the same
  // decision from both rows' lists.
  int cut[RW], hi_r[RW], lo_r[RW];
  int u0 = 0, u1 = -1;
  bool share = false;
  if constexpr (RW == 2) {
    const int64_t g1 = min(gq0 + 1, rows - 1);
    bool same_seq = gq0 / a.L == g1 / a.L;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t gr = min(gq0 + r, rows - 1);
      const int nr = min(max(a.n_sel[gr], 0), a.K_tot);
      const int32_t* ids = a.idx + gr * a.K_tot;
      const int T = contiguous_tail(ids, nr);
      cut[r] = nr - T;
      hi_r[r] = T > 0 ? ids[nr - 1] : -1;
      lo_r[r] = hi_r[r] - T + 1;
      share = (r == 0 || share) && T >= 64;
    }
    if (share && same_seq) {
      u0 = min(lo_r[0], lo_r[1]);
      u1 = max(hi_r[0], hi_r[1]);
      share = u1 - u0 + 1 <= max(hi_r[0] - lo_r[0], hi_r[1] - lo_r[1]) + 1 + 32;
    } else {
      share = false;
    }
  }
  int n1 = n, n1max = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int nr = min(max(a.n_sel[min(gq0 + r, rows - 1)], 0), a.K_tot);
    n1max = max(n1max, share ? cut[r] : nr);
  }
  if (share) n1 = cut[sr];
  const int trips = ((n1max + 31) / 32 + kR - 1) / kR * kR;
  attn_keys<1, TW, kR, true>(Q, true, K, V, a.idx + gq * a.K_tot, 0, n1, trips, a.n_k, a.sl2, gw, st,
                             lds_all + sr * 2 * kBlkLds);
  if (share) {
    __syncthreads();  // every wave is done with its row's buffers
    const int trips2 = ((u1 - u0 + 32) / 32 + kR - 1) / kR * kR;
    attn_keys_range<4, kR>(Q, K, V, u0, u1, lo_r[sr], hi_r[sr], trips2, a.n_k, a.sl2, wv, st, lds_all);
  }
  st.l[0] += shfl_xor_f(st.l[0], 32);  // both key halves
  const int h = gw * 32 + c;
  if (!active || h >= a.H) return;
  const float inv = st.l[0] > 0.f ? 1.f / st.l[0] : 0.f;
  uint16_t* orow = a.o + (gq * a.H + h) * kD;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const v16f& O = st.o[mb][0];
      const uint32_t w0 = pack_bf16x2(O[4 * i4] * inv, O[4 * i4 + 1] * inv);
      const uint32_t w1 = pack_bf16x2(O[4 * i4 + 2] * inv, O[4 * i4 + 3] * inv);
      *(v2u*)(orow + 32 * mb + 8 * i4 + 4 * g) = v2u{w0, w1};
    }
  if (a.lse && g == 0)
    a.lse[gq * a.H + h] = st.l[0] > 0.f ? (st.m[0] + log2f(st.l[0])) * 0.69314718055994531f : -INFINITY;
}

constexpr bool kPrefillShared = true;

hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t st) {
  const int NB = a.H <= 32 ? 1 : 2;
  const int HB = (a.H + 32 * NB - 1) / (32 * NB);
  const int64_t groups = (int64_t)a.B * a.L * HB;
  dim3 grid((unsigned)(((groups + 3) / 4 + 7) / 8 * 8));
  KernelTimer kt("attn_prefill_kernel", st);
  if (kPrefillShared && (a.H == 64 || a.H == 128)) {
    const int TW = a.H / 32, RW = 4 / TW;
    const int64_t wgs = ((int64_t)a.B * a.L + RW - 1) / RW;
    const dim3 g2((unsigned)((wgs + 7) / 8 * 8));
    if (TW == 2) hipLaunchKernelGGL(attn_prefill_shared<2>, g2, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(attn_prefill_shared<4>, g2, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (NB == 1) hipLaunchKernelGGL(attn_prefill_kernel<1>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_prefill_kernel<2>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int TW, int KS>
__global__ __launch_bounds__(64 * TW * KS) void attn_decode_partial(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_all[DecodeCfg<TW, KS>::kBytes];
  int bx = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
  const int nx = gridDim.x, ny = gridDim.y;
  const int64_t total = (int64_t)nx * ny * gridDim.z;
  if (nx == 2 && total % 16 == 0) {
    // workgroups go to the 8 XCDs in turn: the two workgroups of a part
    // (which gather the same blocks) take consecutive slots of one XCD, so
    // the second finds the blocks in that XCD's L2
    const int64_t id = blockIdx.x + (int64_t)nx * (blockIdx.y + (int64_t)ny * blockIdx.z);
    const int64_t j = (id % 8) * (total / 8) + id / 8;
    bx = (int)(j % 2);
    split = (int)((j / 2) % ny);
    b = (int)(j / 2 / ny);
  }
  decode_partial_body<TW, KS>(a, bx, split, b, lds_all);
}

// One row per 16 threads, 8 output dims per thread.
template <int NS>
__global__ __launch_bounds__(256) void attn_decode_merge(DecodeArgs a) {
  const int64_t brow = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (brow >= (int64_t)a.B * a.n_q * a.H) return;
  decode_merge_row<NS>(a, brow, 8 * (threadIdx.x & 15));
}


size_t decode_ws_bytes(int B, int n_q, int H, int n_split) {
  const size_t rows = (size_t)B * n_split * n_q * H;
  return rows * (2 * sizeof(float) + kD * sizeof(uint16_t)) + 256;
}

template <int TW, int KS>
static void launch_partial_tk(const DecodeArgs& a, int T, hipStream_t st) {
  dim3 grid((T + TW - 1) / TW, a.n_split, a.B);
  KernelTimer kt("attn_decode_partial", st);
  hipLaunchKernelGGL((attn_decode_partial<TW, KS>), grid, dim3(64 * TW * KS), 0, st, a);
}

static hipError_t launch_partial(const DecodeArgs& a, hipStream_t st) {
  const int HB = (a.H + 31) / 32;
  const int T = a.n_q * HB;
  // waves sharing K/V must read the same index row: with one index per
  // query row, a workgroup stays within the head groups of one row
  const int TW = a.n_idx == 1 ? (T >= 4 ? 4 : T >= 2 ? 2 : 1) : HB;
  // subranges per part: 8 waves per workgroup (4 when one row group, to stay
  // within LDS); with eight or more head groups, workgroups of four waves
  // (one per SIMD) without subranges
  switch (TW) {
    case 8: launch_partial_tk<8, 1>(a, T, st); break;
    case 4:
      if (T >= 8) launch_partial_tk<4, 1>(a, T, st);
      else launch_partial_tk<4, 2>(a, T, st);
      break;
    case 2: launch_partial_tk<2, 4>(a, T, st); break;
    default: launch_partial_tk<1, 4>(a, T, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t st) {
  hipError_t e = launch_partial(a, st);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(((int64_t)a.B * a.n_q * a.H + 15) / 16));
  KernelTimer kt("attn_decode_merge", st);
  if (a.n_split <= 1) hipLaunchKernelGGL(attn_decode_merge<1>, grid, dim3(256), 0, st, a);
  else if (a.n_split <= 2) hipLaunchKernelGGL(attn_decode_merge<2>, grid, dim3(256), 0, st, a);
  else if (a.n_split <= 4) hipLaunchKernelGGL(attn_decode_merge<4>, grid, dim3(256), 0, st, a);
  else if (a.n_split <= 8) hipLaunchKernelGGL(attn_decode_merge<8>, grid, dim3(256), 0, st, a);
  else if (a.n_split <= 16) hipLaunchKernelGGL(attn_decode_merge<16>, grid, dim3(256), 0, st, a);
  else if (a.n_split <= 32) hipLaunchKernelGGL(attn_decode_merge<32>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_decode_merge<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
