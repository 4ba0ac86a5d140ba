// Sparse attention backward on bf16 MFMA (gfx950), deterministic.
//
// Training pairs the LSA operator with deterministic attention operators
// ("如何在 5 万张国产芯片训练出 1.6T 万亿参数模型？", section "④ 痛点③：长上下文训练三招";
// the LongCat-2.0 release article, section "长上下文训练"); the haoling.cc
// article (section 三) describes a deterministic attention backward that had
// serialised its accumulation, and scatter operators redesigned as
// deterministic parallel algorithms. Here the scatter of the key gradients is
// made order-independent instead of ordered.
//
// Row-major, as the forward: a wave takes 32 heads of one query row, the TW =
// H / 32 waves of the row share one LDS gather of each 32-key K/V block, and
// the row's selected keys are walked 32 at a time. Per block, with the
// probabilities recomputed from the forward's log-sum-exp:
//   S^T  = K . Q^T              A = K rows from LDS, B = Q^T in registers
//   dP^T = V . dO^T             A = V rows from LDS, B = dO^T in registers
//   P^T  = 2^(S^T sl2 - lse2), dS^T = P^T (dP^T - Delta)      (lane = head)
//   dQ^T += K^T . dS^T          A = K^T by transposed LDS reads, B = dS^T in place
// with Delta = sum_d dO . o per head; dQ stays in registers for the whole
// row. The row's waves then put P^T and dS^T into one LDS tile of all H heads
// and wave gw takes the dims [128 gw / TW, 128 (gw + 1) / TW) over every head:
//   dV = P . dO,  dK = dS . Q (x scale)   A = P / dS by transposed tile reads
// so each (row, key) pair's contribution to dk and dv comes out complete
// (256 values) and is stored once, in bf16, through an LDS transpose that
// makes the stores 128-byte rows.
//
// The scatter of those contributions to the keys is made order-independent
// rather than ordered: the pairs of each key are listed (integer counts, an
// exclusive scan, a fill whose order does not matter), and each key's
// contributions are summed as int64 fixed point (value * 2^32, exact for
// bf16 values at or above 2^-24 in magnitude). Integer sums do not depend on
// the order of their terms, so the totals, and the fp32 gradients converted
// from them, are bit-identical from run to run, with no float atomics. Rows
// are processed in chunks so that the contribution buffer stays bounded.
#include <math.h>

#include <algorithm>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int kD = 128;
// LDS bytes per K or V row: 76 dwords, so that both the 16-byte row reads
// (row c at 76c dwords: 16 distinct bank groups over 16 rows) and the 8-byte
// transposed reads (4 rows 12 banks apart) are free of bank conflicts
constexpr int kRowB = 304;
constexpr int kBlkB = 32 * kRowB;  // 32 rows of K (or V)
// LDS bytes per head row of a 32 x 32 bf16 P^T / dS^T tile (24 dwords)
constexpr int kTileP = 96;
constexpr int kTileB = 32 * kTileP;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v8bf ld8(const uint16_t* p) { return *(const v8bf*)p; }

// round-half-even(x * 2^32) as an int64 (|x| < 2^31): x * 2^32 and its
// rounding are exact in fp64; the high word is floor(y / 2^32) and the low
// word y - high * 2^32, an integer in [0, 2^32).
__device__ __forceinline__ uint64_t to_fixed32(float x) {
  const double y = __builtin_rint((double)x * 4294967296.0);
  const double hi = __builtin_floor(y * (1.0 / 4294967296.0));
  const double lo = __builtin_fma(hi, -4294967296.0, y);
  return ((uint64_t)(uint32_t)(int32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

// K and V rows of one 32-key block staged in registers: thread gt = 64 * gw +
// lane of the row's TW waves loads, for i < 8 / TW, the 16 bytes at 16 * (lane
// % 16) of the rows of key 4 * gw + lane / 16 + 4 * TW * i. Buffer loads over
// the sequence's cache: a position outside [0, n_k) reads zeros (and its
// probability is set to 0 before use).
template <int TW>
struct Stage {
  v4u k[8 / TW], v[8 / TW];
};

template <int TW>
__device__ __forceinline__ void gather(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int pos, int gw,
                                       Stage<TW>& s) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8 / TW; ++i) {
    const int pe = __shfl(pos, 4 * gw + (l >> 4) + 4 * TW * i, 64);
    const uint32_t off = (uint32_t)pe * (uint32_t)(kD * 2) + 16u * (uint32_t)(l & 15);
    s.k[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)off, 0, 0));
    s.v[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(vr, (int)off, 0, 0));
  }
}

template <int TW>
__device__ __forceinline__ void store(const Stage<TW>& s, char* kb, char* vb, int gw) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8 / TW; ++i) {
    const int key = 4 * gw + (l >> 4) + 4 * TW * i;
    *(v4u*)(kb + key * kRowB + 16 * (l & 15)) = s.k[i];
    *(v4u*)(vb + key * kRowB + 16 * (l & 15)) = s.v[i];
  }
}

// Per-row operands of one wave (heads h0 .. h0 + 31 of the row for S^T, dP^T
// and dQ; every head, over the wave's dims d0 .. d0 + 128/TW - 1, for dK, dV).
template <int TW>
struct RowOps {
  static constexpr int NT = 4 / TW;  // 32-dim tiles of the wave's dims
  static constexpr int KS = 2 * TW;  // 16-head steps over all H = 32 TW heads
  v8bf Qb[8], dOb[8];          // lane (g, c): head h0 + c, dims 64g + 8j + {0..7}
  v8bf Qt[NT][KS], dOt[NT][KS];  // lane (g, c): dim d0 + 32nt + c, heads 16ks + 4g + {0..3, 8..11}
  float dlt, lse2;             // Delta and lse * log2(e) of head h0 + c
};

template <int TW>
__device__ __forceinline__ void load_row_ops(const BwdArgs& a, int64_t gq, int h0, int d0, RowOps<TW>& r) {
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const uint16_t* qr = a.q + gq * a.H * kD;
  const uint16_t* dr = a.d_o + gq * a.H * kD;
  const uint16_t* orw = a.o + gq * a.H * kD;
  float dl = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int off = (h0 + c) * kD + 64 * g + 8 * j;
    r.Qb[j] = ld8(qr + off);
    r.dOb[j] = ld8(dr + off);
    const v8bf ov = ld8(orw + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) dl = fmaf((float)r.dOb[j][e], (float)ov[e], dl);
  }
  r.dlt = dl + shfl_xor_f(dl, 32);
#pragma unroll
  for (int nt = 0; nt < RowOps<TW>::NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < RowOps<TW>::KS; ++ks) {
      v8bf x, y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int h = 16 * ks + 4 * g + (e & 3) + 8 * (e >> 2);
        x[e] = __builtin_bit_cast(__bf16, qr[h * kD + d0 + 32 * nt + c]);
        y[e] = __builtin_bit_cast(__bf16, dr[h * kD + d0 + 32 * nt + c]);
      }
      r.Qt[nt][ks] = x;
      r.dOt[nt][ks] = y;
    }
  r.lse2 = a.lse[gq * a.H + h0 + c] * kLog2e;
}

// Part one of a 32-key block: lane c (and c + 32) holds the position of key
// c. dQ is updated; P^T and dS^T of the wave's heads go to the row's tiles.
template <int TW>
__device__ __forceinline__ void bwd_block_rows(const BwdArgs& a, const RowOps<TW>& r, const char* kb,
                                               const char* vb, char* ptile, char* stile, int h0, int pos,
                                               v16f (&dQ)[4]) {
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const bool valid = (unsigned)pos < (unsigned)a.n_k;
  const uint32_t vmask = (uint32_t)__ballot(valid);
  v16f S = v16f{}, dP = v16f{};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const v8bf ka = *(const v8bf*)(kb + c * kRowB + g * 128 + 16 * j);
    const v8bf va = *(const v8bf*)(vb + c * kRowB + g * 128 + 16 * j);
    S = mfma_bf16_32x32x16(ka, r.Qb[j], S);
    dP = mfma_bf16_32x32x16(va, r.dOb[j], dP);
  }
  // lane (g, c): head h0 + c; entry i is key 8(i/4) + 4g + i%4
  v8bf Pb[2], Sb[2];
#pragma unroll
  for (int js = 0; js < 2; ++js)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * js + e;
      const int kt = 8 * (i >> 2) + 4 * g + (i & 3);
      const float p = ((vmask >> kt) & 1u) ? __builtin_amdgcn_exp2f(fmaf(S[i], a.sl2, -r.lse2)) : 0.f;
      Pb[js][e] = (__bf16)p;
      Sb[js][e] = (__bf16)(p * (dP[i] - r.dlt));
    }
  // dQ^T += K^T . dS^T
  const int kt_off = tr_lane_off(kRowB);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int js = 0; js < 2; ++js)
      dQ[mb] = mfma_bf16_32x32x16(read_tr(kb + kt_off + 16 * js * kRowB + 64 * mb, kRowB), Sb[js], dQ[mb]);
  // tile rows h0 + c (head), 8-byte runs of keys 16js + 4g + {0..3} and
  // 16js + 8 + 4g + {0..3}
#pragma unroll
  for (int js = 0; js < 2; ++js) {
    const v4u pu = __builtin_bit_cast(v4u, Pb[js]), su = __builtin_bit_cast(v4u, Sb[js]);
    char* pp = ptile + (h0 + c) * kTileP + (16 * js + 4 * g) * 2;
    char* sp = stile + (h0 + c) * kTileP + (16 * js + 4 * g) * 2;
    *(v2u*)pp = v2u{pu[0], pu[1]};
    *(v2u*)(pp + 16) = v2u{pu[2], pu[3]};
    *(v2u*)sp = v2u{su[0], su[1]};
    *(v2u*)(sp + 16) = v2u{su[2], su[3]};
  }
}

// Part two, once every wave of the row has written its tile rows: the
// block's dk and dv contributions over all heads for the wave's dims,
// through the wave's transpose buffer xb ([32 keys][128 / TW dims] bf16) to
// 16-byte stores of contrib rows cb + key (keys >= cnt are not stored).
template <int TW>
__device__ __forceinline__ void bwd_block_keys(const BwdArgs& a, const RowOps<TW>& r, const char* ptile,
                                               const char* stile, char* xb, int d0, uint16_t* cb, int cnt) {
  constexpr int NT = RowOps<TW>::NT, KS = RowOps<TW>::KS, ND = 128 / TW;
  constexpr int XP = 2 * ND + 16;  // transpose buffer pitch (bytes)
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int t_off = tr_lane_off(kTileP);
#pragma unroll
  for (int which = 0; which < 2; ++which) {  // 0: dk (dS . Q x scale), 1: dv (P . dO)
    const char* tile = which == 0 ? stile : ptile;
    v8bf A[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) A[ks] = read_tr(tile + t_off + 16 * ks * kTileP, kTileP);
    const float mul = which == 0 ? a.scale : 1.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      v16f acc = v16f{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = mfma_bf16_32x32x16(A[ks], which == 0 ? r.Qt[nt][ks] : r.dOt[nt][ks], acc);
      // lane (g, c): dim 32nt + c of the wave's dims, entry i key 8(i/4) + 4g + i%4
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *(__bf16*)(xb + (8 * (i >> 2) + 4 * g + (i & 3)) * XP + 2 * (32 * nt + c)) = (__bf16)(acc[i] * mul);
    }
    // 32 keys x ND dims back as 16-byte pieces: piece q is key q / (ND / 8),
    // dims 8 (q % (ND / 8)) .. + 7
#pragma unroll
    for (int u = 0; u < ND / 16; ++u) {
      const int q = 64 * u + l;
      const int key = q / (ND / 8), part = q % (ND / 8);
      const v4u x = *(const v4u*)(xb + key * XP + 16 * part);
      if (key < cnt) *(v4u*)(cb + (int64_t)key * 256 + 128 * which + d0 + 8 * part) = x;
    }
  }
}

template <int TW>
__global__ __launch_bounds__(256) void attn_bwd_kernel(BwdArgs a) {
  constexpr int RW = 4 / TW;  // query rows per workgroup
  constexpr int H = 32 * TW;
  constexpr int XB = 32 * (2 * (128 / TW) + 16);  // one wave's transpose buffer
  __shared__ __attribute__((aligned(16))) char lds_kv[RW * 2 * kBlkB];
  __shared__ __attribute__((aligned(16))) char lds_t[RW * 2 * H * kTileP];
  __shared__ __attribute__((aligned(16))) char lds_x[4 * XB];
  const int wv = wave_id(), gw = wv % TW, sr = wv / TW;
  // each XCD walks a contiguous range of the chunk's rows (the grid is a
  // multiple of 8)
  const int64_t per = gridDim.x / 8, bx = blockIdx.x;
  const int64_t tile = (bx % 8) * per + bx / 8;
  const int64_t gq0 = a.r0 + tile * RW;
  if (gq0 >= a.r1) return;  // the same for every wave of the workgroup
  const bool active = gq0 + sr < a.r1;
  const int64_t gq = active ? gq0 + sr : a.r1 - 1;
  const int b = (int)(gq / a.L);
  const int c = lane_id() & 31;
  const int h0 = gw * 32, d0 = gw * (128 / TW);
  int nmax = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r)
    if (gq0 + r < a.r1) nmax = max(nmax, min(max(a.n_sel[gq0 + r], 0), a.K_tot));
  const int n = active ? min(max(a.n_sel[gq], 0), a.K_tot) : 0;
  RowOps<TW> ro;
  load_row_ops<TW>(a, gq, h0, d0, ro);
  const int32_t* ids = a.idx + gq * a.K_tot;
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const uint16_t* V = a.v + (int64_t)b * a.n_k * kD;
  const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(K, (uint32_t)a.n_k * (uint32_t)(kD * 2));
  const __amdgpu_buffer_rsrc_t vr = uniform_rsrc(V, (uint32_t)a.n_k * (uint32_t)(kD * 2));
  char* kb = lds_kv + sr * 2 * kBlkB;
  char* vb = kb + kBlkB;
  char* ptile = lds_t + sr * 2 * H * kTileP;
  char* stile = ptile + H * kTileP;
  char* xb = lds_x + wv * XB;
  uint16_t* crow = a.contrib + (gq - a.r0) * a.K_tot * 256;
  v16f dQ[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) dQ[mb] = v16f{};
  const int nblk = (nmax + 31) / 32;
  int pos = c < n ? ids[c] : -1;
  Stage<TW> stg;
  gather<TW>(kr, vr, pos, gw, stg);
  for (int bi = 0; bi < nblk; ++bi) {
    __syncthreads();  // the previous block's K / V rows and tiles are no longer read
    store<TW>(stg, kb, vb, gw);
    const int pcur = pos;
    const int s1 = 32 * (bi + 1) + c;
    pos = s1 < n ? ids[s1] : -1;
    gather<TW>(kr, vr, pos, gw, stg);  // the next block's rows load during this one
    __syncthreads();
    const bool live = 32 * bi < n;  // the same for the TW waves of the row
    if (live) bwd_block_rows<TW>(a, ro, kb, vb, ptile, stile, h0, pcur, dQ);
    __syncthreads();  // the row's tiles are complete
    if (live) bwd_block_keys<TW>(a, ro, ptile, stile, xb, d0, crow + (int64_t)32 * bi * 256, min(32, n - 32 * bi));
  }
  if (!active) return;
  const int g = lane_id() >> 5;
  uint16_t* dqrow = a.dq + (gq * a.H + h0 + c) * kD;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const v16f& D = dQ[mb];
      const uint32_t w0 = pack_bf16x2(D[4 * i4] * a.scale, D[4 * i4 + 1] * a.scale);
      const uint32_t w1 = pack_bf16x2(D[4 * i4 + 2] * a.scale, D[4 * i4 + 3] * a.scale);
      *(v2u*)(dqrow + 32 * mb + 8 * i4 + 4 * g) = v2u{w0, w1};
    }
}

// ---------------------------------------------------------------- scatter
// Pairs of the chunk: p = (row - r0) * K_tot + slot, for slots below the
// row's n_sel holding a position in [0, n_k); key = b * n_k + position.
__device__ __forceinline__ int pair_key(const ScatterArgs& a, int64_t p) {
  const int64_t t = a.r0 + p / a.K_tot;
  const int j = (int)(p % a.K_tot);
  const int n = min(max(a.n_sel[t], 0), a.K_tot);
  if (j >= n) return -1;
  const int s = a.idx[t * a.K_tot + j];
  if ((unsigned)s >= (unsigned)a.n_k) return -1;
  return (int)(t / a.L) * a.n_k + s;
}

__global__ __launch_bounds__(256) void bwd_count_kernel(ScatterArgs a) {
  const int64_t np = (a.r1 - a.r0) * a.K_tot;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < np; p += (int64_t)gridDim.x * 256) {
    const int key = pair_key(a, p);
    if (key >= 0) atomicAdd(&a.cnt[key], 1);
  }
}

// Exclusive scan of cnt into cur, in blocks of kScanBlock (1024 threads x 4);
// tot gets each block's sum.
__global__ __launch_bounds__(1024) void bwd_scan_blocks_kernel(ScatterArgs a) {
  __shared__ int32_t wsum[16];
  const int base = blockIdx.x * kScanBlock + threadIdx.x * 4;
  int v[4], s = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = base + e < a.n_keys ? a.cnt[base + e] : 0;
    s += v[e];
  }
  const int incl = wave_incl_scan(s);
  if (lane_id() == 63) wsum[wave_id()] = incl;
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    off += w < wave_id() ? wsum[w] : 0;
    total += wsum[w];
  }
  int run = off + incl - s;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (base + e < a.n_keys) a.cur[base + e] = run;
    run += v[e];
  }
  if (threadIdx.x == 0) a.tot[blockIdx.x] = total;
}

// Exclusive scan of the block sums (one workgroup; at most kScanBlock).
__global__ __launch_bounds__(1024) void bwd_scan_totals_kernel(ScatterArgs a, int nb) {
  __shared__ int32_t wsum[16];
  const int base = threadIdx.x * 4;
  int v[4], s = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = base + e < nb ? a.tot[base + e] : 0;
    s += v[e];
  }
  const int incl = wave_incl_scan(s);
  if (lane_id() == 63) wsum[wave_id()] = incl;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) off += w < wave_id() ? wsum[w] : 0;
  int run = off + incl - s;
  __syncthreads();  // every block sum is read before it is replaced
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (base + e < nb) a.tot[base + e] = run;
    run += v[e];
  }
}

__global__ __launch_bounds__(256) void bwd_scan_add_kernel(ScatterArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < a.n_keys) a.cur[i] += a.tot[i / kScanBlock];
}

// Each pair takes a slot in its key's segment (the order within a segment
// varies from run to run; the sums below do not depend on it).
__global__ __launch_bounds__(256) void bwd_fill_kernel(ScatterArgs a) {
  const int64_t np = (a.r1 - a.r0) * a.K_tot;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < np; p += (int64_t)gridDim.x * 256) {
    const int key = pair_key(a, p);
    if (key < 0) continue;
    const int slot = atomicAdd(&a.cur[key], 1);
    a.lkey[slot] = key;
    a.lpair[slot] = (int)p;
  }
}

// bf16 bits to int64 fixed point (value * 2^32)
__device__ __forceinline__ uint64_t bf16_fixed(uint32_t bits16) {
  return to_fixed32(__uint_as_float(bits16 << 16));
}

__device__ __forceinline__ void flush_key(const ScatterArgs& a, int key, const uint64_t (&acc)[4]) {
  const int l = lane_id();
  int64_t* dst = (l < 32 ? a.dk_acc : a.dv_acc) + (int64_t)key * kD + 4 * (l & 31);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    __hip_atomic_fetch_add((unsigned long long*)(dst + e), (unsigned long long)acc[e], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Wave w sums the listed entries [w * kReduceRun, (w + 1) * kReduceRun) of
// the total (cur[n_keys - 1] after the fill): lane l keeps the 4 values at
// 4l of each contribution (lanes 0-31 dk, 32-63 dv) as int64 and adds them
// to the accumulators whenever the key changes and at the end. Keys are
// contiguous in the list, so a wave flushes once per key it meets.
constexpr int kReduceRun = 1024;

__global__ __launch_bounds__(256) void bwd_reduce_kernel(ScatterArgs a) {
  const int total = a.cur[a.n_keys - 1];  // the fill advanced every segment to its end
  const int64_t w = (int64_t)blockIdx.x * 4 + wave_id();
  const int e0 = (int)min<int64_t>(w * kReduceRun, total), e1 = (int)min<int64_t>(e0 + (int64_t)kReduceRun, total);
  if (e0 >= e1) return;
  const int l = lane_id();
  uint64_t acc[4] = {0, 0, 0, 0};
  int ck = -1;
  for (int b0 = e0; b0 < e1; b0 += 64) {
    const int m = min(64, e1 - b0);
    const int lk = l < m ? a.lkey[b0 + l] : -1;
    const int lp = l < m ? a.lpair[b0 + l] : 0;
    for (int i0 = 0; i0 < m; i0 += 8) {
      v2u x[8];
      int kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        kk[u] = __shfl(lk, i0 + u, 64);
        const int pr = __shfl(lp, i0 + u, 64);
        x[u] = i0 + u < m ? *(const v2u*)(a.contrib + (int64_t)pr * 256 + 4 * l) : v2u{0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u >= m) break;
        if (kk[u] != ck) {
          if (ck >= 0) flush_key(a, ck, acc);
          ck = kk[u];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = 0;
        }
        acc[0] += bf16_fixed(x[u][0] & 0xffffu);
        acc[1] += bf16_fixed(x[u][0] >> 16);
        acc[2] += bf16_fixed(x[u][1] & 0xffffu);
        acc[3] += bf16_fixed(x[u][1] >> 16);
      }
    }
  }
  if (ck >= 0) flush_key(a, ck, acc);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(v4u* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) p[i] = v4u{};
}

// int64 fixed point (value * 2^32) to fp32
__global__ __launch_bounds__(256) void attn_bwd_finish_kernel(const int64_t* acc, float* out, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint64_t u = (uint64_t)acc[i];
    const double d = (double)(int32_t)(uint32_t)(u >> 32) * 4294967296.0 + (double)(uint32_t)u;
    out[i] = (float)(d * (1.0 / 4294967296.0));
  }
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 256 * 16);
  KernelTimer kt("fill_zero_kernel", st);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, st, (v4u*)p, n16);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t st) {
  const int TW = a.H / 32, RW = 4 / TW;
  const int64_t wgs = (a.r1 - a.r0 + RW - 1) / RW;
  const dim3 grid((unsigned)((wgs + 7) / 8 * 8));
  KernelTimer kt("attn_bwd_kernel", st);
  if (TW == 1) hipLaunchKernelGGL(attn_bwd_kernel<1>, grid, dim3(256), 0, st, a);
  else if (TW == 2) hipLaunchKernelGGL(attn_bwd_kernel<2>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_bwd_kernel<4>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_scatter(const ScatterArgs& a, hipStream_t st) {
  if (a.n_keys <= 0 || a.n_keys > kMaxScanKeys) return hipErrorInvalidValue;
  hipError_t e = launch_fill_zero(a.cnt, ((size_t)a.n_keys * 4 + 15) / 16 * 16, st);
  if (e != hipSuccess) return e;
  const int64_t np = (a.r1 - a.r0) * a.K_tot;
  const unsigned gp = (unsigned)std::min<int64_t>((np + 255) / 256, 256 * 64);
  const int nb = (a.n_keys + kScanBlock - 1) / kScanBlock;
  {
    KernelTimer kt("bwd_count_kernel", st);
    hipLaunchKernelGGL(bwd_count_kernel, dim3(gp), dim3(256), 0, st, a);
  }
  {
    KernelTimer kt("bwd_scan_kernel", st);
    hipLaunchKernelGGL(bwd_scan_blocks_kernel, dim3(nb), dim3(1024), 0, st, a);
    hipLaunchKernelGGL(bwd_scan_totals_kernel, dim3(1), dim3(1024), 0, st, a, nb);
    hipLaunchKernelGGL(bwd_scan_add_kernel, dim3((a.n_keys + 255) / 256), dim3(256), 0, st, a);
  }
  {
    KernelTimer kt("bwd_fill_kernel", st);
    hipLaunchKernelGGL(bwd_fill_kernel, dim3(gp), dim3(256), 0, st, a);
  }
  KernelTimer kt("bwd_reduce_kernel", st);
  const int64_t waves = (np + kReduceRun - 1) / kReduceRun;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_finish(const int64_t* acc, float* out, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 256 * 16);
  KernelTimer kt("attn_bwd_finish_kernel", st);
  hipLaunchKernelGGL(attn_bwd_finish_kernel, dim3(grid), dim3(256), 0, st, acc, out, n);
  return hipGetLastError();
}

}  // namespace lsa
