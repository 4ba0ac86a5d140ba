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
//   dV    = P . dO              A = P by transposed reads of the wave's P^T tile
//   dK    = dS . Q (x scale)    A = dS the same way
// with Delta = sum_d dO . o per head. dQ stays in registers for the whole
// row. dK and dV of a block are added into int64 fixed-point accumulators
// (value * 2^32 rounded to nearest even) by integer atomics: integer addition
// is associative, so the totals are the same whatever order the rows arrive
// in, and repeated runs are bit-identical with no float atomics. A last pass
// converts the totals to fp32.
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

__device__ __forceinline__ void add_fixed(int64_t* p, float x) {
  __hip_atomic_fetch_add((unsigned long long*)p, (unsigned long long)to_fixed32(x), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
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

// Per-row operands of one wave (heads h0 .. h0 + 31 of the row).
struct RowOps {
  v8bf Qb[8], dOb[8];     // B of S^T / dP^T: lane (g, c) head h0 + c, dims 64g + 8j + {0..7}
  v8bf Qt[4][2], dOt[4][2];  // B of dK / dV: lane (g, c) dim 32nb + c, heads 16js + 4g + {0..3, 8..11}
  float dlt, lse2;        // Delta and lse * log2(e) of head h0 + c
};

__device__ __forceinline__ void load_row_ops(const BwdArgs& a, int64_t gq, int h0, RowOps& r) {
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
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      v8bf x, y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int h = h0 + 16 * js + 4 * g + (e & 3) + 8 * (e >> 2);
        x[e] = __builtin_bit_cast(__bf16, qr[h * kD + 32 * nb + c]);
        y[e] = __builtin_bit_cast(__bf16, dr[h * kD + 32 * nb + c]);
      }
      r.Qt[nb][js] = x;
      r.dOt[nb][js] = y;
    }
  r.lse2 = a.lse[gq * a.H + h0 + c] * kLog2e;
}

// One 32-key block: lane c (and c + 32) holds the position of key c.
__device__ __forceinline__ void bwd_block(const BwdArgs& a, const RowOps& r, const char* kb, const char* vb,
                                          char* ptile, char* stile, int pos, int b, v16f (&dQ)[4]) {
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
  // the P^T and dS^T tiles of this wave: row = head c, 8-byte runs of keys
  // 16js + 4g + {0..3} and 16js + 8 + 4g + {0..3}
#pragma unroll
  for (int js = 0; js < 2; ++js) {
    const v4u pu = __builtin_bit_cast(v4u, Pb[js]), su = __builtin_bit_cast(v4u, Sb[js]);
    char* pp = ptile + c * kTileP + (16 * js + 4 * g) * 2;
    char* sp = stile + c * kTileP + (16 * js + 4 * g) * 2;
    *(v2u*)pp = v2u{pu[0], pu[1]};
    *(v2u*)(pp + 16) = v2u{pu[2], pu[3]};
    *(v2u*)sp = v2u{su[0], su[1]};
    *(v2u*)(sp + 16) = v2u{su[2], su[3]};
  }
  // the block's keys in accumulator row order, for the scatter
  int pk[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pk[i] = __shfl(pos, 8 * (i >> 2) + 4 * g + (i & 3), 64);
  const int t_off = tr_lane_off(kTileP);
  int64_t* dvb = a.dv_acc + (int64_t)b * a.n_k * kD;
  int64_t* dkb = a.dk_acc + (int64_t)b * a.n_k * kD;
  // dV = P . dO, then dK = dS . Q: lane (g, c) holds dim 32nb + c of keys pk[i]
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const char* tile = which == 0 ? ptile : stile;
    const v8bf A0 = read_tr(tile + t_off, kTileP), A1 = read_tr(tile + t_off + 16 * kTileP, kTileP);
    int64_t* dst = which == 0 ? dvb : dkb;
    const float mul = which == 0 ? 1.f : a.scale;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      v16f acc = v16f{};
      acc = mfma_bf16_32x32x16(A0, which == 0 ? r.dOt[nb][0] : r.Qt[nb][0], acc);
      acc = mfma_bf16_32x32x16(A1, which == 0 ? r.dOt[nb][1] : r.Qt[nb][1], acc);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((unsigned)pk[i] < (unsigned)a.n_k) add_fixed(dst + (int64_t)pk[i] * kD + 32 * nb + c, acc[i] * mul);
    }
  }
}

template <int TW>
__global__ __launch_bounds__(256) void attn_bwd_kernel(BwdArgs a) {
  constexpr int RW = 4 / TW;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) char lds_kv[RW * 2 * kBlkB];
  __shared__ __attribute__((aligned(16))) char lds_t[4 * 2 * kTileB];
  const int wv = wave_id(), gw = wv % TW, sr = wv / TW;
  // each XCD walks a contiguous range of rows (the grid is a multiple of 8)
  const int64_t per = gridDim.x / 8, bx = blockIdx.x;
  const int64_t tile = (bx % 8) * per + bx / 8;
  const int64_t rows = (int64_t)a.B * a.L;
  const int64_t gq0 = tile * RW;
  if (gq0 >= rows) return;  // the same for every wave of the workgroup
  const bool active = gq0 + sr < rows;
  const int64_t gq = active ? gq0 + sr : rows - 1;
  const int b = (int)(gq / a.L);
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int h0 = gw * 32;
  int nmax = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r)
    if (gq0 + r < rows) nmax = max(nmax, min(max(a.n_sel[gq0 + r], 0), a.K_tot));
  const int n = active ? min(max(a.n_sel[gq], 0), a.K_tot) : 0;
  RowOps ro;
  load_row_ops(a, gq, h0, ro);
  const int32_t* ids = a.idx + gq * a.K_tot;
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const uint16_t* V = a.v + (int64_t)b * a.n_k * kD;
  const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(K, (uint32_t)a.n_k * (uint32_t)(kD * 2));
  const __amdgpu_buffer_rsrc_t vr = uniform_rsrc(V, (uint32_t)a.n_k * (uint32_t)(kD * 2));
  char* kb = lds_kv + sr * 2 * kBlkB;
  char* vb = kb + kBlkB;
  char* ptile = lds_t + wv * 2 * kTileB;
  char* stile = ptile + kTileB;
  v16f dQ[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) dQ[mb] = v16f{};
  const int nblk = (nmax + 31) / 32;
  int pos = c < n ? ids[c] : -1;
  Stage<TW> stg;
  gather<TW>(kr, vr, pos, gw, stg);
  for (int bi = 0; bi < nblk; ++bi) {
    __syncthreads();  // the previous block's K / V rows are no longer read
    store<TW>(stg, kb, vb, gw);
    const int pcur = pos;
    const int s1 = 32 * (bi + 1) + c;
    pos = s1 < n ? ids[s1] : -1;
    gather<TW>(kr, vr, pos, gw, stg);  // the next block's rows load during this one
    __syncthreads();
    if (32 * bi < n) bwd_block(a, ro, kb, vb, ptile, stile, pcur, b, dQ);
  }
  if (!active) return;
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
  const int64_t wgs = ((int64_t)a.B * a.L + RW - 1) / RW;
  const dim3 grid((unsigned)((wgs + 7) / 8 * 8));
  KernelTimer kt("attn_bwd_kernel", st);
  if (TW == 1) hipLaunchKernelGGL(attn_bwd_kernel<1>, grid, dim3(256), 0, st, a);
  else if (TW == 2) hipLaunchKernelGGL(attn_bwd_kernel<2>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_bwd_kernel<4>, grid, dim3(256), 0, st, a);
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
