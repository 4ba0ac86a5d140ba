// LSA warm-up KL operator on bf16 MFMA (gfx950).
//
// The LongCat-2.0 release article (section "长上下文训练", paragraph "LSA 算子与
// 前向优化") describes a KL-loss operator for LSA's warm-up in which a single
// forward pass yields both the KL loss and its gradient. For each query row
// t with key list S_t (the selected keys, or every key 0..t for a dense
// warm-up) and indexer logits l[t, j] for those keys:
//   p_s  = (1/H) sum_h exp(scale q_h . k_s - lse_h)     the attention
//          distribution of the row averaged over its H heads, with lse the
//          forward's log-sum-exp over the same list
//   KL_t = sum_s p_s (log p_s - log softmax(l)_s),  dKL_t/dl = softmax(l) - p
// Nothing runs backward through the attention: P comes from the same K rows
// and q as the forward, and the forward's lse normalises it.
//
// A wave takes 32 heads of one row; the TW = H / 32 waves of the row share
// one LDS gather of each 32-key block of K. S = Q . K^T puts the key on the
// lane and 16 heads in the lane's accumulator entries, so the head sum of a
// key is a sum over the lane's entries, one lane-half exchange and, across
// the row's waves, a fixed-order sum through LDS (deterministic).
#include <math.h>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int kD = 128;
constexpr int kRowK = 272;  // LDS bytes per K row (conflict-free 16-byte reads)
constexpr int kBlkK = 32 * kRowK;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <int TW>
__global__ __launch_bounds__(256) void kl_warmup_kernel(KlArgs a) {
  constexpr int RW = 4 / TW;  // rows per workgroup
  __shared__ __attribute__((aligned(16))) char lds_k[RW * kBlkK];
  __shared__ float xbuf[2][4][32];  // per block parity: each wave's head sums of the block's keys
  const int wv = wave_id(), gw = wv % TW, sr = wv / TW;
  const int64_t per = gridDim.x / 8, bx = blockIdx.x;
  const int64_t tile = (bx % 8) * per + bx / 8;
  const int64_t rows = (int64_t)a.B * a.L;
  const int64_t gq0 = tile * RW;
  if (gq0 >= rows) return;  // the same for every wave of the workgroup
  const bool active = gq0 + sr < rows;
  const int64_t gq = active ? gq0 + sr : rows - 1;
  const int b = (int)(gq / a.L);
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int h0 = 32 * gw;
  int nmax = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r)
    if (gq0 + r < rows) nmax = max(nmax, min(max(a.n_sel[gq0 + r], 0), a.K_tot));
  const int n = active ? min(max(a.n_sel[gq], 0), a.K_tot) : 0;
  // A operand of S = Q . K^T: lane (g, c) head h0 + c, dims 64g + 8j + {0..7}
  const uint16_t* qrow = a.q + gq * a.H * kD;
  v8bf Q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) Q[j] = *(const v8bf*)(qrow + (h0 + c) * kD + 64 * g + 8 * j);
  // lse (base 2) of the heads of accumulator entry i: h0 + 8(i/4) + 4g + i%4
  float lse2[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lse2[i] = a.lse[gq * a.H + h0 + 8 * (i >> 2) + 4 * g + (i & 3)] * kLog2e;
  // log of the indexer's softmax normaliser over the row's n logits, in a
  // fixed order (lane-strided partials, then a fixed butterfly)
  const float* lg = a.logits + gq * a.K_tot;
  float mx = -INFINITY;
  for (int j = l; j < n; j += 64) mx = fmaxf(mx, lg[j]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, d));
  float z = 0.f;
  for (int j = l; j < n; j += 64) z += __builtin_amdgcn_exp2f((lg[j] - mx) * kLog2e);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) z += shfl_xor_f(z, d);
  const float lnZ = n > 0 ? mx + log2f(z) * kLn2 : 0.f;
  const int32_t* ids = a.idx + gq * a.K_tot;
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(K, (uint32_t)a.n_k * (uint32_t)(kD * 2));
  char* kb = lds_k + sr * kBlkK;
  float* dl = a.dlogits + gq * a.K_tot;
  const float inv_h = 1.f / (float)a.H;
  float kl = 0.f;
  // the previous block's head sums become the KL terms and gradient of its
  // keys once every wave of the row has written them (after the next barrier)
  auto emit = [&](int bi) {
    if (gw != 0 || g != 0 || !active) return;
    const int j = 32 * bi + c;
    if (j >= n) return;
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < TW; ++w) p += xbuf[bi & 1][sr * TW + w][c];
    p *= inv_h;
    const float logq = lg[j] - lnZ;
    if (p > 0.f) kl += p * (log2f(p) * kLn2 - logq);
    dl[j] = __builtin_amdgcn_exp2f(logq * kLog2e) - p;
  };
  const int nblk = (nmax + 31) / 32;
  // K rows of one block: thread 64 * gw + lane loads 16 bytes of row
  // 4 * gw + lane / 16 + 4 * TW * i, i < 8 / TW
  v4u stg[8 / TW];
  auto gather = [&](int bi) {
    const int s = 32 * bi + c;
    const int pos = s < n ? ids[s] : -1;
#pragma unroll
    for (int i = 0; i < 8 / TW; ++i) {
      const int pe = __shfl(pos, 4 * gw + (l >> 4) + 4 * TW * i, 64);
      const uint32_t off = (uint32_t)pe * (uint32_t)(kD * 2) + 16u * (uint32_t)(l & 15);
      stg[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)off, 0, 0));
    }
    return pos;
  };
  int pos = gather(0);
  for (int bi = 0; bi < nblk; ++bi) {
    __syncthreads();  // the previous block's K rows and head sums are read
    if (bi > 0) emit(bi - 1);
#pragma unroll
    for (int i = 0; i < 8 / TW; ++i) *(v4u*)(kb + (4 * gw + (l >> 4) + 4 * TW * i) * kRowK + 16 * (l & 15)) = stg[i];
    const int pcur = pos;
    pos = gather(bi + 1);
    __syncthreads();
    // S = Q . K^T: lane (g, c) key c, entry i head h0 + 8(i/4) + 4g + i%4
    v16f S = v16f{};
#pragma unroll
    for (int j = 0; j < 8; ++j) S = mfma_bf16_32x32x16(Q[j], *(const v8bf*)(kb + c * kRowK + g * 128 + 16 * j), S);
    float ps = 0.f;
    if ((unsigned)pcur < (unsigned)a.n_k) {
#pragma unroll
      for (int i = 0; i < 16; ++i) ps += __builtin_amdgcn_exp2f(fmaf(S[i], a.sl2, -lse2[i]));
    }
    ps += shfl_xor_f(ps, 32);
    if (g == 0) xbuf[bi & 1][wv][c] = ps;
  }
  __syncthreads();
  if (nblk > 0) emit(nblk - 1);
  if (gw != 0 || !active) return;
  // fixed-order lane sum of the KL terms (lanes 0..31 hold them)
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) kl += shfl_xor_f(kl, d);
  if (l == 0) a.kl[gq] = kl;
  for (int j = n + l; j < a.K_tot; j += 64) dl[j] = 0.f;
}

}  // namespace

hipError_t launch_kl_warmup(const KlArgs& a, hipStream_t st) {
  const int TW = a.H / 32, RW = 4 / TW;
  const int64_t wgs = ((int64_t)a.B * a.L + RW - 1) / RW;
  const dim3 grid((unsigned)((wgs + 7) / 8 * 8));
  KernelTimer kt("kl_warmup_kernel", st);
  if (TW == 1) hipLaunchKernelGGL(kl_warmup_kernel<1>, grid, dim3(256), 0, st, a);
  else if (TW == 2) hipLaunchKernelGGL(kl_warmup_kernel<2>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(kl_warmup_kernel<4>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
