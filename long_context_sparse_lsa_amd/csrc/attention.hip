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
// so softmax probabilities go from accumulator to operand in place. The V
// tile is transposed through a per-wave LDS buffer (4x4 register transposes,
// 8-byte LDS writes and reads). Online softmax runs in fp32 in base 2.
//
// Decode splits the selected list into n_split contiguous parts (the one-GPU
// form of the KV-cache parallel decode of the "③ KVP 解码切分示意" section) and
// merges the (max, sum, output) partials with a fixed-shape binary tree.
#include <math.h>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

constexpr int kD = 128;
constexpr int kKRow = 272;                   // bytes per K row in LDS: 256 + pad, conflict-free 16-byte reads
constexpr int kVRow = 320;                   // bytes per V row in LDS: 256 + pad, conflict-free transposed reads
constexpr int kVOff = 32 * kKRow;            // V rows follow the K rows of a block
constexpr int kBlkLds = kVOff + 32 * kVRow;  // one 32-key block of K and V rows
constexpr int kWaveLds = 2 * kBlkLds;        // two blocks per wave
constexpr float kSlack = 8.f;                // softmax reference slack, log2 units

template <int NB>
struct AttnState {
  v16f o[4][NB];
  float m[NB], l[NB];
};

__device__ __forceinline__ v8bf load_v8bf(const uint16_t* p) { return *(const v8bf*)p; }

template <int NB>
__device__ __forceinline__ void attn_init(AttnState<NB>& st) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    st.m[nb] = -INFINITY;
    st.l[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st.o[mb][nb] = v16f{};
  }
}

// Load the B operand Q^T for heads [h0, h0 + 32*NB) of one query row
// (row base pointer qrow -> [H][128]); heads >= H are zero.
template <int NB>
__device__ __forceinline__ void load_q(const uint16_t* qrow, int h0, int H, v8bf (&Q)[NB][8]) {
  const int l = lane_id(), g = l >> 5, c = l & 31;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int h = h0 + 32 * nb + c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (h < H) Q[nb][j] = load_v8bf(qrow + (int64_t)h * kD + g * 64 + 8 * j);
      else Q[nb][j] = v8bf{};
    }
  }
}

// K and V rows of one 32-key block, staged through registers on their way
// to LDS: load i of lane l holds bytes 16 * (l % 16) of the rows of key
// 4i + l/16. A key outside [0, n_k) loads row 0 instead: its score is set to
// -inf and its probability to 0 before use, so only finiteness matters and
// the loads need no masking.
struct KVStage {
  v4u k[8], v[8];
};

__device__ __forceinline__ void gather_kv(const uint16_t* K, const uint16_t* V, int pos, int n_k,
                                          KVStage& s) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pe = __shfl(pos, 4 * i + (l >> 4), 64);
    const int64_t p = (unsigned)pe < (unsigned)n_k ? pe : 0;
    s.k[i] = *(const v4u*)(K + p * kD + 8 * (l & 15));
    s.v[i] = *(const v4u*)(V + p * kD + 8 * (l & 15));
  }
}

// The staged rows into one LDS block buffer (K rows, then V rows).
__device__ __forceinline__ void store_kv(const KVStage& s, char* blk) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = 4 * i + (l >> 4);
    *(v4u*)(blk + key * kKRow + 16 * (l & 15)) = s.k[i];
    *(v4u*)(blk + kVOff + key * kVRow + 16 * (l & 15)) = s.v[i];
  }
}

// The V^T operand of the PV product for dims 32mb.. and key slice js, read
// transposed from the row-major V block with two ds_read_b64_tr_b16. The
// transposing read gives lane j of each 16-lane group element j % 4 of the
// 8-byte pieces addressed by lanes j / 4 + 4s of the group (s = 0..3), so a
// lane addresses key row 4(G / 2) + j / 4 (+ the slice and half offsets) at
// dims 16(G % 2) + 4(j % 4) (G = lane / 16). Lane (g, c) then holds dim c of
// keys 16js + 4g + {0..3} and 16js + 8 + 4g + {0..3}: the key order of the P^T
// operand.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v8bf read_vt(const char* vblk, int lane_off, int mb, int js) {
  const char* p = vblk + lane_off + 16 * js * kVRow + 64 * mb;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 8 * kVRow));
  const v4u u = v4u{__builtin_bit_cast(v2u, lo)[0], __builtin_bit_cast(v2u, lo)[1], __builtin_bit_cast(v2u, hi)[0],
                    __builtin_bit_cast(v2u, hi)[1]};
  return __builtin_bit_cast(v8bf, u);
}

// Attend the wave's rows over keys ids[kb .. ke) of one sequence, 32 keys
// per block. The block's K and V rows sit in one of two per-wave LDS buffers
// (kWaveLds bytes at lds). Loads run two blocks ahead: while block i is
// computed from its buffer, the rows of block i + 2 are in flight in one
// register stage and those of block i + 1 (in flight since the previous
// block) go from the other stage into the second buffer at the end.
template <int NB>
__device__ __forceinline__ void attn_block(const v8bf (&Q)[NB][8], const char* blk, int pos, int n_k,
                                           float sl2, int vt_off, AttnState<NB>& st);

template <int NB>
__device__ void attn_keys(const v8bf (&Q)[NB][8], const uint16_t* K, const uint16_t* V,
                          const int32_t* ids, int kb, int ke, int n_k, float sl2,
                          AttnState<NB>& st, char* lds) {
  const int l = lane_id(), c = l & 31;
  const int G = l >> 4, jj = l & 15;
  const int vt_off = kVOff + (4 * (G >> 1) + (jj >> 2)) * kVRow + (16 * (G & 1) + 4 * (jj & 3)) * 2;
  auto pos_at = [&](int s0) { return s0 + c < ke ? ids[s0 + c] : -1; };
  if (kb >= ke) return;
  KVStage sa, sb;
  int p0 = pos_at(kb), p1 = pos_at(kb + 32), p2 = pos_at(kb + 64);
  gather_kv(K, V, p0, n_k, sa);
  store_kv(sa, lds);
  if (kb + 32 < ke) gather_kv(K, V, p1, n_k, sb);
  // two blocks per trip so that the stages and buffers swap roles statically
  for (int s0 = kb; s0 < ke; s0 += 64) {
    {
      const int p3 = pos_at(s0 + 96);
      if (s0 + 64 < ke) gather_kv(K, V, p2, n_k, sa);
      attn_block<NB>(Q, lds, p0, n_k, sl2, vt_off, st);
      if (s0 + 32 < ke) store_kv(sb, lds + kBlkLds);
      p0 = p1;
      p1 = p2;
      p2 = p3;
    }
    if (s0 + 32 < ke) {
      const int p3 = pos_at(s0 + 128);
      if (s0 + 96 < ke) gather_kv(K, V, p2, n_k, sb);
      attn_block<NB>(Q, lds + kBlkLds, p0, n_k, sl2, vt_off, st);
      if (s0 + 64 < ke) store_kv(sa, lds);
      p0 = p1;
      p1 = p2;
      p2 = p3;
    }
  }
}

// One 32-key block: scores, softmax update, PV product. pos: this lane's key
// position (lane % 32); K and V rows in LDS at blk.
template <int NB>
__device__ __forceinline__ void attn_block(const v8bf (&Q)[NB][8], const char* blk, int pos, int n_k,
                                           float sl2, int vt_off, AttnState<NB>& st) {
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const bool valid = (unsigned)pos < (unsigned)n_k;
  const uint32_t vmask = (uint32_t)__ballot(valid);

  // ---- S^T = K * Q^T (A operand: key row c, dims g*64 + 8j from LDS)
  v16f S[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) S[nb] = v16f{};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const v8bf Ka = *(const v8bf*)(blk + c * kKRow + g * 128 + 16 * j);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) S[nb] = mfma_bf16_32x32x16(Ka, Q[nb][j], S[nb]);
  }

    // ---- softmax numerators in base 2 against a per-head reference st.m:
    // p = 2^(S * sl2 - m). The reference moves up only when a block's max
    // exceeds it by more than kSlack, so p < 2^kSlack and the O / l rescale
    // is rare; o / l does not depend on the reference. l is kept per lane
    // half (16 of the 32 keys) and the halves are added at the end.
    const bool full = (uint32_t)vmask == 0xffffffffu;
    if (!full) {
      // a block with invalid keys (the ragged tail): scores to -inf
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kt = 8 * (i >> 2) + 4 * g + (i & 3);
          if (!((vmask >> kt) & 1u)) S[nb][i] = -INFINITY;
        }
    }
    float mx[NB];
    bool need = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float m = S[nb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = fmaxf(m, S[nb][i]);
      mx[nb] = fmaxf(m, shfl_xor_f(m, 32)) * sl2;
      need = need || mx[nb] > st.m[nb] + kSlack;
    }
    if (__any(need)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mnew = mx[nb] > st.m[nb] + kSlack ? mx[nb] : st.m[nb];
        const float alpha = __builtin_amdgcn_exp2f(st.m[nb] - mnew);  // 0 when st.m is -inf
        st.l[nb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st.o[mb][nb] *= alpha;
        st.m[nb] = mnew;
      }
    }
    // p = 2^(S*sl2 - m) (exp2 of -inf is 0); l sums p in fp32, and P is
    // rounded to bf16 for the PV product
    v8bf P[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float nm = -st.m[nb];
      float rs = 0.f;
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        v8bf x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[nb][8 * js + e], sl2, nm));
          rs += p;
          x[e] = (__bf16)p;
        }
        P[nb][js] = x;
      }
      st.l[nb] += rs;
    }

    // ---- O^T += V^T * P^T
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        const v8bf Va = read_vt(blk, vt_off, mb, js);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) st.o[mb][nb] = mfma_bf16_32x32x16(Va, P[nb][js], st.o[mb][nb]);
      }
    }
}

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
  attn_keys<NB>(Q, K, V, a.idx + gq * a.K_tot, 0, n, a.n_k, a.sl2, st, lds_all + wv * kWaveLds);
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

hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t st) {
  const int NB = a.H <= 32 ? 1 : 2;
  const int HB = (a.H + 32 * NB - 1) / (32 * NB);
  const int64_t groups = (int64_t)a.B * a.L * HB;
  dim3 grid((unsigned)(((groups + 3) / 4 + 7) / 8 * 8));
  if (NB == 1) hipLaunchKernelGGL(attn_prefill_kernel<1>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_prefill_kernel<2>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode
// Partials: ws_m / ws_l [B, n_split, R], ws_o [B, n_split, R, 128] with
// R = n_q * H; o is unnormalised, m in base-2 units.
template <int NB>
__global__ __launch_bounds__(256) void attn_decode_partial(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds_all[4 * kWaveLds];
  const int wv = wave_id();
  const int HB = (a.H + 32 * NB - 1) / (32 * NB);
  const int gi = blockIdx.x * 4 + wv;
  if (gi >= a.n_q * HB) return;
  const int qr = gi / HB, hb = gi % HB;
  const int split = blockIdx.y, b = blockIdx.z;
  const int l = lane_id(), g = l >> 5, c = l & 31;
  const int R = a.n_q * a.H;
  v8bf Q[NB][8];
  load_q<NB>(a.q + ((int64_t)b * a.n_q + qr) * a.H * kD, hb * 32 * NB, a.H, Q);
  AttnState<NB> st;
  attn_init(st);
  const int irow = a.n_idx == 1 ? 0 : qr;
  const int64_t ibase = (int64_t)b * a.n_idx + irow;
  const int n = min(max(a.n_sel[ibase], 0), a.K_tot);
  const int cs = (n + a.n_split - 1) / a.n_split;
  const int kb = min(n, split * cs), ke = min(n, (split + 1) * cs);
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const uint16_t* V = a.v + (int64_t)b * a.n_k * kD;
  attn_keys<NB>(Q, K, V, a.idx + ibase * a.K_tot, kb, ke, a.n_k, a.sl2, st, lds_all + wv * kWaveLds);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.l[nb] += shfl_xor_f(st.l[nb], 32);  // both key halves

  const int64_t pbase = ((int64_t)b * a.n_split + split) * R;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int h = hb * 32 * NB + 32 * nb + c;
    if (h >= a.H) continue;
    const int64_t row = pbase + (int64_t)qr * a.H + h;
    if (g == 0) {
      a.ws_m[row] = st.m[nb];
      a.ws_l[row] = st.l[nb];
    }
    float* orow = a.ws_o + row * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v16f& O = st.o[mb][nb];
        *(v4f*)(orow + 32 * mb + 8 * i4 + 4 * g) =
            v4f{O[4 * i4], O[4 * i4 + 1], O[4 * i4 + 2], O[4 * i4 + 3]};
      }
  }
}

constexpr int kMaxSplit = 64;

// One block per (sequence, row); thread = output dim. Weighted sums over the
// splits use a fixed 64-leaf binary tree (absent splits are exact zeros).
__global__ __launch_bounds__(128) void attn_decode_merge(DecodeArgs a) {
  const int R = a.n_q * a.H;
  const int64_t brow = blockIdx.x;
  const int b = (int)(brow / R), r = (int)(brow % R);
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int j = 0; j < a.n_split; ++j) M = fmaxf(M, a.ws_m[((int64_t)b * a.n_split + j) * R + r]);
  float lv[kMaxSplit], ov[kMaxSplit];
#pragma unroll
  for (int j = 0; j < kMaxSplit; ++j) {
    lv[j] = 0.f;
    ov[j] = 0.f;
    if (j < a.n_split && M != -INFINITY) {
      const int64_t row = ((int64_t)b * a.n_split + j) * R + r;
      const float wj = exp2f(a.ws_m[row] - M);
      lv[j] = wj * a.ws_l[row];
      ov[j] = wj * a.ws_o[row * kD + d];
    }
  }
#pragma unroll
  for (int s = 1; s < kMaxSplit; s <<= 1)
#pragma unroll
    for (int j = 0; j + s < kMaxSplit; j += 2 * s) {
      lv[j] += lv[j + s];
      ov[j] += ov[j + s];
    }
  const float Lam = lv[0];
  const float out = Lam > 0.f ? ov[0] / Lam : 0.f;
  a.o[brow * kD + d] = (uint16_t)f32_to_bf16_bits(out);
  if (a.lse && d == 0) a.lse[brow] = Lam > 0.f ? (M + log2f(Lam)) * 0.69314718055994531f : -INFINITY;
}

size_t decode_ws_bytes(int B, int n_q, int H, int n_split) {
  const size_t rows = (size_t)B * n_split * n_q * H;
  return rows * sizeof(float) * (2 + kD) + 256;
}

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t st) {
  const int NB = a.H <= 32 ? 1 : 2;
  const int HB = (a.H + 32 * NB - 1) / (32 * NB);
  const int groups = a.n_q * HB;
  dim3 grid((groups + 3) / 4, a.n_split, a.B);
  if (NB == 1) hipLaunchKernelGGL(attn_decode_partial<1>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_decode_partial<2>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_merge, dim3((unsigned)((int64_t)a.B * a.n_q * a.H)), dim3(kD), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
