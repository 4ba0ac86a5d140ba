// Sparse attention device code shared by the attention kernels and the
// fused HI decode step: the gathered K/V block pipeline, the per-block
// softmax update on bf16 MFMA, the split-KV part of a decode row group and
// the log-sum-exp merge. The method and the measured design choices are
// described in attention.hip.
#pragma once
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
// to LDS, gathered by a group of TW waves that share the block: thread gt
// of the group (gt = 64 * wave-in-group + lane) loads, for i < 8 / TW, the
// 16 bytes at 16 * (gt % 16) of the K row and of the V row of key
// gt / 16 + 4 * TW * i. The loads are buffer loads over one sequence's
// cache (a 32-bit byte offset from a wave-uniform base, range-checked by the
// hardware): a key outside [0, n_k) reads zeros, or, where its offset wraps
// past 2^32, some row of the cache. Its score is set to -inf and its
// probability to 0 before use, so only finiteness matters and the loads need
// no masking. The 32-bit offsets bound a cache at kMaxCacheKeys rows.
template <int TW>
struct KVStage {
  v4u k[8 / TW], v[8 / TW];
};

// Rows [0, n_k) of one sequence's K or V cache.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cache_rsrc(const uint16_t* base, int n_k) {
  return uniform_rsrc(base, (uint32_t)n_k * (uint32_t)(kD * 2));
}

// 16 bytes at part 16 * part of row pos (unsigned offset arithmetic: a
// negative or huge pos wraps, and lands out of range or on some row)
__device__ __forceinline__ v4u load_row16(__amdgpu_buffer_rsrc_t r, int pos, int part) {
  const uint32_t off = (uint32_t)pos * (uint32_t)(kD * 2) + 16u * (uint32_t)part;
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// pos: lane c (and c + 32) holds the cache position of key c of the block.
template <int TW>
__device__ __forceinline__ void gather_kv(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int pos, int gw,
                                          KVStage<TW>& s) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8 / TW; ++i) {
    const int pe = __shfl(pos, 4 * gw + (l >> 4) + 4 * TW * i, 64);
    s.k[i] = load_row16(kr, pe, l & 15);
    s.v[i] = load_row16(vr, pe, l & 15);
  }
}

// The staged pieces into one LDS block buffer (K rows, then V rows).
template <int TW>
__device__ __forceinline__ void store_kv(const KVStage<TW>& s, char* blk, int gw) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8 / TW; ++i) {
    const int key = 4 * gw + (l >> 4) + 4 * TW * i;
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
__device__ __forceinline__ v8bf read_vt(const char* vblk, int lane_off, int mb, int js) {
  const char* p = vblk + lane_off + 16 * js * kVRow + 64 * mb;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 8 * kVRow));
  const v4u u = v4u{__builtin_bit_cast(v2u, lo)[0], __builtin_bit_cast(v2u, lo)[1], __builtin_bit_cast(v2u, hi)[0],
                    __builtin_bit_cast(v2u, hi)[1]};
  return __builtin_bit_cast(v8bf, u);
}

template <int NB>
__device__ __forceinline__ void attn_block(const v8bf (&Q)[NB][8], const char* blk, int pos, int n_k,
                                           float sl2, int vt_off, AttnState<NB>& st);

// Attend the wave's rows over keys ids[sb .. se), 32 keys per block, with
// the block's K and V rows in one of two LDS buffers (kBlkLds bytes each at
// lds) shared by the TW waves of a group (SYNC: a workgroup barrier orders
// the buffers; a single-wave group needs none, its LDS accesses execute in
// order). Gathers run R blocks ahead through a ring of R register stages:
// step i issues the loads of block i + R, computes block i and moves block
// i + 1 from its stage into the other buffer. No load sits under a branch
// and no loaded value is used before it has to be (masking is applied at
// use), so the memory counter waits only for the stage being moved, not for
// the loads still in flight. trips: the number of steps, a multiple of R and at least
// the number of blocks; the same for all waves that meet at barriers.
template <int NB, int TW, int R, bool SYNC>
__device__ void attn_keys(const v8bf (&Q)[NB][8], bool active, const uint16_t* K, const uint16_t* V,
                          const int32_t* ids, int sb, int se, int trips, int n_k, float sl2, int gw,
                          AttnState<NB>& st, char* lds) {
  static_assert(R % 2 == 0, "block parity selects the LDS buffer");
  const int l = lane_id(), c = l & 31;
  const int G = l >> 4, jj = l & 15;
  const int vt_off = kVOff + (4 * (G >> 1) + (jj >> 2)) * kVRow + (16 * (G & 1) + 4 * (jj & 3)) * 2;
  // positions through a buffer over ids[0, se): entries past se read 0 (and
  // eff replaces them by -1)
  const __amdgpu_buffer_rsrc_t ir = uniform_rsrc(ids, (uint32_t)max(se, 0) * 4u);
  auto raw_at = [&](int s0) { return __builtin_amdgcn_raw_buffer_load_b32(ir, (s0 + c) * 4, 0, 0); };
  auto eff = [&](int s0, int raw) { return s0 + c < se ? raw : -1; };
  // The memory counter is in order: waiting for a position also waits for
  // every gather issued before it. Positions are therefore loaded P blocks
  // ahead, far enough that this never waits for a stage before it is due.
  constexpr int P = R > 2 ? 2 * R - 2 : R;
  KVStage<TW> stg[R];
  int pr[P + 1];  // raw positions of blocks i .. i + P
#pragma unroll
  for (int j = 0; j <= P; ++j) pr[j] = raw_at(sb + 32 * j);
  const __amdgpu_buffer_rsrc_t kr = cache_rsrc(K, n_k), vr = cache_rsrc(V, n_k);
#pragma unroll
  for (int j = 0; j < R; ++j) gather_kv<TW>(kr, vr, eff(sb + 32 * j, pr[j]), gw, stg[j]);
  store_kv<TW>(stg[0], lds, gw);
  for (int it = 0; it < trips; it += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int s0 = sb + 32 * (it + u);
      if constexpr (SYNC) __syncthreads();  // block it+u in its buffer for all; the other buffer free
      const int pnew = raw_at(s0 + 32 * (P + 1));
      gather_kv<TW>(kr, vr, eff(s0 + 32 * R, pr[R]), gw, stg[u]);
      if (active && s0 < se) attn_block<NB>(Q, lds + (u & 1) * kBlkLds, eff(s0, pr[0]), n_k, sl2, vt_off, st);
      store_kv<TW>(stg[(u + 1) % R], lds + ((u + 1) & 1) * kBlkLds, gw);
#pragma unroll
      for (int j = 0; j < P; ++j) pr[j] = pr[j + 1];
      pr[P] = pnew;
    }
  }
}

// The same pipeline with the positions already in LDS (pos: the chunk's
// positions, -1 from entry cnt on, readable up to entry 32 * (trips + R)).
// The block loop then issues no global load but the gathers, so the memory
// counter holds nothing else and a stage waits only on its own loads. Used
// where positions would otherwise chain their load latency into every step.
// trips_used: the key span of the chunk's longest subrange (the same for all
// waves of the workgroup); steps past its last block are not run.
template <int TW>
__device__ __forceinline__ void gather_kv_lds(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, const int* pb,
                                              int gw, KVStage<TW>& s) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 8 / TW; ++i) {
    const int pe = pb[4 * gw + (l >> 4) + 4 * TW * i];
    s.k[i] = load_row16(kr, pe, l & 15);
    s.v[i] = load_row16(vr, pe, l & 15);
  }
}

template <int NB, int TW, int R>
__device__ void attn_keys_lds(const v8bf (&Q)[NB][8], bool active, const uint16_t* K, const uint16_t* V,
                              const int* pos, int cnt, int trips, int trips_used, int n_k, float sl2, int gw,
                              AttnState<NB>& st, char* lds) {
  static_assert(R % 2 == 0, "block parity selects the LDS buffer");
  const int l = lane_id(), c = l & 31;
  const int G = l >> 4, jj = l & 15;
  const int vt_off = kVOff + (4 * (G >> 1) + (jj >> 2)) * kVRow + (16 * (G & 1) + 4 * (jj & 3)) * 2;
  KVStage<TW> stg[R];
  const __amdgpu_buffer_rsrc_t kr = cache_rsrc(K, n_k), vr = cache_rsrc(V, n_k);
#pragma unroll
  for (int j = 0; j < R; ++j) gather_kv_lds<TW>(kr, vr, pos + 32 * j, gw, stg[j]);
  store_kv<TW>(stg[0], lds, gw);
  const int nsteps = (trips_used + 31) / 32;  // the blocks of the chunk's longest subrange
  for (int it = 0; it < trips; it += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int bi = it + u;
      if (bi >= nsteps) break;  // the same for every wave of the workgroup
      __syncthreads();  // block bi in its buffer for all; the other buffer free
      gather_kv_lds<TW>(kr, vr, pos + 32 * (bi + R), gw, stg[u]);
      if (active && 32 * bi < cnt) attn_block<NB>(Q, lds + (u & 1) * kBlkLds, pos[32 * bi + c], n_k, sl2, vt_off, st);
      store_kv<TW>(stg[(u + 1) % R], lds + ((u + 1) & 1) * kBlkLds, gw);
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

  // ---- S^T = K * Q^T (A operand: key row c, dims g*64 + 8j from LDS). With
  // 64 heads per wave (one wave per SIMD, registers to spare) every operand
  // read of the block is issued before the products that consume it, so LDS
  // latency is paid once per block rather than once per fragment.
  v16f S[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) S[nb] = v16f{};
  constexpr bool kAhead = NB == 2;
  v8bf Ka[8];
  if constexpr (kAhead) {
#pragma unroll
    for (int j = 0; j < 8; ++j) Ka[j] = *(const v8bf*)(blk + c * kKRow + g * 128 + 16 * j);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (!kAhead) Ka[j] = *(const v8bf*)(blk + c * kKRow + g * 128 + 16 * j);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) S[nb] = mfma_bf16_32x32x16(Ka[j], Q[nb][j], S[nb]);
  }
  if constexpr (kAhead) {
    // keep the eight K reads ahead of the sixteen products in the schedule
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  }
  v8bf Va[4][2];
  if constexpr (kAhead) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int js = 0; js < 2; ++js) Va[mb][js] = read_vt(blk, vt_off, mb, js);
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
      mx[nb] = xor32_max(m) * sl2;
      need = need || mx[nb] > st.m[nb] + kSlack;
    }
    if (__any(need)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mnew = mx[nb] > st.m[nb] + kSlack ? mx[nb] : st.m[nb];
        // 0 when st.m is -inf; 1 when the reference stays (also -inf - -inf)
        const float alpha = mnew == st.m[nb] ? 1.f : __builtin_amdgcn_exp2f(st.m[nb] - mnew);
        st.l[nb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st.o[mb][nb] *= alpha;
        st.m[nb] = mnew;
      }
    }
    // p = 2^(S*sl2 - m) (exp2 of -inf is 0); l sums p in fp32, and P is
    // rounded to bf16 for the PV product. A block whose keys are all masked
    // while nothing has been seen yet (m still -inf) adds zeros: the
    // reference is taken as 0 there, not +inf (which would make -inf + inf).
    v8bf P[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float nm = st.m[nb] == -INFINITY ? 0.f : -st.m[nb];
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
        if constexpr (!kAhead) Va[mb][js] = read_vt(blk, vt_off, mb, js);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) st.o[mb][nb] = mfma_bf16_32x32x16(Va[mb][js], P[nb][js], st.o[mb][nb]);
      }
    }
}

// ------------------------------------------------------------------ decode
// Partials: ws_m / ws_l [B, n_split, R] fp32, ws_o [B, n_split, R, 128] fp16
// with R = n_q * H; o is the part's output normalised by its own l, m in
// base-2 units.
//
// Decode runs 32 heads per wave (a row group: one query row x 32 heads), so
// that a wave needs at most 256 registers and two waves share each SIMD:
// one wave's MFMAs then overlap the other's softmax. A workgroup of W = TW *
// KS waves takes one part of one index row; wave w has row group w % TW of
// the workgroup's TW and key subrange w / TW of the part's KS. The TW waves
// of a subrange need the same K/V rows, so they gather each 32-key block
// together into one shared LDS buffer pair (one request per row instead of
// one per wave). With KS > 1 the subrange states of a row group are combined
// through LDS in a fixed binary tree before the part's partial is written.

// (x0 + x1) or (x0 + x1) + (x2 + x3)
template <int N>
__device__ __forceinline__ float tree_sum(const float (&x)[N]) {
  static_assert(N == 2 || N == 4, "two or four subranges");
  if constexpr (N == 2) return x[0] + x[1];
  else return (x[0] + x[1]) + (x[2] + x[3]);
}

template <int NB>
__device__ __forceinline__ void store_partial(const AttnState<NB>& st, const DecodeArgs& a, int64_t rbase, int h0,
                                              int mb_lo, int mb_hi, bool ml) {
  const int l = lane_id(), g = l >> 5, c = l & 31;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int h = h0 + 32 * nb + c;
    if (h >= a.H) continue;
    const int64_t row = rbase + h;
    if (ml && g == 0) {
      a.ws_m[row] = st.m[nb];
      a.ws_l[row] = st.l[nb];
    }
    // the part's output normalised by its own sum (so each value is a convex
    // combination of V entries), in fp16 rounded to nearest (11 significant
    // bits: a quarter of a bf16 output's rounding); the merge weighs it by
    // l * 2^(m - M)
    const float inv = st.l[nb] > 0.f ? 1.f / st.l[nb] : 0.f;
    _Float16* orow = a.ws_o + row * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < mb_lo || mb >= mb_hi) continue;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v16f& O = st.o[mb][nb];
        *(v4h*)(orow + 32 * mb + 8 * i4 + 4 * g) =
            v4h{(_Float16)(O[4 * i4] * inv), (_Float16)(O[4 * i4 + 1] * inv), (_Float16)(O[4 * i4 + 2] * inv),
                (_Float16)(O[4 * i4 + 3] * inv)};
      }
    }
  }
}

template <int TW, int KS>
struct DecodeCfg {
  static constexpr int W = TW * KS;                        // waves per workgroup
  static constexpr int R = TW >= 8 ? 6 : TW >= 4 ? 4 : 2;  // register stages of 64 / TW VGPRs
  static constexpr int kCap = KS >= 4 ? 512 : 2048;        // positions per chunk
  static constexpr int kPosN = kCap + 64 * R;              // with the -1 tail the pipeline reads
  static constexpr int kKvOnly = KS * 2 * kBlkLds;
  static constexpr int kKv = kKvOnly + KS * kPosN * 4;
  // subrange states: per wave, o as [mb][i][lane] and m, l as [lane]
  static constexpr int kStO = 4 * 16 * 64 * 4;
  static constexpr int kStW = kStO + 2 * 64 * 4;
  static constexpr int kSt = KS > 1 ? W * kStW : 0;
  static constexpr int kBytes = kKv > kSt ? kKv : kSt;
  static_assert(kBytes <= 160 * 1024, "LDS");
};

// One workgroup of TW * KS waves: row groups bx * TW .. bx * TW + TW - 1 (of
// n_q * H / 32), part `split` of sequence b; lds_all holds
// DecodeCfg<TW, KS>::kBytes.
template <int TW, int KS>
__device__ __forceinline__ void decode_partial_body(const DecodeArgs& a, int bx, int split, int b, char* lds_all) {
  using Cfg = DecodeCfg<TW, KS>;
  constexpr int NB = 1;
  const int wv = wave_id(), gw = wv % TW, sr = wv / TW;
  const int HB = (a.H + 31) / 32;
  const int T = a.n_q * HB;
  const int t = bx * TW + gw;
  const bool active = t < T;
  const int qr = active ? t / HB : 0, hb = active ? t % HB : 0;
  const int l = lane_id();
  const int R = a.n_q * a.H;
  v8bf Q[NB][8];
  if (active) load_q<NB>(a.q + ((int64_t)b * a.n_q + qr) * a.H * kD, hb * 32, a.H, Q);
  AttnState<NB> st;
  attn_init(st);
  // every row group of a workgroup reads the same index row
  const int irow = a.n_idx == 1 ? 0 : (bx * TW) / HB;
  const int64_t ibase = (int64_t)b * a.n_idx + irow;
  const int n = min(max(a.n_sel[ibase], 0), a.K_tot);
  const int cs = (n + a.n_split - 1) / a.n_split;
  const int kb = min(n, split * cs), ke = min(n, (split + 1) * cs);
  const int nblk = (ke - kb + 31) / 32;
  const int bps = (nblk + KS - 1) / KS;
  const int sb = min(ke, kb + 32 * bps * sr), se = min(ke, sb + 32 * bps);
  const uint16_t* K = a.k + (int64_t)b * a.n_k * kD;
  const uint16_t* V = a.v + (int64_t)b * a.n_k * kD;
  // positions go to LDS a chunk at a time (one chunk for parts up to kCap
  // keys); chunk and trip counts derive from bps alone, so every wave meets
  // the same barriers
  constexpr int kR = Cfg::R;
  int* posg = (int*)(lds_all + Cfg::kKvOnly) + sr * Cfg::kPosN;
  const int32_t* ids = a.idx + ibase * a.K_tot;
  const int span = 32 * bps;
  const int gt = 64 * gw + l;
  for (int ch = 0; ch * Cfg::kCap < span; ++ch) {
    const int cb = sb + ch * Cfg::kCap;
    const int cnt = min(max(se - cb, 0), Cfg::kCap);
    const int tr = (min(Cfg::kCap, span - ch * Cfg::kCap) / 32 + kR - 1) / kR * kR;
    if (ch > 0) __syncthreads();  // the previous chunk's positions and buffers no longer read
    for (int i = gt; i < Cfg::kPosN; i += 64 * TW) posg[i] = i < cnt ? ids[cb + i] : -1;
    __syncthreads();
    attn_keys_lds<NB, TW, kR>(Q, active, K, V, posg, cnt, tr, min(Cfg::kCap, span - ch * Cfg::kCap), a.n_k, a.sl2,
                              gw, st, lds_all + sr * 2 * kBlkLds);
  }
  if (a.tgt_pos != nullptr && split == a.n_split - 1) {
    // MTP rows with causal tails: the last part also holds the positions
    // tgt + 1 .. tgt + n_q - 1 (the drafts' keys); row qr sees the first qr
    // of them. One block, gathered by the first subrange's waves.
    const int tgt = a.tgt_pos[b];
    const int l2 = lane_id(), G = l2 >> 4, jj = l2 & 15;
    const int vt_off = kVOff + (4 * (G >> 1) + (jj >> 2)) * kVRow + (16 * (G & 1) + 4 * (jj & 3)) * 2;
    const int p = c_lane() < a.n_q - 1 ? tgt + 1 + c_lane() : -1;
    __syncthreads();  // every wave is done with its buffers
    if (sr == 0) {
      KVStage<TW> stg;
      gather_kv<TW>(cache_rsrc(K, a.n_k), cache_rsrc(V, a.n_k), p, gw, stg);
      store_kv<TW>(stg, lds_all, gw);
    }
    __syncthreads();
    if (sr == 0 && active)
      attn_block<NB>(Q, lds_all, c_lane() < qr ? p : -1, a.n_k, a.sl2, vt_off, st);
  }
  st.l[0] += shfl_xor_f(st.l[0], 32);  // both key halves
  const int64_t rbase = ((int64_t)b * a.n_split + split) * R + (int64_t)qr * a.H;
  if constexpr (KS == 1) {
    if (active) store_partial<NB>(st, a, rbase, hb * 32, 0, 4, true);
  } else {
    // combine the KS subrange states of each row group; wave sr of the row
    // group then owns the dim blocks [sr * 4 / KS, (sr + 1) * 4 / KS)
    __syncthreads();  // K/V buffers no longer read
    float* so = (float*)(lds_all + wv * Cfg::kStW);
    float* sm = (float*)(lds_all + wv * Cfg::kStW + Cfg::kStO);
    sm[l] = st.m[0];
    sm[64 + l] = st.l[0];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) so[(mb * 16 + i) * 64 + l] = st.o[mb][0][i];
    __syncthreads();
    float ms[KS], ws[KS], ls[KS];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float* smw = (const float*)(lds_all + (s * TW + gw) * Cfg::kStW + Cfg::kStO);
      ms[s] = smw[l];
      ls[s] = smw[64 + l];
      M = fmaxf(M, ms[s]);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      ws[s] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
      ls[s] *= ws[s];
    }
    st.m[0] = M;
    st.l[0] = tree_sum<KS>(ls);
    constexpr int MBW = 4 / KS;  // dim blocks per wave
    const int mb_lo = sr * MBW;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < mb_lo || mb >= mb_lo + MBW) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float os[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const float* sow = (const float*)(lds_all + (s * TW + gw) * Cfg::kStW);
          os[s] = ws[s] * sow[(mb * 16 + i) * 64 + l];
        }
        st.o[mb][0][i] = tree_sum<KS>(os);
      }
    }
    if (active) store_partial<NB>(st, a, rbase, hb * 32, mb_lo, mb_lo + MBW, sr == 0);
  }
}

// One row per 16 threads, 8 output dims per thread. Weighted sums over the
// NS >= n_split leaves (absent parts are exact zeros) use a fixed binary
// tree; for NS up to 64 the leaves beyond the next power of two above
// n_split add exact zeros only, so every NS gives the same result.
// Merge of row brow (of B * n_q * H), dims d .. d + 7.
template <int NS>
__device__ __forceinline__ void decode_merge_row(const DecodeArgs& a, int64_t brow, int d) {
  // products and sums each rounded to fp32 (no fused multiply-add), so the
  // result is set by the tree alone
#pragma clang fp contract(off)
  const int R = a.n_q * a.H;
  const int b = (int)(brow / R), r = (int)(brow % R);
  const int64_t row0 = (int64_t)b * a.n_split * R + r;
  const float* pm = a.ws_m + row0;
  const float* pl = a.ws_l + row0;
  const _Float16* po = a.ws_o + row0 * kD + d;
  float mj[NS], lv[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bool in = j < a.n_split;
    const int jr = in ? j * R : 0;
    mj[j] = in ? pm[jr] : -INFINITY;
    lv[j] = in ? pl[jr] : 0.f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < NS; ++j) M = fmaxf(M, mj[j]);
  // each part's normalised output weighed by l * 2^(m - M), summed in a
  // fixed binary tree in fp32 (pairs of parts, then pairs of pairs, ...).
  // The tree is evaluated part by part, keeping one pending subtree sum per
  // level: part j closes the subtrees of the levels where j has a one bit.
  constexpr int LG = NS <= 1 ? 0 : NS <= 2 ? 1 : NS <= 4 ? 2 : NS <= 8 ? 3 : NS <= 16 ? 4 : NS <= 32 ? 5 : 6;
  static_assert((1 << LG) == NS, "NS is a power of two up to 64");
  float sl[LG + 1], so[LG + 1][8];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bool in = j < a.n_split;
    const v8h ov = in ? *(const v8h*)(po + (int64_t)j * R * kD) : v8h{};
    const float wj = (in && M != -INFINITY) ? __builtin_amdgcn_exp2f(mj[j] - M) : 0.f;
    float cl = lv[j] * wj, co[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) co[e] = (float)ov[e] * cl;
    int lvl = 0;
#pragma unroll
    for (; lvl < LG && ((j >> lvl) & 1); ++lvl) {
      cl = sl[lvl] + cl;
#pragma unroll
      for (int e = 0; e < 8; ++e) co[e] = so[lvl][e] + co[e];
    }
    sl[lvl] = cl;
#pragma unroll
    for (int e = 0; e < 8; ++e) so[lvl][e] = co[e];
  }
  const float Lam = sl[LG];
  const float inv = Lam > 0.f ? 1.f / Lam : 0.f;
  v4u out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(so[LG][2 * e] * inv, so[LG][2 * e + 1] * inv);
  *(v4u*)(a.o + brow * kD + d) = out;
  if (a.lse && d == 0) a.lse[brow] = Lam > 0.f ? (M + log2f(Lam)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace lsa
