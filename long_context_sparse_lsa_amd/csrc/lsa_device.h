// Device-side helpers shared by the LSA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int32_t kMasked = INT32_MIN;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int c_lane() { return threadIdx.x & 31; }

// 32x32x32 int8 MFMA: each lane brings 16 int8 of A (row lane%32) and of B
// (column lane%32); lanes 0-31 and 32-63 bring two disjoint halves of the
// contraction. Output: lane holds column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4.
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA, fp32 accumulate, same operand/output lane layout.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// float -> bfloat16 bits, round to nearest even (inputs here are finite).
// Lane-half exchange without LDS (v_permlane32_swap_b32): lanes 0-31 get
// lo[l] + lo[l + 32] and lanes 32-63 get hi[l - 32] + hi[l], i.e. lane half
// g holds the full 64-lane pair sum of its own operand.
__device__ __forceinline__ int pair_sum32(int lo, int hi) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)lo, (unsigned)hi, false, false);
  return (int)r[0] + (int)r[1];
}
// max(v[l], v[l ^ 32]) in every lane (float), through the same lane swap.
__device__ __forceinline__ float xor32_max(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
// v[l] + v[l ^ 32] in every lane.
__device__ __forceinline__ int xor32_sum(int v) { return pair_sum32(v, v); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
  return r >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Buffer resource over `bytes` bytes at base. Base and size are wave-uniform
// at every use; readfirstlane lets the compiler keep the resource in scalar
// registers. Loads through it at offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const int nb = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, nb, 0x00020000);
}

typedef short v4s __attribute__((ext_vector_type(4)));

// Transposed MFMA operand from a row-major bf16 matrix in LDS (rows = the
// contraction index, `pitch` bytes apart; 32 columns from the start of p):
// two ds_read_b64_tr_b16 give lane (g, c) column c and the 8 contraction rows
// 4g + {0..3} and 8 + 4g + {0..3} of the 16 at p. The lane's address offset
// is tr_lane_off(pitch). This row order is the row order of a 32x32 MFMA
// accumulator's lane entries 0..7 (and, 16 rows on, 8..15), so the operand
// pairs with one taken from an accumulator in place.
__device__ __forceinline__ int tr_lane_off(int pitch) {
  const int l = lane_id(), G = l >> 4, jj = l & 15;
  return (4 * (G >> 1) + (jj >> 2)) * pitch + (16 * (G & 1) + 4 * (jj & 3)) * 2;
}
__device__ __forceinline__ v8bf read_tr(const char* p, int pitch) {
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p + 8 * pitch));
  const v4u u = v4u{__builtin_bit_cast(v2u, lo)[0], __builtin_bit_cast(v2u, lo)[1], __builtin_bit_cast(v2u, hi)[0],
                    __builtin_bit_cast(v2u, hi)[1]};
  return __builtin_bit_cast(v8bf, u);
}

// Order-preserving map of int32 scores to uint32 (INT32_MIN -> 0).
__device__ __forceinline__ uint32_t score_key(int32_t s) { return (uint32_t)s ^ 0x80000000u; }

// Inclusive prefix sum over a wave (fixed shuffle order, integer only).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (l >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

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

}  // namespace lsa
