// Peak-rate probe of the matrix cores (a measurement aid, not part of the
// method): every wave issues independent chains of one MFMA instruction on
// register operands, with no memory traffic in the loop, so the launch's
// duration gives the rate the chip sustains for that instruction at its
// current clock. The indexer and attention kernels are measured against it
// next to the published peaks.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int kChains = 8;  // independent accumulators per wave

// kind 0: v_mfma_i32_32x32x32_i8 (65536 int8 ops each);
// kind 1: v_mfma_f32_32x32x16_bf16 (32768 flop each)
template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, int* sink) {
  const int l = lane_id();
  int acc_sum = 0;
  if constexpr (KIND == 0) {
    const v4i a = v4i{l, l + 1, l + 2, l + 3};
    const v4i b = v4i{3 * l, l ^ 5, l + 7, 11};
    v16i acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = v16i{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < kChains; ++j) acc[j] = mfma_i8_32x32x32(a, b, acc[j]);
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_sum += acc[j][e];
  } else {
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)(l + e);
      b[e] = (__bf16)(float)(e - l);
    }
    v16f acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = v16f{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < kChains; ++j) acc[j] = mfma_bf16_32x32x16(a, b, acc[j]);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
    acc_sum = (int)s;
  }
  // keeps the products live; the sink holds one int per workgroup
  if (threadIdx.x == 0) sink[blockIdx.x] = acc_sum;
}

// The same chains with operands taken from caller data: each lane loads 8
// A and 8 B fragments (16 bytes each) from the given arrays, and chain j
// multiplies A fragment j by B fragment j + 1, so consecutive instructions
// see different operands drawn from the data's value distribution. The
// matrix cores' power draw, and with it the clock the chip holds, depends on
// how many operand bits switch from one instruction to the next: this rate is
// the ceiling for kernels that multiply such data.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_data_kernel(int iters, const uint4* a_src, int64_t a_n,
                                                              const uint4* b_src, int64_t b_n, int* sink) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 ua[kChains], ub[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    ua[j] = a_src[(t * kChains + j) % a_n];
    ub[j] = b_src[(t * kChains + j + 3) % b_n];
  }
  int acc_sum = 0;
  if constexpr (KIND == 0) {
    v16i acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = v16i{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        acc[j] = mfma_i8_32x32x32(__builtin_bit_cast(v4i, ua[j]), __builtin_bit_cast(v4i, ub[(j + 1) % kChains]),
                                  acc[j]);
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_sum += acc[j][e];
  } else {
    v16f acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = v16f{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        acc[j] = mfma_bf16_32x32x16(__builtin_bit_cast(v8bf, ua[j]), __builtin_bit_cast(v8bf, ub[(j + 1) % kChains]),
                                    acc[j]);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
    acc_sum = (int)s;
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = acc_sum;
}

}  // namespace

}  // namespace lsa

extern "C" int32_t lsa_probe_mfma(int32_t kind, int32_t n_wg, int32_t iters, int32_t* sink, double* ops,
                                  void* stream) {
  if (sink == nullptr || ((uintptr_t)sink & 3u) != 0 || n_wg <= 0 || iters <= 0) return LSA_INVALID_ARG;
  if (kind != 0 && kind != 1) return LSA_UNSUPPORTED;
  const double per = kind == 0 ? 65536.0 : 32768.0;
  if (ops) *ops = per * lsa::kChains * (double)iters * 4.0 * n_wg;  // 4 waves per workgroup
  hipStream_t st = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL(lsa::mfma_probe_kernel<0>, dim3(n_wg), dim3(256), 0, st, iters, sink);
  else hipLaunchKernelGGL(lsa::mfma_probe_kernel<1>, dim3(n_wg), dim3(256), 0, st, iters, sink);
  return hipGetLastError() == hipSuccess ? LSA_OK : LSA_HIP;
}

extern "C" int32_t lsa_probe_mfma_data(int32_t kind, int32_t n_wg, int32_t iters, const void* a, int64_t a_bytes,
                                       const void* b, int64_t b_bytes, int32_t* sink, double* ops, void* stream) {
  if (sink == nullptr || ((uintptr_t)sink & 3u) != 0 || n_wg <= 0 || iters <= 0) return LSA_INVALID_ARG;
  if (a == nullptr || b == nullptr || ((uintptr_t)a & 15u) != 0 || ((uintptr_t)b & 15u) != 0 || a_bytes < 16 ||
      b_bytes < 16)
    return LSA_INVALID_ARG;
  if (kind != 0 && kind != 1) return LSA_UNSUPPORTED;
  const double per = kind == 0 ? 65536.0 : 32768.0;
  if (ops) *ops = per * lsa::kChains * (double)iters * 4.0 * n_wg;
  hipStream_t st = (hipStream_t)stream;
  const uint4* pa = (const uint4*)a;
  const uint4* pb = (const uint4*)b;
  if (kind == 0)
    hipLaunchKernelGGL(lsa::mfma_probe_data_kernel<0>, dim3(n_wg), dim3(256), 0, st, iters, pa, a_bytes / 16, pb,
                       b_bytes / 16, sink);
  else
    hipLaunchKernelGGL(lsa::mfma_probe_data_kernel<1>, dim3(n_wg), dim3(256), 0, st, iters, pa, a_bytes / 16, pb,
                       b_bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? LSA_OK : LSA_HIP;
}
