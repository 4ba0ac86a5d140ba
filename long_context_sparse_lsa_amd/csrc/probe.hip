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
