// Per-row key lists of an MTP decode step whose draft rows also see the drafts
// before them (gfx950).
//
// The CLI paragraph of the LongCat-2.0 release article (section "LongCat 稀疏注
// 意力") has the three MTP draft steps reuse the target's index. When the
// drafts' keys and values are already appended to the cache, draft j (at
// position tgt + j) may also attend to positions tgt + 1 .. tgt + j. Row j's
// list is the target's selected list (positions <= tgt, ascending) followed by
// those positions, so it stays ascending; row 0 is the target's list itself.
//
// One workgroup per (row, sequence) copies the list and writes the tail and
// the -1 padding.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

__global__ __launch_bounds__(256) void mtp_index_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ n_sel, int K_tot, int n_q,
                                                        const int32_t* __restrict__ tgt_pos,
                                                        int32_t* __restrict__ idx_rows,
                                                        int32_t* __restrict__ n_sel_rows) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int K2 = K_tot + n_q - 1;
  const int n = min(max(n_sel[b], 0), K_tot);
  const int tgt = tgt_pos[b];
  const int32_t* src = idx + (int64_t)b * K_tot;
  int32_t* dst = idx_rows + ((int64_t)b * n_q + j) * K2;
  for (int i = threadIdx.x; i < K2; i += 256) {
    int v;
    if (i < n) v = src[i];
    else if (i < n + j) v = tgt + 1 + (i - n);
    else v = -1;
    dst[i] = v;
  }
  if (threadIdx.x == 0) n_sel_rows[(int64_t)b * n_q + j] = n + j;
}

hipError_t launch_mtp_index(const int32_t* idx, const int32_t* n_sel, int B, int K_tot, int n_q,
                            const int32_t* tgt_pos, int32_t* idx_rows, int32_t* n_sel_rows, hipStream_t st) {
  KernelTimer kt("mtp_index_kernel", st);
  hipLaunchKernelGGL(mtp_index_kernel, dim3(n_q, B), dim3(256), 0, st, idx, n_sel, K_tot, n_q, tgt_pos, idx_rows,
                     n_sel_rows);
  return hipGetLastError();
}

}  // namespace lsa
