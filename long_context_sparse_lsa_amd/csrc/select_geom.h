// Row geometry of the selection kernels: which candidates a row of a
// selection launch has and how many it keeps, and the cache position of a
// candidate. Host-callable too, so the host tests can check it in every mode.
#pragma once
#include "lsa_internal.h"

namespace lsa {

struct RowGeom {
  int trivial;
  int t;
  int c_lo, nc;
  int k;
};

__host__ __device__ inline RowGeom row_geom(const SelectArgs& a, int r) {
  RowGeom gm{0, 0, 0, 0, 0};
  if (a.mode == SEL_FLAT) {
    const int t = a.q_off + (a.row0 + r) % a.n_q + seq_shift(a.shift, (a.row0 + r) / a.n_q);
    gm.t = t;
    if (t + 1 <= a.n_sink + a.n_window + a.k_dyn) {
      gm.trivial = 1;
      return gm;
    }
    gm.c_lo = a.n_sink;
    gm.nc = t - a.n_window - a.n_sink + 1;
    gm.k = a.k_dyn;
  } else if (a.mode == SEL_RAW) {
    int hi = a.raw_hi;
    if (a.shift.ctx_len != nullptr) {
      const int hp = a.raw_hi_pos + seq_shift(a.shift, a.row0 + r);
      hi = min(hp >= 0 ? hp / a.raw_div : -1, a.raw_hi);
    }
    gm.c_lo = a.raw_lo;
    gm.nc = max(0, hi - a.raw_lo + 1);
    gm.k = a.raw_k;
  } else {
    gm.t = a.t_fixed;
    gm.c_lo = 0;
    gm.nc = a.n_virt;
    gm.k = a.k_dyn;
    if (a.shift.ctx_len != nullptr) {
      gm.t += seq_shift(a.shift, a.row0 + r);
      gm.trivial = gm.t + 1 <= a.n_sink + a.n_window + a.k_dyn;
    }
  }
  return gm;
}

__host__ __device__ inline int pos_of(const SelectArgs& a, int r, int v) {
  if (a.mode != SEL_INDIRECT) return v;
  const int bi = a.blocks[(int64_t)r * a.nbr + v / a.blk];
  return bi * a.blk + v % a.blk;
}

}  // namespace lsa
