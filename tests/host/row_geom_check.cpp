// Host check of the selection row geometry (select_geom.h) in every mode:
// its result equals a form that returns as soon as a row is known to keep
// every key, field by field, on random launches with and without per-sequence
// lengths; the candidate ranges it gives stay inside the row's visible keys;
// and pos_of maps every candidate of a recalled block into the cache.
// Prints "ok <cases>" and exits 0, or names the first difference and exits 1.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "select_geom.h"

using namespace lsa;

// The same geometry written with early returns.
static RowGeom geom_early(const SelectArgs& a, int r) {
  RowGeom gm{0, 0, 0, 0, 0};
  const int K_tot = a.n_sink + a.n_window + a.k_dyn;
  if (a.mode == SEL_FLAT) {
    gm.t = a.q_off + (a.row0 + r) % a.n_q + seq_shift(a.shift, (a.row0 + r) / a.n_q);
    if (gm.t + 1 <= K_tot) {
      gm.trivial = 1;
      return gm;
    }
    gm.c_lo = a.n_sink;
    gm.nc = gm.t - a.n_window - a.n_sink + 1;
    gm.k = a.k_dyn;
    return gm;
  }
  if (a.mode == SEL_RAW) {
    int hi = a.raw_hi;
    if (a.shift.ctx_len != nullptr) {
      const int hp = a.raw_hi_pos + seq_shift(a.shift, a.row0 + r);
      hi = hp >= 0 ? hp / a.raw_div : -1;
      if (hi > a.raw_hi) hi = a.raw_hi;
    }
    gm.c_lo = a.raw_lo;
    gm.nc = hi - a.raw_lo + 1 > 0 ? hi - a.raw_lo + 1 : 0;
    gm.k = a.raw_k;
    return gm;
  }
  gm.t = a.t_fixed;
  if (a.shift.ctx_len != nullptr) {
    gm.t += seq_shift(a.shift, a.row0 + r);
    if (gm.t + 1 <= K_tot) {
      gm.trivial = 1;
      gm.c_lo = 0;
      gm.nc = a.n_virt;
      gm.k = a.k_dyn;
      return gm;
    }
  }
  gm.c_lo = 0;
  gm.nc = a.n_virt;
  gm.k = a.k_dyn;
  return gm;
}

static bool same(const RowGeom& x, const RowGeom& y) {
  return x.trivial == y.trivial && x.t == y.t && x.c_lo == y.c_lo && x.nc == y.nc && x.k == y.k;
}

int main() {
  std::mt19937_64 rng(2026);
  auto U = [&](int lo, int hi) { return (int)(lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1))); };
  long cases = 0;
  for (int trial = 0; trial < 20000; ++trial) {
    SelectArgs a{};
    a.mode = trial % 3;
    a.n_sink = U(0, 8);
    a.n_window = U(0, 600);
    a.k_dyn = U(0, 3000);
    const int K_tot = a.n_sink + a.n_window + a.k_dyn;
    const int n_k = U(1, 1 << 20);
    const int B = U(1, 6);
    a.n_q = U(1, 4);
    a.n_rows = B * a.n_q;
    a.row0 = 0;
    std::vector<int32_t> ctx(B);
    for (int b = 0; b < B; ++b) ctx[b] = U(-5, n_k + 100);
    const bool ragged = rng() & 1;
    a.shift = SeqShift{ragged ? ctx.data() : nullptr, a.mode == SEL_FLAT ? a.n_q : 1, n_k};
    if (a.mode == SEL_FLAT) {
      a.q_off = n_k - a.n_q;
      if (a.q_off < 0) continue;
    } else if (a.mode == SEL_RAW) {
      a.n_rows = B;
      a.raw_div = 32 * U(1, 32);
      a.raw_lo = U(0, 4);
      a.raw_hi_pos = n_k - 1 - a.n_window;
      a.raw_hi = a.raw_hi_pos >= 0 ? a.raw_hi_pos / a.raw_div : -1;
      a.raw_k = U(1, 300);
    } else {
      a.n_rows = B;
      a.blk = 32 * U(1, 32);
      a.nbr = U(1, 64);
      a.n_virt = a.nbr * a.blk;
      a.t_fixed = n_k - 1;
    }
    for (int r = 0; r < a.n_rows; ++r) {
      const RowGeom g = row_geom(a, r), e = geom_early(a, r);
      ++cases;
      if (!same(g, e)) {
        std::printf("differs: mode %d trial %d row %d: trivial %d/%d t %d/%d c_lo %d/%d nc %d/%d k %d/%d\n", a.mode,
                    trial, r, g.trivial, e.trivial, g.t, e.t, g.c_lo, e.c_lo, g.nc, e.nc, g.k, e.k);
        return 1;
      }
      if (a.mode == SEL_FLAT && !g.trivial) {
        // candidates n_sink .. t - W inside the row's visible keys 0 .. t < n_k
        const int L = ragged ? std::min(std::max(ctx[r / a.n_q], a.n_q), n_k) : n_k;
        if (g.t != L - a.n_q + r % a.n_q || g.c_lo + g.nc - 1 != g.t - a.n_window || g.t >= n_k || g.nc < 1 ||
            g.t + 1 <= K_tot) {
          std::printf("flat range: trial %d row %d\n", trial, r);
          return 1;
        }
      }
      if (a.mode == SEL_RAW && (g.nc < 0 || (g.nc > 0 && g.c_lo + g.nc - 1 > a.raw_hi))) {
        std::printf("raw range: trial %d row %d\n", trial, r);
        return 1;
      }
      if (a.mode == SEL_INDIRECT && !g.trivial) {
        // every virtual candidate of a recalled block maps into the cache
        std::vector<int32_t> blocks(a.n_rows * a.nbr);
        const int nblocks = (n_k + a.blk - 1) / a.blk;
        for (auto& x : blocks) x = U(0, nblocks - 1);
        a.blocks = blocks.data();
        for (int v = 0; v < g.nc; v += U(1, 97)) {
          const int p = pos_of(a, r, v);
          if (p < 0 || p >= nblocks * a.blk) {
            std::printf("pos_of: trial %d row %d v %d -> %d\n", trial, r, v, p);
            return 1;
          }
        }
        a.blocks = nullptr;
      }
    }
  }
  std::printf("ok %ld\n", cases);
  return 0;
}
