// C ABI of the training-side LSA operators: the deterministic sparse
// attention backward and the warm-up KL operator. Argument checks run before
// the first launch; workspace comes from the caller.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "lsa.h"
#include "lsa_internal.h"

using namespace lsa;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool al16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }
int32_t hip_status(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_HIP; }

}  // namespace

// Bytes of (row, slot) contributions one backward chunk may hold.
constexpr size_t kContribCap = (size_t)8 << 30;

extern "C" int32_t lsa_sparse_attn_backward(const lsa_bf16* q, const lsa_bf16* k, const lsa_bf16* v,
                                            const int32_t* idx, const int32_t* n_sel, const lsa_bf16* o,
                                            const float* lse, const lsa_bf16* d_o, int32_t B, int32_t L,
                                            int32_t n_k, int32_t H, int32_t D, int32_t K_tot, float scale,
                                            lsa_bf16* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                            size_t* ws_needed, void* stream) {
  if (B <= 0 || L <= 0 || n_k <= 0 || K_tot <= 0 || !(scale > 0.f) || !isfinite(scale)) return LSA_INVALID_ARG;
  if (D != 128 || (H != 32 && H != 64 && H != 128) || n_k > kMaxCacheKeys) return LSA_UNSUPPORTED;
  const int64_t n_keys = (int64_t)B * n_k;
  if (n_keys > kMaxScanKeys || K_tot > (1 << 20)) return LSA_UNSUPPORTED;
  // rows per chunk: contributions of 512 bytes per (row, slot) within
  // kContribCap, pair ids within int32
  const int64_t rows = (int64_t)B * L;
  const int64_t rc = std::max<int64_t>(
      1, std::min<int64_t>({rows, (int64_t)(kContribCap / ((size_t)K_tot * 512)), (int64_t)INT32_MAX / K_tot}));
  const size_t n_acc = (size_t)n_keys * 128;
  const size_t n_pairs = (size_t)rc * K_tot;
  const size_t sz_acc = align_up(n_acc * sizeof(int64_t));
  const size_t sz_contrib = align_up(n_pairs * 512);
  const size_t sz_keys = align_up((size_t)n_keys * sizeof(int32_t));
  const size_t sz_tot = align_up((size_t)(n_keys + kScanBlock - 1) / kScanBlock * sizeof(int32_t));
  const size_t sz_list = align_up(n_pairs * sizeof(int32_t));
  const size_t need = 2 * sz_acc + sz_contrib + 2 * sz_keys + sz_tot + 2 * sz_list;
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al16(q) || !al16(k) || !al16(v) || !al4(idx) || !al4(n_sel) || !al16(o) || !al4(lse) || !al16(d_o) ||
      !al16(dq) || !al16(dk) || !al16(dv) || !al16(ws))
    return LSA_INVALID_ARG;
  if (ws_bytes < need) return LSA_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* p = (char*)ws;
  BwdArgs a{};
  ScatterArgs sa{};
  sa.dk_acc = (int64_t*)p;
  p += sz_acc;
  sa.dv_acc = (int64_t*)p;
  p += sz_acc;
  a.contrib = (uint16_t*)p;
  p += sz_contrib;
  sa.cnt = (int32_t*)p;
  p += sz_keys;
  sa.cur = (int32_t*)p;
  p += sz_keys;
  sa.tot = (int32_t*)p;
  p += sz_tot;
  sa.lkey = (int32_t*)p;
  p += sz_list;
  sa.lpair = (int32_t*)p;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.d_o = d_o;
  a.lse = lse;
  a.idx = idx;
  a.n_sel = n_sel;
  a.B = B;
  a.L = L;
  a.n_k = n_k;
  a.H = H;
  a.K_tot = K_tot;
  a.scale = scale;
  a.sl2 = scale * 1.4426950408889634f;
  a.dq = dq;
  sa.idx = idx;
  sa.n_sel = n_sel;
  sa.L = L;
  sa.n_k = n_k;
  sa.K_tot = K_tot;
  sa.n_keys = (int)n_keys;
  sa.contrib = a.contrib;
  int32_t s = hip_status(launch_fill_zero(sa.dk_acc, 2 * sz_acc, st));
  if (s != LSA_OK) return s;
  for (int64_t r0 = 0; r0 < rows; r0 += rc) {
    a.r0 = sa.r0 = r0;
    a.r1 = sa.r1 = std::min(rows, r0 + rc);
    s = hip_status(launch_attn_bwd(a, st));
    if (s != LSA_OK) return s;
    s = hip_status(launch_bwd_scatter(sa, st));
    if (s != LSA_OK) return s;
  }
  s = hip_status(launch_attn_bwd_finish(sa.dk_acc, dk, n_acc, st));
  if (s != LSA_OK) return s;
  return hip_status(launch_attn_bwd_finish(sa.dv_acc, dv, n_acc, st));
}

extern "C" int32_t lsa_kl_warmup(const lsa_bf16* q, const lsa_bf16* k, const int32_t* idx, const int32_t* n_sel,
                                 const float* lse, const float* logits, int32_t B, int32_t L, int32_t n_k,
                                 int32_t H, int32_t D, int32_t K_tot, float scale, float* kl, float* dlogits,
                                 void* stream) {
  if (!al16(q) || !al16(k) || !al4(idx) || !al4(n_sel) || !al4(lse) || !al4(logits) || !al4(kl) ||
      !al4(dlogits))
    return LSA_INVALID_ARG;
  if (B <= 0 || L <= 0 || n_k <= 0 || K_tot <= 0 || !(scale > 0.f) || !isfinite(scale)) return LSA_INVALID_ARG;
  if (D != 128 || (H != 32 && H != 64 && H != 128) || n_k > kMaxCacheKeys) return LSA_UNSUPPORTED;
  KlArgs a{};
  a.q = q;
  a.k = k;
  a.lse = lse;
  a.idx = idx;
  a.n_sel = n_sel;
  a.logits = logits;
  a.B = B;
  a.L = L;
  a.n_k = n_k;
  a.H = H;
  a.K_tot = K_tot;
  a.sl2 = scale * 1.4426950408889634f;
  a.kl = kl;
  a.dlogits = dlogits;
  return hip_status(launch_kl_warmup(a, (hipStream_t)stream));
}
