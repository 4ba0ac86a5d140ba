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

extern "C" int32_t lsa_sparse_attn_backward(const lsa_bf16* q, const lsa_bf16* k, const lsa_bf16* v,
                                            const int32_t* idx, const int32_t* n_sel, const lsa_bf16* o,
                                            const float* lse, const lsa_bf16* d_o, int32_t B, int32_t L,
                                            int32_t n_k, int32_t H, int32_t D, int32_t K_tot, float scale,
                                            lsa_bf16* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                            size_t* ws_needed, void* stream) {
  if (B <= 0 || L <= 0 || n_k <= 0 || K_tot <= 0 || !(scale > 0.f) || !isfinite(scale)) return LSA_INVALID_ARG;
  if (D != 128 || (H != 32 && H != 64 && H != 128) || n_k > kMaxCacheKeys) return LSA_UNSUPPORTED;
  const size_t n_acc = (size_t)B * n_k * 128;
  const size_t need = 2 * align_up(n_acc * sizeof(int64_t));
  if (ws_needed) *ws_needed = need;
  if (ws == nullptr) return ws_needed ? LSA_OK : LSA_WORKSPACE;  // size query
  if (!al16(q) || !al16(k) || !al16(v) || !al4(idx) || !al4(n_sel) || !al16(o) || !al4(lse) || !al16(d_o) ||
      !al16(dq) || !al16(dk) || !al16(dv) || !al16(ws))
    return LSA_INVALID_ARG;
  if (ws_bytes < need) return LSA_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  BwdArgs a{};
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
  a.dk_acc = (int64_t*)ws;
  a.dv_acc = (int64_t*)((char*)ws + align_up(n_acc * sizeof(int64_t)));
  int32_t s = hip_status(launch_fill_zero(ws, need, st));
  if (s != LSA_OK) return s;
  s = hip_status(launch_attn_bwd(a, st));
  if (s != LSA_OK) return s;
  s = hip_status(launch_attn_bwd_finish(a.dk_acc, dk, n_acc, st));
  if (s != LSA_OK) return s;
  return hip_status(launch_attn_bwd_finish(a.dv_acc, dv, n_acc, st));
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
