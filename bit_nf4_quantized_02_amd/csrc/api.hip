// Host side of the C ABI declared in include/qlora.h: argument checks,
// workspace carving and kernel dispatch. Nothing here allocates, frees or
// synchronizes; every device call is enqueued on the caller's stream.
#include <cstdint>

#include "common.h"
#include "kernels.h"
#include "qlora.h"

using namespace qlora;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qlora_status hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

qlora_status check_weight(const qlora_nf4_weight* w) {
  if (w == nullptr) return QLORA_ERR_INVALID_ARG;
  if (w->n < 1 || w->k < 1 || (w->k % QLORA_BLOCK) != 0) return QLORA_ERR_SHAPE;
  if (!w->codes || !w->code8 || !w->s2 || !w->mean || !w->codebook) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(w->codes) || !aligned16(w->code8) || !aligned16(w->s2) || !aligned16(w->mean) ||
      !aligned16(w->codebook))
    return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

Nf4View view_of(const qlora_nf4_weight* w) {
  return Nf4View{w->n, w->k, w->codes, w->code8, w->s2, w->mean, w->codebook};
}

// Bump allocator over the caller's workspace (256-byte aligned regions).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t bytes) {
    if (bytes == 0) return nullptr;
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += align256(bytes);
    return p;
  }
};

bool small_m(int64_t M) { return M <= 16; }

size_t fwd_ws(int64_t M, int64_t n, int64_t k, int r, bool have_tsave, Carver* c,
              float** T, uint16_t** TS, float** part) {
  Carver local(nullptr);
  Carver& cv = c ? *c : local;
  float* t = nullptr;
  uint16_t* ts = nullptr;
  float* pt = nullptr;
  if (r > 0) {
    if (small_m(M)) {
      if (!have_tsave) t = cv.take<float>((size_t)M * r * 4);
    } else {
      ts = cv.take<uint16_t>((size_t)M * lora_extra_cols(r) * 2);
    }
    pt = cv.take<float>(rowdot_ws_bytes(M, k, r));
  }
  (void)n;
  if (T) *T = t;
  if (TS) *TS = ts;
  if (part) *part = pt;
  return cv.used;
}

struct BwdWs {
  float* T = nullptr;
  uint16_t* BT = nullptr;
  float* U = nullptr;
  uint16_t* US = nullptr;
  float* part = nullptr;
  float* colpart = nullptr;
};

size_t bwd_ws(int64_t M, int64_t n, int64_t k, int r, bool have_tsaved, Carver& cv, BwdWs& o) {
  if (r > 0) {
    if (!have_tsaved) o.T = cv.take<float>((size_t)M * r * 4);
    o.BT = cv.take<uint16_t>((size_t)n * r * 2);
    o.U = cv.take<float>((size_t)M * r * 4);
    o.US = cv.take<uint16_t>((size_t)M * lora_extra_cols(r) * 2);
    const size_t p1 = rowdot_ws_bytes(M, n, r), p2 = rowdot_ws_bytes(M, k, r);
    o.part = cv.take<float>(p1 > p2 ? p1 : p2);
    const size_t c1 = coldot_ws_bytes(M, k, r), c2 = coldot_ws_bytes(M, n, r);
    o.colpart = cv.take<float>(c1 > c2 ? c1 : c2);
  }
  return cv.used;
}

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_ERR_INVALID_ARG: return "QLORA_ERR_INVALID_ARG: NULL, misaligned or invalid argument";
    case QLORA_ERR_SHAPE: return "QLORA_ERR_SHAPE: unsupported or inconsistent shape";
    case QLORA_ERR_UNSUPPORTED: return "QLORA_ERR_UNSUPPORTED";
    case QLORA_ERR_WORKSPACE: return "QLORA_ERR_WORKSPACE: workspace too small";
    case QLORA_ERR_HIP: return "QLORA_ERR_HIP: a HIP launch or runtime call failed";
    default: return "QLORA_ERR_UNKNOWN";
  }
}

size_t qlora_nf4_packed_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 1 || k % QLORA_BLOCK) return 0;
  const int64_t nb = n * k / QLORA_BLOCK;
  const int64_t nc = (nb + QLORA_DQ_BLOCK - 1) / QLORA_DQ_BLOCK;
  return (size_t)(n * k / 2 + nb + 4 * nc + 4);
}

size_t qlora_quantize_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 1 || k % QLORA_BLOCK) return 0;
  return quantize_ws_bytes(n * k / QLORA_BLOCK);
}

qlora_status qlora_quantize_nf4(const void* W, int w_dtype, const qlora_nf4_weight* out, void* ws, size_t ws_bytes,
                                void* stream) {
  const qlora_status s = check_weight(out);
  if (s != QLORA_OK) return s;
  if (W == nullptr || !aligned16(W)) return QLORA_ERR_INVALID_ARG;
  if (w_dtype != QLORA_DT_BF16 && w_dtype != QLORA_DT_FP32) return QLORA_ERR_INVALID_ARG;
  const size_t need = qlora_quantize_workspace_bytes(out->n, out->k);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  return hip_status(launch_quantize(W, w_dtype == QLORA_DT_BF16, out->n, out->k, out->codebook, out->codes,
                                    out->code8, out->s2, out->mean, ws, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_dequant(const qlora_nf4_weight* w, void* out, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (out == nullptr || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_dequant(view_of(w), static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd) {
  if (M < 0 || n < 1 || k < 1 || k % QLORA_BLOCK || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (M == 0) return 0;
  if (!is_bwd) return fwd_ws(M, n, k, r, /*have_tsave=*/false, nullptr, nullptr, nullptr, nullptr);
  Carver cv(nullptr);
  BwdWs o;
  return bwd_ws(M, n, k, r, /*have_tsaved=*/false, cv, o);
}

qlora_status qlora_linear_fwd(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A, const void* B,
                              int r, float scale, void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream) {
  qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !aligned16(X) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if (T_save && !aligned16(T_save)) return QLORA_ERR_INVALID_ARG;
  const size_t need = fwd_ws(M, w->n, w->k, r, T_save != nullptr, nullptr, nullptr, nullptr, nullptr);
  if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  float* Tws = nullptr;
  uint16_t* TS = nullptr;
  float* part = nullptr;
  fwd_ws(M, w->n, w->k, r, T_save != nullptr, &cv, &Tws, &TS, &part);
  const Nf4View v = view_of(w);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  uint16_t* y = static_cast<uint16_t*>(Y);
  hipError_t e = hipSuccess;
  if (small_m(M)) {
    float* T = T_save ? T_save : Tws;
    if (r > 0) e = launch_rowdot_impl(x, M, w->k, a, r, T, nullptr, scale, part, st);
    if (e == hipSuccess) e = launch_gemv(v, x, M, T, b, r, scale, y, st);
  } else {
    if (r > 0) e = launch_rowdot_impl(x, M, w->k, a, r, T_save, TS, scale, part, st);
    if (e == hipSuccess) e = launch_gemm_fwd(v, x, M, TS, b, r, y, st);
  }
  return hip_status(e);
}

qlora_status qlora_linear_bwd(const qlora_nf4_weight* w, const void* X, const float* T_saved, const void* dY,
                              int64_t M, const void* A, const void* B, int r, float scale, void* dX, float* dA,
                              float* dB, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  if (!dY || !aligned16(dY)) return QLORA_ERR_INVALID_ARG;
  if (dX && !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if (r == 0) { dA = nullptr; dB = nullptr; }
  const bool need_x = (dA != nullptr) || (dB != nullptr && T_saved == nullptr);
  if (need_x && (!X || !aligned16(X))) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if ((dA && !aligned16(dA)) || (dB && !aligned16(dB)) || (T_saved && !aligned16(T_saved)))
    return QLORA_ERR_INVALID_ARG;
  Carver probe(nullptr);
  BwdWs tmp;
  const size_t need = bwd_ws(M, w->n, w->k, r, T_saved != nullptr, probe, tmp);
  if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  BwdWs o;
  bwd_ws(M, w->n, w->k, r, T_saved != nullptr, cv, o);
  const Nf4View v = view_of(w);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* dy = static_cast<const uint16_t*>(dY);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  hipError_t e = hipSuccess;
  if (r > 0 && (dX || dA)) {
    e = launch_transpose(b, w->n, r, o.BT, st);
    if (e == hipSuccess) e = launch_rowdot_impl(dy, M, w->n, o.BT, r, o.U, o.US, scale, o.part, st);
  }
  if (e == hipSuccess && dX)
    e = launch_gemm_dx(v, dy, M, r > 0 ? o.US : nullptr, a, r, static_cast<uint16_t*>(dX), st);
  if (e == hipSuccess && dA)
    e = launch_coldot(x, M, w->k, o.U, r, scale, dA, /*g_sc=*/1, /*g_sj=*/w->k, accumulate, o.colpart, st);
  if (e == hipSuccess && dB) {
    const float* T = T_saved;
    if (T == nullptr) {
      e = launch_rowdot_impl(x, M, w->k, a, r, o.T, nullptr, scale, o.part, st);
      T = o.T;
    }
    if (e == hipSuccess)
      e = launch_coldot(dy, M, w->n, T, r, scale, dB, /*g_sc=*/r, /*g_sj=*/1, accumulate, o.colpart, st);
  }
  return hip_status(e);
}

qlora_status qlora_silu_mul_fwd(const void* G, const void* Up, void* H, int64_t count, void* stream) {
  if (count < 0) return QLORA_ERR_SHAPE;
  if (count == 0) return QLORA_OK;
  if (!G || !Up || !H || !aligned16(G) || !aligned16(Up) || !aligned16(H)) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_silu_fwd(static_cast<const uint16_t*>(G), static_cast<const uint16_t*>(Up),
                                    static_cast<uint16_t*>(H), count, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_silu_mul_bwd(const void* G, const void* Up, const void* dH, void* dG, void* dUp, int64_t count,
                                void* stream) {
  if (count < 0) return QLORA_ERR_SHAPE;
  if (count == 0) return QLORA_OK;
  if (!G || !Up || !dH || !dG || !dUp || !aligned16(G) || !aligned16(Up) || !aligned16(dH) || !aligned16(dG) ||
      !aligned16(dUp))
    return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_silu_bwd(static_cast<const uint16_t*>(G), static_cast<const uint16_t*>(Up),
                                    static_cast<const uint16_t*>(dH), static_cast<uint16_t*>(dG),
                                    static_cast<uint16_t*>(dUp), count, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
