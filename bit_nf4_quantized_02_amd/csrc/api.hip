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
  // code8 NULL: no double quantization (s2 holds one fp32 scale per block,
  // or one bf16 bit pattern per block with scale_bf16 = 1; mean is not read)
  if (!w->codes || !w->s2 || !w->codebook || (w->code8 && !w->mean)) return QLORA_ERR_INVALID_ARG;
  if (w->scale_bf16 != 0 && (w->scale_bf16 != 1 || w->code8)) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(w->codes) || !aligned16(w->s2) || !aligned16(w->codebook)) return QLORA_ERR_INVALID_ARG;
  if (w->code8 && (!aligned16(w->code8) || !aligned16(w->mean))) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

Nf4View view_of(const qlora_nf4_weight* w) {
  return Nf4View{w->n, w->k, w->codes, w->code8, w->s2, w->mean, w->codebook, w->scale_bf16 == 1};
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

// Kernel choice per pass (the rule qlora_linear_path documents).
// fp16 compute (the ablation) runs the GEMV for M <= 16 in the forward and the
// expanded path otherwise; -1 where that path cannot take the shape.
int path_of_f16(int64_t M, int64_t n, int64_t k, int r, bool bwd) {
  if (!bwd && small_m(M)) return gemv_fits(n, k) ? QLORA_PATH_GEMV : -1;
  const int xc = lora_extra_cols(r);
  const bool fits = bwd ? gemm_bf16_offsets_fit(M, n, xc, k) : gemm_bf16_offsets_fit(M, k, xc, n);
  return fits && (!bwd || n % 8 == 0) ? QLORA_PATH_EXPANDED : -1;
}

int path_of(int64_t M, int64_t n, int64_t k, int r, bool bwd) {
  // forward GEMV (codes under 4 GiB, else the fused kernel); backward: dX GEMV
  if (small_m(M) && (bwd || gemv_fits(n, k))) return QLORA_PATH_GEMV;
  const int xc = lora_extra_cols(r);
  const bool fits = bwd ? gemm_bf16_offsets_fit(M, n, xc, k) : gemm_bf16_offsets_fit(M, k, xc, n);
  if (M >= QLORA_EXPAND_MIN_M && fits && (!bwd || n % 8 == 0)) return QLORA_PATH_EXPANDED;
  return QLORA_PATH_FUSED;
}

// ---- building-block workspaces
size_t project_ws(int64_t M, int64_t C, int r) {
  const size_t b = rowdot_ws_bytes(M, C, r);
  return b > 0 ? b : 256;  // a non-empty region keeps the workspace pointer checks uniform
}
size_t grad_ws(int64_t M, int64_t C, int r) { return coldot_ws_bytes(M, C, r); }

// T = P Q^T (q_layout 0, Q [r, C]) or P Q (q_layout 1, Q [C, r]); optional split.
hipError_t do_project(const uint16_t* P, int64_t M, int64_t C, const uint16_t* Q, int q_layout, int r, float scale,
                      float* out, uint16_t* split, void* ws, hipStream_t st, const uint8_t* pmask = nullptr,
                      bool f16 = false) {
  return launch_rowdot(P, M, C, Q, q_layout, r, out, split, scale, static_cast<float*>(ws), st, pmask, f16);
}

hipError_t do_grad(const uint16_t* P, int64_t M, int64_t C, const float* Q, int r, float scale, float* G,
                   int g_layout, int accumulate, void* ws, hipStream_t st, const uint8_t* pmask = nullptr,
                   bool f16 = false) {
  const int64_t g_sc = g_layout == 0 ? 1 : r;
  const int64_t g_sj = g_layout == 0 ? C : 1;
  return launch_coldot(P, M, C, Q, r, scale, G, g_sc, g_sj, accumulate, static_cast<float*>(ws), st, pmask, f16);
}

// ---- whole-layer workspaces (layouts shared by the size query and the call)
struct FwdWs {
  void* xp = nullptr;     // activations in the GEMV's operand order (M <= 16)
  float* T = nullptr;
  uint16_t* TS = nullptr;
  void* proj = nullptr;
  uint16_t* F = nullptr;  // expanded operand (large M)
  float* part = nullptr;  // split-K partial sums of its GEMM (few output tiles)
};

size_t fwd_ws(int64_t M, int64_t n, int64_t k, int r, bool have_tsave, Carver& cv, FwdWs& o, bool f16 = false) {
  const int path = f16 ? path_of_f16(M, n, k, r, false) : path_of(M, n, k, r, false);
  if (r > 0) {
    if (path == QLORA_PATH_GEMV) {
      if (!have_tsave) o.T = cv.take<float>((size_t)M * r * 4);
    } else {
      o.TS = cv.take<uint16_t>((size_t)M * lora_extra_cols(r) * 2);
    }
    o.proj = cv.take<char>(project_ws(M, k, r));
  }
  if (path == QLORA_PATH_GEMV) o.xp = cv.take<char>(gemv_ws_bytes(k));
  if (path == QLORA_PATH_EXPANDED) {
    o.F = cv.take<uint16_t>(expand_ws_bytes(n, k, r, false));
    const size_t pb = gemm_bf16_ws_bytes(M, k, lora_extra_cols(r), n);
    if (pb > 0) o.part = cv.take<float>(pb);
  }
  return cv.used;
}

struct BwdWs {
  float* T = nullptr;
  float* U = nullptr;
  uint16_t* US = nullptr;
  void* proj = nullptr;
  void* grad = nullptr;
  uint16_t* F = nullptr;  // expanded transposed operand (large M)
  float* part = nullptr;  // split-K partial sums of its GEMM (few output tiles), or of the dX GEMV (M <= 16)
};

size_t bwd_ws(int64_t M, int64_t n, int64_t k, int r, bool have_tsaved, Carver& cv, BwdWs& o, bool f16 = false) {
  const bool gemv = !f16 && path_of(M, n, k, r, true) == QLORA_PATH_GEMV;
  if (r > 0) {
    if (!have_tsaved) o.T = cv.take<float>((size_t)M * r * 4);
    o.U = cv.take<float>((size_t)M * r * 4);
    if (!gemv) o.US = cv.take<uint16_t>((size_t)M * lora_extra_cols(r) * 2);
    const size_t p1 = project_ws(M, n, r), p2 = project_ws(M, k, r);
    o.proj = cv.take<char>(p1 > p2 ? p1 : p2);
    const size_t g1 = grad_ws(M, k, r), g2 = grad_ws(M, n, r);
    o.grad = cv.take<char>(g1 > g2 ? g1 : g2);
  }
  if ((f16 ? path_of_f16(M, n, k, r, true) : path_of(M, n, k, r, true)) == QLORA_PATH_EXPANDED) {
    o.F = cv.take<uint16_t>(expand_ws_bytes(n, k, r, true));
    const size_t pb = gemm_bf16_ws_bytes(M, n, lora_extra_cols(r), k);
    if (pb > 0) o.part = cv.take<float>(pb);
  }
  if (gemv) o.part = cv.take<float>(gemv_dx_ws_bytes(n, k));
  return cv.used;
}

// Zeros for the adapter gradients of an empty batch (a kernel, not a memset,
// so the call stays capturable in a graph).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  zero_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
  return hipGetLastError();
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
    case QLORA_ERR_SCRATCH:
      return "QLORA_ERR_SCRATCH: the call needs more than the library's static scratch (QLORA_SCRATCH_BYTES)";
    default: return "QLORA_ERR_UNKNOWN";
  }
}

size_t qlora_nf4_packed_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 1 || k % QLORA_BLOCK) return 0;
  const int64_t nb = n * k / QLORA_BLOCK;
  const int64_t nc = (nb + QLORA_DQ_BLOCK - 1) / QLORA_DQ_BLOCK;
  return (size_t)(n * k / 2 + nb + 4 * nc + 4);
}

size_t qlora_nf4_storage_bytes(int64_t n, int64_t k, int scale_form) {
  if (scale_form < 0 || scale_form > 2) return 0;
  if (scale_form == QLORA_SCALE_DQ) return qlora_nf4_packed_bytes(n, k);
  if (n < 1 || k < 1 || k % QLORA_BLOCK) return 0;
  const int64_t per_block = scale_form == QLORA_SCALE_BF16 ? 2 : 4;
  return (size_t)(n * k / 2 + per_block * (n * k / QLORA_BLOCK));
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
                                    out->code8, out->s2, out->mean, ws, static_cast<hipStream_t>(stream),
                                    out->scale_bf16 == 1));
}

qlora_status qlora_dequant(const qlora_nf4_weight* w, void* out, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (out == nullptr || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_dequant(view_of(w), static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

qlora_status qlora_dequant_f16(const qlora_nf4_weight* w, void* out, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (out == nullptr || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  return hip_status(
      launch_dequant(view_of(w), static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream), /*f16=*/true));
}

qlora_status qlora_adapter_merge(const qlora_nf4_weight* w, const void* A, const void* B, int r, float scale,
                                 void* out, int out_dtype, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (out_dtype != QLORA_DT_BF16 && out_dtype != QLORA_DT_FP32) return QLORA_ERR_INVALID_ARG;
  if (out == nullptr || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  const Nf4View v = view_of(w);
  return hip_status(launch_merge(&v, nullptr, w->n, w->k, static_cast<const uint16_t*>(A),
                                 static_cast<const uint16_t*>(B), r, scale, out_dtype == QLORA_DT_FP32, out,
                                 static_cast<hipStream_t>(stream)));
}

qlora_status qlora_adapter_unmerge(const void* merged, int64_t n, int64_t k, const void* A, const void* B, int r,
                                   float scale, void* out, void* stream) {
  if (n < 1 || k < QLORA_BLOCK || k % QLORA_BLOCK || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (!merged || !out || !aligned16(merged) || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_merge(nullptr, static_cast<const uint16_t*>(merged), n, k, static_cast<const uint16_t*>(A),
                                 static_cast<const uint16_t*>(B), r, scale, false, out,
                                 static_cast<hipStream_t>(stream)));
}

static size_t linear_ws_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd, bool f16) {
  if (M < 0 || n < 1 || k < 1 || k % QLORA_BLOCK || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (is_bwd != 0 && is_bwd != 1) return 0;
  if (M == 0) return 0;
  Carver cv(nullptr);
  if (!is_bwd) {
    FwdWs o;
    return fwd_ws(M, n, k, r, /*have_tsave=*/false, cv, o, f16);
  }
  BwdWs o;
  return bwd_ws(M, n, k, r, /*have_tsaved=*/false, cv, o, f16);
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd) {
  return linear_ws_bytes(M, n, k, r, is_bwd, false);
}

}  // extern "C"

size_t qlora::linear_fwd_ws_bytes(int64_t M, int64_t n, int64_t k, int r, bool have_tsave) {
  if (M < 1 || n < 1 || k < 1 || k % QLORA_BLOCK || r < 0 || r > QLORA_MAX_RANK) return 0;
  Carver cv(nullptr);
  FwdWs o;
  return fwd_ws(M, n, k, r, have_tsave, cv, o, false);
}

extern "C" {

size_t qlora_linear_f16_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd) {
  return linear_ws_bytes(M, n, k, r, is_bwd, true);
}

int qlora_lowrank_split_cols(int r) { return (r < 0 || r > QLORA_MAX_RANK) ? 0 : lora_extra_cols(r); }

size_t qlora_lowrank_project_workspace_bytes(int64_t M, int64_t C, int r) {
  if (M < 1 || C < 1 || r < 1 || r > QLORA_MAX_RANK) return 0;
  return project_ws(M, C, r);
}

qlora_status qlora_lowrank_project(const void* P, int64_t M, int64_t C, const void* Q, int q_layout, int r,
                                   float scale, float* out, void* split, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || C < 1 || r < 1 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (q_layout != 0 && q_layout != 1) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  if (!P || !Q || !aligned16(P) || !aligned16(Q)) return QLORA_ERR_INVALID_ARG;
  if ((out && !aligned16(out)) || (split && !aligned16(split)) || (!out && !split)) return QLORA_ERR_INVALID_ARG;
  if (ws == nullptr || !aligned16(ws) || ws_bytes < project_ws(M, C, r)) return QLORA_ERR_WORKSPACE;
  return hip_status(do_project(static_cast<const uint16_t*>(P), M, C, static_cast<const uint16_t*>(Q), q_layout, r,
                               scale, out, static_cast<uint16_t*>(split), ws, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_nf4_gemm_fwd(const qlora_nf4_weight* w, const void* X, int64_t M, const void* split,
                                const void* B, int r, void* Y, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !aligned16(X) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!split || !B || !aligned16(split) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_gemm_fwd(view_of(w), static_cast<const uint16_t*>(X), M,
                                    static_cast<const uint16_t*>(split), static_cast<const uint16_t*>(B), r,
                                    static_cast<uint16_t*>(Y), static_cast<hipStream_t>(stream)));
}

qlora_status qlora_nf4_gemm_dx(const qlora_nf4_weight* w, const void* dY, int64_t M, const void* split,
                               const void* A, int r, void* dX, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!dY || !dX || !aligned16(dY) || !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!split || !A || !aligned16(split) || !aligned16(A))) return QLORA_ERR_INVALID_ARG;
  return hip_status(launch_gemm_dx(view_of(w), static_cast<const uint16_t*>(dY), M,
                                   static_cast<const uint16_t*>(split), static_cast<const uint16_t*>(A), r,
                                   static_cast<uint16_t*>(dX), static_cast<hipStream_t>(stream)));
}

size_t qlora_nf4_gemv_workspace_bytes(int64_t k) {
  if (k < 1 || k % QLORA_BLOCK) return 0;
  return gemv_ws_bytes(k);
}

qlora_status qlora_nf4_gemv_fwd(const qlora_nf4_weight* w, const void* X, int64_t M, const float* T, const void* B,
                                int r, float scale, void* Y, void* ws, size_t ws_bytes, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || M > 16 || r < 0 || r > QLORA_MAX_RANK || !gemv_fits(w->n, w->k)) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !aligned16(X) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!T || !B || !aligned16(T) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if (ws == nullptr || !aligned16(ws) || ws_bytes < gemv_ws_bytes(w->k)) return QLORA_ERR_WORKSPACE;
  return hip_status(launch_gemv(view_of(w), static_cast<const uint16_t*>(X), M, T, static_cast<const uint16_t*>(B),
                                r, scale, static_cast<uint16_t*>(Y), ws, static_cast<hipStream_t>(stream)));
}

size_t qlora_nf4_gemv_dx_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 1 || k % QLORA_BLOCK) return 0;
  return gemv_dx_ws_bytes(n, k);
}

qlora_status qlora_nf4_gemv_dx(const qlora_nf4_weight* w, const void* dY, int64_t M, const float* U, const void* A,
                               int r, float scale, void* dX, void* ws, size_t ws_bytes, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || M > 16 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!dY || !dX || !aligned16(dY) || !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!U || !A || !aligned16(U) || !aligned16(A))) return QLORA_ERR_INVALID_ARG;
  if (ws == nullptr || !aligned16(ws) || ws_bytes < gemv_dx_ws_bytes(w->n, w->k)) return QLORA_ERR_WORKSPACE;
  return hip_status(launch_gemv_dx(view_of(w), static_cast<const uint16_t*>(dY), M, U,
                                   static_cast<const uint16_t*>(A), r, scale, static_cast<uint16_t*>(dX), ws,
                                   static_cast<hipStream_t>(stream)));
}

int qlora_linear_path(int64_t M, int64_t n, int64_t k, int r, int is_bwd) {
  if (M < 0 || n < 1 || k < 1 || (k % QLORA_BLOCK) != 0 || r < 0 || r > QLORA_MAX_RANK) return -1;
  if (is_bwd != 0 && is_bwd != 1) return -1;
  return path_of(M, n, k, r, is_bwd == 1);
}

size_t qlora_nf4_expand_bytes(int64_t n, int64_t k, int r, int transposed) {
  if (n < 1 || k < 1 || (k % QLORA_BLOCK) != 0 || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (transposed == 2) return n % 64 == 0 ? expand_nn_bytes(n, k, r) : 0;
  if (transposed != 0 && transposed != 1) return 0;
  return expand_ws_bytes(n, k, r, transposed == 1);
}

qlora_status qlora_nf4_expand(const qlora_nf4_weight* w, const void* lr, int r, int transposed, void* out,
                              size_t out_bytes, void* stream) {
  const qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (transposed != 0 && transposed != 1 && transposed != 2) return QLORA_ERR_INVALID_ARG;
  if (transposed == 2 && w->n % 64 != 0) return QLORA_ERR_SHAPE;
  if (!out || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!lr || !aligned16(lr))) return QLORA_ERR_INVALID_ARG;
  if (out_bytes < qlora_nf4_expand_bytes(w->n, w->k, r, transposed)) return QLORA_ERR_WORKSPACE;
  if (transposed == 2)
    return hip_status(launch_expand_nn(view_of(w), static_cast<const uint16_t*>(lr), r, static_cast<uint16_t*>(out),
                                       static_cast<hipStream_t>(stream)));
  return hip_status(launch_expand(view_of(w), static_cast<const uint16_t*>(lr), r, transposed == 1,
                                  static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

size_t qlora_bf16_gemm_workspace_bytes(int64_t M, int64_t kc, int r, int64_t nout) {
  if (M < 1 || kc < 8 || (kc % 8) != 0 || nout < 1 || r < 0 || r > QLORA_MAX_RANK) return 0;
  return gemm_bf16_ws_bytes(M, kc, lora_extra_cols(r), nout);
}

qlora_status qlora_bf16_gemm(const void* act, int64_t M, int64_t kc, const void* split, int r, const void* F,
                             int64_t nout, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || kc < 8 || (kc % 8) != 0 || nout < 1 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!act || !F || !out || !aligned16(act) || !aligned16(F) || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!split || !aligned16(split))) return QLORA_ERR_INVALID_ARG;
  if (!gemm_bf16_offsets_fit(M, kc, lora_extra_cols(r), nout)) return QLORA_ERR_SHAPE;
  const size_t need = gemm_bf16_ws_bytes(M, kc, lora_extra_cols(r), nout);
  if (need > 0 && (!ws || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  return hip_status(launch_gemm_bf16(static_cast<const uint16_t*>(act), M, kc, static_cast<const uint16_t*>(split),
                                     lora_extra_cols(r), static_cast<const uint16_t*>(F), nout,
                                     static_cast<uint16_t*>(out), need > 0 ? static_cast<float*>(ws) : nullptr,
                                     static_cast<hipStream_t>(stream)));
}

qlora_status qlora_bf16_gemm_nn(const void* act, int64_t M, int64_t kc, const void* split, int r, const void* F,
                                int64_t nout, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || kc < 64 || (kc % 64) != 0 || nout < 8 || (nout % 8) != 0 || r < 0 || r > QLORA_MAX_RANK)
    return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!act || !F || !out || !aligned16(act) || !aligned16(F) || !aligned16(out)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!split || !aligned16(split))) return QLORA_ERR_INVALID_ARG;
  const int xc = lora_extra_cols(r);
  if (!gemm_bf16_offsets_fit(M, kc, xc, nout) || (kc + xc) * nout * 2 >= ((int64_t)1 << 32)) return QLORA_ERR_SHAPE;
  const size_t need = gemm_bf16_ws_bytes(M, kc, xc, nout);
  if (need > 0 && (!ws || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  const uint16_t* f = static_cast<const uint16_t*>(F);
  return hip_status(launch_gemm_bf16_ext(static_cast<const uint16_t*>(act), M, kc, static_cast<const uint16_t*>(split),
                                         xc, f, nout, f + kc * nout, nout, nout, static_cast<uint16_t*>(out),
                                         need > 0 ? static_cast<float*>(ws) : nullptr,
                                         static_cast<hipStream_t>(stream), nullptr, 1.0f, false, /*nn=*/true));
}

size_t qlora_lowrank_grad_workspace_bytes(int64_t M, int64_t C, int r) {
  if (M < 1 || C < 1 || r < 1 || r > QLORA_MAX_RANK) return 0;
  return grad_ws(M, C, r);
}

qlora_status qlora_lowrank_grad(const void* P, int64_t M, int64_t C, const float* Q, int r, float scale, float* G,
                                int g_layout, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || C < 1 || r < 1 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if ((g_layout != 0 && g_layout != 1) || (accumulate != 0 && accumulate != 1)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  if (!G || !aligned16(G) || !P || !Q || !aligned16(P) || !aligned16(Q)) return QLORA_ERR_INVALID_ARG;
  if (ws == nullptr || !aligned16(ws) || ws_bytes < grad_ws(M, C, r)) return QLORA_ERR_WORKSPACE;
  return hip_status(do_grad(static_cast<const uint16_t*>(P), M, C, Q, r, scale, G, g_layout, accumulate, ws,
                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// The layer calls with and without dropout on the adapter's input (mask NULL:
// none). With dropout the branch's kernels read X through the mask (dropped
// entries as zero) and keep_scale folds into the branch's scale: T_save
// receives (X . mask) A^T. (Also the body of the forward that runs in the
// library's static scratch, noalloc.hip.)
qlora_status qlora::linear_fwd_impl(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A,
                                    const void* B, int r, float scale, const uint8_t* mask, float keep_scale,
                                    void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream, bool f16) {
  qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !aligned16(X) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if (T_save && !aligned16(T_save)) return QLORA_ERR_INVALID_ARG;
  const bool drop = mask != nullptr && r > 0;
  if (f16 && (drop || path_of_f16(M, w->n, w->k, r, false) < 0)) return QLORA_ERR_UNSUPPORTED;
  {
    Carver probe(nullptr);
    FwdWs tmp;
    const size_t need = fwd_ws(M, w->n, w->k, r, T_save != nullptr, probe, tmp, f16);
    if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  FwdWs o;
  fwd_ws(M, w->n, w->k, r, T_save != nullptr, cv, o, f16);
  const Nf4View v = view_of(w);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  uint16_t* y = static_cast<uint16_t*>(Y);
  hipError_t e = hipSuccess;
  // the branch's input mask and scale
  const uint8_t* pm = drop ? mask : nullptr;
  const float sb = drop ? scale * keep_scale : scale;
  const int path = f16 ? path_of_f16(M, w->n, w->k, r, false) : path_of(M, w->n, w->k, r, false);
  if (path == QLORA_PATH_GEMV) {
    float* T = T_save ? T_save : o.T;
    if (r > 0) e = do_project(x, M, w->k, a, 0, r, sb, T, nullptr, o.proj, st, pm, f16);
    if (e == hipSuccess) e = launch_gemv(v, x, M, T, b, r, sb, y, o.xp, st, f16);
  } else {
    if (r > 0) e = do_project(x, M, w->k, a, 0, r, sb, T_save, o.TS, o.proj, st, pm, f16);
    if (path == QLORA_PATH_FUSED) {
      if (e == hipSuccess) e = launch_gemm_fwd(v, x, M, o.TS, b, r, y, st);
    } else {
      if (e == hipSuccess) e = launch_expand(v, b, r, false, o.F, st, f16);
      if (e == hipSuccess)
        e = launch_gemm_bf16(x, M, w->k, o.TS, lora_extra_cols(r), o.F, w->n, y, o.part, st, nullptr, 1.0f, f16);
    }
  }
  return hip_status(e);
}

static qlora_status linear_bwd_impl(const qlora_nf4_weight* w, const void* X, const float* T_saved,
                                    const void* dY, int64_t M, const void* A, const void* B, int r, float scale,
                                    const uint8_t* mask, float keep_scale, void* dX, float* dA, float* dB,
                                    int accumulate, void* ws, size_t ws_bytes, void* stream, bool f16 = false) {
  qlora_status s = check_weight(w);
  if (s != QLORA_OK) return s;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return QLORA_ERR_INVALID_ARG;
  if (M == 0) {
    // an empty batch: dA and dB are empty sums (zeros), unless accumulating
    if (accumulate || r == 0) return QLORA_OK;
    if ((dA && !aligned16(dA)) || (dB && !aligned16(dB))) return QLORA_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = dA ? zero_f32(dA, (int64_t)r * w->k, st) : hipSuccess;
    if (e == hipSuccess && dB) e = zero_f32(dB, w->n * (int64_t)r, st);
    return hip_status(e);
  }
  if (!dY || !aligned16(dY)) return QLORA_ERR_INVALID_ARG;
  if (dX && !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if (r == 0) { dA = nullptr; dB = nullptr; }
  const bool drop = mask != nullptr && r > 0;
  const bool need_x = (dA != nullptr) || (dB != nullptr && T_saved == nullptr);
  if (need_x && (!X || !aligned16(X))) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if ((dA && !aligned16(dA)) || (dB && !aligned16(dB)) || (T_saved && !aligned16(T_saved)))
    return QLORA_ERR_INVALID_ARG;
  if (f16 && dX && path_of_f16(M, w->n, w->k, r, true) < 0) return QLORA_ERR_UNSUPPORTED;
  if (f16 && mask != nullptr && r > 0) return QLORA_ERR_UNSUPPORTED;
  {
    Carver probe(nullptr);
    BwdWs tmp;
    const size_t need = bwd_ws(M, w->n, w->k, r, T_saved != nullptr, probe, tmp, f16);
    if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  BwdWs o;
  bwd_ws(M, w->n, w->k, r, T_saved != nullptr, cv, o, f16);
  const Nf4View v = view_of(w);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* dy = static_cast<const uint16_t*>(dY);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  hipError_t e = hipSuccess;
  const uint8_t* dmask = drop ? mask : nullptr;  // dX: dropout on its low-rank term
  const bool gemv = !f16 && path_of(M, w->n, w->k, r, true) == QLORA_PATH_GEMV;
  if (r > 0 && (dX || dA))
    e = do_project(dy, M, w->n, b, 1, r, scale, o.U, (dX && !gemv) ? o.US : nullptr, o.proj, st, nullptr, f16);
  if (e == hipSuccess && dX && gemv) {
    e = launch_gemv_dx(v, dy, M, o.U, a, r, scale, static_cast<uint16_t*>(dX), o.part, st, dmask, keep_scale);
  } else if (e == hipSuccess && dX) {
    if (!f16 && dmask == nullptr && path_of(M, w->n, w->k, r, true) == QLORA_PATH_EXPANDED &&
        w->n % 64 == 0) {
      // W' expanded as the forward does ([n, k], contraction-major for dX)
      // and read by the GEMM's NN form through transposing LDS reads, the
      // low-rank rows [A ; A ; 0] after it (qlora_nf4_expand with
      // transposed = 2, then qlora_bf16_gemm_nn). This takes the transposed
      // expansion's workspace: (n + xc) k = k (np + xc) for n % 64 == 0.
      const int xc = lora_extra_cols(r);
      uint16_t* const fl = o.F + (size_t)w->n * w->k;
      e = launch_expand_nn(v, a, r, o.F, st);
      if (e == hipSuccess)
        e = launch_gemm_bf16_ext(dy, M, w->n, r > 0 ? o.US : nullptr, xc, o.F, w->k, fl, w->k, w->k,
                                 static_cast<uint16_t*>(dX), o.part, st, nullptr, 1.0f, false, /*nn=*/true);
    } else if (f16 || path_of(M, w->n, w->k, r, true) == QLORA_PATH_EXPANDED) {
      e = launch_expand(v, a, r, true, o.F, st, f16);
      if (e == hipSuccess)
        e = launch_gemm_bf16(dy, M, w->n, r > 0 ? o.US : nullptr, lora_extra_cols(r), o.F, w->k,
                             static_cast<uint16_t*>(dX), o.part, st, dmask, keep_scale, f16);
    } else {
      e = launch_gemm_dx(v, dy, M, r > 0 ? o.US : nullptr, a, r, static_cast<uint16_t*>(dX), st, dmask, keep_scale);
    }
  }
  // the branch's input mask and scale for the adapter gradients
  const uint8_t* pm = drop ? mask : nullptr;
  const float sb = drop ? scale * keep_scale : scale;
  if (e == hipSuccess && dA && dB && pm == nullptr && coldot_pairable(M, w->k, w->n)) {
    // few tokens: dA and dB in one launch
    const float* T = T_saved;
    if (T == nullptr) {
      e = do_project(x, M, w->k, a, 0, r, scale, o.T, nullptr, o.proj, st, nullptr, f16);
      T = o.T;
    }
    if (e == hipSuccess)
      e = launch_coldot_pair(x, w->k, o.U, dA, 1, w->k, dy, w->n, T, dB, r, 1, M, r, sb, accumulate, st, f16);
    return hip_status(e);
  }
  if (e == hipSuccess && dA) e = do_grad(x, M, w->k, o.U, r, sb, dA, 0, accumulate, o.grad, st, pm, f16);
  if (e == hipSuccess && dB) {
    const float* T = T_saved;
    if (T == nullptr) {
      e = do_project(x, M, w->k, a, 0, r, scale, o.T, nullptr, o.proj, st, pm, f16);
      T = o.T;
    }
    if (e == hipSuccess) e = do_grad(dy, M, w->n, T, r, sb, dB, 1, accumulate, o.grad, st, nullptr, f16);
  }
  return hip_status(e);
}

extern "C" {

qlora_status qlora_linear_fwd(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A, const void* B,
                              int r, float scale, void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream) {
  return linear_fwd_impl(w, X, M, A, B, r, scale, nullptr, 1.0f, Y, T_save, ws, ws_bytes, stream);
}

qlora_status qlora_linear_bwd(const qlora_nf4_weight* w, const void* X, const float* T_saved, const void* dY,
                              int64_t M, const void* A, const void* B, int r, float scale, void* dX, float* dA,
                              float* dB, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(w, X, T_saved, dY, M, A, B, r, scale, nullptr, 1.0f, dX, dA, dB, accumulate, ws,
                         ws_bytes, stream);
}

qlora_status qlora_linear_fwd_f16(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A, const void* B,
                                  int r, float scale, void* Y, float* T_save, void* ws, size_t ws_bytes,
                                  void* stream) {
  return linear_fwd_impl(w, X, M, A, B, r, scale, nullptr, 1.0f, Y, T_save, ws, ws_bytes, stream, true);
}

qlora_status qlora_linear_bwd_f16(const qlora_nf4_weight* w, const void* X, const float* T_saved, const void* dY,
                                  int64_t M, const void* A, const void* B, int r, float scale, void* dX, float* dA,
                                  float* dB, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(w, X, T_saved, dY, M, A, B, r, scale, nullptr, 1.0f, dX, dA, dB, accumulate, ws,
                         ws_bytes, stream, true);
}

qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A,
                                      const void* B, int r, float scale, const void* mask, float keep_scale,
                                      void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream) {
  if (M > 0 && r > 0 && (mask == nullptr || !aligned16(mask))) return QLORA_ERR_INVALID_ARG;
  if (!(keep_scale >= 1.0f) || keep_scale == INFINITY) return QLORA_ERR_INVALID_ARG;
  return linear_fwd_impl(w, X, M, A, B, r, scale, static_cast<const uint8_t*>(mask), keep_scale, Y, T_save, ws,
                         ws_bytes, stream);
}

qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const void* X, const float* T_saved, const void* dY,
                                      int64_t M, const void* A, const void* B, int r, float scale, const void* mask,
                                      float keep_scale, void* dX, float* dA, float* dB, int accumulate, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (M > 0 && r > 0 && (mask == nullptr || !aligned16(mask))) return QLORA_ERR_INVALID_ARG;
  if (!(keep_scale >= 1.0f) || keep_scale == INFINITY) return QLORA_ERR_INVALID_ARG;
  return linear_bwd_impl(w, X, T_saved, dY, M, A, B, r, scale, static_cast<const uint8_t*>(mask), keep_scale, dX,
                         dA, dB, accumulate, ws, ws_bytes, stream);
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

// ---- the same layer over a bf16 base weight (LoRA without quantization, the
// pages' comparison point). Same low-rank kernels; the forward multiplies W as
// stored (the plain GEMM with the low-rank operand as a separate matrix), and
// so does dX (the same GEMM reading W's tiles contraction-major).
namespace {

bool lora_shape_ok(int64_t n, int64_t k, int r) {
  return n >= 1 && k >= QLORA_BLOCK && k % QLORA_BLOCK == 0 && r >= 0 && r <= QLORA_MAX_RANK;
}

struct LoraFwdWs {
  uint16_t* TS = nullptr;
  void* proj = nullptr;
  uint16_t* Bx = nullptr;  // [n, xc] low-rank operand rows
  float* part = nullptr;
};

size_t lora_fwd_ws(int64_t M, int64_t n, int64_t k, int r, Carver& cv, LoraFwdWs& o) {
  const int xc = lora_extra_cols(r);
  if (r > 0) {
    o.TS = cv.take<uint16_t>((size_t)M * xc * 2);
    o.proj = cv.take<char>(project_ws(M, k, r));
    o.Bx = cv.take<uint16_t>((size_t)n * xc * 2);
  }
  const size_t pb = gemm_bf16_ws_bytes(M, k, xc, n);
  if (pb > 0) o.part = cv.take<float>(pb);
  return cv.used;
}

// dX over the bf16 base: the plain GEMM reading W's tiles as stored
// (contraction-major) when dY's rows allow direct copies (n % 8 == 0) and the
// operands fit its 32-bit offsets; the fused kernel otherwise.
bool lora_dx_nn(int64_t M, int64_t n, int64_t k, int r) {
  return n % 8 == 0 && gemm_bf16_offsets_fit(M, n, lora_extra_cols(r), k);
}

size_t lora_bwd_ws(int64_t M, int64_t n, int64_t k, int r, bool have_tsaved, Carver& cv, BwdWs& o) {
  if (lora_dx_nn(M, n, k, r)) {
    if (r > 0) o.F = cv.take<uint16_t>((size_t)lora_extra_cols(r) * k * 2);  // [A ; A ; 0]
    const size_t pb = gemm_bf16_ws_bytes(M, n, lora_extra_cols(r), k);
    if (pb > 0) o.part = cv.take<float>(pb);
  }
  if (r > 0) {
    if (!have_tsaved) o.T = cv.take<float>((size_t)M * r * 4);
    o.U = cv.take<float>((size_t)M * r * 4);
    o.US = cv.take<uint16_t>((size_t)M * lora_extra_cols(r) * 2);
    const size_t p1 = project_ws(M, n, r), p2 = project_ws(M, k, r);
    o.proj = cv.take<char>(p1 > p2 ? p1 : p2);
    const size_t g1 = grad_ws(M, k, r), g2 = grad_ws(M, n, r);
    o.grad = cv.take<char>(g1 > g2 ? g1 : g2);
  }
  return cv.used;
}

}  // namespace

extern "C" {

size_t qlora_lora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd) {
  if (M < 1 || !lora_shape_ok(n, k, r) || (is_bwd != 0 && is_bwd != 1)) return 0;
  Carver cv(nullptr);
  if (!is_bwd) {
    LoraFwdWs o;
    return lora_fwd_ws(M, n, k, r, cv, o);
  }
  BwdWs o;
  return lora_bwd_ws(M, n, k, r, false, cv, o);
}

qlora_status qlora_lora_linear_fwd(const void* W, int64_t n, int64_t k, const void* X, int64_t M, const void* A,
                                   const void* B, int r, float scale, void* Y, float* T_save, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (M < 0 || !lora_shape_ok(n, k, r)) return QLORA_ERR_SHAPE;
  if (M == 0) return QLORA_OK;
  if (!W || !X || !Y || !aligned16(W) || !aligned16(X) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if (T_save && !aligned16(T_save)) return QLORA_ERR_INVALID_ARG;
  const int xc = lora_extra_cols(r);
  if (!gemm_bf16_offsets_fit(M, k, xc, n)) return QLORA_ERR_SHAPE;
  {
    Carver probe(nullptr);
    LoraFwdWs tmp;
    const size_t need = lora_fwd_ws(M, n, k, r, probe, tmp);
    if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  LoraFwdWs o;
  lora_fwd_ws(M, n, k, r, cv, o);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* w = static_cast<const uint16_t*>(W);
  hipError_t e = hipSuccess;
  if (r > 0) {
    e = do_project(x, M, k, static_cast<const uint16_t*>(A), 0, r, scale, T_save, o.TS, o.proj, st);
    if (e == hipSuccess) e = launch_lowrank_rows(static_cast<const uint16_t*>(B), n, r, o.Bx, st);
  }
  if (e == hipSuccess)
    e = launch_gemm_bf16_ext(x, M, k, o.TS, xc, w, k, o.Bx, xc, n, static_cast<uint16_t*>(Y), o.part, st);
  return hip_status(e);
}

qlora_status qlora_lora_linear_bwd(const void* W, int64_t n, int64_t k, const void* X, const float* T_saved,
                                   const void* dY, int64_t M, const void* A, const void* B, int r, float scale,
                                   void* dX, float* dA, float* dB, int accumulate, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (M < 0 || !lora_shape_ok(n, k, r)) return QLORA_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return QLORA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 0) {
    if (accumulate || r == 0) return QLORA_OK;
    if ((dA && !aligned16(dA)) || (dB && !aligned16(dB))) return QLORA_ERR_INVALID_ARG;
    hipError_t e = dA ? zero_f32(dA, (int64_t)r * k, st) : hipSuccess;
    if (e == hipSuccess && dB) e = zero_f32(dB, n * (int64_t)r, st);
    return hip_status(e);
  }
  if (!W || !aligned16(W) || !dY || !aligned16(dY)) return QLORA_ERR_INVALID_ARG;
  if (dX && !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if (r == 0) { dA = nullptr; dB = nullptr; }
  const bool need_x = (dA != nullptr) || (dB != nullptr && T_saved == nullptr);
  if (need_x && (!X || !aligned16(X))) return QLORA_ERR_INVALID_ARG;
  if (r > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return QLORA_ERR_INVALID_ARG;
  if ((dA && !aligned16(dA)) || (dB && !aligned16(dB)) || (T_saved && !aligned16(T_saved)))
    return QLORA_ERR_INVALID_ARG;
  {
    Carver probe(nullptr);
    BwdWs tmp;
    const size_t need = lora_bwd_ws(M, n, k, r, T_saved != nullptr, probe, tmp);
    if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  }
  Carver cv(ws);
  BwdWs o;
  lora_bwd_ws(M, n, k, r, T_saved != nullptr, cv, o);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* dy = static_cast<const uint16_t*>(dY);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  hipError_t e = hipSuccess;
  if (r > 0 && (dX || dA)) e = do_project(dy, M, n, b, 1, r, scale, o.U, dX ? o.US : nullptr, o.proj, st);
  if (e == hipSuccess && dX) {
    if (lora_dx_nn(M, n, k, r)) {
      const int xc = lora_extra_cols(r);
      if (r > 0) e = launch_lowrank_cols(a, r, k, o.F, st);
      if (e == hipSuccess)
        e = launch_gemm_bf16_ext(dy, M, n, r > 0 ? o.US : nullptr, xc, static_cast<const uint16_t*>(W), k, o.F, k, k,
                                 static_cast<uint16_t*>(dX), o.part, st, nullptr, 1.0f, false, /*nn=*/true);
    } else {
      e = launch_gemm_w16_dx(static_cast<const uint16_t*>(W), n, k, dy, M, r > 0 ? o.US : nullptr, a, r,
                             static_cast<uint16_t*>(dX), st);
    }
  }
  if (e == hipSuccess && dA) e = do_grad(x, M, k, o.U, r, scale, dA, 0, accumulate, o.grad, st);
  if (e == hipSuccess && dB) {
    const float* T = T_saved;
    if (T == nullptr) {
      e = do_project(x, M, k, a, 0, r, scale, o.T, nullptr, o.proj, st);
      T = o.T;
    }
    if (e == hipSuccess) e = do_grad(dy, M, n, T, r, scale, dB, 1, accumulate, o.grad, st);
  }
  return hip_status(e);
}

}  // extern "C"
