// Internal launch functions of libqlora (host side). Each enqueues kernels on
// `stream` and returns hipGetLastError(); argument checking happens before,
// in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qlora.h"

namespace qlora {

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// ---- encoder workspace: absmax fp32 [nb], run sums fp64 [ceil(nb/256)]
inline size_t quantize_ws_absmax_bytes(int64_t nb) { return align256((size_t)nb * 4); }
inline size_t quantize_ws_runsum_bytes(int64_t nb) { return align256((size_t)((nb + 255) / 256) * 8); }
inline size_t quantize_ws_bytes(int64_t nb) {
  return quantize_ws_absmax_bytes(nb) + quantize_ws_runsum_bytes(nb) + align256((size_t)((nb + 255) / 256) * 4);
}

// code8 NULL: no double quantization, s2 receives one scale per block, fp32
// or (s2_bf16) the bf16 rounding of the block absmax, which the codes are
// then taken against.
hipError_t launch_quantize(const void* W, bool w_bf16, int64_t n, int64_t k, const float* codebook,
                           uint8_t* codes, uint8_t* code8, float* s2, float* mean, void* ws,
                           hipStream_t stream, bool s2_bf16 = false);

// Encoded weight as the kernels see it (s2_bf16: without double
// quantization, s2 holds bf16 bit patterns, one per block).
struct Nf4View {
  int64_t n, k;
  const uint8_t* codes;
  const uint8_t* code8;
  const float* s2;
  const float* mean;
  const float* codebook;
  bool s2_bf16 = false;
};

hipError_t launch_dequant(const Nf4View& w, uint16_t* out, hipStream_t stream, bool f16 = false);

// Columns of the LoRA "extra" contraction region: [hi | lo] halves of the
// scaled low-rank activation, padded with zeros to a multiple of 64.
inline int lora_extra_cols(int r) { return r > 0 ? ((2 * r + 63) / 64) * 64 : 0; }

// out[m, j] = sum_c P[m, c] Q(c, j), P bf16 [M, C]; Q bf16 [r, C] (q_layout
// 0) or [C, r] (q_layout 1); fp32 out [M, r] (nullable). If split != NULL it
// also receives rows [bf16(scale*out) | bf16(scale*out - hi) | 0 ...] of
// lora_extra_cols(r) elements. part: workspace of rowdot_ws_bytes (may be 0).
size_t rowdot_ws_bytes(int64_t M, int64_t C, int r);
// pmask (uint8 [M, C], q_layout 0 and C % 8 == 0 only; NULL: none): P's
// elements whose byte is 0 read as zero (dropout on the adapter's input).
hipError_t launch_rowdot(const uint16_t* P, int64_t M, int64_t C, const uint16_t* Q, int q_layout, int r,
                         float* out, uint16_t* split, float scale, float* part, hipStream_t stream,
                         const uint8_t* pmask = nullptr, bool f16 = false);

// Column reduction over M in fixed order, for the adapter gradients:
//   G[c, j] (+)= scale * sum_m P[m, c] * Q[m, j]    P bf16 [M, C], Q fp32 [M, r]
// written at G[c * g_sc + j * g_sj]. partial (fp32, [splits, C, r]) is workspace.
size_t coldot_ws_bytes(int64_t M, int64_t C, int r);
hipError_t launch_coldot(const uint16_t* P, int64_t M, int64_t C, const float* Q, int r, float scale,
                         float* G, int64_t g_sc, int64_t g_sj, int accumulate, float* partial,
                         hipStream_t stream, const uint8_t* pmask = nullptr, bool f16 = false);
// dA and dB of one layer in one launch (both with a single token split, no
// mask): products (P0, C0, Q0 -> G0 with strides g_sc0, g_sj0) and (P1, ...),
// the same arithmetic as two launch_coldot calls. coldot_pairable tells when
// it applies.
bool coldot_pairable(int64_t M, int64_t C0, int64_t C1);
hipError_t launch_coldot_pair(const uint16_t* P0, int64_t C0, const float* Q0, float* G0, int64_t g_sc0,
                              int64_t g_sj0, const uint16_t* P1, int64_t C1, const float* Q1, float* G1,
                              int64_t g_sc1, int64_t g_sj1, int64_t M, int r, float scale, int accumulate,
                              hipStream_t stream, bool f16);

// Y = RN_bf16(X W'^T + [sT_hi | sT_lo] [B | B]^T): fused dequant + MFMA GEMM.
hipError_t launch_gemm_fwd(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* TS,
                           const uint16_t* B, int r, uint16_t* Y, hipStream_t stream);

// dX = RN_bf16(dY W' + [sU_hi | sU_lo] [A ; A]): fused transposed dequant + MFMA GEMM.
hipError_t launch_gemm_dx(const Nf4View& w, const uint16_t* dY, int64_t M, const uint16_t* US,
                          const uint16_t* A, int r, uint16_t* dX, hipStream_t stream,
                          const uint8_t* mask = nullptr, float keep_scale = 1.0f);

// dX = RN_bf16(dY W + [sU_hi | sU_lo] [A ; A]) for a bf16 base weight W [n, k]
// (k % 64 == 0): the fused kernel's dX with the weight tile copied instead of
// expanded.
hipError_t launch_gemm_w16_dx(const uint16_t* W, int64_t n, int64_t k, const uint16_t* dY, int64_t M,
                              const uint16_t* US, const uint16_t* A, int r, uint16_t* dX, hipStream_t stream);

// Expanded bf16 operand of the plain GEMM (forward [n, k + xc], or dX
// [k, np + xc] with np = n rounded up to 64), LoRA factor appended.
int64_t expand_pad_rows(int64_t n);
size_t expand_ws_bytes(int64_t n, int64_t k, int r, bool transposed);
hipError_t launch_expand(const Nf4View& w, const uint16_t* lr, int r, bool transposed, uint16_t* out,
                         hipStream_t stream, bool f16 = false);
// The dX operand in contraction-major form for the GEMM's NN form (n % 64
// == 0): out [n + xc, k], rows 0 .. n-1 W' as the forward expansion writes
// them, then the low-rank rows [A ; A ; 0].
size_t expand_nn_bytes(int64_t n, int64_t k, int r);
hipError_t launch_expand_nn(const Nf4View& w, const uint16_t* A, int r, uint16_t* out, hipStream_t stream);

// [n, lora_extra_cols(r)] rows [B | B | 0] (bf16), the low-rank operand of
// the forward GEMM when the weight operand is a separate matrix.
hipError_t launch_lowrank_rows(const uint16_t* B, int64_t n, int r, uint16_t* out, hipStream_t stream);

// out = RN_bf16([act | split] F^T) over an expanded operand F [nout, kcp + kx].
// The kernel addresses each operand with 32-bit byte offsets: every operand
// must be smaller than 4 GiB (gemm_bf16_offsets_fit). When the last wave of
// 256 tiles holds at most 128 (all of them, for small outputs), those tiles
// are split along the contraction over gemm_bf16_splits() workgroups each,
// whose fp32 partials (gemm_bf16_ws_bytes() of workspace, `part`) are added
// in split order and rounded once; part may be NULL when that size is 0.
bool gemm_bf16_offsets_fit(int64_t M, int64_t kc, int kx, int64_t nout);
int gemm_bf16_splits(int64_t M, int64_t kc, int kx, int64_t nout);
size_t gemm_bf16_ws_bytes(int64_t M, int64_t kc, int kx, int64_t nout);
// mask (uint8 [M, nout], may be NULL): dropout on the low-rank term, which is
// multiplied by keep_scale where mask is set and dropped where it is not,
// before the main contraction is added (one rounding of the whole sum).
hipError_t launch_gemm_bf16(const uint16_t* act, int64_t M, int64_t kc, const uint16_t* split, int kx,
                            const uint16_t* f, int64_t nout, uint16_t* out, float* part, hipStream_t stream,
                            const uint8_t* mask = nullptr, float keep_scale = 1.0f, bool f16 = false);

// The same GEMM with the weight operand and the low-rank operand as separate
// row-major matrices: f [nout, ldf] (the base contraction in its first kc
// columns; kc % 64 == 0 or the columns up to the next multiple of 64 zero)
// and fx [nout, ldx] (kx low-rank columns). A bf16 base weight W [n, k] is
// such an f for the forward as it is stored.
// nn: f is stored [contraction][output] instead ([kc rows, ldf], kc % 64 == 0,
// and fx [kx rows, ldx]): dX over a bf16 base weight W [n, k] as stored, the
// fragments read through the transposing LDS read (bf16, no mask).
hipError_t launch_gemm_bf16_ext(const uint16_t* act, int64_t M, int64_t kc, const uint16_t* split, int kx,
                                const uint16_t* f, int64_t ldf, const uint16_t* fx, int64_t ldx, int64_t nout,
                                uint16_t* out, float* part, hipStream_t stream, const uint8_t* mask = nullptr,
                                float keep_scale = 1.0f, bool f16 = false, bool nn = false);

// [lora_extra_cols(r), k] rows [A ; A ; 0] (bf16), the low-rank operand of the
// nn GEMM (dX over a bf16 base).
hipError_t launch_lowrank_cols(const uint16_t* A, int r, int64_t k, uint16_t* out, hipStream_t stream);

// Adapter merge: out = round(W' + scale * B A) (w != NULL; bf16, or fp32 if
// out_f32) or unmerge: out = RN_bf16(Wm - scale * B A) (w == NULL, Wm bf16).
size_t merge_smem_bytes(int r);
hipError_t launch_merge(const Nf4View* w, const uint16_t* Wm, int64_t n, int64_t k, const uint16_t* A,
                        const uint16_t* B, int r, float scale, bool out_f32, void* out, hipStream_t stream);

// Small-M dequant-GEMV: Y = RN_bf16(X W'^T + scale * T B^T), M <= 16. ws:
// gemv_ws_bytes(k) bytes for the activations in operand order.
size_t gemv_ws_bytes(int64_t k);
// The GEMV addresses the codes with 32-bit buffer offsets: n k / 2 bytes
// (plus one workgroup's rows past n) under 4 GiB.
bool gemv_fits(int64_t n, int64_t k);
hipError_t launch_gemv(const Nf4View& w, const uint16_t* X, int64_t M, const float* T,
                       const uint16_t* B, int r, float scale, uint16_t* Y, void* ws, hipStream_t stream,
                       bool f16 = false);

// The layer forward behind qlora_linear_fwd and its dropout / fp16 forms
// (api.hip), and the workspace it carves for a bf16 call with or without a
// caller-provided T_save.
qlora_status linear_fwd_impl(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A, const void* B,
                             int r, float scale, const uint8_t* mask, float keep_scale, void* Y, float* T_save,
                             void* ws, size_t ws_bytes, void* stream, bool f16 = false);
size_t linear_fwd_ws_bytes(int64_t M, int64_t n, int64_t k, int r, bool have_tsave);

// Small-M dX through the frozen base (M <= 16): dX = RN_bf16(dY W' + scale
// (U A) [. mask * keep]) with U = dY B fp32 [M, r] (nullable when r == 0)
// and A bf16 [r, k]; ws: gemv_dx_ws_bytes(n, k) bytes of fp32 partials.
size_t gemv_dx_ws_bytes(int64_t n, int64_t k);
hipError_t launch_gemv_dx(const Nf4View& w, const uint16_t* dY, int64_t M, const float* U, const uint16_t* A, int r,
                          float scale, uint16_t* dX, void* ws, hipStream_t stream, const uint8_t* mask = nullptr,
                          float keep = 1.0f);

hipError_t launch_silu_fwd(const uint16_t* G, const uint16_t* U, uint16_t* H, int64_t count,
                           hipStream_t stream);
hipError_t launch_silu_bwd(const uint16_t* G, const uint16_t* U, const uint16_t* dH, uint16_t* dG,
                           uint16_t* dU, int64_t count, hipStream_t stream);

}  // namespace qlora
