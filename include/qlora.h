/*
 * qlora.h — C ABI of libqlora.so: the frozen-base NF4 linear layer with a
 * LoRA branch, for AMD Instinct MI355X (gfx950).
 *
 *   Y  = X W'^T + s (X A^T) B^T          forward
 *   dX = dY W' + s (dY B) A              backward through the frozen base
 *   dA = s (dY B)^T X,  dB = s dY^T (X A^T)   adapter gradients (no dW)
 *
 * W' is the bf16 expansion of a weight stored as 4-bit NF4 codes in blocks of
 * 64 consecutive weights, each block with an absmax scale that is itself
 * quantized to 8 bits ("double quantization").
 *
 * Sources (web pages on QLoRA, cited by title and section):
 *   [QQ] "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev):
 *        three-piece summary (4-bit storage, 16-bit compute on 64-weight
 *        blocks expanded on the fly, learning only in the adapter), the worked
 *        8-weight block, "NF4: a 4-bit format matched to weight statistics",
 *        the double-quantization paragraph, "Batched 4-bit matmuls".
 *   [QX] "QLoRA Explained: Fine-Tune 70B+ LLMs on a Single GPU" (gamut.so):
 *        "4-Bit NormalFloat (NF4) Quantization", "Double Quantization",
 *        "Step 3: Configure and Apply LoRA Adapters".
 *   [WQ] "What is QLoRA?" (qubittool.com), "Key Characteristics".
 *
 * Conventions shared by every call
 *   - Memory: every pointer marked (device) is device memory owned by the
 *     caller; (host) is host memory. The library never allocates or frees,
 *     keeps no state between calls, and writes only the outputs and the
 *     workspace it is given.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream). Every device call only enqueues work on that stream and
 *     returns; none synchronizes the host.
 *   - Layouts: all matrices are dense row-major with the last index
 *     contiguous and no padding: X [M,K], Y [M,N], dY [M,N], dX [M,K],
 *     A [r,K], B [N,r], T [M,r], dA [r,K], dB [N,r]. W is [N,K] (out x in),
 *     as a linear layer stores it.
 *   - Types: X, Y, dY, dX, A, B are bf16 (IEEE binary32 truncated to 16 bits,
 *     stored as uint16). T, dA, dB are fp32. bf16 outputs are rounded once,
 *     to nearest-even, from an fp32 accumulator that already includes the
 *     LoRA term.
 *   - Alignment: every device pointer must be 16-byte aligned.
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     on any error nothing is launched and a negative qlora_status returns.
 *     A failed launch returns QLORA_ERR_HIP. No C++ exception crosses the
 *     ABI. qlora_status_string() names each status.
 *   - Sizes: M = 0 launches nothing and returns QLORA_OK, except that a
 *     backward with accumulate = 0 writes zeros to dA and dB (the gradient
 *     of an empty batch). r = 0 means no LoRA branch (A, B, T, dA, dB may
 *     then be NULL).
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_BLOCK 64      /* weights per first-level block [QQ] */
#define QLORA_DQ_BLOCK 256  /* first-level scales per second-level block */
#define QLORA_MAX_RANK 128  /* largest supported LoRA rank */

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1, /* NULL where a buffer is needed, bad enum, misaligned */
  QLORA_ERR_SHAPE = -2,       /* K % 64 != 0, negative sizes, rank out of range */
  QLORA_ERR_UNSUPPORTED = -3, /* valid request the library does not implement */
  QLORA_ERR_WORKSPACE = -4,   /* workspace smaller than the matching *_workspace_bytes() */
  QLORA_ERR_HIP = -5,         /* a HIP launch or runtime call failed */
  QLORA_ERR_SCRATCH = -6      /* the call needs more than QLORA_SCRATCH_BYTES of library scratch */
} qlora_status;

typedef enum { QLORA_DT_BF16 = 0, QLORA_DT_FP32 = 1 } qlora_dtype;

/*
 * One encoded weight W [n, k]. All pointers are (device), owned by the caller.
 * Block b covers the 64 weights W[b / (k/64)][64 (b % (k/64)) ...], i.e. the
 * row-major flattening cut into runs of 64; blocks never straddle rows.
 *   codes    [n*k/2]  bytes; weight 2t in the low nibble of byte t, weight
 *                     2t+1 in the high nibble; a code indexes `codebook`.
 *   code8    [n*k/64] bytes; OCP FP8 E4M3 bit pattern of block b's centred,
 *                     scaled absmax [QX "Double Quantization"].
 *   s2       [ceil(n*k/64/256)] fp32 second-level scales, one per 256 blocks.
 *   mean     [1]      fp32 mean of all block absmax values.
 * Without double quantization (the ablation the pages weigh it against, QX
 * "Double Quantization"): code8 = NULL, s2 [n*k/64] holds every block's fp32
 * absmax and mean is not read (may be NULL); then c'_b = s2[b]. With
 * scale_bf16 = 1 as well (QQ's worked block and its 65B arithmetic: "one
 * BF16 scalar per 64-weight block", 4.25 bit per weight), s2 points to
 * n*k/64 uint16 bf16 bit patterns, c_b = RN_bf16(block absmax), the codes
 * are the nearest levels to w / c_b for that stored c_b, and c'_b = c_b
 * widened to fp32 (a block whose c_b is 0 stores code 7). scale_bf16 must be
 * 0 when code8 is set.
 *   codebook [16]     fp32 NF4 levels, ascending (from
 *                     qlora_build_nf4_codebook, copied to the device).
 * Block b's scale is c'_b = RN32(RN32(fp8(code8[b]) * s2[b/256]) + mean[0])
 * (two separately rounded fp32 operations) and its weight i expands to
 * w' = RN_bf16(RN32(codebook[code] * c'_b)).
 */
typedef struct {
  int64_t n;
  int64_t k;
  uint8_t *codes;
  uint8_t *code8;
  float *s2;
  float *mean;
  const float *codebook;
  int32_t scale_bf16; /* 0, or 1: per-block bf16 scales in s2 (code8 NULL only) */
} qlora_nf4_weight;

/* Storage forms of the block scales, for qlora_nf4_storage_bytes. */
typedef enum {
  QLORA_SCALE_FP32 = 0, /* one fp32 absmax per block (no double quantization) */
  QLORA_SCALE_DQ = 1,   /* double-quantized: code8 + s2 + mean */
  QLORA_SCALE_BF16 = 2  /* one bf16 absmax per block (no double quantization) */
} qlora_scale_form;

/* Name of a status code (static string, never NULL). */
const char *qlora_status_string(int status);

/*
 * The 16 NF4 levels into levels_out (host, 16 floats), ascending: index 0 is
 * -1, index 7 is exactly 0, index 15 is +1 [QQ "NF4: a 4-bit format matched
 * to weight statistics"; QX "4-Bit NormalFloat (NF4) Quantization"]. Eight
 * positive levels are standard-normal quantiles at the probabilities
 * 1/2 + (j/8)(delta - 1/2), j = 1..8, seven negative levels mirror the
 * quantiles at 1/2 + (j/7)(delta - 1/2), j = 1..7, with
 * delta = ((1 - 1/30) + (1 - 1/32)) / 2; all are divided by the quantile of
 * delta, evaluated in fp64 and rounded once to fp32. Pure host code; no HIP
 * call. Errors: INVALID_ARG if levels_out is NULL.
 */
qlora_status qlora_build_nf4_codebook(float *levels_out);

/* Bytes of the encoded weight (codes + code8 + s2 + mean, codebook excluded).
 * Returns 0 if k % 64 != 0 or a size is not positive. */
size_t qlora_nf4_packed_bytes(int64_t n, int64_t k);

/* Bytes of an encoded weight in a qlora_scale_form: QLORA_SCALE_DQ as
 * qlora_nf4_packed_bytes; QLORA_SCALE_FP32 codes + 4 bytes per block (4.5
 * bit per weight); QLORA_SCALE_BF16 codes + 2 bytes per block (4.25 bit,
 * QQ's "one BF16 scalar per 64-weight block"). 0 on bad arguments. */
size_t qlora_nf4_storage_bytes(int64_t n, int64_t k, int scale_form);

/*
 * The 16 levels of the uniform INT4 grid, the ablation the pages contrast
 * NF4 with (QQ "NF4: a 4-bit format matched to weight statistics": evenly
 * spaced code points), into levels_out (host, 16 floats): (i - 7) / 7 rounded
 * once to fp32, i = 0..15 -- -1 at index 0, exactly 0 at index 7 (the level
 * all-zero blocks and padding use), +1 at index 14; 8/7 at index 15 is never
 * chosen for absmax-scaled weights. Any 16 ascending levels with an exact 0
 * at index 7 can serve as a codebook. Pure host code.
 * Errors: INVALID_ARG if levels_out is NULL.
 */
qlora_status qlora_build_uniform4_codebook(float *levels_out);

/* Workspace bytes qlora_quantize_nf4 needs for an [n, k] weight (0 on bad shape). */
size_t qlora_quantize_workspace_bytes(int64_t n, int64_t k);

/*
 * Encode W (device, [n, k] row-major, bf16 or fp32 per w_dtype, finite) into
 * the buffers of *out (out->n, out->k must equal the shape; out->codebook must
 * hold the 16 levels) [QQ worked 8-weight block and "NF4: ..."; QX "Double
 * Quantization"]:
 *   c_b   = max |w| over block b (fp32, exact);
 *   code  = nearest level to w / c_b, ties to the lower level, evaluated as
 *           #{j : w > (L_j + L_{j+1})/2 * c_b} in exact fp64; c_b = 0 gives 7;
 *   mean  = (sum of c_b, added in fp64 left to right within each run of 256
 *           blocks, then run totals left to right) / nb, rounded to fp32;
 *   d_b   = RN32(c_b - mean); s2_j = RN32(max |d_b| over run j / 448);
 *   code8 = E4M3 pattern of the finite E4M3 value nearest to d_b / s2_j, ties
 *           to the lower value, -0 never produced; s2_j = 0 gives 0x00.
 * With out->code8 = NULL the second level is skipped: s2[b] = c_b; with
 * out->scale_bf16 = 1 as well, s2 (as uint16) receives RN_bf16(c_b) and the
 * codes are taken against that stored value.
 * ws (device) must hold qlora_quantize_workspace_bytes(n, k) bytes. The result
 * is deterministic and independent of the launch configuration.
 * Errors: INVALID_ARG (NULL/misaligned pointers, bad dtype), SHAPE (k % 64,
 * n or k < 1, shape mismatch), WORKSPACE, HIP.
 */
qlora_status qlora_quantize_nf4(const void *W, int w_dtype, const qlora_nf4_weight *out,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * Expand the whole weight to bf16: out (device, [n, k] bf16) receives exactly
 * the values the forward and backward kernels feed to the matrix cores
 * [QQ three-piece summary, piece 2 (compute in 16 bits)].
 * Errors: INVALID_ARG, SHAPE, HIP.
 */
qlora_status qlora_dequant(const qlora_nf4_weight *w, void *out, void *stream);

/* Workspace bytes for qlora_linear_fwd (is_bwd = 0) or qlora_linear_bwd
 * (is_bwd = 1) at this M, weight shape and rank (0 on bad arguments). */
size_t qlora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd);

/*
 * Forward [QQ three-piece summary and the storage/compute/learning diagram]:
 *   T = X A^T (fp32, written to T_save if not NULL),
 *   Y = RN_bf16( X W'^T + scale * T B^T ), accumulated in fp32.
 * X (device) [M, k] bf16; A (device) [r, k] bf16; B (device) [n, r] bf16;
 * Y (device) [M, n] bf16; T_save (device, nullable) [M, r] fp32;
 * scale = alpha / r, the LoRA scale [QX "Step 3"]. The kernels depend on M
 * (qlora_linear_path): a bandwidth-oriented dequant-GEMV for M <= 16, a
 * matrix-core GEMM expanding each 64-block in on-chip memory for medium M,
 * and for large M one expansion into workspace followed by a bf16 GEMM.
 * ws (device) must hold qlora_linear_workspace_bytes(M, n, k, r, 0) bytes.
 * Errors: INVALID_ARG, SHAPE, WORKSPACE, HIP.
 */
qlora_status qlora_linear_fwd(const qlora_nf4_weight *w, const void *X, int64_t M,
                              const void *A, const void *B, int r, float scale,
                              void *Y, float *T_save, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, kernels and results as qlora_linear_fwd;
 * the regions qlora_linear_fwd carves from ws come from a device array the
 * library owns instead: QLORA_SCRATCH_BYTES (64 MiB) per device, held from
 * the first call on that device until the process ends (the only memory the
 * library keeps; nothing is allocated or freed). The device is the one
 * `stream` belongs to. Every call on a device shares that device's array and
 * leaves its contents behind: calls that overlap on one device (two streams,
 * two host threads) race and must be serialized by the caller.
 * Errors: as qlora_linear_fwd; SCRATCH (before anything is enqueued) when
 * qlora_linear_workspace_bytes(M, n, k, r, 0) would exceed QLORA_SCRATCH_BYTES
 * (e.g. the expanded path of a large weight: use qlora_linear_fwd with a
 * workspace there).
 */
#define QLORA_SCRATCH_BYTES (64 << 20)
qlora_status qlora_linear_fwd_scratch(const qlora_nf4_weight *w, const void *X, int64_t M,
                                      const void *A, const void *B, int r, float scale,
                                      void *Y, float *T_save, void *stream);

/*
 * Backward [WQ "Key Characteristics": backpropagation through quantized
 * weights, adapters trained in full precision; QQ: the base gets no gradient]:
 *   U  = dY B                          (fp32, internal)
 *   dX = RN_bf16( dY W' + scale * U A ) (fp32 accumulate)   if dX != NULL
 *   dA = scale * U^T X                  (fp32, [r, k])       if dA != NULL
 *   dB = scale * dY^T T                 (fp32, [n, r])       if dB != NULL
 * T_saved (device, nullable) is the forward's T; if NULL it is recomputed from
 * X and A. X is needed when dA != NULL or T_saved == NULL. accumulate = 0
 * overwrites dA and dB, 1 adds to them (gradient accumulation). There is no
 * weight gradient. dA and dB are reduced in a fixed order: reruns are
 * bit-identical.
 * ws (device) must hold qlora_linear_workspace_bytes(M, n, k, r, 1) bytes.
 * Errors: INVALID_ARG, SHAPE, WORKSPACE, HIP.
 */
qlora_status qlora_linear_bwd(const qlora_nf4_weight *w, const void *X, const float *T_saved,
                              const void *dY, int64_t M, const void *A, const void *B, int r,
                              float scale, void *dX, float *dA, float *dB, int accumulate,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * The layer calls with dropout on the adapter's input, the LoRA dropout of the
 * pages' training configuration ("QLoRA Explained ..." (gamut.so), "Step 3:
 * Configure and Apply LoRA Adapters": 0.05):
 *   Y  = RN_bf16( X W'^T + scale ((X . D) A^T) B^T ),   D = mask * keep_scale
 *   dX = RN_bf16( dY W' + scale (U A) . D ),  U = dY B
 *   dA = scale U^T (X . D),   dB = scale dY^T ((X . D) A^T)
 * mask (device, uint8 [M, k], 16-byte aligned): nonzero keeps an element of X
 * for the branch; the caller draws it. keep_scale (>= 1, finite) is
 * 1 / (1 - p). The base product uses X itself. T_save / T_saved hold
 * (X . mask) A^T (without keep_scale; the backward applies it). Workspace:
 * qlora_linear_workspace_bytes, as for the plain calls; the branch's kernels
 * read X through the mask. Everything else, including the kernels chosen, is
 * as for qlora_linear_fwd / qlora_linear_bwd; r = 0 ignores mask.
 * Errors: as those calls, and INVALID_ARG for a NULL or misaligned mask or a
 * keep_scale below 1 or not finite.
 */
qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight *w, const void *X, int64_t M, const void *A,
                                      const void *B, int r, float scale, const void *mask, float keep_scale,
                                      void *Y, float *T_save, void *ws, size_t ws_bytes, void *stream);
qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight *w, const void *X, const float *T_saved,
                                      const void *dY, int64_t M, const void *A, const void *B, int r, float scale,
                                      const void *mask, float keep_scale, void *dX, float *dA, float *dB,
                                      int accumulate, void *ws, size_t ws_bytes, void *stream);

/*
 * The layer in fp16 instead of bf16, the other 16-bit compute type the pages
 * use ("QLoRA vs LoRA: How Quantized Low-Rank Adaptation Reduces Memory ..."
 * (instagit.com), "Implementation Guide", "QLoRA Fine-Tuning with 4-Bit
 * Quantization": a float16 compute dtype for the 4-bit base; "QLoRA
 * Explained ..." (gamut.so), the LoRA / QLoRA / full fine-tuning table:
 * fp16 or bf16 16-bit precision). Same storage, same arithmetic, with every 16-bit
 * value read or written in IEEE binary16 (round to nearest even):
 *   w'  = RN_fp16(RN32(L[code] * c'))            (qlora_dequant_f16)
 *   Y   = RN_fp16( X W'^T + scale * T B^T ),  dX = RN_fp16( dY W' + scale * U A )
 * X, A, B, Y, dY, dX and out (device) are fp16 in the layouts of the bf16
 * calls; T_save / T_saved, dA and dB stay fp32. The low-rank term enters the
 * products as fp16 hi / lo pairs of scale * T (and scale * U). Kernels: the
 * dequant-GEMV for M <= 16 in the forward, otherwise one expansion into
 * workspace followed by the 16-bit GEMM (the medium-M fused kernel is bf16
 * only). Workspace: qlora_linear_f16_workspace_bytes (is_bwd as for
 * qlora_linear_workspace_bytes). Values beyond the fp16 range (65504)
 * become infinities, as in any fp16 arithmetic; the caller scales.
 * Errors: as qlora_linear_fwd / qlora_linear_bwd, and UNSUPPORTED for a
 * backward with dX whose n is not a multiple of 8 (dA and dB alone are
 * computed at any n).
 */
qlora_status qlora_dequant_f16(const qlora_nf4_weight *w, void *out, void *stream);
size_t qlora_linear_f16_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd);
qlora_status qlora_linear_fwd_f16(const qlora_nf4_weight *w, const void *X, int64_t M,
                                  const void *A, const void *B, int r, float scale,
                                  void *Y, float *T_save, void *ws, size_t ws_bytes, void *stream);
qlora_status qlora_linear_bwd_f16(const qlora_nf4_weight *w, const void *X, const float *T_saved,
                                  const void *dY, int64_t M, const void *A, const void *B, int r,
                                  float scale, void *dX, float *dA, float *dB, int accumulate,
                                  void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Building blocks. qlora_linear_fwd and qlora_linear_bwd are compositions of
 * the calls below (same kernels, same order); they are exported so a caller
 * can reuse a low-rank activation it already has, or time each step.
 * ------------------------------------------------------------------------ */

/* Columns of the bf16 "split" rows the fused GEMMs take: 2r rounded up to a
 * multiple of 64 (0 for r = 0). */
int qlora_lowrank_split_cols(int r);

/* Workspace bytes of qlora_lowrank_project (0 on bad arguments). */
size_t qlora_lowrank_project_workspace_bytes(int64_t M, int64_t C, int r);

/*
 * Low-rank projection of an activation [QQ three-piece summary, piece 3]:
 *   out[m, j] = sum_c P[m, c] Q(c, j)        (fp32; T = X A^T or U = dY B)
 * P (device) [M, C] bf16; Q (device) bf16, q_layout 0: Q is [r, C] (j-major,
 * as A), 1: Q is [C, r] (as B). out (device, nullable) [M, r] fp32. If split
 * (device, nullable, [M, qlora_lowrank_split_cols(r)] bf16) is given, row m
 * receives [hi | lo | zeros] with hi_j = RN_bf16(scale * out[m, j]) and
 * lo_j = RN_bf16(scale * out[m, j] - hi_j): the 2r extra contraction columns
 * the fused GEMMs use to add the low-rank term in fp32. bf16 products, fp32
 * sums; the contraction is split over workgroups and added in a fixed order.
 * Errors: INVALID_ARG, SHAPE (r < 1 or > QLORA_MAX_RANK), WORKSPACE, HIP.
 */
qlora_status qlora_lowrank_project(const void *P, int64_t M, int64_t C, const void *Q, int q_layout, int r,
                                   float scale, float *out, void *split, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * Fused forward GEMM [QQ three-piece summary, piece 2; "Batched 4-bit matmuls"]:
 *   Y = RN_bf16( X W'^T + split [B | B]^T )
 * i.e. the base product with every 64-block expanded to bf16 on chip, plus the
 * low-rank term when split = qlora_lowrank_project(X, A, scale) and B
 * (device, [n, r] bf16). r = 0: split and B are ignored. M >= 1, any size.
 * Errors: INVALID_ARG, SHAPE, HIP.
 */
qlora_status qlora_nf4_gemm_fwd(const qlora_nf4_weight *w, const void *X, int64_t M, const void *split,
                                const void *B, int r, void *Y, void *stream);

/*
 * Fused backward-data GEMM through the frozen base [WQ "Key Characteristics"]:
 *   dX = RN_bf16( dY W' + split [A ; A] )
 * dY (device) [M, n] bf16; split = qlora_lowrank_project(dY, B, scale) rows;
 * A (device) [r, k] bf16. The contraction runs over n, so each 64-block is
 * expanded transposed into on-chip memory. Errors: INVALID_ARG, SHAPE, HIP.
 */
qlora_status qlora_nf4_gemm_dx(const qlora_nf4_weight *w, const void *dY, int64_t M, const void *split,
                               const void *A, int r, void *dX, void *stream);

/* Workspace bytes of qlora_nf4_gemv_fwd for a weight with k columns (0 on a
 * bad k): the activations rewritten in the kernel's operand order. */
size_t qlora_nf4_gemv_workspace_bytes(int64_t k);

/*
 * Bandwidth-oriented forward for M <= 16 tokens:
 *   Y = RN_bf16( X W'^T + scale T B^T ),   T (device, [M, r] fp32) = X A^T.
 * One pass over the packed codes, addressed with 32-bit offsets: the codes
 * plus 256 rows' worth ((n + 256) k / 2 bytes) must stay under 4 GiB. ws
 * (device, 16-byte aligned) holds qlora_nf4_gemv_workspace_bytes(k) bytes.
 * Errors: INVALID_ARG, SHAPE (M > 16, or the codes too large), WORKSPACE, HIP.
 */
qlora_status qlora_nf4_gemv_fwd(const qlora_nf4_weight *w, const void *X, int64_t M, const float *T,
                                const void *B, int r, float scale, void *Y, void *ws, size_t ws_bytes,
                                void *stream);

/* Workspace bytes of qlora_nf4_gemv_dx for an [n, k] weight (0 on bad
 * arguments): fp32 partial sums of the contraction's row ranges. */
size_t qlora_nf4_gemv_dx_workspace_bytes(int64_t n, int64_t k);

/*
 * Bandwidth-oriented dX for M <= 16 tokens [WQ "Key Characteristics";
 * QQ "Batched 4-bit matmuls"]:
 *   dX = RN_bf16( dY W' + scale U A ),   U (device, [M, r] fp32) = dY B.
 * dY (device) [M, n] bf16, A (device) [r, k] bf16, dX (device) [M, k] bf16.
 * One pass over the packed codes: row ranges of the contraction each write
 * fp32 partials (ws, qlora_nf4_gemv_dx_workspace_bytes(n, k) bytes), added in
 * range order with the low-rank term (fp32) and rounded once.
 * Errors: INVALID_ARG, SHAPE (M > 16), WORKSPACE, HIP.
 */
qlora_status qlora_nf4_gemv_dx(const qlora_nf4_weight *w, const void *dY, int64_t M, const float *U,
                               const void *A, int r, float scale, void *dX, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Which kernels a pass uses at this size; qlora_linear_fwd (is_bwd = 0) and
 * qlora_linear_bwd (is_bwd = 1, the dX product) make exactly this choice:
 *   QLORA_PATH_GEMV      M <= 16: qlora_nf4_gemv_fwd (codes within its
 *                        4 GiB limit; else the forward is FUSED), or for dX
 *                        qlora_nf4_gemv_dx (one pass over the packed codes,
 *                        bandwidth-bound);
 *   QLORA_PATH_FUSED     qlora_nf4_gemm_fwd / qlora_nf4_gemm_dx (each 64-block
 *                        expanded in on-chip memory, once per 256-row tile);
 *   QLORA_PATH_EXPANDED  M >= QLORA_EXPAND_MIN_M (and n % 8 == 0 for dX, and
 *                        every operand of the bf16 GEMM under 4 GiB):
 *                        qlora_nf4_expand once into workspace, then
 *                        qlora_bf16_gemm (each weight expanded once per pass
 *                        instead of M / 256 times); for dX with n % 64 == 0
 *                        (bf16, no dropout) qlora_nf4_expand with
 *                        transposed = 2, then qlora_bf16_gemm_nn.
 * r is the LoRA rank. Returns -1 on bad arguments.
 */
#define QLORA_PATH_GEMV 0
#define QLORA_PATH_FUSED 1
#define QLORA_PATH_EXPANDED 2
#define QLORA_EXPAND_MIN_M 128
int qlora_linear_path(int64_t M, int64_t n, int64_t k, int r, int is_bwd);

/* Bytes of the expanded operand of qlora_nf4_expand (0 on bad arguments). */
size_t qlora_nf4_expand_bytes(int64_t n, int64_t k, int r, int transposed);

/*
 * Expand the encoded weight once to the bf16 operand of qlora_bf16_gemm
 * [QQ three-piece summary, piece 2: expand to 16 bits right before the
 * multiply], with the LoRA factor appended as xc = qlora_lowrank_split_cols(r)
 * extra contraction columns:
 *   transposed = 0 (forward): out [n, k + xc],  out[i, c] = W'[i, c],
 *       out[i, k + j] = B[i, j mod r] for j < 2r, else 0;  lr = B [n, r].
 *   transposed = 1 (dX): np = n rounded up to 64, out [k, np + xc],
 *       out[c, i] = W'[i, c] (0 for n <= i < np),
 *       out[c, np + j] = A[j mod r, c] for j < 2r, else 0;  lr = A [r, k].
 *   transposed = 2 (dX, contraction-major operand of qlora_bf16_gemm_nn;
 *       n % 64 == 0, else SHAPE): out [n + xc, k], out[i, c] = W'[i, c],
 *       out[n + j, c] = A[j mod r, c] for j < 2r, else 0;  lr = A [r, k].
 *       The W' rows are the forward's layout, which expands with 16-byte
 *       stores along rows instead of a transpose through on-chip memory.
 * W' values are bit-identical to qlora_dequant's. out (device) must hold
 * qlora_nf4_expand_bytes(n, k, r, transposed) bytes (out_bytes).
 * Errors: INVALID_ARG, SHAPE, WORKSPACE (out_bytes too small), HIP.
 */
qlora_status qlora_nf4_expand(const qlora_nf4_weight *w, const void *lr, int r, int transposed, void *out,
                              size_t out_bytes, void *stream);

/* Workspace bytes of qlora_bf16_gemm (0: none needed, or bad arguments). */
size_t qlora_bf16_gemm_workspace_bytes(int64_t M, int64_t kc, int r, int64_t nout);

/*
 * bf16 MFMA GEMM over an expanded operand F from qlora_nf4_expand:
 *   out[m, j] = RN_bf16( sum_{c < kc} act[m, c] F[j, c] + sum_x split[m, x] F[j, kcp + x] )
 * act (device) [M, kc] bf16 (X with kc = k for the forward, dY with kc = n
 * for dX; kc % 8 == 0); kcp = kc rounded up to 64; split (device) [M, xc]
 * bf16 rows from qlora_lowrank_project (ignored for r = 0); F (device)
 * [nout, kcp + xc]; out (device) [M, nout] bf16 (nout = n forward, k for dX).
 * Each operand (act, split, F) must be smaller than 4 GiB.
 * The 256 x 256 output tiles run in waves of 256 (one per compute unit).
 * When the last wave holds at most 128 tiles (all of them, for outputs of at
 * most 128 tiles), each of those tiles has its contraction split over 2-8
 * workgroups: their fp32 partial sums go to ws
 * (device, qlora_bf16_gemm_workspace_bytes; may be NULL when that is 0) and
 * are added in split order, then rounded once. Results are deterministic;
 * they can differ in the last bits from an unsplit sum.
 * Errors: INVALID_ARG, SHAPE, WORKSPACE, HIP.
 */
qlora_status qlora_bf16_gemm(const void *act, int64_t M, int64_t kc, const void *split, int r, const void *F,
                             int64_t nout, void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * The same product over a contraction-major operand F from qlora_nf4_expand
 * with transposed = 2 [QQ three-piece summary, piece 2; the dX product of the
 * backward pass]:
 *   out[m, j] = RN_bf16( sum_{c < kc} act[m, c] F[c, j] + sum_x split[m, x] F[kc + x, j] )
 * act (device) [M, kc] bf16 (dY, kc = n, kc % 64 == 0); split (device)
 * [M, xc] bf16 from qlora_lowrank_project (ignored for r = 0); F (device)
 * [kc + xc, nout] (nout = k, nout % 8 == 0); out (device) [M, nout] bf16.
 * Workspace and splitting as qlora_bf16_gemm
 * (qlora_bf16_gemm_workspace_bytes(M, kc, r, nout)). Each operand must be
 * smaller than 4 GiB. Deterministic; may differ in the last bits from
 * qlora_bf16_gemm over the transposed operand (a different summation order
 * inside each 64-wide step).
 * Errors: INVALID_ARG, SHAPE, WORKSPACE, HIP.
 */
qlora_status qlora_bf16_gemm_nn(const void *act, int64_t M, int64_t kc, const void *split, int r, const void *F,
                                int64_t nout, void *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of qlora_lowrank_grad (0 on bad arguments). */
size_t qlora_lowrank_grad_workspace_bytes(int64_t M, int64_t C, int r);

/*
 * Adapter gradient, a reduction over the M tokens [QQ: all updates land on the
 * low-rank branch]:
 *   G(c, j) (+)= scale * sum_m P[m, c] Q[m, j]
 * P (device) [M, C] bf16; Q (device) [M, r] fp32; G (device) fp32 with
 * g_layout 0: G is [r, C] (dA = s U^T X), 1: G is [C, r] (dB = s dY^T T).
 * accumulate 0 overwrites, 1 adds. fp32 products and sums, reduced over M in
 * a fixed order (bit-identical reruns).
 * Errors: INVALID_ARG, SHAPE, WORKSPACE, HIP.
 */
qlora_status qlora_lowrank_grad(const void *P, int64_t M, int64_t C, const float *Q, int r, float scale, float *G,
                                int g_layout, int accumulate, void *ws, size_t ws_bytes, void *stream);

/*
 * The same layer over a bf16 base weight (LoRA without quantization): the
 * comparison the pages draw for QLoRA's speed ("QLoRA Explained ..."
 * (gamut.so), "QLoRA vs LoRA: Memory, Speed, and Quality Tradeoffs": a 16-bit
 * base trains faster, no dequantization overhead; QQ "Two prices to know",
 * price 1: every QLoRA matmul pays for unpacking).
 *   forward:  T = X A^T,  Y = RN_bf16( X W^T + scale * T B^T )
 *   backward: U = dY B,  dX = RN_bf16( dY W + scale * U A ),
 *             dA = scale * U^T X,  dB = scale * dY^T T
 * W (device) [n, k] bf16 row-major, k % 64 == 0; every other argument, the
 * nullable outputs, accumulate and the workspace rules as in
 * qlora_linear_fwd / qlora_linear_bwd, workspace sizes from
 * qlora_lora_linear_workspace_bytes (0 on bad arguments). The low-rank
 * kernels are the QLoRA layer's; the forward multiplies W as stored, dX
 * copies W's tiles where the QLoRA layer expands 4-bit ones.
 * Errors: INVALID_ARG, SHAPE (also when k % 64 != 0), WORKSPACE, HIP.
 */
size_t qlora_lora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r, int is_bwd);
qlora_status qlora_lora_linear_fwd(const void *W, int64_t n, int64_t k, const void *X, int64_t M,
                                   const void *A, const void *B, int r, float scale, void *Y,
                                   float *T_save, void *ws, size_t ws_bytes, void *stream);
qlora_status qlora_lora_linear_bwd(const void *W, int64_t n, int64_t k, const void *X,
                                   const float *T_saved, const void *dY, int64_t M, const void *A,
                                   const void *B, int r, float scale, void *dX, float *dA, float *dB,
                                   int accumulate, void *ws, size_t ws_bytes, void *stream);

/*
 * The gated-MLP join used between the gate/up and down linears of the MLP
 * workloads (not a QLoRA operation; provided so a whole MLP block runs on
 * this library):
 *   forward:  H = RN_bf16( silu(G) * Up ),  silu(g) = g / (1 + exp(-g))
 *   backward: dG = RN_bf16( dH * Up * silu'(g) ), dUp = RN_bf16( dH * silu(g) )
 * All tensors (device) bf16 with `count` elements; math in fp32.
 * Errors: INVALID_ARG, SHAPE, HIP.
 */
qlora_status qlora_silu_mul_fwd(const void *G, const void *Up, void *H, int64_t count, void *stream);
qlora_status qlora_silu_mul_bwd(const void *G, const void *Up, const void *dH, void *dG, void *dUp,
                                int64_t count, void *stream);

/*
 * Adapter merge for deployment ["QLoRA: Quantized Low-Rank Adaptation"
 * (completesystemdesign.dev), the two prices, price 2: a 4-bit base cannot
 * absorb the trained delta, so the adapter is added onto a dequantized copy;
 * "QLoRA vs LoRA ..." (instagit.com), converting back to full precision]:
 *   out[i, c] = round( W'[i, c] + scale * sum_j B[i, j] A[j, c] )
 * W' = the bf16 expansion of w (bit-identical to qlora_dequant); A (device)
 * [r, k] bf16, B (device) [n, r] bf16 (the trained adapter), scale = alpha / r
 * as in the forward pass; out (device) [n, k] of out_dtype: QLORA_DT_BF16
 * (rounded once, nearest-even) or QLORA_DT_FP32. The sum over j is an fp32
 * matrix-core sum of exact bf16 products; scale * sum and the addition are
 * single fp32 operations. r = 0 writes W' (A, B may be NULL).
 * Errors: INVALID_ARG, SHAPE, HIP.
 */
qlora_status qlora_adapter_merge(const qlora_nf4_weight *w, const void *A, const void *B, int r, float scale,
                                 void *out, int out_dtype, void *stream);

/*
 * Inverse of the bf16 merge (swap adapters on a merged copy):
 *   out[i, c] = RN_bf16( merged[i, c] - scale * sum_j B[i, j] A[j, c] )
 * merged, out (device) [n, k] bf16, k % 64 == 0; out may equal merged (each
 * tile is read whole before it is written). The result equals W' only where
 * that rounding lands back on it: the merged copy was itself rounded.
 * Errors: INVALID_ARG, SHAPE, HIP.
 */
qlora_status qlora_adapter_unmerge(const void *merged, int64_t n, int64_t k, const void *A, const void *B, int r,
                                   float scale, void *out, void *stream);

/*
 * One AdamW step over the adapter's parameters ["QLoRA Explained ..."
 * (gamut.so), "Paged Optimizers" and the quick reference: the 32-bit paged
 * AdamW; "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
 * paged optimizers: states in pinned CPU RAM]. Per element, fp32, each
 * operation rounded separately:
 *   m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g g,
 *   theta <- theta - lr ( (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) + wd theta )
 * (1 - b1, 1 - b2 and the bias corrections are formed in fp64 on the host and
 * rounded once). theta (device, fp32 master copy), grad (device, fp32, e.g.
 * dA or dB), m and v (fp32 states: device memory, or host memory pinned with
 * hipHostMalloc, updated in place through its device mapping) hold `count`
 * elements; theta16 (device, nullable) receives RN_bf16(theta), the adapter
 * copy the layer calls read. step t >= 1 (bias correction); lr is the
 * learning rate of this step (the schedule is the caller's).
 * All pointers 16-byte aligned. Errors: INVALID_ARG (NULL, misaligned,
 * hyperparameters out of range, states in pageable host memory), SHAPE
 * (count < 0, step < 1), HIP.
 */
qlora_status qlora_adamw_step(float *theta, uint16_t *theta16, const float *grad, float *m, float *v, int64_t count,
                              int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                              void *stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers (not part of the layer): attainable peaks on the box at
 * hand, reported beside the published ones.
 *
 * qlora_calib_mfma: `blocks` workgroups of 8 waves; each wave runs `iters`
 * rounds of 8 independent v_mfma_f32_32x32x16_bf16 with no memory traffic.
 * Work = blocks * 8 * iters * 8 * 32768 flops. `sink` (device, 1 fp32) is
 * written only in a case that never occurs (it keeps the work alive).
 * Errors: INVALID_ARG (blocks or iters < 1, sink NULL), HIP.
 *
 * qlora_calib_stream_read: reads `bytes` (multiple of 16) of `buf` (device,
 * 16-byte aligned) once with 16-byte loads, grid-stride, four loads in flight
 * per thread; `sink` as above. Errors: INVALID_ARG, SHAPE (alignment or size),
 * HIP.
 * ------------------------------------------------------------------------- */
qlora_status qlora_calib_mfma(int blocks, int iters, float *sink, void *stream);
qlora_status qlora_calib_stream_read(const void *buf, int64_t bytes, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
