// Expansion of an encoded NF4 weight, once per pass, into the bf16 operand of
// the plain MFMA GEMM used at large token counts.
//
// "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// three-piece summary, piece 2, and "Batched 4-bit matmuls": storage stays
// 4-bit, and the weight is expanded to bf16 right before the 16-bit multiply.
// At large M a fused kernel would expand every weight once per 256-row output
// tile (M / 256 times); expanding it once into workspace and streaming the
// bf16 copy through a plain GEMM costs 2 extra bytes written and read per
// weight instead.
//
// The LoRA factor rides along as extra contraction columns, so the GEMM
// rounds its output once (see the low-rank split in lora.hip):
//   forward operand  F [n, k + xc]:    F[i, c] = W'[i, c]           c <  k
//                                      F[i, k + j] = B[i, j mod r]  j <  2r, else 0
//   dX operand       G [k, np + xc]:   G[c, i] = W'[i, c]           i <  n, 0 for n <= i < np
//                                      G[c, np + j] = A[j mod r, c] j <  2r, else 0
// with xc = lora_extra_cols(r) and np = n rounded up to a multiple of 64.
// Values are bit-identical to qlora_dequant's.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

// Row expansion: one thread per 16-byte output chunk column (8 bf16 = one
// 32-bit code word) of kRows consecutive weight rows. Workgroup (x, y) covers
// chunks 256 y .. 256 y + 255 of rows kRows x .. kRows x + kRows - 1: every
// store instruction of a wavefront writes 1 KB of contiguous output, and a
// thread issues all kRows code-word and scale loads before its first store,
// so each workgroup keeps kRows round trips to memory in flight instead of
// one. Workgroups with y equal to the number of code-chunk blocks write the
// LoRA columns of their rows.
constexpr int kRows = 8;

// kF16 (both expansions): the operand written in fp16 instead of bf16, w'
// and the low-rank columns alike (the compute-type ablation).
template <bool kF16>
__global__ __launch_bounds__(256) void expand_rows_kernel(const uint32_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ code8,
                                                          const float* __restrict__ s2,
                                                          const float* __restrict__ mean_p,
                                                          const float* __restrict__ codebook, bool s2_bf16,
                                                          int64_t n, int64_t k, const uint16_t* __restrict__ B, int r,
                                                          int xc, u32x4* __restrict__ out) {
  const int t = threadIdx.x;
  const int64_t kw = k / 8;
  const int64_t ldc = (k + xc) / 8;  // output row pitch in chunks
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  if ((int64_t)blockIdx.y * 256 >= kw) {
    // LoRA columns of rows r0 .. r0 + kRows - 1 (kRows * xc / 8 <= 256 threads for r <= 128)
    const int cpr = xc / 8;
    if (t >= kRows * cpr) return;
    const int64_t rr = r0 + t / cpr;
    const int j0 = (t % cpr) * 8;
    if (rr >= n) return;
    u32x4 v;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int j = j0 + 2 * p + e;
        h[e] = j < 2 * r ? (uint32_t)B[rr * r + (j % r)] : 0u;
      }
      v[p] = h[0] | (h[1] << 16);
    }
    out[rr * ldc + kw + t % cpr] = v;
    return;
  }
  __shared__ float lut[16];
  if (t < 16) lut[t] = codebook[t];
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.y * 256 + t;
  if (c >= kw) return;
  const float mean = weight_mean(code8, mean_p);
  uint32_t word[kRows], c8[kRows];
  float s2v[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t row = r0 + i < n ? r0 + i : n - 1;  // rows past n repeat the last one (not stored)
    const int64_t wi = row * kw + c;                  // code word index
    word[i] = codes[wi];
    scale_fields(code8, s2, s2_bf16, wi >> 3, c8[i], s2v[i]);
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    if (r0 + i < n) out[(r0 + i) * ldc + c] = dequant8<kF16>(word[i], lut, decode_block_scale(c8[i], s2v[i], mean));
}

// Transposing expansion, straight from registers. Workgroup (tn, kb) covers
// weight rows n0 .. n0+255 and k-block kb: thread t takes rows 2 (t % 128)
// and +1, half (t / 128) of the block (32 weights each), and for every one of
// its 32 k writes the (row pair) as one 4-byte word of output row k. A
// wavefront's 64 lanes thus write 256 contiguous bytes per store. Rows in
// [n, np) are written as zeros; workgroups with tn == number of n tiles write
// the low-rank columns of their 64 k rows.
// Order: the four k-blocks of one 128-byte code line (kb = 4 g .. 4 g + 3)
// get workgroup ids 8 apart, i.e. the same XCD (ids go to XCDs round-robin)
// at nearly the same time, so each line is fetched into one L2 once.
constexpr int kXT = 256;  // weight rows per tile

__device__ __forceinline__ bool cols_unit(int64_t ntiles1, int64_t kblocks, int64_t& tn, int64_t& kb) {
  const int64_t b = blockIdx.x;
  const int64_t x = b % 8, q = b / 8;
  const int64_t j = q % 4, p = q / 4;
  const int64_t kg = cdiv(kblocks, (int64_t)4);
  const int64_t u = p * 8 + x;  // (tile, line group) unit
  if (u >= ntiles1 * kg) return false;
  tn = u / kg;
  kb = 4 * (u % kg) + j;
  return kb < kblocks;
}

template <bool kF16>
__global__ __launch_bounds__(256) void expand_cols_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ code8,
                                                          const float* __restrict__ s2,
                                                          const float* __restrict__ mean_p,
                                                          const float* __restrict__ codebook, bool s2_bf16,
                                                          int64_t n, int64_t k, int64_t np,
                                                          const uint16_t* __restrict__ A, int r, int xc,
                                                          uint16_t* __restrict__ out) {
  __shared__ float lut[16];
  const int t = threadIdx.x;
  const int64_t ldo = np + xc;
  const int64_t ntiles = (np + kXT - 1) / kXT;
  int64_t tn, kb;
  if (!cols_unit(ntiles + (xc > 0 ? 1 : 0), k / kBlock, tn, kb)) return;
  if (tn == ntiles) {
    // low-rank columns: out[kb*64 + row, np + j]
    for (int idx = t; idx < 64 * xc; idx += 256) {
      const int row = idx / xc, j = idx - row * xc;
      const int64_t c = kb * kBlock + row;
      out[c * ldo + np + j] = j < 2 * r ? A[(int64_t)(j % r) * k + c] : (uint16_t)0;
    }
    return;
  }
  if (t < 16) lut[t] = codebook[t];
  __syncthreads();
  const float mean = weight_mean(code8, mean_p);
  const int64_t n0 = tn * kXT;
  const int pr = t & 127, half = t >> 7;
  const int64_t na = n0 + 2 * pr, nb = na + 1;
  if (na >= np) return;  // np is a multiple of 64: the pair is in or out together
  u32x4 qa = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
  u32x4 qb = qa;
  float ca = 0.0f, cb = 0.0f;
  const int64_t kblocks = k / kBlock;
  if (na < n) {
    qa = *reinterpret_cast<const u32x4*>(codes + na * (k / 2) + kb * 32 + half * 16);
    ca = block_scale(code8, s2, s2_bf16, mean, na * kblocks + kb);
  }
  if (nb < n) {
    qb = *reinterpret_cast<const u32x4*>(codes + nb * (k / 2) + kb * 32 + half * 16);
    cb = block_scale(code8, s2, s2_bf16, mean, nb * kblocks + kb);
  }
  // rows past n decode code 7 (level 0) times scale 0: exact zeros
  uint32_t* dst = reinterpret_cast<uint32_t*>(out + (kb * kBlock + half * 32) * ldo + na);
  const int64_t ldw = ldo / 2;  // output row pitch in 4-byte words
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float va = nf4_scaled(lut[(qa[w] >> (4 * e)) & 0xF], ca);
      const float vb = nf4_scaled(lut[(qb[w] >> (4 * e)) & 0xF], cb);
      dst[(w * 8 + e) * ldw] = pack2<kF16>(va, vb);
    }
}

// Low-rank operand rows alone, [n, xc]: row i = [B[i, :] | B[i, :] | 0 ...]
// (the columns the row expansion appends to W'), for a GEMM whose weight
// operand is a separate matrix. One thread per 8 output columns.
__global__ __launch_bounds__(256) void lowrank_rows_kernel(const uint16_t* __restrict__ B, int64_t n, int r, int xc,
                                                           u32x4* __restrict__ out) {
  const int cpr = xc / 8;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n * cpr) return;
  const int64_t i = q / cpr;
  const int j0 = (int)(q % cpr) * 8;
  u32x4 v;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = j0 + 2 * p + e;
      h[e] = j < 2 * r ? (uint32_t)B[i * r + (j % r)] : 0u;
    }
    v[p] = h[0] | (h[1] << 16);
  }
  out[q] = v;
}

// [xc, k] rows [A ; A ; 0]: row x is A's row x % r for x < 2r, zeros after.
__global__ __launch_bounds__(256) void lowrank_cols_kernel(const uint16_t* __restrict__ A, int r, int xc, int64_t k,
                                                           u32x4* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = k / 8;
  if (q >= (int64_t)xc * cpr) return;
  const int x = (int)(q / cpr);
  const int64_t c = (q % cpr) * 8;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (x < 2 * r) v = *reinterpret_cast<const u32x4*>(A + (int64_t)(x % r) * k + c);
  out[q] = v;
}

}  // namespace

hipError_t launch_lowrank_cols(const uint16_t* A, int r, int64_t k, uint16_t* out, hipStream_t stream) {
  const int xc = lora_extra_cols(r);
  if (xc == 0 || k == 0) return hipSuccess;
  const int64_t total = (int64_t)xc * (k / 8);
  lowrank_cols_kernel<<<(unsigned)cdiv(total, (int64_t)256), 256, 0, stream>>>(A, r, xc, k,
                                                                               reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_lowrank_rows(const uint16_t* B, int64_t n, int r, uint16_t* out, hipStream_t stream) {
  const int xc = lora_extra_cols(r);
  if (xc == 0 || n == 0) return hipSuccess;
  const int64_t total = n * (xc / 8);
  lowrank_rows_kernel<<<(unsigned)cdiv(total, (int64_t)256), 256, 0, stream>>>(B, n, r, xc,
                                                                               reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

int64_t expand_pad_rows(int64_t n) { return cdiv(n, (int64_t)kBlock) * kBlock; }

size_t expand_ws_bytes(int64_t n, int64_t k, int r, bool transposed) {
  const int xc = lora_extra_cols(r);
  if (!transposed) return align256((size_t)n * (size_t)(k + xc) * 2);
  return align256((size_t)k * (size_t)(expand_pad_rows(n) + xc) * 2);
}

hipError_t launch_expand(const Nf4View& w, const uint16_t* lr, int r, bool transposed, uint16_t* out,
                         hipStream_t stream, bool f16) {
  const int xc = lora_extra_cols(r);
  if (!transposed) {
    const int64_t kw = w.k / 8;
    const dim3 grid((unsigned)cdiv(w.n, (int64_t)kRows), (unsigned)(cdiv(kw, (int64_t)256) + (xc > 0 ? 1 : 0)));
    auto* cw = reinterpret_cast<const uint32_t*>(w.codes);
    auto* o4 = reinterpret_cast<u32x4*>(out);
    if (f16)
      expand_rows_kernel<true><<<grid, 256, 0, stream>>>(cw, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16, w.n, w.k,
                                                         lr, r, xc, o4);
    else
      expand_rows_kernel<false><<<grid, 256, 0, stream>>>(cw, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16, w.n, w.k,
                                                          lr, r, xc, o4);
  } else {
    const int64_t np = expand_pad_rows(w.n);
    const int64_t ntiles = cdiv(np, (int64_t)kXT);
    const int64_t units = (ntiles + (xc > 0 ? 1 : 0)) * cdiv(w.k / kBlock, (int64_t)4);
    const dim3 grid((unsigned)(cdiv(units, (int64_t)8) * 8 * 4));
    if (f16)
      expand_cols_kernel<true><<<grid, 256, 0, stream>>>(w.codes, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16, w.n,
                                                         w.k, np, lr, r, xc, out);
    else
      expand_cols_kernel<false><<<grid, 256, 0, stream>>>(w.codes, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16, w.n,
                                                          w.k, np, lr, r, xc, out);
  }
  return hipGetLastError();
}

size_t expand_nn_bytes(int64_t n, int64_t k, int r) {
  return align256((size_t)(n + lora_extra_cols(r)) * (size_t)k * 2);
}

hipError_t launch_expand_nn(const Nf4View& w, const uint16_t* A, int r, uint16_t* out, hipStream_t stream) {
  hipError_t e = launch_expand(w, nullptr, 0, false, out, stream);
  if (e == hipSuccess && r > 0) e = launch_lowrank_cols(A, r, w.k, out + w.n * w.k, stream);
  return e;
}

}  // namespace qlora
