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

// One thread per 16-byte output chunk (8 bf16): consecutive threads write
// consecutive chunks of a row, and read consecutive 32-bit code words.
__global__ __launch_bounds__(256) void expand_rows_kernel(const uint32_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ code8,
                                                          const float* __restrict__ s2,
                                                          const float* __restrict__ mean_p,
                                                          const float* __restrict__ codebook, int64_t n, int64_t k,
                                                          const uint16_t* __restrict__ B, int r, int xc,
                                                          u32x4* __restrict__ out) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const float mean = mean_p[0];
  const int64_t row_chunks = (k + xc) / 8;
  const int64_t total = n * row_chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / row_chunks;
    const int64_t c = (i - row * row_chunks) * 8;
    u32x4 v;
    if (c < k) {
      const float cp = block_scale(code8, s2, mean, row * (k / kBlock) + c / kBlock);
      v = dequant8(codes[(row * k + c) / 8], lut, cp);
    } else {
      const int j0 = (int)(c - k);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = j0 + 2 * p + e;
          h[e] = j < 2 * r ? (uint32_t)B[row * r + (j % r)] : 0u;
        }
        v[p] = h[0] | (h[1] << 16);
      }
    }
    out[i] = v;
  }
}

// Transposing expansion. Workgroup (tn, kb) expands k-block kb (64 weights)
// of 256 weight rows n0 .. n0+255 into LDS as [64 k][256 n] and writes the 64
// output rows' 512-byte segments. Thread t takes weight rows 2 (t % 128) and
// +1 and half (t / 128) of the block, so its LDS writes are (row pair) dwords
// and a wavefront writes 64 consecutive dwords of one k row. Workgroups with
// tn == number of n tiles write the low-rank columns of their 64 k rows.
constexpr int kXT = 256;  // weight rows per tile

__global__ __launch_bounds__(256) void expand_cols_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ code8,
                                                          const float* __restrict__ s2,
                                                          const float* __restrict__ mean_p,
                                                          const float* __restrict__ codebook, int64_t n, int64_t k,
                                                          int64_t np, const uint16_t* __restrict__ A, int r, int xc,
                                                          uint16_t* __restrict__ out) {
  __shared__ float lut[16];
  __shared__ __attribute__((aligned(16))) uint32_t tile[64][kXT / 2];
  const int t = threadIdx.x;
  const int64_t ldo = np + xc;
  const int64_t kb = blockIdx.y;
  const int64_t ntiles = (np + kXT - 1) / kXT;
  if ((int64_t)blockIdx.x == ntiles) {
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
  const float mean = mean_p[0];
  const int64_t n0 = (int64_t)blockIdx.x * kXT;
  const int pr = t & 127, half = t >> 7;
  const int64_t na = n0 + 2 * pr, nb = na + 1;
  uint32_t qa[4] = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
  uint32_t qb[4] = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
  float ca = 0.0f, cb = 0.0f;
  const int64_t kblocks = k / kBlock;
  if (na < n) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes + na * (k / 2) + kb * 32 + half * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) qa[j] = v[j];
    ca = block_scale(code8, s2, mean, na * kblocks + kb);
  }
  if (nb < n) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes + nb * (k / 2) + kb * 32 + half * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = v[j];
    cb = block_scale(code8, s2, mean, nb * kblocks + kb);
  }
  // rows past n decode code 7 (level 0) times scale 0: exact zeros
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float va = nf4_scaled(lut[(qa[w] >> (4 * e)) & 0xF], ca);
      const float vb = nf4_scaled(lut[(qb[w] >> (4 * e)) & 0xF], cb);
      tile[half * 32 + w * 8 + e][pr] = pack_bf16x2(va, vb);
    }
  __syncthreads();
  // 64 rows x 512 bytes = 2048 chunks of 16 B; chunk q: row q / 32, col chunk q % 32
  const int64_t ncols = np - n0 < kXT ? np - n0 : kXT;  // multiple of 64
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 5, ch = q & 31;
    if (ch * 8 < ncols) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[row][ch * 4]);
      *reinterpret_cast<u32x4*>(out + (kb * kBlock + row) * ldo + n0 + ch * 8) = v;
    }
  }
}

}  // namespace

int64_t expand_pad_rows(int64_t n) { return cdiv(n, (int64_t)kBlock) * kBlock; }

size_t expand_ws_bytes(int64_t n, int64_t k, int r, bool transposed) {
  const int xc = lora_extra_cols(r);
  if (!transposed) return align256((size_t)n * (size_t)(k + xc) * 2);
  return align256((size_t)k * (size_t)(expand_pad_rows(n) + xc) * 2);
}

hipError_t launch_expand(const Nf4View& w, const uint16_t* lr, int r, bool transposed, uint16_t* out,
                         hipStream_t stream) {
  const int xc = lora_extra_cols(r);
  if (!transposed) {
    const int64_t total = w.n * (w.k + xc) / 8;
    int64_t blocks = cdiv(total, (int64_t)256);
    if (blocks > 256 * 64) blocks = 256 * 64;
    expand_rows_kernel<<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<const uint32_t*>(w.codes), w.code8,
                                                             w.s2, w.mean, w.codebook, w.n, w.k, lr, r, xc,
                                                             reinterpret_cast<u32x4*>(out));
  } else {
    const int64_t np = expand_pad_rows(w.n);
    const int64_t ntiles = cdiv(np, (int64_t)kXT);
    const dim3 grid((unsigned)(ntiles + (xc > 0 ? 1 : 0)), (unsigned)(w.k / kBlock));
    expand_cols_kernel<<<grid, 256, 0, stream>>>(w.codes, w.code8, w.s2, w.mean, w.codebook, w.n, w.k, np, lr, r,
                                                 xc, out);
  }
  return hipGetLastError();
}

}  // namespace qlora
