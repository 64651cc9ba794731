// Whole-tensor expansion of an encoded NF4 weight to bf16.
//
// "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// three-piece summary, piece 2: a 64-weight block is expanded back to bf16
// right before it is multiplied. This kernel writes exactly the values the
// GEMM kernels build in LDS, so the expansion can be checked bit for bit.
//
// One thread expands 8 weights (one 32-bit code word, 16 output bytes);
// consecutive threads take consecutive words, so both the code reads and the
// bf16 writes are contiguous across the wavefront. HBM-bound: 0.5 B read and
// 2 B written per weight, plus 1/64 B of code8.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

// kF16: each w' rounded to fp16 instead of bf16 (the compute-type ablation).
template <bool kF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ code8,
                                                      const float* __restrict__ s2,
                                                      const float* __restrict__ mean_p,
                                                      const float* __restrict__ codebook, bool s2_bf16,
                                                      int64_t nwords, u32x4* __restrict__ out) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const float mean = weight_mean(code8, mean_p);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) {
    const int64_t blk = i >> 3;  // 8 words per 64-weight block
    const float cp = block_scale(code8, s2, s2_bf16, mean, blk);
    out[i] = dequant8<kF16>(codes[i], lut, cp);
  }
}

}  // namespace

hipError_t launch_dequant(const Nf4View& w, uint16_t* out, hipStream_t stream, bool f16) {
  const int64_t nwords = w.n * w.k / 8;
  int64_t blocks = cdiv(nwords, 256);
  if (blocks > 256 * 64) blocks = 256 * 64;
  auto* cw = reinterpret_cast<const uint32_t*>(w.codes);
  auto* o4 = reinterpret_cast<u32x4*>(out);
  if (f16)
    dequant_kernel<true><<<(unsigned)blocks, 256, 0, stream>>>(cw, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16,
                                                               nwords, o4);
  else
    dequant_kernel<false><<<(unsigned)blocks, 256, 0, stream>>>(cw, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16,
                                                                nwords, o4);
  return hipGetLastError();
}

}  // namespace qlora
