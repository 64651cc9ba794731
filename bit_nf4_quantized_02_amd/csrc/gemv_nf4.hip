// Dequant-GEMV for small token counts (M <= 16): bandwidth-bound path.
//
// With a handful of tokens every packed weight byte is used for at most 16
// multiply-adds, so the layer costs one pass over the 4-bit codes
// ("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// "Batched 4-bit matmuls"; "QLoRA vs LoRA: ..." (instagit.com), "Training
// Speed and Computational Efficiency": lower memory traffic).
//
//   Y = RN_bf16( X W'^T + s T B^T ),   T = X A^T precomputed (fp32)
//
// Each workgroup owns NT output rows (n) and the whole contraction; its 4
// waves split the contraction into quarters. A wave walks its quarter in
// 128-wide chunks: every lane loads 16 contiguous bytes of codes (32 weights
// of one row, one 64-block, one scale), expands them to bf16 in registers
// through the LDS codebook and feeds them straight to
// v_mfma_f32_16x16x32_bf16 as the B operand; X (padded to 16 rows with zeros)
// is the A operand. The contraction order inside a chunk is permuted the same
// way on both operands (lane group g takes columns 32 g .. 32 g + 31), which
// leaves the sum unchanged and makes each lane's code load contiguous.
// Partial sums of the 4 waves are added in a fixed order through LDS, the
// low-rank term is added in fp32, and Y is rounded to bf16 once.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

template <int NT, bool kLora>
__global__ __launch_bounds__(256) void gemv_nf4_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ code8,
                                                       const float* __restrict__ s2,
                                                       const float* __restrict__ mean_p,
                                                       const float* __restrict__ codebook, int64_t N,
                                                       int64_t K, const uint16_t* __restrict__ X, int64_t M,
                                                       const float* __restrict__ T,
                                                       const uint16_t* __restrict__ B, int r, float scale,
                                                       uint16_t* __restrict__ Y) {
  constexpr int kTiles = NT / 16;
  __shared__ float lut[16];
  __shared__ float red[4][kTiles][16][16];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  if (t < 16) lut[t] = codebook[t];
  __syncthreads();
  const float mean = mean_p[0];
  const int64_t n0 = (int64_t)blockIdx.x * NT;
  const int64_t kq = cdiv(cdiv(K, 4), 128) * 128;  // per-wave share, multiple of 128
  const int64_t kb = wave * kq;
  const int64_t ke = (kb + kq < K) ? kb + kq : K;
  const int grp = lane >> 4;   // 0..3: which 32 columns of a 128-chunk
  const int col = lane & 15;   // A: token row m; B: weight row within a tile
  const int64_t kblocks = K / kBlock;

  f32x4 acc[kTiles];
#pragma unroll
  for (int i = 0; i < kTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kb; k0 < ke; k0 += 128) {
    const int64_t k = k0 + 32 * grp;
    const bool kin = k < ke;  // ke is a multiple of 32 (K % 64 == 0)
    bf16x8 af[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kin && col < M) v = *reinterpret_cast<const u32x4*>(X + col * K + k + 8 * s);
      af[s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
      const int64_t n = n0 + i * 16 + col;
      u32x4 cw = {0u, 0u, 0u, 0u};
      float cp = 0.0f;
      if (kin && n < N) {
        cw = *reinterpret_cast<const u32x4*>(codes + n * (K / 2) + k / 2);
        cp = block_scale(code8, s2, mean, n * kblocks + k / kBlock);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 bw = dequant8(cw[s], lut, cp);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], __builtin_bit_cast(bf16x8, bw), acc[i], 0, 0, 0);
      }
    }
  }
  // D[m][n]: lane -> n = lane & 15, m = 4 (lane >> 4) + v
#pragma unroll
  for (int i = 0; i < kTiles; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][i][4 * (lane >> 4) + v][lane & 15] = acc[i][v];
  __syncthreads();
  for (int o = t; o < 16 * NT; o += 256) {
    const int m = o / NT, nl = o % NT;
    const int64_t n = n0 + nl;
    if (m >= M || n >= N) continue;
    const int i = nl >> 4, nc = nl & 15;
    float y = ((red[0][i][m][nc] + red[1][i][m][nc]) + red[2][i][m][nc]) + red[3][i][m][nc];
    if constexpr (kLora) {
      float l = 0.0f;
      for (int j = 0; j < r; ++j) l = fmaf(T[m * r + j], bf16_bits_to_f32(B[n * r + j]), l);
      y = fmaf(scale, l, y);
    }
    Y[m * N + n] = to_bf16_bits(y);
  }
}

}  // namespace

hipError_t launch_gemv(const Nf4View& w, const uint16_t* X, int64_t M, const float* T, const uint16_t* B, int r,
                       float scale, uint16_t* Y, hipStream_t stream) {
  const bool lora = r > 0;
#define QLORA_GEMV(NT)                                                                                        \
  {                                                                                                           \
    const dim3 grid((unsigned)cdiv(w.n, NT));                                                                 \
    if (lora)                                                                                                 \
      gemv_nf4_kernel<NT, true><<<grid, 256, 0, stream>>>(w.codes, w.code8, w.s2, w.mean, w.codebook, w.n,   \
                                                           w.k, X, M, T, B, r, scale, Y);                     \
    else                                                                                                      \
      gemv_nf4_kernel<NT, false><<<grid, 256, 0, stream>>>(w.codes, w.code8, w.s2, w.mean, w.codebook, w.n,  \
                                                            w.k, X, M, T, B, r, scale, Y);                    \
  }
  if (w.n / 64 >= 512) QLORA_GEMV(64)
  else if (w.n / 32 >= 512) QLORA_GEMV(32)
  else QLORA_GEMV(16)
#undef QLORA_GEMV
  return hipGetLastError();
}

}  // namespace qlora
