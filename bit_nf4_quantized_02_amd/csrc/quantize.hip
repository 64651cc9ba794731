// Offline encoder: blockwise NF4 codes + double quantization of the block
// absmax constants.
//
// Sources: "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev):
// the worked 8-weight block (scale = the block's largest magnitude, every
// weight snapped to the nearest of the 16 levels, half a byte each) and
// "NF4: a 4-bit format matched to weight statistics" (64-weight absmax
// blocks). "QLoRA Explained ..." (gamut.so), "Double Quantization": the block
// constants are quantized again to 8 bits.
//
// Every decision is taken by exact comparisons in fp64, so the result does not
// depend on the launch configuration:
//   code  = #{ j : w > mu_j * c_b },   mu_j = (L_j + L_{j+1}) / 2
//   code8 = E4M3 index #{ k : d_b > nu_k * s2 },  nu_k = midpoint of the k-th
//           and (k+1)-th finite E4M3 values in ascending order.
// Both products are exact in fp64 (<= 29 and <= 50 significant bits).
//
// Kernels, in launch order:
//   nf4_codes_kernel   8 lanes per 64-block: absmax, 64 codes, packed bytes
//   dq_runsum_kernel   one thread per run of 256 blocks: fp64 sum in order
//   dq_mean_kernel     one thread: run sums in order -> fp32 mean
//   dq_encode_kernel   one workgroup per run: s2 and the 256 code8 bytes
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

// Eight consecutive weights of the input as fp32 (bf16 widens exactly).
template <bool kBf16>
__device__ __forceinline__ void load8(const void* __restrict__ W, int64_t idx, float (&w)[8]) {
  if constexpr (kBf16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = __uint_as_float(v[i] << 16);
      w[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(W) + idx);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[i] = a[i]; w[4 + i] = b[i]; }
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void nf4_codes_kernel(const void* __restrict__ W, int64_t nb,
                                                        const float* __restrict__ codebook,
                                                        uint32_t* __restrict__ codes,
                                                        float* __restrict__ absmax) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = g >> 3;         // block
  const int part = (int)(g & 7);    // which 8 of its 64 weights
  // midpoints between adjacent levels, exact in fp64
  double mid[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) mid[j] = ((double)codebook[j] + (double)codebook[j + 1]) * 0.5;

  float w[8];
  float m = 0.0f;
  if (b < nb) {
    load8<kBf16>(W, b * kBlock + part * 8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(w[i]));
  }
  // max over the 8 lanes of this block (lanes 8-aligned inside the wavefront)
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 8));
  if (b >= nb) return;

  const double c = (double)m;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t code = 7;
    if (m != 0.0f) {
      const double x = (double)w[i];
      code = 0;
#pragma unroll
      for (int j = 0; j < 15; ++j) code += (x > mid[j] * c) ? 1u : 0u;
    }
    word |= code << (4 * i);
  }
  codes[b * 8 + part] = word;
  if (part == 0) absmax[b] = m;
}

__global__ __launch_bounds__(256) void dq_runsum_kernel(const float* __restrict__ absmax, int64_t nb,
                                                        int64_t nruns, double* __restrict__ runsum) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nruns) return;
  const int64_t b0 = j * kDqBlock;
  const int64_t b1 = (b0 + kDqBlock < nb) ? b0 + kDqBlock : nb;
  double s = 0.0;
  for (int64_t b = b0; b < b1; ++b) s += (double)absmax[b];  // left to right
  runsum[j] = s;
}

__global__ void dq_mean_kernel(const double* __restrict__ runsum, int64_t nruns, int64_t nb,
                               float* __restrict__ mean) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  double s = 0.0;
  for (int64_t j = 0; j < nruns; ++j) s += runsum[j];  // left to right
  mean[0] = (float)(s / (double)nb);
}

// Ascending index (0..252) of the finite E4M3 values -> bit pattern:
// 0..125 are the negatives from -448 up, 126 is +0, 127..252 the positives.
__device__ __forceinline__ uint32_t e4m3_bits_of_index(int idx) {
  return idx < 126 ? (0x80u | (uint32_t)(126 - idx)) : (uint32_t)(idx - 126);
}

__device__ __forceinline__ double e4m3_value_of_index(int idx) {
  return (double)e4m3_to_f32(e4m3_bits_of_index(idx));
}

__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ absmax, int64_t nb,
                                                        const float* __restrict__ mean_p,
                                                        float* __restrict__ s2_out,
                                                        uint8_t* __restrict__ code8) {
  __shared__ float red[256];
  const int64_t run = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t b = run * kDqBlock + t;
  const float mean = mean_p[0];
  float d = 0.0f;
  if (b < nb) d = absmax[b] - mean;  // one fp32 subtraction
  red[t] = fabsf(d);
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  const float a2 = red[0];
  const float s2 = a2 / 448.0f;  // fp32 division, correctly rounded
  if (t == 0) s2_out[run] = s2;
  if (b >= nb) return;
  uint32_t bits = 0;
  if (s2 != 0.0f) {
    const double x = (double)d;
    const double sc = (double)s2;
    // count of midpoints below x: binary search over the 252 midpoints
    int lo = 0;  // answer in [0, 252]
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1) {
      const int k = lo + step - 1;  // midpoint between values k and k+1
      if (k < 252) {
        const double nu = (e4m3_value_of_index(k) + e4m3_value_of_index(k + 1)) * 0.5;
        if (x > nu * sc) lo += step;
      }
    }
    bits = e4m3_bits_of_index(lo);
  }
  code8[b] = (uint8_t)bits;
}

}  // namespace

hipError_t launch_quantize(const void* W, bool w_bf16, int64_t n, int64_t k, const float* codebook,
                           uint8_t* codes, uint8_t* code8, float* s2, float* mean, void* ws,
                           hipStream_t stream) {
  const int64_t nb = n * k / kBlock;
  const int64_t nruns = cdiv(nb, kDqBlock);
  float* absmax = reinterpret_cast<float*>(ws);
  double* runsum = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) + quantize_ws_absmax_bytes(nb));
  const int64_t threads = nb * 8;
  const dim3 grid((unsigned)cdiv(threads, 256));
  if (w_bf16)
    nf4_codes_kernel<true><<<grid, 256, 0, stream>>>(W, nb, codebook, reinterpret_cast<uint32_t*>(codes), absmax);
  else
    nf4_codes_kernel<false><<<grid, 256, 0, stream>>>(W, nb, codebook, reinterpret_cast<uint32_t*>(codes), absmax);
  dq_runsum_kernel<<<(unsigned)cdiv(nruns, 256), 256, 0, stream>>>(absmax, nb, nruns, runsum);
  dq_mean_kernel<<<1, 1, 0, stream>>>(runsum, nruns, nb, mean);
  dq_encode_kernel<<<(unsigned)nruns, 256, 0, stream>>>(absmax, nb, mean, s2, code8);
  return hipGetLastError();
}

}  // namespace qlora
