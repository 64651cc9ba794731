// Gated-MLP join between the gate/up and down linears of the MLP workloads:
//   H = silu(G) * Up,  silu(g) = g * sigmoid(g)
// and its backward. Not a QLoRA operation: it lets a whole MLP block
// (gate, up -> join -> down) run on this library. fp32 math on bf16 inputs,
// one bf16 rounding per output. HBM-bound: 8 elements (16 B) per thread.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

__device__ __forceinline__ float sigmoid(float g) { return 1.0f / (1.0f + expf(-g)); }

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

__global__ __launch_bounds__(256) void silu_fwd_kernel(const u32x4* __restrict__ G, const u32x4* __restrict__ U,
                                                       u32x4* __restrict__ H, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  float g[8], u[8], h[8];
  unpack8(G[i], g);
  unpack8(U[i], u);
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = g[e] * sigmoid(g[e]) * u[e];
  H[i] = pack8(h);
}

__global__ __launch_bounds__(256) void silu_bwd_kernel(const u32x4* __restrict__ G, const u32x4* __restrict__ U,
                                                       const u32x4* __restrict__ dH, u32x4* __restrict__ dG,
                                                       u32x4* __restrict__ dU, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  float g[8], u[8], dh[8], dg[8], du[8];
  unpack8(G[i], g);
  unpack8(U[i], u);
  unpack8(dH[i], dh);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float sg = sigmoid(g[e]);
    const float silu = g[e] * sg;
    du[e] = dh[e] * silu;
    dg[e] = dh[e] * u[e] * (sg * (1.0f + g[e] * (1.0f - sg)));
  }
  dG[i] = pack8(dg);
  dU[i] = pack8(du);
}

// Tail (count % 8) elements, one per thread.
__global__ void silu_tail_kernel(const uint16_t* __restrict__ G, const uint16_t* __restrict__ U,
                                 const uint16_t* __restrict__ dH, uint16_t* __restrict__ H, uint16_t* __restrict__ dG,
                                 uint16_t* __restrict__ dU, int64_t begin, int64_t count) {
  const int64_t i = begin + threadIdx.x;
  if (i >= count) return;
  const float g = bf16_bits_to_f32(G[i]), u = bf16_bits_to_f32(U[i]);
  const float sg = sigmoid(g);
  if (dH == nullptr) {
    H[i] = to_bf16_bits(g * sg * u);
  } else {
    const float dh = bf16_bits_to_f32(dH[i]);
    dU[i] = to_bf16_bits(dh * (g * sg));
    dG[i] = to_bf16_bits(dh * u * (sg * (1.0f + g * (1.0f - sg))));
  }
}

}  // namespace

hipError_t launch_silu_fwd(const uint16_t* G, const uint16_t* U, uint16_t* H, int64_t count, hipStream_t stream) {
  const int64_t n8 = count / 8;
  if (n8 > 0)
    silu_fwd_kernel<<<(unsigned)cdiv(n8, 256), 256, 0, stream>>>(reinterpret_cast<const u32x4*>(G),
                                                                 reinterpret_cast<const u32x4*>(U),
                                                                 reinterpret_cast<u32x4*>(H), n8);
  if (count % 8)
    silu_tail_kernel<<<1, 8, 0, stream>>>(G, U, nullptr, H, nullptr, nullptr, n8 * 8, count);
  return hipGetLastError();
}

hipError_t launch_silu_bwd(const uint16_t* G, const uint16_t* U, const uint16_t* dH, uint16_t* dG, uint16_t* dU,
                           int64_t count, hipStream_t stream) {
  const int64_t n8 = count / 8;
  if (n8 > 0)
    silu_bwd_kernel<<<(unsigned)cdiv(n8, 256), 256, 0, stream>>>(
        reinterpret_cast<const u32x4*>(G), reinterpret_cast<const u32x4*>(U), reinterpret_cast<const u32x4*>(dH),
        reinterpret_cast<u32x4*>(dG), reinterpret_cast<u32x4*>(dU), n8);
  if (count % 8)
    silu_tail_kernel<<<1, 8, 0, stream>>>(G, U, dH, nullptr, dG, dU, n8 * 8, count);
  return hipGetLastError();
}

}  // namespace qlora
