// Attainable-peak probes for the roofline report: a matrix-core loop with no
// memory traffic and a streaming read of a device buffer. They measure what
// the chip sustains on the box at hand (clocks under load, achievable HBM
// read rate), printed beside the published peaks; they are not part of the
// layer and compute nothing the layer uses.
#include "common.h"
#include "qlora.h"

namespace qlora {
namespace {

constexpr int kCalibThreads = 512;  // 8 waves, two per SIMD
constexpr int kCalibChains = 8;     // independent accumulators per wave

// Each wave runs `iters` rounds of kCalibChains independent
// v_mfma_f32_32x32x16_bf16 (32768 flops each). The result is stored only if
// it equals a value it never takes, so the work cannot be dropped.
__global__ __launch_bounds__(kCalibThreads) void calib_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(e + 1));
  }
  f32x16 acc[kCalibChains];
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (s == -1.2345e-30f) sink[0] = s;
}

// Grid-stride read of n16 16-byte chunks, four loads in flight per thread.
__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                         float* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < n16 ? p[j] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (x == 0x9E3779B9u) sink[0] = (float)x;
}

}  // namespace
}  // namespace qlora

extern "C" qlora_status qlora_calib_mfma(int blocks, int iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr) return QLORA_ERR_INVALID_ARG;
  qlora::calib_mfma_kernel<<<blocks, qlora::kCalibThreads, 0, (hipStream_t)stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

extern "C" qlora_status qlora_calib_stream_read(const void* buf, int64_t bytes, float* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes < 16) return QLORA_ERR_INVALID_ARG;
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return QLORA_ERR_SHAPE;
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  qlora::calib_read_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(
      reinterpret_cast<const qlora::u32x4*>(buf), n16, sink);
  return hipGetLastError() == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}
