// Dropout on the adapter's input ("QLoRA Explained ..." (gamut.so), "Step 3:
// Configure and Apply LoRA Adapters": LoRA dropout 0.05): the low-rank branch
// sees X . D with D = mask * keep_scale, mask drawn by the caller. The keep
// scale factors out of every product the branch forms, so the kernels here
// only zero the dropped entries (exact in bf16) and the scale is applied to
// the products' fp32 results: T = keep_scale (X . mask) A^T, and so on.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

// Xd = X where mask != 0, else +0; 8 elements per thread (16-byte X, 8-byte
// mask loads), grid-stride.
__global__ __launch_bounds__(256) void dropout_apply_kernel(const u32x4* __restrict__ X,
                                                            const uint2* __restrict__ mask, u32x4* __restrict__ Xd,
                                                            int64_t count8) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count8; i += stride) {
    const u32x4 x = X[i];
    const uint2 m = mask[i];
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t mb = (w < 2 ? m.x : m.y) >> (16 * (w & 1));  // mask bytes of elements 2w, 2w+1
      const uint32_t lo = (mb & 0xFFu) ? 0x0000FFFFu : 0u;
      const uint32_t hi = (mb & 0xFF00u) ? 0xFFFF0000u : 0u;
      o[w] = x[w] & (lo | hi);
    }
    Xd[i] = o;
  }
}

}  // namespace

hipError_t launch_dropout_apply(const uint16_t* X, const uint8_t* mask, uint16_t* Xd, int64_t count,
                                hipStream_t stream) {
  const int64_t count8 = count / 8;
  int64_t blocks = cdiv(count8, (int64_t)256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  dropout_apply_kernel<<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<const u32x4*>(X),
                                                             reinterpret_cast<const uint2*>(mask),
                                                             reinterpret_cast<u32x4*>(Xd), count8);
  return hipGetLastError();
}

}  // namespace qlora
