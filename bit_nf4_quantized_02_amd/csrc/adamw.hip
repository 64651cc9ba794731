// AdamW step on the adapter with fp32 ("32-bit") states that may live in
// host-pinned memory ("paged" optimizer states).
//
// "QLoRA Explained ..." (gamut.so), "Paged Optimizers": the optimizer states
// (momentum, variance) move between GPU and CPU memory to absorb memory
// spikes; "Step 4" / quick reference: the 32-bit paged AdamW at lr 2e-4.
// "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev), paged
// optimizers (states in pinned CPU RAM) and piece 3 (only the adapter learns).
//
// Per element, in fp32 with every operation rounded separately:
//   m <- b1 m + (1 - b1) g
//   v <- b2 v + (1 - b2) (g g)
//   theta <- theta - lr ( (m / bc1) / (sqrt(v / bc2) + eps) + wd theta )
// with bc1 = 1 - b1^t, bc2 = 1 - b2^t and 1 - b1, 1 - b2 formed on the host in
// fp64 and rounded once; optionally also theta16 = RN_bf16(theta), the copy
// the layer kernels read. States in host-pinned memory are read and written
// in place over the host link, which then bounds the step.
#include <cmath>

#include "common.h"
#include "qlora.h"

namespace qlora {
namespace {

struct AdamwC {
  float b1, b2, omb1, omb2, lr, eps, wd, bc1, bc2;
};

__device__ __forceinline__ void adamw_one(float& th, float g, float& m, float& v, const AdamwC& c) {
#pragma clang fp contract(off)
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * (g * g);
  const float mhat = m / c.bc1;
  const float vhat = v / c.bc2;
  const float u = mhat / (sqrtf(vhat) + c.eps) + c.wd * th;
  th = th - c.lr * u;
}

// Four elements per thread (16-byte accesses when every array is 16-byte
// aligned), grid-stride; the last count % 4 elements one per thread.
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ theta, uint16_t* __restrict__ theta16,
                                                    const float* __restrict__ grad, float* __restrict__ m,
                                                    float* __restrict__ v, int64_t n, AdamwC c) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 th = reinterpret_cast<float4*>(theta)[i];
    const float4 g = reinterpret_cast<const float4*>(grad)[i];
    float4 mm = reinterpret_cast<float4*>(m)[i];
    float4 vv = reinterpret_cast<float4*>(v)[i];
    adamw_one(th.x, g.x, mm.x, vv.x, c);
    adamw_one(th.y, g.y, mm.y, vv.y, c);
    adamw_one(th.z, g.z, mm.z, vv.z, c);
    adamw_one(th.w, g.w, mm.w, vv.w, c);
    reinterpret_cast<float4*>(theta)[i] = th;
    reinterpret_cast<float4*>(m)[i] = mm;
    reinterpret_cast<float4*>(v)[i] = vv;
    if (theta16 != nullptr) {
      uint2 o;
      o.x = pack_bf16x2(th.x, th.y);
      o.y = pack_bf16x2(th.z, th.w);
      reinterpret_cast<uint2*>(theta16)[i] = o;
    }
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float th = theta[i], mm = m[i], vv = v[i];
    adamw_one(th, grad[i], mm, vv, c);
    theta[i] = th;
    m[i] = mm;
    v[i] = vv;
    if (theta16 != nullptr) theta16[i] = to_bf16_bits(th);
  }
}

// Device address of an optimizer-state buffer: device memory as is, pinned
// host memory through its device mapping; anything else (pageable host
// memory, unknown pointers) is rejected.
bool state_ptr(float* p, float** dev) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error the failed query leaves behind
    return false;
  }
  if (a.type == hipMemoryTypeDevice) {
    *dev = p;
    return true;
  }
  if (a.type == hipMemoryTypeHost) {
    // only memory from hipHostMalloc: its flags are known and it has a device mapping
    unsigned int flags = 0;
    void* d = nullptr;
    if (hipHostGetFlags(&flags, p) != hipSuccess || hipHostGetDevicePointer(&d, p, 0) != hipSuccess ||
        d == nullptr) {
      (void)hipGetLastError();
      return false;
    }
    *dev = static_cast<float*>(d);
    return true;
  }
  return false;
}

}  // namespace
}  // namespace qlora

extern "C" qlora_status qlora_adamw_step(float* theta, uint16_t* theta16, const float* grad, float* m, float* v,
                                         int64_t count, int64_t step, float lr, float beta1, float beta2, float eps,
                                         float weight_decay, void* stream) {
  using namespace qlora;
  if (count < 0 || step < 1) return QLORA_ERR_SHAPE;
  if (count == 0) return QLORA_OK;
  if (!theta || !grad || !m || !v) return QLORA_ERR_INVALID_ARG;
  if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f && eps >= 0.0f && lr >= 0.0f &&
        weight_decay >= 0.0f))
    return QLORA_ERR_INVALID_ARG;
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (!al16(theta) || !al16(grad) || !al16(m) || !al16(v) || (theta16 && !al16(theta16))) return QLORA_ERR_INVALID_ARG;
  float *md = nullptr, *vd = nullptr;
  if (!state_ptr(m, &md) || !state_ptr(v, &vd)) return QLORA_ERR_INVALID_ARG;
  AdamwC c;
  c.b1 = beta1;
  c.b2 = beta2;
  c.omb1 = (float)(1.0 - (double)beta1);
  c.omb2 = (float)(1.0 - (double)beta2);
  c.lr = lr;
  c.eps = eps;
  c.wd = weight_decay;
  c.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  c.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  if (!(c.bc1 > 0.0f) || !(c.bc2 > 0.0f)) return QLORA_ERR_INVALID_ARG;
  int64_t blocks = (count / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  adamw_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(theta, theta16, grad, md, vd, count, c);
  return hipGetLastError() == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}
