// Adapter merge for deployment, and its inverse.
//
// "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev), the two
// prices, price 2: the trained adapter cannot be folded into the 4-bit base
// (no 4-bit level lies between the allowed ones), so it is added onto a
// dequantized copy; "QLoRA vs LoRA ..." (instagit.com), converting back to
// full precision: merge, then dequantize to a higher precision.
//
//   merge:    out[i, c] = round( W'[i, c] + s * sum_j B[i, j] A[j, c] )
//   unmerge:  out[i, c] = round_bf16( Wm[i, c] - s * sum_j B[i, j] A[j, c] )
//
// W' is the bf16 expansion (bit-identical to qlora_dequant), Wm a bf16 merged
// weight. The products of bf16 numbers are exact in fp32; the sum over j runs
// on the matrix cores in fp32, then s * sum and the addition are single fp32
// operations and the result is rounded once (bf16, nearest-even; or kept as
// fp32 for the fp32 copy).
//
// Workgroup: a 64-row x 128-column tile of the weight, 4 waves of 16 rows.
//  1. The tile's W' (from the codes) or Wm is written to an fp32 LDS tile; the
//     A columns of the tile, rows j < rp (rank rounded up to 32, zero rows
//     past r), go to a bf16 LDS tile.
//  2. Each wave forms its 16 x 128 block of B A with v_mfma_f32_16x16x32_bf16:
//     B rows from global memory in operand layout, A read transposed from LDS
//     (ds_read_b64_tr_b16), and adds s * (B A) into the fp32 tile in place.
//  3. The tile is rounded and written with 16-byte row-contiguous stores.
// Bytes per weight: 0.5 code + 2 (bf16) or 4 (fp32) out for merge; 2 + 2 for
// unmerge; A and B are re-read from cache by the tiles that share them.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kGT = 64;          // weight rows per workgroup
constexpr int kGK = 128;         // weight columns per workgroup
constexpr int kWPitch = kGK + 4;  // fp32 words per LDS weight row (4-bank shift per row)
constexpr int kAPitch = kGK * 2 + 32;  // bytes per LDS A row

template <bool kFromNf4, bool kOutF32>
__global__ __launch_bounds__(256) void merge_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ code8,
                                                    const float* __restrict__ s2, const float* __restrict__ mean_p,
                                                    const float* __restrict__ codebook,
                                                    const uint16_t* __restrict__ Wm, int64_t n, int64_t k,
                                                    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    int r, int rp, float scale, void* __restrict__ out) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* wt = reinterpret_cast<float*>(smem);          // [kGT][kWPitch] fp32
  char* at = smem + kGT * kWPitch * 4;                  // [rp][kAPitch bytes] bf16
  __shared__ float lut[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t i0 = (int64_t)blockIdx.y * kGT, c0 = (int64_t)blockIdx.x * kGK;
  const int kcols = (int)(k - c0 < kGK ? k - c0 : kGK);  // 64 or 128 (k % 64 == 0)

  // 1a. A columns c0 .. c0 + kcols - 1 of rows j < rp (zeros past r or past kcols)
  for (int idx = t; idx < rp * (kGK / 8); idx += 256) {
    const int j = idx / (kGK / 8), ch = idx % (kGK / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < r && ch * 8 < kcols) v = *reinterpret_cast<const u32x4*>(A + (int64_t)j * k + c0 + ch * 8);
    *reinterpret_cast<u32x4*>(at + j * kAPitch + ch * 16) = v;
  }
  // 1b. the weight tile as fp32: thread t takes row t / 4, columns 32 (t % 4) .. + 31
  {
    const int row = t >> 2, q = t & 3;
    const int64_t gi = i0 + row;
    float* dst = wt + row * kWPitch + 32 * q;
    const bool ok = gi < n && 32 * q < kcols;
    if constexpr (kFromNf4) {
      if (t < 16) lut[t] = codebook[t];
      __syncthreads();
      u32x4 w = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      float cp = 0.0f;
      if (ok) {
        w = *reinterpret_cast<const u32x4*>(codes + gi * (k / 2) + (c0 + 32 * q) / 2);
        cp = block_scale(code8, s2, mean_p[0], (gi * k + c0 + 32 * q) / kBlock);
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const u32x4 b = dequant8(w[h], lut, cp);  // 8 bf16 = W' values (exact in fp32)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[8 * h + 2 * e] = __uint_as_float(b[e] << 16);
          dst[8 * h + 2 * e + 1] = __uint_as_float(b[e] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        u32x4 b = {0u, 0u, 0u, 0u};
        if (ok) b = *reinterpret_cast<const u32x4*>(Wm + gi * k + c0 + 32 * q + 8 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[8 * h + 2 * e] = __uint_as_float(b[e] << 16);
          dst[8 * h + 2 * e + 1] = __uint_as_float(b[e] & 0xFFFF0000u);
        }
      }
    }
  }
  __syncthreads();

  // 2. s * (B A) for this wave's rows 16 wave .. + 15, added in place
  if (rp > 0) {
    const int64_t bi = i0 + 16 * wave + (lane & 15);  // B row of this lane's operand
    constexpr int kMaxChunks = 4;  // ranks up to 128
    bf16x8 bop[kMaxChunks];
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
      u32x4 v = {0u, 0u, 0u, 0u};
      const int j0 = 32 * ch + 8 * (lane >> 4);
      if (32 * ch < rp && bi < n) {
        if ((r & 7) == 0) {
          if (j0 < r) v = *reinterpret_cast<const u32x4*>(B + bi * r + j0);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) e[x] = j0 + x < r ? (uint32_t)B[bi * r + j0 + x] : 0u;
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = e[2 * x] | (e[2 * x + 1] << 16);
        }
      }
      bop[ch] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int ct = 0; ct < kGK / 16; ++ct) {
      f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ch = 0; ch < kMaxChunks; ++ch)
        if (32 * ch < rp) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop[ch], tr_rows8(at + 32 * ch * kAPitch, kAPitch,
                                                                                         16 * ct, lane), d, 0, 0, 0);
      // D layout: lane -> column 16 ct + lane % 16, rows 4 (lane / 16) + v
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float* p = wt + (16 * wave + 4 * (lane >> 4) + v) * kWPitch + 16 * ct + (lane & 15);
        *p = *p + scale * d[v];
      }
    }
  }
  __syncthreads();

  // 3. round and store: thread t writes row t / 4, columns 32 (t % 4) .. + 31
  {
    const int row = t >> 2, q = t & 3;
    const int64_t gi = i0 + row;
    if (gi >= n || 32 * q >= kcols) return;
    const float* src = wt + row * kWPitch + 32 * q;
    if constexpr (kOutF32) {
      float* o = static_cast<float*>(out) + gi * k + c0 + 32 * q;
#pragma unroll
      for (int h = 0; h < 8; ++h)
        *reinterpret_cast<float4*>(o + 4 * h) = make_float4(src[4 * h], src[4 * h + 1], src[4 * h + 2], src[4 * h + 3]);
    } else {
      uint16_t* o = static_cast<uint16_t*>(out) + gi * k + c0 + 32 * q;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(src[8 * h + 2 * e], src[8 * h + 2 * e + 1]);
        *reinterpret_cast<u32x4*>(o + 8 * h) = v;
      }
    }
  }
}

}  // namespace

size_t merge_smem_bytes(int r) {
  const int rp = r > 0 ? (int)cdiv(r, 32) * 32 : 0;
  return (size_t)kGT * kWPitch * 4 + (size_t)rp * kAPitch;
}

hipError_t launch_merge(const Nf4View* w, const uint16_t* Wm, int64_t n, int64_t k, const uint16_t* A,
                        const uint16_t* B, int r, float scale, bool out_f32, void* out, hipStream_t stream) {
  const int rp = r > 0 ? (int)cdiv(r, 32) * 32 : 0;
  const dim3 grid((unsigned)cdiv(k, (int64_t)kGK), (unsigned)cdiv(n, (int64_t)kGT));
  const size_t smem = merge_smem_bytes(r);
  if (smem > 65536) {
    // more than the default dynamic LDS limit (ranks above 96)
    const void* fns[3] = {reinterpret_cast<const void*>(&merge_kernel<true, true>),
                          reinterpret_cast<const void*>(&merge_kernel<true, false>),
                          reinterpret_cast<const void*>(&merge_kernel<false, false>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
    }
  }
  if (w != nullptr) {
    if (out_f32)
      merge_kernel<true, true><<<grid, 256, smem, stream>>>(w->codes, w->code8, w->s2, w->mean, w->codebook, nullptr,
                                                            n, k, A, B, r, rp, scale, out);
    else
      merge_kernel<true, false><<<grid, 256, smem, stream>>>(w->codes, w->code8, w->s2, w->mean, w->codebook, nullptr,
                                                             n, k, A, B, r, rp, scale, out);
  } else {
    merge_kernel<false, false><<<grid, 256, smem, stream>>>(nullptr, nullptr, nullptr, nullptr, nullptr, Wm, n, k, A,
                                                            B, r, rp, -scale, out);
  }
  return hipGetLastError();
}

}  // namespace qlora
