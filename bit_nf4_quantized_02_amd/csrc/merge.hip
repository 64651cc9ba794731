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
// Workgroup: a 128-column strip of the weight, walked in 4 tiles of 64 rows,
// 4 waves. The strip's A columns, rows j < rp (rank rounded up to 32, zero
// rows past r), are staged in LDS once as bf16. Per tile:
//  1. each wave forms its 16 x 128 block of B A with v_mfma_f32_16x16x32_bf16
//     (B rows from global memory in operand layout, A read transposed from
//     LDS with ds_read_b64_tr_b16) and writes s * (B A) to an fp32 LDS tile;
//  2. each thread expands (or holds) the 4 x 8 base weights it will store and
//     issues the next tile's loads;
//  3. it adds the delta from LDS, rounds once and stores; a store
//     instruction covers whole 256-byte row segments.
// A wave only ever reads the delta rows it wrote itself, so the tile loop has
// no workgroup barrier and the four waves proceed independently.
// Bytes per weight: 0.5 code + 2 (bf16) or 4 (fp32) out for merge; 2 + 2 for
// unmerge; A and B are re-read from cache by the tiles that share them.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kGT = 64;                // weight rows per tile
constexpr int kGK = 128;               // weight columns per tile (the workgroup's column strip)
constexpr int kTiles = 4;              // row tiles per workgroup (the A strip is staged once)
constexpr int kDPitch = kGK + 4;       // fp32 words per LDS delta row (4-bank shift per row)
constexpr int kAPitch = kGK * 2 + 32;  // bytes per LDS A row
constexpr int kMaxChunks = 4;          // 32-deep rank chunks, ranks up to 128

// What one thread loads for a tile: its B row in MFMA operand layout, and the
// source of the 4 x 8 weights it stores (rows 16 wave + lane / 16 + 4 i,
// columns 8 (lane % 16) .. + 7): four code words and their block scales, or
// four 16-byte bf16 chunks of the merged weight.
template <bool kFromNf4>
struct TileSrc {
  bf16x8 bop[kMaxChunks];
  u32x4 v[kFromNf4 ? 1 : 4];
  float cp[kFromNf4 ? 4 : 1];
};

template <bool kFromNf4>
__device__ __forceinline__ void load_src(TileSrc<kFromNf4>& x, const uint8_t* __restrict__ codes,
                                         const uint8_t* __restrict__ code8, const float* __restrict__ s2, bool s2_bf16,
                                         float mean, const uint16_t* __restrict__ Wm, int64_t n, int64_t k, int64_t i0, int64_t c0,
                                         int kcols, int t, const uint16_t* __restrict__ B, int r, int rp) {
  {
    // B rows i0 + 16 wave + lane % 16, ranks 32 ch + 8 (lane / 16) .. + 7
    const int lane = t & 63, wave = t >> 6;
    const int64_t bi = i0 + 16 * wave + (lane & 15);
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
          for (int q = 0; q < 8; ++q) e[q] = j0 + q < r ? (uint32_t)B[bi * r + j0 + q] : 0u;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = e[2 * q] | (e[2 * q + 1] << 16);
        }
      }
      x.bop[ch] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const int cc = t & 15;
  const int64_t c = c0 + 8 * cc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gi = i0 + 16 * (t >> 6) + ((t & 63) >> 4) + 4 * i;
    const bool ok = gi < n && 8 * cc < kcols;
    if constexpr (kFromNf4) {
      x.v[0][i] = 0x77777777u;  // level 0 (not stored)
      x.cp[i] = 0.0f;
      if (ok) {
        x.v[0][i] = *reinterpret_cast<const uint32_t*>(codes + gi * (k / 2) + c / 2);
        x.cp[i] = block_scale(code8, s2, s2_bf16, mean, (gi * k + c) / kBlock);
      }
    } else {
      x.v[i] = u32x4{0u, 0u, 0u, 0u};
      if (ok) x.v[i] = *reinterpret_cast<const u32x4*>(Wm + gi * k + c);
    }
  }
}

template <bool kFromNf4, bool kOutF32, int kHold>
__global__ __launch_bounds__(256) void merge_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ code8,
                                                    const float* __restrict__ s2, const float* __restrict__ mean_p,
                                                    const float* __restrict__ codebook, bool s2_bf16,
                                                    const uint16_t* __restrict__ Wm, int64_t n, int64_t k,
                                                    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    int r, int rp, float scale, void* __restrict__ out) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* dl = reinterpret_cast<float*>(smem);          // [kGT][kDPitch] fp32: scale * (B A)
  char* at = smem + kGT * kDPitch * 4;                  // [rp][kAPitch bytes] bf16
  __shared__ float lut[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kGK;
  const int64_t ibase = (int64_t)blockIdx.y * kGT * kTiles;
  const int kcols = (int)(k - c0 < kGK ? k - c0 : kGK);  // 64 or 128 (k % 64 == 0)
  const float mean = kFromNf4 ? weight_mean(code8, mean_p) : 0.0f;
  const int cc = t & 15;

  if (kFromNf4 && t < 16) lut[t] = codebook[t];
  // A columns c0 .. c0 + kcols - 1 of rows j < rp (zeros past r or past kcols), once
  for (int idx = t; idx < rp * (kGK / 8); idx += 256) {
    const int j = idx / (kGK / 8), ch = idx % (kGK / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < r && ch * 8 < kcols) v = *reinterpret_cast<const u32x4*>(A + (int64_t)j * k + c0 + ch * 8);
    *reinterpret_cast<u32x4*>(at + j * kAPitch + ch * 16) = v;
  }
  TileSrc<kFromNf4> cur;
  load_src<kFromNf4>(cur, codes, code8, s2, s2_bf16, mean, Wm, n, k, ibase, c0, kcols, t, B, r, rp);

  __syncthreads();  // lut and the A strip are written
  // Each wave works on its own 16 rows of every tile and its own region of
  // dl, so the tile loop needs no barrier: a wave's LDS operations complete in
  // order.
  float* const dw = dl + 16 * wave * kDPitch;
  // For ranks up to 32 kHold the strip's MFMA operands (the same for every
  // tile) are read from LDS once into registers.
  bf16x8 aop[kHold > 0 ? kHold * (kGK / 16) : 1];
#pragma unroll
  for (int ch = 0; ch < kHold; ++ch)
#pragma unroll
    for (int ct = 0; ct < kGK / 16; ++ct) aop[ch * (kGK / 16) + ct] = tr_rows8(at + 32 * ch * kAPitch, kAPitch, 16 * ct, lane);
  for (int tile = 0; tile < kTiles; ++tile) {
    const int64_t i0 = ibase + (int64_t)tile * kGT;
    if (i0 >= n) break;  // uniform
    // 1. scale * (B A) for this wave's rows 16 wave .. + 15 into its dl rows
    //    (the empty asm statements keep the compiler from moving this wave's
    //    LDS writes and reads across each other: other lanes read what a lane
    //    writes, which the compiler cannot see)
    asm volatile("" ::: "memory");
    if (rp > 0) {
#pragma unroll
      for (int ct = 0; ct < kGK / 16; ++ct) {
        f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ch = 0; ch < kMaxChunks; ++ch) {
          if (32 * ch >= rp) continue;
          const bf16x8 ao = ch < kHold ? aop[ch * (kGK / 16) + ct]
                                       : tr_rows8(at + 32 * ch * kAPitch, kAPitch, 16 * ct, lane);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.bop[ch], ao, d, 0, 0, 0);
        }
        // D layout: lane -> column 16 ct + lane % 16, rows 4 (lane / 16) + v
#pragma unroll
        for (int v = 0; v < 4; ++v) dw[(4 * (lane >> 4) + v) * kDPitch + 16 * ct + (lane & 15)] = scale * d[v];
      }
    }
    // 2. this thread's 32 base weights (fp32 values of bf16 numbers)
    u32x4 wb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wb[i] = kFromNf4 ? dequant8(cur.v[0][i], lut, cur.cp[i]) : cur.v[i];
    // the next tile's loads are in flight while this one is finished
    if (tile + 1 < kTiles && i0 + kGT < n)
      load_src<kFromNf4>(cur, codes, code8, s2, s2_bf16, mean, Wm, n, k, i0 + kGT, c0, kcols, t, B, r, rp);
    asm volatile("" ::: "memory");
    // 3. add, round once, store: rows 16 wave + lane / 16 + 4 i, columns
    //    8 cc .. + 7; a store instruction covers whole 256-byte row segments
    if (8 * cc < kcols) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (lane >> 4) + 4 * i;  // within the wave's 16 rows
        const int64_t gi = i0 + 16 * wave + row;
        if (gi >= n) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(wb[i][e] << 16);
          v[2 * e + 1] = __uint_as_float(wb[i][e] & 0xFFFF0000u);
        }
        if (rp > 0) {
          const float4* src = reinterpret_cast<const float4*>(dw + row * kDPitch + 8 * cc);
          const float4 a0 = src[0], a1 = src[1];
          v[0] = v[0] + a0.x; v[1] = v[1] + a0.y; v[2] = v[2] + a0.z; v[3] = v[3] + a0.w;
          v[4] = v[4] + a1.x; v[5] = v[5] + a1.y; v[6] = v[6] + a1.z; v[7] = v[7] + a1.w;
        }
        if constexpr (kOutF32) {
          float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + gi * k + c0 + 8 * cc);
          o[0] = make_float4(v[0], v[1], v[2], v[3]);
          o[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + gi * k + c0 + 8 * cc) = pk;
        }
      }
    }
  }
}

}  // namespace

size_t merge_smem_bytes(int r) {
  const int rp = r > 0 ? (int)cdiv(r, 32) * 32 : 0;
  return (size_t)kGT * kDPitch * 4 + (size_t)rp * kAPitch;
}

hipError_t launch_merge(const Nf4View* w, const uint16_t* Wm, int64_t n, int64_t k, const uint16_t* A,
                        const uint16_t* B, int r, float scale, bool out_f32, void* out, hipStream_t stream) {
  const int rp = r > 0 ? (int)cdiv(r, 32) * 32 : 0;
  const dim3 grid((unsigned)cdiv(k, (int64_t)kGK), (unsigned)cdiv(n, (int64_t)kGT * kTiles));
  const size_t smem = merge_smem_bytes(r);
  if (smem > 65536) {
    // more than the default dynamic LDS limit (ranks above 96)
    const void* fns[3] = {reinterpret_cast<const void*>(&merge_kernel<true, true, 0>),
                          reinterpret_cast<const void*>(&merge_kernel<true, false, 0>),
                          reinterpret_cast<const void*>(&merge_kernel<false, false, 0>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
    }
  }
#define QLORA_MERGE(NF4, F32, H)                                                                               \
  merge_kernel<NF4, F32, H><<<grid, 256, smem, stream>>>(                                                      \
      NF4 ? w->codes : nullptr, NF4 ? w->code8 : nullptr, NF4 ? w->s2 : nullptr, NF4 ? w->mean : nullptr,      \
      NF4 ? w->codebook : nullptr, NF4 && w->s2_bf16, Wm, n, k, A, B, r, rp, NF4 ? scale : -scale, out)
#define QLORA_MERGE_H(NF4, F32)          \
  if (rp == 32) QLORA_MERGE(NF4, F32, 1); \
  else if (rp == 64) QLORA_MERGE(NF4, F32, 2); \
  else QLORA_MERGE(NF4, F32, 0);
  if (w != nullptr) {
    if (out_f32) { QLORA_MERGE_H(true, true) }
    else { QLORA_MERGE_H(true, false) }
  } else {
    QLORA_MERGE_H(false, false)
  }
#undef QLORA_MERGE_H
#undef QLORA_MERGE
  return hipGetLastError();
}

}  // namespace qlora
