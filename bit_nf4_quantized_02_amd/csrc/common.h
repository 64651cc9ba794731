// Shared device helpers for the gfx950 kernels of libqlora.
//
// Storage format (per 64-weight block b of the row-major weight, see
// include/qlora.h): packed nibble codes, an 8-bit E4M3 code for the block's
// centred absmax, one fp32 second-level scale per 256 blocks, one fp32 mean.
// Sources: "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// three-piece summary and "NF4: a 4-bit format matched to weight
// statistics"; "QLoRA Explained ..." (gamut.so), "Double Quantization".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;     // weights per first-level block
constexpr int kDqBlock = 256;  // blocks per second-level scale

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values -> packed bf16 pair (lo in bits 0..15), round to nearest
// even. gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// The 16-bit compute type as a template flag: bf16 (kF16 = false, the
// default everywhere) or fp16 (the compute-type ablation). Operands travel
// as 16-byte bit patterns (bf16x8) either way; only the roundings and the
// MFMA instruction differ. Both roundings are to nearest, ties to even.
template <bool kF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (kF16) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <bool kF16>
__device__ __forceinline__ uint16_t to16(float x) {
  if constexpr (kF16) return __builtin_bit_cast(uint16_t, (_Float16)x);
  else return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <bool kF16>
__device__ __forceinline__ float from16(uint32_t b16) {
  if constexpr (kF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
  else return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// OCP FP8 E4M3 bit pattern -> fp32, from the format's definition: sign bit,
// 4-bit exponent with bias 7, 3-bit mantissa, subnormals at exponent 0.
// Exact for every finite pattern (the encoder never writes the NaN pattern).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 0xFu;
  const uint32_t m = b & 0x7u;
  // both cases computed, one selected: no divergent branch
  const float sub = (float)m * 0.001953125f;  // m/8 * 2^-6 = m * 2^-9, exact
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float mag = e == 0 ? sub : nrm;
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// c'_b = RN32(RN32(fp8 * s2) + mean): two separately rounded fp32 operations.
// The pragma keeps the compiler from fusing them into one FMA.
__device__ __forceinline__ float decode_block_scale(uint32_t code8, float s2, float mean) {
#pragma clang fp contract(off)
  const float v = e4m3_to_f32(code8);
  const float p = v * s2;
  return p + mean;
}

// An encoded weight keeps its block scales double-quantized (code8 set) or
// as one value per block in s2 (code8 NULL: no double quantization), fp32
// or, with s2_bf16 set, a bf16 bit pattern per block ("QLoRA: Quantized
// Low-Rank Adaptation" (completesystemdesign.dev): one BF16 scalar per
// 64-weight block). In the per-block forms the loads below return the E4M3
// code of 1.0 and a zero mean, for which decode_block_scale returns the
// stored scale exactly (1.0 * s and s + 0 are exact for s >= 0; a bf16 value
// widens to fp32 exactly), so every kernel decodes all three forms with the
// same arithmetic.
constexpr uint32_t kE4m3One = 0x38;

__device__ __forceinline__ float weight_mean(const uint8_t* code8, const float* __restrict__ mean_p) {
  return code8 ? mean_p[0] : 0.0f;
}

__device__ __forceinline__ void scale_fields(const uint8_t* __restrict__ code8, const float* __restrict__ s2,
                                             bool s2_bf16, int64_t blk, uint32_t& c8, float& s2v) {
  if (code8) {
    c8 = code8[blk];
    s2v = s2[blk / kDqBlock];
  } else if (s2_bf16) {
    c8 = kE4m3One;
    s2v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s2)[blk]);
  } else {
    c8 = kE4m3One;
    s2v = s2[blk];
  }
}

// Scale of block `blk` (global block index) read from the encoded weight.
__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ code8,
                                             const float* __restrict__ s2, bool s2_bf16, float mean,
                                             int64_t blk) {
  uint32_t c8;
  float s2v;
  scale_fields(code8, s2, s2_bf16, blk, c8, s2v);
  return decode_block_scale(c8, s2v, mean);
}

// One weight: w' = RN_bf16(RN32(L[code] * c')); the product is a single
// fp32 multiply (nothing to fuse it with), the bf16 rounding is RNE.
__device__ __forceinline__ float nf4_scaled(float level, float cprime) {
#pragma clang fp contract(off)
  return level * cprime;
}

// Eight codes of one 32-bit word (code 2t in the low nibble of byte t) ->
// eight bf16 values as four packed pairs, levels looked up in `lut`
// (16 fp32 entries, normally in LDS).
template <bool kF16 = false>
__device__ __forceinline__ u32x4 dequant8(uint32_t word, const float* lut, float cprime) {
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = nf4_scaled(lut[(word >> (8 * p)) & 0xF], cprime);
    const float b = nf4_scaled(lut[(word >> (8 * p + 4)) & 0xF], cprime);
    out[p] = pack2<kF16>(a, b);
  }
  return out;
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <bool kF16>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool kF16>
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight bf16 values with the ones whose mask byte is 0 cleared (mask bytes in
// element order, little-endian in mk): dropout on the adapter's input.
__device__ __forceinline__ u32x4 apply_mask8(u32x4 v, uint2 mk) {
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t mb = (w < 2 ? mk.x : mk.y) >> (16 * (w & 1));  // bytes of elements 2w, 2w + 1
    const uint32_t lo = (mb & 0xFFu) ? 0x0000FFFFu : 0u;
    const uint32_t hi = (mb & 0xFF00u) ? 0xFFFF0000u : 0u;
    o[w] = v[w] & (lo | hi);
  }
  return o;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Operand of v_mfma_f32_16x16x32_bf16 from a [row][col] bf16 tile in LDS:
// lane gets column c0 + lane % 16, rows 8 (lane / 16) .. +7 (the contraction
// index runs over rows). Inside each 16-lane group lane i addresses row
// base + i / 4, columns 4 (i % 4) .. +3, and ds_read_b64_tr_b16 hands each
// lane its own column of the 4 rows.
__device__ __forceinline__ bf16x8 tr_rows8(const char* tile, int pitch, int c0, int lane) {
  const int i = lane & 15;
  const char* p = tile + (8 * (lane >> 4) + (i >> 2)) * pitch + (c0 + 4 * (i & 3)) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 4 * pitch));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Direct buffer load into LDS (16 bytes per lane, LDS address from the wave-
// uniform destination), declared through its LLVM intrinsic so the compiler
// keeps track of the LDS region written and does not wait for these copies
// before reading the other buffer.
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) uint32_t* lds, int size, int voffset,
                                    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer descriptor for a whole operand: base address, size in bytes (the
// offsets of every copy stay below it), raw 32-bit dword format.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = (int)(uint32_t)(bytes < (int64_t)0xFFFFFFFF ? bytes : (int64_t)0xFFFFFFFF);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from a buffer straight into LDS at dst (wave-uniform;
// lane i lands at dst + 16 i). Offsets at or past the descriptor's size
// read as zero.
__device__ __forceinline__ void copy16(const i32x4& r, uint32_t voff, int soff, char* dst) {
  raw_buffer_load_lds(r, (__attribute__((address_space(3))) uint32_t*)dst, 16, (int)voff, soff, 0, 0);
}

// 16 bytes per lane from a buffer into registers; offsets at or past the
// descriptor's size read as zero.
__device__ u32x4 raw_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");

// Buffer loads of one byte / half-word / word (zero past the descriptor's
// size). Unlike plain loads the compiler keeps them where they are issued:
// a plain load whose value is used only after the loop's exit test gets
// sunk past it, right before its use, which drains the prefetch.
__device__ uint8_t raw_buffer_load_u8(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i8");
__device__ uint16_t raw_buffer_load_u16(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i16");
__device__ uint32_t raw_buffer_load_u32(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i32");

}  // namespace qlora
