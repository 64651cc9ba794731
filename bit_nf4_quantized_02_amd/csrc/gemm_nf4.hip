// Fused NF4-dequant + bf16 MFMA GEMMs for large token counts (gfx950).
//
// "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev): storage
// stays 4-bit while the math is 16-bit -- a 64-weight block is expanded to
// bf16 right before the multiply (three-piece summary, piece 2; "Batched
// 4-bit matmuls"); the same expansion serves the backward pass through the
// frozen base ("What is QLoRA?" (qubittool.com), "Key Characteristics").
//
//   forward   Y  = RN_bf16( X W'^T  + [sT_hi | sT_lo] [B | B]^T )
//   backward  dX = RN_bf16( dY W'   + [sU_hi | sU_lo] [A ; A]   )
//
// The low-rank term is folded into the same fp32 accumulator as 2r extra
// contraction columns (hi/lo bf16 halves of the scaled fp32 T or U), so the
// output is rounded to bf16 exactly once.
//
// Workgroup tile 256 x 256 outputs, 64-deep contraction steps (one NF4 block
// per weight row per step), 512 threads = 8 waves (two per SIMD) in a 2 x 4
// grid, each wave a 128 x 64 sub-tile of v_mfma_f32_32x32x16_bf16 (8 tiles,
// 128 accumulator registers). Two waves per SIMD let one wave's MFMAs run
// while the other waits on LDS or does its share of the dequantization. LDS holds two buffers of each operand tile (4 x 32 KB), so one
// barrier per step suffices and the next step's tiles are built while the
// current step's MFMAs run:
//   * activation tile [256 x 64] bf16: copied one step ahead straight from
//     global memory into LDS (global_load_lds_dwordx4; the swizzle is applied
//     by permuting each lane's source address), no registers involved;
//   * weight tile: packed nibbles, code8 byte and s2 loaded two steps ahead
//     (0.5 B/weight); for the step after the current one each block's scale c'
//     is rebuilt, every nibble is looked up in the 16-entry codebook held in
//     LDS (lookups issued one quarter-step before their use), multiplied by c'
//     in fp32, rounded to bf16 and written to LDS row-major [n][k] for both
//     passes. dX contracts over n, so its MFMA operand needs 8 consecutive n
//     per lane: gfx950's transposing LDS read (ds_read_b64_tr_b16) gathers
//     them from the [n][k] tile, 4 rows per read. The dequant VALU/LDS work is
//     placed between the current step's MFMAs so the matrix core and the VALU
//     work at the same time.
// Tiles use an XOR swizzle of the 16-byte chunk index with the row, so the 32
// rows one fragment read touches fall in distinct LDS banks.
// Workgroups are ordered so that consecutive tiles of one XCD share operand
// rows (each XCD has its own L2).
#include <type_traits>

#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace qlora {

namespace {

using namespace gt;
// dX weight tile: 64 contraction rows (n) x 256 output columns (k), bf16,
// rows padded from 512 to 544 bytes so the 4 rows one transposing read
// touches start 8 banks apart.
constexpr int kDxPitch = 544;
constexpr int kDxTileBytes = 64 * kDxPitch;
constexpr int kBTileBytes = kDxTileBytes > kTileBytes ? kDxTileBytes : kTileBytes;

struct GemmArgs {
  // activation operand (rows = output rows), bf16, row stride lda, kc columns
  const uint16_t* act;
  int64_t lda;
  int64_t M;
  int64_t kc;             // contraction length of the base part (K fwd, N for dX)
  // low-rank extra contraction columns: [M, kx] bf16
  const uint16_t* act_x;
  int kx;
  // encoded weight [wn, wk]
  const uint8_t* codes;
  const uint8_t* code8;
  const float* s2;
  const float* mean;
  const float* codebook;
  bool s2_bf16;           // per-block bf16 scales (no double quantization)
  // a bf16 base weight [wn, wk] instead (kW16 kernels): its tile is copied as
  // it is, nothing to expand (the 16-bit-base LoRA layer the pages compare
  // QLoRA with)
  const uint16_t* w16;
  int64_t wn, wk;
  // low-rank second factor: B [wn, r] (forward) or A [r, wk] (dX)
  const uint16_t* lr;
  int r;
  // output [M, nout] bf16
  uint16_t* out;
  int64_t nout;
  // dX only: dropout on the low-rank term, uint8 [M, nout] (NULL: none)
  const uint8_t* mask;
  float keep_scale;
};

// ------------------------------------------------------------ activation tile
// 256 rows x 8 chunks of 16 B: thread t owns chunks t + 512 i, i = 0..3
// (each wavefront instruction covers 8 full rows).
constexpr int kActChunks = 256 * 8 / kThreads;
struct ActStage {
  u32x4 v[kActChunks];
};

// Branch-free: out-of-range rows / columns read a clamped in-range address and
// are then zeroed with a select, so the pipelined loop stays one basic block
// (which lets its MFMA and VALU instructions be interleaved).
template <bool kVec>
__device__ __forceinline__ void load_act(const GemmArgs& a, int64_t m0, int step, int nk_main, ActStage& st) {
  const int t = threadIdx.x;
  const bool extra = step >= nk_main;
  const uint16_t* src = extra ? a.act_x : a.act;
  const int64_t ld = extra ? (int64_t)a.kx : a.lda;
  const int64_t cols = extra ? (int64_t)a.kx : a.kc;
  const int64_t c0 = (int64_t)(extra ? step - nk_main : step) * kBK;
#pragma unroll
  for (int i = 0; i < kActChunks; ++i) {
    const int q = t + i * kThreads;
    const int row = q >> 3, ch = q & 7;
    const int64_t m = m0 + row;
    const int64_t mc = m < a.M ? m : a.M - 1;
    const int64_t c = c0 + ch * 8;
    u32x4 v;
    if (extra || kVec) {
      const int64_t cc = c < cols ? c : cols - 8;
      v = *reinterpret_cast<const u32x4*>(src + mc * ld + cc);
      const bool ok = (m < a.M) && (c < cols);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = ok ? v[j] : 0u;
    } else {
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t cj = c + j < cols ? c + j : cols - 1;
        const uint32_t x = src[mc * ld + cj];
        e[j] = (m < a.M && c + j < cols) ? x : 0u;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = e[2 * j] | (e[2 * j + 1] << 16);
    }
    st.v[i] = v;
  }
}

// Direct global -> LDS copy of the activation tile for `step` (16-B rows
// required: the forward always, dX when n % 8 == 0): the base operand for the
// first nk_main steps, then the low-rank split columns. Chunks past the last
// contraction column re-read the last in-range chunk; the weight rows they
// meet are exactly zero and the data are finite.
__device__ __forceinline__ void issue_act_lds(const GemmArgs& a, int64_t m0, int step, int nk_main, char* As) {
  // selects, not a branch: the pipelined loop body stays one basic block
  const bool extra = step >= nk_main;
  const uint16_t* src = extra ? a.act_x : a.act;
  const int64_t ld = extra ? (int64_t)a.kx : a.lda;
  const int64_t cols = extra ? (int64_t)a.kx : a.kc;
  const int64_t c0 = (int64_t)(extra ? step - nk_main : step) * kBK;
  issue_tile_lds(src, ld, a.M, m0, cols, c0, As);
}

__device__ __forceinline__ void store_act(char* As, const ActStage& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kActChunks; ++i) {
    const int q = t + i * kThreads;
    *reinterpret_cast<u32x4*>(As + swz(q >> 3, q & 7)) = st.v[i];
  }
}

// ------------------------------------------------------------ weight tile
// Both passes expand the tile in its stored orientation, half a block per
// thread: 16 bytes of codes (32 weights, one scale) -> 4 chunks of 8 bf16,
// one 16-byte LDS write each.
// Forward: 256 rows (n) x 64 (k); thread t: row t / 2, columns 32 (t % 2) ...
// dX: 64 rows (n, the contraction) x 256 columns (k, the output); thread t:
// row t / 8, columns 32 (t % 8) ...; 8 consecutive threads cover 128
// contiguous bytes of one code row.
struct WStage {
  uint32_t q[4];  // 4 code words (32 weights)
  uint32_t c8;    // raw code8 byte of the block
  float s2v;      // raw second-level scale of the block
  u32x4 w[4];     // kW16: the 32 bf16 weights themselves
};

// Rows outside the weight get code 7 (the zero level) so they contribute
// exactly zero wherever they enter a contraction.
template <bool kDX, bool kW16 = false>
__device__ __forceinline__ void load_w(const GemmArgs& a, int64_t n0, int step, WStage& st) {
  const int t = threadIdx.x;
  const int64_t kblocks = a.wk / kBlock;
  int64_t n, k;
  if constexpr (!kDX) {
    n = n0 + (t >> 1);
    k = (int64_t)step * kBK + (t & 1) * 32;
  } else {
    n = (int64_t)step * kBK + (t >> 3);
    k = n0 + (t & 7) * 32;  // n0 is the output-column origin for dX
  }
  const bool ok = n < a.wn && k < a.wk;
  const int64_t nc = n < a.wn ? n : a.wn - 1;
  const int64_t kc = k < a.wk ? k : a.wk - 32;
  if constexpr (kW16) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.w16 + nc * a.wk + kc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = src[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) st.w[j][e] = ok ? v[e] : 0u;
    }
    return;
  }
  const u32x4 q = *reinterpret_cast<const u32x4*>(a.codes + nc * (a.wk / 2) + kc / 2);
  const int64_t blk = nc * kblocks + kc / kBlock;
  scale_fields(a.code8, a.s2, a.s2_bf16, blk, st.c8, st.s2v);
#pragma unroll
  for (int j = 0; j < 4; ++j) st.q[j] = ok ? q[j] : 0x77777777u;
}

// Codebook lookups of quarter `part` (8 weights, one code word).
__device__ __forceinline__ void lookup_part(const float* lut, const WStage& st, int part, float (&lv)[8]) {
  const uint32_t word = st.q[part];
#pragma unroll
  for (int e = 0; e < 8; ++e) lv[e] = lut[(word >> (4 * e)) & 0xF];
}

// Scale, round to bf16 and write quarter `part` (one 16-byte chunk) into LDS.
template <bool kDX>
__device__ __forceinline__ void finish_part(char* Bs, const float (&lv)[8], float cp, int part) {
  const int t = threadIdx.x;
  u32x4 v;
#pragma unroll
  for (int p2 = 0; p2 < 4; ++p2) v[p2] = pack_bf16x2(nf4_scaled(lv[2 * p2], cp), nf4_scaled(lv[2 * p2 + 1], cp));
  if constexpr (!kDX) {
    *reinterpret_cast<u32x4*>(Bs + swz(t >> 1, (t & 1) * 4 + part)) = v;
  } else {
    *reinterpret_cast<u32x4*>(Bs + (t >> 3) * kDxPitch + ((t & 7) * 32 + part * 8) * 2) = v;
  }
}

__device__ __forceinline__ float decode_scale(const WStage& st, float mean) {
  return decode_block_scale(st.c8, st.s2v, mean);
}

// kW16: quarter `part` of the copied bf16 weights into LDS, where
// finish_part would put the expanded ones.
template <bool kDX>
__device__ __forceinline__ void store_part16(char* Bs, const WStage& st, int part) {
  const int t = threadIdx.x;
  if constexpr (!kDX) {
    *reinterpret_cast<u32x4*>(Bs + swz(t >> 1, (t & 1) * 4 + part)) = st.w[part];
  } else {
    *reinterpret_cast<u32x4*>(Bs + (t >> 3) * kDxPitch + ((t & 7) * 32 + part * 8) * 2) = st.w[part];
  }
}

// Whole tile at once (prologue).
template <bool kDX, bool kW16 = false>
__device__ __forceinline__ void store_w_all(char* Bs, const float* lut, const WStage& st, float mean) {
  if constexpr (kW16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) store_part16<kDX>(Bs, st, p);
    return;
  }
  const float cp = decode_scale(st, mean);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float lv[8];
    lookup_part(lut, st, p, lv);
    finish_part<kDX>(Bs, lv, cp, p);
  }
}

// Low-rank step `xs` (64 of the 2r extra contraction columns): write the tile
// of [B | B] (forward, [n][j]) or [A ; A] (dX, [k][j]) straight into LDS.
template <bool kDX>
__device__ __forceinline__ void store_lowrank_w(char* Bs, const GemmArgs& a, int64_t n0, int xs) {
  const int t = threadIdx.x;
  if constexpr (!kDX) {
    // rows n of [B | B]: 64 extra contraction columns j per row
    const int row = t >> 1, half = t & 1;
    const int j0 = xs * kBK + half * 32;
    const int64_t g = n0 + row;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 v;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = j0 + c * 8 + 2 * p + e;
          h[e] = (g < a.wn && j < 2 * a.r) ? (uint32_t)a.lr[g * a.r + (j % a.r)] : 0u;
        }
        v[p] = h[0] | (h[1] << 16);
      }
      *reinterpret_cast<u32x4*>(Bs + swz(row, half * 4 + c)) = v;
    }
  } else {
    // rows j of [A ; A] (the contraction), 256 output columns k per row
    const int row = t >> 3;
    const int j = xs * kBK + row;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t k = n0 + (t & 7) * 32 + c * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (j < 2 * a.r && k < a.wk) v = *reinterpret_cast<const u32x4*>(a.lr + (int64_t)(j % a.r) * a.wk + k);
      *reinterpret_cast<u32x4*>(Bs + row * kDxPitch + ((t & 7) * 32 + c * 8) * 2) = v;
    }
  }
}

// B-operand fragment of v_mfma_f32_32x32x16_bf16 for dX: output column
// c = cb + lane % 32, contraction rows r0 + 8 (lane / 32) .. +7 of the [n][k]
// tile. Two transposing reads of 4 rows each: inside every 16-lane group,
// lane i addresses row base + i / 4, columns 4 (i % 4) .. +3 of its 16-column
// slice, and receives its own column of the 4 rows.
__device__ __forceinline__ bf16x8 dx_b_frag(const char* Bc, int cb, int r0, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int i = lane & 15;
  const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
  const int row = r0 + 8 * (lane >> 5) + (i >> 2);
  const char* p = Bc + row * kDxPitch + col * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 4 * kDxPitch));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------ one step
// MFMAs of the current step on (Ac, Bc) while the next step's weight tile is
// expanded into Bn and its activation tile is copied into An. The four LDS
// buffers are passed as restrict pointers: the compiler then knows the
// direct copies into An cannot alias the fragment reads of Ac, and does not
// wait for those copies before reading.

template <bool kDX, bool kVec, bool kW16>
__device__ __forceinline__ void pipelined_step(const GemmArgs& a, int step, int nk_main, int64_t m0, int64_t n0,
                                               const char* __restrict__ Ac, const char* __restrict__ Bc,
                                               char* __restrict__ An, char* __restrict__ Bn, const float* lut,
                                               float mean, WStage& wcur, WStage& wnxt, ActStage& ast,
                                               f32x16 (&acc)[kTM][kTN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  const int s1 = step + 1 < nk_main ? step + 1 : nk_main - 1;
  const int s2 = step + 2 < nk_main ? step + 2 : nk_main - 1;
  bf16x8 af[2][kTM], bfr[2][kTN];
  auto read_frags = [&](int kk, int buf) {
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
      af[buf][i] = *reinterpret_cast<const bf16x8*>(Ac + swz(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      if constexpr (!kDX)
        bfr[buf][j] = *reinterpret_cast<const bf16x8*>(Bc + swz(wn0 + j * 32 + (lane & 31), ch));
      else
        bfr[buf][j] = dx_b_frag(Bc, wn0 + j * 32, 16 * kk, lane);
    }
  };
  // first consume what the previous step loaded, before issuing new loads
  const float cp = kW16 ? 0.0f : decode_scale(wnxt, mean);
  float lv[2][8];
  if constexpr (!kW16) lookup_part(lut, wnxt, 0, lv[0]);
  read_frags(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kVec) issue_act_lds(a, m0, s1, nk_main, An);
  __builtin_amdgcn_sched_barrier(0);  // the copies stay ahead of the weight loads
  load_w<kDX, kW16>(a, n0, s2, wcur);
  __builtin_amdgcn_sched_barrier(0);  // issue the weight loads now, a full step ahead of their use
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    const int cb = kk & 1;
    // next quarter's fragments and codebook lookups go out before this
    // quarter's MFMAs, so their LDS latency is covered by the MFMAs
    if (kk < 3) {
      read_frags(kk + 1, cb ^ 1);
      if constexpr (!kW16) lookup_part(lut, wnxt, kk + 1, lv[cb ^ 1]);
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bfr[cb][j], acc[i][j], 0, 0, 0);
    if constexpr (kW16)
      store_part16<kDX>(Bn, wnxt, kk);
    else
      finish_part<kDX>(Bn, lv[cb], cp, kk);
  }
  if constexpr (!kVec) {
    store_act(An, ast);
    load_act<kVec>(a, m0, s2, nk_main, ast);
  }
  if constexpr (kVec) {
    step_barrier<3>();  // weight loads per thread after the copies: codes, code8, s2
  } else {
    __syncthreads();
  }
}

// ------------------------------------------------------------ kernel
template <bool kDX, bool kVec, bool kW16 = false>
__global__ __launch_bounds__(kThreads) void gemm_nf4_kernel(GemmArgs a) {
  constexpr int TM = kTM, TN = kTN;
  // four separate arrays (not one [2][...] array) so the compiler can tell the
  // buffer being filled by direct global->LDS copies from the one being read
  __shared__ __attribute__((aligned(16))) char As0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char As1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs0[kBTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs1[kBTileBytes];
  __shared__ float lut[16];
  char* const As[2] = {As0, As1};
  char* const Bs[2] = {Bs0, Bs1};

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  int64_t tm, tn;
  tile_of(tm, tn, cdiv(a.M, kBM), cdiv(a.nout, kBN));
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  if (!kW16 && t < 16) lut[t] = a.codebook[t];

  const int nk_main = (int)cdiv(a.kc, kBK);
  const int nk = nk_main + a.kx / kBK;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto mfma_step = [&](const char* Ac, const char* Bc, auto&& between) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(Ac + swz(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (!kDX)
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bc + swz(wn0 + j * 32 + (lane & 31), ch));
        else
          bfr[j] = dx_b_frag(Bc, wn0 + j * 32, 16 * kk, lane);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      between(kk);
    }
  };

  ActStage ast;
  WStage wst[2];
  const float mean = weight_mean(a.code8, a.mean);
  // low-rank extra steps (1 or 2 for r <= 64): not pipelined
  auto lowrank_steps = [&]() {
    for (int xs = 0; xs < nk - nk_main; ++xs) {
      load_act<kVec>(a, m0, nk_main + xs, nk_main, ast);
      store_act(As[0], ast);
      store_lowrank_w<kDX>(Bs[0], a, n0, xs);
      __syncthreads();
      mfma_step(As[0], Bs[0], [](int) {});
      __syncthreads();
    }
  };
  // dropout (dX): the low-rank term alone first, masked and scaled, then the
  // main contraction on top of it
  const bool masked = kDX && a.mask != nullptr && nk > nk_main;
  if (masked) {
    lowrank_steps();
    mask_acc(acc, a.mask, a.keep_scale, a.M, a.nout, m0, n0, wm0, wn0, lane);
  }
  // prologue: step 0 into buffer 0; step 1 activations and weights staged
  if constexpr (kVec) {
    issue_act_lds(a, m0, 0, nk_main, As[0]);
  } else {
    load_act<kVec>(a, m0, 0, nk_main, ast);
  }
  load_w<kDX, kW16>(a, n0, 0, wst[0]);
  load_w<kDX, kW16>(a, n0, nk_main > 1 ? 1 : 0, wst[1]);
  __syncthreads();  // lut
  if constexpr (!kVec) {
    store_act(As[0], ast);
    load_act<kVec>(a, m0, nk_main > 1 ? 1 : 0, nk_main, ast);
  }
  store_w_all<kDX, kW16>(Bs[0], lut, wst[0], mean);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // The stage index and buffers are compile-time choices (loop unrolled by 2),
  // so staging registers are never indexed dynamically. Loads for steps past
  // the last one use a clamped step index (re-reading the last step); the LDS
  // writes they feed land in a buffer no later step reads, keeping the body
  // free of branches.
  for (int step = 0; step < nk_main; step += 2) {
    pipelined_step<kDX, kVec, kW16>(a, step, nk_main, m0, n0, As0, Bs0, As1, Bs1, lut, mean, wst[0], wst[1], ast,
                                    acc);
    if (step + 1 < nk_main)
      pipelined_step<kDX, kVec, kW16>(a, step + 1, nk_main, m0, n0, As1, Bs1, As0, Bs0, lut, mean, wst[1], wst[0],
                                      ast, acc);
  }
  if (!masked) lowrank_steps();

  // D layout: lane -> column (lane & 31); register v -> row 8 (v/4) + 4 (lane/32) + v%4
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn0 + j * 32 + (lane & 31);
      if (n >= a.nout) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < a.M) a.out[m * a.nout + n] = to_bf16_bits(acc[i][j][v]);
      }
    }
}

}  // namespace

hipError_t launch_gemm_fwd(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* TS, const uint16_t* B,
                           int r, uint16_t* Y, hipStream_t stream) {
  GemmArgs a{};
  a.act = X; a.lda = w.k; a.M = M; a.kc = w.k;
  a.act_x = TS; a.kx = lora_extra_cols(r);
  a.codes = w.codes; a.code8 = w.code8; a.s2 = w.s2; a.mean = w.mean; a.codebook = w.codebook;
  a.s2_bf16 = w.s2_bf16;
  a.wn = w.n; a.wk = w.k;
  a.lr = B; a.r = r;
  a.out = Y; a.nout = w.n;
  const dim3 grid((unsigned)(cdiv(w.n, kBN) * cdiv(M, kBM)));
  gemm_nf4_kernel<false, true><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const Nf4View& w, const uint16_t* dY, int64_t M, const uint16_t* US, const uint16_t* A,
                          int r, uint16_t* dX, hipStream_t stream, const uint8_t* mask, float keep_scale) {
  GemmArgs a{};
  a.mask = mask;
  a.keep_scale = keep_scale;
  a.act = dY; a.lda = w.n; a.M = M; a.kc = w.n;
  a.act_x = US; a.kx = lora_extra_cols(r);
  a.codes = w.codes; a.code8 = w.code8; a.s2 = w.s2; a.mean = w.mean; a.codebook = w.codebook;
  a.s2_bf16 = w.s2_bf16;
  a.wn = w.n; a.wk = w.k;
  a.lr = A; a.r = r;
  a.out = dX; a.nout = w.k;
  const dim3 grid((unsigned)(cdiv(w.k, kBN) * cdiv(M, kBM)));
  if (w.n % 8 == 0)
    gemm_nf4_kernel<true, true><<<grid, kThreads, 0, stream>>>(a);
  else
    gemm_nf4_kernel<true, false><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_w16_dx(const uint16_t* W, int64_t n, int64_t k, const uint16_t* dY, int64_t M,
                              const uint16_t* US, const uint16_t* A, int r, uint16_t* dX, hipStream_t stream) {
  GemmArgs a{};
  a.act = dY; a.lda = n; a.M = M; a.kc = n;
  a.act_x = US; a.kx = lora_extra_cols(r);
  a.w16 = W;
  a.wn = n; a.wk = k;
  a.lr = A; a.r = r;
  a.out = dX; a.nout = k;
  const dim3 grid((unsigned)(cdiv(k, kBN) * cdiv(M, kBM)));
  if (n % 8 == 0)
    gemm_nf4_kernel<true, true, true><<<grid, kThreads, 0, stream>>>(a);
  else
    gemm_nf4_kernel<true, false, true><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qlora
