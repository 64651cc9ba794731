// Tile machinery shared by the two large-M GEMM kernels (fused NF4 dequant
// and expanded bf16): workgroup shape, LDS tile layout, direct global->LDS
// copies, XCD-aware tile order and the step barrier.
//
// Workgroup tile 256 x 256 outputs, 64-deep contraction steps, 512 threads =
// 8 waves (two per SIMD) in a 2 x 4 grid, each wave a 128 x 64 sub-tile of
// v_mfma_f32_32x32x16_bf16. An operand tile is 256 rows x 64 bf16 (128 B per
// row = 8 chunks of 16 B); chunk c of row r is stored at chunk c ^ key(r),
// key(r) = (r & 7) ^ ((r >> 3) & 1). A fragment read sends 16 consecutive
// rows of one logical chunk to the LDS per cycle (256 B across its 64 banks):
// consecutive rows alternate 128-B halves, and the key gives rows r and r + 8
// (same half) different chunks, so the 16 reads hit 16 distinct 16-B bank
// groups. (The plain r & 7 key maps r and r + 8 to the same banks: measured
// as one conflict cycle per LDS cycle.)
#pragma once

#include "common.h"

namespace qlora {
namespace gt {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kTileBytes = 256 * 128;  // one 256-row x 64-col bf16 tile
constexpr int kTM = 4, kTN = 2;        // 32x32 MFMA tiles per wave (128 x 64 outputs)

__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_key(row)) << 4); }

// Direct global -> LDS copy of one 256 x 64 tile: rows r0 .. r0+255 and
// columns c0 .. c0+63 of a row-major bf16 matrix with leading dimension ld
// (rows and ld*2 bytes must keep every 16-byte chunk 16-byte aligned). Each
// wavefront instruction fills one contiguous 1 KB of LDS = 8 tile rows; lane l
// lands at row 8 b + l / 8, physical chunk l % 8, so it fetches logical chunk
// (l % 8) ^ key(row). Every address stays inside the matrix: rows past
// `rows` read the last row and chunks past `cols` read the last chunk; the
// caller makes those positions harmless (outputs never stored, or the other
// operand is zero there).
__device__ __forceinline__ void issue_tile_lds(const uint16_t* src, int64_t ld, int64_t rows, int64_t r0,
                                               int64_t cols, int64_t c0, char* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 32 / kWaves; ++i) {
    const int blk = wave * (32 / kWaves) + i;
    const int row = blk * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz_key(row);
    const int64_t m = r0 + row;
    const int64_t mc = m < rows ? m : rows - 1;
    const int64_t c = c0 + 8 * lc;
    const int64_t cc = c < cols ? c : cols - 8;
    const uint16_t* g = src + mc * ld + cc;
    __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)(dst + blk * 1024), 16,
                                     0, 0);
  }
}

// Logical tile index of workgroup `bid`: hardware dispatches workgroup i to
// XCD i % 8, so give each XCD a contiguous range of logical tiles; within the
// range, walk groups of 8 activation row-tiles column by column.
__device__ __forceinline__ void tile_of(int64_t& tm, int64_t& tn, int64_t mt, int64_t nt, int64_t bid) {
  const int64_t total = mt * nt;
  int64_t lin = bid;
  if (total % 8 == 0) lin = (bid % 8) * (total / 8) + bid / 8;
  constexpr int64_t G = 8;
  const int64_t group = lin / (G * nt);
  const int64_t first_m = group * G;
  const int64_t gm = (mt - first_m < G) ? mt - first_m : G;
  const int64_t in = lin % (G * nt);
  tm = first_m + in % gm;
  tn = in / gm;
}
__device__ __forceinline__ void tile_of(int64_t& tm, int64_t& tn, int64_t mt, int64_t nt) {
  tile_of(tm, tn, mt, nt, (int64_t)blockIdx.x);
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8. Waits until at most `vm` vector-memory operations are
// outstanding and all LDS operations are done; expcnt is left free.
template <int vm>
constexpr int waitcnt_vm_lgkm0() {
  return (vm & 0xF) | (0x7 << 4) | (0x0 << 8) | (((vm >> 4) & 0x3) << 14);
}

// End of a pipelined step: this wave's LDS traffic is done and all but the
// last `vm_after` vector-memory operations (its direct copies included) have
// completed; then all waves meet. The empty asm statements keep the compiler
// from moving memory operations across the barrier.
template <int vm_after>
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<vm_after>());
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row-major fragment of a swizzled 256 x 64 tile for v_mfma_f32_32x32x16_bf16:
// lane l holds row rb + l % 32, contraction elements 16 kk + 8 (l / 32) .. +7.
__device__ __forceinline__ bf16x8 tile_frag(const char* T, int rb, int kk, int lane) {
  return *reinterpret_cast<const bf16x8*>(T + swz(rb + (lane & 31), 2 * kk + (lane >> 5)));
}

// Accumulators -> bf16 outputs. D layout of v_mfma_f32_32x32x16: lane ->
// column (lane & 31); register v -> row 8 (v / 4) + 4 (lane / 32) + v % 4.
__device__ __forceinline__ void store_acc_bf16(const f32x16 (&acc)[kTM][kTN], uint16_t* out, int64_t ldo,
                                               int64_t M, int64_t N, int64_t m0, int64_t n0, int wm0, int wn0,
                                               int lane) {
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int64_t n = n0 + wn0 + j * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M) out[m * ldo + n] = to_bf16_bits(acc[i][j][v]);
      }
    }
}

// Dropout on the low-rank term of a tile: while the accumulators hold only
// that term (its contraction steps run first), each output (m, n) is
// multiplied by keep_scale where mask[m, n] is set and cleared where it is
// not (mask: uint8 [M, N], row-major).
__device__ __forceinline__ void mask_acc(f32x16 (&acc)[kTM][kTN], const uint8_t* __restrict__ mask, float keep_scale,
                                         int64_t M, int64_t N, int64_t m0, int64_t n0, int wm0, int wn0, int lane) {
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int64_t n = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const bool keep = m < M && n < N && mask[m * N + n] != 0;
        acc[i][j][v] = keep ? acc[i][j][v] * keep_scale : 0.0f;
      }
    }
}

}  // namespace gt
}  // namespace qlora
