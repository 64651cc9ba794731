// Plain bf16 MFMA GEMM over an expanded weight operand (large token counts).
//
//   out[m, j] = RN_bf16( sum_c act[m, c] F[j, c] + sum_x split[m, x] F[j, kcp + x] )
//
// with F the operand written by expand.hip ([n, k + xc] for the forward, the
// transposed [k, np + xc] for dX) and kcp the contraction length rounded up to
// 64. The low-rank columns are the hi/lo halves of s*T or s*U, so the output
// is rounded once from an fp32 accumulator holding the whole sum
// ("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// three-piece summary, pieces 2 and 3).
//
// Same tile shape as the fused kernel (gemm_tile.h): 256 x 256 outputs per
// workgroup, 8 waves each computing 128 x 64 with v_mfma_f32_32x32x16_bf16,
// 64-deep steps. Both operand tiles go global -> LDS with direct buffer loads
// into LDS (no registers, no VALU): the activation tile in two buffers, the
// weight tile in three (160 KB of LDS). Step s issues the activation copies of
// step s + 1 and the weight copies of step s + 2, so a weight copy has two
// steps to land, and one barrier per step (after its third substep)
// separates filling a buffer from reading it; the buffers rotate with period
// six. Activations above 128 MB take the mirrored ring (activation in three
// buffers, weight in two).
//
// Per-step cost is kept off the vector ALU: every lane's byte offset inside
// each operand (row, swizzled chunk) is computed once, and a step only moves
// a scalar offset by 128 bytes. The copies are buffer loads into LDS (one
// descriptor per operand, 32-bit lane offset + scalar step offset): measured
// 4-8% faster for the whole GEMM than the same copies issued as global loads
// into LDS, which need a 64-bit address per lane. Inside a step the next substep's
// fragment reads are interleaved one-to-one with the current substep's MFMAs
// (scheduling groups), so LDS latency hides behind the matrix core. The
// epilogue stages each wave's bf16 outputs through LDS and writes full 16-byte
// row segments.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace qlora {

namespace {

using namespace gt;

struct BfArgs {
  const uint16_t* act;   // [M, kc] bf16
  int64_t M, kc;
  const uint16_t* act_x; // [M, kx] low-rank split columns
  int kx;
  const uint16_t* f;     // [nout, ldf] weight operand (rows = outputs), ldf >= 64 * nk_main
  int64_t ldf, nout;
  const uint16_t* fx;    // [nout, ldx] low-rank operand rows [B | B | 0] or [A ; A ; 0]^T (kx columns)
  int64_t ldx;
  uint16_t* out;         // [M, nout]
  // Workgroups [0, full) compute whole tiles (tiles 0 .. full-1 in tile_of
  // order); the `tail` tiles after them are each split over `splits`
  // workgroups along the contraction, whose fp32 sums go to `part`
  // ([splits][tail][256 x 256], tile-local row-major).
  float* part;
  int64_t full, tail;
  int splits;
  // dropout on the low-rank term (the masked kernel only): uint8 [M, nout]
  const uint8_t* mask;
  float keep_scale;
};

constexpr int kCopies = 32 / kWaves;  // 1 KB copies per wave per operand tile

// Byte offsets of this lane's copies, relative to the operands' base pointer
// advanced to the step's first column. For the last base step of a ragged
// contraction (kc % 64 != 0) the column is clamped to the last in-range chunk
// (the F rows it meets there are exactly zero).
// (Vectors, not arrays: an array in a struct may be placed in LDS by the
// compiler, which would turn every copy into an LDS read first.)
static_assert(kCopies == 4, "one u32x4 of offsets per operand");
struct CopyPlan {
  u32x4 a;      // activation, base steps
  u32x4 alast;  // activation, last base step (clamped columns)
  u32x4 x;      // low-rank split columns
  u32x4 f;      // weight operand, base steps
  u32x4 fx;     // low-rank operand
};

// kNN: the weight operand is stored [contraction][output] (a bf16 base W
// [n, k] for dX): its tile is 64 contraction rows x 256 output columns, 512 B
// per row, and an instruction copies two rows; 16-byte chunk c of row r sits
// at c ^ (4 (r & 3)), so the four rows one transposing fragment read touches
// fall on distinct banks.
__device__ __forceinline__ int nn_key(int row) { return 4 * (row & 3); }

template <bool kNN>
__device__ __forceinline__ void make_plan(const BfArgs& a, int64_t m0, int64_t n0, int nk_main, int wave, CopyPlan& p) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int row = (wave * kCopies + i) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz_key(row);
    const int64_t m = m0 + row < a.M ? m0 + row : a.M - 1;
    p.a[i] = (uint32_t)((m * a.kc + 8 * lc) * 2);
    const int64_t cl = (int64_t)(nk_main - 1) * kBK + 8 * lc;
    const int64_t cc = cl < a.kc ? cl : a.kc - 8;
    p.alast[i] = (uint32_t)((m * a.kc + cc - (int64_t)(nk_main - 1) * kBK) * 2);
    p.x[i] = (uint32_t)((m * a.kx + 8 * lc) * 2);
    if constexpr (!kNN) {
      const int64_t n = n0 + row < a.nout ? n0 + row : a.nout - 1;
      p.f[i] = (uint32_t)((n * a.ldf + 8 * lc) * 2);
      p.fx[i] = (uint32_t)((n * a.ldx + 8 * lc) * 2);
    } else {
      // rows 2 blk, 2 blk + 1 of the step's 64; output columns past nout read
      // other data (those outputs are never stored), rows past the end of the
      // operand read zeros (buffer range check)
      const int blk = wave * kCopies + i;
      const int r = 2 * blk + (lane >> 5);
      const int c = (lane & 31) ^ nn_key(r);
      p.f[i] = (uint32_t)((r * a.ldf + n0 + 8 * c) * 2);
      p.fx[i] = (uint32_t)((r * a.ldx + n0 + 8 * c) * 2);
    }
  }
}

// B-operand fragment of v_mfma_f32_32x32x16_bf16 from a kNN tile: output
// column cb + lane % 32, contraction rows 16 kk + 8 (lane / 32) .. +7. Two
// transposing reads of 4 rows each: in every 16-lane group lane i addresses
// row base + i / 4, columns 4 (i % 4) .. +3 of its 16 columns.
__device__ __forceinline__ bf16x8 nn_frag(const char* T, int cb, int kk, int lane) {
  const int i = lane & 15;
  const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
  const int row = 16 * kk + 8 * (lane >> 5) + (i >> 2);
  const char* p = T + row * 512 + (((col >> 3) ^ nn_key(row)) << 4) + (col & 7) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 4 * 512));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <bool kNN>
__device__ __forceinline__ bf16x8 b_frag(const char* Bc, int cb, int kk, int lane) {
  if constexpr (kNN)
    return nn_frag(Bc, cb, kk, lane);
  else
    return tile_frag(Bc, cb, kk, lane);
}

struct Rsrc {
  i32x4 act, x, f, fx;
};

// Copies of step `step` into (As, Bs). The operand choice is wave-uniform
// (it depends on the step only), so descriptors and step offsets stay scalar.
template <bool kNN>
__device__ __forceinline__ void issue_step(const Rsrc& rs, const CopyPlan& p, int step, int nk_main, int wave,
                                           char* As, char* Bs, int64_t ldf, int64_t ldx) {
  // the weight operand advances 64 columns (NT) or 64 rows (NN) per step
  // (32-bit scalar offsets: unsigned arithmetic, operands under 4 GiB)
  const uint32_t fstep = kNN ? (uint32_t)(kBK * ldf * 2) : (uint32_t)(kBK * 2);
  const uint32_t xstep = kNN ? (uint32_t)(kBK * ldx * 2) : (uint32_t)(kBK * 2);
  char* const as = As + wave * kCopies * 1024;
  char* const bs = Bs + wave * kCopies * 1024;
  if (step < nk_main) {
    const u32x4 off = step == nk_main - 1 ? p.alast : p.a;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(rs.act, off[i], step * (kBK * 2), as + i * 1024);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(rs.f, p.f[i], (int)((uint32_t)step * fstep), bs + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(rs.x, p.x[i], (step - nk_main) * (kBK * 2), as + i * 1024);
#pragma unroll
    for (int i = 0; i < kCopies; ++i)
      copy16(rs.fx, p.fx[i], (int)((uint32_t)(step - nk_main) * xstep), bs + i * 1024);
  }
}

// The two operands' copies of step `step` issued separately (the weight
// side runs one step further ahead).
template <bool kNN>
__device__ __forceinline__ void issue_act(const Rsrc& rs, const CopyPlan& p, int step, int nk_main, int wave,
                                          char* As) {
  char* const as = As + wave * kCopies * 1024;
  if (step < nk_main) {
    const u32x4 off = step == nk_main - 1 ? p.alast : p.a;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(rs.act, off[i], step * (kBK * 2), as + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(rs.x, p.x[i], (step - nk_main) * (kBK * 2), as + i * 1024);
  }
}

template <bool kNN>
__device__ __forceinline__ void issue_wt(const Rsrc& rs, const CopyPlan& p, int step, int nk_main, int wave,
                                         char* Bs, int64_t ldf, int64_t ldx) {
  const uint32_t fstep = kNN ? (uint32_t)(kBK * ldf * 2) : (uint32_t)(kBK * 2);
  const uint32_t xstep = kNN ? (uint32_t)(kBK * ldx * 2) : (uint32_t)(kBK * 2);
  char* const bs = Bs + wave * kCopies * 1024;
  if (step < nk_main) {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(rs.f, p.f[i], (int)((uint32_t)step * fstep), bs + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kCopies; ++i)
      copy16(rs.fx, p.fx[i], (int)((uint32_t)(step - nk_main) * xstep), bs + i * 1024);
  }
}

// Fragments of one substep: 4 activation row blocks and 2 weight column
// blocks of the wave's 128 x 64 sub-tile.
struct StepFrags {
  bf16x8 af[2][kTM], bfr[2][kTN];  // double-buffered by substep parity
};

template <bool kNN>
__device__ __forceinline__ void read_substep(StepFrags& f, const char* Ac, const char* Bc, int wm0, int wn0, int kk,
                                             int buf, int lane) {
#pragma unroll
  for (int i = 0; i < kTM; ++i) f.af[buf][i] = tile_frag(Ac, wm0 + i * 32, kk, lane);
#pragma unroll
  for (int j = 0; j < kTN; ++j) f.bfr[buf][j] = b_frag<kNN>(Bc, wn0 + j * 32, kk, lane);
}

// One step: MFMAs on (Ac, Bc) while the activation copies of step + 1 fill
// An and the weight copies of step + 2 fill Bn2. Substeps 0-2 multiply, each
// with the next substep's fragment reads interleaved one-to-one with its
// MFMAs; then the copies of step + 1 (both operands) have landed, the weight
// copies of step + 2 may still be in flight, and all waves meet; then
// substep 3 multiplies while substep 0 of step + 1 is read from (An, Bn1),
// so the LDS latency after the barrier hides behind MFMAs. Restrict pointers
// tell the compiler the copies cannot alias the fragment reads, so it does
// not wait for them before reading. On entry f holds substep 0 (buffer 0);
// after the last step that read finds a repeated copy (valid data, not used).
// Measured in the 65B-class layer step (same box, each against the form
// before it): the weight copied two steps ahead with all four substeps
// before the barrier and raised issue priority, for operands above the
// last-level cache, 997 -> 981 ms (the six 22016-wide GEMMs 1181 -> 1158 us;
// the raised priority had made the two-buffer form 4-6% faster there); the
// same three buffers with this schedule for the cache-resident operands,
// 972.9 -> 967 ms (8192 x 8192 GEMMs 404-417 -> 400-402 us); this schedule
// for the larger operands too, 969.0 -> 951.2 ms (22016-wide GEMMs 1150 ->
// 1108 us; with the raised priority kept, 952.2 ms).
template <bool kF16, bool kNN>
__device__ __forceinline__ void bf16_step(const BfArgs& a, const Rsrc& rs, const CopyPlan& p, int step, int nk,
                                            int nk_main, int wave, const char* __restrict__ Ac,
                                            const char* __restrict__ Bc, char* __restrict__ An,
                                            const char* __restrict__ Bn1, char* __restrict__ Bn2,
                                            f32x16 (&acc)[kTM][kTN], StepFrags& f) {
  const int lane = threadIdx.x & 63;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  const int s1 = step + 1 < nk ? step + 1 : nk - 1;
  const int s2 = step + 2 < nk ? step + 2 : nk - 1;
  issue_act<kNN>(rs, p, s1, nk_main, wave, An);
  issue_wt<kNN>(rs, p, s2, nk_main, wave, Bn2, a.ldf, a.ldx);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kReads = kTM + (kNN ? 2 : 1) * kTN, kMfma = kTM * kTN;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    const int cb = kk & 1;
    read_substep<kNN>(f, Ac, Bc, wm0, wn0, kk + 1, cb ^ 1, lane);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32<kF16>(f.af[cb][i], f.bfr[cb][j], acc[i][j]);
  }
#pragma unroll
  for (int kk = 0; kk < 3; ++kk)
#pragma unroll
    for (int g = 0; g < kMfma; ++g) {
      if (g < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
    }
  __builtin_amdgcn_sched_barrier(0);
  step_barrier<kCopies>();
  __builtin_amdgcn_sched_barrier(0);
  read_substep<kNN>(f, An, Bn1, wm0, wn0, 0, 0, lane);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32<kF16>(f.af[1][i], f.bfr[1][j], acc[i][j]);
#pragma unroll
  for (int g = 0; g < kMfma; ++g) {
    if (g < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The same step with the roles of the operands swapped (activation tile in
// three buffers, copied two steps ahead; weight tile in two), for
// activations larger than the last-level cache holds beside the weight: the
// weight copies of step + 1 fill Bn, the activation copies of step + 2 fill
// An2, and after the barrier substep 0 of step + 1 is read from (An1, Bn).
// Measured in the 65B-class layer step: down's forward (activation H, 180 MB)
// 1101.6 -> 1084.8 us, the dX of gate / up (activation dG / dU) 1091-1094 ->
// 1058-1061 us, the step 946.9 -> 939.7 ms.
template <bool kF16, bool kNN>
__device__ __forceinline__ void bf16_step_a3(const BfArgs& a, const Rsrc& rs, const CopyPlan& p, int step, int nk,
                                             int nk_main, int wave, const char* __restrict__ Ac,
                                             const char* __restrict__ Bc, char* __restrict__ Bn,
                                             const char* __restrict__ An1, char* __restrict__ An2,
                                             f32x16 (&acc)[kTM][kTN], StepFrags& f) {
  const int lane = threadIdx.x & 63;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  const int s1 = step + 1 < nk ? step + 1 : nk - 1;
  const int s2 = step + 2 < nk ? step + 2 : nk - 1;
  issue_wt<kNN>(rs, p, s1, nk_main, wave, Bn, a.ldf, a.ldx);
  issue_act<kNN>(rs, p, s2, nk_main, wave, An2);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kReads = kTM + (kNN ? 2 : 1) * kTN, kMfma = kTM * kTN;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    const int cb = kk & 1;
    read_substep<kNN>(f, Ac, Bc, wm0, wn0, kk + 1, cb ^ 1, lane);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32<kF16>(f.af[cb][i], f.bfr[cb][j], acc[i][j]);
  }
#pragma unroll
  for (int kk = 0; kk < 3; ++kk)
#pragma unroll
    for (int g = 0; g < kMfma; ++g) {
      if (g < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
    }
  __builtin_amdgcn_sched_barrier(0);
  step_barrier<kCopies>();
  __builtin_amdgcn_sched_barrier(0);
  read_substep<kNN>(f, An1, Bn, wm0, wn0, 0, 0, lane);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32<kF16>(f.af[1][i], f.bfr[1][j], acc[i][j]);
#pragma unroll
  for (int g = 0; g < kMfma; ++g) {
    if (g < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <bool kNN>
__device__ __forceinline__ void prologue_a3(const BfArgs& a, const Rsrc& rs, const CopyPlan& p, int sbeg, int nk,
                                            int nk_main, int wave, char* __restrict__ A0, char* __restrict__ B0,
                                            char* __restrict__ A1) {
  issue_act<kNN>(rs, p, sbeg, nk_main, wave, A0);
  issue_wt<kNN>(rs, p, sbeg, nk_main, wave, B0, a.ldf, a.ldx);
  issue_act<kNN>(rs, p, sbeg + 1 < nk ? sbeg + 1 : nk - 1, nk_main, wave, A1);
  step_barrier<kCopies>();
}

// First copies: step sbeg of both operands and the
// weight of step sbeg + 1 (restrict pointers, as in the steps, so the
// compiler can tell these copies from the fragment reads of the loop).
template <bool kNN>
__device__ __forceinline__ void prologue(const BfArgs& a, const Rsrc& rs, const CopyPlan& p, int sbeg, int nk,
                                          int nk_main, int wave, char* __restrict__ A0, char* __restrict__ B0,
                                          char* __restrict__ B1) {
  issue_act<kNN>(rs, p, sbeg, nk_main, wave, A0);
  issue_wt<kNN>(rs, p, sbeg, nk_main, wave, B0, a.ldf, a.ldx);
  issue_wt<kNN>(rs, p, sbeg + 1 < nk ? sbeg + 1 : nk - 1, nk_main, wave, B1, a.ldf, a.ldx);
  step_barrier<kCopies>();
}

// One step without copies in flight: fragments of (Ac, Bc) and their MFMAs.
template <bool kF16, bool kNN>
__device__ __forceinline__ void plain_step(const char* Ac, const char* Bc, int wave, f32x16 (&acc)[kTM][kTN]) {
  const int lane = threadIdx.x & 63;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    bf16x8 af[kTM], bfr[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) af[i] = tile_frag(Ac, wm0 + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < kTN; ++j) bfr[j] = b_frag<kNN>(Bc, wn0 + j * 32, kk, lane);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = mfma32<kF16>(af[i], bfr[j], acc[i][j]);
  }
}

// The tile's 256 x 256 mask bytes, rows 0-127 into lo and 128-255 into hi
// (32 KB each, row-major), with direct copies: 8 of 1 KB (4 rows) per wave.
// Rows past M repeat the last row (never read back); nout is a multiple of
// 64 for dX, so a 16-byte piece never crosses the end of a row.
__device__ __forceinline__ void issue_mask_lds(const BfArgs& a, int64_t m0, int64_t n0, int wave, char* lo,
                                               char* hi) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave * 8 + i;                // 1 KB block: rows 4 blk .. +3
    const int row = blk * 4 + (lane >> 4);
    const int64_t m = m0 + row < a.M ? m0 + row : a.M - 1;
    const int64_t c = n0 + (lane & 15) * 16;
    const int64_t cc = c + 16 <= a.nout ? c : a.nout - 16;
    char* dst = (blk < 32 ? lo : hi) + (blk & 31) * 1024;
    __builtin_amdgcn_global_load_lds((const void*)(a.mask + m * a.nout + cc),
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  }
}

// Dropout on the accumulators while they hold only the low-rank term: keep
// scale where the staged mask byte is set, zero where it is not.
__device__ __forceinline__ void mask_acc_lds(f32x16 (&acc)[kTM][kTN], const char* lo, const char* hi,
                                             float keep_scale, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                             int wm0, int wn0, int lane) {
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int c = wn0 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const uint8_t mb = *reinterpret_cast<const uint8_t*>((rr < 128 ? lo : hi) + (rr & 127) * 256 + c);
        const bool keep = m0 + rr < M && n0 + c < N && mb != 0;
        acc[i][j][v] = keep ? acc[i][j][v] * keep_scale : 0.0f;
      }
    }
}

// kMask: dropout on the low-rank term. A workgroup whose step range holds the
// low-rank steps runs them first (unpipelined, 1-4 steps) on buffers 0 while
// the tile's mask bytes land in buffers 1, masks and scales the accumulators
// from there, then runs its main steps as usual.
// kF16: fp16 operands and output (the compute-type ablation), else bf16.
// kA3: the mirrored ring (bf16_step_a3; plain bf16 only).
template <bool kMask, bool kF16, bool kNN = false, bool kA3 = false>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(BfArgs a) {
  // four separate arrays so the compiler can tell the buffer being filled by
  // direct copies from the one being read
  __shared__ __attribute__((aligned(16))) char As0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char As1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs2[kTileBytes];  // third weight buffer

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  const int64_t mt = cdiv(a.M, (int64_t)kBM), nt = cdiv(a.nout, (int64_t)kBN);
  // workgroup -> whole tile, or (split, tail tile): split units come after
  // every whole tile, split 0 of all tail tiles first
  // (integer division leaves its result in vector registers: the values the
  // step loop and the copy offsets depend on are made wave-uniform again, so
  // descriptors and step offsets stay scalar)
  const int b = (int)blockIdx.x;
  const bool whole = b < a.full;
  const int unit = whole ? 0 : b - (int)a.full;
  const int tail_i = whole ? 0 : __builtin_amdgcn_readfirstlane(unit % (int)a.tail);
  const int split = whole ? 0 : __builtin_amdgcn_readfirstlane(unit / (int)a.tail);
  int64_t tm, tn;
  tile_of(tm, tn, mt, nt, whole ? (int64_t)b : a.full + tail_i);
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int nk_main = (int)cdiv(a.kc, (int64_t)kBK);
  const int nk_all = nk_main + a.kx / kBK;
  // this workgroup's contiguous range of 64-deep steps
  const int chunk = whole ? nk_all : __builtin_amdgcn_readfirstlane((nk_all + a.splits - 1) / a.splits);
  const int sbeg = split * chunk;
  const int nk = sbeg + chunk < nk_all ? sbeg + chunk : nk_all;  // exclusive end

  CopyPlan plan;
  make_plan<kNN>(a, m0, n0, nk_main, wave, plan);
  Rsrc rs;
  rs.act = make_rsrc(a.act, a.M * a.kc * 2);
  rs.x = make_rsrc(a.act_x, a.M * (int64_t)a.kx * 2);
  rs.f = make_rsrc(a.f, (kNN ? a.kc : a.nout) * a.ldf * 2);
  rs.fx = make_rsrc(a.fx, (kNN ? (int64_t)a.kx : a.nout) * a.ldx * 2);

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  int nk_end = nk;  // exclusive end of the pipelined range
  if constexpr (kMask) {
    if (nk > nk_main) {
      issue_mask_lds(a, m0, n0, wave, As1, Bs1);
      for (int step = sbeg > nk_main ? sbeg : nk_main; step < nk; ++step) {
        issue_step<kNN>(rs, plan, step, nk_main, wave, As0, Bs0, a.ldf, a.ldx);
        step_barrier<0>();  // (the first one also waits for the mask bytes)
        plain_step<kF16, kNN>(As0, Bs0, wave, acc);
        __syncthreads();  // every wave's reads done before the next copies land
      }
      mask_acc_lds(acc, As1, Bs1, a.keep_scale, a.M, a.nout, m0, n0, wm0, wn0, lane);
      __syncthreads();  // mask reads done before the main steps' copies reuse buffers 1
      nk_end = nk_main;
    }
  }
  if constexpr (kA3) {
    // activation ring of three (As0, As1, Bs2), weight ring of two (Bs0, Bs1)
    char* const A2 = Bs2;
    if (sbeg < nk_end) {
      prologue_a3<kNN>(a, rs, plan, sbeg, nk_end, nk_main, wave, As0, Bs0, As1);
      StepFrags f;
      read_substep<kNN>(f, As0, Bs0, wm0, wn0, 0, 0, lane);
      bf16_step_a3<kF16, kNN>(a, rs, plan, sbeg, nk_end, nk_main, wave, As0, Bs0, Bs1, As1, A2, acc, f);
      int s = sbeg + 1;
      for (; s + 6 <= nk_end; s += 6) {
        bf16_step_a3<kF16, kNN>(a, rs, plan, s, nk_end, nk_main, wave, As1, Bs1, Bs0, A2, As0, acc, f);
        bf16_step_a3<kF16, kNN>(a, rs, plan, s + 1, nk_end, nk_main, wave, A2, Bs0, Bs1, As0, As1, acc, f);
        bf16_step_a3<kF16, kNN>(a, rs, plan, s + 2, nk_end, nk_main, wave, As0, Bs1, Bs0, As1, A2, acc, f);
        bf16_step_a3<kF16, kNN>(a, rs, plan, s + 3, nk_end, nk_main, wave, As1, Bs0, Bs1, A2, As0, acc, f);
        bf16_step_a3<kF16, kNN>(a, rs, plan, s + 4, nk_end, nk_main, wave, A2, Bs1, Bs0, As0, As1, acc, f);
        bf16_step_a3<kF16, kNN>(a, rs, plan, s + 5, nk_end, nk_main, wave, As0, Bs0, Bs1, As1, A2, acc, f);
      }
      const int rem = nk_end - s;
      if (rem > 0) bf16_step_a3<kF16, kNN>(a, rs, plan, s, nk_end, nk_main, wave, As1, Bs1, Bs0, A2, As0, acc, f);
      if (rem > 1) bf16_step_a3<kF16, kNN>(a, rs, plan, s + 1, nk_end, nk_main, wave, A2, Bs0, Bs1, As0, As1, acc, f);
      if (rem > 2) bf16_step_a3<kF16, kNN>(a, rs, plan, s + 2, nk_end, nk_main, wave, As0, Bs1, Bs0, As1, A2, acc, f);
      if (rem > 3) bf16_step_a3<kF16, kNN>(a, rs, plan, s + 3, nk_end, nk_main, wave, As1, Bs0, Bs1, A2, As0, acc, f);
      if (rem > 4) bf16_step_a3<kF16, kNN>(a, rs, plan, s + 4, nk_end, nk_main, wave, A2, Bs1, Bs0, As0, As1, acc, f);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
      __syncthreads();
    }
  } else {
    if (sbeg < nk_end) {  // (every split range is non-empty for the split counts split_plan picks)
      prologue<kNN>(a, rs, plan, sbeg, nk_end, nk_main, wave, As0, Bs0, Bs1);
      StepFrags f;
      read_substep<kNN>(f, As0, Bs0, wm0, wn0, 0, 0, lane);
      bf16_step<kF16, kNN>(a, rs, plan, sbeg, nk_end, nk_main, wave, As0, Bs0, As1, Bs1, Bs2, acc, f);
      int s = sbeg + 1;
      for (; s + 6 <= nk_end; s += 6) {
        bf16_step<kF16, kNN>(a, rs, plan, s, nk_end, nk_main, wave, As1, Bs1, As0, Bs2, Bs0, acc, f);
        bf16_step<kF16, kNN>(a, rs, plan, s + 1, nk_end, nk_main, wave, As0, Bs2, As1, Bs0, Bs1, acc, f);
        bf16_step<kF16, kNN>(a, rs, plan, s + 2, nk_end, nk_main, wave, As1, Bs0, As0, Bs1, Bs2, acc, f);
        bf16_step<kF16, kNN>(a, rs, plan, s + 3, nk_end, nk_main, wave, As0, Bs1, As1, Bs2, Bs0, acc, f);
        bf16_step<kF16, kNN>(a, rs, plan, s + 4, nk_end, nk_main, wave, As1, Bs2, As0, Bs0, Bs1, acc, f);
        bf16_step<kF16, kNN>(a, rs, plan, s + 5, nk_end, nk_main, wave, As0, Bs0, As1, Bs1, Bs2, acc, f);
      }
      const int rem = nk_end - s;
      if (rem > 0) bf16_step<kF16, kNN>(a, rs, plan, s, nk_end, nk_main, wave, As1, Bs1, As0, Bs2, Bs0, acc, f);
      if (rem > 1) bf16_step<kF16, kNN>(a, rs, plan, s + 1, nk_end, nk_main, wave, As0, Bs2, As1, Bs0, Bs1, acc, f);
      if (rem > 2) bf16_step<kF16, kNN>(a, rs, plan, s + 2, nk_end, nk_main, wave, As1, Bs0, As0, Bs1, Bs2, acc, f);
      if (rem > 3) bf16_step<kF16, kNN>(a, rs, plan, s + 3, nk_end, nk_main, wave, As0, Bs1, As1, Bs2, Bs0, acc, f);
      if (rem > 4) bf16_step<kF16, kNN>(a, rs, plan, s + 4, nk_end, nk_main, wave, As1, Bs2, As0, Bs0, Bs1, acc, f);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
      __syncthreads();
    }
  }

  if (!whole) {
    // split unit: this range's fp32 sums go to the partial buffer (tile-local
    // layout), added in split order by gemm_bf16_reduce_kernel
    float* const pp = a.part + ((int64_t)split * a.tail + tail_i) * (kBM * kBN);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int c = wn0 + j * 32 + (lane & 31);
        if (n0 + c >= a.nout) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (m0 + rr < a.M) pp[rr * kBN + c] = acc[i][j][v];
        }
      }
    return;
  }

  // Epilogue: each wave writes its 128 x 64 bf16 block (16 KB) into its own
  // LDS region (all copies have landed and all fragment reads are done: the
  // step loop ends with a barrier after waiting for both), then stores
  // 16-byte row segments.
  {
    char* const bufs0 = wave < 4 ? (wave < 2 ? As0 : As1) : (wave < 6 ? Bs0 : Bs1);
    uint16_t* reg = reinterpret_cast<uint16_t*>(bufs0 + (wave & 1) * 16384);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          reg[rr * 64 + j * 32 + (lane & 31)] = to16<kF16>(acc[i][j][v]);
        }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<63>());  // this wave's LDS writes are done
    // 128 rows x 8 chunks of 16 B
#pragma unroll 4
    for (int q = lane; q < 128 * 8; q += 64) {
      const int rr = q >> 3, cc = q & 7;
      const int64_t m = m0 + wm0 + rr, n = n0 + wn0 + cc * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + rr * 64 + cc * 8);
      if (m < a.M) {
        if (n + 8 <= a.nout && (a.nout & 7) == 0) {
          *reinterpret_cast<u32x4*>(a.out + m * a.nout + n) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t h = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            if (n + e < a.nout) a.out[m * a.nout + n + e] = (uint16_t)h;
          }
        }
      }
    }
  }
}

// Tail tiles: out = RN_bf16(part[0] + part[1] + ... + part[S-1]), added in
// split order (deterministic; one rounding). Four adjacent outputs of one
// tile row per thread.
template <bool kF16>
__global__ __launch_bounds__(256) void gemm_bf16_reduce_kernel(const float* __restrict__ part, int64_t full,
                                                               int64_t tail, int splits, int64_t M, int64_t nout,
                                                               uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  constexpr int kTile = kBM * kBN;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 4
  const int64_t ti = g / (kTile / 4);
  if (ti >= tail) return;
  const int loc = (int)(g % (kTile / 4)) * 4;
  const int64_t mt = cdiv(M, (int64_t)kBM), nt = cdiv(nout, (int64_t)kBN);
  int64_t tm, tn;
  tile_of(tm, tn, mt, nt, full + ti);
  const int64_t m = tm * kBM + loc / kBN, n = tn * kBN + loc % kBN;
  if (m >= M || n >= nout) return;
  const float* p0 = part + ti * kTile + loc;
  float4 s = *reinterpret_cast<const float4*>(p0);
  for (int p = 1; p < splits; ++p) {
    const float4 v = *reinterpret_cast<const float4*>(p0 + (int64_t)p * tail * kTile);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  uint16_t* const o = out + m * nout + n;
  if (n + 4 <= nout && (nout & 3) == 0) {
    uint2 w;
    w.x = pack2<kF16>(s.x, s.y);
    w.y = pack2<kF16>(s.z, s.w);
    *reinterpret_cast<uint2*>(o) = w;
  } else {
    const float e[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < nout) o[i] = to16<kF16>(e[i]);
  }
}

struct SplitPlan {
  int64_t full, tail;
  int splits;
};

// One 256 x 256 workgroup fits a CU at a time (128 KB of LDS), so the 256
// CUs of an MI355X take the tiles in waves of 256. When the last wave holds
// at most 128 tiles, those tiles are split along the contraction: the
// largest power of two S <= 8 with tail * S <= 256 and at least 8 steps per
// split, so the last wave takes about 1/S of a whole tile's time (with fewer
// than 129 tiles in all, every tile is a tail tile).
constexpr int64_t kWaveTiles = 256;

SplitPlan split_plan(int64_t M, int64_t kc, int kx, int64_t nout) {
  const int64_t tiles = cdiv(M, (int64_t)kBM) * cdiv(nout, (int64_t)kBN);
  const int64_t nk = cdiv(kc, (int64_t)kBK) + kx / kBK;
  const int64_t rem = tiles % kWaveTiles;
  SplitPlan p{tiles, 0, 1};
  if (rem == 0 || rem > kWaveTiles / 2) return p;
  int s = 1;
  while (s < 8 && rem * s * 2 <= kWaveTiles && nk >= (int64_t)16 * s) s *= 2;
  if (s > 1) {
    p.full = tiles - rem;
    p.tail = rem;
    p.splits = s;
  }
  return p;
}

}  // namespace

int gemm_bf16_splits(int64_t M, int64_t kc, int kx, int64_t nout) { return split_plan(M, kc, kx, nout).splits; }

size_t gemm_bf16_ws_bytes(int64_t M, int64_t kc, int kx, int64_t nout) {
  const SplitPlan p = split_plan(M, kc, kx, nout);
  return p.splits > 1 ? align256((size_t)p.splits * (size_t)p.tail * kBM * kBN * 4) : 0;
}

bool gemm_bf16_offsets_fit(int64_t M, int64_t kc, int kx, int64_t nout) {
  const int64_t ldf = cdiv(kc, (int64_t)kBK) * kBK + kx;
  const int64_t lim = (int64_t)1 << 32;
  return M * kc * 2 < lim && M * (int64_t)kx * 2 < lim && nout * ldf * 2 < lim;
}

// activation bytes above which the activation takes the three-buffer ring
// (bf16_step_a3): more than half the 256 MB last-level cache, so it streams
// from HBM beside the weight instead of staying resident for its re-reads
constexpr int64_t kActStreamBytes = 128LL << 20;

hipError_t launch_gemm_bf16_ext(const uint16_t* act, int64_t M, int64_t kc, const uint16_t* split, int kx,
                                const uint16_t* f, int64_t ldf, const uint16_t* fx, int64_t ldx, int64_t nout,
                                uint16_t* out, float* part, hipStream_t stream, const uint8_t* mask, float keep_scale,
                                bool f16, bool nn) {
  BfArgs a{};
  a.mask = mask;
  a.keep_scale = keep_scale;
  a.act = act; a.M = M; a.kc = kc;
  a.act_x = split; a.kx = kx;
  a.f = f; a.ldf = ldf; a.nout = nout;
  a.fx = kx > 0 ? fx : f; a.ldx = kx > 0 ? ldx : ldf;
  a.out = out;
  const SplitPlan sp = split_plan(M, kc, kx, nout);
  a.full = sp.full; a.tail = sp.tail; a.splits = sp.splits;
  a.part = part;
  if (a.splits > 1 && part == nullptr) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.full + a.tail * a.splits));
  if (nn) {
    // the weight operand stored [contraction][output] (bf16 base, dX)
    if (mask != nullptr || f16) return hipErrorInvalidValue;
    if (M * kc * 2 > kActStreamBytes)
      gemm_bf16_kernel<false, false, true, true><<<grid, kThreads, 0, stream>>>(a);
    else
      gemm_bf16_kernel<false, false, true><<<grid, kThreads, 0, stream>>>(a);
  } else if (f16) {
    if (mask != nullptr && kx > 0)
      gemm_bf16_kernel<true, true><<<grid, kThreads, 0, stream>>>(a);
    else
      gemm_bf16_kernel<false, true><<<grid, kThreads, 0, stream>>>(a);
  } else {
    if (mask != nullptr && kx > 0)
      gemm_bf16_kernel<true, false><<<grid, kThreads, 0, stream>>>(a);
    else if (M * kc * 2 > kActStreamBytes)
      gemm_bf16_kernel<false, false, false, true><<<grid, kThreads, 0, stream>>>(a);
    else
      gemm_bf16_kernel<false, false><<<grid, kThreads, 0, stream>>>(a);
  }
  if (a.splits > 1) {
    const int64_t groups = a.tail * (kBM * kBN / 4);
    if (f16)
      gemm_bf16_reduce_kernel<true><<<dim3((unsigned)cdiv(groups, (int64_t)256)), 256, 0, stream>>>(
          part, a.full, a.tail, a.splits, M, nout, out);
    else
      gemm_bf16_reduce_kernel<false><<<dim3((unsigned)cdiv(groups, (int64_t)256)), 256, 0, stream>>>(
          part, a.full, a.tail, a.splits, M, nout, out);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* act, int64_t M, int64_t kc, const uint16_t* split, int kx,
                            const uint16_t* f, int64_t nout, uint16_t* out, float* part, hipStream_t stream,
                            const uint8_t* mask, float keep_scale, bool f16) {
  // the expanded operand holds the low-rank rows right after the padded base
  // columns of each row: [W' (kcp) | low-rank (kx)]
  const int64_t kcp = cdiv(kc, (int64_t)kBK) * kBK;
  const int64_t ldf = kcp + kx;
  return launch_gemm_bf16_ext(act, M, kc, split, kx, f, ldf, f + kcp, ldf, nout, out, part, stream, mask, keep_scale,
                              f16, false);
}

}  // namespace qlora
