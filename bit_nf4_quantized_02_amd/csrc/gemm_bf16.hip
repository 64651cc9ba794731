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
// 64-deep steps. Both operand tiles go global -> LDS with
// global_load_lds_dwordx4 (no registers, no VALU), double-buffered: the copies
// for step s + 1 are issued at the start of step s and waited for at its end,
// so one barrier per step separates filling a buffer from reading it.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace qlora {

namespace {

using namespace gt;

struct BfArgs {
  const uint16_t* act;   // [M, lda] bf16, kc columns used
  int64_t lda, M, kc;
  const uint16_t* act_x; // [M, kx] low-rank split columns
  int kx;
  const uint16_t* f;     // [nout, ldf] expanded operand, ldf = 64 * nk_main + kx
  int64_t ldf, nout;
  uint16_t* out;         // [M, nout]
};

__device__ __forceinline__ void issue_step(const BfArgs& a, int64_t m0, int64_t n0, int step, int nk_main,
                                           char* As, char* Bs) {
  const bool extra = step >= nk_main;
  const uint16_t* src = extra ? a.act_x : a.act;
  const int64_t ld = extra ? (int64_t)a.kx : a.lda;
  const int64_t cols = extra ? (int64_t)a.kx : a.kc;
  const int64_t c0 = (int64_t)(extra ? step - nk_main : step) * kBK;
  issue_tile_lds(src, ld, a.M, m0, cols, c0, As);
  issue_tile_lds(a.f, a.ldf, a.nout, n0, a.ldf, (int64_t)step * kBK, Bs);
}

// One step: MFMAs on (Ac, Bc) while the copies of step + 1 fill (An, Bn).
// Restrict pointers tell the compiler the copies cannot alias the fragment
// reads, so it does not wait for them before reading.
__device__ __forceinline__ void bf16_step(const BfArgs& a, int step, int nk, int nk_main, int64_t m0, int64_t n0,
                                          const char* __restrict__ Ac, const char* __restrict__ Bc,
                                          char* __restrict__ An, char* __restrict__ Bn, f32x16 (&acc)[kTM][kTN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  // past the last step the copy repeats the last step into a buffer no later
  // step reads: keeps the body free of branches
  const int s1 = step + 1 < nk ? step + 1 : nk - 1;
  bf16x8 af[2][kTM], bfr[2][kTN];
  auto read_frags = [&](int kk, int buf) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) af[buf][i] = tile_frag(Ac, wm0 + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < kTN; ++j) bfr[buf][j] = tile_frag(Bc, wn0 + j * 32, kk, lane);
  };
  read_frags(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_step(a, m0, n0, s1, nk_main, An, Bn);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    const int cb = kk & 1;
    if (kk < 3) read_frags(kk + 1, cb ^ 1);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bfr[cb][j], acc[i][j], 0, 0, 0);
  }
  step_barrier<0>();
}

__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(BfArgs a) {
  // four separate arrays so the compiler can tell the buffer being filled by
  // direct copies from the one being read
  __shared__ __attribute__((aligned(16))) char As0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char As1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char Bs1[kTileBytes];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;
  int64_t tm, tn;
  tile_of(tm, tn, cdiv(a.M, (int64_t)kBM), cdiv(a.nout, (int64_t)kBN));
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int nk_main = (int)cdiv(a.kc, (int64_t)kBK);
  const int nk = nk_main + a.kx / kBK;

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  issue_step(a, m0, n0, 0, nk_main, As0, Bs0);
  step_barrier<0>();
  for (int step = 0; step < nk; step += 2) {
    bf16_step(a, step, nk, nk_main, m0, n0, As0, Bs0, As1, Bs1, acc);
    if (step + 1 < nk) bf16_step(a, step + 1, nk, nk_main, m0, n0, As1, Bs1, As0, Bs0, acc);
  }
  store_acc_bf16(acc, a.out, a.nout, a.M, a.nout, m0, n0, wm0, wn0, lane);
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* act, int64_t M, int64_t kc, const uint16_t* split, int kx,
                            const uint16_t* f, int64_t nout, uint16_t* out, hipStream_t stream) {
  BfArgs a{};
  a.act = act; a.lda = kc; a.M = M; a.kc = kc;
  a.act_x = split; a.kx = kx;
  a.f = f; a.ldf = cdiv(kc, (int64_t)kBK) * kBK + kx; a.nout = nout;
  a.out = out;
  const dim3 grid((unsigned)(cdiv(nout, (int64_t)kBN) * cdiv(M, (int64_t)kBM)));
  gemm_bf16_kernel<<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qlora
