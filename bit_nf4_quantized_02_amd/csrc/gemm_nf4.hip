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
// Tile: BM x BN outputs per 256-thread workgroup, 64-deep contraction steps
// (one NF4 block per weight row and step); 4 waves in a 2 x 2 grid, each a
// (BM/2) x (BN/2) sub-tile of v_mfma_f32_32x32x16_bf16. Per step:
//   * the activation tile [BM x 64] bf16 is copied global -> registers -> LDS;
//   * the weight tile is read as packed nibbles (0.5 B/weight, 16-B or 4-B
//     loads, coalesced along rows), each block's scale c' is rebuilt from its
//     code8 byte, s2 and the mean, every nibble is looked up in the 16-entry
//     codebook held in LDS, multiplied by c' in fp32 and rounded to bf16, and
//     the bf16 tile is written to LDS: row-major [n][k] for the forward,
//     transposed [k][n] for dX (the contraction runs over n there);
//   * MFMA operands are read from LDS with 16-B reads; tiles use an XOR swizzle
//     of the 16-B chunk index with the row, so the 32 rows a fragment read
//     touches fall in distinct banks.
// The next step's global loads are issued before the current step's MFMAs.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

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
  int64_t wn, wk;
  // low-rank second factor: B [wn, r] (forward) or A [r, wk] (dX)
  const uint16_t* lr;
  int r;
  // output [M, nout] bf16
  uint16_t* out;
  int64_t nout;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int BM>
struct ActStage {
  static constexpr int kChunks = BM * 8 / kThreads;  // 16-B chunks per thread
  u32x4 v[kChunks];
};

// Load the activation tile for contraction columns [c0, c0 + 64).
template <int BM, bool kVec>
__device__ __forceinline__ void load_act(const GemmArgs& a, int64_t m0, int step, int nk_main,
                                         ActStage<BM>& st) {
  const int t = threadIdx.x;
  const bool extra = step >= nk_main;
  const uint16_t* src = extra ? a.act_x : a.act;
  const int64_t ld = extra ? (int64_t)a.kx : a.lda;
  const int64_t cols = extra ? (int64_t)a.kx : a.kc;
  const int64_t c0 = (int64_t)(extra ? step - nk_main : step) * kBK;
#pragma unroll
  for (int i = 0; i < ActStage<BM>::kChunks; ++i) {
    const int q = t + i * kThreads;
    const int row = q >> 3, ch = q & 7;
    const int64_t m = m0 + row;
    const int64_t c = c0 + ch * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < a.M) {
      const uint16_t* p = src + m * ld + c;
      if (extra || kVec) {
        if (c < cols) v = *reinterpret_cast<const u32x4*>(p);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = (c + j < cols) ? p[j] : (uint16_t)0;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
      }
    }
    st.v[i] = v;
  }
}

template <int BM>
__device__ __forceinline__ void store_act(char* As, const ActStage<BM>& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < ActStage<BM>::kChunks; ++i) {
    const int q = t + i * kThreads;
    *reinterpret_cast<u32x4*>(As + swz(q >> 3, q & 7)) = st.v[i];
  }
}

// ---------------------------------------------------------------- forward B
// Weight tile for the forward: BN rows (n) x 64 (k). BN = 128: thread t takes
// row t/2, half t%2 (32 weights = 16 B of codes, one block scale). In a
// low-rank step the same thread holds 32 bf16 of [B | B] instead.
struct FwdWStage {
  u32x4 q[4];  // q[0]: packed codes (NF4 step); q[0..3]: 32 bf16 (low-rank step)
  float cp;
};

template <int BN>
__device__ __forceinline__ void load_w_fwd(const GemmArgs& a, int64_t n0, int step, int nk_main,
                                           FwdWStage& st) {
  static_assert(BN * 2 == kThreads, "forward weight mapping needs BN = 128");
  const int t = threadIdx.x;
  const int row = t >> 1, half = t & 1;
  const int64_t n = n0 + row;
  if (step < nk_main) {
    st.q[0] = u32x4{0u, 0u, 0u, 0u};
    st.cp = 0.0f;
    if (n < a.wn) {
      st.q[0] = *reinterpret_cast<const u32x4*>(a.codes + n * (a.wk / 2) + (int64_t)step * 32 + half * 16);
      st.cp = block_scale(a.code8, a.s2, a.mean[0], n * (a.wk / kBlock) + step);
    }
  } else {
    const int j0 = (step - nk_main) * kBK + half * 32;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = j0 + w * 8 + p * 2 + e;
          h[e] = (n < a.wn && j < 2 * a.r) ? (uint32_t)a.lr[n * a.r + (j % a.r)] : 0u;
        }
        st.q[w][p] = h[0] | (h[1] << 16);
      }
  }
}

template <int BN>
__device__ __forceinline__ void store_w_fwd(char* Bs, const float* lut, int step, int nk_main,
                                            const FwdWStage& st) {
  const int t = threadIdx.x;
  const int row = t >> 1, half = t & 1;
  if (step < nk_main) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      *reinterpret_cast<u32x4*>(Bs + swz(row, half * 4 + w)) = dequant8(st.q[0][w], lut, st.cp);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4*>(Bs + swz(row, half * 4 + w)) = st.q[w];
  }
}

// ---------------------------------------------------------------- dX B
// Weight tile for dX: contraction rows n (64) x output columns k (BN = 128),
// stored in LDS transposed as [k][n]. Thread t takes the 4 rows
// n = 4 (t/16) .. +3 and the 8 columns k = 8 (t%16) .. +7 (4 bytes of codes
// per row, one block scale per row); each of its 8 columns becomes 4
// consecutive n values, one 8-byte LDS write. In a low-rank step the rows are
// rows of [A ; A] (8 bf16 per row).
struct DxWStage {
  u32x4 q[4];  // q[i][0]: code word of row i (NF4 step); q[i]: 8 bf16 of row i (low-rank)
  float cp[4];
};

template <int BN>
__device__ __forceinline__ void load_w_dx(const GemmArgs& a, int64_t k0, int step, int nk_main,
                                          DxWStage& st) {
  static_assert(BN == 128, "dX weight mapping needs BN = 128");
  const int t = threadIdx.x;
  const int g = t >> 4, kcol = t & 15;
  const int64_t k = k0 + kcol * 8;
  if (step < nk_main) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = (int64_t)step * kBK + 4 * g + i;
      st.q[i][0] = 0u;
      st.cp[i] = 0.0f;
      if (n < a.wn && k < a.wk) {
        st.q[i][0] = *reinterpret_cast<const uint32_t*>(a.codes + n * (a.wk / 2) + k / 2);
        st.cp[i] = block_scale(a.code8, a.s2, a.mean[0], n * (a.wk / kBlock) + k / kBlock);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = (step - nk_main) * kBK + 4 * g + i;
      st.q[i] = u32x4{0u, 0u, 0u, 0u};
      if (j < 2 * a.r && k < a.wk)
        st.q[i] = *reinterpret_cast<const u32x4*>(a.lr + (int64_t)(j % a.r) * a.wk + k);
    }
  }
}

template <int BN>
__device__ __forceinline__ void store_w_dx(char* Bs, const float* lut, int step, int nk_main,
                                           const DxWStage& st) {
  const int t = threadIdx.x;
  const int g = t >> 4, kcol = t & 15;
  const int nrow = 4 * g;  // first of the 4 contraction rows, in [0, 64)
  if (step < nk_main) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = nf4_scaled(lut[(st.q[i][0] >> (4 * e)) & 0xF], st.cp[i]);
      const int krow = kcol * 8 + e;
      u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(Bs + swz(krow, nrow >> 3) + (nrow & 7) * 2) = pk;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (st.q[i][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
      const int krow = kcol * 8 + e;
      u32x2 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *reinterpret_cast<u32x2*>(Bs + swz(krow, nrow >> 3) + (nrow & 7) * 2) = pk;
    }
  }
}

// ---------------------------------------------------------------- kernel
template <int BM, int BN, bool kDX, bool kVec>
__global__ __launch_bounds__(kThreads) void gemm_nf4_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ __attribute__((aligned(16))) char As[BM * 128];
  __shared__ __attribute__((aligned(16))) char Bs[BN * 128];
  __shared__ float lut[16];

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int64_t n0 = (int64_t)blockIdx.x * BN;  // output columns
  const int64_t m0 = (int64_t)blockIdx.y * BM;  // output rows
  if (t < 16) lut[t] = a.codebook[t];

  const int nk_main = (int)cdiv(a.kc, kBK);
  const int nk = nk_main + a.kx / kBK;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  ActStage<BM> ast;
  FwdWStage fst;
  DxWStage dst;
  load_act<BM, kVec>(a, m0, 0, nk_main, ast);
  if constexpr (kDX) load_w_dx<BN>(a, n0, 0, nk_main, dst);
  else load_w_fwd<BN>(a, n0, 0, nk_main, fst);
  __syncthreads();  // lut

  for (int step = 0; step < nk; ++step) {
    store_act<BM>(As, ast);
    if constexpr (kDX) store_w_dx<BN>(Bs, lut, step, nk_main, dst);
    else store_w_fwd<BN>(Bs, lut, step, nk_main, fst);
    __syncthreads();
    if (step + 1 < nk) {
      load_act<BM, kVec>(a, m0, step + 1, nk_main, ast);
      if constexpr (kDX) load_w_dx<BN>(a, n0, step + 1, nk_main, dst);
      else load_w_fwd<BN>(a, n0, step + 1, nk_main, fst);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + swz(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn0 + j * 32 + (lane & 31), ch));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

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

constexpr int kBM = 256, kBN = 128;

}  // namespace

hipError_t launch_gemm_fwd(const Nf4View& w, const uint16_t* X, int64_t M, const uint16_t* TS, const uint16_t* B,
                           int r, uint16_t* Y, hipStream_t stream) {
  GemmArgs a{};
  a.act = X; a.lda = w.k; a.M = M; a.kc = w.k;
  a.act_x = TS; a.kx = lora_extra_cols(r);
  a.codes = w.codes; a.code8 = w.code8; a.s2 = w.s2; a.mean = w.mean; a.codebook = w.codebook;
  a.wn = w.n; a.wk = w.k;
  a.lr = B; a.r = r;
  a.out = Y; a.nout = w.n;
  const dim3 grid((unsigned)cdiv(w.n, kBN), (unsigned)cdiv(M, kBM));
  gemm_nf4_kernel<kBM, kBN, false, true><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const Nf4View& w, const uint16_t* dY, int64_t M, const uint16_t* US, const uint16_t* A,
                          int r, uint16_t* dX, hipStream_t stream) {
  GemmArgs a{};
  a.act = dY; a.lda = w.n; a.M = M; a.kc = w.n;
  a.act_x = US; a.kx = lora_extra_cols(r);
  a.codes = w.codes; a.code8 = w.code8; a.s2 = w.s2; a.mean = w.mean; a.codebook = w.codebook;
  a.wn = w.n; a.wk = w.k;
  a.lr = A; a.r = r;
  a.out = dX; a.nout = w.k;
  const dim3 grid((unsigned)cdiv(w.k, kBN), (unsigned)cdiv(M, kBM));
  if (w.n % 8 == 0)
    gemm_nf4_kernel<kBM, kBN, true, true><<<grid, kThreads, 0, stream>>>(a);
  else
    gemm_nf4_kernel<kBM, kBN, true, false><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qlora
