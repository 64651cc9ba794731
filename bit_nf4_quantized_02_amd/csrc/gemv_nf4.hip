// Dequant-GEMV for small token counts (M <= 16): bandwidth-bound path.
//
// With a handful of tokens every packed weight byte is used for at most 16
// multiply-adds, so the layer costs one pass over the 4-bit codes
// ("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// "Batched 4-bit matmuls"; "QLoRA vs LoRA: ..." (instagit.com), "Training
// Speed and Computational Efficiency": lower memory traffic).
//
//   Y = RN_bf16( X W'^T + s T B^T ),   T = X A^T precomputed (fp32)
//
// Each workgroup owns NT output rows (n) and the whole contraction; its kW
// waves split the contraction into kW parts. A wave walks its quarter in
// 256-wide chunks, keeping the loads of the next chunk in flight while it
// works on one: every lane loads 32 contiguous bytes of codes (one whole
// 64-block of one row, one scale), expands them to bf16 in registers
// through an LDS table indexed by whole code bytes (one read yields the
// levels of two weights; the products are those of the 16-entry codebook)
// and feeds them straight to
// v_mfma_f32_16x16x32_bf16 as the B operand; X (padded to 16 rows with zeros)
// is the A operand. The contraction order inside a chunk is permuted the same
// way on both operands (lane group g takes columns 64 g .. 64 g + 63), which
// leaves the sum unchanged and makes each lane's code load contiguous. A
// first small kernel writes X in exactly that operand order (per 256-column
// chunk, per MFMA, per lane: 16 bytes), so each activation load instruction
// reads 1 KB in one run; read in place, the 16 token rows and 4 column groups
// of one instruction fall in 64 different cache lines.
// Partial sums of the waves are added in a fixed order through LDS; the
// low-rank term T B^T is formed with fp32 MFMAs (one 16-row tile per wave,
// T and B exact in fp32) and added in fp32, and Y is rounded to bf16 once.
#include "common.h"
#include "kernels.h"

#ifndef QLORA_GEMV_XP_MIN_M
#define QLORA_GEMV_XP_MIN_M 5
#endif

namespace qlora {

namespace {

// Xp[q][s][lane] = X[lane % 16][256 q + 64 (lane / 16) + 8 s .. +7] (16 bytes),
// zero for token rows >= M or columns >= K.
__global__ __launch_bounds__(256) void gemv_xperm_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                         u32x4* __restrict__ Xp, int64_t entries) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= entries) return;
  const int lane = (int)(e & 63), s = (int)((e >> 6) & 7);
  const int64_t q = e >> 9;
  const int64_t m = lane & 15, c = 256 * q + 64 * (lane >> 4) + 8 * s;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M && c < K) v = *reinterpret_cast<const u32x4*>(X + m * K + c);
  Xp[e] = v;
}

// kXp: activations from the operand-ordered copy Xp (else read in place from X).
// kF16: fp16 activations, weights, B and output (the compute-type ablation).
template <int NT, int kW, bool kLora, bool kXp, bool kF16>
__global__ __launch_bounds__(64 * kW) void gemv_nf4_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ code8,
                                                       const float* __restrict__ s2,
                                                       const float* __restrict__ mean_p,
                                                       const float* __restrict__ codebook, bool s2_bf16,
                                                       int64_t N, int64_t K, const uint16_t* __restrict__ X,
                                                       const u32x4* __restrict__ Xp, int64_t M,
                                                       const float* __restrict__ T,
                                                       const uint16_t* __restrict__ B, int r, float scale,
                                                       uint16_t* __restrict__ Y) {
  constexpr int kTiles = NT / 16;
  __shared__ float2 lut2[256];
  __shared__ float red[kW][kTiles][16][16];
  __shared__ float lred[kLora ? kTiles : 1][16][16];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  for (int i = t; i < 256; i += 64 * kW)
    lut2[i] = float2{codebook[i & 15], codebook[i >> 4]};  // levels of the two codes in byte i
  __syncthreads();
  const float mean = weight_mean(code8, mean_p);
  const int64_t n0 = (int64_t)blockIdx.x * NT;
  constexpr int kChunk = 256;                            // columns per wave iteration
  const int64_t kq = cdiv(cdiv(K, kW), kChunk) * kChunk;  // per-wave share
  const int64_t kb = wave * kq;
  const int64_t ke = (kb + kq < K) ? kb + kq : K;        // multiple of 64
  const int grp = lane >> 4;   // 0..3: which 64-block of a 256-column chunk
  const int col = lane & 15;   // A: token row m; B: weight row within a tile
  const int64_t kblocks = K / kBlock;
  const int64_t nq = cdiv(K, (int64_t)kChunk);  // chunks of the operand-ordered activations
  const bool xtok = col < M;                     // lanes of token rows past M load nothing
  const uint16_t* xrow = X + (int64_t)(col < M ? col : M - 1) * K;

  f32x4 acc[kTiles];
#pragma unroll
  for (int i = 0; i < kTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane row bases, computed once. Every load below reads a clamped,
  // in-range address; out-of-range rows / blocks / tokens are then replaced
  // by code 7 (level 0) or zero activations with selects, so the loop body is
  // one basic block and the next chunk's loads stay in flight while a chunk
  // is expanded and multiplied. Lane group g takes the whole 64-block g of
  // the chunk (32 code bytes, one scale): a row's 128-byte code line is read
  // by one wave in one iteration. The 64 columns are fed to 8 MFMAs, 8 per
  // MFMA; the activations follow the same column permutation, which leaves
  // the sum unchanged.
  const uint8_t* crow[kTiles];
  int64_t bbase[kTiles];
  bool rowok[kTiles];
#pragma unroll
  for (int i = 0; i < kTiles; ++i) {
    const int64_t n = n0 + i * 16 + col;
    const int64_t nc = n < N ? n : N - 1;
    rowok[i] = n < N;
    crow[i] = codes + nc * (K / 2);
    bbase[i] = nc * kblocks;
  }

  struct Stage {
    u32x4 cw[kTiles][2];
    uint32_t c8[kTiles];
    float s2v[kTiles];
    u32x4 xa[8];
    bool kin;
  };
  auto load = [&](int64_t k0, Stage& st) {
    const int64_t k = k0 + 64 * grp;
    st.kin = k < ke;
    const int64_t kc = st.kin ? k : ke - 64;  // a valid block of this wave's range
    // this chunk's operands, in order (a prefetch past the last chunk reads
    // the last one again: every group then has kin false and code 7)
    if constexpr (kXp) {
      const int64_t q = k0 / kChunk < nq ? k0 / kChunk : nq - 1;
      const u32x4* xq = Xp + q * 512 + lane;
#pragma unroll
      for (int s = 0; s < 8; ++s) st.xa[s] = xtok ? xq[64 * s] : u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) st.xa[s] = *reinterpret_cast<const u32x4*>(xrow + kc + 8 * s);
    }
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
      st.cw[i][0] = *reinterpret_cast<const u32x4*>(crow[i] + kc / 2);
      st.cw[i][1] = *reinterpret_cast<const u32x4*>(crow[i] + kc / 2 + 16);
      const int64_t blk = bbase[i] + kc / kBlock;
      scale_fields(code8, s2, s2_bf16, blk, st.c8[i], st.s2v[i]);
    }
  };
  auto compute = [&](const Stage& st) {
    const bool xuse = st.kin && xtok;
    bf16x8 xa[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = st.xa[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = xuse ? v[e] : 0u;
      xa[s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
      const bool use = st.kin && rowok[i];
      const float cp = decode_block_scale(st.c8[i], st.s2v[i], mean);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t word = use ? st.cw[i][s >> 2][s & 3] : 0x77777777u;  // code 7: level 0
        const u32x4 bw = dequant8_pairs<kF16>(word, lut2, cp);
        acc[i] = mfma16<kF16>(xa[s], __builtin_bit_cast(bf16x8, bw), acc[i]);
      }
    }
  };
  if (kb < ke) {  // (a wave may have no columns when K is tiny)
    Stage st0, st1;
    load(kb, st0);
    for (int64_t k0 = kb; k0 < ke; k0 += 2 * kChunk) {
      // the scheduling barriers keep each chunk's loads issued ahead of the
      // work on the previous chunk (the compiler would otherwise sink them to
      // their first use)
      load(k0 + kChunk, st1);
      __builtin_amdgcn_sched_barrier(0);
      compute(st0);
      if (k0 + kChunk >= ke) break;
      load(k0 + 2 * kChunk, st0);
      __builtin_amdgcn_sched_barrier(0);
      compute(st1);
    }
  }
  // D[m][n]: lane -> n = lane & 15, m = 4 (lane >> 4) + v
#pragma unroll
  for (int i = 0; i < kTiles; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][i][4 * (lane >> 4) + v][lane & 15] = acc[i][v];
  if constexpr (kLora) {
    // L[m][n] = sum_j T[m][j] B[n][j] for tile i on wave i (mod kW), 4 ranks
    // per v_mfma_f32_16x16x4_f32: A = T (lane: token lane % 16, rank lane / 16),
    // B = B^T (lane: weight row lane % 16, same rank); rows past M or N and
    // ranks past r read as zero
    for (int i = wave; i < kTiles; i += kW) {
      f32x4 l = f32x4{0.f, 0.f, 0.f, 0.f};
      const int m = lane & 15;
      const int64_t n = n0 + i * 16 + (lane & 15);
      for (int j0 = 0; j0 < r; j0 += 4) {
        const int j = j0 + (lane >> 4);
        const float a = (m < M && j < r) ? T[m * r + j] : 0.0f;
        const float b = (n < N && j < r) ? from16<kF16>(B[n * r + j]) : 0.0f;
        l = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, l, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) lred[i][4 * (lane >> 4) + v][lane & 15] = l[v];
    }
  }
  __syncthreads();
  for (int o = t; o < 16 * NT; o += 64 * kW) {
    const int m = o / NT, nl = o % NT;
    const int64_t n = n0 + nl;
    if (m >= M || n >= N) continue;
    const int i = nl >> 4, nc = nl & 15;
    float y = red[0][i][m][nc];
#pragma unroll
    for (int w2 = 1; w2 < kW; ++w2) y += red[w2][i][m][nc];  // in wave order
    if constexpr (kLora) y = fmaf(scale, lred[i][m][nc], y);
    Y[m * N + n] = to16<kF16>(y);
  }
}

}  // namespace

size_t gemv_ws_bytes(int64_t k) { return align256((size_t)cdiv(k, 256) * 512 * 16); }

// Token counts from which the activations are first rewritten in operand
// order: below it the few distinct rows an activation load touches cost less
// than the extra pass (measured on the 70B-class shapes). Weights with fewer
// than kXpMinN rows never take it: their workgroups re-read X only a few
// times, and the extra launch costs more (a 1024 x 1024 layer at M = 16).
constexpr int64_t kXpMinM = QLORA_GEMV_XP_MIN_M;
constexpr int64_t kXpMinN = 4096;

hipError_t launch_gemv(const Nf4View& w, const uint16_t* X, int64_t M, const float* T, const uint16_t* B, int r,
                       float scale, uint16_t* Y, void* ws, hipStream_t stream, bool f16) {
  u32x4* Xp = static_cast<u32x4*>(ws);
  const bool xp = M >= kXpMinM && w.n >= kXpMinN;
  if (xp) {
    const int64_t entries = cdiv(w.k, (int64_t)256) * 512;
    gemv_xperm_kernel<<<(unsigned)cdiv(entries, (int64_t)256), 256, 0, stream>>>(X, M, w.k, Xp, entries);
  }
  // Rows and waves per workgroup, measured on the 70B-class shapes: 64 rows
  // and 4 waves for 28672 rows (448 workgroups), 32 rows and 8 waves for
  // 8192 rows (256 workgroups, each wave an eighth of the 28672-long
  // contraction), 16 rows and 4 waves below.
  const bool lora = r > 0;
#define QLORA_GEMV3(NT, W, L, XP, H)                                                                           \
  gemv_nf4_kernel<NT, W, L, XP, H><<<dim3((unsigned)cdiv(w.n, NT)), 64 * W, 0, stream>>>(                      \
      w.codes, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16, w.n, w.k, X, Xp, M, T, B, r, scale, Y)
#define QLORA_GEMV2(NT, W, L, XP) \
  if (f16) QLORA_GEMV3(NT, W, L, XP, true); else QLORA_GEMV3(NT, W, L, XP, false);
#define QLORA_GEMV(NT, W)                                                   \
  {                                                                         \
    if (lora) { if (xp) { QLORA_GEMV2(NT, W, true, true) } else { QLORA_GEMV2(NT, W, true, false) } } \
    else { if (xp) { QLORA_GEMV2(NT, W, false, true) } else { QLORA_GEMV2(NT, W, false, false) } }    \
  }
  if (w.n / 64 >= 448) QLORA_GEMV(64, 4)
  else if (w.n / 32 >= 256) QLORA_GEMV(32, 8)
  else QLORA_GEMV(16, 4)
#undef QLORA_GEMV
#undef QLORA_GEMV2
#undef QLORA_GEMV3
  return hipGetLastError();
}

}  // namespace qlora
