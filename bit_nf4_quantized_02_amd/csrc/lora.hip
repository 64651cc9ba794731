// Low-rank branch kernels: the skinny products around the frozen base.
//
// "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev): the
// three-piece summary (only the low-rank pair learns, the base gets no
// gradient) and the storage / compute / learning diagram (gradients flow back
// into the adapter only). "What is QLoRA?" (qubittool.com), "Key
// Characteristics": adapters are trained in full precision.
//
//   rowdot  out[m, j] = sum_c P[m, c] Q[j, c]     T = X A^T,  U = dY B
//           (bf16 x bf16 on the matrix cores, fp32 accumulate; the
//           contraction is split over workgroups and the pieces are added in
//           a fixed order, so reruns are bit-identical)
//   coldot  G[c, j] = s sum_m P[m, c] Q[m, j]      dA = s U^T X, dB = s dY^T T
//           (fp32 FMAs with an fp32 Q, split over M, fixed-order reduction)
//
// rowdot's finalize step also writes the scaled value s*out as a bf16 hi/lo
// pair, [hi | lo | zero pad] per row: hi = RN_bf16(s*out), lo =
// RN_bf16(s*out - hi). The main GEMMs consume this pair as 2r extra
// contraction columns, so the low-rank term enters their fp32 accumulator
// with about 16 significant bits and Y / dX are rounded to bf16 only once.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kRowTile = 16;   // rows of P per workgroup (one 16x16x32 MFMA row block)
constexpr int kMaxRank = 128;

// Each workgroup: 16 rows, columns [c0, c1) of the contraction, all r outputs.
// 4 waves split [c0, c1) into quarters; lanes read P and Q straight from
// global memory in the MFMA operand layout (8 consecutive bf16 per lane).
template <bool kVec, int kRP>
__global__ __launch_bounds__(256) void rowdot_kernel(const uint16_t* __restrict__ P, int64_t M, int64_t C,
                                                     const uint16_t* __restrict__ Q, int r,
                                                     int64_t cchunk, float* __restrict__ part) {
  __shared__ float red[4][kRowTile][kRP];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t m0 = (int64_t)blockIdx.x * kRowTile;
  const int64_t cs = blockIdx.y;
  const int64_t cbeg = cs * cchunk;
  const int64_t cend = (cbeg + cchunk < C) ? cbeg + cchunk : C;
  const int64_t qlen = cdiv(cend - cbeg, 4 * 32) * 32;  // per-wave length, multiple of 32
  const int64_t w0 = cbeg + wave * qlen;
  const int64_t w1 = (w0 + qlen < cend) ? w0 + qlen : cend;

  const int row = lane & 15;
  const int ko = (lane >> 4) * 8;
  const int64_t m = m0 + row;
  constexpr int kTiles = kRP / 16;
  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 4 chunks of 32 columns per iteration: all loads first, then the MFMAs,
  // so each lane keeps several 16-byte loads in flight
  constexpr int kU = 4;
  for (int64_t c = w0; c < w1; c += 32 * kU) {
    u32x4 a[kU];
    u32x4 b[kU][kTiles];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t cc = c + 32 * u + ko;
      a[u] = u32x4{0u, 0u, 0u, 0u};
      if (m < M) {
        if constexpr (kVec) {
          if (cc < w1) a[u] = *reinterpret_cast<const u32x4*>(P + m * C + cc);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = (cc + i < w1) ? P[m * C + cc + i] : (uint16_t)0;
#pragma unroll
          for (int i = 0; i < 4; ++i) a[u][i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
        }
      }
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const int j = t * 16 + row;
        b[u][t] = u32x4{0u, 0u, 0u, 0u};
        if (j < r) {
          if constexpr (kVec) {
            if (cc < w1) b[u][t] = *reinterpret_cast<const u32x4*>(Q + (int64_t)j * C + cc);
          } else {
            uint16_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = (cc + i < w1) ? Q[(int64_t)j * C + cc + i] : (uint16_t)0;
#pragma unroll
            for (int i = 0; i < 4; ++i) b[u][t][i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                         __builtin_bit_cast(bf16x8, b[u][t]), acc[t], 0, 0, 0);
  }
  // D layout: lane -> column (lane & 15), rows 4 * (lane >> 4) + v
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * (lane >> 4) + v][t * 16 + (lane & 15)] = acc[t][v];
  __syncthreads();
  for (int i = threadIdx.x; i < kRowTile * kRP; i += 256) {
    const int rr = i / kRP, j = i % kRP;
    const int64_t mm = m0 + rr;
    if (mm < M && j < r) {
      const float s = ((red[0][rr][j] + red[1][rr][j]) + red[2][rr][j]) + red[3][rr][j];
      part[(cs * M + mm) * r + j] = s;
    }
  }
}

// Sum the contraction pieces in order; write out (fp32) and the bf16 hi/lo pair.
__global__ __launch_bounds__(256) void rowdot_finalize_kernel(const float* __restrict__ part, int64_t M, int r,
                                                              int64_t nsplit, float* __restrict__ out,
                                                              uint16_t* __restrict__ split, int xcols,
                                                              float scale) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (split == nullptr) {
    if (i >= M * (int64_t)r) return;
    const int64_t m = i / r;
    const int j = (int)(i % r);
    float s = 0.0f;
    for (int64_t p = 0; p < nsplit; ++p) s += part[(p * M + m) * r + j];
    out[i] = s;
    return;
  }
  if (i >= M * (int64_t)xcols) return;
  const int64_t m = i / xcols;
  const int col = (int)(i % xcols);
  uint16_t v = 0;
  if (col < 2 * r) {
    const int j = col < r ? col : col - r;
    float s = 0.0f;
    for (int64_t p = 0; p < nsplit; ++p) s += part[(p * M + m) * r + j];
    if (col < r && out != nullptr) out[m * r + j] = s;
    const float ss = scale * s;
    const uint16_t hi = to_bf16_bits(ss);
    v = (col < r) ? hi : to_bf16_bits(ss - bf16_bits_to_f32(hi));  // exact difference, then RNE
  }
  split[i] = v;
}

// G partial on the matrix cores: Gp[s][j][c] = sum_{m in split s} Q[m, j] P[m, c].
// v_mfma_f32_16x16x32_bf16 with rows = j (rank), columns = c, contraction =
// 32 tokens: every lane gathers 8 consecutive tokens of one column of P (2-byte
// loads; across the wave they cover 16 columns x 32 tokens) and of one column
// of Q, so neither operand is transposed through LDS. Q is fp32: each value is
// split into bf16 hi + lo and both halves are multiplied, so the products
// carry ~16 significant bits of Q. Each wave owns 64 columns; a workgroup
// 256 columns and one token split.
template <int kRP>
__global__ __launch_bounds__(256) void coldot_mfma_kernel(const uint16_t* __restrict__ P, int64_t M, int64_t C,
                                                          const float* __restrict__ Q, int r, int64_t mchunk,
                                                          float* __restrict__ partial) {
#pragma clang fp contract(off)
  constexpr int kJT = kRP / 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t c0 = (int64_t)blockIdx.x * 256 + wave * 64;
  const int64_t s = blockIdx.y;
  const int64_t m0 = s * mchunk;
  const int64_t m1 = (m0 + mchunk < M) ? m0 + mchunk : M;
  const int col = lane & 15;
  const int mo = (lane >> 4) * 8;
  f32x4 acc[kJT][4];
#pragma unroll
  for (int a = 0; a < kJT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t mb = m0; mb < m1; mb += 32) {
    // B operands: 4 column tiles x 8 tokens of P
    bf16x8 pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t c = c0 + t * 16 + col;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t m = mb + mo + e;
        h[e] = (c < C && m < m1) ? (uint32_t)P[m * C + c] : 0u;
      }
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = h[2 * e] | (h[2 * e + 1] << 16);
      pb[t] = __builtin_bit_cast(bf16x8, v);
    }
    // A operands: rank tiles x 8 tokens of Q, split into hi and lo
#pragma unroll
    for (int a = 0; a < kJT; ++a) {
      const int j = a * 16 + col;
      u32x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t hh[2], ll[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int64_t m = mb + mo + 2 * e + f;
          const float q = (j < r && m < m1) ? Q[m * r + j] : 0.0f;
          const uint16_t qh = to_bf16_bits(q);
          hh[f] = qh;
          ll[f] = to_bf16_bits(q - bf16_bits_to_f32(qh));
        }
        hi[e] = hh[0] | (hh[1] << 16);
        lo[e] = ll[0] | (ll[1] << 16);
      }
      const bf16x8 ah = __builtin_bit_cast(bf16x8, hi), al = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, pb[t], acc[a][t], 0, 0, 0);
        acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, pb[t], acc[a][t], 0, 0, 0);
      }
    }
  }
  // D[j][c]: lane -> c = col, j = 4 (lane >> 4) + v
#pragma unroll
  for (int a = 0; a < kJT; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t c = c0 + t * 16 + col;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = a * 16 + 4 * (lane >> 4) + v;
        if (c < C && j < r) partial[(s * r + j) * C + c] = acc[a][t][v];
      }
    }
}

__global__ __launch_bounds__(256) void coldot_reduce_kernel(const float* __restrict__ partial, int64_t C, int r,
                                                            int64_t nsplit, float scale, float* __restrict__ G,
                                                            int64_t g_sc, int64_t g_sj, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= C * r) return;
  const int64_t j = i / C, c = i % C;
  float s = 0.0f;
  for (int64_t p = 0; p < nsplit; ++p) s += partial[(p * r + j) * C + c];
  float* g = G + c * g_sc + j * g_sj;
  const float v = scale * s;
  *g = accumulate ? (*g + v) : v;
}

}  // namespace

static int rowdot_splits(int64_t M, int64_t C) {
  const int64_t tiles = cdiv(M, kRowTile);
  int64_t s = cdiv(512, tiles);
  const int64_t maxs = cdiv(C, 4 * 128);  // keep >= 128 columns per wave
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

size_t rowdot_ws_bytes(int64_t M, int64_t C, int r) {
  return align256((size_t)rowdot_splits(M, C) * (size_t)M * (size_t)r * 4);
}

hipError_t launch_rowdot_impl(const uint16_t* P, int64_t M, int64_t C, const uint16_t* Q, int r, float* out,
                              uint16_t* split, float scale, float* part, hipStream_t stream) {
  const int ns = rowdot_splits(M, C);
  const int64_t cchunk = cdiv(cdiv(C, ns), 32) * 32;
  const dim3 grid((unsigned)cdiv(M, kRowTile), (unsigned)ns);
  const bool vec = (C % 8) == 0;
#define QLORA_ROWDOT(RP)                                                                          \
  if (vec) rowdot_kernel<true, RP><<<grid, 256, 0, stream>>>(P, M, C, Q, r, cchunk, part);       \
  else rowdot_kernel<false, RP><<<grid, 256, 0, stream>>>(P, M, C, Q, r, cchunk, part);
  if (r <= 16) { QLORA_ROWDOT(16) }
  else if (r <= 32) { QLORA_ROWDOT(32) }
  else if (r <= 64) { QLORA_ROWDOT(64) }
  else { QLORA_ROWDOT(128) }
#undef QLORA_ROWDOT
  const int xcols = lora_extra_cols(r);
  const int64_t total = split ? M * xcols : M * r;
  rowdot_finalize_kernel<<<(unsigned)cdiv(total, 256), 256, 0, stream>>>(part, M, r, ns, out, split, xcols, scale);
  return hipGetLastError();
}

int coldot_splits(int64_t M) {
  int64_t s = M / 256;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  return (int)s;
}

size_t coldot_ws_bytes(int64_t M, int64_t C, int r) {
  return align256((size_t)coldot_splits(M) * (size_t)C * (size_t)r * 4);
}

hipError_t launch_coldot(const uint16_t* P, int64_t M, int64_t C, const float* Q, int r, float scale, float* G,
                         int64_t g_sc, int64_t g_sj, int accumulate, float* partial, hipStream_t stream) {
  const int ns = coldot_splits(M);
  const int64_t mchunk = cdiv(cdiv(M, ns), 32) * 32;
  const dim3 grid((unsigned)cdiv(C, 256), (unsigned)ns);
  if (r <= 16) coldot_mfma_kernel<16><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);
  else if (r <= 32) coldot_mfma_kernel<32><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);
  else if (r <= 64) coldot_mfma_kernel<64><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);
  else coldot_mfma_kernel<128><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);
  coldot_reduce_kernel<<<(unsigned)cdiv(C * r, 256), 256, 0, stream>>>(partial, C, r, ns, scale, G, g_sc, g_sj,
                                                                      accumulate);
  return hipGetLastError();
}

// B [n, r] -> B^T [r, n], so dY B is a rowdot with a contiguous second operand.
namespace {
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ B, int64_t n, int r,
                                                        uint16_t* __restrict__ BT) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * r) return;
  const int64_t j = i / n, c = i % n;
  BT[i] = B[c * r + j];
  (void)j;
}
}  // namespace

hipError_t launch_transpose(const uint16_t* B, int64_t n, int r, uint16_t* BT, hipStream_t stream) {
  transpose_kernel<<<(unsigned)cdiv(n * r, 256), 256, 0, stream>>>(B, n, r, BT);
  return hipGetLastError();
}

}  // namespace qlora
