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

constexpr int kMaxRank = 128;

// Each workgroup: RT x 16 rows, columns [c0, c1) of the contraction, all r
// outputs. Wave w takes row tile w % RT and part w / RT of the column range
// (4 / RT parts); lanes read P and Q straight from global memory in the MFMA
// operand layout (8 consecutive bf16 per lane), 8 column chunks per
// iteration so each lane keeps eight 16-byte loads in flight. With RT = 4 the
// four waves share one slice of Q (read once per 64 rows instead of per 16).
template <bool kVec, int kRP, int RT>
__global__ __launch_bounds__(256) void rowdot_kernel(const uint16_t* __restrict__ P, int64_t M, int64_t C,
                                                     const uint16_t* __restrict__ Q, int r,
                                                     int64_t cchunk, float* __restrict__ part) {
  constexpr int kParts = 4 / RT;
  __shared__ float red[4][16][kRP];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int rt = wave % RT, cpart = wave / RT;
  const int64_t m0 = (int64_t)blockIdx.x * (16 * RT) + 16 * rt;
  const int64_t cs = blockIdx.y;
  const int64_t cbeg = cs * cchunk;
  const int64_t cend = (cbeg + cchunk < C) ? cbeg + cchunk : C;
  const int64_t qlen = cdiv(cend - cbeg, kParts * 32) * 32;  // per-wave length, multiple of 32
  const int64_t w0 = cbeg + cpart * qlen;
  const int64_t w1 = (w0 + qlen < cend) ? w0 + qlen : cend;

  const int row = lane & 15;
  const int ko = (lane >> 4) * 8;
  const int64_t m = m0 + row;
  constexpr int kTiles = kRP / 16;
  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kU = kTiles >= 4 ? 2 : 8 / kTiles;
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
  const int64_t mw = (int64_t)blockIdx.x * (16 * RT);
  for (int i = threadIdx.x; i < 16 * RT * kRP; i += 256) {
    const int rr = i / kRP, j = i % kRP;
    const int64_t mm = mw + rr;
    if (mm < M && j < r) {
      const int rtile = rr / 16, rin = rr % 16;
      float sum = red[rtile][rin][j];
#pragma unroll
      for (int pp = 1; pp < kParts; ++pp) sum += red[rtile + pp * RT][rin][j];  // parts in order
      part[(cs * M + mm) * r + j] = sum;
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
// The contraction runs over the tokens m, which are the slow index of both
// operands, so each 32-token step is staged in LDS in its stored orientation
// -- P as [32][256 columns] bf16 (coalesced 16-byte loads), Q as [32][r] bf16
// hi and lo halves of the fp32 value -- and both MFMA operands are gathered
// with the transposing read ds_read_b64_tr_b16 (8 consecutive tokens of one
// column per lane). v_mfma_f32_16x16x32_bf16: rows = j, columns = c; the hi
// and lo halves of Q are multiplied separately, so the products carry ~16
// significant bits of Q. Each wave owns 64 columns; a workgroup 256 columns
// and one token split. The next step's P is loaded into registers while the
// current step's MFMAs run.
constexpr int kPPitch = 512 + 32;  // bytes per staged P row (256 bf16 + pad)

template <int kRP>
struct ColdotSmem {
  static constexpr int kQPitch = kRP * 2 + (kRP >= 32 ? 32 : 0);
  char p[32 * kPPitch];
  char qh[32 * kQPitch];
  char ql[32 * kQPitch];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Operand of v_mfma_f32_16x16x32_bf16 from a [token][col] bf16 tile: lane
// gets column c0 + lane % 16, tokens 8 (lane / 16) .. +7. Inside each 16-lane
// group lane i addresses token base + i / 4, columns 4 (i % 4) .. +3 and
// receives its own column of the 4 tokens.
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int pitch, int c0, int lane) {
  const int i = lane & 15;
  const char* p = tile + (8 * (lane >> 4) + (i >> 2)) * pitch + (c0 + 4 * (i & 3)) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 4 * pitch));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int kRP, bool kVec>
__global__ __launch_bounds__(256) void coldot_mfma_kernel(const uint16_t* __restrict__ P, int64_t M, int64_t C,
                                                          const float* __restrict__ Q, int r, int64_t mchunk,
                                                          float* __restrict__ partial) {
#pragma clang fp contract(off)
  constexpr int kJT = kRP / 16;
  using Smem = ColdotSmem<kRP>;
  constexpr int kQP = Smem::kQPitch;
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int64_t cw = (int64_t)blockIdx.x * 256;
  const int64_t s = blockIdx.y;
  const int64_t m0 = s * mchunk;
  const int64_t m1 = (m0 + mchunk < M) ? m0 + mchunk : M;
  f32x4 acc[kJT][4];
#pragma unroll
  for (int a = 0; a < kJT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // P tile: 32 rows x 32 chunks of 16 B; thread t owns chunk t % 32 of rows
  // t / 32 + 8 i (i = 0..3). Out-of-range rows / columns load zeros.
  auto load_p = [&](int64_t mb, u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb + (t >> 5) + 8 * i;
      const int64_t c = cw + (t & 31) * 8;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (m < m1) {
        if constexpr (kVec) {
          if (c < C) v[i] = *reinterpret_cast<const u32x4*>(P + m * C + c);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = (c + q < C) ? (uint32_t)P[m * C + c + q] : 0u;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[i][q] = e[2 * q] | (e[2 * q + 1] << 16);
        }
      }
    }
  };
  u32x4 pv[4];
  load_p(m0, pv);
  for (int64_t mb = m0; mb < m1; mb += 32) {
    // stage this step: P from registers, Q converted to bf16 hi / lo
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(sm.p + ((t >> 5) + 8 * i) * kPPitch + (t & 31) * 16) = pv[i];
    for (int e = t; e < 32 * kRP; e += 256) {
      const int mm = e / kRP, j = e % kRP;
      const int64_t m = mb + mm;
      const float q = (j < r && m < m1) ? Q[m * r + j] : 0.0f;
      const uint16_t qh = to_bf16_bits(q);
      const uint16_t ql = to_bf16_bits(q - bf16_bits_to_f32(qh));
      *reinterpret_cast<uint16_t*>(sm.qh + mm * kQP + j * 2) = qh;
      *reinterpret_cast<uint16_t*>(sm.ql + mm * kQP + j * 2) = ql;
    }
    __syncthreads();
    if (mb + 32 < m1) load_p(mb + 32, pv);  // in flight during the MFMAs
    bf16x8 pb[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) pb[ct] = tr_operand(sm.p, kPPitch, wave * 64 + ct * 16, lane);
#pragma unroll
    for (int a = 0; a < kJT; ++a) {
      const bf16x8 ah = tr_operand(sm.qh, kQP, a * 16, lane);
      const bf16x8 al = tr_operand(sm.ql, kQP, a * 16, lane);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, pb[ct], acc[a][ct], 0, 0, 0);
        acc[a][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, pb[ct], acc[a][ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // D[j][c]: lane -> c = lane % 16, j = 4 (lane / 16) + v
#pragma unroll
  for (int a = 0; a < kJT; ++a)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t c = cw + wave * 64 + ct * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = a * 16 + 4 * (lane >> 4) + v;
        if (c < C && j < r) partial[(s * r + j) * C + c] = acc[a][ct][v];
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

static int rowdot_rt(int64_t M) { return M >= 256 ? 4 : 1; }

static int rowdot_splits(int64_t M, int64_t C) {
  const int64_t tiles = cdiv(M, 16 * rowdot_rt(M));
  int64_t s = cdiv(512, tiles);
  const int64_t maxs = cdiv(C, 256);  // keep >= 256 columns per split
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
  const int rt = rowdot_rt(M);
  const int64_t cchunk = cdiv(cdiv(C, ns), 32) * 32;
  const dim3 grid((unsigned)cdiv(M, 16 * rt), (unsigned)ns);
  const bool vec = (C % 8) == 0;
#define QLORA_ROWDOT2(RP, RT)                                                                          \
  if (vec) rowdot_kernel<true, RP, RT><<<grid, 256, 0, stream>>>(P, M, C, Q, r, cchunk, part);        \
  else rowdot_kernel<false, RP, RT><<<grid, 256, 0, stream>>>(P, M, C, Q, r, cchunk, part);
#define QLORA_ROWDOT(RP) \
  if (rt == 4) { QLORA_ROWDOT2(RP, 4) } else { QLORA_ROWDOT2(RP, 1) }
  if (r <= 16) { QLORA_ROWDOT(16) }
  else if (r <= 32) { QLORA_ROWDOT(32) }
  else if (r <= 64) { QLORA_ROWDOT(64) }
  else { QLORA_ROWDOT(128) }
#undef QLORA_ROWDOT
#undef QLORA_ROWDOT2
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
  const bool vec = C % 8 == 0;
#define QLORA_COLDOT(RP)                                                                             \
  if (vec) coldot_mfma_kernel<RP, true><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);  \
  else coldot_mfma_kernel<RP, false><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);
  if (r <= 16) { QLORA_COLDOT(16) }
  else if (r <= 32) { QLORA_COLDOT(32) }
  else if (r <= 64) { QLORA_COLDOT(64) }
  else { QLORA_COLDOT(128) }
#undef QLORA_COLDOT
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
