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

// kMask (16-byte P rows only): P's elements whose byte in pmask [M, C] is 0
// read as zero (dropout on the adapter's input).
// kF16: fp16 P and fp16 hi/lo halves of Q (the compute-type ablation).
template <int kRP, bool kVec, bool kMask = false, bool kF16 = false>
__global__ __launch_bounds__(256) void coldot_mfma_kernel(const uint16_t* __restrict__ P, int64_t M, int64_t C,
                                                          const float* __restrict__ Q, int r, int64_t mchunk,
                                                          float* __restrict__ partial,
                                                          const uint8_t* __restrict__ pmask = nullptr) {
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
  auto load_p = [&](int64_t mb, u32x4 (&v)[4], uint2 (&mk)[kMask ? 4 : 1]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb + (t >> 5) + 8 * i;
      const int64_t c = cw + (t & 31) * 8;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (kMask) mk[i] = uint2{0u, 0u};
      if (m < m1) {
        if constexpr (kVec) {
          if (c < C) {
            v[i] = *reinterpret_cast<const u32x4*>(P + m * C + c);
            if constexpr (kMask) mk[i] = *reinterpret_cast<const uint2*>(pmask + m * C + c);
          }
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
  // Q of one step (32 tokens x kRP, fp32): thread t owns elements t + 256 e
  constexpr int kQE = 32 * kRP / 256;
  auto load_q = [&](int64_t mb, float (&qv)[kQE]) {
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const int idx = t + 256 * e;
      const int mm = idx / kRP, j = idx % kRP;
      const int64_t m = mb + mm;
      qv[e] = (j < r && m < m1) ? Q[m * r + j] : 0.0f;
    }
  };
  // Several steps of P and Q in flight: a ring of register stages with
  // compile-time indices (the loop is unrolled by the ring length), each
  // refilled for the step kDepth ahead right after it has been staged into
  // LDS. Four stages up to r = 32; one for larger ranks (register budget).
  constexpr int kDepth = kRP <= 32 ? 4 : 1;
  struct Stage {
    u32x4 p[4];
    uint2 mk[kMask ? 4 : 1];
    float q[kQE];
  };
  auto step = [&](int64_t mb, Stage& stg) {
    // stage this step: P from registers, Q converted to bf16 hi / lo
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(sm.p + ((t >> 5) + 8 * i) * kPPitch + (t & 31) * 16) =
          kMask ? apply_mask8(stg.p[i], stg.mk[i]) : stg.p[i];
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const int idx = t + 256 * e;
      const int mm = idx / kRP, j = idx % kRP;
      const uint16_t qh = to16<kF16>(stg.q[e]);
      const uint16_t ql = to16<kF16>(stg.q[e] - from16<kF16>(qh));
      *reinterpret_cast<uint16_t*>(sm.qh + mm * kQP + j * 2) = qh;
      *reinterpret_cast<uint16_t*>(sm.ql + mm * kQP + j * 2) = ql;
    }
    __syncthreads();
    if (mb + kDepth * 32 < m1) {
      load_p(mb + kDepth * 32, stg.p, stg.mk);
      load_q(mb + kDepth * 32, stg.q);
    }
    bf16x8 pb[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) pb[ct] = tr_operand(sm.p, kPPitch, wave * 64 + ct * 16, lane);
#pragma unroll
    for (int a = 0; a < kJT; ++a) {
      const bf16x8 ah = tr_operand(sm.qh, kQP, a * 16, lane);
      const bf16x8 al = tr_operand(sm.ql, kQP, a * 16, lane);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[a][ct] = mfma16<kF16>(ah, pb[ct], acc[a][ct]);
        acc[a][ct] = mfma16<kF16>(al, pb[ct], acc[a][ct]);
      }
    }
    __syncthreads();
  };
  if constexpr (kDepth == 4) {
    Stage s0, s1, s2, s3;
    load_p(m0, s0.p, s0.mk); load_q(m0, s0.q);
    load_p(m0 + 32, s1.p, s1.mk); load_q(m0 + 32, s1.q);
    load_p(m0 + 64, s2.p, s2.mk); load_q(m0 + 64, s2.q);
    load_p(m0 + 96, s3.p, s3.mk); load_q(m0 + 96, s3.q);
    for (int64_t mb = m0; mb < m1; mb += 4 * 32) {
      step(mb, s0);
      if (mb + 32 >= m1) break;
      step(mb + 32, s1);
      if (mb + 64 >= m1) break;
      step(mb + 64, s2);
      if (mb + 96 >= m1) break;
      step(mb + 96, s3);
    }
  } else {
    Stage s0;
    load_p(m0, s0.p, s0.mk); load_q(m0, s0.q);
    for (int64_t mb = m0; mb < m1; mb += 32) step(mb, s0);
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
  // partials added in split order; loaded eight at a time so the loads of a
  // batch are in flight together
  float s = 0.0f;
  int64_t p = 0;
  for (; p + 8 <= nsplit; p += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[((p + u) * r + j) * C + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; p < nsplit; ++p) s += partial[(p * r + j) * C + c];
  float* g = G + c * g_sc + j * g_sj;
  const float v = scale * s;
  *g = accumulate ? (*g + v) : v;
}

}  // namespace

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
                         int64_t g_sc, int64_t g_sj, int accumulate, float* partial, hipStream_t stream,
                         const uint8_t* pmask, bool f16) {
  const int ns = coldot_splits(M);
  const int64_t mchunk = cdiv(cdiv(M, ns), 32) * 32;
  const dim3 grid((unsigned)cdiv(C, 256), (unsigned)ns);
  const bool vec = C % 8 == 0;
  if (pmask != nullptr && !vec) return hipErrorInvalidValue;
  if (pmask != nullptr && f16) return hipErrorInvalidValue;
#define QLORA_COLDOT(RP)                                                                                    \
  if (f16 && vec)                                                                                          \
    coldot_mfma_kernel<RP, true, false, true><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);   \
  else if (f16)                                                                                            \
    coldot_mfma_kernel<RP, false, false, true><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);  \
  else if (pmask != nullptr)                                                                               \
    coldot_mfma_kernel<RP, true, true><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial, pmask);   \
  else if (vec) coldot_mfma_kernel<RP, true><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial);    \
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

}  // namespace qlora
