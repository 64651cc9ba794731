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

// G partial on the matrix cores: Gp[s][j][c] = sum_{m in split s} Q[m, j] P[m, c].
// The contraction runs over the tokens m, which are the slow index of both
// operands, so each 32-token step is staged in LDS in its stored orientation
// -- P as [32][4 kCW columns] bf16 (coalesced 16-byte loads), Q as [32][r]
// bf16 hi and lo halves of the fp32 value -- and both MFMA operands are
// gathered with the transposing read ds_read_b64_tr_b16 (8 consecutive tokens
// of one column per lane). v_mfma_f32_16x16x32_bf16: rows = j, columns = c;
// the hi and lo halves of Q are multiplied separately, so the products carry
// ~16 significant bits of Q. Each of the 4 waves owns kCW columns (64 or 32);
// a workgroup 4 kCW columns and one token split. The next steps' P and Q are
// loaded into registers (a ring of kDepth stages) while the current step's
// MFMAs run.
constexpr int kColdotDepth64 = 1;  // register stages in flight at ranks 33..64 (more stages cost occupancy)

template <int kRP, int kCW>
struct ColdotSmem {
  static constexpr int kPPitch = 4 * kCW * 2 + 32;  // bytes per staged P row (+ pad)
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

// kDirect (a single token split): the workgroup writes scale * its sums to G
// itself, (c, j) at G[c * g_sc + j * g_sj], added to G when accumulating --
// the value the reduce kernel would compute from one partial -- instead of a
// partial for a second launch.
// kCW: columns per wave (64 or 32). kVec: 16-byte P rows (C % 8 == 0); then
// every load is issued from a clamped, in-range address (rows past the split
// read its last row, columns past C the last 8) and the step that reaches
// past either end zeroes those values before staging them.
// kMask (16-byte P rows only): P's elements whose byte in pmask [M, C] is 0
// read as zero (dropout on the adapter's input).
// kF16: fp16 P and fp16 hi/lo halves of Q (the compute-type ablation).
// The second product of a paired launch (kPair: dA and dB of one layer in a
// single direct launch, blockIdx.y picking the product).
struct ColdotSecond {
  const uint16_t* P;
  int64_t C;
  const float* Q;
  float* G;
  int64_t g_sc, g_sj;
};

template <int kRP, int kCW, bool kVec, bool kMask = false, bool kF16 = false, bool kDirect = false, bool kPair = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void coldot_mfma_kernel(
    const uint16_t* __restrict__ P, int64_t M, int64_t C, const float* __restrict__ Q, int r, int64_t mchunk,
    float* __restrict__ partial, const uint8_t* __restrict__ pmask, float scale, float* __restrict__ G, int64_t g_sc,
    int64_t g_sj, int accumulate, ColdotSecond second = {}) {
#pragma clang fp contract(off)
  static_assert(!kPair || (kDirect && !kMask), "a paired launch writes G directly and takes no mask");
  if constexpr (kPair) {
    if (blockIdx.y == 1) {
      P = second.P; C = second.C; Q = second.Q; G = second.G; g_sc = second.g_sc; g_sj = second.g_sj;
    }
    if ((int64_t)blockIdx.x * (4 * kCW) >= C) return;  // (the grid covers the wider product)
  }
  constexpr int kJT = kRP / 16;
  constexpr int kCT = kCW / 16;              // 16-column tiles per wave
  constexpr int kCPR = kCW / 2;              // 16-byte chunks per staged P row (4 kCW columns)
  constexpr int kRPT = 256 / kCPR;           // P rows covered by one pass of the 256 threads
  constexpr int kPL = 32 / kRPT;             // P chunks per thread per step
  using Smem = ColdotSmem<kRP, kCW>;
  constexpr int kPP = Smem::kPPitch;
  constexpr int kQP = Smem::kQPitch;
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int64_t cw = (int64_t)blockIdx.x * (4 * kCW);
  const int64_t s = kPair ? 0 : blockIdx.y;
  const int64_t m0 = s * mchunk;
  const int64_t m1 = (m0 + mchunk < M) ? m0 + mchunk : M;
  f32x4 acc[kJT][kCT];
#pragma unroll
  for (int a = 0; a < kJT; ++a)
#pragma unroll
    for (int b = 0; b < kCT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // P tile: thread t owns chunk t % kCPR of rows t / kCPR + kRPT i (i < kPL).
  const int pc = (t % kCPR) * 8;
  const int pr = t / kCPR;
  const int64_t cp = cw + pc;
  const int64_t cpl = cp < C ? cp : C - 8;  // kVec: clamped column
  constexpr int kQE = 32 * kRP / 256;       // Q elements of one step per thread: t + 256 e
  struct Stage {
    u32x4 p[kPL];
    uint2 mk[kMask ? kPL : 1];
    float q[kQE];
  };
  // kBuf (16-byte rows, no mask): buffer loads through descriptors that
  // start at the split's first token and end after its last, each lane's
  // offsets fixed for the whole split and a scalar offset per step. Tokens
  // past the split then read as zero, and no address is recomputed or
  // clamped per step (64-bit address arithmetic and clamps were most of the
  // step's vector instructions). Columns past C read the next token's row
  // (or zero) and are zeroed in the tail step; Q columns j >= r read other
  // entries of Q, whose products land in rows j >= r of the result, which
  // are never stored. The launch keeps each split's P bytes under 4 GiB.
  constexpr bool kBuf = kVec && !kMask;
  i32x4 prs = {}, qrs = {};
  uint32_t poff[kBuf ? kPL : 1], qoff[kBuf ? kQE : 1];
  if constexpr (kBuf) {
    // (a split that starts past M has no tokens: empty descriptors, whose
    // loads read zero without touching memory)
    const int64_t mt = m1 > m0 ? m1 - m0 : 0;
    prs = make_rsrc(mt > 0 ? P + m0 * C : P, mt * C * 2);
    qrs = make_rsrc(mt > 0 ? Q + m0 * r : Q, mt * (int64_t)r * 4);
#pragma unroll
    for (int i = 0; i < kPL; ++i) poff[i] = (uint32_t)(((pr + kRPT * i) * C + cp) * 2);
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const int idx = t + 256 * e;
      qoff[e] = (uint32_t)(((idx / kRP) * r + idx % kRP) * 4);
    }
  }
  auto load = [&](int64_t mb, Stage& st) {
    if constexpr (kBuf) {
      const int sp = (int)(uint32_t)((mb - m0) * C * 2), sq = (int)(uint32_t)((mb - m0) * r * 4);
#pragma unroll
      for (int i = 0; i < kPL; ++i) st.p[i] = raw_buffer_load_b128(prs, (int)poff[i], sp, 0);
#pragma unroll
      for (int e = 0; e < kQE; ++e) st.q[e] = __builtin_bit_cast(float, raw_buffer_load_u32(qrs, (int)qoff[e], sq, 0));
      return;
    }
#pragma unroll
    for (int i = 0; i < kPL; ++i) {
      const int64_t m = mb + pr + kRPT * i;
      if constexpr (kVec) {
        const int64_t ml = m < m1 ? m : m1 - 1;
        st.p[i] = *reinterpret_cast<const u32x4*>(P + ml * C + cpl);
        if constexpr (kMask) st.mk[i] = *reinterpret_cast<const uint2*>(pmask + ml * C + cpl);
      } else {
        st.p[i] = u32x4{0u, 0u, 0u, 0u};
        if (m < m1) {
          uint32_t e[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) e[x] = (cp + x < C) ? (uint32_t)P[m * C + cp + x] : 0u;
#pragma unroll
          for (int x = 0; x < 4; ++x) st.p[i][x] = e[2 * x] | (e[2 * x + 1] << 16);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const int idx = t + 256 * e;
      const int mm = idx / kRP, j = idx % kRP;
      const int64_t m = mb + mm;
      // rows past the split read its last row (zeroed below); columns j >= r
      // read column r - 1: their products land in rows j >= r of the result,
      // which are never stored
      st.q[e] = Q[(m < m1 ? m : m1 - 1) * r + (j < r ? j : r - 1)];
    }
  };
  constexpr int kDepth = kRP <= 32 ? 4 : kRP <= 64 ? kColdotDepth64 : 1;
  // (kBuf: tokens past the split already read as zero; the workgroup whose
  // columns reach past C zeroes those, a fixed set of lanes)
  const bool ctail = cw + 4 * kCW > C;
  auto step = [&](int64_t mb, Stage& st) {
    if constexpr (kBuf) {
      if (ctail) {
        if (cp >= C) {
#pragma unroll
          for (int i = 0; i < kPL; ++i) st.p[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else if (mb + 32 > m1 || (kVec && ctail)) {
      // the step that reaches past the split's last token or past C: zero those values
#pragma unroll
      for (int i = 0; i < kPL; ++i)
        if (mb + pr + kRPT * i >= m1 || cp >= C) st.p[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < kQE; ++e)
        if (mb + (t + 256 * e) / kRP >= m1) st.q[e] = 0.0f;
    }
    // stage this step: P from registers, Q converted to bf16 hi / lo
#pragma unroll
    for (int i = 0; i < kPL; ++i)
      *reinterpret_cast<u32x4*>(sm.p + (pr + kRPT * i) * kPP + pc * 2) =
          kMask ? apply_mask8(st.p[i], st.mk[i]) : st.p[i];
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const int idx = t + 256 * e;
      const int mm = idx / kRP, j = idx % kRP;
      const uint16_t qh = to16<kF16>(st.q[e]);
      const uint16_t ql = to16<kF16>(st.q[e] - from16<kF16>(qh));
      *reinterpret_cast<uint16_t*>(sm.qh + mm * kQP + j * 2) = qh;
      *reinterpret_cast<uint16_t*>(sm.ql + mm * kQP + j * 2) = ql;
    }
    __syncthreads();
    if (mb + kDepth * 32 < m1) load(mb + kDepth * 32, st);
    bf16x8 pb[kCT];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) pb[ct] = tr_operand(sm.p, kPP, wave * kCW + ct * 16, lane);
#pragma unroll
    for (int a = 0; a < kJT; ++a) {
      const bf16x8 ah = tr_operand(sm.qh, kQP, a * 16, lane);
      const bf16x8 al = tr_operand(sm.ql, kQP, a * 16, lane);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        acc[a][ct] = mfma16<kF16>(ah, pb[ct], acc[a][ct]);
        acc[a][ct] = mfma16<kF16>(al, pb[ct], acc[a][ct]);
      }
    }
    __syncthreads();
  };
  if constexpr (kDepth == 4) {
    Stage s0, s1, s2, s3;
    load(m0, s0);
    if (m0 + 32 < m1) load(m0 + 32, s1);
    if (m0 + 64 < m1) load(m0 + 64, s2);
    if (m0 + 96 < m1) load(m0 + 96, s3);
    for (int64_t mb = m0; mb < m1; mb += 4 * 32) {
      step(mb, s0);
      if (mb + 32 >= m1) break;
      step(mb + 32, s1);
      if (mb + 64 >= m1) break;
      step(mb + 64, s2);
      if (mb + 96 >= m1) break;
      step(mb + 96, s3);
    }
  } else if constexpr (kDepth == 2) {
    Stage s0, s1;
    load(m0, s0);
    if (m0 + 32 < m1) load(m0 + 32, s1);
    for (int64_t mb = m0; mb < m1; mb += 2 * 32) {
      step(mb, s0);
      if (mb + 32 >= m1) break;
      step(mb + 32, s1);
    }
  } else {
    Stage s0;
    load(m0, s0);
    for (int64_t mb = m0; mb < m1; mb += 32) step(mb, s0);
  }
  // D[j][c]: lane -> c = lane % 16, j = 4 (lane / 16) + v
#pragma unroll
  for (int a = 0; a < kJT; ++a)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const int64_t c = cw + wave * kCW + ct * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = a * 16 + 4 * (lane >> 4) + v;
        if (c < C && j < r) {
          if constexpr (kDirect) {
            float* g = G + c * g_sc + j * g_sj;
            const float val = scale * acc[a][ct][v];
            *g = accumulate ? (*g + val) : val;
          } else {
            partial[(s * r + j) * C + c] = acc[a][ct][v];
          }
        }
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

// Token splits: the fewest that give about 512 workgroups of 256 columns
// (each split >= 128 tokens, at most 32 splits). Measured: half as many,
// longer-running workgroups (or 128-column ones) were slower -- the kernel is
// bound by the latency of its per-step barriers -- although they write fewer
// partial sums.
constexpr int kColdotCW = 64;  // columns per wave
constexpr int64_t kColdotTargetWG = 512;

// The buffer-load form addresses one split's P rows with 32-bit offsets.
bool coldot_buf_fits(int64_t mchunk, int64_t C) { return mchunk * C * 2 < ((int64_t)1 << 32) - 256; }

int coldot_splits(int64_t M, int64_t C) {
  int64_t s = cdiv(kColdotTargetWG, cdiv(C, (int64_t)(4 * kColdotCW)));
  int64_t cap = M / 128;
  if (cap > 32) cap = 32;
  if (s > cap) s = cap;
  return (int)(s < 1 ? 1 : s);
}

size_t coldot_ws_bytes(int64_t M, int64_t C, int r) {
  return align256((size_t)coldot_splits(M, C) * (size_t)C * (size_t)r * 4);
}

hipError_t launch_coldot(const uint16_t* P, int64_t M, int64_t C, const float* Q, int r, float scale, float* G,
                         int64_t g_sc, int64_t g_sj, int accumulate, float* partial, hipStream_t stream,
                         const uint8_t* pmask, bool f16) {
  const int ns = coldot_splits(M, C);
  const int64_t mchunk = cdiv(cdiv(M, ns), 32) * 32;
  const dim3 grid((unsigned)cdiv(C, 4 * kColdotCW), (unsigned)ns);
  // 16-byte rows; without a mask they are read through per-split buffer
  // descriptors (32-bit offsets), so a split's P bytes stay under 4 GiB
  const bool vec = C % 8 == 0 && (pmask != nullptr || coldot_buf_fits(mchunk, C));
  if (pmask != nullptr && !vec) return hipErrorInvalidValue;
  if (pmask != nullptr && f16) return hipErrorInvalidValue;
  const bool direct = ns == 1;
#define QLORA_COLDOT3(RP, CW, VEC, MASK, F16, D)                                                                \
  coldot_mfma_kernel<RP, CW, VEC, MASK, F16, D><<<grid, 256, 0, stream>>>(P, M, C, Q, r, mchunk, partial, pmask, \
                                                                           scale, G, g_sc, g_sj, accumulate)
#define QLORA_COLDOT2(RP, CW, D)                                  \
  if (f16 && vec) QLORA_COLDOT3(RP, CW, true, false, true, D);    \
  else if (f16) QLORA_COLDOT3(RP, CW, false, false, true, D);     \
  else if (pmask != nullptr) QLORA_COLDOT3(RP, CW, true, true, false, D); \
  else if (vec) QLORA_COLDOT3(RP, CW, true, false, false, D);     \
  else QLORA_COLDOT3(RP, CW, false, false, false, D);
#define QLORA_COLDOT(RP)                                  \
  {                                                       \
    if (direct) { QLORA_COLDOT2(RP, kColdotCW, true) }    \
    else { QLORA_COLDOT2(RP, kColdotCW, false) }          \
  }
  if (r <= 16) QLORA_COLDOT(16)
  else if (r <= 32) QLORA_COLDOT(32)
  else if (r <= 64) QLORA_COLDOT(64)
  else QLORA_COLDOT(128)
#undef QLORA_COLDOT
#undef QLORA_COLDOT2
#undef QLORA_COLDOT3
  if (!direct)
    coldot_reduce_kernel<<<(unsigned)cdiv(C * r, 256), 256, 0, stream>>>(partial, C, r, ns, scale, G, g_sc, g_sj,
                                                                        accumulate);
  return hipGetLastError();
}

bool coldot_pairable(int64_t M, int64_t C0, int64_t C1) {
  return coldot_splits(M, C0) == 1 && coldot_splits(M, C1) == 1;
}

hipError_t launch_coldot_pair(const uint16_t* P0, int64_t C0, const float* Q0, float* G0, int64_t g_sc0,
                              int64_t g_sj0, const uint16_t* P1, int64_t C1, const float* Q1, float* G1,
                              int64_t g_sc1, int64_t g_sj1, int64_t M, int r, float scale, int accumulate,
                              hipStream_t stream, bool f16) {
  if (!coldot_pairable(M, C0, C1)) return hipErrorInvalidValue;
  const int64_t mchunk = cdiv(M, (int64_t)32) * 32;
  const int64_t cmax = C0 > C1 ? C0 : C1;
  const dim3 grid((unsigned)cdiv(cmax, 4 * kColdotCW), 2u);
  const ColdotSecond sec{P1, C1, Q1, G1, g_sc1, g_sj1};
  const bool vec = C0 % 8 == 0 && C1 % 8 == 0 && coldot_buf_fits(mchunk, cmax);
#define QLORA_PAIR3(RP, VEC, F16)                                                                              \
  coldot_mfma_kernel<RP, kColdotCW, VEC, false, F16, true, true><<<grid, 256, 0, stream>>>(                      \
      P0, M, C0, Q0, r, mchunk, nullptr, nullptr, scale, G0, g_sc0, g_sj0, accumulate, sec)
#define QLORA_PAIR(RP)                                   \
  {                                                      \
    if (f16) { if (vec) QLORA_PAIR3(RP, true, true); else QLORA_PAIR3(RP, false, true); }    \
    else { if (vec) QLORA_PAIR3(RP, true, false); else QLORA_PAIR3(RP, false, false); }      \
  }
  if (r <= 16) QLORA_PAIR(16)
  else if (r <= 32) QLORA_PAIR(32)
  else if (r <= 64) QLORA_PAIR(64)
  else QLORA_PAIR(128)
#undef QLORA_PAIR
#undef QLORA_PAIR3
  return hipGetLastError();
}

}  // namespace qlora
