// Low-rank projection of an activation: the skinny product on the way into
// the adapter ("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// three-piece summary, piece 3: only the low-rank pair learns; "What is
// QLoRA?" (qubittool.com), "Key Characteristics": adapters in full precision).
//
//   out[m, j] = sum_c P[m, c] Q(c, j)       T = X A^T (Q = A, [r, C]),  U = dY B (Q = B, [C, r])
//
// bf16 products on the matrix cores (v_mfma_f32_16x16x32_bf16), fp32 sums.
// Optionally the scaled value s*out is also written as a bf16 hi/lo pair per
// row, [hi | lo | zero pad] with hi = RN_bf16(s*out), lo = RN_bf16(s*out - hi):
// the 2r extra contraction columns through which the main GEMMs add the
// low-rank term to their fp32 accumulator, so Y and dX are rounded once.
//
// Workgroup: kMR 16-row tiles of P and a range of columns, NW waves splitting
// the range into contiguous parts; every wave multiplies all kMR row tiles,
// so each Q fragment it loads serves kMR tiles (kMR = 4 at large M: Q, the
// whole low-rank factor, is then read once per 64 rows instead of once per
// 16, which at r = 64 was four times the bytes of P itself). Lanes read P in
// the MFMA operand layout (8 consecutive bf16 per lane, 16-byte loads, kU
// column steps in flight). Q as [r, C] is read the same way. Q as [C, r] (j contiguous) is staged per
// wave in LDS as a [32 c][r] tile and read back with the transposing read
// ds_read_b64_tr_b16, which hands each lane 4 consecutive c of its column j.
// The waves' partial sums are added in a fixed order in LDS. With the whole
// contraction in one workgroup (large M) the result and its split are written
// directly; for small M the contraction is also split over workgroups, each
// writes its partial, and a finalize kernel adds the partials in a fixed
// (split-major, then group) order. Reruns are bit-identical either way.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kMaxRankPad = 128;

// 8 bf16 starting at p (element index e0 of a row with `lim` valid elements):
// one 16-byte load when the row is 16-byte aligned (kVec), else 8 guarded loads.
template <bool kVec>
__device__ __forceinline__ u32x4 load8(const uint16_t* __restrict__ row, int64_t e0, int64_t lim) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (kVec) {
    if (e0 < lim) v = *reinterpret_cast<const u32x4*>(row + e0);
  } else {
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (e0 + i < lim) ? (uint32_t)row[e0 + i] : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = e[2 * i] | (e[2 * i + 1] << 16);
  }
  return v;
}

// Tall form (kMR > 1): waves per workgroup, workgroups aimed for, and the
// fewest contraction columns per split.
constexpr int kTallWaves = 8;
constexpr int kTallMR = 4;
constexpr int64_t kTallTargetWG = 256;
constexpr int64_t kTallMinCols = 1024;
constexpr int kTallDepth = 2;
constexpr bool kTallInterleave = true;

template <int kRP, int kMR>
constexpr int rowdot_threads() { return (kMR > 1 ? kTallWaves : kRP <= 64 ? 8 : 4) * 64; }

template <int kRP, int kQL, int kMR>
struct RowdotCfg {
  static constexpr int kTiles = kRP / 16;
  static constexpr int kRows = 16 * kMR;                             // rows of P per workgroup
  static constexpr int kU = kMR > 1 ? (kTiles >= 2 ? 1 : 2)          // column steps per load batch
                                    : (kTiles >= 8 ? 1 : 8 / kTiles);
  static constexpr int kNW = rowdot_threads<kRP, kMR>() / 64;        // waves per workgroup
  static constexpr int kDepth = kMR > 1 ? kTallDepth : 2;             // batches in the load ring
  static constexpr int kQPitch = kRP * 2 + (kRP >= 32 ? 32 : 0);     // bytes per staged Q row
  static constexpr int kStage = kU * 32 * kQPitch;                   // staged Q bytes per wave
  static constexpr int kRed = kNW * kRows * kRP * 4;                 // partial sums of the waves
  static constexpr int kSmem = (kQL == 1 && kNW * kStage > kRed) ? kNW * kStage : kRed;
};

// kQL: 0 = Q is [r, C], 1 = Q is [C, r]. kVecP / kVecQ: 16-byte rows.
// kDirect: write out / split (single column split), else write partials.
// kMask (Q = A only): P's elements whose byte in pmask [M, C] is 0 read as zero
// (dropout on the adapter's input).
// kF16: fp16 operands and split (the compute-type ablation), else bf16.
// kMR: 16-row tiles per workgroup, all multiplied by every wave.
template <int kRP, int kQL, bool kVecP, bool kVecQ, bool kDirect, bool kMask = false, bool kF16 = false, int kMR = 1>
__global__ __launch_bounds__((rowdot_threads<kRP, kMR>())) __attribute__((amdgpu_waves_per_eu(kMR > 1 ? 2 : 1))) void rowdot_kernel(
    const uint16_t* __restrict__ P, int64_t M, int64_t C, const uint16_t* __restrict__ Q, int r, int64_t cchunk,
    float* __restrict__ out, uint16_t* __restrict__ split, int xc, float scale, float* __restrict__ part,
    const uint8_t* __restrict__ pmask = nullptr) {
#pragma clang fp contract(off)
  using Cfg = RowdotCfg<kRP, kQL, kMR>;
  constexpr int kTiles = Cfg::kTiles, kU = Cfg::kU, kNW = Cfg::kNW, kRows = Cfg::kRows;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::kSmem];
  // wave-uniform (scalar) so that the column range and loop tests are too
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t m0 = (int64_t)blockIdx.x * kRows;
  const int64_t cs = blockIdx.y;
  const int64_t cbeg = cs * cchunk;
  const int64_t cend = (cbeg + cchunk < C) ? cbeg + cchunk : C;
  // Columns of this wave: a contiguous part of the range, or (kIL) every
  // kNW-th column step, so that the waves of a workgroup read adjacent
  // pieces of the same rows at the same time.
  constexpr bool kIL = kMR > 1 && kTallInterleave;
  constexpr int64_t kStep = 32 * kU;
  const int64_t qlen = cdiv(cend - cbeg, (int64_t)kNW * 32) * 32;  // per-wave length, multiple of 32
  const int64_t w0 = kIL ? cbeg + wave * kStep : cbeg + wave * qlen;
  const int64_t w1 = kIL ? cend : (w0 + qlen < cend) ? w0 + qlen : cend;
  const int64_t cstride = kIL ? kNW * kStep : kStep;

  const int row = lane & 15;
  const int ko = (lane >> 4) * 8;
  const uint16_t* prow[kMR];
  const uint8_t* mrow[kMR];
  bool mok[kMR];
#pragma unroll
  for (int i = 0; i < kMR; ++i) {
    const int64_t m = m0 + 16 * i + row;
    mok[i] = m < M;
    prow[i] = P + (m < M ? m : M - 1) * C;
    mrow[i] = kMask ? pmask + (m < M ? m : M - 1) * C : nullptr;
  }
  char* const stage = smem + wave * Cfg::kStage;

  f32x4 acc[kMR][kTiles];
#pragma unroll
  for (int i = 0; i < kMR; ++i)
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One batch = kU column steps of 32: the P operands and the raw Q values.
  // Two batches rotate (the loop is unrolled by two), so the next batch's
  // loads are in flight while the current one is multiplied.
  constexpr int kChunks = 32 * kRP / 8;  // 16-byte chunks of one staged [32][kRP] Q tile
  constexpr int kQL1 = kQL == 1 ? kU * (kChunks / 64) : 1;
  struct Batch {
    u32x4 a[kU][kMR];
    uint2 mk[kMask ? kU : 1][kMask ? kMR : 1];
    u32x4 q0[kQL == 0 ? kU * kTiles : 1];  // Q = [r, C]: operand layout
    u32x4 q1[kQL1];                        // Q = [C, r]: raw chunks for the LDS tile
    int64_t c0;                            // first column of the batch
  };
  // 16-byte rows (kFast): every load is issued unconditionally from a
  // clamped, in-range address -- rows past M read row M - 1 and Q rows past r
  // read row r - 1 (their results are never stored), columns past w1 read the
  // last in-range group and are zeroed before the multiply, in the tail batch
  // only -- so no load sits behind a branch that waits for it, and the next
  // batch stays in flight while this one is multiplied.
  constexpr bool kFast = kVecP && kVecQ && kMR > 1;
  auto load = [&](int64_t c, Batch& bt) {
    bt.c0 = c;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e0 = c + 32 * u + ko;
      const int64_t ec = e0 < w1 ? e0 : w1 - 8;
#pragma unroll
      for (int i = 0; i < kMR; ++i) {
        if constexpr (kFast) {
          bt.a[u][i] = *reinterpret_cast<const u32x4*>(prow[i] + ec);
          if constexpr (kMask) bt.mk[u][i] = *reinterpret_cast<const uint2*>(mrow[i] + ec);
        } else {
          bt.a[u][i] = load8<kVecP>(prow[i], e0, w1);
          if (!mok[i]) bt.a[u][i] = u32x4{0u, 0u, 0u, 0u};
          if constexpr (kMask) bt.mk[u][i] = e0 < w1 ? *reinterpret_cast<const uint2*>(mrow[i] + e0) : uint2{0u, 0u};
        }
      }
    }
    if constexpr (kQL == 0) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t e0 = c + 32 * u + ko;
        const int64_t ec = e0 < w1 ? e0 : w1 - 8;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const int j = t * 16 + row;
          if constexpr (kFast) {
            bt.q0[u * kTiles + t] = *reinterpret_cast<const u32x4*>(Q + (int64_t)(j < r ? j : r - 1) * C + ec);
          } else {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (j < r) v = load8<kVecQ>(Q + (int64_t)j * C, e0, w1);
            bt.q0[u * kTiles + t] = v;
          }
        }
      }
    } else {
      // Q[c + 32 u + cc][jc .. jc + 7] for chunk q = lane + 64 i (zeros past w1 / r)
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int i = 0; i < kChunks / 64; ++i) {
          const int q = lane + 64 * i;
          const int cc = q / (kRP / 8), jc = (q % (kRP / 8)) * 8;
          const int64_t cq = c + 32 * u + cc;
          u32x4 v = {0u, 0u, 0u, 0u};
          if constexpr (kFast) {
            v = *reinterpret_cast<const u32x4*>(Q + (cq < w1 ? cq : w1 - 1) * r + (jc < r ? jc : r - 8));
          } else if (cq < w1) {
            if constexpr (kVecQ) {
              if (jc < r) v = *reinterpret_cast<const u32x4*>(Q + cq * r + jc);
            } else {
              uint32_t e[8];
#pragma unroll
              for (int x = 0; x < 8; ++x) e[x] = (jc + x < r) ? (uint32_t)Q[cq * r + jc + x] : 0u;
#pragma unroll
              for (int x = 0; x < 4; ++x) v[x] = e[2 * x] | (e[2 * x + 1] << 16);
            }
          }
          bt.q1[u * (kChunks / 64) + i] = v;
        }
    }
  };
  // the tail batch of the fast path: zero what lies past w1 (wave-uniform test)
  auto clip = [&](Batch& bt) {
    if (bt.c0 + kStep <= w1) return;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = bt.c0 + 32 * u + ko < w1;
#pragma unroll
      for (int i = 0; i < kMR; ++i) {
        if (!ok) bt.a[u][i] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (kMask) if (!ok) bt.mk[u][i] = uint2{0u, 0u};
      }
      if constexpr (kQL == 0) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
          if (!ok) bt.q0[u * kTiles + t] = u32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int i = 0; i < kChunks / 64; ++i) {
          const int cc = (lane + 64 * i) / (kRP / 8);
          if (bt.c0 + 32 * u + cc >= w1) bt.q1[u * (kChunks / 64) + i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  // the batch's MFMAs (a batch that reaches past w1 is clipped first)
  auto compute = [&](Batch& bt) {
    bf16x8 b[kU][kTiles];
    if constexpr (kQL == 0) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int t = 0; t < kTiles; ++t) b[u][t] = __builtin_bit_cast(bf16x8, bt.q0[u * kTiles + t]);
    } else {
      // The staged region is rewritten every batch: the empty asm keeps the
      // compiler from moving these stores above the previous batch's
      // transposing reads (or the reads above the stores), which it might
      // otherwise treat as unrelated accesses.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int i = 0; i < kChunks / 64; ++i) {
          const int q = lane + 64 * i;
          const int cc = q / (kRP / 8), jc = (q % (kRP / 8)) * 8;
          *reinterpret_cast<u32x4*>(stage + u * 32 * Cfg::kQPitch + cc * Cfg::kQPitch + jc * 2) =
              bt.q1[u * (kChunks / 64) + i];
        }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int t = 0; t < kTiles; ++t) b[u][t] = tr_rows8(stage + u * 32 * Cfg::kQPitch, Cfg::kQPitch, t * 16, lane);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < kMR; ++i) {
        const bf16x8 pa = __builtin_bit_cast(bf16x8, kMask ? apply_mask8(bt.a[u][i], bt.mk[u][i]) : bt.a[u][i]);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) acc[i][t] = mfma16<kF16>(pa, b[u][t], acc[i][t]);
      }
  };
  if constexpr (!kVecP || !kVecQ) {
    // element-wise loads hold several registers per value: no second batch
    for (int64_t c = w0; c < w1; c += cstride) {
      Batch b0;
      load(c, b0);
      compute(b0);
    }
  } else if constexpr (kMR == 1) {
    // 16-row workgroups: a ring of two batches, the loads of batch j + 1
    // issued before batch j is multiplied (past w1 the loads read zeros). The
    // grouped loop below raised these forms' register count past the step
    // that halves their workgroups per CU.
    if (w0 < w1) {
      constexpr int kD = 2;
      Batch bt[kD];
      load(w0, bt[0]);
      for (int64_t c = w0; c < w1; c += kD * cstride) {
#pragma unroll
        for (int j = 0; j < kD; ++j) {
          load(c + (j + kD - 1) * cstride, bt[(j + kD - 1) % kD]);
          __builtin_amdgcn_sched_barrier(0);
          compute(bt[j]);
          if (c + (j + 1) * cstride >= w1) break;
        }
      }
    }
  } else if (w0 < w1) {
    // 64-row workgroups: a ring of kD batches, the loads of batch j + kD - 1
    // issued before batch j is multiplied. Only the wave's last batch can
    // reach past w1, so the loop takes whole groups of kD batches that end
    // before it, with no exit and no clip inside (an exit inside the unrolled
    // group made the compiler wait for every load in flight at the back edge,
    // which emptied the ring every kD batches); the last 1..kD batches follow
    // the loop. Loads past w1 read clamped in-range addresses.
    constexpr int kD = Cfg::kDepth;
    const int64_t nb = cdiv(w1 - w0, cstride);  // >= 1, wave-uniform
    Batch bt[kD];
#pragma unroll
    for (int i = 0; i < kD - 1; ++i) load(w0 + i * cstride, bt[i]);
    int64_t j = 0;
    for (; j + kD < nb; j += kD) {
#pragma unroll
      for (int i = 0; i < kD; ++i) {
        load(w0 + (j + i + kD - 1) * cstride, bt[(i + kD - 1) % kD]);
        __builtin_amdgcn_sched_barrier(0);
        compute(bt[i]);
      }
    }
    load(w0 + (j + kD - 1) * cstride, bt[kD - 1]);
#pragma unroll
    for (int i = 0; i < kD; ++i)
      if (j + i < nb) {
        if constexpr (kFast) clip(bt[i]);
        compute(bt[i]);
      }
  }
  __syncthreads();  // all staged-Q reads done before the region is reused
  // D layout: lane -> column (lane & 15), rows 4 (lane >> 4) + v of tile i
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < kMR; ++i)
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[(wave * kRows + 16 * i + 4 * (lane >> 4) + v) * kRP + t * 16 + (lane & 15)] = acc[i][t][v];
  __syncthreads();
  if constexpr (kDirect) {
    // one thread per (row, split column): columns [0, r) hi, [r, 2r) lo, rest 0
    if (split != nullptr) for (int i = threadIdx.x; i < kRows * xc; i += kNW * 64) {
      const int rr = i / xc, col = i - rr * xc;
      const int64_t mm = m0 + rr;
      if (mm >= M) continue;
      if (col < 2 * r) {
        const int j = col < r ? col : col - r;
        float s = red[rr * kRP + j];
#pragma unroll
        for (int w = 1; w < kNW; ++w) s += red[(w * kRows + rr) * kRP + j];  // parts in order
        if (col < r && out != nullptr) out[mm * r + j] = s;
        const float ss = scale * s;
        const uint16_t hi = to16<kF16>(ss);
        split[mm * xc + col] = col < r ? hi : to16<kF16>(ss - from16<kF16>(hi));
      } else {
        split[mm * xc + col] = 0;
      }
    }
    else {
      for (int i = threadIdx.x; i < kRows * r; i += kNW * 64) {
        const int rr = i / r, j = i - rr * r;
        const int64_t mm = m0 + rr;
        if (mm >= M) continue;
        float s = red[rr * kRP + j];
#pragma unroll
        for (int w = 1; w < kNW; ++w) s += red[(w * kRows + rr) * kRP + j];
        out[mm * r + j] = s;
      }
    }
  } else {
    for (int i = threadIdx.x; i < kRows * r; i += kNW * 64) {
      const int rr = i / r, j = i - rr * r;
      const int64_t mm = m0 + rr;
      if (mm >= M) continue;
      float s = red[rr * kRP + j];
#pragma unroll
      for (int w = 1; w < kNW; ++w) s += red[(w * kRows + rr) * kRP + j];
      part[(cs * M + mm) * r + j] = s;
    }
  }
}

// Partials of the small-M case -> out / split. Block = one row m; G = 256 / r
// thread groups each add splits g, g + G, ... in order; then thread j adds the
// G group sums in order.
template <bool kF16>
__global__ __launch_bounds__(256) void rowdot_finalize_kernel(const float* __restrict__ part, int64_t M, int r,
                                                              int64_t nsplit, float* __restrict__ out,
                                                              uint16_t* __restrict__ split, int xc, float scale) {
#pragma clang fp contract(off)
  __shared__ float gsum[256];
  __shared__ float tot[kMaxRankPad];
  const int t = threadIdx.x;
  const int64_t m = blockIdx.x;
  const int G = 256 / r;
  if (t < G * r) {
    const int j = t % r, g = t / r;
    // splits g, g + G, ... in order, loaded four at a time
    float s = 0.0f;
    int64_t p = g;
    for (; p + 3 * G < nsplit; p += 4 * G) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part[((p + u * G) * M + m) * r + j];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; p < nsplit; p += G) s += part[(p * M + m) * r + j];
    gsum[g * r + j] = s;
  }
  __syncthreads();
  if (t < r) {
    float s = gsum[t];
    for (int g = 1; g < G; ++g) s += gsum[g * r + t];
    tot[t] = s;
    if (out != nullptr) out[m * r + t] = s;
  }
  __syncthreads();
  if (split != nullptr) {
    for (int col = t; col < xc; col += 256) {
      uint16_t v = 0;
      if (col < 2 * r) {
        const float ss = scale * tot[col < r ? col : col - r];
        const uint16_t hi = to16<kF16>(ss);
        v = col < r ? hi : to16<kF16>(ss - from16<kF16>(hi));
      }
      split[m * xc + col] = v;
    }
  }
}

// Contractions up to this length are not split over workgroups: each wave
// then walks at most 256 columns, and the finalize launch would cost more
// than the split saves (a 1024-wide layer at M = 16).
constexpr int64_t kShortContraction = 2048;

int rowdot_splits(int64_t M, int64_t C) {
  const int64_t tiles = cdiv(M, (int64_t)16);
  if (tiles >= 128) return 1;                // enough row tiles: whole contraction per workgroup
  if (C <= kShortContraction) return 1;      // short rows: one pass per tile beats a second launch
  int64_t s = cdiv((int64_t)256, tiles);
  const int64_t maxs = cdiv(C, (int64_t)256);  // keep >= 256 columns per split
  if (s > maxs) s = maxs;
  return (int)(s < 1 ? 1 : s);
}

// Row tiles per workgroup and contraction splits. From 2048 rows (ranks up
// to 64) a workgroup takes 64 rows, and the contraction is split until there
// are about 256 workgroups, keeping >= 1024 columns per split; below that,
// one 16-row tile per workgroup as before.
constexpr int64_t kTallMinRows = 2048;
constexpr int kTallMinRank = 17;

struct RowdotPlan {
  int mr;  // 16-row tiles per workgroup
  int ns;  // contraction splits (partials + finalize when > 1)
};

RowdotPlan rowdot_plan(int64_t M, int64_t C, int r) {
  if (M >= kTallMinRows && r >= kTallMinRank && r <= 64) {
    const int64_t tiles = cdiv(M, (int64_t)(16 * kTallMR));
    int64_t s = cdiv(kTallTargetWG, tiles);
    const int64_t maxs = C / kTallMinCols;
    if (s > maxs) s = maxs;
    return {kTallMR, (int)(s < 1 ? 1 : s)};
  }
  return {1, rowdot_splits(M, C)};
}

template <int kRP, int kQL, int kMR>
hipError_t launch_rp(const uint16_t* P, int64_t M, int64_t C, const uint16_t* Q, int r, float* out,
                     uint16_t* split, float scale, float* part, hipStream_t stream, const uint8_t* pmask, bool f16,
                     int ns) {
  constexpr int kNW = RowdotCfg<kRP, kQL, kMR>::kNW;
  constexpr int kRows = RowdotCfg<kRP, kQL, kMR>::kRows;
  const int64_t cchunk = cdiv(cdiv(C, (int64_t)ns), (int64_t)32) * 32;
  const dim3 grid((unsigned)cdiv(M, (int64_t)kRows), (unsigned)ns);
  const int xc = lora_extra_cols(r);
  const bool vp = C % 8 == 0;
  const bool vq = kQL == 0 ? (C % 8 == 0) : (r % 8 == 0);
#define QLORA_RD(VP, VQ, D)                                                                                \
  rowdot_kernel<kRP, kQL, VP, VQ, D, false, false, kMR><<<grid, kNW * 64, 0, stream>>>(P, M, C, Q, r, cchunk, \
                                                                                      out, split, xc, scale, part)
#define QLORA_RDM(VQ, D)                                                                                   \
  rowdot_kernel<kRP, 0, true, VQ, D, true, false, kMR><<<grid, kNW * 64, 0, stream>>>(P, M, C, Q, r, cchunk, out, \
                                                                                     split, xc, scale, part, pmask)
#define QLORA_RDF(VP, VQ, D)                                                                               \
  rowdot_kernel<kRP, kQL, VP, VQ, D, false, true, kMR><<<grid, kNW * 64, 0, stream>>>(P, M, C, Q, r, cchunk, out, \
                                                                                     split, xc, scale, part)
#define QLORA_RD2(D)                                           \
  if (f16) {                                                   \
    if (pmask != nullptr) return hipErrorInvalidValue;         \
    if (vp && vq) QLORA_RDF(true, true, D);                    \
    else if (vp) QLORA_RDF(true, false, D);                    \
    else if (vq) QLORA_RDF(false, true, D);                    \
    else QLORA_RDF(false, false, D);                           \
  } else if constexpr (kQL == 0) {                             \
    if (pmask != nullptr) {                                    \
      if (!vp) return hipErrorInvalidValue;                    \
      if (vq) QLORA_RDM(true, D); else QLORA_RDM(false, D);    \
    } else if (vp && vq) QLORA_RD(true, true, D);              \
    else if (vp) QLORA_RD(true, false, D);                     \
    else if (vq) QLORA_RD(false, true, D);                     \
    else QLORA_RD(false, false, D);                            \
  } else {                                                     \
    if (pmask != nullptr) return hipErrorInvalidValue;         \
    if (vp && vq) QLORA_RD(true, true, D);                     \
    else if (vp) QLORA_RD(true, false, D);                     \
    else if (vq) QLORA_RD(false, true, D);                     \
    else QLORA_RD(false, false, D);                            \
  }
  if (ns == 1) {
    QLORA_RD2(true)
    return hipGetLastError();
  }
  QLORA_RD2(false)
#undef QLORA_RD2
#undef QLORA_RDF
#undef QLORA_RDM
#undef QLORA_RD
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f16)
    rowdot_finalize_kernel<true><<<(unsigned)M, 256, 0, stream>>>(part, M, r, ns, out, split, xc, scale);
  else
    rowdot_finalize_kernel<false><<<(unsigned)M, 256, 0, stream>>>(part, M, r, ns, out, split, xc, scale);
  return hipGetLastError();
}

template <int kRP, int kQL>
hipError_t launch_rq(const uint16_t* P, int64_t M, int64_t C, const uint16_t* Q, int r, float* out,
                     uint16_t* split, float scale, float* part, hipStream_t stream, const uint8_t* pmask, bool f16) {
  const RowdotPlan pl = rowdot_plan(M, C, r);
  if constexpr (kRP <= 64) {
    if (pl.mr > 1)
      return launch_rp<kRP, kQL, kTallMR>(P, M, C, Q, r, out, split, scale, part, stream, pmask, f16, pl.ns);
  }
  return launch_rp<kRP, kQL, 1>(P, M, C, Q, r, out, split, scale, part, stream, pmask, f16, pl.ns);
}

}  // namespace

size_t rowdot_ws_bytes(int64_t M, int64_t C, int r) {
  const int ns = rowdot_plan(M, C, r).ns;
  return ns > 1 ? align256((size_t)ns * (size_t)M * (size_t)r * 4) : 0;
}

hipError_t launch_rowdot(const uint16_t* P, int64_t M, int64_t C, const uint16_t* Q, int q_layout, int r,
                         float* out, uint16_t* split, float scale, float* part, hipStream_t stream,
                         const uint8_t* pmask, bool f16) {
#define QLORA_RP(RP)                                                                                  \
  return q_layout == 0 ? launch_rq<RP, 0>(P, M, C, Q, r, out, split, scale, part, stream, pmask, f16) \
                       : launch_rq<RP, 1>(P, M, C, Q, r, out, split, scale, part, stream, pmask, f16);
  if (r <= 16) { QLORA_RP(16) }
  if (r <= 32) { QLORA_RP(32) }
  if (r <= 64) { QLORA_RP(64) }
  QLORA_RP(128)
#undef QLORA_RP
}

}  // namespace qlora
