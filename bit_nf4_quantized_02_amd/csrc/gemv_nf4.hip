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
// Each workgroup owns 16 kT output rows (n) and the whole contraction; its
// kW waves take its 256-wide chunks in turn (wave w: chunks w, w + kW, ...). The codes of a chunk (kT tiles x 16 rows x 128 bytes) go from HBM
// straight into LDS (buffer loads into LDS, no registers held), into a ring
// of three per wave: one chunk is worked on while the next two are in
// flight, which keeps about 64 KB of codes per CU on the way. A lane takes
// one whole 64-block of one row (32 bytes, one scale) from the ring, expands
// it to bf16 in registers through an LDS table indexed by whole code bytes
// (one read yields the levels of two weights; the products are those of the
// 16-entry codebook) and feeds it straight to v_mfma_f32_16x16x32_bf16 as the
// B operand; X (padded to 16 rows with zeros) is the A operand. The
// contraction order inside a chunk is permuted the same way on both operands
// (lane group g takes columns 64 g .. 64 g + 63), which leaves the sum
// unchanged and makes each lane's codes contiguous. From 5 tokens a first
// small kernel writes X in exactly that operand order (per 256-column chunk,
// per MFMA, per lane: 16 bytes), so each activation load instruction reads
// 1 KB in one run; read in place, the 16 token rows and 4 column groups of
// one instruction fall in 64 different cache lines.
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

// Level table: entry b (a code byte) holds the level pair (L[b & 15],
// L[b >> 4]) of its two codes, kLutCopies times side by side, so that lane l
// reads copy l % kLutCopies: the 16 lanes that share the LDS banks in one
// cycle of an 8-byte read then hit 16 different bank pairs whatever codes
// they look up (with one shared copy, random codes collide).
// With eight waves per workgroup (one workgroup per CU) the table holds 32
// copies, 256 bytes per entry: a lane's address is then its code byte in bits
// 8..15 and its copy offset in bits 0..7, formed by one byte permute instead
// of an extract and a shift-or; 32 copies also leave no bank conflict at all.
template <int kW>
constexpr int lut_copies() { return kW == 8 ? 32 : 16; }
constexpr int kRingDepth = 3;  // chunks of codes per wave: one worked on, two in flight

// s_waitcnt immediate that waits for LDS / scalar-memory operations only
// (lgkmcnt <= n; vmcnt and expcnt left at their maxima)
constexpr int lgkm_wait(int n) { return 0xC07F | (n << 8); }

// Swizzle of a 128-byte code line in LDS: row r of a 16-row tile keeps its
// 16-byte segment g at position g ^ sw(r). The 8 (or 16) lanes that read one
// segment of 8 (16) consecutive rows in one LDS cycle then hit distinct banks
// whether the LDS serves 128 or 256 bytes per cycle.
__device__ __forceinline__ int code_swz(int r) { return (r ^ (r >> 3)) & 7; }

// Scale fields of block blk in one of the three stored forms, without
// branches (kForm 0: double-quantized, E4M3 code + fp32 second-level scale
// per 256 blocks; 1: fp32 per block; 2: bf16 per block), as scale_fields.
// c8r / s2r: descriptors of the code and scale arrays.
template <int kForm>
__device__ __forceinline__ void scale_fields_of(const i32x4& c8r, const i32x4& s2r, uint32_t blk, uint32_t& c8,
                                                float& s2v) {
  if constexpr (kForm == 0) {
    c8 = raw_buffer_load_u8(c8r, (int)blk, 0, 0);
    s2v = __builtin_bit_cast(float, raw_buffer_load_u32(s2r, (int)((blk / kDqBlock) * 4), 0, 0));
  } else if constexpr (kForm == 1) {
    c8 = kE4m3One;
    s2v = __builtin_bit_cast(float, raw_buffer_load_u32(s2r, (int)(blk * 4), 0, 0));
  } else {
    c8 = kE4m3One;
    s2v = bf16_bits_to_f32(raw_buffer_load_u16(s2r, (int)(blk * 2), 0, 0));
  }
}

// Scale fields of one 256-column chunk for the lane's rows, and its
// activation operand.
template <int kT>
struct GvStage {
  uint32_t c8[kT];
  float s2v[kT];
  u32x4 xa[8];
};

// kT: 16-row tiles per workgroup (each wave covers all of them over its
// share of the contraction); kW: waves. kXp: activations from the
// operand-ordered copy Xp (else read in place from X). kF16: fp16
// activations, weights, B and output (the compute-type ablation). kForm: the
// block-scale form (scale_fields_of).
template <int kT, int kW, bool kXp, bool kF16, int kForm>
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
  constexpr int NT = 16 * kT;
  constexpr int kSlot = kT * 2048;  // one wave's codes of one chunk: kT tiles x 16 rows x 128 bytes
  // three separate ring arrays, so the compiler can tell the one being read
  // from the ones being filled by direct copies (and waits only for the copy
  // of the chunk it reads)
  constexpr int kLutCopies = lut_copies<kW>();
  __shared__ __attribute__((aligned(16))) char lut[256 * kLutCopies * 8];
  __shared__ __attribute__((aligned(16))) char ring0[kW * kSlot];
  __shared__ __attribute__((aligned(16))) char ring1[kW * kSlot];
  __shared__ __attribute__((aligned(16))) char ring2[kW * kSlot];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // the 16 levels pass through the first ring (not yet in use) so that the
  // table fill below reads LDS, not 16 rounds of global loads per thread
  float* const levels = reinterpret_cast<float*>(ring0);
  if (t < 16) levels[t] = codebook[t];
  __syncthreads();
  for (int i = t; i < 256 * kLutCopies; i += 64 * kW) {
    const int e = i / kLutCopies;
    reinterpret_cast<float2*>(lut)[i] = float2{levels[e & 15], levels[e >> 4]};
  }
  const float mean = weight_mean(code8, mean_p);
  const int64_t n0 = (int64_t)blockIdx.x * NT;
  // this wave's contiguous range of 256-column chunks (a multiple-of-64 tail
  // in the last one)
  const int nq = (int)cdiv(K, (int64_t)256);
  // chunks wave, wave + kW, wave + 2 kW, ...: the waves of a workgroup read
  // neighbouring chunks of the same rows at about the same time (kW x 128
  // contiguous bytes per row) rather than far-apart pieces of each row
  const int cnt = wave < nq ? (nq - 1 - wave) / kW + 1 : 0;
  const int grp = lane >> 4;  // 0..3: which 64-block of a chunk
  const int col = lane & 15;  // A: token row m; B: weight row within a tile
  const int64_t kblocks = K / kBlock;

  // Copies: lane l of copy h of tile i fills row 8 h + l / 8 of the tile at
  // swizzled position l % 8, i.e. logical segment (l % 8) ^ sw(row). Rows past
  // N lie past the end of the codes and read as zero (their outputs are not
  // stored); columns past K in the last chunk read the next row's codes and
  // meet zero activations.
  const i32x4 crs = make_rsrc(codes, N * (K / 2));
  uint32_t cvoff[kT][2];
#pragma unroll
  for (int i = 0; i < kT; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = 8 * h + (lane >> 3);
      const int g = (lane & 7) ^ code_swz(rr);
      cvoff[i][h] = (uint32_t)((n0 + 16 * i + rr) * (K / 2) + 16 * g);
    }
  // reads: row col, logical segments 2 grp and 2 grp + 1 (64 codes)
  const uint32_t rd0 = (uint32_t)(col * 128 + 16 * ((2 * grp) ^ code_swz(col)));
  const uint32_t lane_off = (uint32_t)(lane % kLutCopies) * 8;
  // scale rows (clamped: rows past N are computed and dropped)
  uint32_t bbase[kT];  // (blocks < 2^27: the codes stay under 4 GiB)
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int64_t n = n0 + 16 * i + col;
    bbase[i] = (uint32_t)((n < N ? n : N - 1) * kblocks);
  }
  // activations: Xp[q][s][lane] (operand order), or X[col][256 q + 64 grp +
  // 8 s ..] in place, token rows past M and columns past K reading as zero
  const i32x4 xrs = kXp ? make_rsrc(Xp, (int64_t)nq * 512 * 16) : make_rsrc(X, M * K * 2);
  const uint32_t xvoff = kXp ? (uint32_t)lane * 16 : (uint32_t)(col * K * 2 + 128 * grp);

  // scale arrays (blocks < 2^30: 32-bit byte offsets)
  const int64_t nblk = N * kblocks;
  const i32x4 c8rs = make_rsrc(code8, kForm == 0 ? nblk : 0);
  const i32x4 s2rs = make_rsrc(s2, kForm == 0 ? cdiv(nblk, (int64_t)kDqBlock) * 4 : nblk * (kForm == 1 ? 4 : 2));

  auto issue = [&](int j, char* R, GvStage<kT>& st) {
    const int q = wave + kW * (j < cnt ? j : cnt - 1);  // past the range: the last chunk again
    char* const dst = R + wave * kSlot;
#pragma unroll
    for (int i = 0; i < kT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) copy16(crs, cvoff[i][h], q * 128, dst + i * 2048 + h * 1024);
    const int kc = q * 256 + 64 * grp;
    const uint32_t bq = (uint32_t)(kc < K ? kc / kBlock : kblocks - 1);
#pragma unroll
    for (int i = 0; i < kT; ++i) scale_fields_of<kForm>(c8rs, s2rs, bbase[i] + bq, st.c8[i], st.s2v[i]);
    if constexpr (kXp) {
#pragma unroll
      for (int s = 0; s < 8; ++s) st.xa[s] = raw_buffer_load_b128(xrs, (int)xvoff, q * 8192 + s * 1024, 0);
    } else {
      const uint32_t v = kc < K ? xvoff : 0x80000000u;
#pragma unroll
      for (int s = 0; s < 8; ++s) st.xa[s] = raw_buffer_load_b128(xrs, (int)(v + 16 * s), q * 512, 0);
    }
  };

  f32x4 acc[kT];
#pragma unroll
  for (int i = 0; i < kT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Work on one chunk, in groups of kGw code words (8 kGw weights of one
  // row per lane): the level-table reads of group g + 1 are issued before
  // the products of group g, so about 4 kGw + 4 reads per wave are in
  // flight instead of the 4 that one word's expansion waits for.
  constexpr int kGw = 2;
  constexpr int kGroups = kT * 8 / kGw;
  auto compute = [&](const char* R, const GvStage<kT>& st) {
    const char* const src = R + wave * kSlot;
    bf16x8 xa[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) xa[s] = __builtin_bit_cast(bf16x8, st.xa[s]);
    uint32_t cw[kT][8];
    float cp[kT];
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(src + i * 2048 + rd0);
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(src + i * 2048 + (rd0 ^ 16u));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cw[i][e] = c0[e];
        cw[i][4 + e] = c1[e];
      }
      cp[i] = decode_block_scale(st.c8[i], st.s2v[i], mean);
    }
    float2 lv[2][4 * kGw];
    auto gather = [&](int g, float2 (&out)[4 * kGw]) {
      const int i = g / (8 / kGw), s0 = (g % (8 / kGw)) * kGw;
#pragma unroll
      for (int w = 0; w < kGw; ++w)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t addr;
          if constexpr (kLutCopies == 32) {
            // bytes of the result: lane_off (byte 0 of the second operand),
            // code byte p (byte p of the first), zero, zero
            addr = __builtin_amdgcn_perm(cw[i][s0 + w], lane_off, 0x0C0C0400u + ((uint32_t)p << 8));
          } else {
            addr = (((cw[i][s0 + w] >> (8 * p)) & 0xFFu) * (kLutCopies * 8)) | lane_off;
          }
          out[4 * w + p] = *reinterpret_cast<const float2*>(lut + addr);
        }
    };
    gather(0, lv[0]);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (g + 1 < kGroups) {
        gather(g + 1, lv[(g + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(lgkm_wait(4 * kGw));  // group g's reads (one wait for all of them)
      } else {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(lgkm_wait(0));
      }
      __builtin_amdgcn_sched_barrier(0);
      const int i = g / (8 / kGw), s0 = (g % (8 / kGw)) * kGw;
#pragma unroll
      for (int w = 0; w < kGw; ++w) {
        u32x4 bw;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float2 l = lv[g & 1][4 * w + p];
          bw[p] = pack2<kF16>(nf4_scaled(l.x, cp[i]), nf4_scaled(l.y, cp[i]));
        }
        acc[i] = mfma16<kF16>(xa[s0 + w], __builtin_bit_cast(bf16x8, bw), acc[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __syncthreads();  // the level table (and the levels read before the copies reuse the first ring)
  if (cnt > 0) {
    GvStage<kT> st0, st1, st2;
    issue(0, ring0, st0);
    issue(1, ring1, st1);
    // whole groups of three chunks, with no exit inside a group: an exit
    // between the chunks leaves a path on which a chunk's loads are still
    // pending at the loop head, and the compiler then waits for every load
    // in flight there
    int j = 0;
    for (; j + kRingDepth <= cnt; j += kRingDepth) {
      // the scheduling barriers keep each chunk's copies and loads issued
      // ahead of the work on the chunk before them
      issue(j + 2, ring2, st2);
      __builtin_amdgcn_sched_barrier(0);
      compute(ring0, st0);
      __builtin_amdgcn_sched_barrier(0);
      issue(j + 3, ring0, st0);
      __builtin_amdgcn_sched_barrier(0);
      compute(ring1, st1);
      __builtin_amdgcn_sched_barrier(0);
      issue(j + 4, ring1, st1);
      __builtin_amdgcn_sched_barrier(0);
      compute(ring2, st2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the last one or two chunks, already in rings 0 and 1
    if (j < cnt) compute(ring0, st0);
    if (j + 1 < cnt) compute(ring1, st1);
  }
  // copies past the range may still be landing: all done before the rings
  // are reused below
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // partial sums and the low-rank tiles reuse the rings
  float(*red)[kT][16][16] = reinterpret_cast<float(*)[kT][16][16]>(ring0);  // [kW]
  float(*lred)[16][16] = reinterpret_cast<float(*)[16][16]>(ring1);          // [kT]
  static_assert(sizeof(float) * kW * kT * 256 <= kW * kSlot, "partials fit the ring");
  // D[m][n]: lane -> n = lane & 15, m = 4 (lane >> 4) + v
#pragma unroll
  for (int i = 0; i < kT; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][i][4 * (lane >> 4) + v][lane & 15] = acc[i][v];
  if (r > 0) {
    // L[m][n] = sum_j T[m][j] B[n][j] for tile i on wave i (mod kW), 4 ranks
    // per v_mfma_f32_16x16x4_f32: A = T (lane: token lane % 16, rank lane / 16),
    // B = B^T (lane: weight row lane % 16, same rank); rows past M or N and
    // ranks past r read as zero
    for (int i = wave; i < kT; i += kW) {
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
    if (r > 0) y = fmaf(scale, lred[i][m][nc], y);
    Y[m * N + n] = to16<kF16>(y);
  }
}

}  // namespace

bool gemv_fits(int64_t n, int64_t k) { return (n + 256) * (k / 2) < ((int64_t)1 << 32); }

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
  if (!gemv_fits(w.n, w.k)) return hipErrorInvalidValue;
  u32x4* Xp = static_cast<u32x4*>(ws);
  const bool xp = M >= kXpMinM && w.n >= kXpMinN;
  if (xp) {
    const int64_t entries = cdiv(w.k, (int64_t)256) * 512;
    gemv_xperm_kernel<<<(unsigned)cdiv(entries, (int64_t)256), 256, 0, stream>>>(X, M, w.k, Xp, entries);
  }
  // Tiles and waves per workgroup: two 16-row tiles where that still gives
  // every CU a workgroup, else one; four waves (two workgroups per CU) where
  // there are at least two workgroups per CU, else eight (one per CU, the
  // contraction split eight ways).
  const int64_t t2 = cdiv(w.n, (int64_t)32);
  const int kt = t2 >= 256 ? 2 : 1;
  const int64_t wgs = kt == 2 ? t2 : cdiv(w.n, (int64_t)16);
  const int kw = kt == 2 && wgs >= 512 ? 4 : 8;
#define QLORA_GEMV4(KT, W, XP, H, F)                                                                           \
  gemv_nf4_kernel<KT, W, XP, H, F><<<dim3((unsigned)wgs), 64 * W, 0, stream>>>(                                \
      w.codes, w.code8, w.s2, w.mean, w.codebook, w.s2_bf16, w.n, w.k, X, Xp, M, T, B, r, scale, Y)
#define QLORA_GEMV3(KT, W, XP, H)          \
  {                                        \
    if (form == 0) QLORA_GEMV4(KT, W, XP, H, 0); \
    else if (form == 1) QLORA_GEMV4(KT, W, XP, H, 1); \
    else QLORA_GEMV4(KT, W, XP, H, 2);     \
  }
#define QLORA_GEMV2(KT, W, XP) \
  if (f16) QLORA_GEMV3(KT, W, XP, true) else QLORA_GEMV3(KT, W, XP, false)
#define QLORA_GEMV(KT, W)                                                   \
  {                                                                         \
    if (xp) { QLORA_GEMV2(KT, W, true) } else { QLORA_GEMV2(KT, W, false) } \
  }
  const int form = w.code8 ? 0 : (w.s2_bf16 ? 2 : 1);
  if (kt == 2) {
    if (kw == 4) QLORA_GEMV(2, 4) else QLORA_GEMV(2, 8)
  } else QLORA_GEMV(1, 8)
#undef QLORA_GEMV
#undef QLORA_GEMV2
#undef QLORA_GEMV3
#undef QLORA_GEMV4
  return hipGetLastError();
}

}  // namespace qlora
