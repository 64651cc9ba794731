// dX for small token counts (M <= 16): the backward's pass through the
// frozen 4-bit base as a bandwidth-bound kernel, like the forward GEMV
// ("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
// "Batched 4-bit matmuls"; the gradient flows back through the quantized
// weights, "What is QLoRA?" (qubittool.com), "Key Characteristics").
//
//   dX = RN_bf16( dY W' + s (U A) [. mask * keep] ),   U = dY B (fp32)
//
// dX contracts over the weight's rows n, while the codes of a row are
// contiguous along k. A workgroup owns 256 output columns and a range of
// rows, and walks it 32 rows at a time: each thread expands one half block
// (16 code bytes: 32 weights of one row, one scale) into a bf16 [32][256]
// tile in LDS, so a row's 128 code bytes are read by 8 consecutive threads;
// four waves each multiply 64 of the columns with v_mfma_f32_16x16x32_bf16,
// dY (16 token rows, zero past M) as the A operand straight from memory and
// the tile's columns as the B operand through the transposing LDS read
// (ds_read_b64_tr_b16). The next step's codes are in flight while a step is
// expanded and multiplied. Row ranges split the contraction; each writes its
// fp32 partial [16][k] slice, and a second kernel adds the partials in range
// order, adds the low-rank term s (U A) in fp32 (with dropout, multiplied by
// keep where the mask is set and dropped where it is not) and rounds once.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kCols = 256;             // output columns per workgroup
constexpr int kStepRows = 32;          // contraction rows per step
constexpr int kPitch = kCols * 2 + 32;  // bytes per tile row (pad: the 4 rows of a transposing read on distinct banks)

struct DxStage {
  u32x4 q;       // 16 code bytes: 32 weights
  uint32_t c8;
  float s2v;
};

// kVec: dY rows are 16-byte aligned (n % 8 == 0) and read 16 bytes at a time.
// kDirect (one row range covers all n): the workgroup finishes its outputs
// itself -- the low-rank term and the rounding, with the finalize kernel's
// arithmetic -- instead of writing a partial for a second launch.
template <bool kVec, bool kDirect = false>
__global__ __launch_bounds__(256) void gemv_dx_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ code8,
                                                      const float* __restrict__ s2, bool s2_bf16,
                                                      const float* __restrict__ mean_p,
                                                      const float* __restrict__ codebook, int64_t n, int64_t k,
                                                      const uint16_t* __restrict__ dY, int64_t M, int64_t rows_per,
                                                      float* __restrict__ part, const float* __restrict__ U,
                                                      const uint16_t* __restrict__ A, int r, float scale,
                                                      const uint8_t* __restrict__ mask, float keep,
                                                      uint16_t* __restrict__ dX) {
  __shared__ float lut[16];
  __shared__ __attribute__((aligned(16))) char tile0[kStepRows * kPitch];
  __shared__ __attribute__((aligned(16))) char tile1[kStepRows * kPitch];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  if (t < 16) lut[t] = codebook[t];
  const float mean = weight_mean(code8, mean_p);
  const int64_t j0 = (int64_t)blockIdx.x * kCols;
  const int64_t nb = (int64_t)blockIdx.y * rows_per;
  const int64_t ne = nb + rows_per < n ? nb + rows_per : n;
  const int nsteps = (int)cdiv(ne - nb, (int64_t)kStepRows);
  // this thread's half block: row t / 8 of a step, columns 32 (t % 8) .. +31
  const int rr = t >> 3;
  const int64_t jc = j0 + 32 * (t & 7);
  const bool colok = jc < k;
  const int64_t jcl = colok ? jc : k - 32;
  const int64_t kblocks = k / kBlock;
  auto load = [&](int step, DxStage& st) {
    const int64_t row = nb + (int64_t)step * kStepRows + rr;
    const int64_t rc = row < ne ? row : ne - 1;  // clamped: an in-range row
    st.q = *reinterpret_cast<const u32x4*>(codes + rc * (k / 2) + jcl / 2);
    scale_fields(code8, s2, s2_bf16, rc * kblocks + jcl / kBlock, st.c8, st.s2v);
    if (!(row < ne && colok)) st.q = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};  // level 0
  };
  auto expand = [&](const DxStage& st, char* tile) {
    const float cp = decode_block_scale(st.c8, st.s2v, mean);
    char* dst = tile + rr * kPitch + (t & 7) * 64;
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4*>(dst + 16 * w) = dequant8(st.q[w], lut, cp);
  };
  // A operand: token row lane % 16, contraction rows 8 (lane / 16) .. +7 of the step
  const int am = lane & 15;
  const bool mok = am < M;
  const uint16_t* yrow = dY + (mok ? am : 0) * n;
  auto a_operand = [&](int step) {
    const int64_t r0 = nb + (int64_t)step * kStepRows + 8 * (lane >> 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if constexpr (kVec) {
      if (mok && r0 + 8 <= n) v = *reinterpret_cast<const u32x4*>(yrow + r0);
    } else {
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = (mok && r0 + i < n) ? (uint32_t)yrow[r0 + i] : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = e[2 * i] | (e[2 * i + 1] << 16);
    }
    // rows past ne of this range meet zero weights; rows past n are zero here
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  DxStage s0, s1;
  load(0, s0);
  load(nsteps > 1 ? 1 : 0, s1);
  __syncthreads();  // lut
  expand(s0, tile0);
  load(nsteps > 2 ? 2 : nsteps - 1, s0);
  __syncthreads();
  auto step_body = [&](int step, const char* cur, char* nxt, DxStage& stn, DxStage& stl) {
    // stn: step + 1 (landed or in flight) -> nxt; stl: receives step + 3
    bf16x8 a = a_operand(step);
    expand(stn, nxt);
    const int s3 = step + 3 < nsteps ? step + 3 : nsteps - 1;
    load(s3, stn);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 b = tr_rows8(cur, kPitch, 64 * wave + 16 * c, lane);
      acc[c] = mfma16<false>(a, b, acc[c]);
    }
    (void)stl;
    __syncthreads();
  };
  // step s reads tile (s & 1); the expansion of step s + 1 goes to the other
  // tile; stages alternate so the loads of step s + 2 are already in flight
  for (int step = 0; step < nsteps; step += 2) {
    step_body(step, tile0, tile1, s1, s0);
    if (step + 1 < nsteps) step_body(step + 1, tile1, tile0, s0, s1);
  }
  // D layout of v_mfma_f32_16x16x32: lane -> column lane % 16, rows 4 (lane / 16) + v
  if constexpr (kDirect) {
#pragma clang fp contract(off)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t j = j0 + 64 * wave + 16 * c + (lane & 15);
      if (j >= k) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * (lane >> 4) + v;
        if (m >= M) continue;
        float l = 0.0f;
        for (int t = 0; t < r; ++t) l = fmaf(U[m * r + t], bf16_bits_to_f32(A[(int64_t)t * k + j]), l);
        const float f = mask != nullptr ? (mask[m * k + j] ? scale * keep : 0.0f) : scale;
        dX[m * k + j] = to_bf16_bits(acc[c][v] + f * l);
      }
    }
  } else {
    float* p = part + (int64_t)blockIdx.y * 16 * k;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t j = j0 + 64 * wave + 16 * c + (lane & 15);
      if (j >= k) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * (lane >> 4) + v;
        if (m < M) p[(int64_t)m * k + j] = acc[c][v];
      }
    }
  }
}

// dX[m, j] = RN_bf16( sum_p part[p][m][j] + scale * sum_t U[m, t] A[t, j] ),
// partials added in range order, the low-rank sum in t order; with a mask the
// low-rank term is multiplied by keep where mask[m, j] is set and dropped
// where it is not. Four adjacent columns per thread.
__global__ __launch_bounds__(256) void gemv_dx_finalize_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                               int64_t k, const float* __restrict__ U,
                                                               const uint16_t* __restrict__ A, int r, float scale,
                                                               const uint8_t* __restrict__ mask, float keep,
                                                               uint16_t* __restrict__ dX) {
#pragma clang fp contract(off)
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t groups = k / 4;
  if (g >= M * groups) return;
  const int64_t m = g / groups, j = (g % groups) * 4;
  // loads issued eight at a time (clamped to the last valid index, the
  // extra values unused), sums still taken in range / rank order
  float4 s = *reinterpret_cast<const float4*>(part + m * k + j);
  for (int p0 = 1; p0 < splits; p0 += 8) {
    float4 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = p0 + e < splits ? p0 + e : splits - 1;
      v[e] = *reinterpret_cast<const float4*>(part + ((int64_t)p * 16 + m) * k + j);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (p0 + e < splits) {
        s.x += v[e].x; s.y += v[e].y; s.z += v[e].z; s.w += v[e].w;
      }
  }
  float l[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < r; t0 += 8) {
    float u[8];
    uint2 a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + e < r ? t0 + e : r - 1;
      u[e] = U[m * r + t];
      a[e] = *reinterpret_cast<const uint2*>(A + (int64_t)t * k + j);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (t0 + e < r) {
        l[0] = fmaf(u[e], bf16_bits_to_f32(a[e].x & 0xFFFFu), l[0]);
        l[1] = fmaf(u[e], bf16_bits_to_f32(a[e].x >> 16), l[1]);
        l[2] = fmaf(u[e], bf16_bits_to_f32(a[e].y & 0xFFFFu), l[2]);
        l[3] = fmaf(u[e], bf16_bits_to_f32(a[e].y >> 16), l[3]);
      }
  }
  float f[4];
  if (mask != nullptr) {
    const uint32_t mk = *reinterpret_cast<const uint32_t*>(mask + m * k + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = ((mk >> (8 * e)) & 0xFFu) ? scale * keep : 0.0f;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = scale;
  }
  const float o[4] = {s.x + f[0] * l[0], s.y + f[1] * l[1], s.z + f[2] * l[2], s.w + f[3] * l[3]};
  uint2 w;
  w.x = pack_bf16x2(o[0], o[1]);
  w.y = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dX + m * k + j) = w;
}

struct DxSplit {
  int64_t rows_per;
  int splits;
};

// Row ranges: about 512 workgroups in all, at least 128 rows per range (a
// single range, n <= 128, finishes its outputs without the finalize launch;
// making a 1024 x 1024 weight one range to save that launch took 42 instead
// of 15 us: four workgroups walking 1024 rows each).
DxSplit dx_split(int64_t n, int64_t k) {
  const int64_t cg = cdiv(k, (int64_t)kCols);
  int64_t s = cdiv((int64_t)512, cg);
  const int64_t smax = cdiv(n, (int64_t)128);
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  const int64_t rows_per = cdiv(cdiv(n, s), (int64_t)kStepRows) * kStepRows;
  return DxSplit{rows_per, (int)cdiv(n, rows_per)};
}

}  // namespace

size_t gemv_dx_ws_bytes(int64_t n, int64_t k) {
  const DxSplit d = dx_split(n, k);
  return align256((size_t)d.splits * 16 * (size_t)k * 4);
}

hipError_t launch_gemv_dx(const Nf4View& w, const uint16_t* dY, int64_t M, const float* U, const uint16_t* A, int r,
                          float scale, uint16_t* dX, void* ws, hipStream_t stream, const uint8_t* mask, float keep) {
  const DxSplit d = dx_split(w.n, w.k);
  float* part = static_cast<float*>(ws);
  const dim3 grid((unsigned)cdiv(w.k, (int64_t)kCols), (unsigned)d.splits);
  const float* u = r > 0 ? U : nullptr;
#define QLORA_GDX(V, D)                                                                                          \
  gemv_dx_kernel<V, D><<<grid, 256, 0, stream>>>(w.codes, w.code8, w.s2, w.s2_bf16, w.mean, w.codebook, w.n, w.k, \
                                                 dY, M, d.rows_per, part, u, A, u ? r : 0, scale, mask, keep, dX)
  if (d.splits == 1) {
    if (w.n % 8 == 0) QLORA_GDX(true, true); else QLORA_GDX(false, true);
    return hipGetLastError();
  }
  if (w.n % 8 == 0) QLORA_GDX(true, false); else QLORA_GDX(false, false);
#undef QLORA_GDX
  const int64_t groups = M * (w.k / 4);
  gemv_dx_finalize_kernel<<<(unsigned)cdiv(groups, (int64_t)256), 256, 0, stream>>>(
      part, d.splits, M, w.k, r > 0 ? U : nullptr, A, r, scale, mask, keep, dX);
  return hipGetLastError();
}

}  // namespace qlora
