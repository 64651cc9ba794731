// Offline encoder: blockwise NF4 codes + double quantization of the block
// absmax constants.
//
// Sources: "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev):
// the worked 8-weight block (scale = the block's largest magnitude, every
// weight snapped to the nearest of the 16 levels, half a byte each) and
// "NF4: a 4-bit format matched to weight statistics" (64-weight absmax
// blocks). "QLoRA Explained ..." (gamut.so), "Double Quantization": the block
// constants are quantized again to 8 bits.
//
// Every decision is taken by exact comparisons in fp64 (an fp32 estimate only
// chooses which comparisons to make), so the result does not depend on the
// launch configuration:
//   code  = #{ j : w > mu_j * c_b },   mu_j = (L_j + L_{j+1}) / 2
//   code8 = E4M3 index #{ k : d_b > nu_k * s2 },  nu_k = midpoint of the k-th
//           and (k+1)-th finite E4M3 values in ascending order.
// Both products are exact in fp64 (<= 29 and <= 50 significant bits).
//
// Kernels, in launch order:
//   nf4_codes_kernel   workgroups looping over runs of 256 blocks, 8 lanes per
//                      block: absmax, 64 codes, packed bytes; each run's sum
//   dq_mean_kernel     fp32 mean of all absmax values, equal to the fp64 sum
//                      in order (runs summed in order, each run in order)
//   dq_encode_kernel   one workgroup per run: s2 and the 256 code8 bytes
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

// Eight consecutive weights of the input as fp32 (bf16 widens exactly).
template <bool kBf16>
__device__ __forceinline__ void load8(const void* __restrict__ W, int64_t idx, float (&w)[8]) {
  if constexpr (kBf16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = __uint_as_float(v[i] << 16);
      w[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(W) + idx);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[i] = a[i]; w[4 + i] = b[i]; }
  }
}

// Per-workgroup lookup tables for the code search (built from the codebook
// at kernel start):
//   lut[i]   for x in [(i - 64) / 64, (i - 63) / 64): the number of fp32
//            midpoints below the interval and the one midpoint inside it
//            (+inf if none; midpoints are >= 0.08 apart, intervals 1/64 wide)
//   pair[c]  the exact fp64 midpoints around code c: (mu_{c-1}, mu_c), with
//            -inf / +inf at the ends
//   mid[j]   the 15 exact fp64 midpoints
struct CodeTables {
  uint2 lut[128];
  double2 pair[16];  // (lo, hi)
  double mid[15];
};

__device__ void build_tables(const float* cb, CodeTables& tb) {
  const int t = threadIdx.x;
  if (t < 15) tb.mid[t] = ((double)cb[t] + (double)cb[t + 1]) * 0.5;
  if (t < 16) {
    tb.pair[t].x = t == 0 ? -INFINITY : ((double)cb[t - 1] + (double)cb[t]) * 0.5;
    tb.pair[t].y = t == 15 ? INFINITY : ((double)cb[t] + (double)cb[t + 1]) * 0.5;
  }
  if (t < 128) {
    const float lo = (float)(t - 64) / 64.0f, hi = (float)(t - 63) / 64.0f;
    uint32_t below = 0;
    float inside = INFINITY;
    for (int j = 0; j < 15; ++j) {
      const float mf = (float)(((double)cb[j] + (double)cb[j + 1]) * 0.5);
      if (mf < lo) ++below;
      else if (mf < hi) inside = mf;
    }
    tb.lut[t] = make_uint2(below, __float_as_uint(inside));
  }
}

// codes = #{ j : x > mu_j * c } for the 8 weights a lane holds, packed 4
// bits each. An fp32 estimate of x / c picks each weight's candidate interval
// from the table; two exact fp64 comparisons confirm it. The estimate's error
// is far below the midpoint spacing, so they fail only for degenerate scales
// (an fp32-denormal absmax, whose reciprocal overflows): those weights are
// flagged in *bad for the full count. Written in stages over the 8 weights so
// the table reads of all 8 are in flight together.
__device__ __forceinline__ uint32_t nf4_codes8(const float (&w)[8], float rc, double cd, const CodeTables& tb,
                                               uint32_t* bad) {
  float xf[8];
  uint2 e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xf[i] = w[i] * rc;
    int j = (int)fmaf(xf[i], 64.0f, 64.0f);  // x >= -1: truncation is the floor
    j = j < 0 ? 0 : (j > 127 ? 127 : j);
    e[i] = tb.lut[j];
  }
  double2 pr[8];
  uint32_t est[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    est[i] = e[i].x + (xf[i] > __uint_as_float(e[i].y) ? 1u : 0u);
    pr[i] = tb.pair[est[i]];
  }
  uint32_t word = 0, fail = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double x = (double)w[i];
    const bool ok = (x > pr[i].x * cd) & !(x > pr[i].y * cd);
    word |= est[i] << (4 * i);
    fail |= ok ? 0u : 1u << i;
  }
  *bad = fail;
  return word;
}

__device__ __forceinline__ uint32_t nf4_code_full(float w, double cd, const CodeTables& tb) {
  const double x = (double)w;
  uint32_t code = 0;
#pragma unroll 1
  for (int j = 0; j < 15; ++j) code += (x > tb.mid[j] * cd) ? 1u : 0u;
  return code;
}

// Biased exponent of a block absmax for the exactness test of the mean
// (max(E, 1): denormals share the smallest normal's spacing); 255 = none.
__device__ __forceinline__ int absmax_exp(float m) {
  const int e = (int)((__float_as_uint(m) >> 23) & 0xFF);
  return m == 0.0f ? 255 : (e < 1 ? 1 : e);
}

// Workgroups loop over runs of 256 blocks: 8 lanes per block, 32 blocks per
// pass, the loads of 4 passes issued before any of them is encoded. Writes the packed codes, every
// block's absmax, and for each run the fp64 sum of its absmax values (in any
// order: it is used only when every partial sum is exact, see
// dq_mean_kernel) and the smallest exponent among them.
// kBf16Scale (no double quantization, bf16 block scales): each block's scale
// is c = RN_bf16(absmax), the codes are taken against that c (the value the
// dequant will multiply by), and absmax receives c's bf16 bit patterns
// (uint16 per block) instead of fp32 values. A block whose c is zero stores
// code 7 throughout.
template <bool kBf16, bool kBf16Scale>
__global__ __launch_bounds__(256, 4) void nf4_codes_kernel(const void* __restrict__ W, int64_t nb, int64_t nruns,
                                                        const float* __restrict__ codebook,
                                                        uint32_t* __restrict__ codes,
                                                        float* __restrict__ absmax, double* __restrict__ runsum,
                                                        int* __restrict__ runexp) {
  __shared__ float cb[16];
  __shared__ CodeTables tb;
  __shared__ double wsum[4];
  __shared__ int wexp[4];
  const int t = threadIdx.x;
  if (t < 16) cb[t] = codebook[t];
  __syncthreads();
  build_tables(cb, tb);
  __syncthreads();

  const int sub = t >> 3, part = t & 7, wave = t >> 6;
  constexpr int kPasses = 4;  // passes of 32 blocks whose loads are in flight together
  for (int64_t run = blockIdx.x; run < nruns; run += gridDim.x) {
    double rs = 0.0;
    int re = 255;
#pragma unroll 1
    for (int64_t b0 = run * kDqBlock; b0 < (run + 1) * kDqBlock; b0 += kPasses * 32) {
      float w[kPasses][8];
#pragma unroll
      for (int it = 0; it < kPasses; ++it) {
        const int64_t b = b0 + it * 32 + sub;
        if (b < nb) {
          load8<kBf16>(W, b * kBlock + part * 8, w[it]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) w[it][i] = 0.0f;
        }
      }
#pragma unroll
      for (int it = 0; it < kPasses; ++it) {
        const int64_t b = b0 + it * 32 + sub;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(w[it][i]));
        // max over the 8 lanes of this block (lanes 8-aligned inside the wavefront)
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 8));
        // the scale the codes are taken against
        const float c = kBf16Scale ? bf16_bits_to_f32(to_bf16_bits(m)) : m;
        uint32_t word = 0x77777777u;  // all-zero block (or zero scale): every code is 7
        if (c != 0.0f) {
          const float rc = __builtin_amdgcn_rcpf(c);
          const double cd = (double)c;
          uint32_t bad;
          word = nf4_codes8(w[it], rc, cd, tb, &bad);
          if (bad) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (bad >> i & 1u) word = (word & ~(0xFu << (4 * i))) | nf4_code_full(w[it][i], cd, tb) << (4 * i);
          }
        }
        if (b < nb) {
          codes[b * 8 + part] = word;
          if (part == 0) {
            if constexpr (kBf16Scale)
              reinterpret_cast<uint16_t*>(absmax)[b] = to_bf16_bits(m);
            else
              absmax[b] = m;
            rs += (double)m;
            const int e = absmax_exp(m);
            re = re < e ? re : e;
          }
        }
      }
    }
    // the run's sum and smallest exponent: lanes 0, 8, .., 56 of each wave,
    // then the 4 waves
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
      rs += __shfl_xor(rs, off);
      const int o = __shfl_xor(re, off);
      re = re < o ? re : o;
    }
    if ((t & 63) == 0) {
      wsum[wave] = rs;
      wexp[wave] = re;
    }
    __syncthreads();
    if (t == 0) {
      runsum[run] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
      int e = wexp[0] < wexp[1] ? wexp[0] : wexp[1];
      e = e < wexp[2] ? e : wexp[2];
      runexp[run] = e < wexp[3] ? e : wexp[3];
    }
    __syncthreads();
  }
}

// mean = RN_fp32(S / nb), S the fp64 sum of the run sums in order, each run
// summed in order. Every absmax is a multiple of 2^(emin - 150) (emin: the
// smallest exponent field among them), so when the total stays below
// 2^(emin - 98) every partial sum, in any order, is a multiple of that below
// 2^53 times it: exact, and the ordered sum equals the tree sum of the runs'
// tree sums. Otherwise one thread takes the ordered sums themselves.
__global__ __launch_bounds__(1024) void dq_mean_kernel(const double* __restrict__ runsum,
                                                      const int* __restrict__ runexp, int64_t nruns,
                                                      const float* __restrict__ absmax, int64_t nb,
                                                      float* __restrict__ mean) {
  __shared__ double ssum[1024];
  __shared__ int sexp[1024];
  const int t = threadIdx.x;
  double s = 0.0;
  int e = 255;
  for (int64_t j = t; j < nruns; j += 1024) {
    s += runsum[j];
    e = e < runexp[j] ? e : runexp[j];
  }
  ssum[t] = s;
  sexp[t] = e;
  __syncthreads();
  for (int h = 512; h > 0; h >>= 1) {
    if (t < h) {
      ssum[t] += ssum[t + h];
      sexp[t] = sexp[t] < sexp[t + h] ? sexp[t] : sexp[t + h];
    }
    __syncthreads();
  }
  if (t != 0) return;
  double S = ssum[0];
  const int emin = sexp[0];
  const bool exact = emin == 255 || S < ldexp(1.0, emin - 98);
  if (!exact) {
    S = 0.0;
    for (int64_t j = 0; j < nruns; ++j) {
      const int64_t b1 = (j + 1) * kDqBlock < nb ? (j + 1) * kDqBlock : nb;
      double P = 0.0;
      for (int64_t b = j * kDqBlock; b < b1; ++b) P += (double)absmax[b];  // left to right
      S += P;
    }
  }
  mean[0] = (float)(S / (double)nb);
}

// Ascending index (0..252) of the finite E4M3 values -> bit pattern:
// 0..125 are the negatives from -448 up, 126 is +0, 127..252 the positives.
__device__ __forceinline__ uint32_t e4m3_bits_of_index(int idx) {
  return idx < 126 ? (0x80u | (uint32_t)(126 - idx)) : (uint32_t)(idx - 126);
}

__device__ __forceinline__ double e4m3_value_of_index(int idx) {
  return (double)e4m3_to_f32(e4m3_bits_of_index(idx));
}

__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ absmax, int64_t nb,
                                                        const float* __restrict__ mean_p,
                                                        float* __restrict__ s2_out,
                                                        uint8_t* __restrict__ code8) {
  __shared__ float red[256];
  const int64_t run = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t b = run * kDqBlock + t;
  const float mean = mean_p[0];
  float d = 0.0f;
  if (b < nb) d = absmax[b] - mean;  // one fp32 subtraction
  red[t] = fabsf(d);
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  const float a2 = red[0];
  const float s2 = a2 / 448.0f;  // fp32 division, correctly rounded
  if (t == 0) s2_out[run] = s2;
  if (b >= nb) return;
  uint32_t bits = 0;
  if (s2 != 0.0f) {
    const double x = (double)d;
    const double sc = (double)s2;
    // count of midpoints below x: binary search over the 252 midpoints
    int lo = 0;  // answer in [0, 252]
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1) {
      const int k = lo + step - 1;  // midpoint between values k and k+1
      if (k < 252) {
        const double nu = (e4m3_value_of_index(k) + e4m3_value_of_index(k + 1)) * 0.5;
        if (x > nu * sc) lo += step;
      }
    }
    bits = e4m3_bits_of_index(lo);
  }
  code8[b] = (uint8_t)bits;
}

}  // namespace

hipError_t launch_quantize(const void* W, bool w_bf16, int64_t n, int64_t k, const float* codebook,
                           uint8_t* codes, uint8_t* code8, float* s2, float* mean, void* ws,
                           hipStream_t stream, bool s2_bf16) {
  const int64_t nb = n * k / kBlock;
  const int64_t nruns = cdiv(nb, kDqBlock);
  // without double quantization (code8 NULL) the block absmax values are the
  // stored scales: written straight to s2, and the second level is skipped
  const bool dq = code8 != nullptr;
  float* absmax = dq ? reinterpret_cast<float*>(ws) : s2;
  double* runsum = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) + quantize_ws_absmax_bytes(nb));
  int* runexp = reinterpret_cast<int*>(reinterpret_cast<char*>(runsum) + quantize_ws_runsum_bytes(nb));
  // 4 workgroups per CU of an MI355X, each looping over runs
  const dim3 grid((unsigned)(nruns < 1024 ? nruns : 1024));
  auto* cw = reinterpret_cast<uint32_t*>(codes);
  const bool bs = !dq && s2_bf16;
  if (w_bf16) {
    if (bs)
      nf4_codes_kernel<true, true><<<grid, 256, 0, stream>>>(W, nb, nruns, codebook, cw, absmax, runsum, runexp);
    else
      nf4_codes_kernel<true, false><<<grid, 256, 0, stream>>>(W, nb, nruns, codebook, cw, absmax, runsum, runexp);
  } else {
    if (bs)
      nf4_codes_kernel<false, true><<<grid, 256, 0, stream>>>(W, nb, nruns, codebook, cw, absmax, runsum, runexp);
    else
      nf4_codes_kernel<false, false><<<grid, 256, 0, stream>>>(W, nb, nruns, codebook, cw, absmax, runsum, runexp);
  }
  if (dq) {
    dq_mean_kernel<<<1, 1024, 0, stream>>>(runsum, runexp, nruns, absmax, nb, mean);
    dq_encode_kernel<<<(unsigned)nruns, 256, 0, stream>>>(absmax, nb, mean, s2, code8);
  }
  return hipGetLastError();
}

}  // namespace qlora
