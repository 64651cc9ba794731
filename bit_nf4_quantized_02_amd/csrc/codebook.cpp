// NF4 codebook, host side.
//
// The levels are standard-normal quantiles rescaled to [-1, 1] with an exact
// zero ("QLoRA Explained ..." (gamut.so), "4-Bit NormalFloat (NF4)
// Quantization"; "QLoRA: Quantized Low-Rank Adaptation"
// (completesystemdesign.dev), "NF4: a 4-bit format matched to weight
// statistics"). Construction: 8 positive quantiles at evenly spaced
// probabilities in (1/2, delta], 7 negative ones mirrored from evenly spaced
// probabilities in (1/2, delta], one zero; every level divided by the quantile
// of delta = ((1 - 1/30) + (1 - 1/32)) / 2; fp64 throughout, one final
// rounding to fp32.
//
// The inverse normal CDF is solved numerically: bisection on
// Phi(x) = erfc(-x / sqrt 2) / 2 (C library erfc) to bracket the root, then
// Newton's method x <- x - (Phi(x) - p) / phi(x) to full double precision.
// Each level lies several hundredths of an fp32 ulp away from an fp32
// rounding boundary, so any quantile with relative error below 1e-9 yields
// the same table.
#include <cmath>

#include "qlora.h"

namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int i = 0; i < 40; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int i = 0; i < 4; ++i) x -= (normal_cdf(x) - p) / normal_pdf(x);
  return x;
}

}  // namespace

extern "C" qlora_status qlora_build_uniform4_codebook(float* levels_out) {
  if (levels_out == nullptr) return QLORA_ERR_INVALID_ARG;
  // (i - 7) / 7: both operands exact in fp32, the division rounded once
  for (int i = 0; i < 16; ++i) levels_out[i] = (float)(i - 7) / 7.0f;
  return QLORA_OK;
}

extern "C" qlora_status qlora_build_nf4_codebook(float* levels_out) {
  if (levels_out == nullptr) return QLORA_ERR_INVALID_ARG;
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  const double top = normal_quantile(delta);
  double lv[16];
  // ascending: 7 negative (largest magnitude first), zero, 8 positive
  for (int j = 7; j >= 1; --j) lv[7 - j] = -normal_quantile(0.5 + (j / 7.0) * (delta - 0.5)) / top;
  lv[7] = 0.0;
  for (int j = 1; j <= 8; ++j) lv[7 + j] = normal_quantile(0.5 + (j / 8.0) * (delta - 0.5)) / top;
  for (int i = 0; i < 16; ++i) levels_out[i] = (float)lv[i];
  return QLORA_OK;
}
