// ln(beta) correctly rounded to float32, shared by the kernels that store
// it (the prefill planes, the per-step append, and the append folded into
// the selection's first kernel), so every path stores the same bits.
// TRIM-KV page, section 2: beta is produced once, when the token is created.
#pragma once
#include "common.h"
#include "ln_table.h"

namespace trimkv {

// ln(x) correctly rounded to float32 for x in [0, 1].
// A float64 log (error far below 8 float64 ulps) rounds to the correct
// float32 unless the true value lies close to a float32 rounding midpoint;
// those few inputs (ln within 40 float64 ulps of a midpoint) are listed in
// ln_table.h with their correctly rounded logarithm.  The check below flags
// every input whose float64 log lies within |y| * 2^-48 (16..32 ulps) of a
// midpoint, which covers every listed input and nothing that could round
// wrongly otherwise.
__device__ __forceinline__ float ln_f32_cr(float x) {
  double y = log((double)x);
  float f = (float)y;
  if (!(y < 0.0) || isinf(y)) return f;  // x == 1 -> +0, x == 0 -> -inf
  uint32_t fb = __float_as_uint(f);      // f < 0
  double fd = (double)f;
  double toward0 = (double)__uint_as_float(fb - 1u);
  double away = (double)__uint_as_float(fb + 1u);
  double thr = fabs(y) * 0x1p-48;
  if (fabs(y - 0.5 * (fd + toward0)) < thr || fabs(y - 0.5 * (fd + away)) < thr) {
    uint32_t xb = __float_as_uint(x);
    int lo = 0, hi = TRIMKV_LN_TABLE_N;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (kLnHardIn[mid] < xb) lo = mid + 1; else hi = mid;
    }
    if (lo < TRIMKV_LN_TABLE_N && kLnHardIn[lo] == xb) return __uint_as_float(kLnHardOut[lo]);
  }
  return f;
}

}  // namespace trimkv
