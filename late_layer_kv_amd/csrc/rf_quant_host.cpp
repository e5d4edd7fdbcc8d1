// Host quantizer for the int8 map format.
//
// "RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill",
// section 2.2 ("Size and cost") and section 4.2: int8 codes with one bf16
// scale for each 128-weight block of a row.  Absmax per block: the scale is the bf16
// value (nearest even) of the fp32 value nearest max|a| / 127, and each code is
// a / s rounded to the nearest integer, ties to even, in double precision,
// clipped to [-127, 127].  An all-zero block gets scale 0 and codes 0.
#include <cfenv>
#include <cmath>
#include <cstring>

#include "../../include/rf.h"
#include "rf_error.h"

namespace {

rf_status qfail(rf_status st, const char* msg) {
  rf::set_last_error(msg);
  return st;
}

uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

double bf16_value(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

}  // namespace

extern "C" rf_status rf_map_quantize_q8(const float* a, int32_t d_out, int32_t d_in, int8_t* q, uint16_t* scale) {
  if (!a || !q || !scale) return qfail(RF_E_ARG, "null argument");
  if (d_out < 1 || d_in < 1 || d_in % 128) return qfail(RF_E_SHAPE, "d_out must be >= 1 and d_in a positive multiple of 128");
  const int nb = d_in / 128;
  const size_t n = static_cast<size_t>(d_out) * d_in;
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(a[i])) return qfail(RF_E_ARG, "map holds a non-finite weight");
  const int mode = std::fegetround();
  std::fesetround(FE_TONEAREST);
  for (int o = 0; o < d_out; ++o) {
    for (int b = 0; b < nb; ++b) {
      const float* blk = a + static_cast<size_t>(o) * d_in + static_cast<size_t>(b) * 128;
      int8_t* qb = q + static_cast<size_t>(o) * d_in + static_cast<size_t>(b) * 128;
      float m = 0.0f;
      for (int k = 0; k < 128; ++k) m = std::fmax(m, std::fabs(blk[k]));
      const uint16_t sb = f32_to_bf16_rne(static_cast<float>(static_cast<double>(m) / 127.0));
      scale[static_cast<size_t>(o) * nb + b] = sb;
      const double s = bf16_value(sb);
      for (int k = 0; k < 128; ++k) {
        double r = (s > 0.0) ? std::nearbyint(static_cast<double>(blk[k]) / s) : 0.0;
        r = std::fmin(127.0, std::fmax(-127.0, r));
        qb[k] = static_cast<int8_t>(r);
      }
    }
  }
  std::fesetround(mode);
  return RF_OK;
}
