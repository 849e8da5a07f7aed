// Shared device/host helpers of the SemKV HIP library (gfx950).
//
// Row format (SemKV page, Table 6 fixes only the code-bit rates; the layout
// is ours): g base-L codes per b-bit field, field value sum_i code[g*j+i]*L^i,
// fields LSB-first in a little-endian bit stream, R = ceil(ceil(128/g)*b/8)
// bytes per 128-value row.  Meta = {scale, min} as two fp16 per row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace semkv {

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 8;   // query heads per KV head supported by decode

struct RowFmt {
  int32_t L;   // level count
  int32_t g;   // codes per field
  int32_t b;   // bits per field
  int32_t R;   // packed bytes per row
};

__host__ __device__ inline RowFmt row_fmt(int32_t L) {
  RowFmt f;
  f.L = L;
  switch (L) {
    case 3: f.g = 5; f.b = 8; break;     // 3^5 = 243 <= 256
    case 4: f.g = 4; f.b = 8; break;     // plain 2-bit codes
    case 5: f.g = 3; f.b = 7; break;     // 5^3 = 125 <= 128
    case 6: f.g = 3; f.b = 8; break;     // 6^3 = 216 <= 256
    case 8: f.g = 1; f.b = 3; break;
    case 16: f.g = 2; f.b = 8; break;    // nibbles
    case 65536: f.g = 1; f.b = 16; break;
    default: {
      int b = 0;
      while ((1 << b) < L) ++b;
      f.g = 1;
      f.b = b;
    }
  }
  const int nf = (kHeadDim + f.g - 1) / f.g;
  f.R = (nf * f.b + 7) / 8;
  return f;
}

// ---- fp16 bit helpers (exact conversions; f32 -> f16 rounds to nearest even)
__device__ __forceinline__ float h2f(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Smallest fp16 >= (hi - lo) / (L - 1), as bits; 0 when hi == lo.
// d = hi - lo is exact in double (float operands), and so is f * (L - 1) for
// an fp16 f, so the ceiling is settled by exact comparisons of those
// products with d, starting from the fp16 nearest the quotient.
__device__ inline uint16_t scale_ceil_bits(float lo, float hi, int L) {
  const double d = (double)hi - (double)lo;
  const double lm = (double)(L - 1);
  if (!(d > 0.0)) return 0;
  uint16_t h = f2h((float)(d / lm));
  while ((double)h2f(h) * lm < d) ++h;                     // next fp16 up (d > 0)
  while (h > 1 && (double)h2f((uint16_t)(h - 1)) * lm >= d) --h;
  return h;
}

// Largest fp16 <= v, as a float (v within the fp16 range).
__device__ inline float fp16_floor(float v) {
  uint16_t h = f2h(v);                                     // nearest
  if (h2f(h) > v) h = (h & 0x8000u) ? (uint16_t)(h + 1)   // negative: away from zero
                      : (h == 0 ? (uint16_t)0x8001u : (uint16_t)(h - 1));
  return h2f(h);
}

}  // namespace semkv
