// MXFP8 encoding helpers shared by the forward GEMMs (mxfp8.hip) and the backward
// quantisers and GEMMs (mxfp8_bwd.hip): OCP Microscaling Formats v1.0 E4M3 elements with
// one E8M0 scale per block of 32, the block scale chosen so that no element saturates.
#ifndef LIBMOE_MX_COMMON_H
#define LIBMOE_MX_COMMON_H

#include <math.h>

#include "moe_internal.h"

namespace moe {

typedef uint32_t mx_u32x4_t __attribute__((ext_vector_type(4)));

// fp32 (already divided by its block scale) -> E4M3 code, round to nearest even,
// saturating to +-448 (NaN -> 0x7F).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a != a) return 0x7Fu;
  if (!(a < 448.0f)) return sign | 0x7Eu;
  const uint32_t ua = __float_as_uint(a);
  if (ua < 0x00800000u) return sign;                 // below 2^-126: rounds to zero
  const int e = (int)(ua >> 23) - 127;
  const uint32_t full = (ua & 0x7FFFFFu) | 0x800000u;
  const int shift = e >= -6 ? 20 : 20 + (-6 - e);
  if (shift > 24) return sign;                       // below 2^-10: rounds to zero
  uint32_t keep = full >> shift;
  const uint32_t rem = full & ((1u << shift) - 1u), half = 1u << (shift - 1);
  keep += (rem > half || (rem == half && (keep & 1u))) ? 1u : 0u;
  if (e >= -6) {
    int ef = e + 7;
    if (keep == 16u) {
      ++ef;
      keep = 8u;
    }
    return sign | ((uint32_t)ef << 3) | (keep - 8u);
  }
  return sign | keep;                                // subnormal grid (keep == 8: 2^-6)
}

// E8M0 scale 2^se of one MX block whose largest magnitude is amax: the smallest power of
// two X with amax / X <= 448, the largest E4M3 value, so that no element of the block
// saturates.  (The conversion OCP MX v1.0 suggests, X = 2^(floor(log2 amax) - 8), leaves
// amax / X in [256, 512) and clamps a block's largest elements to 448 whenever amax / X
// exceeds 448; both give the same X otherwise.)  All-zero blocks get code 0 (2^-127),
// non-finite ones code 255 (NaN).
__device__ __forceinline__ void mx_block_scale(float amax, int& se, uint32_t& scode) {
  if (amax == 0.0f) {
    se = -127;
    scode = 0;
  } else if (!(amax <= 3.0e38f)) {
    se = 0;
    scode = 255;
  } else {
    int e = ilogbf(amax) - 8;
    if (ldexpf(amax, -e) > 448.0f) ++e;   // exact: a power-of-two scaling
    se = min(max(e, -127), 127);
    scode = (uint32_t)(se + 127);
  }
}

// Requantise one row's 32-feature MX block (this value and the 31 other lanes of the
// half wavefront) and store its code and the block's scale (mx_block_scale).
__device__ __forceinline__ void mx_store_h(float h, bool live, uint8_t* code, uint8_t* scale,
                                           bool first) {
  float amax = fabsf(h);
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int se;
  uint32_t scode;
  mx_block_scale(amax, se, scode);
  if (live) {
    *code = (uint8_t)e4m3_rne_sat(ldexpf(h, -se));
    if (first) *scale = (uint8_t)scode;
  }
}

// Requantise one MX block (32 consecutive fp32 features of a row, at `src` in LDS, read
// by one lane) and store its 32 codes (two 16-byte stores) and its scale.  Same scale
// rule (mx_block_scale) and encoding as mx_store_h.  Two passes over LDS (the block's
// amax, then the codes) keep few values live.
__device__ __forceinline__ void mx_store_block(const uint8_t* src, uint8_t* code, uint8_t* scale) {
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float4 t = *(const float4*)(src + 16 * c);
    amax = fmaxf(fmaxf(amax, fmaxf(fabsf(t.x), fabsf(t.y))), fmaxf(fabsf(t.z), fabsf(t.w)));
  }
  int se;
  uint32_t scode;
  mx_block_scale(amax, se, scode);
  // v_cvt_pk_fp8_f32 rounds to nearest even onto the OCP E4M3 grid; with its input
  // clamped to +-448 it equals e4m3_rne_sat (checked on every rounding boundary of
  // every binade from 2^-20 to 2^10, the subnormal grid, +-0 and the infinities), and
  // NaN is kept as 0x7F explicitly
  mx_u32x4_t w[2];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float4 t = *(const float4*)(src + 16 * c);
    const float v[4] = {ldexpf(t.x, -se), ldexpf(t.y, -se), ldexpf(t.z, -se), ldexpf(t.w, -se)};
    int d = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v[0], -448.0f), 448.0f),
                                            fminf(fmaxf(v[1], -448.0f), 448.0f), 0, false);
    d = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v[2], -448.0f), 448.0f),
                                        fminf(fmaxf(v[3], -448.0f), 448.0f), d, true);
    uint32_t du = (uint32_t)d;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (v[b] != v[b]) du = (du & ~(0xFFu << (8 * b))) | (0x7Fu << (8 * b));
    w[c >> 2][c & 3] = du;
  }
  *(mx_u32x4_t*)code = w[0];
  *(mx_u32x4_t*)(code + 16) = w[1];
  *scale = (uint8_t)scode;
}

// Four fp32 values already divided by their block scale -> four E4M3 codes packed into
// one word (value i in byte i), as mx_store_block encodes them.
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.0f), 448.0f), fminf(fmaxf(b, -448.0f), 448.0f), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -448.0f), 448.0f), fminf(fmaxf(d, -448.0f), 448.0f), w, true);
  uint32_t u = (uint32_t)w;
  const float v[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (v[i] != v[i]) u = (u & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i));
  return u;
}

// Value of an E4M3 code (finite codes; 0x7F / 0xFF decode to NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e == 0 ? (float)m * 0x1p-9f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  return (c & 0x80u) ? -v : v;
}

// Exact-input versions for values held in float64: the block scale of mx_block_scale and
// the nearest-even E4M3 code of v / X (|v / X| <= 448 by that scale).
__device__ __forceinline__ void mx_block_scale_f64(double amax, int& se, uint32_t& scode) {
  if (amax == 0.0) {
    se = -127;
    scode = 0;
  } else if (!(amax <= 3.0e38)) {
    se = 0;
    scode = 255;
  } else {
    int e = ilogb(amax) - 8;
    if (ldexp(amax, -e) > 448.0) ++e;
    se = min(max(e, -127), 127);
    scode = (uint32_t)(se + 127);
  }
}
__device__ __forceinline__ uint32_t e4m3_rne_f64(double v) {
  const uint32_t sign = signbit(v) ? 0x80u : 0u;
  const double a = fabs(v);
  if (a != a) return 0x7Fu;
  if (!(a < 448.0)) return sign | 0x7Eu;
  if (a == 0.0) return sign;
  int ee = ilogb(a);
  if (ee < -6) ee = -6;                                  // subnormal grid below 2^-6
  uint32_t m = (uint32_t)rint(ldexp(a, 3 - ee));         // steps of 2^(ee - 3), ties to even
  if (ee == -6 && m < 8) return sign | m;                // subnormal (or zero)
  if (m == 16) {
    ++ee;
    m = 8;
  }
  return sign | ((uint32_t)(ee + 7) << 3) | (m - 8);
}

}  // namespace moe

#endif  // LIBMOE_MX_COMMON_H
