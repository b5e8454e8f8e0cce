// Per-token FP8 quantisation of activations (the quantisation bullet of the
// "Tile Kernels" section of youleyou, "DeepSeek 模型更新解读 Tile Kernels 与
// DeepEP V2 新特性": per-token FP8 quantisation), the step in front of the
// router when the layer receives BF16 activations.
//
// For each token and 128-channel block: amax = max |x|; the scale is
// s = fl32(amax / 448) (a zero block gets 1), or the smallest power of two
// with 448 s >= amax (clamped to 2^-127 .. 2^127, an E8M0 number); codes
// are the E4M3 round-to-nearest-even, saturating, of x * fl32(1 / s) (with a
// power-of-two scale the product is exact).  The E4M3 conversion is the
// one the GEMM epilogue's re-quantisation uses.
//
// Mapping: 16 lanes (one DPP row) per block, 8 channels per lane (one
// 16-byte BF16 load, or two fp32 loads); the block maximum is a DPP row max.
// HBM-bound: 2 (or 4) bytes read and 1 written per element.
#pragma once
#include "device_common.h"

namespace moe {

enum { QIN_BF16 = 0, QIN_F32 = 1 };

// Scale of a block with maximum amax (>= 0), and the multiplier its values
// are scaled by: (s, fl32(1/s)) or (2^e, 2^-e).  Integer arithmetic for the
// power-of-two exponent: amax = 1.f * 2^(E-127) gives e = E - 135 + (f > 0.75)
// (448 = 1.75 * 2^8), exact for every fp32 amax, then clamped.
DEV void block_scale(float amax, bool pow2, float* s, float* inv) {
  if (!(amax > 0.f)) {
    *s = 1.f;
    *inv = 1.f;
    return;
  }
  if (!pow2) {
    const float sc = amax / 448.0f;          // correctly rounded
    *s = sc;
    *inv = 1.0f / sc;                         // correctly rounded
    return;
  }
  const uint32_t u = __float_as_uint(amax);
  const int E = (int)(u >> 23), frac = (int)(u & 0x7FFFFFu);
  int e = (E == 0) ? -127 : E - 135 + (frac > 0x600000 ? 1 : 0);
  e = max(-127, min(127, e));
  // 2^e and 2^-e as fp32 (2^-127 is the subnormal 0x00400000)
  auto pow2f = [](int k) -> float {
    return __uint_as_float(k >= -126 ? (uint32_t)(k + 127) << 23 : 0x00400000u);
  };
  *s = pow2f(e);
  *inv = pow2f(-e);
}

// Quantise 128-channel blocks [b0, b1) of x ([T][H], b = t * H/128 + c/128)
// with `nthreads` threads of the calling group (a multiple of 64, 16 per
// block per pass).  xq [T][H] E4M3 bytes, xs [T][H/128] fp32 scales, stored
// with cache policy CP (kCoherent: written through, for readers on other
// XCDs inside the same kernel).
template <int IN, int CP = 0>
DEV void quant_blocks(const void* x, int T, int H, int b0, int b1, bool pow2, uint8_t* xq, float* xs, int tid,
                      int nthreads) {
  const int nb = H / 128;
  const rsrc_t qrs = make_rsrc_u(xq, (uint32_t)T * (uint32_t)H);
  const rsrc_t srs = make_rsrc_u(xs, (uint32_t)T * (uint32_t)nb * 4u);
  const int li = tid & 15;
  for (int b = b0 + tid / 16; b < b1; b += nthreads / 16) {
    const int t = b / nb, c = (b % nb) * 128 + li * 8;
    const size_t e0 = (size_t)t * H + c;
    float v[8];
    if (IN == QIN_BF16) {
      const v4i q = ld16(reinterpret_cast<const uint16_t*>(x) + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint32_t)q[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32((uint32_t)q[i] >> 16);
      }
    } else {
      const v4i q0 = ld16(reinterpret_cast<const float*>(x) + e0);
      const v4i q1 = ld16(reinterpret_cast<const float*>(x) + e0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = __int_as_float(q0[i]);
        v[4 + i] = __int_as_float(q1[i]);
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
    mx = row_max16(mx);
    float s, inv;
    block_scale(mx, pow2, &s, &inv);
    const uint32_t lo = f32x4_to_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = f32x4_to_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    buf_st8<CP>(qrs, (uint32_t)e0, v2u{lo, hi});
    if (li == 0) buf_stf<CP>(srs, (uint32_t)(t * nb + c / 128) * 4u, s);
  }
}

// ------------------------------------------------------------------ E5M6
// The third format of the same quantisation bullet, read as the
// IEEE-754-style binary format with 1 sign, 5 exponent (bias 15) and 6
// fraction bits (subnormals at exponent 0, exponent 31 reserved), largest
// finite 65024; 12-bit codes, two to three bytes, little-endian (the 8
// codes of a lane are one 96-bit little-endian word).  Per token and
// 128-channel block as above with 65024 in place of 448.  No matrix-core
// instruction takes E5M6: it is a storage format (every value is exactly a
// BF16 and an fp32 number), converted here in both directions.

// Scale of a block for E5M6: (fl32(amax / 65024), fl32(1/s)), or the
// smallest power of two with 65024 s >= amax (65024 = 1.984375 * 2^15:
// e = E - 142 + (fraction > 0.984375), clamped) and its inverse.
DEV void block_scale_e5m6(float amax, bool pow2, float* s, float* inv) {
  if (!(amax > 0.f)) {
    *s = 1.f;
    *inv = 1.f;
    return;
  }
  if (!pow2) {
    const float sc = amax / 65024.0f;        // correctly rounded
    *s = sc;
    *inv = 1.0f / sc;
    return;
  }
  const uint32_t u = __float_as_uint(amax);
  const int E = (int)(u >> 23), frac = (int)(u & 0x7FFFFFu);
  int e = (E == 0) ? -127 : E - 142 + (frac > 0x7E0000 ? 1 : 0);
  e = max(-127, min(127, e));
  auto pow2f = [](int k) -> float {
    return __uint_as_float(k >= -126 ? (uint32_t)(k + 127) << 23 : 0x00400000u);
  };
  *s = pow2f(e);
  *inv = pow2f(-e);
}

// fp32 (finite) -> E5M6 code, round to nearest even, saturating to 65024.
// Normal range (|v| >= 2^-14): the top 6 fraction bits, rounded on the 17
// dropped ones (a carry into the exponent is the next code up).  Below it:
// the multiple of 2^-20 nearest |v| (|v| * 2^20 is exact; rint rounds half
// to even).
DEV uint32_t f32_to_e5m6(float v) {
  const uint32_t u = __float_as_uint(v), sign = (u >> 20) & 0x800u, a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x38800000u) {                     // 2^-14
    const uint32_t E = a >> 23, frac = a & 0x7FFFFFu;
    code = ((E - 112u) << 6) | (frac >> 17);
    const uint32_t rem = frac & 0x1FFFFu;
    code += (rem > 0x10000u || (rem == 0x10000u && (code & 1u))) ? 1u : 0u;
    code = min(code, 0x7BFu);                 // also every fp32 exponent past 2^15
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 1048576.0f);   // 0 .. 64
  }
  return code | sign;
}

// E5M6 code -> fp32 (exact).
DEV float e5m6_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x800u) << 20, exp = (c >> 6) & 0x1Fu, man = c & 0x3Fu;
  if (exp == 0) return __uint_as_float(__float_as_uint((float)man * 9.5367431640625e-07f) | sign);   // m * 2^-20
  if (exp == 31) return __uint_as_float(sign | 0x7F800000u | (man << 17));
  return __uint_as_float(sign | ((exp + 112u) << 23) | (man << 17));
}

typedef int v3i __attribute__((ext_vector_type(3)));

// Quantise 128-channel blocks [b0, b1) of x ([T][H]) to E5M6: xq [T][3H/2]
// bytes, xs [T][H/128] fp32 scales; 16 lanes per block, 8 channels (12
// bytes of codes) per lane.
template <int IN>
DEV void quant_blocks_e5m6(const void* x, int T, int H, int b0, int b1, bool pow2, uint8_t* xq, float* xs, int tid,
                           int nthreads) {
  const int nb = H / 128;
  const int li = tid & 15;
  for (int b = b0 + tid / 16; b < b1; b += nthreads / 16) {
    const int t = b / nb, c = (b % nb) * 128 + li * 8;
    const size_t e0 = (size_t)t * H + c;
    float v[8];
    if (IN == QIN_BF16) {
      const v4i q = ld16(reinterpret_cast<const uint16_t*>(x) + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint32_t)q[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32((uint32_t)q[i] >> 16);
      }
    } else {
      const v4i q0 = ld16(reinterpret_cast<const float*>(x) + e0);
      const v4i q1 = ld16(reinterpret_cast<const float*>(x) + e0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = __int_as_float(q0[i]);
        v[4 + i] = __int_as_float(q1[i]);
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
    mx = row_max16(mx);
    float s, inv;
    block_scale_e5m6(mx, pow2, &s, &inv);
    uint32_t k[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = f32_to_e5m6(v[i] * inv);
    v3i w;
    w[0] = (int)(k[0] | (k[1] << 12) | (k[2] << 24));
    w[1] = (int)((k[2] >> 8) | (k[3] << 4) | (k[4] << 16) | (k[5] << 28));
    w[2] = (int)((k[5] >> 4) | (k[6] << 8) | (k[7] << 20));
    *reinterpret_cast<v3i*>(xq + e0 / 2 * 3) = w;
    if (li == 0) xs[t * nb + c / 128] = s;
  }
}

// out [T][H] fp32 = fl32(value(code) * s) of E5M6 codes xq [T][3H/2] with
// scales xs [T][H/128]; 8 channels per thread.
DEV void dequant_e5m6(const uint8_t* xq, const float* xs, int T, int H, size_t i8, float* out) {
  const size_t e0 = i8 * 8;
  if (e0 >= (size_t)T * H) return;
  const v3i w = *reinterpret_cast<const v3i*>(xq + e0 / 2 * 3);
  const uint32_t w0 = (uint32_t)w[0], w1 = (uint32_t)w[1], w2 = (uint32_t)w[2];
  const uint32_t k[8] = {w0 & 0xFFFu,         (w0 >> 12) & 0xFFFu, (w0 >> 24) | ((w1 & 0xFu) << 8),
                         (w1 >> 4) & 0xFFFu,  (w1 >> 16) & 0xFFFu, (w1 >> 28) | ((w2 & 0xFFu) << 4),
                         (w2 >> 8) & 0xFFFu,  w2 >> 20};
  const float s = xs[e0 / 128];               // row t, block c: (t * H + c) / 128 = t * H/128 + c/128
  v4f o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = e5m6_to_f32(k[i]) * s;
    o1[i] = e5m6_to_f32(k[4 + i]) * s;
  }
  *reinterpret_cast<v4f*>(out + e0) = o0;
  *reinterpret_cast<v4f*>(out + e0 + 4) = o1;
}

}  // namespace moe
