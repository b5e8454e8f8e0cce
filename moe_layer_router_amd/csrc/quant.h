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

}  // namespace moe
