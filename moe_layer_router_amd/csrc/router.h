// Gating: router logits and top-k selection with renormalised softmax weights.
//
// Gating is "top-k expert selection and scoring" (youleyou, "DeepSeek 模型更新
// 解读 Tile Kernels 与 DeepEP V2 新特性", section "Tile Kernels", gating bullet).
// The score is a softmax over the logits; the k selected weights are the
// softmax restricted to the selection, which equals the full softmax
// renormalised over it.  Experts are ranked by logit descending, equal logits
// going to the lower expert index.
#pragma once
#include "device_common.h"

namespace moe {

struct RouterArgs {
  const uint8_t* x;        // [T][H] E4M3 bytes, or BF16 (2 bytes per element)
  const float* x_scales;   // [T][H/128] (FP8 activations) or nullptr
  const uint16_t* wr;      // [E][H] BF16
  const float* bias;       // [E] or nullptr
  float* logits;           // [T][E]
  int T, H, E;
  int act_fp8;
};

constexpr int kRouterTokens = 64;    // tokens per router tile
constexpr int kRouterExperts = 64;   // experts per router tile
constexpr int kRouterLds = 2 * 64 * 256;

// Logits of tokens [t0, t0+64) x experts [e0, e0+64) on 256 threads.
//
// Both operands go through LDS as BF16 (E4M3 -> BF16 is exact), 128 K per
// step.  Each 256-byte LDS row holds 16 chunks of 8 BF16; chunk c of row r
// sits at position c ^ (r & 15) so that the 16 rows read by one MFMA operand
// fetch hit distinct banks.  Wave w owns tokens 16w..16w+15 and all 64
// experts (four 16x16 accumulators).  MFMA i of a step takes K elements
// 32*g + 8*i .. +7 in lane group g for both operands, so each lane reads
// whole 16-byte chunks.  For FP8 activations the per-128 scale multiplies
// each step's partial sum (fp32), as the scale changes every 128 channels.
DEV void router_tile(const RouterArgs& a, int t0, int e0, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  char* xs = lds;
  char* ws = lds + 64 * 256;
  const int nsteps = a.H / 128;

  const int lrow = tid >> 2, lpart = tid & 3;
  const int ltok = t0 + lrow, lexp = e0 + lrow;
  const bool tok_ok = ltok < a.T, exp_ok = lexp < a.E;

  v4i xr[4], wrr[4];
  auto load = [&](int s) __attribute__((always_inline)) {
    if (a.act_fp8) {
      const uint8_t* p = a.x + (size_t)ltok * a.H + s * 128 + lpart * 32;
      xr[0] = tok_ok ? ld16(p) : v4i{0, 0, 0, 0};
      xr[1] = tok_ok ? ld16(p + 16) : v4i{0, 0, 0, 0};
    } else {
      const uint8_t* p = a.x + ((size_t)ltok * a.H + s * 128 + lpart * 32) * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = tok_ok ? ld16(p + 16 * i) : v4i{0, 0, 0, 0};
    }
    const uint8_t* q = reinterpret_cast<const uint8_t*>(a.wr) + ((size_t)lexp * a.H + s * 128 + lpart * 32) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) wrr[i] = exp_ok ? ld16(q + 16 * i) : v4i{0, 0, 0, 0};
  };
  auto store = [&]() __attribute__((always_inline)) {
    const int sw = lrow & 15;
    if (a.act_fp8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t l0, h0, l1, h1;
        e4m3x4_to_bf16x4((uint32_t)xr[i][0], l0, h0);
        e4m3x4_to_bf16x4((uint32_t)xr[i][1], l1, h1);
        st16(xs + lrow * 256 + (((lpart * 4 + 2 * i) ^ sw) << 4), v4i{(int)l0, (int)h0, (int)l1, (int)h1});
        e4m3x4_to_bf16x4((uint32_t)xr[i][2], l0, h0);
        e4m3x4_to_bf16x4((uint32_t)xr[i][3], l1, h1);
        st16(xs + lrow * 256 + (((lpart * 4 + 2 * i + 1) ^ sw) << 4), v4i{(int)l0, (int)h0, (int)l1, (int)h1});
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) st16(xs + lrow * 256 + (((lpart * 4 + i) ^ sw) << 4), xr[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(ws + lrow * 256 + (((lpart * 4 + i) ^ sw) << 4), wrr[i]);
  };

  v4f acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();          // previous step's LDS reads are done
    store();
    __syncthreads();
    if (s + 1 < nsteps) load(s + 1);
    float sc[4] = {1.f, 1.f, 1.f, 1.f};
    if (a.act_fp8) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 16 * w + 4 * g + v;
        sc[v] = (t < a.T) ? a.x_scales[(size_t)t * (a.H / 128) + s] : 0.f;
      }
    }
    v4f part[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) part[c] = a.act_fp8 ? v4f{0.f, 0.f, 0.f, 0.f} : acc[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = (g * 4 + i) ^ c16;
      const v8bf av = as_v8bf(*reinterpret_cast<const v4i*>(xs + (16 * w + c16) * 256 + (chunk << 4)));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const v8bf bv = as_v8bf(*reinterpret_cast<const v4i*>(ws + (16 * c + c16) * 256 + (chunk << 4)));
        part[c] = mfma_bf16(av, bv, part[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (a.act_fp8) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][v] += part[c][v] * sc[v];
      } else {
        acc[c] = part[c];
      }
    }
  }

  // accumulator element v of tile c: token row 4g+v, expert column c16
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = e0 + 16 * c + c16;
    if (e >= a.E) continue;
    const float b = a.bias ? a.bias[e] : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 16 * w + 4 * g + v;
      if (t < a.T) a.logits[(size_t)t * a.E + e] = acc[c][v] + b;
    }
  }
}

// Top-k of one token's logits by one wave.  Keys pack the order-preserving
// image of the logit in the high word and (E-1-e) in the low word, so the
// largest key is the largest logit with the lowest index.  E <= 1024, k <= 16.
DEV void topk_token(const float* lrow, int E, int k, int32_t* ids, float* wts) {
  const int lane = threadIdx.x & 63;
  uint64_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)f32_order_key(lrow[e]) << 32) | (uint32_t)(E - 1 - e)) : 0ull;
  }
  int my_id = 0;
  float my_val = 0.f, top = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = E - 1 - (int)(uint32_t)best;
      const float val = f32_from_order_key((uint32_t)(best >> 32));
      if (j == 0) top = val;
      if (lane == j) { my_id = e; my_val = val; }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (lane + 64 * i == e) key[i] = 0ull;
    }
  }
  float ex = (lane < k) ? expf(my_val - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) sum += __shfl_xor(sum, m);
  sum = __shfl(sum, 0);
  if (lane < k) {
    ids[lane] = my_id;
    wts[lane] = ex / sum;
  }
}

// Top-k for `count` consecutive tokens starting at t0, one wave per token in turn.
DEV void topk_tokens(const float* logits, int E, int k, int t0, int count, int32_t* ids, float* wts) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i = w; i < count; i += nw) {
    const int t = t0 + i;
    topk_token(logits + (size_t)t * E, E, k, ids + (size_t)t * k, wts + (size_t)t * k);
  }
}

}  // namespace moe
