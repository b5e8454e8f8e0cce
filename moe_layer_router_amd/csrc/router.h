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

constexpr int kRouterTokens = 128;   // tokens per router tile
constexpr int kRouterExperts = 64;   // experts per router tile
constexpr int kRouterStages = 3;     // LDS stages (loads run two steps ahead)
// One LDS stage (128 K): router weights [64 experts][256 B], activations
// [128 tokens][128 B (E4M3) or 256 B (BF16)], activation scales [4 waves][64].
constexpr int kRouterW = 0;
constexpr int kRouterX = kRouterW + 64 * 256;
constexpr int kRouterSc = kRouterX + 128 * 256;
constexpr int kRouterStage = kRouterSc + 4 * 256;
constexpr int kRouterLds = kRouterStages * kRouterStage;
// The wide tile (128 experts, E4M3 activations only): weights [128][256 B],
// activations [128][128 B], scales; the same LDS total.
constexpr int kRouterExpertsWide = 128;
template <int AF, int NE>
struct RouterLds {
  static_assert(NE == kRouterExperts || (NE == kRouterExpertsWide && AF == ACT_FP8), "router tile widths");
  static constexpr int kW = 0;
  static constexpr int kX = kW + NE * 256;
  static constexpr int kSc = kX + 128 * ((NE == kRouterExperts) ? 256 : 128);
  static constexpr int kStage = kSc + 4 * 256;
};
static_assert(kRouterStages * RouterLds<ACT_FP8, kRouterExpertsWide>::kStage <= kRouterLds, "wide tile fits");

// Logits of tokens [t0, t0+128) x experts [e0, e0+NE) on 256 threads, over
// the K steps [s0, s1) (128 channels each), written to `out` ([T][E]); the
// bias is added when add_bias (the K slice that starts at channel 0).
//
// The logits are a dense [T, H] x [H, E] product, so the tile runs on 16x16x32
// BF16 MFMAs: E4M3 activations convert exactly to BF16 with the gfx950
// conversion instruction.  Router weights, activations and (E4M3) the per-128
// activation scales are loaded straight into LDS, 128 K per step, two steps
// ahead; each row of 16-byte chunks is stored with chunk c at c ^ (row & 15)
// (c ^ (row & 7) for 128-byte activation rows) so that the 16 rows read by one
// operand fetch fall in distinct banks.  Wave w owns tokens 32w..32w+31 (it
// loads exactly those activation rows and scales itself) and all NE experts:
// 2 x NE/16 accumulator tiles.  The wide tile (NE = 128) halves the router
// weight bytes per flop; it is used where there are enough tiles to fill the
// GPU anyway (E >= 512).  Within a step, lane group g holds K elements
// 32g + 8i .. +7 in MFMA i (the same permutation of K for both operands), so a
// lane reads contiguous bytes.  E4M3: each step's partial sum is scaled by the
// token's scale of that 128-channel block and added to the fp32 logits.
template <int AF, int NE = kRouterExperts>
DEV void router_tile(const RouterArgs& a, int t0, int e0, char* lds, int s0, int s1, float* out, bool add_bias) {
  using L = RouterLds<AF, NE>;
  constexpr int NC = NE / 16;                                // expert subtiles
  constexpr int XB = (AF == ACT_FP8) ? 128 : 256;          // activation bytes per token per step
  constexpr int NW = NE / 16;                                // weight loads per wave per step (1 KB each)
  constexpr int NX = XB * 128 / 1024 / 4;                    // activation loads per wave per step
  constexpr int NS = (AF == ACT_FP8) ? 1 : 0;                // scale loads per wave per step
  constexpr int NLOAD = NW + NX + NS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  const rsrc_t wrs = make_rsrc_u(a.wr, (uint32_t)a.E * (uint32_t)a.H * 2);
  const rsrc_t xrs = make_rsrc_u(a.x, (uint32_t)a.T * (uint32_t)a.H * (XB / 128));
  const rsrc_t srs = make_rsrc_u(a.x_scales, (AF == ACT_FP8) ? (uint32_t)a.T * (uint32_t)(a.H / 128) * 4 : 0u);
  // per-lane global offsets (step 0) of this wave's loads
  uint32_t woff[NW], xoff[NX];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int r = (NE / 4) * w + 4 * j + lane / 16;           // expert row of the tile
    const int c = (lane & 15) ^ (r & 15);                     // logical chunk of physical chunk lane & 15
    woff[j] = (uint32_t)(e0 + r) * (uint32_t)a.H * 2 + c * 16;
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    if (AF == ACT_FP8) {
      const int r = 32 * w + 8 * j + lane / 8;
      const int c = (lane & 7) ^ (r & 7);
      xoff[j] = (uint32_t)(t0 + r) * (uint32_t)a.H + c * 16;
    } else {
      const int r = 32 * w + 4 * j + lane / 16;
      const int c = (lane & 15) ^ (r & 15);
      xoff[j] = (uint32_t)(t0 + r) * (uint32_t)a.H * 2 + c * 16;
    }
  }
  const uint32_t soff = (uint32_t)(t0 + 32 * w + (lane & 31)) * (uint32_t)(a.H / 128) * 4;
  auto issue = [&](int s, int j) __attribute__((always_inline)) {   // load j of step s
    char* st = lds + (s % kRouterStages) * L::kStage;
    if (j < NW) {
      buf_ld16_lds(wrs, st + L::kW + ((NE / 4) * w + 4 * j) * 256, woff[j], uni((uint32_t)s * 256));
    } else if (j < NW + NX) {
      const int jx = j - NW;
      const int rows = (AF == ACT_FP8) ? 8 : 4;
      buf_ld16_lds(xrs, st + L::kX + (32 * w + rows * jx) * XB, xoff[jx], uni((uint32_t)s * 128 * (XB / 128)));
    } else {
      buf_ld4_lds(srs, st + L::kSc + w * 256, soff, uni((uint32_t)s * 4));
    }
  };

  v4f acc[2][NC];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[st][c] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < NLOAD; ++j) issue(s0, j);
#pragma unroll
  for (int j = 0; j < NLOAD; ++j) issue(s0 + 1, j);
  barrier_vmcnt<NLOAD>();

  for (int s = s0; s < s1; ++s) {
    const char* st = lds + (s % kRouterStages) * L::kStage;
    // A operands of both token subtiles
    v8bf av[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = 32 * w + 16 * sub + c16;
      if (AF == ACT_FP8) {
        const v4i q0 = ld16(st + L::kX + row * 128 + (((2 * g) ^ (row & 7)) << 4));
        const v4i q1 = ld16(st + L::kX + row * 128 + (((2 * g + 1) ^ (row & 7)) << 4));
        const int qs[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qs[2 * i], 1.0f, false);
          const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qs[2 * i], 1.0f, true);
          const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qs[2 * i + 1], 1.0f, false);
          const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qs[2 * i + 1], 1.0f, true);
          av[sub][i] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[sub][i] = as_v8bf(ld16(st + L::kX + row * 256 + (((4 * g + i) ^ (row & 15)) << 4)));
      }
    }
    v4f part[2][NC];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = i * NW / 4; j < (i + 1) * NW / 4; ++j) issue(s + 2, j);   // weights of step s+2
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int row = 16 * c + c16;
        const v8bf bv = as_v8bf(ld16(st + L::kW + row * 256 + (((4 * g + i) ^ (row & 15)) << 4)));
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          if (AF == ACT_FP8)
            part[sub][c] = mfma_bf16(av[sub][i], bv, i == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : part[sub][c]);
          else
            acc[sub][c] = mfma_bf16(av[sub][i], bv, acc[sub][c]);
        }
      }
    }
#pragma unroll
    for (int j = NW; j < NLOAD; ++j) issue(s + 2, j);          // activations (and scales) of step s+2
    if (AF == ACT_FP8) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const v4f sc = *reinterpret_cast<const v4f*>(st + L::kSc + w * 256 + (16 * sub + 4 * g) * 4);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[sub][c][v] = __builtin_fmaf(part[sub][c][v], sc[v], acc[sub][c][v]);
      }
    }
    barrier_vmcnt<NLOAD>();
  }
  wait_vmcnt<0>();                                 // loads issued for steps past the end
  __syncthreads();

  // accumulator element v of tile (sub, c): token 32w + 16sub + 4g + v, expert 16c + c16.
  // Write-through buffer stores, with the elements outside [T) x [E) given
  // an offset past the buffer's end, which the hardware drops: stores under
  // a condition would each be a branch with a wait.
  // (the biases are loaded before the first store, which could alias them)
  const rsrc_t ors = make_rsrc_u(out, (uint32_t)a.T * (uint32_t)a.E * 4u);
  float bias[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) bias[c] = (add_bias && a.bias) ? a.bias[min(e0 + 16 * c + c16, a.E - 1)] : 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = e0 + 16 * c + c16;
    const float b = bias[c];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 32 * w + 16 * sub + 4 * g + v;
        const uint32_t off = (t < a.T && e < a.E) ? ((uint32_t)t * (uint32_t)a.E + (uint32_t)e) * 4u : 0xFFFFFFF0u;
        buf_stf<kCoherent>(ors, off, acc[sub][c][v] + b);
      }
  }
}

// Sum of the S channel-slice partials (at a.logits + s*T*E, S <= 8) of
// elements [i0, i1) of the tile (t0, e0) (element i = token i / ne, expert
// i % ne), in slice order, into slice 0.  kB elements per thread and pass,
// consecutive threads on consecutive elements (each load instruction reads
// whole lines); all loads of a pass are in flight together.  The partials
// are read coherently: their writers' stores completed before their counts.
DEV void router_sum_slices(const RouterArgs& a, int t0, int e0, int S, int i0, int i1) {
  const size_t stride = (size_t)a.T * a.E;
  const int ne = min(kRouterExperts, a.E - e0);
  constexpr int kB = 8, kMaxS = 8;
  const int nthr = blockDim.x;
  // write-through buffer stores; an element past i1 gets an offset past the
  // buffer's end, which the hardware drops (a store under a condition would
  // be a branch with a wait)
  const rsrc_t lrs = make_rsrc_u(a.logits, (uint32_t)a.T * (uint32_t)a.E * 4u);
  for (int ib = i0; ib < i1; ib += nthr * kB) {
    float p[kB][kMaxS];
    size_t off[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int i = min(ib + u * nthr + (int)threadIdx.x, i1 - 1);
      off[u] = (size_t)(t0 + i / ne) * a.E + e0 + i % ne;
    }
    // the loads of one slice for all kB elements under one (uniform)
    // condition, before any of them is used
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      if (s < S) {
#pragma unroll
        for (int u = 0; u < kB; ++u) p[u][s] = ld_coh(a.logits + s * stride + off[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      float v = p[u][0];
#pragma unroll
      for (int s = 1; s < kMaxS; ++s)
        if (s < S) v += p[u][s];
      const bool ok = ib + u * nthr + (int)threadIdx.x < i1;
      buf_stf<kCoherent>(lrs, ok ? (uint32_t)off[u] * 4u : 0xFFFFFFF0u, v);
    }
  }
}

// Number of elements of tile (t0, e0).
DEV int router_tile_elems(const RouterArgs& a, int t0, int e0) {
  return min(kRouterTokens, a.T - t0) * min(kRouterExperts, a.E - e0);
}

// With the channels split into S slices, the last of the S tiles of
// (t0, e0) to finish (counted in *tile_cnt) sums the tile's partials.
DEV void router_reduce(const RouterArgs& a, int t0, int e0, int S, int32_t* tile_cnt) {
  __shared__ int s_last;
  wait_stores();                                   // this slice's partials are in memory
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(tile_cnt, 1) == S - 1);
  __syncthreads();
  if (!s_last) return;
  router_sum_slices(a, t0, e0, S, 0, router_tile_elems(a, t0, e0));
}

// Max of a 64-bit key over the 16 lanes of a DPP row (the same four moves as
// row_max16), returned to every lane of the row.
template <int CTRL>
DEV uint64_t dpp_mov64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
DEV uint64_t row_max16_u64(uint64_t v) {
  uint64_t o;
  o = dpp_mov64<0xB1>(v); v = o > v ? o : v;
  o = dpp_mov64<0x4E>(v); v = o > v ? o : v;
  o = dpp_mov64<0x141>(v); v = o > v ? o : v;
  o = dpp_mov64<0x140>(v); v = o > v ? o : v;
  return v;
}
DEV float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// Max of a 64-bit key over the whole wave: row maxima by DPP, then the
// gfx950 lane swaps across row pairs and wave halves.
DEV uint64_t wave_max64(uint64_t v) {
  v = row_max16_u64(v);
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  uint64_t a = ((uint64_t)h16[0] << 32) | l16[0], b = ((uint64_t)h16[1] << 32) | l16[1];
  v = a > b ? a : b;
  lo = (uint32_t)v; hi = (uint32_t)(v >> 32);
  const auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  a = ((uint64_t)h32[0] << 32) | l32[0];
  b = ((uint64_t)h32[1] << 32) | l32[1];
  return a > b ? a : b;
}

// The 16 logits a lane works on, lrow[idx(j)] for j < 16 (every index in
// range), as the sum of the S channel-slice partials at lrow + s*sstride in
// slice order, the same fp32 sum as router_sum_slices (S = 1: the logits
// themselves).  All loads are issued before any is used: coherent loads
// stay in program order with the arithmetic between them, so a sum between
// loads would make each wait for the one before.
template <typename IdxF>
DEV void load_logits16(const float* lrow, int S, size_t sstride, const IdxF& idx, float* v) {
  constexpr int kMaxS = 8;
  float p[kMaxS][16];
#pragma unroll
  for (int s = 0; s < kMaxS; ++s)
    if (s < S)
#pragma unroll
      for (int j = 0; j < 16; ++j) p[s][j] = ld_coh(lrow + s * sstride + idx(j));
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float x = p[0][j];
#pragma unroll
    for (int s = 1; s < kMaxS; ++s)
      if (s < S) x += p[s][j];
    v[j] = x;
  }
}

// Top-k of one token's logits by one wave.  Keys pack the order-preserving
// image of the logit in the high word and (E-1-e) in the low word, so the
// largest key is the largest logit with the lowest index.  E <= 1024, k <= 16.
DEV void topk_token(const float* lrow, int E, int k, int32_t* ids, float* wts, int S, size_t sstride) {
  const int lane = threadIdx.x & 63;
  // All loads first, each from an in-range address, the unused keys
  // cleared afterwards: a load under a condition is a branch that waits for
  // it (see load_logits16).  Lanes whose indices were clamped store nothing.
  float v[16];
  load_logits16(lrow, S, sstride, [&](int i) { return min(lane + 64 * i, E - 1); }, v);
  if (S > 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (lane + 64 * i < E) st_coh(const_cast<float*>(lrow) + lane + 64 * i, v[i]);
  uint64_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)f32_order_key(v[i]) << 32) | (uint32_t)(E - 1 - e)) : 0ull;
  }
  int my_id = 0;
  float my_val = 0.f, top = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max64(best);
      const int e = E - 1 - (int)(uint32_t)best;
      const float val = f32_from_order_key((uint32_t)(best >> 32));
      if (j == 0) top = val;
      if (lane == j) { my_id = e; my_val = val; }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (lane + 64 * i == e) key[i] = 0ull;
    }
  }
  // the k <= 16 selected values sit in lanes 0..k-1 (the first DPP row)
  const float ex = (lane < k) ? expf(my_val - top) : 0.f;
  const float sum = row_sum16(ex);
  if (lane < k) {
    st_coh(ids + lane, my_id);
    st_coh(wts + lane, ex / sum);
  }
}

// Top-k of one token per DPP row (16 lanes), E <= 256, k <= 16: lane i of
// the row holds experts i + 16j.  Same keys and order as topk_token.
DEV void topk_token16(const float* lrow, bool valid, int E, int k, int32_t* ids, float* wts, int S,
                      size_t sstride) {
  const int li = threadIdx.x & 15;
  float v[16];                                     // (loads first: see topk_token)
  load_logits16(lrow, S, sstride, [&](int j) { return min(li + 16 * j, E - 1); }, v);
  if (S > 1 && valid)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (li + 16 * j < E) st_coh(const_cast<float*>(lrow) + li + 16 * j, v[j]);
  uint64_t key[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = li + 16 * j;
    key[j] = (valid && e < E) ? (((uint64_t)f32_order_key(v[j]) << 32) | (uint32_t)(E - 1 - e)) : 0ull;
  }
  int my_id = 0;
  float my_val = 0.f, top = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < k) {
      uint64_t best = key[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) best = key[j] > best ? key[j] : best;
      best = row_max16_u64(best);
      const int e = E - 1 - (int)(uint32_t)best;
      const float val = f32_from_order_key((uint32_t)(best >> 32));
      if (r == 0) top = val;
      if (li == r) { my_id = e; my_val = val; }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (li + 16 * j == e) key[j] = 0ull;
    }
  }
  const float ex = (li < k) ? expf(my_val - top) : 0.f;
  const float sum = row_sum16(ex);
  if (valid && li < k) {
    st_coh(ids + li, my_id);
    st_coh(wts + li, ex / sum);
  }
}

// Top-k for `count` consecutive tokens starting at t0: one token per DPP row
// (16 per workgroup pass) when E <= 256, else one wave per token.  With
// S > 1 the logits are the sums of S channel-slice partials ([S][T][E] from
// `logits`, slice stride sstride = T*E elements, summed in slice order), and
// the sums are stored over slice 0.
DEV void topk_tokens(const float* logits, int E, int k, int t0, int count, int32_t* ids, float* wts, int S = 1,
                     size_t sstride = 0) {

  if (E <= 256) {
    const int rowid = threadIdx.x >> 4, nrows = blockDim.x >> 4;
    for (int i0 = 0; i0 < count; i0 += nrows) {
      const int i = i0 + rowid;
      const bool valid = i < count;
      const int t = t0 + (valid ? i : 0);
      topk_token16(logits + (size_t)t * E, valid, E, k, ids + (size_t)t * k, wts + (size_t)t * k, S, sstride);
    }
    return;
  }
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i = w; i < count; i += nw) {
    const int t = t0 + i;
    topk_token(logits + (size_t)t * E, E, k, ids + (size_t)t * k, wts + (size_t)t * k, S, sstride);
  }
}

}  // namespace moe
