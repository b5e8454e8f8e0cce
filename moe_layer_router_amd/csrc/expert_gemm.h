// Grouped expert GEMMs on gfx950 MFMA, with their fused epilogues.
//
// Linear 1 (gate|up), SwiGLU, linear 2 (down) and the per-token combine are
// the expert half of the MoE block (机器之心, "DeepSeek悄悄更新：Mega MoE、FP4
// Indexer来了", section "Mega MoE 是什么？"); FP8 x FP4 mixed precision is named
// in the same section; quantisation fused with SwiGLU is the quantisation
// bullet of the "Tile Kernels" section of youleyou, "DeepSeek 模型更新解读 Tile
// Kernels 与 DeepEP V2 新特性".
//
// One work item is a row tile of one expert (up to 128 permuted rows) times
// one N block:
//   stage 1: 128 intermediate channels c0..c0+127, i.e. gate rows c0.. and up
//            rows I+c0.. of W_gate_up (256 B-columns), K = H.  Epilogue:
//            a = SiLU(g) * u, then per row an FP8 E4M3 re-quantisation of the
//            128 channels with scale amax/448 (BF16 rounding for BF16 layers),
//            written to the intermediate buffer in permuted row order.
//   stage 2: 256 output channels n0..n0+255 of W_down, K = I.  Epilogue:
//            multiply by the token's routing weight, round to BF16 and store
//            into the staging row of flat index p = t*k + j.
//
// Tiling: 256 threads = 4 waves.  A (activation rows) goes through LDS,
// double-buffered, 128 K per step; wave w reads all 128 rows.  B (weights)
// is streamed from HBM straight into registers: wave w owns 64 B-columns
// (four 16-column MFMA tiles) and no other wave reads them, so weights are
// fetched exactly once per item and never touch LDS.  The next step's B is
// loaded while the current step's MFMAs run.
//
// Accumulation: one 16x16x128 scaled MFMA covers a whole 128-wide K step of a
// 16x16 tile.  FP8 scales (per token per 128 channels for activations, per
// 128x128 block for weights) change every step and are not powers of two, so
// each step's partial product is scaled in fp32 and added to the accumulator
// (acc += P * sA[row] * sB).  The per-row products sA*sB of a step are formed
// once in LDS by the whole workgroup.  FP4 weights carry E8M0 scales per 32 K,
// which go straight into the MFMA's B scale operand.  Rows past the tile's
// valid count repeat a valid row; their results are never stored.
#pragma once
#include "device_common.h"
#include "permute.h"

namespace moe {

enum { ACT_BF16 = 0, ACT_FP8 = 1 };
enum { W_BF16 = 0, W_FP8 = 1, W_FP4 = 2 };

struct GemmArgs {
  const uint8_t* x;          // [T][H] E4M3 or BF16
  const float* x_scales;     // [T][H/128]
  const int32_t* perm;       // [T*k] flat index of each permuted row
  const float* topk_w;       // [T*k] routing weights, flat
  const uint8_t* w_gu;       // [E][2I][H] (FP8 / BF16) or [E][2I][H/2] (FP4)
  const void* w_gu_scales;   // fp32 [E][2I/128][H/128] or E8M0 [E][2I][H/32]
  const uint8_t* w_d;        // [E][H][I] or [E][H][I/2]
  const void* w_d_scales;    // fp32 [E][H/128][I/128] or E8M0 [E][H][I/32]
  uint8_t* aq;               // [T*k][I] E4M3 (or BF16 for BF16 layers)
  float* sa;                 // [T*k][I/128]
  uint16_t* staging;         // [T*k][H] BF16, indexed by flat index p
  int T, H, E, I, k;
};

constexpr int kGemmThreads = 256;

template <int AF>
struct GemmLds {
  static constexpr int kABytes = (AF == ACT_FP8) ? 128 : 256;   // A bytes per row per step
  static constexpr int kA = 0;
  static constexpr int kSC = kA + 2 * kTileRows * kABytes;       // [2][2][128] fp32
  static constexpr int kRowI = kSC + 2 * 2 * kTileRows * 4;      // [128] int
  static constexpr int kRowW = kRowI + kTileRows * 4;            // [128] fp32
  static constexpr int kAmax = kRowW + kTileRows * 4;            // [4][128] fp32
  static constexpr int kRsc = kAmax + 4 * kTileRows * 4;         // [128] fp32 scale
  static constexpr int kRinv = kRsc + kTileRows * 4;             // [128] fp32 1/scale
  static constexpr int kBytes = kRinv + kTileRows * 4;
};

// One step's B fragments: d[cs][i] are 16-byte pieces of column tile cs
// (FP8 uses i = 0..1, FP4 i = 0, BF16 i = 0..3); sc[cs] is the FP4 E8M0 scale.
struct BFrag {
  v4i d[4][4];
  int sc[4];
};

template <int AF, int WF, int STAGE>
DEV void expert_gemm_tile(const GemmArgs& g, int e, int r0, int m, int nb, char* lds) {
  using L = GemmLds<AF>;
  constexpr int AB = L::kABytes;                  // A bytes per row per step
  constexpr int CPR = AB / 16;                    // 16-byte chunks per A row per step
  constexpr int AJ = kTileRows * CPR / kGemmThreads;
  constexpr int ASTAGE = kTileRows * AB;          // bytes of one A stage
  constexpr int ESZ = (AF == ACT_FP8) ? 1 : 2;    // activation element size
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, c16 = lane & 15;
  const int K = (STAGE == 1) ? g.H : g.I;
  const int nsteps = K / 128;
  const int ksb = K / 128;                        // fp32 scale blocks along K

  float* SC = reinterpret_cast<float*>(lds + L::kSC);
  int* ROWI = reinterpret_cast<int*>(lds + L::kRowI);
  float* ROWW = reinterpret_cast<float*>(lds + L::kRowW);

  // ---- N block and weight pointers
  const int c0 = (STAGE == 1) ? nb * 128 : 0;
  const int n0 = (STAGE == 2) ? nb * 256 : 0;
  // Whether this wave's B columns exist.  Always true for stage 1; kept as a
  // runtime test in both stages because the branch it creates also stops the
  // scheduler from interleaving the two halves of the software pipeline
  // (which would raise register pressure past the budget).
  const bool wave_ok = (STAGE == 1) ? (c0 + 32 * w < g.I) : (n0 + 64 * w < g.H);
  const int N = (STAGE == 1) ? 2 * g.I : g.H;
  const size_t wrow = (WF == W_FP8) ? (size_t)K : (WF == W_BF16) ? (size_t)K * 2 : (size_t)K / 2;
  const uint8_t* Wbase = ((STAGE == 1) ? g.w_gu : g.w_d) + (size_t)e * N * wrow;
  const void* Sbase = (STAGE == 1) ? g.w_gu_scales : g.w_d_scales;
  const uint8_t* bptr[4];                         // this lane's weight row, at its K group
  const uint8_t* bscp[4];                         // FP4: this lane's E8M0 scale row
#pragma unroll
  for (int cs = 0; cs < 4; ++cs) {
    const int n = (STAGE == 1) ? ((cs < 2) ? c0 : g.I + c0) + 32 * w + 16 * (cs & 1) + c16
                               : n0 + 64 * w + 16 * cs + c16;
    const int ncl = wave_ok ? n : 0;
    const int goff = (WF == W_FP8) ? gq * 32 : (WF == W_FP4) ? gq * 16 : gq * 64;
    bptr[cs] = Wbase + (size_t)ncl * wrow + goff;
    bscp[cs] = reinterpret_cast<const uint8_t*>(Sbase) + ((size_t)e * N + ncl) * (K / 32) + gq;
  }
  // fp32 weight-scale rows (FP8): two 128-blocks of N per item
  const int sb0 = (STAGE == 1) ? c0 / 128 : n0 / 128;
  const int sb1 = (STAGE == 1) ? (g.I + c0) / 128 : min(n0 / 128 + 1, g.H / 128 - 1);
  const float* wsc = (WF == W_FP8) ? reinterpret_cast<const float*>(Sbase) + (size_t)e * (N / 128) * ksb : nullptr;

  __syncthreads();                                 // LDS of the previous item is free
  if (tid < kTileRows) {
    // clamped so that a malformed permutation can never index out of bounds
    const int p = (tid < m) ? min(max(g.perm[r0 + tid], 0), g.T * g.k - 1) : 0;
    if (STAGE == 1) {
      ROWI[tid] = p / g.k;
    } else {
      ROWI[tid] = p;
      ROWW[tid] = (tid < m) ? g.topk_w[p] : 0.f;
    }
  }
  __syncthreads();

  // ---- per-lane LDS offsets (constants are added at each access)
  // A stores: chunk q = tid + 256*j holds row q / CPR, chunk q % CPR; since
  // 256 is a multiple of CPR the swizzle (chunk ^ row % CPR) is the same for
  // every j and row q / CPR = tid / CPR + j * 256 / CPR.
  const int wr_row = tid / CPR, wr_c = tid % CPR;
  const uint32_t a_wr = opaque(L::kA + wr_row * AB + ((wr_c ^ (wr_row & (CPR - 1))) << 4));
  // A operand reads: row rs*16 + c16; rs*16 is a multiple of CPR's period.
  // 16x16x128 f8f6f4 operand layout (gfx950): an 8-bit operand's lane group g
  // holds K 16g..16g+15 in its first 16 bytes and K 64+16g..64+16g+15 in the
  // next 16; a 4-bit operand's lane group g holds K 32g..32g+31 (even K in the
  // low nibble); the E8M0 scale of lane group g covers K 32g..32g+31.  With
  // FP8 weights both operands use the same (arbitrary) K order, chunks 2g and
  // 2g+1; against FP4 weights the FP8 A operand must follow the 8-bit layout,
  // chunks g and g+4.
  uint32_t a_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int chunk;
    if (AF == ACT_FP8)
      chunk = (i >= 2) ? 0 : (WF == W_FP4) ? gq + 4 * i : 2 * gq + i;
    else
      chunk = 4 * gq + i;
    a_rd[i] = opaque(L::kA + c16 * AB + ((chunk ^ (c16 & (CPR - 1))) << 4));
  }
  const uint32_t sc_rd = opaque(L::kSC + 16 * gq);

  // A source rows (hoisted): token rows of x for stage 1, intermediate rows for stage 2
  // Rows past the tile's valid count load a valid row instead (row 0 of the
  // tile): their results are never stored, so no branch is needed.
  const uint8_t* asrc[AJ];
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    int row = wr_row + j * (kGemmThreads / CPR);
    row = (row < m) ? row : 0;
    if (STAGE == 1)
      asrc[j] = g.x + (size_t)ROWI[row] * g.H * ESZ + wr_c * 16;
    else
      asrc[j] = g.aq + (size_t)(r0 + row) * g.I * ESZ + wr_c * 16;
  }
  const int srow = ((tid & 127) < m) ? (tid & 127) : 0;
  const float* sAp = (AF == ACT_FP8)
      ? ((STAGE == 1) ? g.x_scales + (size_t)ROWI[srow] * (g.H / 128)
                      : g.sa + (size_t)(r0 + srow) * (g.I / 128))
      : nullptr;

  // ---- A loads (global -> registers -> LDS)
  v4i areg[AJ];
  float sA_next = 0.f, sw0_next = 0.f, sw1_next = 0.f;
  auto load_a = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < AJ; ++j) areg[j] = ld16(asrc[j] + (size_t)s * 128 * ESZ);
    if (AF == ACT_FP8) {
      sA_next = sAp[s];
      if (WF == W_FP8) {
        sw0_next = wsc[(size_t)sb0 * ksb + s];
        sw1_next = wsc[(size_t)sb1 * ksb + s];
      }
    }
  };
  auto store_a = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < AJ; ++j) lds_st(lds, a_wr + stage * ASTAGE + j * (kGemmThreads / CPR) * AB, areg[j]);
    if (AF == ACT_FP8) {
      float v = sA_next;
      if (WF == W_FP8) v *= (tid < 128) ? sw0_next : sw1_next;
      SC[stage * 2 * kTileRows + tid] = v;        // [stage][set = tid / 128][row = tid % 128]
    }
  };

  // ---- B loads (straight to registers)
  auto load_b = [&](int s, BFrag& b) __attribute__((always_inline)) {
    if (!wave_ok) return;
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) {
      if (WF == W_FP8) {
        const uint8_t* p = bptr[cs] + (size_t)s * 128;
        b.d[cs][0] = ld16(p);
        b.d[cs][1] = ld16(p + 16);
      } else if (WF == W_FP4) {
        b.d[cs][0] = ld16(bptr[cs] + (size_t)s * 64);
        b.sc[cs] = bscp[cs][s * 4];
      } else {
        const uint8_t* p = bptr[cs] + (size_t)s * 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) b.d[cs][i] = ld16(p + 16 * i);
      }
    }
  };

  v4f acc[8][4];
#pragma unroll
  for (int rs = 0; rs < 8; ++rs)
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) acc[rs][cs] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage, const BFrag& b) __attribute__((always_inline)) {
    if (!wave_ok) return;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rs = 0; rs < 8; ++rs) {
      const uint32_t ao = stage * ASTAGE + rs * 16 * AB;
      // operands of row tile rs are read only once row tile rs-2 is finished
      const float dep = (rs >= 2) ? acc[rs - 2][3][3] : 0.f;
      if (AF == ACT_FP8) {
        const v4i a0 = lds_ld<v4i>(lds, after(a_rd[0], dep) + ao);
        const v4i a1 = lds_ld<v4i>(lds, after(a_rd[1], dep) + ao);
        const v8i av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const uint32_t so = after(sc_rd, dep);
        const v4f s0 = lds_ld<v4f>(lds, so + (stage * 2) * kTileRows * 4 + rs * 64);
        const v4f s1 = lds_ld<v4f>(lds, so + (stage * 2 + 1) * kTileRows * 4 + rs * 64);
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
          v4f p;
          if (WF == W_FP8) {
            const v8i bv = {b.d[cs][0][0], b.d[cs][0][1], b.d[cs][0][2], b.d[cs][0][3],
                            b.d[cs][1][0], b.d[cs][1][1], b.d[cs][1][2], b.d[cs][1][3]};
            p = mfma_fp8_fp8(av, bv, zero);
          } else {
            const v8i bv = {b.d[cs][0][0], b.d[cs][0][1], b.d[cs][0][2], b.d[cs][0][3], 0, 0, 0, 0};
            p = mfma_fp8_fp4(av, bv, zero, b.sc[cs]);
          }
          bool set1;
          if (WF == W_FP4) set1 = false;
          else if (STAGE == 1) set1 = cs >= 2;
          else set1 = (w >= 2);
          const v4f sc = set1 ? s1 : s0;
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rs][cs][v] = __builtin_fmaf(p[v], sc[v], acc[rs][cs][v]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4i a = lds_ld<v4i>(lds, after(a_rd[i], dep) + ao);
#pragma unroll
          for (int cs = 0; cs < 4; ++cs) acc[rs][cs] = mfma_bf16(as_v8bf(a), as_v8bf(b.d[cs][i]), acc[rs][cs]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);          // keep one row tile's operands live at a time
    }
  };

  // ---- main loop: A double-buffered in LDS, B double-buffered in registers
  // (BF16 weights are 4x the bytes per step and stay single-buffered)
  BFrag b0, b1;
  load_a(0);
  store_a(0);
  if (WF == W_BF16) {
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      load_b(s, b0);
      if (s + 1 < nsteps) load_a(s + 1);
      compute(s & 1, b0);
      if (s + 1 < nsteps) store_a((s + 1) & 1);
      __syncthreads();
    }
  } else {
  load_b(0, b0);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    if (s + 1 < nsteps) { load_a(s + 1); load_b(s + 1, b1); }
    compute(0, b0);
    if (s + 1 < nsteps) store_a(1);
    __syncthreads();
    if (s + 1 >= nsteps) break;
    if (s + 2 < nsteps) { load_a(s + 2); load_b(s + 2, b0); }
    compute(1, b1);
    if (s + 2 < nsteps) store_a(0);
    __syncthreads();
  }
  }

  // ---- epilogues (the A region is reused as the output staging tile)
  if (STAGE == 1) {
    // a = SiLU(g) * u, written over the gate accumulators: av[rs][q] = acc[rs][q]
#pragma unroll
    for (int rs = 0; rs < 8; ++rs) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc[rs][q][v], uv = acc[rs][2 + q][v];
          acc[rs][q][v] = gv / (1.0f + __expf(-gv)) * uv;
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    auto av = [&](int rs, int q, int v) __attribute__((always_inline)) { return acc[rs][q][v]; };
    if (AF == ACT_FP8) {
      float* RSC = reinterpret_cast<float*>(lds + L::kRsc);
      const uint32_t amax_wr = opaque(L::kAmax + w * kTileRows * 4 + 16 * gq);
#pragma unroll
      for (int rs = 0; rs < 8; ++rs)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float mx = fmaxf(fabsf(av(rs, 0, v)), fabsf(av(rs, 1, v)));
          mx = wave_max_xor16(mx);
          if (c16 == 0) lds_st(lds, amax_wr + (rs * 16 + v) * 4, mx);
        }
      __syncthreads();
      if (tid < kTileRows) {
        const float* AMAX = reinterpret_cast<const float*>(lds + L::kAmax);
        const float mx = fmaxf(fmaxf(AMAX[tid], AMAX[kTileRows + tid]),
                               fmaxf(AMAX[2 * kTileRows + tid], AMAX[3 * kTileRows + tid]));
        const float sc = (mx > 0.f) ? mx / 448.0f : 1.0f;
        RSC[tid] = sc;
        reinterpret_cast<float*>(lds + L::kRinv)[tid] = 1.0f / sc;
      }
      __syncthreads();
      const uint32_t rinv_rd = opaque(L::kRinv + 16 * gq);
      const uint32_t out_wr = opaque(L::kA + 4 * gq * 128 + 32 * w + c16);
#pragma unroll
      for (int rs = 0; rs < 8; ++rs)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float inv = lds_ld<float>(lds, rinv_rd + (rs * 16 + v) * 4);
          const uint32_t o = out_wr + (rs * 16 + v) * 128;
          lds_st(lds, o, (uint8_t)f32_to_e4m3(av(rs, 0, v) * inv));
          lds_st(lds, o + 16, (uint8_t)f32_to_e4m3(av(rs, 1, v) * inv));
        }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = tid + kGemmThreads * j;
        const int row = q >> 3, c = q & 7;
        if (row < m) st16(g.aq + (size_t)(r0 + row) * g.I + c0 + c * 16, ld16(lds + L::kA + row * 128 + c * 16));
      }
      if (tid < m) g.sa[(size_t)(r0 + tid) * (g.I / 128) + c0 / 128] = RSC[tid];
    } else {
      const uint32_t out_wr = opaque(L::kA + (4 * gq * 128 + 32 * w + c16) * 2);
#pragma unroll
      for (int rs = 0; rs < 8; ++rs)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t o = out_wr + (rs * 16 + v) * 256;
          lds_st(lds, o, (uint16_t)f32_to_bf16_rne(av(rs, 0, v)));
          lds_st(lds, o + 32, (uint16_t)f32_to_bf16_rne(av(rs, 1, v)));
        }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = tid + kGemmThreads * j;
        const int row = q >> 4, c = q & 15;
        if (row < m)
          st16(g.aq + ((size_t)(r0 + row) * g.I + c0) * 2 + c * 16, ld16(lds + L::kA + row * 256 + c * 16));
      }
    }
  } else {
    const uint32_t out_wr = opaque(L::kA + (4 * gq * 256 + 64 * w + c16) * 2);
    const uint32_t roww_rd = opaque(L::kRowW + 16 * gq);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) __syncthreads();                 // first half's copy-out is done
      if (wave_ok) {
#pragma unroll
        for (int rs = 4 * h; rs < 4 * h + 4; ++rs)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float rw = lds_ld<float>(lds, roww_rd + (rs * 16 + v) * 4);
#pragma unroll
            for (int cs = 0; cs < 4; ++cs)
              lds_st(lds, out_wr + ((rs - 4 * h) * 16 + v) * 512 + cs * 32,
                     (uint16_t)f32_to_bf16_rne(acc[rs][cs][v] * rw));
          }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = tid + kGemmThreads * j;
        const int rl = q >> 5, c = q & 31;
        const int row = 64 * h + rl, col = n0 + c * 8;
        if (row < m && col < g.H)
          st16(reinterpret_cast<uint8_t*>(g.staging) + ((size_t)ROWI[row] * g.H + col) * 2,
               ld16(lds + L::kA + rl * 512 + c * 16));
      }
    }
  }
}

// y[t, n0:n1] = BF16( sum_j staging[t*k + j, n0:n1] ) for tokens [t0, t1),
// fp32 sums in ascending j; 8 channels (16 bytes) per thread and step.
DEV void combine_rows(const uint16_t* staging, uint16_t* y, int H, int k, int t0, int t1, int n0, int n1) {
  const int cpt = (n1 - n0) / 8;
  const int total = (t1 - t0) * cpt;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int t = t0 + idx / cpt, c = n0 + (idx % cpt) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const v4i v = ld16(reinterpret_cast<const uint8_t*>(staging) + ((size_t)(t * k + j) * H + c) * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[2 * i] += bf16_to_f32((uint32_t)v[i] & 0xFFFFu);
        s[2 * i + 1] += bf16_to_f32((uint32_t)v[i] >> 16);
      }
    }
    v4i o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (int)(f32_to_bf16_rne(s[2 * i]) | (f32_to_bf16_rne(s[2 * i + 1]) << 16));
    st16(reinterpret_cast<uint8_t*>(y) + ((size_t)t * H + c) * 2, o);
  }
}

}  // namespace moe
