// Grouped expert GEMMs on gfx950 MFMA, with their fused epilogues.
//
// Linear 1 (gate|up), SwiGLU, linear 2 (down) and the per-token combine are
// the expert half of the MoE block (机器之心, "DeepSeek悄悄更新：Mega MoE、FP4
// Indexer来了", section "Mega MoE 是什么？"); FP8 x FP4 mixed precision is named
// in the same section; quantisation fused with SwiGLU is the quantisation
// bullet of the "Tile Kernels" section of youleyou, "DeepSeek 模型更新解读 Tile
// Kernels 与 DeepEP V2 新特性".
//
// One work item is a row tile of one expert (up to 256 permuted rows for FP8
// activations, 128 for BF16) times one N block:
//   stage 1: 128 intermediate channels c0..c0+127, i.e. gate rows c0.. and up
//            rows I+c0.. of W_gate_up (256 B-columns), K = H.  Epilogue:
//            a = SiLU(g) * u, then per row an FP8 E4M3 re-quantisation of the
//            128 channels with scale amax/448 (BF16 rounding for BF16 layers),
//            written to the intermediate buffer in permuted row order.
//   stage 2: 256 output channels n0..n0+255 of W_down, K = I.  Epilogue:
//            multiply by the token's routing weight, round to BF16 and store
//            into the staging row of flat index p = t*k + j.
//
// Tiling: 256 threads = 4 waves, one per SIMD (512 VGPRs each).  A
// (activation rows, gathered by token for stage 1) is copied HBM -> LDS by
// direct buffer loads into two stages, one step ahead, 128 K per step; wave
// w reads all rows.  B (weights)
// is streamed from HBM straight into registers: wave w owns 64 B-columns
// (four 16-column MFMA tiles) and no other wave reads them, so weights are
// fetched exactly once per item and never touch LDS.  B is loaded two steps
// ahead of the MFMAs that use it.  All loads use buffer
// resources with 32-bit offsets (loads past a buffer's end read zero).
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
#include "quant.h"

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
  float* sa;                 // [I/128][T*k] (K block major, permuted rows)
  const float* sxp;          // [H/128][T*k] x_scales in permuted row order, or NULL
  uint16_t* staging;         // [H/256][T*k][256] BF16: N block, then flat index p, then column
  int T, H, E, I, k;
  int pow2;                  // re-quantise the intermediate with power-of-two scales
  int pow2_x;                // the activation scales are powers of two (the layer's own quantisation)
  int wchan;                 // FP8 weights: one fp32 scale per output channel ([E][N]), not per block
};

constexpr int kGemmThreads = 256;

// Full tiles: 128 rows for FP8 activations, 64 for BF16.  With one wave per
// SIMD a wave holds 16*RS x 64 fp32 accumulators (4*RS*4 VGPRs), which must
// stay in VALU-addressable registers for the per-128-K promotion, next to
// three (FP8) or two (BF16) steps of B fragments.  144-row FP8 tiles: an
// expert with up to 288 rows (a DeepSeek-V3-shaped layer has 256 +- 15 per
// expert) needs two tiles, each streaming the expert's weight slab once,
// instead of two full tiles and a small remainder that streams it again.
constexpr int kGemmMaxRsFp8 = 9;
constexpr int kGemmMaxRsBf16 = 4;

template <int AF>
struct GemmLds {
  static constexpr int kABytes = (AF == ACT_FP8) ? 128 : 256;   // A bytes per row per step
  static constexpr int kMaxRs = (AF == ACT_FP8) ? kGemmMaxRsFp8 : kGemmMaxRsBf16;
  static constexpr int kRows = kMaxRs * 16;                      // rows of a full tile
  static constexpr int kASlot = kRows * kABytes;                 // one A stage
  static constexpr int kA = 0;                                   // [2] A stages
  static constexpr int kScRows = kGemmThreads;                   // every thread writes a scale
  // SC position stride of a row: subtile-minor, padded to a multiple of four
  // so that a lane's run of scales starts 16-byte aligned
  static constexpr int kScStride = (kMaxRs + 3) / 4 * 4;
  static_assert(16 * kScStride + 64 <= kScRows, "scale positions and the spare slots fit");
  static constexpr int kSaRows = (kRows + 63) / 64 * 64;         // rows of an activation-scale slot
  // Prefetch distance (steps) of gate|up, which sets the LDS stages.  The
  // down GEMM (K = I, 8 to 16 steps at DeepSeek-V3-like shapes) runs two
  // steps ahead: measured 0.5-2.6% faster than three on every workload.
  static constexpr int kPd = (AF == ACT_FP8) ? 3 : 2;
  static constexpr int kPdDown = 2;                               // <= kPd
  static constexpr int kAStages = kPd + 1;
  static constexpr int kSC = kA + kAStages * kASlot;             // [2][2][kScRows] fp32 row scales
  static constexpr int kRowI = kSC + 2 * 2 * kScRows * 4;        // [kRows] int
  static constexpr int kRowW = kRowI + kRows * 4;                // [kRows] fp32
  static constexpr int kAmax = kRowW + kRows * 4;                // [4][kRows] fp32
  static constexpr int kRsc = kAmax + 4 * kRows * 4;             // [kRows] fp32 scale
  static constexpr int kRinv = kRsc + kRows * 4;                 // [kRows] fp32 1/scale
  static constexpr int kScw = kRinv + kRows * 4;                 // [2][128] fp32 weight block scales
  static constexpr int kSaSlots = kPd + 1;
  static constexpr int kSA = kScw + 2 * 128 * 4;                 // [kSaSlots][kSaRows] fp32 activation scales
  static constexpr int kBytes = kSA + kSaSlots * kSaRows * 4;
};

// One step's B fragments: d[cs][i] are 16-byte pieces of column tile cs
// (FP8 uses i = 0..1, FP4 i = 0, BF16 i = 0..3); with FP4, byte cs of sc is
// the E8M0 scale of column tile cs (one load for the wave's four tiles).
struct BFrag {
  v4i d[4][4];
  uint32_t sc;
};

// 16-byte chunk position of logical chunk c of A row `row` in LDS.  FP8 rows
// (8 chunks): c ^ (row & 7) ^ ((row >> 3) & 1), so that the 16 rows read by
// one MFMA operand fetch fall in distinct banks whether LDS serves 8 or 16
// lanes per cycle, and the swizzle of row rs*16 + r depends on r only.
// BF16 rows (16 chunks): c ^ (row & 15).
template <int CPR>
DEV int a_swz(int row, int c) {
  if (CPR == 8) return c ^ (row & 7) ^ ((row >> 3) & 1);
  return c ^ (row & 15);
}

// Copy a staged output tile from LDS to global memory: N pieces of 16 bytes,
// `piece(q, &lds_off, &dst_off)` gives the offsets of piece q and whether
// it is stored.  A thread issues all of its LDS reads before its stores, so
// it waits for LDS once rather than once per piece.
template <int N, int CP, typename F>
DEV void copy_pieces(rsrc_t dst, const char* lds, const F& piece) {
  constexpr int NQ = (N + kGemmThreads - 1) / kGemmThreads;
  v4i d[NQ];
  uint32_t off[NQ];
  bool ok[NQ];
#pragma unroll
  for (int it = 0; it < NQ; ++it) {
    const int q = threadIdx.x + it * kGemmThreads;
    uint32_t lo = 0;
    ok[it] = (N % kGemmThreads == 0 || q < N) && piece(q, &lo, &off[it]);
    d[it] = ld16(lds + lo);
  }
#pragma unroll
  for (int it = 0; it < NQ; ++it)
    if (ok[it]) buf_st16<CP>(dst, off[it], d[it]);
}

struct NoHook {
  DEV void operator()() const {}
};

// One work item: `RS` 16-row subtiles (rows [r0, r0+m), m <= 16*RS) of
// expert e times one N block nb.  256 threads, one wave per SIMD.  With COH
// (inside the persistent kernel, where producer and consumer items may run
// on different XCDs) the outputs are stored write-through (kCoherent), so
// that they are in memory once the producer's counter is signalled.  The
// consumer reads the intermediate codes with ordinary, cached loads: each
// 128-byte line of them belongs to one (row, N block), is written once per
// launch and is read only after its writer's counter is complete, so no L2
// can hold an older copy of it.  The intermediate's scales (one K block of
// 32 consecutive permuted rows per 128-byte line, so a line can hold rows of
// two tiles) are read coherently.  `signal_prev` (may be NULL) is a
// counter to increment once the stores of this workgroup's previous item
// have completed: the prologue's barrier below waits for every older memory
// operation of each wave, so the previous item is signalled without a wait
// of its own.
// `at_loop_end()` is called by every thread once the K loop has ended,
// before the epilogue.
// E8 (FP4 weights with power-of-two activation scales): every scale of the
// product is a power of two, so the activation scale goes into the MFMA's
// B scale operand next to the weights' E8M0 scales, and the MFMA accumulates
// in place: no fp32 promotion.
template <int AF, int WF, int STAGE, int RS, int COH, int E8, typename Hook>
DEV void expert_gemm_tile(const GemmArgs& g, int e, int r0, int m, int nb, char* lds, int32_t* signal_prev,
                          const Hook& at_loop_end) {
  static_assert(!E8 || (WF == W_FP4 && AF == ACT_FP8), "power-of-two products need FP4 weights");
  constexpr int CP = COH ? kCoherent : 0;            // cache policy of cross-item data
  using L = GemmLds<AF>;
  static_assert(RS >= 1 && RS <= L::kMaxRs, "row subtiles");
  constexpr int AB = L::kABytes;                  // A bytes per row per step
  constexpr int CPR = AB / 16;                    // 16-byte chunks per A row per step
  constexpr int RPD = 1024 / AB;                  // rows per wave-wide 1 KB DMA
  constexpr int R = RS * 16;                      // rows computed
  constexpr int NDMA = (R * AB + 4095) / 4096;    // DMA instructions per thread per step
  constexpr int ESZ = (AF == ACT_FP8) ? 1 : 2;    // activation element size
  constexpr int NB = (WF == W_BF16) ? 16 : (WF == W_FP8) ? 8 : 5;   // B load instructions per lane per step
  constexpr int PD = (STAGE == 2) ? L::kPdDown : L::kPd;   // A and scales: loaded PD (+1) steps ahead
  constexpr int AST = PD + 1;                      // A stages and activation-scale slots in use
  static_assert(PD <= L::kPd, "stages fit the LDS layout");
  constexpr int NBUF = (WF == W_BF16) ? 2 : PD + 1; // B register buffers (B distance NBUF - 1)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, c16 = lane & 15;
  const int K = (STAGE == 1) ? g.H : g.I;
  const int nsteps = K / 128;
  const int ksb = K / 128;                        // fp32 scale blocks along K

  float* SC = reinterpret_cast<float*>(lds + L::kSC);
  float* SCW = reinterpret_cast<float*>(lds + L::kScw);
  int* ROWI = reinterpret_cast<int*>(lds + L::kRowI);
  float* ROWW = reinterpret_cast<float*>(lds + L::kRowW);

  // ---- N block and weights
  const int c0 = (STAGE == 1) ? nb * 128 : 0;
  const int n0 = (STAGE == 2) ? nb * 256 : 0;
  // Whether this wave's B columns exist (only the last down-projection block
  // can be half empty).  Waves without columns still run the main loop on a
  // clamped row so that it stays branch-free; their results are not stored.
  const bool wave_ok = (STAGE == 1) || (n0 + 64 * w < g.H);
  const int N = (STAGE == 1) ? 2 * g.I : g.H;
  const uint32_t wrow = (WF == W_FP8) ? K : (WF == W_BF16) ? K * 2 : K / 2;
  const uint8_t* Wexp = ((STAGE == 1) ? g.w_gu : g.w_d) + (size_t)e * N * wrow;
  const rsrc_t wrs = make_rsrc(Wexp, (uint32_t)N * wrow);
  const void* Sbase = (STAGE == 1) ? g.w_gu_scales : g.w_d_scales;
  const rsrc_t srs = make_rsrc(reinterpret_cast<const uint8_t*>(Sbase) + (size_t)e * N * (K / 32),
                               (WF == W_FP4) ? (uint32_t)N * (K / 32) : 0u);
  // Weights are in the MFMA-tiled layout (see moe_pack_weights): for each
  // 128-K step s and 16-row tile t, a block of 16*BS bytes at
  // (s*(N/16) + t)*16*BS made of 1 KB pieces, piece p holding in its 16
  // bytes at 16*l the row 16t + l%16, bytes BS*s + 64p + 16*(l/16) .. +15 of
  // the row-major matrix.  One piece is exactly one B operand load of a
  // wave: 1 KB contiguous; the blocks of one step are adjacent.
  constexpr uint32_t BS = (WF == W_FP8) ? 128 : (WF == W_BF16) ? 256 : 64;   // bytes per row per K step
  uint32_t boff[4];                                // this lane's piece offsets
#pragma unroll
  for (int cs = 0; cs < 4; ++cs) {
    const int nt = ((STAGE == 1) ? ((cs < 2) ? c0 : g.I + c0) + 32 * w + 16 * (cs & 1) : n0 + 64 * w + 16 * cs) / 16;
    const int ntc = wave_ok ? nt : 0;
    boff[cs] = (uint32_t)ntc * 16u * BS + 16u * lane;
  }
  // FP4 E8M0 scales (see moe_pack_weights): per K step, quads of 256 bytes,
  // 4 bytes per lane, byte c the scale of the quad's tile c: for gate|up the
  // gate tiles 2q, 2q+1 and up tiles 2q, 2q+1, for down the tiles 4q..4q+3.
  // A wave's four column tiles are exactly one quad.
  const uint32_t bsoff = (uint32_t)(wave_ok ? ((STAGE == 1) ? c0 / 32 + w : n0 / 64 + w) : 0) * 256u + 4u * lane;
  // fp32 weight-scale rows (FP8): two 128-blocks of N per item; or, with
  // per-channel scales, the scales of the item's 256 B-columns (applied in
  // the epilogue, after the K sum)
  const int sb0 = (STAGE == 1) ? c0 / 128 : n0 / 128;
  const int sb1 = (STAGE == 1) ? (g.I + c0) / 128 : min(n0 / 128 + 1, g.H / 128 - 1);
  const bool wchan = WF == W_FP8 && g.wchan != 0;
  const float* wsc = (WF == W_FP8) ? reinterpret_cast<const float*>(Sbase) +
                                         (size_t)e * (wchan ? (size_t)N : (size_t)(N / 128) * ksb)
                                   : nullptr;

  __syncthreads();                                 // LDS of the previous item is free
  if (tid < R) {
    // clamped so that a malformed permutation can never index out of bounds
    const int p = (tid < m) ? min(max(g.perm[r0 + tid], 0), g.T * g.k - 1) : 0;
    if (STAGE == 1) {
      ROWI[tid] = p / g.k;
    } else {
      ROWI[tid] = p;
      ROWW[tid] = (tid < m) ? g.topk_w[p] : 0.f;
    }
  }
  // the item's two rows of FP8 weight block scales (K <= 16384: <= 128
  // blocks), or its columns' channel scales: SCW[c] for item column c
  // (gate|up: gate channel c0 + c for c < 128, up channel I + c0 + c - 128;
  // down: output column n0 + c, past H reading the last one)
  if (WF == W_FP8 && AF == ACT_FP8) {
    const int set = tid >> 7, kb = tid & 127;
    if (wchan)
      SCW[tid] = wsc[(STAGE == 1) ? (set ? g.I : 0) + c0 + kb : min(n0 + tid, g.H - 1)];
    else if (kb < nsteps)
      SCW[tid] = wsc[(size_t)(set ? sb1 : sb0) * ksb + kb];
  }
  __syncthreads();

  // ---- A rows: direct-to-LDS loads.  Wave w's DMA j fills rows
  // RPD*(4j+w) .. +RPD of a stage; lane l writes row + l / CPR, physical
  // chunk l % CPR, i.e. logical chunk a_swz(row, l % CPR).  Rows past the
  // tile's valid count repeat row 0 (their results are never stored).  A
  // DMA whose rows lie past the variant's R rows (R not a multiple of 4*RPD)
  // repeats the wave's DMA 0 instead (same bytes to the same place), so that
  // every wave issues the same number of loads per step.
  const rsrc_t ars = (STAGE == 1) ? make_rsrc(g.x, (uint32_t)((size_t)g.T * g.H * ESZ))
                                  : make_rsrc(g.aq, (uint32_t)((size_t)g.T * g.k * g.I * ESZ));
  uint32_t aoff[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int row = RPD * (4 * j + w) + lane / CPR;
    const int c = a_swz<CPR>(row, lane % CPR);
    const int rowc = (row < m) ? row : 0;
    const uint32_t rbase = (STAGE == 1) ? (uint32_t)ROWI[rowc] * g.H : (uint32_t)(r0 + rowc) * g.I;
    aoff[j] = rbase * ESZ + c * 16;
  }
  // stage `slot` (= s % AST) receives A(s).  Steps past the last
  // (issued so that the step stays branch-free) load the last step again:
  // an unclamped offset would reach into the next permuted row, which in
  // the persistent kernel may belong to a tile whose gate|up item has not
  // yet written it, and an ordinary load would leave that stale line in
  // this XCD's L2 for a later reader.
  auto dma_a = [&](int s, int slot, int j) __attribute__((always_inline)) {
    char* dst = lds + L::kA + slot * L::kASlot + w * 1024;
    const bool in = (R % (4 * RPD) == 0) || RPD * (4 * j + w) < R;      // wave-uniform
    buf_ld16_lds<0>(ars, dst + (in ? j : 0) * 4096, in ? aoff[j] : aoff[0],
                    (uint32_t)min(s, nsteps - 1) * 128 * ESZ);
  };

  // ---- per-row scales (FP8 activations).  The activation scales of step s
  // are loaded straight into LDS slot s % AST, PD + 1 steps ahead: wave w
  // loads rows 64*(w % NSW) + lane (NSW waves cover the tile; the others
  // write the same values as wave w % NSW), so that thread tid < kRows finds
  // the scale of row tid.  SC[par][set] holds sA[row] * sB[set] for the
  // tile's rows, stored subtile-minor (row rs*16 + i at position
  // i*kScStride + rs), so that a lane reads the scales of its row i for every
  // subtile with one to three 16-byte LDS reads.
  constexpr int NSW = L::kSaRows / 64;
  const int arow = 64 * (w % NSW) + lane;
  const int srow = (arow < m) ? arow : 0;
  // The intermediate's scales, and the activation scales when a permuted
  // copy exists (g.sxp), are K block major over the permuted rows
  // ([K/128][T*k]): the scales of one step for a tile's rows are contiguous.
  // Otherwise each row reads its token's row of x_scales.
  const uint32_t nrows_all = (uint32_t)(g.T * g.k);
  const bool permuted = (STAGE == 2) || g.sxp != nullptr;
  const rsrc_t sars = (AF != ACT_FP8) ? make_rsrc(nullptr, 0)
                      : (STAGE == 2) ? make_rsrc(g.sa, nrows_all * (uint32_t)(g.I / 128) * 4)
                      : permuted     ? make_rsrc(g.sxp, nrows_all * (uint32_t)(g.H / 128) * 4)
                                     : make_rsrc(g.x_scales, (uint32_t)g.T * (g.H / 128) * 4);
  const uint32_t saoff = permuted ? (uint32_t)(r0 + srow) * 4 : (uint32_t)ROWI[srow] * (uint32_t)(g.H / 128) * 4;
  const uint32_t sastep = permuted ? nrows_all * 4 : 4u;
  auto dma_sa = [&](int s, int slot) __attribute__((always_inline)) {   // slot = s % AST
    buf_ld4_lds<STAGE == 2 ? CP : 0>(sars, lds + L::kSA + slot * (L::kSaRows * 4) + (w % NSW) * 256, saoff,
                                     (uint32_t)min(s, nsteps - 1) * sastep);
  };
  auto read_sa = [&](int slot) __attribute__((always_inline)) -> float {
    return (AF == ACT_FP8) ? lds_ld<float>(lds, L::kSA + slot * (L::kSaRows * 4) + (tid % L::kSaRows) * 4) : 1.f;
  };
  auto store_scale = [&](int s, int par, float sa) __attribute__((always_inline)) {   // par = s & 1
    if (AF != ACT_FP8) return;
    const int sc = min(s, nsteps - 1);             // steps past the end are never used
    const float w0 = (WF == W_FP8 && !wchan) ? SCW[sc] : 1.f;
    const float w1 = (WF == W_FP8 && !wchan) ? SCW[128 + sc] : 1.f;
    // no branch here: a conditional block would let the compiler sink the
    // step's MFMAs below the step's closing barrier
    // spare threads write to the unused positions past 16 * kScStride
    const int pos = (tid < L::kRows) ? (tid & 15) * L::kScStride + (tid >> 4) : 16 * L::kScStride + (tid & 63);
    SC[(par * 2 + 0) * L::kScRows + pos] = sa * w0;
    SC[(par * 2 + 1) * L::kScRows + pos] = sa * w1;
  };

  // ---- B loads (HBM straight to registers), one instruction per piece q.
  // Steps past the last (issued so that the step stays branch-free) load
  // the last step again.
  auto bstep = [&](int s) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)min(s, nsteps - 1) * (uint32_t)N * BS;
  };
  auto load_b_piece = [&](int s, BFrag& b, int q) __attribute__((always_inline)) {
    if (WF == W_FP8) {
      b.d[q >> 1][q & 1] = buf_ld16(wrs, boff[q >> 1] + 1024 * (q & 1), bstep(s));
    } else if (WF == W_FP4) {
      if (q < 4) b.d[q][0] = buf_ld16(wrs, boff[q], bstep(s));
      else b.sc = __float_as_uint(buf_ldf(srs, bsoff, (uint32_t)min(s, nsteps - 1) * (uint32_t)N * 4u));
    } else {
      b.d[q >> 2][q & 3] = buf_ld16(wrs, boff[q >> 2] + 1024 * (q & 3), bstep(s));
    }
  };

  // ---- MFMA operand offsets.  16x16x128 f8f6f4 operand layout (gfx950): an
  // 8-bit operand's lane group g holds K 16g..16g+15 in its first 16 bytes
  // and K 64+16g..64+16g+15 in the next 16; a 4-bit operand's lane group g
  // holds K 32g..32g+31 (even K in the low nibble); the E8M0 scale of lane
  // group g covers K 32g..32g+31.  So an FP8 operand of lane group g is
  // 16-byte chunks g and g+4 of the 128-byte K step, an FP4 operand is chunk
  // g of the 64-byte step.  16x16x32 BF16: lane group g holds K 8g..8g+7 of
  // each 32-K MFMA i, i.e. chunk 4i+g of the 256-byte step.  Each B load
  // instruction thereby reads 64 contiguous bytes of every weight row it
  // touches (one L1 request per row instead of four scattered pieces).
  uint32_t a_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int chunk;
    if (AF == ACT_FP8)
      chunk = (i >= 2) ? 0 : gq + 4 * i;
    else
      chunk = 4 * i + gq;
    a_rd[i] = opaque(L::kA + c16 * AB + (a_swz<CPR>(c16, chunk) << 4));
  }
  // With FP8 activations the product is formed transposed: the weights are
  // the MFMA's A operand and the activation rows its B operand, so output
  // lane l holds row l%16 of the subtile (channels 4*(l/16) + v) and the
  // promotion scale of its four values is one number per lane and subtile.
  constexpr int NSET = (STAGE == 1 && WF == W_FP8) ? 2 : 1;
  const uint32_t sc_rd = opaque(L::kSC + c16 * L::kScStride * 4 +
                                ((STAGE == 2 && WF == W_FP8 && w >= 2) ? L::kScRows * 4 : 0));

  v4f acc[RS][4];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) acc[rs][cs] = v4f{0.f, 0.f, 0.f, 0.f};

  // The step's MFMAs and FMAs have no memory side effects, so the compiler
  // may sink them below the step's closing barrier (an asm statement), which
  // would serialise the loads behind it with the math.  An empty volatile asm
  // that "modifies" every accumulator keeps them above it.
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        float x0 = acc[rs][cs][0], x1 = acc[rs][cs][1], x2 = acc[rs][cs][2], x3 = acc[rs][cs][3];
        asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
        acc[rs][cs] = v4f{x0, x1, x2, x3};
      }
  };

  // Software pipeline over row subtiles, one scheduling region per subtile
  // (sched_barrier keeps the compiler from hoisting every LDS read to the
  // top, which would need registers for all subtiles at once): region rs
  // issues a share of the step's global loads, the LDS reads of subtile
  // rs+1, the MFMAs of rs and the fp32 promotion of rs-1, so the vector ALU
  // scales and the memory pipeline accepts new loads while the matrix core
  // works.  `issue(j)` issues global load j of the step (0 <= j < nload).
  auto compute = [&](int slot, int par, const BFrag& b, int nload, auto&& issue) __attribute__((always_inline)) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t so = (uint32_t)slot * L::kASlot;
    const uint32_t sco = (uint32_t)par * 2 * L::kScRows * 4;
    constexpr int NREG = (AF == ACT_FP8) ? RS + 1 : RS;
    auto issue_share = [&](int r) __attribute__((always_inline)) {
#pragma unroll
      for (int j = r * nload / NREG; j < (r + 1) * nload / NREG; ++j) issue(j);
    };
    if (AF == ACT_FP8) {
      constexpr int NC = (RS + 3) / 4;
      v4i a0[3], a1[3];
      v4f p[2][4], scv[NSET][NC];
#pragma unroll
      for (int st = 0; st < NSET; ++st)
#pragma unroll
        for (int c = 0; c < NC; ++c) scv[st][c] = lds_ld<v4f>(lds, sc_rd + sco + st * L::kScRows * 4 + c * 16);
      auto lda = [&](int rs) __attribute__((always_inline)) {
        const uint32_t ao = so + rs * 16 * AB;
        a0[rs % 3] = lds_ld<v4i>(lds, a_rd[0] + ao);
        a1[rs % 3] = lds_ld<v4i>(lds, a_rd[1] + ao);
      };
      // A operands are read two subtiles ahead (three register sets), which
      // gives each LDS read about two subtiles of MFMA time to land
      lda(0);
      if (RS > 1) lda(1);
#pragma unroll
      for (int rs = 0; rs <= RS; ++rs) {
        __builtin_amdgcn_sched_barrier(0);
        issue_share(rs);
        if (rs + 2 < RS) lda(rs + 2);
        if (rs < RS) {
          const v4i x0 = a0[rs % 3], x1 = a1[rs % 3];
          const v8i av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
          for (int cs = 0; cs < 4; ++cs) {
            if (WF == W_FP8) {
              const v8i bv = {b.d[cs][0][0], b.d[cs][0][1], b.d[cs][0][2], b.d[cs][0][3],
                              b.d[cs][1][0], b.d[cs][1][1], b.d[cs][1][2], b.d[cs][1][3]};
              p[rs & 1][cs] = mfma_fp8_fp8(bv, av, zero);
            } else if (E8) {
              const v8i bv = {b.d[cs][0][0], b.d[cs][0][1], b.d[cs][0][2], b.d[cs][0][3], 0, 0, 0, 0};
              acc[rs][cs] = mfma_fp4_fp8(bv, av, acc[rs][cs], (int)((b.sc >> (8 * cs)) & 0xFFu),
                                         e8m0_of_pow2(scv[0][rs >> 2][rs & 3]));
            } else {
              const v8i bv = {b.d[cs][0][0], b.d[cs][0][1], b.d[cs][0][2], b.d[cs][0][3], 0, 0, 0, 0};
              p[rs & 1][cs] = mfma_fp4_fp8(bv, av, zero, (int)((b.sc >> (8 * cs)) & 0xFFu));
            }
          }
        }
        if (rs > 0 && !E8) {
          const int q = rs - 1;
#pragma unroll
          for (int cs = 0; cs < 4; ++cs) {
            const float sc = scv[(NSET == 2 && cs >= 2) ? 1 : 0][q >> 2][q & 3];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[q][cs][v] = __builtin_fmaf(p[q & 1][cs][v], sc, acc[q][cs][v]);
          }
        }
        // One wave per SIMD: the matrix core only overlaps vector ALU work
        // that sits between MFMAs in the instruction stream, so interleave
        // each MFMA with a share of the promotion FMAs, LDS reads and loads.
        if (rs < RS) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      pin_acc();
    } else {
      v4i a[2][4];
      auto lda = [&](int rs) __attribute__((always_inline)) {
        const uint32_t ao = so + rs * 16 * AB;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[rs & 1][i] = lds_ld<v4i>(lds, a_rd[i] + ao);
      };
      lda(0);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        __builtin_amdgcn_sched_barrier(0);
        issue_share(rs);
        if (rs + 1 < RS) lda(rs + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int cs = 0; cs < 4; ++cs)
            acc[rs][cs] = mfma_bf16(as_v8bf(a[rs & 1][i]), as_v8bf(b.d[cs][i]), acc[rs][cs]);
      }
      __builtin_amdgcn_sched_barrier(0);
      pin_acc();
    }
  };

  // ---- main loop.  A (PD + 1 LDS stages, direct loads) is loaded PD steps
  // ahead, the activation scales PD + 1 steps ahead, B NBUF - 1 steps ahead
  // (NBUF register buffers).  Step s: read the scales of s+1, compute s while
  // issuing scale(s+PD+1), A(s+PD) and B(s+NBUF-1), spread over the compute,
  // publish the row scales of s+1, then a barrier that first waits until
  // only the loads of the last PD-1 steps may still be in flight: A(s+1) has
  // then landed in LDS for every wave, and so has scale(s+2).  The vector
  // memory counter completes in order, so every load gets about PD-1 steps
  // of latency.  Loads for steps past the end are issued anyway (buffer
  // loads past a buffer's end read zero, and those stages are never
  // computed): the step stays straight-line, which keeps the compiler's wait
  // counts exact.  The prologue issues its loads in the steady state's order
  // and group sizes, so the barrier's count means the same from step 0 on.
  constexpr int NSA = (AF == ACT_FP8) ? 1 : 0;
  constexpr int NLOAD = NSA + NDMA + NB;           // global loads issued per step
  static_assert((PD - 1) * NLOAD < 64 && PD * NLOAD < 64, "vmcnt range");
  static_assert(NBUF - 1 == PD || NSA == 0, "with activation scales, B runs PD steps ahead");
  BFrag bb[NBUF];
  auto issue_a = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) dma_a(s, s % AST, j);
  };
  auto load_b = [&](int s, BFrag& b) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NB; ++q) load_b_piece(s, b, q);
  };
  // Prologue: scale(0), then groups v = 0..PD-1 of {scale(v+1), A(v), B(v)
  // if v < NBUF-1}.  (sched_barrier keeps the compiler from reordering the
  // groups, which would make its wait counts for B at the loop head nearly a
  // full drain.)
  if (NSA) dma_sa(0, 0);
#pragma unroll
  for (int v = 0; v < PD; ++v) {
    if (NSA) dma_sa(v + 1, (v + 1) % AST);
    issue_a(v);
    __builtin_amdgcn_sched_barrier(0);
    if (v < NBUF - 1) load_b(v, bb[v]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // loads issued after scale(0), and after the last load of A(0)
  constexpr int AFTER_SA0 = PD * (NSA + NDMA) + (NBUF - 1 < PD ? NBUF - 1 : PD) * NB;
  constexpr int AFTER_A0 = AFTER_SA0 - NSA - NDMA;
  static_assert(AFTER_SA0 < 64, "vmcnt range");
  if (NSA) {
    wait_vmcnt<AFTER_SA0>();                       // scale(0) is in LDS
    store_scale(0, 0, read_sa(0));
  }
  barrier_vmcnt<AFTER_A0>();                       // A(0) is in LDS for every wave
  if (signal_prev && tid == 0) __hip_atomic_fetch_add(signal_prev, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // The loop body is UNR steps, a multiple of NBUF (B buffer rotation), of
  // 2 (scale parity) and of AST (A stage and scale slot rotation), so
  // every buffer and LDS slot index in it is a compile-time constant; a long
  // body also makes the loop head, where the compiler's wait counts are
  // merged from two paths and come out conservative, rarer.  Step s reads
  // the scales of step s+1 into a register within the step: no loaded value
  // is carried across the loop's back edge, where the compiler would drain
  // every load in flight.
  constexpr int UNR = (AF == ACT_FP8) ? (AST == 4 ? 16 : 12) : 6;
  static_assert(UNR % NBUF == 0 && UNR % 2 == 0 && UNR % AST == 0, "loop unroll");
  auto step = [&](int s, int u) __attribute__((always_inline)) {
    const float sa_next = read_sa((u + 1) % AST);
    compute(u % AST, u & 1, bb[u % NBUF], NLOAD, [&](int j) __attribute__((always_inline)) {
      if (j < NSA) dma_sa(s + PD + 1, (u + PD + 1) % AST);
      else if (j < NSA + NDMA) dma_a(s + PD, (u + PD) % AST, j - NSA);
      else load_b_piece(s + NBUF - 1, bb[(u + NBUF - 1) % NBUF], j - NSA - NDMA);
    });
    store_scale(s + 1, (u + 1) & 1, sa_next);
    barrier_vmcnt<(PD - 1) * NLOAD>();
  };
  for (int s = 0; s < nsteps; s += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (u > 0 && s + u >= nsteps) break;
      step(s + u, u);
    }
  }
  wait_vmcnt<0>();                                 // the last steps' overrun loads
  __syncthreads();
  at_loop_end();

  // ---- epilogues (the A stages are reused as the output staging tile)
  const uint32_t nrows = (uint32_t)(g.T * g.k);
  const rsrc_t aqw = make_rsrc(g.aq, nrows * (uint32_t)g.I * ESZ);
  const rsrc_t saw = make_rsrc(g.sa, nrows * (uint32_t)(g.I / 128) * 4);
  const rsrc_t stw = make_rsrc(g.staging, nrows * (uint32_t)((g.H + 255) / 256) * 512u);
  if (STAGE == 1) {
    if (WF == W_FP8 && AF == ACT_FP8 && wchan) {
      // per-channel weight scales: lane holds channels 32w + 16q + 4gq + v
      // of the item's gate (acc[rs][q]) and up (acc[rs][2 + q]) columns
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const v4f sg = lds_ld<v4f>(lds, L::kScw + (32 * w + 16 * q + 4 * gq) * 4);
        const v4f su = lds_ld<v4f>(lds, L::kScw + (128 + 32 * w + 16 * q + 4 * gq) * 4);
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[rs][q][v] *= sg[v];
            acc[rs][2 + q][v] *= su[v];
          }
      }
    }
    // a = SiLU(g) * u, written over the gate accumulators: av[rs][q] = acc[rs][q]
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc[rs][q][v], uv = acc[rs][2 + q][v];
          acc[rs][q][v] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        }
    }
    auto av = [&](int rs, int q, int v) __attribute__((always_inline)) { return acc[rs][q][v]; };
    if (AF == ACT_FP8) {
      // lane: row rs*16 + c16, channels 32w + 16q + 4gq + v of the item's 128
      float* RSC = reinterpret_cast<float*>(lds + L::kRsc);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        float mx = 0.f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx = fmaxf(mx, fabsf(av(rs, q, v)));
        mx = max_row_groups(mx);
        if (gq == 0) lds_st(lds, L::kAmax + (w * L::kRows + rs * 16 + c16) * 4, mx);
      }
      __syncthreads();
      if (tid < R) {
        const float* AMAX = reinterpret_cast<const float*>(lds + L::kAmax);
        const float mx = fmaxf(fmaxf(AMAX[tid], AMAX[L::kRows + tid]),
                               fmaxf(AMAX[2 * L::kRows + tid], AMAX[3 * L::kRows + tid]));
        float sc, inv;
        block_scale(mx, g.pow2 != 0, &sc, &inv);
        RSC[tid] = sc;
        reinterpret_cast<float*>(lds + L::kRinv)[tid] = inv;
      }
      __syncthreads();
      // Staging rows of 128 codes hold their 16-byte chunks permuted: chunk c
      // of row r at c ^ ((r >> 1) & 7), so that the 16 rows of one 4-byte
      // write (one per lane group position) spread over the LDS banks.
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        const int r = rs * 16 + c16;
        const float inv = lds_ld<float>(lds, L::kRinv + r * 4);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t codes = f32x4_to_e4m3x4(av(rs, q, 0) * inv, av(rs, q, 1) * inv, av(rs, q, 2) * inv,
                                                 av(rs, q, 3) * inv);
          lds_st(lds, L::kA + r * 128 + (((2 * w + q) ^ ((r >> 1) & 7)) << 4) + 4 * gq, codes);
        }
      }
      __syncthreads();
      copy_pieces<R * 8, CP>(aqw, lds, [&](int q, uint32_t* lo, uint32_t* go) {
        const int row = q >> 3, c = q & 7;
        *lo = L::kA + row * 128 + ((c ^ ((row >> 1) & 7)) << 4);
        *go = (uint32_t)(r0 + row) * g.I + c0 + c * 16;
        return row < m;
      });
      if (tid < m) buf_stf<CP>(saw, ((uint32_t)(c0 / 128) * nrows + (uint32_t)(r0 + tid)) * 4, RSC[tid]);
    } else {
      // chunk c of staging row r at c ^ (((r >> 2) & 3) << 1) (bank spread)
      const uint32_t lo = 2 * (c16 & 7), hc = c16 >> 3;
      const uint32_t wr0 = opaque(L::kA + 4 * gq * 256 + 16 * ((4 * w + hc) ^ (2 * gq)) + lo);
      const uint32_t wr1 = opaque(L::kA + 4 * gq * 256 + 16 * ((4 * w + 2 + hc) ^ (2 * gq)) + lo);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          lds_st(lds, wr0 + (rs * 16 + v) * 256, (uint16_t)f32_to_bf16_rne(av(rs, 0, v)));
          lds_st(lds, wr1 + (rs * 16 + v) * 256, (uint16_t)f32_to_bf16_rne(av(rs, 1, v)));
        }
      __syncthreads();
      copy_pieces<R * 16, CP>(aqw, lds, [&](int q, uint32_t* lo, uint32_t* go) {
        const int row = q >> 4, c = q & 15;
        *lo = L::kA + row * 256 + (c ^ (((row >> 2) & 3) << 1)) * 16;
        *go = ((uint32_t)(r0 + row) * g.I + c0) * 2 + c * 16;
        return row < m;
      });
    }
  } else if (AF == ACT_FP8) {
    if (WF == W_FP8 && wchan) {
      // per-channel weight scales of the lane's columns 64w + 16cs + 4gq + v
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        const v4f sn = lds_ld<v4f>(lds, L::kScw + (64 * w + 16 * cs + 4 * gq) * 4);
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rs][cs][v] *= sn[v];
      }
    }
    // lane: row rs*16 + c16, columns 64w + 16cs + 4gq + v of the N block.
    // The whole tile (up to 128 rows x 256 columns of BF16 = 64 KB, the A
    // stages' space) is staged at once; chunk c (16 bytes) of staging row r
    // at c ^ (r & 15), so that the 16 rows of one 8-byte write spread over
    // the LDS banks.
    constexpr int CH = RS;
    static_assert(CH * 16 * 512 <= L::kAStages * L::kASlot, "staging fits the A stages");
#pragma unroll
    for (int h = 0; h < RS / CH; ++h) {
      if (h > 0) __syncthreads();                  // previous chunk's copy-out is done
#pragma unroll
      for (int rs = CH * h; rs < CH * h + CH; ++rs) {
        const int rl = (rs - CH * h) * 16 + c16;
        const float rw = lds_ld<float>(lds, L::kRowW + (rs * 16 + c16) * 4);
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
          const uint32_t lo = bf16x2_rne(acc[rs][cs][0] * rw, acc[rs][cs][1] * rw);
          const uint32_t hi = bf16x2_rne(acc[rs][cs][2] * rw, acc[rs][cs][3] * rw);
          const int c = 8 * w + 2 * cs + (gq >> 1);
          lds_st(lds, L::kA + rl * 512 + ((c ^ (rl & 15)) << 4) + 8 * (gq & 1), v2u{lo, hi});
        }
      }
      __syncthreads();
      copy_pieces<CH * 16 * 32, CP>(stw, lds, [&](int q, uint32_t* lo, uint32_t* go) {
        const int rl = q >> 5, c = q & 31;
        const int row = CH * 16 * h + rl, col = n0 + c * 8;
        *lo = L::kA + rl * 512 + ((c ^ (rl & 15)) << 4);
        *go = (((uint32_t)nb * nrows + (uint32_t)ROWI[row]) * 256u + (uint32_t)(c * 8)) * 2;
        return row < m && col < g.H;
      });
    }
  } else {
    // BF16 activations (product not transposed): lane holds rows 4gq + v,
    // column 16cs + c16 of its 64.  Chunks of CH row subtiles (at most 64
    // rows x 256 columns of BF16 = 32 KB); chunk c of staging row r at
    // c ^ (((r >> 2) & 3) << 1) (bank spread).
    constexpr int CH = (RS < 4) ? RS : 4;
    uint32_t wrc[4];
#pragma unroll
    for (int cs = 0; cs < 4; ++cs)
      wrc[cs] = opaque(L::kA + 4 * gq * 512 + 16 * ((8 * w + 2 * cs + (c16 >> 3)) ^ (2 * gq)) + 2 * (c16 & 7));
    const uint32_t roww_rd = opaque(L::kRowW + 16 * gq);
#pragma unroll
    for (int h = 0; h < RS / CH; ++h) {
      if (h > 0) __syncthreads();                  // previous chunk's copy-out is done
#pragma unroll
      for (int rs = CH * h; rs < CH * h + CH; ++rs)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float rw = lds_ld<float>(lds, roww_rd + (rs * 16 + v) * 4);
#pragma unroll
          for (int cs = 0; cs < 4; ++cs)
            lds_st(lds, wrc[cs] + ((rs - CH * h) * 16 + v) * 512,
                   (uint16_t)f32_to_bf16_rne(acc[rs][cs][v] * rw));
        }
      __syncthreads();
      copy_pieces<CH * 16 * 32, CP>(stw, lds, [&](int q, uint32_t* lo, uint32_t* go) {
        const int rl = q >> 5, c = q & 31;
        const int row = CH * 16 * h + rl, col = n0 + c * 8;
        *lo = L::kA + rl * 512 + (c ^ (((rl >> 2) & 3) << 1)) * 16;
        *go = (((uint32_t)nb * nrows + (uint32_t)ROWI[row]) * 256u + (uint32_t)(c * 8)) * 2;
        return row < m && col < g.H;
      });
    }
  }
}

// Dispatch a tile to the GEMM variant with the tile's number of row subtiles.
template <int AF, int WF, int STAGE, int COH, int E8, typename Hook>
DEV void expert_gemm_rs(const GemmArgs& g, const Tile& t, int nb, char* lds, int32_t* signal_prev,
                        const Hook& at_loop_end) {
  constexpr int FULL = GemmLds<AF>::kMaxRs;
  if (t.rs <= 1)
    expert_gemm_tile<AF, WF, STAGE, 1, COH, E8>(g, t.e, t.r0, t.rows, nb, lds, signal_prev, at_loop_end);
  else if (t.rs <= 4)
    expert_gemm_tile<AF, WF, STAGE, 4, COH, E8>(g, t.e, t.r0, t.rows, nb, lds, signal_prev, at_loop_end);
  else if (FULL > 8 && t.rs <= 8)
    expert_gemm_tile<AF, WF, STAGE, (FULL > 8 ? 8 : FULL), COH, E8>(g, t.e, t.r0, t.rows, nb, lds, signal_prev,
                                                                    at_loop_end);
  else
    expert_gemm_tile<AF, WF, STAGE, FULL, COH, E8>(g, t.e, t.r0, t.rows, nb, lds, signal_prev, at_loop_end);
}
template <int AF, int WF, int STAGE, int COH, typename Hook = NoHook>
DEV void expert_gemm_item(const GemmArgs& g, const Tile& t, int nb, char* lds, int32_t* signal_prev = nullptr,
                          const Hook& at_loop_end = Hook{}) {
  // FP4 weights with power-of-two activation scales (the intermediate for
  // the down GEMM, the layer's own input quantisation for gate|up)
  const bool e8 = (STAGE == 1) ? g.pow2_x != 0 : g.pow2 != 0;
  if (WF == W_FP4 && AF == ACT_FP8 && e8)
    expert_gemm_rs<AF, WF, STAGE, COH, (WF == W_FP4 && AF == ACT_FP8) ? 1 : 0>(g, t, nb, lds, signal_prev, at_loop_end);
  else
    expert_gemm_rs<AF, WF, STAGE, COH, 0>(g, t, nb, lds, signal_prev, at_loop_end);
}

// y[t, n0:n1] = BF16( sum_j staging[t*k + j, n0:n1] ) for tokens [t0, t1),
// fp32 sums in ascending j; 8 channels (16 bytes) per thread and step.
// Staging is N-block major ([H/256][T*k][256]), so the k rows of a token in
// one N block, and the rows of consecutive tokens, are adjacent: a combine
// item reads one contiguous run per N block.
// Ordinary loads also in the persistent kernel: a 128-byte line of staging
// lies in one (row, 256-column block), written once per launch, write-through,
// before the block's counter that the caller waits for.
DEV void combine_rows(const uint16_t* staging, uint16_t* y, int T, int H, int k, int t0, int t1, int n0, int n1) {
  const uint32_t P = (uint32_t)T * (uint32_t)k;
  const rsrc_t srs = make_rsrc_u(staging, P * (uint32_t)((H + 255) / 256) * 512u);
  const int cpt = (n1 - n0) / 8;
  const int total = (t1 - t0) * cpt;
  // U (token, 8-channel) pairs per thread and pass, rows read four j at a
  // time: up to 16 loads in flight per thread
  constexpr int U = 4;
  const int nthr = blockDim.x;
  for (int i0 = threadIdx.x; i0 < total; i0 += U * nthr) {
    uint32_t off[U];
    int tt[U], cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = min(i0 + u * nthr, total - 1);
      tt[u] = t0 + idx / cpt;
      cc[u] = n0 + (idx % cpt) * 8;
      off[u] = (((uint32_t)(cc[u] >> 8) * P + (uint32_t)tt[u] * (uint32_t)k) * 256u + (uint32_t)(cc[u] & 255)) * 2;
    }
    float s[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) s[u][i] = 0.f;
    auto add = [&](int u, const v4i& v) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[u][2 * i] += bf16_to_f32((uint32_t)v[i] & 0xFFFFu);
        s[u][2 * i + 1] += bf16_to_f32((uint32_t)v[i] >> 16);
      }
    };
    const uint32_t row = 512u;                     // staging rows of one N block are adjacent
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      v4i v[4][U];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int u = 0; u < U; ++u) v[jj][u] = buf_ld16(srs, off[u] + (uint32_t)(j + jj) * row, 0);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int u = 0; u < U; ++u) add(u, v[jj][u]);
    }
    for (; j < k; ++j) {
      v4i v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = buf_ld16(srs, off[u] + (uint32_t)j * row, 0);
#pragma unroll
      for (int u = 0; u < U; ++u) add(u, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * nthr >= total) continue;
      v4i o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (int)bf16x2_rne(s[u][2 * i], s[u][2 * i + 1]);
      st16(reinterpret_cast<uint8_t*>(y) + ((size_t)tt[u] * H + cc[u]) * 2, o);
    }
  }
}

}  // namespace moe
