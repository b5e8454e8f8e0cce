// Backward pass of the MoE layer for BF16 layers, with the routing of the
// forward pass held fixed and the forward pass's roundings passed straight
// through (the layer's gradient as a trainable layer: the model-layer bullet
// of the "Tile Kernels" section of youleyou, "DeepSeek 模型更新解读 Tile
// Kernels 与 DeepEP V2 新特性"; DeepEP V2's training workload in the same
// page's "DeepEP V2" section).
//
// With P = T*k permuted rows (row p holding flat index perm[p] = t*k + j of
// token t = tok(p) and expert e), the backward pass is seven grouped GEMMs
// with fp32 accumulation, and small kernels (x and dy gathered into
// permuted row order for the weight-gradient products, the row and router
// steps, the sums):
//   GU   [P][2I] = x[tok(p)] W_gu[e]^T                   (recomputed linear 1)
//   dAu  [P][I]  = dy[tok(p)] W_d[e]                     (unweighted d intermediate)
//   rows:         a = SwiGLU(g, u), dw_p = <dAu_p, a>, dA = w_p dAu,
//                 dG|dU = (dA u SiLU'(g) | dA SiLU(g)), Aw = w_p a
//   dXr  [P][H]  = [dG|dU] W_gu[e]                       (linear-1 input gradient per row)
//   dW_gu[e]     = sum_p [dG|dU]_p^T x[tok(p)]           (K = the expert's rows)
//   dW_d[e]      = sum_p dy[tok(p)]^T Aw_p                (formed transposed: Aw is the fp32 operand)
//   router:       dl[t][e_j] = w_j (dw_j - sum_i w_i dw_i), db[e] = sum_t dl[t][e]
//   dW_r = dl^T x,  dxr = dl W_r
//   dx[t] = sum_j dXr[row(t, j)] + dxr[t]               (fp32, ascending j)
//
// The GEMM: one workgroup of 256 threads (four waves, 2 x 2) computes a
// 128 x 128 tile of C, each wave 64 x 64 (4 x 4 tiles of 16 x 16, the
// 16x16x32 BF16 MFMA), in steps of 64 K.  Operands are described as stored
// matrices S[r][c] with a leading dimension, optionally transposed, and with
// an optional map of the stored row of a K-contiguous operand (row' =
// map[row] / div: the permuted row to its token).  Each step's tiles go to
// LDS as [128 rows][64 K] BF16 with no padding; the 16-byte chunk c
// (K 8c..8c+7) of row r sits at chunk c ^ ((r ^ r/8) mod 8), so that the
// MFMA operand reads (16 B, 8 rows at a time), the K-contiguous stores (8
// chunks of one row) and the transposed stores (8 B, 8 rows apart) all fall
// in distinct banks.  A K-contiguous
// operand is staged as pieces of 8 K of one row; a transposed one (stored
// [K][rows]: the weight-gradient products and the weights used as their
// stored transpose) as 4 K x 8 rows per thread, loaded as four 16-byte runs
// of stored rows and transposed in registers into 8-byte stores.  The next
// step's global loads are in flight during the current step's MFMAs.
// B is BF16 (inputs and weights, exact).  A is BF16 too, or an fp32
// intermediate (dG|dU, w a, dl), which its producer stores as two BF16
// parts, hi = bf16(v) and lo = bf16(v - hi), multiplied with one MFMA each:
// v - hi - lo is below 2^-17 |v|, so the product is as accurate as the fp32
// value (a single BF16 rounding of these operands would put a 2^-9 relative
// error on every term of the weight gradients' sums).
//
// Workgroups take their tiles in an order made for the L2 of each of the
// eight XCDs (consecutive workgroup ids go to different XCDs): each XCD gets
// a contiguous range of the logical order, and in that order the row tiles
// of a grouped-row product come in pairs (an expert's 256-row average load
// is two tiles) that visit the column blocks together, so a pair reads the
// expert's weight column slab once and each row tile is reused by every
// column block while it stays in the cache.
#pragma once
#include "device_common.h"
#include "permute.h"

namespace moe {

struct BwdOperand {
  const void* p;           // BF16 storage (a split A operand: its hi part)
  const void* p_lo;        // a split A operand's lo part (same layout), else NULL
  long ld;                 // elements between stored rows
  int trans;               // A: stored [K][M] (else [M][K]); B: stored [N][K] (else [K][N])
  const int32_t* map;      // stored-row map, or NULL
  int div;                 // row' = map[row] / div
  long gstride;            // elements between groups (per-expert matrices), 0 for one matrix
};

enum { BWD_GROUP_NONE = 0, BWD_GROUP_ROWS = 1, BWD_GROUP_K = 2 };

struct BwdGemm {
  BwdOperand a, b;
  float* c;                // fp32 [M][N] row-major, ldc (c_trans: [N][M])
  int c_trans;
  long ldc;
  long c_gstride;          // per-group C stride (BWD_GROUP_K)
  int M, N, K;             // fixed dimensions (M unused with BWD_GROUP_ROWS, K unused with BWD_GROUP_K)
  int group;               // BWD_GROUP_*
  const Tile* tiles;       // BWD_GROUP_ROWS: row tiles (e, r0, rows), count at *ntiles
  const int32_t* ntiles;
  const int32_t* offsets;  // BWD_GROUP_K: [E+1] K range of group e
  long a_bytes, b_bytes;   // operand buffer sizes (A: each part; B: per group), for the direct-load kernel
  int gx, gy, gz;          // grouped rows: row-tile slots (a multiple of 16), column blocks;
                           // grouped K: row blocks, column blocks, groups (the grid holds
                           // gx * ceil(gy / kBwdTpb) * (gz rounded up to 8) workgroups);
                           // else row, column blocks
};

constexpr int kBwdBM = 128, kBwdBN = 128, kBwdBK = 64;
constexpr int kBwdTpb = 8;                               // column tiles per workgroup of a grouped-K product
constexpr int kBwdTile = 128 * 64;                       // BF16 elements of one staged operand tile
template <int AF32>
constexpr int bwd_lds_bytes() { return (AF32 ? 3 : 2) * kBwdTile * 2; }   // A hi, (A lo,) B

typedef int v2i __attribute__((ext_vector_type(2)));

DEV v4i bwd_pack(const uint16_t (&v)[8]) {
  v4i out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = (int)((uint32_t)v[2 * i] | ((uint32_t)v[2 * i + 1] << 16));
  return out;
}

// Element offset of chunk c (K 8c..8c+7) of row r in a staged tile.
DEV int bwd_off(int r, int c) { return r * 64 + ((c ^ ((r ^ (r >> 3)) & 7)) << 3); }

// This thread's place in a staged tile.  K-contiguous: pieces q = 0..3 are
// row tid/8 + 32q, chunk tid%8.  Transposed: K 4kq..4kq+3 (q-th: 4kq + q) of
// rows 8ro..8ro+7, with eight consecutive lanes on consecutive row octets
// (one 128-byte run of a stored row) and lanes 8 apart on the next K quad.
struct BwdPos {
  int kr, kc;        // K-contiguous: row of piece 0, chunk
  int ro, kq;        // transposed: row octet, K quad
};
DEV BwdPos bwd_pos(int tid) {
  const int lane = tid & 63, w = tid >> 6;
  return BwdPos{tid >> 3, tid & 7, (lane & 7) | ((w & 1) << 3), (lane >> 3) | ((w >> 1) << 3)};
}

// Where this thread's pieces of an operand come from, fixed for the whole
// K loop.  K-contiguous: the (mapped) stored row of each piece, -1 outside
// the tile's logical rows.  Transposed (never mapped): the first stored
// column of the row octet and how many of its 8 columns lie inside (0..8).
struct BwdSrc {
  long row[4];
  long col;
  int ncol;
};

DEV void bwd_src_init(const BwdOperand& o, bool kc, const BwdPos& ps, long row0, long nrows, BwdSrc& s) {
  if (kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long gr = row0 + ps.kr + 32 * q;
      s.row[q] = gr < nrows ? (o.map ? (long)(o.map[gr] / o.div) : gr) : -1;
    }
  } else {
    s.col = row0 + 8 * ps.ro;
    s.ncol = (int)min(max(nrows - s.col, 0L), 8L);
  }
}


// Eight consecutive BF16 elements from `src`, those at i >= n read as zero
// (n <= 0: all zero); `vec`: src is 16-byte aligned and n >= 8.
DEV v4i bwd_fetch(const uint16_t* src, int n, bool vec) {
  if (vec) return *reinterpret_cast<const v4i*>(src);
  uint16_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = i < n ? src[i] : (uint16_t)0;
  return bwd_pack(h);
}

// This thread's loads of the step at k0 of one 128 x 64 tile: K [k0, nk)
// (zero outside); a transposed operand's stored row is kb + K.
// `ald`: the leading dimension keeps every piece 16-byte aligned.
DEV void bwd_load_tile(const BwdOperand& o, const uint16_t* base, bool kc, bool ald, const BwdPos& ps,
                       const BwdSrc& s, long k0, long nk, long kb, v4i (&raw)[4]) {
  if (kc) {
    const long gk = k0 + 8 * ps.kc;
    const int n = (int)min(nk - gk, 8L);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      raw[q] = bwd_fetch(base + s.row[q] * o.ld + gk, s.row[q] < 0 ? 0 : n, ald && n == 8 && s.row[q] >= 0);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long gk = k0 + 4 * ps.kq + q;
      const bool in = gk < nk;
      raw[q] = bwd_fetch(base + (kb + gk) * o.ld + s.col, in ? s.ncol : 0, ald && in && s.ncol == 8);
    }
  }
}

// Store this thread's loads into a staged tile.
DEV void bwd_store_tile(uint16_t* tile, bool kc, const BwdPos& ps, const v4i (&raw)[4]) {
  if (kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<v4i*>(tile + bwd_off(ps.kr + 32 * q, ps.kc)) = raw[q];
  } else {
    // row 8ro + i takes element i of each of the 4 K: two 32-bit words
    const int c = ps.kq >> 1, half = 4 * (ps.kq & 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sh = 16 * (i & 1), wd = i >> 1;
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = ((uint32_t)raw[q][wd] >> sh) & 0xFFFFu;
      const v2i hv{(int)(h[0] | (h[1] << 16)), (int)(h[2] | (h[3] << 16))};
      *reinterpret_cast<v2i*>(tile + bwd_off(8 * ps.ro + i, c) + half) = hv;
    }
  }
}

// Units of S consecutive logical workgroups (a pair of row tiles, or one
// group) go round-robin to the eight XCDs (consecutive workgroup ids go to
// different XCDs): XCD x takes units x, x + 8, ..., each as S consecutive
// workgroups.  The grid holds a multiple of 8 units.
DEV void bwd_unit(long S, long& unit, long& inner) {
  const long b = blockIdx.x, x = b % 8, slot = b / 8;
  unit = 8 * (slot / S) + x;
  inner = slot % S;
}

// AF32: A has a lo part; CT: C is stored transposed ([N][M]).  The MFMA's
// first operand is the side whose index runs along C's rows in memory, so
// that each lane holds four consecutive elements of a C row: one 16-byte
// store.
template <int AF32, int CT>
__global__ void __launch_bounds__(256) k_bwd_gemm(BwdGemm g) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* Ah = reinterpret_cast<uint16_t*>(lds);
  uint16_t* Bs = Ah + kBwdTile;
  uint16_t* Al = Bs + kBwdTile;                  // fp32 A only
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, gq = lane >> 4, wm = w & 1, wn = w >> 1;

  // ---- this workgroup's group and tiles: nt column tiles n_first,
  // n_first + 128, ... of the same rows (grouped K: up to kBwdTpb of them,
  // so that the short K loops of the weight gradients run back to back with
  // the next tile's first loads in flight)
  long m0, M, n_first, k_base = 0, K = g.K;
  int nt = 1;
  const uint16_t* bbase = static_cast<const uint16_t*>(g.b.p);
  float* cbase = g.c;
  if (g.group == BWD_GROUP_ROWS) {
    long pair, inner;
    bwd_unit(2L * g.gy, pair, inner);
    const int t = (int)(2 * pair + (inner & 1));
    n_first = (inner >> 1) * kBwdBN;
    if (t >= *g.ntiles) return;
    const Tile tl = g.tiles[t];
    m0 = tl.r0;
    M = (long)tl.r0 + tl.rows;                   // rows [r0, r0 + rows) of the whole matrix
    bbase += (long)tl.e * g.b.gstride;
  } else if (g.group == BWD_GROUP_K) {
    const long gyb = (g.gy + kBwdTpb - 1) / kBwdTpb;
    long e, inner;
    bwd_unit((long)g.gx * gyb, e, inner);
    if (e >= g.gz) return;
    m0 = (inner % g.gx) * kBwdBM;
    const long nb = (inner / g.gx) * kBwdTpb;
    n_first = nb * kBwdBN;
    nt = (int)min((long)kBwdTpb, g.gy - nb);
    M = g.M;
    k_base = g.offsets[e];
    K = g.offsets[e + 1] - k_base;
    cbase += e * g.c_gstride;
  } else {
    m0 = ((long)blockIdx.x % g.gx) * kBwdBM;
    n_first = ((long)blockIdx.x / g.gx) * kBwdBN;
    M = g.M;
  }
  const long N = g.N;
  // K grouping is only used with A stored [K][M] and B stored [K][N], whose
  // stored row is the K index; a K-contiguous operand takes no K offset.
  const bool a_kc = !g.a.trans, b_kc = g.b.trans != 0;
  const bool a_ald = (g.a.ld % 8) == 0, b_ald = (g.b.ld % 8) == 0;
  const uint16_t* abase = static_cast<const uint16_t*>(g.a.p);
  const uint16_t* abase_lo = static_cast<const uint16_t*>(g.a.p_lo);
  const BwdPos ps = bwd_pos(tid);
  BwdSrc sa, sb;
  bwd_src_init(g.a, a_kc, ps, m0, M, sa);
  bwd_src_init(g.b, b_kc, ps, n_first, N, sb);

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Store the tile at column n0 and clear the sums.  CT: lane holds rows
  // m = 64wm + 16i + 4gq + v of column n = 64wn + 16j + c16, C[n][m..m+3];
  // else rows m = 64wm + 16i + c16 and columns n = 64wn + 16j + 4gq + v,
  // C[m][n..n+3].
  auto store_c = [&](long n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long r = CT ? n0 + 64 * wn + 16 * j + c16 : m0 + 64 * wm + 16 * i + c16;      // C's stored row
        const long c = CT ? m0 + 64 * wm + 16 * i + 4 * gq : n0 + 64 * wn + 16 * j + 4 * gq;
        const long R = CT ? N : M, Cn = CT ? M : N;
        if (r < R) {
          float* dst = cbase + r * g.ldc + c;
          if (c + 4 <= Cn && (g.ldc % 4) == 0 && (c % 4) == 0) {
            *reinterpret_cast<v4f*>(dst) = acc[i][j];
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (c + v < Cn) dst[v] = acc[i][j][v];
          }
        }
        acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
  };

  const long nsteps = (K + kBwdBK - 1) / kBwdBK;
  if (nsteps == 0) {                             // no rows in this group: zero gradients
    for (int t = 0; t < nt; ++t) store_c(n_first + (long)t * kBwdBN);
    return;
  }
  v4i ra[4], ral[4], rb[4];
  auto load = [&](long k0) {
    bwd_load_tile(g.a, abase, a_kc, a_ald, ps, sa, k0, K, k_base, ra);
    if (AF32) bwd_load_tile(g.a, abase_lo, a_kc, a_ald, ps, sa, k0, K, k_base, ral);
    bwd_load_tile(g.b, bbase, b_kc, b_ald, ps, sb, k0, K, k_base, rb);
  };
  load(0);
  // steps of all nt tiles in one loop: s = step of the tile at column n0
  const long total = nsteps * nt;
  long s = 0, n0 = n_first;
  for (long f = 0; f < total; ++f) {
    if (f > 0) __syncthreads();                  // every wave is done with the previous step's tiles
    bwd_store_tile(Ah, a_kc, ps, ra);
    if (AF32) bwd_store_tile(Al, a_kc, ps, ral);
    bwd_store_tile(Bs, b_kc, ps, rb);
    __syncthreads();
    if (f + 1 < total) {                         // next step's loads in flight during this step's MFMAs
      long s1 = s + 1;
      if (s1 == nsteps) {                        // the next tile's first step
        s1 = 0;
        bwd_src_init(g.b, b_kc, ps, n0 + kBwdBN, N, sb);
      }
      load(s1 * kBwdBK);
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      v8bf bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = as_v8bf(*reinterpret_cast<const v4i*>(Bs + bwd_off(64 * wn + 16 * j + c16, 4 * kh + gq)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = bwd_off(64 * wm + 16 * i + c16, 4 * kh + gq);
        const v8bf ah = as_v8bf(*reinterpret_cast<const v4i*>(Ah + off));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = CT ? mfma_bf16(ah, bf[j], acc[i][j]) : mfma_bf16(bf[j], ah, acc[i][j]);
        if (AF32) {
          const v8bf al = as_v8bf(*reinterpret_cast<const v4i*>(Al + off));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = CT ? mfma_bf16(al, bf[j], acc[i][j]) : mfma_bf16(bf[j], al, acc[i][j]);
        }
      }
    }
    if (++s == nsteps) {
      store_c(n0);
      s = 0;
      n0 += kBwdBN;
    }
  }
}

// ---------------------------------------------------------------------------
// The product with both operands K-contiguous and BF16 (the recomputed
// gate|up GEMM: gathered input rows times the expert's weight rows) with
// both operands loaded straight into LDS (buffer loads to LDS, no staging
// registers), kBwdNs stages deep, one barrier per 64-K step.  The tiles are
// [128 rows][64 K] with the chunk swizzle above, read with 16-byte loads.
// Rows past a tile's end read the tile's first row (their results are never
// stored).  Requires N a multiple of 128, K a multiple of 64, and buffers
// below 2 GiB (32-bit buffer offsets); grouped rows only.
constexpr int kBwdNs = 3;                                // LDS stages
constexpr int kBwdDmaLds = kBwdNs * 2 * kBwdTile * 2;    // bytes: A and B tiles per stage

__global__ void __launch_bounds__(256) k_bwd_gemm_dma(BwdGemm g) {
  constexpr int LA = 8;                                  // DMA instructions per wave per step
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, gq = lane >> 4, wm = w & 1, wn = w >> 1;

  long pair, inner;
  bwd_unit(2L * g.gy, pair, inner);
  const int t = (int)(2 * pair + (inner & 1));
  const long n0 = (inner >> 1) * kBwdBN;
  if (t >= *g.ntiles) return;
  const Tile tl = g.tiles[t];
  const long m0 = tl.r0, M = (long)tl.r0 + tl.rows, K = g.K;
  const uint16_t* bbase = static_cast<const uint16_t*>(g.b.p) + (long)tl.e * g.b.gstride;

  // DMA instruction q of wave w fills 1 KB u = 4q + w of a tile: rows
  // 8u + l/8, physical chunk l % 8, i.e. logical chunk (l % 8) ^ swz(row)
  const rsrc_t ars = make_rsrc(g.a.p, (uint32_t)g.a_bytes);
  const rsrc_t brs = make_rsrc(bbase, (uint32_t)g.b_bytes);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * (4 * q + w) + (lane >> 3), c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    const long ar = m0 + r < M ? m0 + r : m0;
    const long sr = g.a.map ? (long)(g.a.map[ar] / g.a.div) : ar;
    aoff[q] = (uint32_t)(sr * g.a.ld * 2 + 16 * c);
    boff[q] = (uint32_t)((n0 + r) * g.b.ld * 2 + 16 * c);
  }
  const long nsteps = K / kBwdBK;
  auto dma = [&](long s) {                       // step s (clamped) into stage s % kBwdNs
    const uint32_t k0b = (uint32_t)((s < nsteps ? s : nsteps - 1) * kBwdBK * 2);
    char* st = lds + (int)(s % kBwdNs) * 2 * kBwdTile * 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      char* dst = st + (4 * q + w) * 1024;
      buf_ld16_lds<0>(ars, dst, aoff[q], k0b);
      buf_ld16_lds<0>(brs, dst + kBwdTile * 2, boff[q], k0b);
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kBwdNs - 1; ++s) dma(s);
  for (long s = 0; s < nsteps; ++s) {
    // this wave's DMAs of step s are done (later steps' may still be in
    // flight), and every wave is past step s - 1
    barrier_vmcnt<(kBwdNs - 2) * LA>();
    dma(s + kBwdNs - 1);                         // into the stage step s - 1 used
    const uint16_t* At = reinterpret_cast<const uint16_t*>(lds + (int)(s % kBwdNs) * 2 * kBwdTile * 2);
    const uint16_t* Bt = At + kBwdTile;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      v8bf bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = as_v8bf(*reinterpret_cast<const v4i*>(Bt + bwd_off(64 * wn + 16 * j + c16, 4 * kh + gq)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v8bf ah = as_v8bf(*reinterpret_cast<const v4i*>(At + bwd_off(64 * wm + 16 * i + c16, 4 * kh + gq)));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(bf[j], ah, acc[i][j]);
      }
    }
  }
  wait_vmcnt<0>();                               // no DMA into LDS outlives the workgroup
  // lane holds rows m = 64wm + 16i + c16, columns n = 64wn + 16j + 4gq + v
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long m = m0 + 64 * wm + 16 * i + c16, n = n0 + 64 * wn + 16 * j + 4 * gq;
      if (m < M) *reinterpret_cast<v4f*>(g.c + m * g.ldc + n) = acc[i][j];
    }
}

// Store v as its hi = bf16(v) and lo = bf16(v - hi) parts.
DEV void bwd_split_store(uint16_t* hi, uint16_t* lo, size_t i, float v) {
  const uint32_t h = f32_to_bf16_rne(v);
  hi[i] = (uint16_t)h;
  lo[i] = (uint16_t)f32_to_bf16_rne(v - bf16_to_f32(h));
}

// Per permuted row p: a = SwiGLU(g, u) from GU (fp32), dw = <dAu_p, a>,
// dA = w_p dAu_p, dG = dA u SiLU'(g), dU = dA SiLU(g) ([P][2I]),
// Aw = w_p a ([P][I]), both as hi / lo BF16 parts, and dws[perm[p]] = dw
// (the flat index's weight gradient).  One workgroup per row; the dot
// product is summed in fp32 over the workgroup (per-thread partial sums in
// channel order, then a fixed tree).
__global__ void __launch_bounds__(256) k_bwd_rows(const float* GU, const float* dAu, const int32_t* perm,
                                                  const float* topk_w, int I, int P, uint16_t* dgu_hi,
                                                  uint16_t* dgu_lo, uint16_t* aw_hi, uint16_t* aw_lo, float* dws) {
  __shared__ float red[256];
  const int p = blockIdx.x;
  if (p >= P) return;
  const int fi = perm[p];
  const float wp = topk_w[fi];
  const float* gu = GU + (size_t)p * 2 * I;
  const float* da = dAu + (size_t)p * I;
  float part = 0.f;
  for (int i = threadIdx.x; i < I; i += blockDim.x) {
    const float gv = gu[i], uv = gu[I + i];
    const float sg = 1.0f / (1.0f + __expf(-gv));
    const float si = gv * sg;
    const float a = si * uv;
    const float d = da[i];
    part += d * a;
    const float dA = wp * d;
    bwd_split_store(dgu_hi, dgu_lo, (size_t)p * 2 * I + i, dA * uv * (sg * (1.0f + gv * (1.0f - sg))));
    bwd_split_store(dgu_hi, dgu_lo, (size_t)p * 2 * I + I + i, dA * si);
    bwd_split_store(aw_hi, aw_lo, (size_t)p * I + i, wp * a);
  }
  red[threadIdx.x] = part;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) dws[fi] = red[0];
}

// Router part, one thread per token: dl_j = w_j (dw_j - sum_i w_i dw_i) into
// the dense [T][E] gradient of the logits (hi / lo BF16 parts); the other
// entries are left as cleared.
__global__ void __launch_bounds__(256) k_bwd_router(const int32_t* ids, const float* topk_w, const float* dws,
                                                    int T, int E, int k, uint16_t* dl_hi, uint16_t* dl_lo) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += topk_w[(size_t)t * k + j] * dws[(size_t)t * k + j];
  for (int j = 0; j < k; ++j) {
    const size_t f = (size_t)t * k + j;
    const int e = min(max(ids[f], 0), E - 1);
    bwd_split_store(dl_hi, dl_lo, (size_t)t * E + e, topk_w[f] * (dws[f] - s));
  }
}

// db[e] = sum_t dl[t][e] (hi + lo parts): one workgroup per expert,
// per-thread sums over t = tid, tid + 256, ... in ascending t, then a fixed
// tree.
__global__ void __launch_bounds__(256) k_bwd_dbias(const uint16_t* dl_hi, const uint16_t* dl_lo, int T, int E,
                                                   float* db) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) {
    const size_t i = (size_t)t * E + e;
    s += bf16_to_f32(dl_hi[i]) + bf16_to_f32(dl_lo[i]);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) db[e] = red[0];
}

// dx[t][h] = sum_j dXr[row_of[t*k + j]][h] (ascending j) + dxr[t][h]: one
// thread per 4 consecutive h of one token (H is a multiple of 128).
__global__ void __launch_bounds__(256) k_bwd_dx(const float* dXr, const int32_t* row_of, const float* dxr, int T,
                                                int H, int k, float* dx) {
  const int H4 = H / 4;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * H4) return;
  const int t = (int)(i / H4), h = (int)(i % H4) * 4;
  v4f s = v4f{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) s += *reinterpret_cast<const v4f*>(dXr + (size_t)row_of[(size_t)t * k + j] * H + h);
  *reinterpret_cast<v4f*>(dx + (size_t)t * H + h) = s + *reinterpret_cast<const v4f*>(dxr + (size_t)t * H + h);
}

// out[p] = in[perm[p] / k] for the P permuted rows (BF16 rows of H, H a
// multiple of 8): the input and output gradient in permuted row order for
// the weight-gradient products.
__global__ void __launch_bounds__(256) k_bwd_gather(const uint16_t* in, const int32_t* perm, int k, int H, long P,
                                                    uint16_t* out) {
  const long H8 = H / 8;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < P * H8; i += (long)gridDim.x * blockDim.x) {
    const long p = i / H8, c = i % H8;
    *reinterpret_cast<v4i*>(out + p * H + 8 * c) =
        *reinterpret_cast<const v4i*>(in + (long)(perm[p] / k) * H + 8 * c);
  }
}

// Fill n 32-bit words with zero.
__global__ void __launch_bounds__(256) k_bwd_zero(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace moe
