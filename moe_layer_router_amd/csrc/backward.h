// Backward pass of the MoE layer for BF16 layers, with the routing of the
// forward pass held fixed and the forward pass's roundings passed straight
// through (the layer's gradient as a trainable layer: the model-layer bullet
// of the "Tile Kernels" section of youleyou, "DeepSeek 模型更新解读 Tile
// Kernels 与 DeepEP V2 新特性"; DeepEP V2's training workload in the same
// page's "DeepEP V2" section).
//
// With P = T*k permuted rows (row p holding flat index perm[p] = t*k + j of
// token t = tok(p) and expert e), the backward pass is seven grouped GEMMs
// with fp32 accumulation, and three small kernels:
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
// The GEMM: one workgroup of 256 threads (four waves) computes a 64 x 128
// tile of C; wave w owns columns 32w..32w+31 (4 x 2 tiles of 16 x 16, the
// 16x16x32 BF16 MFMA).  A and B tiles of 32 K go to LDS as [row][32 K] with
// rows padded to 80 bytes (the 16 rows of one operand read fall in distinct
// banks); the next step's global loads are issued before the current step's
// MFMAs.  Operands are described as stored matrices S[r][c] with a leading
// dimension, optionally transposed, and with an optional map of the stored
// row (row' = map[row] / div: the permuted row to its token).  B is BF16
// (inputs and weights, exact).  A is BF16 too, or an fp32 intermediate
// (dG|dU, w a, dl), which the tile splits into two BF16 parts, hi = bf16(v)
// and lo = bf16(v - hi), with one MFMA each: v - hi - lo is below 2^-17 |v|,
// so the product is as accurate as the fp32 value (a single BF16 rounding of
// these operands would put a 2^-9 relative error on every term of the weight
// gradients' sums).
#pragma once
#include "device_common.h"
#include "permute.h"

namespace moe {

struct BwdOperand {
  const void* p;           // BF16 storage (fp32 for a split A operand)
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
};

constexpr int kBwdBM = 64, kBwdBN = 128, kBwdBK = 32;
constexpr int kBwdRow = 40;                              // padded LDS row, in BF16 elements (80 bytes)
constexpr int kBwdAStage = kBwdBM * kBwdRow;             // elements
constexpr int kBwdBStage = kBwdBN * kBwdRow;
constexpr int kBwdLds = 2 * (2 * kBwdAStage + kBwdBStage) * 2;   // bytes: two stages of A hi, A lo and B

// Load one piece (8 BF16) of a 32-K step of operand `o`: the tile of ROWS
// logical rows (M rows of A, N columns of B) x 32 K starting at (row0, k0).
// Logical (row, k) is stored at (row, k) when k-contiguous (`kc`), else at
// (k, row); a K-grouped operand's stored K index is offset by kb.  Thread
// piece i: k-contiguous, row i / 4 and K 8 (i % 4) .. +7; otherwise K
// i / (ROWS/8) and rows 8 (i % (ROWS/8)) .. +7.  Either way the 8 values are
// 8 consecutive columns of one stored row: one 16-byte load when they are
// all in range and aligned, else element by element.  Values outside the
// logical [row0, nrows) x [k0, nk) are 0.
template <int ROWS, typename TE>
DEV void bwd_load_piece(const BwdOperand& o, const TE* base, bool kc, int piece, long row0, long nrows, long k0,
                        long nk, long kb, TE (&v)[8]) {
  long srow, col, clim;
  bool ok;
  if (kc) {
    const long gr = row0 + piece / 4, gk = k0 + (piece % 4) * 8;
    ok = gr < nrows;
    srow = gr;
    col = gk;
    clim = nk;
  } else {
    constexpr int PR = ROWS / 8;                   // pieces per K row
    const long gk = k0 + piece / PR, gr = row0 + (piece % PR) * 8;
    ok = gk < nk;
    srow = kb + gk;
    col = gr;
    clim = nrows;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = TE(0);
  if (!ok) return;
  const long rr = o.map ? (long)(o.map[srow] / o.div) : srow;
  const TE* src = base + rr * o.ld;
  if (col + 8 <= clim && (o.ld % 8) == 0 && (col % 8) == 0) {
    constexpr int NV = 8 * (int)sizeof(TE) / 16;   // 16-byte loads
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const v4i w = *reinterpret_cast<const v4i*>(src + col + q * (16 / (int)sizeof(TE)));
      __builtin_memcpy(&v[q * (16 / (int)sizeof(TE))], &w, 16);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (col + i < clim) ? src[col + i] : TE(0);
}

DEV v4i bwd_pack(const uint16_t (&v)[8]) {
  v4i out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = (int)((uint32_t)v[2 * i] | ((uint32_t)v[2 * i + 1] << 16));
  return out;
}

// Store a piece loaded by bwd_load_piece into the LDS tile [ROWS][kBwdRow].
template <int ROWS>
DEV void bwd_store_piece(uint16_t* tile, bool kc, int piece, const v4i& q) {
  if (kc) {
    const int r = piece / 4, k = (piece % 4) * 8;
    *reinterpret_cast<v4i*>(tile + r * kBwdRow + k) = q;
  } else {
    constexpr int PR = ROWS / 8;
    const int k = piece / PR, r = (piece % PR) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[(r + 2 * i) * kBwdRow + k] = (uint16_t)((uint32_t)q[i] & 0xFFFFu);
      tile[(r + 2 * i + 1) * kBwdRow + k] = (uint16_t)((uint32_t)q[i] >> 16);
    }
  }
}

template <int AF32>
__global__ void __launch_bounds__(256) k_bwd_gemm(BwdGemm g) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint16_t* As = reinterpret_cast<uint16_t*>(lds);     // [2 stages][hi, lo]
  uint16_t* Bs = As + 4 * kBwdAStage;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, gq = lane >> 4;

  // ---- this block's group and tile
  long m0, M, k_base = 0, K = g.K;
  const uint16_t* abase = static_cast<const uint16_t*>(g.a.p);
  const float* abase32 = static_cast<const float*>(g.a.p);
  const uint16_t* bbase = static_cast<const uint16_t*>(g.b.p);
  float* cbase = g.c;
  const long n0 = (long)blockIdx.y * kBwdBN;
  if (g.group == BWD_GROUP_ROWS) {
    const int t = blockIdx.x;
    if (t >= *g.ntiles) return;
    const Tile tl = g.tiles[t];
    m0 = tl.r0;
    M = (long)tl.r0 + tl.rows;                     // rows [r0, r0 + rows) of the whole matrix
    bbase += (long)tl.e * g.b.gstride;
  } else {
    m0 = (long)blockIdx.x * kBwdBM;
    M = g.M;
    if (g.group == BWD_GROUP_K) {
      const int e = blockIdx.z;
      k_base = g.offsets[e];
      K = g.offsets[e + 1] - k_base;
      cbase += (long)e * g.c_gstride;
    }
  }
  const long N = g.N;
  // logical A(m, k): k-contiguous when not transposed; the K index of a
  // K-grouped operand is offset by the group's base (and mapped)
  const bool a_kc = !g.a.trans, b_kc = g.b.trans != 0;
  // A: logical rows m in [m0, M); mapped stored row = m (normal) or k_base + k (transposed)
  // B: logical rows n in [n0, N); stored row = n (transposed) or k_base + k (normal)

  // (K grouping is only used with A stored [K][M] and B stored [K][N], whose
  // stored row is the K index; a k-contiguous operand takes no K offset.)
  // A's piece as (hi, lo) BF16 parts (lo = 0 for a BF16 operand)
  auto load_a = [&](long k0, v4i* hi, v4i* lo) {
    if (AF32) {
      float v[8];
      bwd_load_piece<kBwdBM>(g.a, abase32, a_kc, tid, m0, M, k0, K, k_base, v);
      uint16_t h[8], l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        h[i] = (uint16_t)f32_to_bf16_rne(v[i]);
        l[i] = (uint16_t)f32_to_bf16_rne(v[i] - bf16_to_f32(h[i]));
      }
      *hi = bwd_pack(h);
      *lo = bwd_pack(l);
    } else {
      uint16_t h[8];
      bwd_load_piece<kBwdBM>(g.a, abase, a_kc, tid, m0, M, k0, K, k_base, h);
      *hi = bwd_pack(h);
      *lo = v4i{0, 0, 0, 0};
    }
  };
  auto load_b = [&](long k0, int half) -> v4i {
    uint16_t h[8];
    bwd_load_piece<kBwdBN>(g.b, bbase, b_kc, tid + 256 * half, n0, N, k0, K, k_base, h);
    return bwd_pack(h);
  };

  v4f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const long nsteps = (K + kBwdBK - 1) / kBwdBK;
  v4i pah, pal, pb0, pb1;
  load_a(0, &pah, &pal);
  pb0 = load_b(0, 0);
  pb1 = load_b(0, 1);
  for (long s = 0; s < nsteps; ++s) {
    uint16_t* ath = As + (s & 1) * 2 * kBwdAStage;
    uint16_t* atl = ath + kBwdAStage;
    uint16_t* bt = Bs + (s & 1) * kBwdBStage;
    bwd_store_piece<kBwdBM>(ath, a_kc, tid, pah);
    if (AF32) bwd_store_piece<kBwdBM>(atl, a_kc, tid, pal);
    bwd_store_piece<kBwdBN>(bt, b_kc, tid, pb0);
    bwd_store_piece<kBwdBN>(bt, b_kc, tid + 256, pb1);
    __syncthreads();
    if (s + 1 < nsteps) {                          // next step's loads in flight during this step's MFMAs
      load_a((s + 1) * kBwdBK, &pah, &pal);
      pb0 = load_b((s + 1) * kBwdBK, 0);
      pb1 = load_b((s + 1) * kBwdBK, 1);
    }
    v8bf bf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bf[j] = as_v8bf(*reinterpret_cast<const v4i*>(bt + (32 * w + 16 * j + c16) * kBwdRow + 8 * gq));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8bf ah = as_v8bf(*reinterpret_cast<const v4i*>(ath + (16 * i + c16) * kBwdRow + 8 * gq));
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(ah, bf[j], acc[i][j]);
      if (AF32) {
        const v8bf al = as_v8bf(*reinterpret_cast<const v4i*>(atl + (16 * i + c16) * kBwdRow + 8 * gq));
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(al, bf[j], acc[i][j]);
      }
    }
  }
  // ---- store: lane holds rows 16i + 4gq + v, column 32w + 16j + c16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const long m = m0 + 16 * i + 4 * gq + v, n = n0 + 32 * w + 16 * j + c16;
        if (m < M && n < N) cbase[g.c_trans ? n * g.ldc + m : m * g.ldc + n] = acc[i][j][v];
      }
}

// Per permuted row p: a = SwiGLU(g, u) from GU (fp32), dw = <dAu_p, a>,
// dA = w_p dAu_p, dG = dA u SiLU'(g), dU = dA SiLU(g) (fp32 [P][2I]),
// Aw = w_p a (fp32 [P][I]), and dws[perm[p]] = dw (the flat index's weight
// gradient).  One workgroup per row; the dot product is summed in fp32 over
// the workgroup (per-thread partial sums in channel order, then a fixed tree).
__global__ void __launch_bounds__(256) k_bwd_rows(const float* GU, const float* dAu, const int32_t* perm,
                                                  const float* topk_w, int I, int P, float* dGU, float* Aw,
                                                  float* dws) {
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
    dGU[(size_t)p * 2 * I + i] = dA * uv * (sg * (1.0f + gv * (1.0f - sg)));
    dGU[(size_t)p * 2 * I + I + i] = dA * si;
    Aw[(size_t)p * I + i] = wp * a;
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
// the dense [T][E] gradient of the logits; the other entries are left as
// cleared.
__global__ void __launch_bounds__(256) k_bwd_router(const int32_t* ids, const float* topk_w, const float* dws,
                                                    int T, int E, int k, float* dl) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += topk_w[(size_t)t * k + j] * dws[(size_t)t * k + j];
  for (int j = 0; j < k; ++j) {
    const size_t f = (size_t)t * k + j;
    const int e = min(max(ids[f], 0), E - 1);
    const float v = topk_w[f] * (dws[f] - s);
    dl[(size_t)t * E + e] = v;
  }
}

// db[e] = sum_t dl[t][e] in ascending t, one thread per expert.
__global__ void __launch_bounds__(256) k_bwd_dbias(const float* dl, int T, int E, float* db) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int t = 0; t < T; ++t) s += dl[(size_t)t * E + e];
  db[e] = s;
}

// dx[t][h] = sum_j dXr[row_of[t*k + j]][h] (ascending j) + dxr[t][h].
__global__ void __launch_bounds__(256) k_bwd_dx(const float* dXr, const int32_t* row_of, const float* dxr, int T,
                                                int H, int k, float* dx) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * H) return;
  const int t = (int)(i / H), h = (int)(i % H);
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += dXr[(size_t)row_of[(size_t)t * k + j] * H + h];
  dx[i] = s + dxr[i];
}

// Fill n 32-bit words with zero.
__global__ void __launch_bounds__(256) k_bwd_zero(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace moe
