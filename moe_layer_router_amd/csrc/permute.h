// Dispatch as a local permutation: expert histogram, exclusive scan and a
// stable scatter into an expert-contiguous row order.
//
// On one GPU the cross-GPU dispatch of the pages becomes this permutation
// (机器之心, "DeepSeek悄悄更新：Mega MoE、FP4 Indexer来了", section "Mega MoE
// 是什么？": tokens are first dispatched to their experts; youleyou, "DeepSeek
// 模型更新解读 Tile Kernels 与 DeepEP V2 新特性", section "Tile Kernels", MoE
// routing bullet: token-to-expert mapping).  Permuted row r holds the flat
// index p = t*k + j; rows of one expert are contiguous and in ascending token
// order.  Everything is integer and deterministic: the only atomics are LDS
// counters and bit-ors whose results do not depend on their order.
#pragma once
#include "device_common.h"

namespace moe {

constexpr int kPermBlock = 256;      // tokens per histogram / scatter block
constexpr int kTileRows = 128;       // rows per GEMM tile

struct Tile {                        // one GEMM row tile: rows [r0, r0 + rows) of expert e
  int e, r0, rows, pad;
};

// Expert id of entry i, clamped into [0, E): ids produced by the router are
// always in range; given ids outside it are treated as E-1 so that every
// write stays inside its buffer.
DEV int expert_of(const int32_t* ids, size_t i, int E) { return min(max(ids[i], 0), E - 1); }

// Per-block expert histogram: blockcnt[b][e] = number of (t, j) with
// ids[t][j] == e for tokens t of block b.  LDS: E ints.
DEV void perm_count_block(const int32_t* ids, int T, int k, int E, int b, int32_t* blockcnt, int* lds) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) lds[e] = 0;
  __syncthreads();
  const int t0 = b * kPermBlock;
  const int n = min(kPermBlock, T - t0) * k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) atomicAdd(&lds[expert_of(ids, (size_t)t0 * k + i, E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blockcnt[(size_t)b * E + e] = lds[e];
  __syncthreads();
}

// Exclusive scans over blocks and experts, and the GEMM tile list.
//   base[b][e]   = first permuted row of expert e's rows from block b
//   offsets[e]   = first permuted row of expert e (offsets[E] = T*k)
//   tiles        = ceil(count_e / 128) tiles per expert, in expert order
//   meta[0]      = number of tiles
// LDS: 2*E + 64 ints.  Any workgroup size that is a multiple of 64.
DEV void perm_scan(const int32_t* blockcnt, int nblk, int E, int32_t* base, int32_t* offsets,
                   Tile* tiles, int32_t* meta, int* lds) {
  int* cnt = lds;
  int* toff = lds + E;
  int* scratch = lds + 2 * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = blockcnt[(size_t)b * E + e];
      base[(size_t)b * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  // each thread scans a contiguous run of experts, then a workgroup scan
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e_lo = min(E, (int)threadIdx.x * per), e_hi = min(E, e_lo + per);
  int rows = 0, ntile = 0;
  for (int e = e_lo; e < e_hi; ++e) {
    rows += cnt[e];
    ntile += (cnt[e] + kTileRows - 1) / kTileRows;
  }
  int tot_rows, tot_tiles;
  int rows_incl = block_inclusive_scan(rows, scratch, &tot_rows);
  int tiles_incl = block_inclusive_scan(ntile, scratch, &tot_tiles);
  int r = rows_incl - rows, tl = tiles_incl - ntile;
  for (int e = e_lo; e < e_hi; ++e) {
    const int c = cnt[e];
    cnt[e] = r;              // now the expert offset
    toff[e] = tl;
    r += c;
    tl += (c + kTileRows - 1) / kTileRows;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int off = cnt[e];
    const int c = ((e + 1 < E) ? cnt[e + 1] : tot_rows) - off;
    offsets[e] = off;
    for (int b = 0; b < nblk; ++b) base[(size_t)b * E + e] += off;
    int t = toff[e];
    for (int r0 = 0; r0 < c; r0 += kTileRows, ++t) tiles[t] = Tile{e, off + r0, min(kTileRows, c - r0), 0};
  }
  if (threadIdx.x == 0) {
    offsets[E] = tot_rows;
    meta[0] = tot_tiles;
  }
  __syncthreads();
}

// Stable scatter of block b: row base[b][e] + (rank of token t among the
// block's tokens choosing e) receives p = t*k + j.  The rank is a popcount
// of per-wave 64-bit membership masks built with LDS bit-ors.  Needs exactly
// 256 threads: wave w owns tokens 64w .. 64w+63 of the block.
// LDS: 4 * E * 8 bytes.
DEV void perm_scatter_block(const int32_t* ids, int T, int k, int E, int b, const int32_t* base,
                            int32_t* perm, int32_t* row_of, uint64_t* masks) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) masks[i] = 0ull;
  __syncthreads();
  const int t0 = b * kPermBlock;
  const int nt = min(kPermBlock, T - t0);
  const int tl = w * 64 + lane;
  const bool ok = tl < nt;
  if (ok)
    for (int j = 0; j < k; ++j)
      atomicOr((unsigned long long*)&masks[(size_t)w * E + expert_of(ids, (size_t)(t0 + tl) * k + j, E)],
               1ull << lane);
  __syncthreads();
  if (ok) {
    for (int j = 0; j < k; ++j) {
      const int e = expert_of(ids, (size_t)(t0 + tl) * k + j, E);
      int rank = __popcll(masks[(size_t)w * E + e] & ((1ull << lane) - 1ull));
      for (int u = 0; u < w; ++u) rank += __popcll(masks[(size_t)u * E + e]);
      const int r = base[(size_t)b * E + e] + rank;
      const int p = (t0 + tl) * k + j;
      perm[r] = p;
      if (row_of) row_of[p] = r;
    }
  }
  __syncthreads();
}

}  // namespace moe
