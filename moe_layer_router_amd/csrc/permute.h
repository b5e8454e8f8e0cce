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
// counters and bit-ors whose results do not depend on their order.  Data
// handed from one step to the next (ids, block counts, bases, tiles) is
// written and read with device-coherent accesses, so that the persistent
// kernel orders the steps with relaxed counters and no device-wide fence.
#pragma once
#include "device_common.h"

namespace moe {

constexpr int kPermBlock = 256;      // tokens per histogram / scatter block
constexpr int kMinTileRows = 64;     // smallest full GEMM row tile (bounds the tile count)
constexpr int kSmallTileRows = 64;   // rows of the 4-subtile GEMM variant

// One GEMM row tile: rows [r0, r0 + rows) of expert e, computed by the GEMM
// variant with `rs` 16-row subtiles (the smallest of 1, 4 or the full tile
// that covers `rows`).  The tiles of one expert are g0 .. g0 + gn - 1.
struct Tile {
  int e, r0, rows, rs, g0, gn;
};
static_assert(sizeof(Tile) == 6 * sizeof(int32_t), "tile fields are stored one by one");

// Work item i of a GEMM over (tile, N block) pairs with nnb N blocks.  Items
// are ordered expert by expert; an expert's tiles in groups of up to
// kTileGroup, and within a group by N block, then tile.  The items reading
// the same weight slab (one N block of the group's tiles) and those reading
// the same rows (one tile's N blocks) are then all close in the queue and
// run at about the same time, so the later reads hit the caches.  Without
// the groups, an expert with hundreds of tiles (a popular expert under a
// skewed routing) would read each tile's rows once per N block, hundreds of
// items apart, long after the L2 dropped them.  An expert with at most
// kTileGroup tiles is one group: N block, then tile.
// (`tiles` is any pointer to Tile, also one into another address space.)
constexpr int kTileGroup = 4;
template <typename TilePtr>
DEV void gemm_item_of(TilePtr tiles, int nnb, int i, int* t, int* nb) {
  const int j = i / nnb;
  const int g0 = tiles[j].g0, gn = tiles[j].gn;
  const int local = i - g0 * nnb;
  const int q = local / (kTileGroup * nnb);          // group (all before it are full)
  const int r = local - q * kTileGroup * nnb;
  const int sz = min(kTileGroup, gn - q * kTileGroup);
  *nb = r / sz;
  *t = g0 + q * kTileGroup + r % sz;
}

// Variant (16-row subtiles computed) of a tile of `rows` rows whose full size
// is full_rs subtiles: 1, 4, 8 (when the full size is larger) or full_rs.
DEV int tile_variant(int rows, int full_rs) {
  return rows <= 16 ? 1 : rows <= 64 ? 4 : (full_rs > 8 && rows <= 128) ? 8 : full_rs;
}

// The c rows of expert e (permuted rows off .. off + c - 1) as
// gn = ceil(c / tile_rows) tiles g0, g0 + 1, ...  Full tiles and a remainder
// when the remainder fits the 64-row variant; otherwise gn tiles of equal
// size to one row.  Equal siblings run the same GEMM variant at the same
// speed: the items of one N block, adjacent in the queue, then stream the
// weight slab they share in step, and the later reads hit the L2 (a full
// tile and a remainder of more than 64 rows would drift apart by the
// remainder's shorter run time and miss).  A small remainder costs little
// either way, and equal tiles would compute more padded rows.
DEV void store_expert_tiles(Tile* tiles, int e, int off, int c, int g0, int tile_rows) {
  const int gn = (c + tile_rows - 1) / tile_rows;
  const bool even = gn > 1 && c - (gn - 1) * tile_rows > kSmallTileRows;
  const int q = even ? c / gn : tile_rows, rem = even ? c % gn : 0;
  for (int i = 0; i < gn; ++i) {
    const int r0 = i * q + min(i, rem);
    const int rows = min(q + (i < rem ? 1 : 0), c - r0);
    int32_t* tf = reinterpret_cast<int32_t*>(tiles + g0 + i);
    st_coh(tf + 0, e);
    st_coh(tf + 1, off + r0);
    st_coh(tf + 2, rows);
    st_coh(tf + 3, tile_variant(rows, tile_rows / 16));
    st_coh(tf + 4, g0);
    st_coh(tf + 5, gn);
  }
}

// Expert id of entry i, clamped into [0, E): ids produced by the router are
// always in range; given ids outside it are treated as E-1 so that every
// write stays inside its buffer.
DEV int expert_of(const int32_t* ids, size_t i, int E) { return min(max(ld_coh(ids + i), 0), E - 1); }

// cnt[e] += number of entries ids[i0 .. i0 + n) equal to e (LDS atomics),
// by the whole workgroup.  Each thread loads its (up to) 16 entries of a
// pass before counting any: a coherent load between LDS atomics would wait
// for the one before, one memory round trip per entry.
DEV void count_experts(const int32_t* ids, size_t i0, int n, int E, int* cnt) {
  constexpr int kU = 16;
  const int nthr = blockDim.x;
  for (int p0 = 0; p0 < n; p0 += kU * nthr) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) ev[u] = expert_of(ids, i0 + min(p0 + u * nthr + (int)threadIdx.x, n - 1), E);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (p0 + u * nthr + (int)threadIdx.x < n) atomicAdd(&cnt[ev[u]], 1);
  }
}

// Per-block expert histogram: blockcnt[b][e] = number of (t, j) with
// ids[t][j] == e for tokens t of block b.  LDS: E ints.
DEV void perm_count_block(const int32_t* ids, int T, int k, int E, int b, int32_t* blockcnt, int* lds) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) lds[e] = 0;
  __syncthreads();
  const int t0 = b * kPermBlock;
  count_experts(ids, (size_t)t0 * k, min(kPermBlock, T - t0) * k, E, lds);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) st_coh(blockcnt + (size_t)b * E + e, lds[e]);
  __syncthreads();
}

// Number of expert classes: expert e belongs to class e % kXcds, and the
// tiles of class x are worked on first by the workgroups of XCD x, so that
// sibling tiles of one expert (which read the same weights) share an L2.
constexpr int kXcds = 8;

DEV int class_pos(int e, int E8) { return (e % kXcds) * E8 + e / kXcds; }

// In-place exclusive scan of a[0..n) in LDS by the whole workgroup; returns
// the total.  Ends with a barrier.
DEV int lds_exclusive_scan(int* a, int n, int* scratch) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += a[i];
  int tot;
  int run = block_inclusive_scan(sum, scratch, &tot) - sum;
  for (int i = lo; i < hi; ++i) {
    const int c = a[i];
    a[i] = run;
    run += c;
  }
  __syncthreads();
  return tot;
}

// Exclusive scans over blocks and experts, and the GEMM tile list.
//   base[b][e]   = first permuted row of expert e's rows from block b
//   offsets[e]   = first permuted row of expert e (offsets[E] = T*k)
//   tiles        = ceil(count_e / tile_rows) tiles per expert (store_expert_tiles), ordered by
//                  expert class, then expert (each expert's tiles adjacent)
//   meta[0]      = number of tiles; meta[1 + x] = first tile of class x
//                  (x = 0 .. kXcds, the last entry equal to meta[0])
// LDS: (2*E + 8 + 64) ints.  Any workgroup size that is a multiple of 64.
DEV void perm_scan(const int32_t* blockcnt, int nblk, int E, int tile_rows, int32_t* base, int32_t* offsets,
                   Tile* tiles, int32_t* meta, int* lds) {
  const int E8 = (E + kXcds - 1) / kXcds;
  int* cnt = lds;                   // [E] rows per expert, then expert offsets
  int* tcl = lds + E;               // [kXcds * E8] tiles per expert in class order, then first tiles
  int* scratch = tcl + kXcds * E8;  // [64]
  // Blocks are read in batches of kBatch independent loads, so that the
  // per-expert walk over blocks is not a chain of dependent memory round
  // trips.  Pass 1: rows per expert.
  constexpr int kBatch = 16;
  for (int i = threadIdx.x; i < kXcds * E8; i += blockDim.x) tcl[i] = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        // (an in-range address, the value dropped after the load: a load
        // under a condition is a branch that waits for it)
        const int32_t v = ld_coh(blockcnt + (size_t)min(b0 + i, nblk - 1) * E + e);
        c[i] = (b0 + i < nblk) ? v : 0;
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) run += c[i];
    }
    cnt[e] = run;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) tcl[class_pos(e, E8)] = (cnt[e] + tile_rows - 1) / tile_rows;
  __syncthreads();
  const int tot_rows = lds_exclusive_scan(cnt, E, scratch);
  const int tot_tiles = lds_exclusive_scan(tcl, kXcds * E8, scratch);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int off = cnt[e];
    const int c = ((e + 1 < E) ? cnt[e + 1] : tot_rows) - off;
    st_coh(offsets + e, off);
    // pass 2: base[b][e] = off + rows of e in blocks before b
    int run = off;
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int cb[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        // (an in-range address, the value dropped after the load: a load
        // under a condition is a branch that waits for it)
        const int32_t v = ld_coh(blockcnt + (size_t)min(b0 + i, nblk - 1) * E + e);
        cb[i] = (b0 + i < nblk) ? v : 0;
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b0 + i < nblk) st_coh(base + (size_t)(b0 + i) * E + e, run);
        run += cb[i];
      }
    }
    store_expert_tiles(tiles, e, off, c, tcl[class_pos(e, E8)], tile_rows);
  }
  if (threadIdx.x == 0) {
    st_coh(offsets + E, tot_rows);
    st_coh(meta, tot_tiles);
    for (int x = 0; x < kXcds; ++x) st_coh(meta + 1 + x, tcl[x * E8]);
    st_coh(meta + 1 + kXcds, tot_tiles);
  }
  __syncthreads();
}

// Stable scatter of block b: row base(e) + (rank of token t among the
// block's tokens choosing e) receives p = t*k + j.  The rank is a popcount
// of per-wave 64-bit membership masks built with LDS bit-ors.  Needs exactly
// 256 threads: wave w owns tokens 64w .. 64w+63 of the block.
// LDS: 4 * E * 8 bytes.
template <typename BaseF>
DEV void scatter_block(const int32_t* ids, int T, int k, int E, int b, const BaseF& base_of, int32_t* perm,
                       int32_t* row_of, uint64_t* masks) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) masks[i] = 0ull;
  __syncthreads();
  const int t0 = b * kPermBlock;
  const int nt = min(kPermBlock, T - t0);
  const int tl = w * 64 + lane;
  const bool ok = tl < nt;
  // The token's experts, loaded once (k <= 16): every load from an in-range
  // address and all of them before any use (a load under a condition is a
  // branch that waits for it).
  int ev[16];
  const size_t ib = (size_t)min(t0 + tl, T - 1) * k;
#pragma unroll
  for (int j = 0; j < 16; ++j) ev[j] = expert_of(ids, ib + min(j, k - 1), E);
  if (ok)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) atomicOr((unsigned long long*)&masks[(size_t)w * E + ev[j]], 1ull << lane);
  __syncthreads();
  if (ok) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
      const int e = ev[j];
      int rank = __popcll(masks[(size_t)w * E + e] & ((1ull << lane) - 1ull));
      for (int u = 0; u < w; ++u) rank += __popcll(masks[(size_t)u * E + e]);
      const int r = base_of(e) + rank;
      const int p = (t0 + tl) * k + j;
      st_coh(perm + r, p);
      if (row_of) st_coh(row_of + p, r);
    }
  }
  __syncthreads();
}
DEV void perm_scatter_block(const int32_t* ids, int T, int k, int E, int b, const int32_t* base,
                            int32_t* perm, int32_t* row_of, uint64_t* masks) {
  scatter_block(ids, T, k, E, b, [&](int e) { return ld_coh(base + (size_t)b * E + e); }, perm, row_of, masks);
}

// Scan and stable scatter of block b in one step (persistent kernel): the
// block sums the histograms of all nblk blocks itself, both the rows per
// expert and the rows of each expert in blocks before b, so no separate scan
// step, with its hand-off through memory, sits between the histograms and
// the scatters.  With nblk == 1 the block counts its own tokens and needs no
// histogram step at all.  Block 0 also writes offsets, tiles and meta,
// exactly as perm_scan does.  LDS: 4*E*8 bytes + (2*E + 8*ceil(E/8) + 64)
// ints.  Needs exactly 256 threads.
DEV void perm_scan_scatter_block(const int32_t* ids, int T, int k, int E, int b, int nblk, const int32_t* blockcnt,
                                 int tile_rows, int32_t* offsets, Tile* tiles, int32_t* meta, int32_t* perm,
                                 int32_t* row_of, char* lds) {
  const int E8 = (E + kXcds - 1) / kXcds;
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds);
  int* cnt = reinterpret_cast<int*>(lds + (size_t)4 * E * 8);   // [E] rows per expert, then offsets
  int* pre = cnt + E;                                            // [E] rows of e in blocks before b
  int* tcl = pre + E;                                            // [kXcds * E8]
  int* scratch = tcl + kXcds * E8;                               // [64]
  if (nblk == 1) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) { cnt[e] = 0; pre[e] = 0; }
    __syncthreads();
    count_experts(ids, 0, min(kPermBlock, T) * k, E, cnt);
  } else {
    constexpr int kBatch = 16;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      int tot = 0, before = 0;
      for (int b0 = 0; b0 < nblk; b0 += kBatch) {
        int c[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          // (an in-range address, the value dropped after the load: a load
          // under a condition is a branch that waits for it)
          const int32_t v = ld_coh(blockcnt + (size_t)min(b0 + i, nblk - 1) * E + e);
          c[i] = (b0 + i < nblk) ? v : 0;
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          tot += c[i];
          if (b0 + i < b) before += c[i];
        }
      }
      cnt[e] = tot;
      pre[e] = before;
    }
  }
  __syncthreads();
  if (b == 0) {
    for (int i = threadIdx.x; i < kXcds * E8; i += blockDim.x) tcl[i] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) tcl[class_pos(e, E8)] = (cnt[e] + tile_rows - 1) / tile_rows;
    __syncthreads();
  }
  const int tot_rows = lds_exclusive_scan(cnt, E, scratch);      // cnt[e] = first row of expert e
  if (b == 0) {
    const int tot_tiles = lds_exclusive_scan(tcl, kXcds * E8, scratch);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      const int off = cnt[e];
      const int c = ((e + 1 < E) ? cnt[e + 1] : tot_rows) - off;
      st_coh(offsets + e, off);
      store_expert_tiles(tiles, e, off, c, tcl[class_pos(e, E8)], tile_rows);
    }
    if (threadIdx.x == 0) {
      st_coh(offsets + E, tot_rows);
      st_coh(meta, tot_tiles);
      for (int x = 0; x < kXcds; ++x) st_coh(meta + 1 + x, tcl[x * E8]);
      st_coh(meta + 1 + kXcds, tot_tiles);
    }
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) pre[e] += cnt[e];   // base of expert e in block b
  __syncthreads();
  scatter_block(ids, T, k, E, b, [&](int e) { return pre[e]; }, perm, row_of, masks);
}

// Activation scales in permuted row order, K block major: for permuted rows
// [r0, r1) (one per thread), sxp[s][r] = x_scales[perm[r] / k][s] for the
// ns = H/128 blocks, so that a GEMM tile reads the scales of its rows for
// one K step as one contiguous run.  The permutation is read coherently
// (written earlier in the same kernel) and the copy is stored write-through.
DEV void permute_scales(const int32_t* perm, const float* x_scales, int T, int k, int ns, int r0, int r1,
                        float* sxp) {
  const int n = T * k;
  for (int r = r0 + (int)threadIdx.x; r < r1; r += blockDim.x) {
    const int t = min(max(ld_coh(perm + r), 0), n - 1) / k;
    const float* src = x_scales + (size_t)t * ns;
    // A chunk of the row's scales is loaded before any of it is stored: the
    // stores could alias the source, so loads after a store would wait for
    // it, one round trip to memory per scale.  With ns a multiple of 4 (rows
    // 16-byte aligned) 16-byte loads: each lane reads another token's row,
    // so every load instruction touches 64 lines, and wider loads need 4x
    // fewer of them.
    if ((ns & 3) == 0) {
      constexpr int kChunk4 = 16;                    // 64 scales per chunk
      const float4* src4 = reinterpret_cast<const float4*>(src);
      const int ns4 = ns >> 2;
      for (int q0 = 0; q0 < ns4; q0 += kChunk4) {
        float4 v[kChunk4];
#pragma unroll
        for (int j = 0; j < kChunk4; ++j) v[j] = src4[min(q0 + j, ns4 - 1)];
#pragma unroll
        for (int j = 0; j < kChunk4; ++j) {
          if (q0 + j < ns4) {
            float* d = sxp + (size_t)(4 * (q0 + j)) * n + r;
            st_coh(d, v[j].x);
            st_coh(d + n, v[j].y);
            st_coh(d + 2 * (size_t)n, v[j].z);
            st_coh(d + 3 * (size_t)n, v[j].w);
          }
        }
      }
      continue;
    }
    constexpr int kChunk = 32;
    for (int s0 = 0; s0 < ns; s0 += kChunk) {
      float v[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) v[j] = src[min(s0 + j, ns - 1)];
#pragma unroll
      for (int j = 0; j < kChunk; ++j)
        if (s0 + j < ns) st_coh(sxp + (size_t)(s0 + j) * n + r, v[j]);
    }
  }
}

}  // namespace moe
