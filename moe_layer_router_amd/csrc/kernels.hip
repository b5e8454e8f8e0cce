// Kernels of the fused MoE layer: the separate-kernel pipeline and the
// persistent work-queue kernel that runs the whole layer in one launch.
//
// The single-launch form is the Mega MoE idea (机器之心, "DeepSeek悄悄更新：Mega
// MoE、FP4 Indexer来了", section "Mega MoE 是什么？"): dispatch, both linear
// maps, SwiGLU and combine fused into one kernel so that the GPU does not
// alternate between computing and waiting.  On one GPU the dispatch and
// combine are local permutations, and the overlap is between HBM weight
// streaming and MFMA work of different work items running side by side.
#include "kernels.h"
#include "backward.h"

namespace moe {

// ----------------------------------------------------------- separate mode
__global__ void k_zero(int32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

// K slice ks of nks: router steps [s0, s1) of H/128.
DEV void router_slice(int H, int ks, int nks, int* s0, int* s1) {
  const int nsteps = H / 128;
  *s0 = ks * nsteps / nks;
  *s1 = (ks + 1) * nsteps / nks;
}

// Router tiles (blockIdx.x: 64 experts, .y: 128 tokens, .z: K slice); slice
// ks writes its partial logits to a.logits + ks*T*E, and the last slice of a
// tile to finish sums them into slice 0 (tile_cnt: one counter per tile).
// NE experts per tile; the wide tiles (NE = kRouterExpertsWide) run with
// one slice only.
template <int AF, int NE = kRouterExperts>
__global__ void __launch_bounds__(256) k_router(RouterArgs a, int nks, int32_t* tile_cnt) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int s0, s1;
  router_slice(a.H, blockIdx.z, nks, &s0, &s1);
  const int t0 = blockIdx.y * kRouterTokens, e0 = blockIdx.x * NE;
  router_tile<AF, NE>(a, t0, e0, lds, s0, s1, a.logits + (size_t)blockIdx.z * a.T * a.E, blockIdx.z == 0);
  if (NE == kRouterExperts && nks > 1) router_reduce(a, t0, e0, nks, &tile_cnt[blockIdx.y * gridDim.x + blockIdx.x]);
}

constexpr int kTopkTokens = 32;   // tokens per top-k workgroup (separate mode)
// `tpb` tokens per workgroup: kTopkTokens (16-lane rows) for E <= 256, one
// token per wave above (more workgroups in flight for the longer rows).
__global__ void __launch_bounds__(256) k_topk(const float* logits, int T, int E, int k, int32_t* ids, float* wts,
                                              int tpb) {
  const int t0 = blockIdx.x * tpb;
  topk_tokens(logits, E, k, t0, min(tpb, T - t0), ids, wts);
}

__global__ void __launch_bounds__(256) k_count(const int32_t* ids, int T, int k, int E, int32_t* blockcnt) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  perm_count_block(ids, T, k, E, blockIdx.x, blockcnt, reinterpret_cast<int*>(lds));
}

// One workgroup of up to 1024 threads (one expert per thread up to E = 1024).
__global__ void __launch_bounds__(1024) k_scan(const int32_t* blockcnt, int nblk, int E, int tile_rows, int32_t* base,
                                               int32_t* offsets, Tile* tiles, int32_t* meta) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  perm_scan(blockcnt, nblk, E, tile_rows, base, offsets, tiles, meta, reinterpret_cast<int*>(lds));
}

__global__ void __launch_bounds__(256) k_scatter(const int32_t* ids, int T, int k, int E, const int32_t* base,
                                                 int32_t* perm, int32_t* row_of) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  perm_scatter_block(ids, T, k, E, blockIdx.x, base, perm, row_of, reinterpret_cast<uint64_t*>(lds));
}

// Input quantisation: 16 blocks of 128 channels per workgroup and pass.
template <int IN>
__global__ void __launch_bounds__(256) k_quant(const void* x, int T, int H, int pow2, uint8_t* xq, float* xs) {
  const int nblk = T * (H / 128);
  const int per = 16 * 4;                  // blocks per workgroup
  const int b0 = blockIdx.x * per;
  quant_blocks<IN>(x, T, H, b0, min(nblk, b0 + per), pow2 != 0, xq, xs, threadIdx.x, 256);
}

// E5M6 quantisation and dequantisation (same block-to-workgroup mapping).
template <int IN>
__global__ void __launch_bounds__(256) k_quant_e5m6(const void* x, int T, int H, int pow2, uint8_t* xq, float* xs) {
  const int nblk = T * (H / 128);
  const int per = 16 * 4;
  const int b0 = blockIdx.x * per;
  quant_blocks_e5m6<IN>(x, T, H, b0, min(nblk, b0 + per), pow2 != 0, xq, xs, threadIdx.x, 256);
}
__global__ void __launch_bounds__(256) k_dequant_e5m6(const uint8_t* xq, const float* xs, int T, int H, float* out) {
  dequant_e5m6(xq, xs, T, H, (size_t)blockIdx.x * blockDim.x + threadIdx.x, out);
}

// Activation scales in permuted row order (FP8 layers): 256 rows per block.
__global__ void __launch_bounds__(256) k_permute_scales(const int32_t* perm, const float* x_scales, int T, int k,
                                                        int ns, float* sxp) {
  const int r0 = blockIdx.x * 256;
  permute_scales(perm, x_scales, T, k, ns, r0, min(T * k, r0 + 256), sxp);
}

// Persistent grid (one workgroup per CU) over (tile, N block) items taken
// from the per-class queues.  Workgroup b runs on XCD b % 8 (round-robin
// dispatch) and starts on that class.  Thread 0 claims the next item when
// the current one's K loop ends, so the atomic's latency is hidden behind
// the epilogue, and items claimed one after the other also start one after
// the other: the row tiles that share a weight slab and the N blocks that
// share a row tile then stream their common operand through the XCD's L2
// at nearly the same time.  (Claiming a whole item ahead would start each
// item when the workgroup's previous, unrelated item happens to end.)
template <int AF, int WF, int STAGE>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
k_gemm(GemmArgs g, const Tile* tiles, const int32_t* meta, int nnb, int32_t* queues) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_item, s_first[kXcds + 1];
  int cls = blockIdx.x % kXcds;
  if (threadIdx.x <= kXcds) s_first[threadIdx.x] = meta[1 + threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) s_item = pop_class_item(queues, s_first, nnb, &cls);
  __syncthreads();
  for (int i = s_item; i >= 0;) {
    int t, nb;
    gemm_item_of(tiles, nnb, i, &t, &nb);
    // starts with a barrier, after which every thread has read s_item
    expert_gemm_item<AF, WF, STAGE, 0>(g, tiles[t], nb, lds, nullptr, [&]() {
      if (threadIdx.x == 0) s_item = pop_class_item(queues, s_first, nnb, &cls);
    });
    __syncthreads();                                          // s_item is written
    i = s_item;
  }
}

// Row-major [E*N][K] weights -> MFMA-tiled blocks (a byte permutation; the
// layout is defined in moe_layer.h).  One thread per 16-byte unit of the
// destination, in destination order, so that the writes are contiguous.
__global__ void __launch_bounds__(256) k_pack_weights(const uint8_t* src, uint8_t* dst, size_t rows, int n,
                                                      int nsteps, int bs) {
  const int np = bs / 64, nt = n / 16;
  const size_t units = rows * (size_t)nsteps * bs / 16;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < units; i += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    size_t r = i >> 6;                               // (e, s, t, p)
    const int p = (int)(r % np);
    r /= np;
    const int t = (int)(r % nt);
    r /= nt;
    const int s = (int)(r % nsteps);
    const size_t row = (r / nsteps) * n + (size_t)t * 16 + (l & 15);
    st16(dst + i * 16, ld16(src + row * ((size_t)nsteps * bs) + (size_t)bs * s + 64 * p + 16 * (l >> 4)));
  }
}

// E8M0 scales [E*N][K/32] -> per (K step s, quad q) 256 bytes, byte
// 4*l + c the scale of row 16*tile + l%16, K group 4*s + l/16, where tile is
// the quad's c-th 16-row tile: gate|up (gu) 2q + c for c < 2 and
// N/32 + 2q + c - 2 (the up rows) for c >= 2; down 4q + c.
__global__ void __launch_bounds__(256) k_pack_e8m0(const uint8_t* src, uint8_t* dst, size_t rows, int n, int nsteps,
                                                   int gu) {
  const int nq = n / 64;
  const size_t total = rows * (size_t)nsteps * 4;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 3), l = (int)((i >> 2) & 63);
    size_t r = i >> 8;                               // (e, s, q)
    const int q = (int)(r % nq);
    r /= nq;
    const int s = (int)(r % nsteps);
    const int tile = gu ? ((c < 2) ? 2 * q + c : n / 32 + 2 * q + c - 2) : 4 * q + c;
    const size_t row = (r / nsteps) * n + (size_t)tile * 16 + (l & 15);
    dst[i] = src[row * ((size_t)nsteps * 4) + 4 * s + (l >> 4)];
  }
}

// Workgroup (x, nb): tokens [64x, 64x + 64) of N block nb, whose staging
// rows are one contiguous run.
constexpr int kCombineKernelTokens = 64;
__global__ void __launch_bounds__(256) k_combine(const uint16_t* staging, uint16_t* y, int T, int H, int k) {
  const int t0 = blockIdx.x * kCombineKernelTokens, nb = blockIdx.y;
  combine_rows(staging, y, T, H, k, t0, min(T, t0 + kCombineKernelTokens), nb * 256, min(H, nb * 256 + 256));
}

// ------------------------------------------------------- persistent kernel
constexpr unsigned kSpinLimit = 1u << 22;

// Thread 0 waits (bounded) until *c >= target; the workgroup then proceeds
// together.  The spin uses relaxed loads and a single device-scope acquire
// fence follows it: an acquire on every poll would invalidate the caches
// each time, taking cached weights away from every workgroup on the XCD.
// Returns false if the wait timed out or another workgroup reported a failure.
DEV bool wait_counter(const int32_t* c, int target, int32_t* err, int* s_ok, bool acquire = true) {
  if (threadIdx.x == 0) {
    int ok = 1;
    unsigned spins = 0;
    for (;;) {
      // both words read in one round trip per poll
      const int v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v >= target) break;
      if (e != 0) { ok = 0; break; }
      __builtin_amdgcn_s_sleep(8);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
    if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_ok = ok;
  }
  __syncthreads();
  const int ok = *s_ok;
  __syncthreads();
  return ok != 0;
}

// Publish this workgroup's coherent (write-through) stores, then add 1 to
// each counter: each wave waits until its stores have completed, the
// workgroup synchronises, and one thread increments.  No device-wide fence:
// the data was written past the L2, and its readers use coherent loads or
// lines that no cache can hold an older copy of (see expert_gemm_tile), so
// the relaxed counter is the only ordering needed.  A release fence per item
// would write back the XCD's whole L2 and the matching acquire would
// invalidate it, taking cached weights and activations from every
// workgroup on the XCD.
DEV void signal_coherent(int32_t* c0, int32_t* c1 = nullptr) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(c0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c1) __hip_atomic_fetch_add(c1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Three queues, each in dependency order.  An item only ever waits for items
// that precede it in its own queue or belong to an earlier queue, and a
// workgroup moves to the next queue only once every item of the current one
// has been claimed by a running workgroup, so no wait can deadlock whatever
// the grid size:
//   head queue:   router tiles (128 tokens x 64 experts, or one channel
//                   slice of one)                        -> rdone[token tile]
//                 top-k of 16 tokens (summing the slices) -> tkdone[256-token block]
//                 expert histogram of 256 tokens        -> COUNT_DONE
//                   (only with more than one 256-token block)
//                 scan and stable scatter of 256 tokens -> SCATTER_DONE
//                   (block 0 also writes offsets, tiles)
//                 FP8 layers: activation scales of 256 permuted rows,
//                   K block major                       -> SXP_DONE
//   class queues: gate|up items (tile, 128 channels)    -> done1[tile]
//   class queues: down items (tile, 256 columns)        -> done2[N block]
//   tail queue:   combine items (N block, 256 tokens)
// The short phases of the persistent kernel are non-inlined functions, so
// that register allocation sees one phase at a time.  Each declares the
// dynamic LDS array itself so that its accesses compile to LDS instructions.
#define MEGA_LDS extern __shared__ __attribute__((aligned(16))) char lds[]
// Their arguments arrive in vector registers, where the compiler cannot tell
// that they are the same in every lane: buffer accesses would then loop over
// distinct descriptors and loops over plan sizes would run as divergent
// loops.  Every argument is wave-uniform, so each phase starts by taking
// them from the first lane.
DEV int uni_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
// The phases get the plan as a pointer to the persistent kernel's own
// argument in the kernarg segment (constant memory): taken from the first
// lane, its fields come through the scalar cache.  A plan passed by value
// would be copied through every lane's scratch memory on each call.
typedef const __attribute__((address_space(4))) Plan KPlan;
DEV Plan load_plan(KPlan* pv) {
  const uint64_t a = reinterpret_cast<uint64_t>(pv);
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  typedef const __attribute__((address_space(4))) uint32_t KWord;
  KWord* src = (KWord*)u;
  static_assert(sizeof(Plan) % 4 == 0, "plan words");
  Plan p;
  uint32_t* dst = reinterpret_cast<uint32_t*>(&p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Plan) / 4); ++i) dst[i] = src[i];
  return p;
}
// The GEMM items are inlined into the kernel: as a called function they
// would save and restore the callee-saved VGPRs they use on every item.
// Tiles as the GEMM phases read them: through the scalar cache, as k_gemm
// does (where the compiler chooses it by itself, the tiles being read-only
// there).  In the persistent kernel the permutation items write them, in
// lines of their own, before any GEMM item starts, and nothing reads them
// through that cache earlier in the launch (it starts each launch empty), so
// it cannot hold an older copy.  Ordinary loads would put two dependent
// round trips to memory between every two items.
typedef const __attribute__((address_space(4))) Tile KTile;
DEV Tile tile_at(KTile* kt, int t) {
  Tile x;
  x.e = kt[t].e;
  x.r0 = kt[t].r0;
  x.rows = kt[t].rows;
  x.rs = kt[t].rs;
  x.g0 = kt[t].g0;
  x.gn = kt[t].gn;
  return x;
}
template <int AF, int WF, int STAGE, typename Hook>
__device__ __forceinline__ void mega_gemm_item(const Plan& p, Tile tl, int nb, int32_t* signal_prev,
                                               const Hook& at_loop_end) {
  MEGA_LDS;
  expert_gemm_item<AF, WF, STAGE, 1>(gemm_args(p), tl, nb, lds, signal_prev, at_loop_end);
}
template <int AF>
__device__ __noinline__ void mega_router_item(KPlan* pv, int tt_, int et_, int ks_) {
  MEGA_LDS;
  const Plan p = load_plan(pv);
  const int tt = uni_i(tt_), et = uni_i(et_), ks = uni_i(ks_);
  int s0, s1;
  router_slice(p.H, ks, p.nKS, &s0, &s1);
  if (AF == ACT_FP8 && p.quant_in) {       // the router reads the BF16 input
    RouterArgs ra{reinterpret_cast<const uint8_t*>(p.xb), nullptr, p.wr, p.bias, p.logits, p.T, p.H, p.E, 0};
    router_tile<ACT_BF16>(ra, tt * kRouterTokens, et * kRouterExperts, lds, s0, s1,
                          p.logits + (size_t)ks * p.T * p.E, ks == 0);
  } else {
    RouterArgs ra{p.x, p.x_scales, p.wr, p.bias, p.logits, p.T, p.H, p.E, p.act_fp8};
    router_tile<AF>(ra, tt * kRouterTokens, et * kRouterExperts, lds, s0, s1, p.logits + (size_t)ks * p.T * p.E,
                    ks == 0);
  }
}
constexpr int kQuantItemBlocks = 256;     // 128-channel blocks per quantisation item
__device__ __noinline__ void mega_quant_item(KPlan* pv, int i_) {
  const Plan p = load_plan(pv);
  const int b0 = uni_i(i_) * kQuantItemBlocks;
  quant_blocks<QIN_BF16, kCoherent>(p.xb, p.T, p.H, b0, min(p.T * (p.H / 128), b0 + kQuantItemBlocks),
                                    p.pow2 != 0, const_cast<uint8_t*>(p.x), const_cast<float*>(p.x_scales),
                                    threadIdx.x, blockDim.x);
}
constexpr int kTopkItemTokens = 16;        // tokens per top-k item of the persistent kernel
__device__ __noinline__ void mega_topk_item(KPlan* pv, int i) {
  const Plan p = load_plan(pv);
  const int t0 = uni_i(i) * kTopkItemTokens;
  // (with channel slices the partials of slice s are at logits + s*T*E)
  topk_tokens(p.logits, p.E, p.k, t0, min(kTopkItemTokens, p.T - t0), p.ids, p.wts, p.nKS, (size_t)p.T * p.E);
}
__device__ __noinline__ void mega_count_item(KPlan* pv, int b_) {
  MEGA_LDS;
  const Plan p = load_plan(pv);
  const int b = uni_i(b_);
  perm_count_block(p.ids, p.T, p.k, p.E, b, p.blockcnt, reinterpret_cast<int*>(lds));
}
__device__ __noinline__ void mega_scatter_item(KPlan* pv, int b_) {
  MEGA_LDS;
  const Plan p = load_plan(pv);
  const int b = uni_i(b_);
  perm_scan_scatter_block(p.ids, p.T, p.k, p.E, b, p.nblk, p.blockcnt, p.tile_rows, p.offsets, p.tiles, p.meta,
                          p.perm, p.row_of, lds);
}
constexpr int kSxpRows = 256;             // permuted rows per activation-scale item
constexpr int kMegaHeadSplitBlocks = 8;   // 256-token blocks from which the head runs as separate kernels
__device__ __noinline__ void mega_sxp_item(KPlan* pv, int i_) {
  const Plan p = load_plan(pv);
  const int r0 = uni_i(i_) * kSxpRows;
  permute_scales(p.perm, p.x_scales, p.T, p.k, p.H / 128, r0, min(p.T * p.k, r0 + kSxpRows), p.sxp);
}
__device__ __noinline__ void mega_combine_item(KPlan* pv, int nb_, int c) {
  const Plan p = load_plan(pv);
  const int ct = uni_i(p.comb_tokens);
  const int nb = uni_i(nb_), t0 = uni_i(c) * ct;
  combine_rows(p.staging, p.y, p.T, p.H, p.k, t0, min(p.T, t0 + ct), nb * 256,
                  min(p.H, nb * 256 + 256));
}

template <int AF, int WF>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
k_mega(Plan p) {
  __shared__ int s_q, s_ok, s_first[kXcds + 1];
  const int tid = threadIdx.x;
  KPlan* const pk = (KPlan*)__builtin_amdgcn_kernarg_segment_ptr();   // p itself (the only argument)
  trace_stamp(p.trace, 0);
  // (with head_given the separate kernels have done the whole head: no items)
  const bool head = !p.head_given;
  const int nR = (p.routing_given || !head) ? 0 : p.nTR * p.nER * p.nKS;
  const int nK = (p.routing_given || !head) ? 0 : (p.T + kTopkItemTokens - 1) / kTopkItemTokens;
  // histogram items only when there are several 256-token blocks (a single
  // block counts itself in its scatter item)
  const int nC = (head && p.nblk > 1) ? p.nblk : 0;
  const int nS = head ? p.nblk : 0;
  // FP8 layers: the activation scales in permuted row order, after the scatter
  const int nX = (head && p.sxp) ? (p.T * p.k + kSxpRows - 1) / kSxpRows : 0;
  // BF16 input quantised in the layer: quantisation items come first (they
  // depend on nothing; the activation-scale items and the GEMMs wait for them)
  const int nQ = (head && p.quant_in) ? (p.T * (p.H / 128) + kQuantItemBlocks - 1) / kQuantItemBlocks : 0;
  const int q_rt = nQ;
  const int q_topk = q_rt + nR, q_count = q_topk + nK, q_scat = q_count + nC,
            q_sxp = q_scat + nS;
  const int q_end = q_sxp + nX;
  constexpr int kPer = kPermBlock / kTopkItemTokens;   // top-k items per 256-token block
  const int rdone_target = p.nER * p.nKS;          // router items per token tile

  // 1. routing and permutation items from the head queue
  for (;;) {
    if (tid == 0) s_q = __hip_atomic_fetch_add(&p.ctr[CTR_QUEUE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int q = s_q;
    __syncthreads();
    if (q >= q_end) break;
    if (q < q_rt) {
      mega_quant_item(pk, q);
      signal_coherent(&p.ctr[CTR_QUANT_DONE]);
    } else if (q < q_topk) {
      const int r = q - q_rt;
      const int per_tt = p.nER * p.nKS;
      const int tt = r / per_tt, et = (r % per_tt) / p.nKS, ks = r % p.nKS;
      mega_router_item<AF>(pk, tt, et, ks);
      signal_coherent(&p.rdone[tt]);
    } else if (q < q_count) {
      const int i = q - q_topk;                          // tokens [16i, 16i+16)
      if (!wait_counter(&p.rdone[i / (kRouterTokens / kTopkItemTokens)], rdone_target, p.err, &s_ok, false)) return;
      mega_topk_item(pk, i);
      signal_coherent(&p.tkdone[i / (kPermBlock / kTopkItemTokens)]);
    } else if (q < q_scat) {
      const int b = q - q_count;
      if (!p.routing_given && !wait_counter(&p.tkdone[b], min(kPer, nK - kPer * b), p.err, &s_ok, false)) return;
      mega_count_item(pk, b);
      signal_coherent(&p.ctr[CTR_COUNT_DONE]);
    } else if (q >= q_sxp) {
      if (!wait_counter(&p.ctr[CTR_SCATTER_DONE], p.nblk, p.err, &s_ok, false)) return;
      if (nQ > 0 && !wait_counter(&p.ctr[CTR_QUANT_DONE], nQ, p.err, &s_ok, false)) return;
      mega_sxp_item(pk, q - q_sxp);
      signal_coherent(&p.ctr[CTR_SXP_DONE]);
    } else {
      // scan and scatter of one block, once every histogram is in (or, with
      // a single block, once its top-k items are done)
      const int b = q - q_scat;
      if (nC > 0) {
        if (!wait_counter(&p.ctr[CTR_COUNT_DONE], nC, p.err, &s_ok, false)) return;
      } else if (!p.routing_given && !wait_counter(&p.tkdone[0], nK, p.err, &s_ok, false)) {
        return;
      }
      mega_scatter_item(pk, b);
      signal_coherent(&p.ctr[CTR_SCATTER_DONE]);
    }
  }

  trace_stamp(p.trace, 1);

  // 2. gate|up items from the per-class queues (every head item has been
  // claimed by a running workgroup, so these waits end).  The GEMM items
  // read the permutation, tiles and weights with ordinary loads: one acquire
  // per workgroup here drops any older copy of them from the L2.
  if (nQ > 0 && !wait_counter(&p.ctr[CTR_QUANT_DONE], nQ, p.err, &s_ok, false)) return;
  if (nX > 0) {
    if (!wait_counter(&p.ctr[CTR_SXP_DONE], nX, p.err, &s_ok)) return;     // (after every scatter item)
  } else if (head && !wait_counter(&p.ctr[CTR_SCATTER_DONE], p.nblk, p.err, &s_ok)) {
    return;
  }
  if (tid <= kXcds) s_first[tid] = __hip_atomic_load(&p.meta[1 + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int ntiles = s_first[kXcds];
  trace_stamp(p.trace, 2);
  int cls = blockIdx.x % kXcds;
  int32_t* pending = nullptr;              // counter of the previous item, not yet signalled
  int n_items = 0;
  if (tid == 0) s_q = pop_class_item(p.ctr + CTR_Q1, s_first, p.nnb1, &cls);
  __syncthreads();
  // (the next item is claimed when the current one's K loop ends, as in k_gemm)
  KTile* const ktiles = (KTile*)p.tiles;
  for (int i = s_q; i >= 0;) {
    int t, nb;
    gemm_item_of(ktiles, p.nnb1, uni_i(i), &t, &nb);
    mega_gemm_item<AF, WF, 1>(p, tile_at(ktiles, t), nb, pending, [&]() {
      if (tid == 0) s_q = pop_class_item(p.ctr + CTR_Q1, s_first, p.nnb1, &cls);
    });
    pending = &p.done1[t];                 // signalled once its stores have completed
    ++n_items;
    __syncthreads();
    i = s_q;
  }
  if (pending) signal_coherent(pending);
  pending = nullptr;
  trace_stamp(p.trace, 3);
  trace_count(p.trace, 6, n_items);
  n_items = 0;

  // 3. down items from the per-class queues (all gate|up items have been
  // claimed); an item waits for the gate|up items of its tile.  Relaxed
  // waits suffice (see signal_coherent).
  cls = blockIdx.x % kXcds;
  __syncthreads();
  if (tid == 0) s_q = pop_class_item(p.ctr + CTR_Q2, s_first, p.nnb2, &cls);
  __syncthreads();
  for (int i = s_q; i >= 0;) {
    int t, nb;
    gemm_item_of(ktiles, p.nnb2, uni_i(i), &t, &nb);
    if (!wait_counter(&p.done1[t], p.nnb1, p.err, &s_ok, false)) return;
    mega_gemm_item<AF, WF, 2>(p, tile_at(ktiles, t), nb, pending, [&]() {
      if (tid == 0) s_q = pop_class_item(p.ctr + CTR_Q2, s_first, p.nnb2, &cls);
    });
    pending = &p.done2[nb];
    ++n_items;
    __syncthreads();
    i = s_q;
  }
  if (pending) signal_coherent(pending);
  trace_stamp(p.trace, 4);
  trace_count(p.trace, 7, n_items);

  // 4. combine items (N block, comb_tokens tokens) once every down item of the N
  // block is done (all down items have been claimed)
  for (;;) {
    __syncthreads();
    if (tid == 0) s_q = __hip_atomic_fetch_add(&p.ctr[CTR_QUEUE2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int i = s_q;
    if (i >= p.nnb2 * p.nCT) break;
    const int nb = i / p.nCT, c = i % p.nCT;
    if (!wait_counter(&p.done2[nb], ntiles, p.err, &s_ok, false)) return;
    mega_combine_item(pk, nb, c);
  }
  trace_stamp(p.trace, 5);
}

}  // namespace moe

// ===================================================================== host
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "moe_layer.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t err, zero_begin, ctr, rdone, rtile, tkdone, done1, done2, zero_end;
  size_t logits, blockcnt, base, offsets, perm, row_of, tiles, meta, aq, sa, sxp, xq, xs, staging, trace, total;
  int nblk, nTR, nER, nKS, max_tiles, nnb1, nnb2;
};

Layout make_layout(const moe_desc* d) {
  Layout L{};
  const size_t T = d->T, E = d->E, k = d->top_k, H = d->H, I = d->I;
  L.nblk = (int)((T + kPermBlock - 1) / kPermBlock);
  L.nTR = (int)((T + kRouterTokens - 1) / kRouterTokens);
  L.nER = (int)((E + kRouterExperts - 1) / kRouterExperts);
  // K slices of the router: when the token x expert tiles are too few to
  // fill the GPU (small T, as in decode), each tile's channels are split
  // into up to H/512 slices (at most 8), whose partial logits the last
  // slice of each tile to finish sums
  {
    const int tiles = L.nTR * L.nER, nsteps = (int)(H / 128);
    int s = 1;
    if (tiles < 128) {
      s = (256 + tiles - 1) / tiles;
      s = s < nsteps / 4 ? s : nsteps / 4;
      s = s < 8 ? s : 8;
      s = s > 1 ? s : 1;
    }
    L.nKS = s;
  }
  L.max_tiles = (int)(E + (T * k + kMinTileRows - 1) / kMinTileRows);
  L.nnb1 = (int)(I / 128);
  L.nnb2 = (int)((H + 255) / 256);
  size_t o = 0;
  L.err = o; o += 256;
  L.zero_begin = o;
  L.ctr = o; o += CTR_NUM * 4;
  L.rdone = o; o += (size_t)L.nTR * 4;
  L.rtile = o; o += (size_t)L.nTR * L.nER * 4;
  L.tkdone = o; o += (size_t)L.nblk * 4;
  L.done1 = o; o += (size_t)L.max_tiles * 4;
  L.done2 = o; o += (size_t)L.nnb2 * 4;
  L.zero_end = o;
  o = align256(o);
  L.logits = o; o = align256(o + (size_t)L.nKS * T * E * 4);
  L.blockcnt = o; o = align256(o + (size_t)L.nblk * E * 4);
  L.base = o; o = align256(o + (size_t)L.nblk * E * 4);
  L.offsets = o; o = align256(o + (E + 1) * 4);
  L.perm = o; o = align256(o + T * k * 4);
  L.row_of = o; o = align256(o + T * k * 4);
  L.tiles = o; o = align256(o + (size_t)L.max_tiles * sizeof(Tile));
  L.meta = o; o = align256(o + 64);
  L.aq = o; o = align256(o + T * k * I * (d->weight_dtype != MOE_DTYPE_BF16 ? 1 : 2));
  L.sa = o; o = align256(o + T * k * (I / 128) * 4);
  const bool quant_in = d->act_dtype == MOE_DTYPE_BF16 && d->weight_dtype != MOE_DTYPE_BF16;
  const bool fp8_experts = d->act_dtype == MOE_DTYPE_FP8_E4M3 || quant_in;
  L.sxp = o; if (fp8_experts && L.nblk > 1) o = align256(o + T * k * (H / 128) * 4);
  L.xq = o; if (quant_in) o = align256(o + T * H);
  L.xs = o; if (quant_in) o = align256(o + T * (H / 128) * 4);
  L.staging = o; o = align256(o + T * k * (size_t)L.nnb2 * 256 * 2);
  L.trace = o; if (d->flags & MOE_FLAG_TRACE) o = align256(o + (size_t)kTraceGroups * kTraceFields * 8);
  L.total = o;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARGUMENT, "descriptor is NULL");
  if (d->T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 1 (got %d)", d->T);
  if (d->H < 128 || d->H % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (got %d)", d->H);
  if (d->I < 128 || d->I % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "I must be a positive multiple of 128 (got %d)", d->I);
  if (d->E < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "E must be >= 1 (got %d)", d->E);
  if (d->top_k < 1 || d->top_k > d->E) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be in [1, E] (got %d)", d->top_k);
  if (d->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E > 1024 is not supported (got %d)", d->E);
  if (d->top_k > 16) return fail(MOE_ERR_UNSUPPORTED, "top_k > 16 is not supported (got %d)", d->top_k);
  if (d->H > 16384) return fail(MOE_ERR_UNSUPPORTED, "H > 16384 is not supported (got %d)", d->H);
  if (d->I > 16384) return fail(MOE_ERR_UNSUPPORTED, "I > 16384 is not supported (got %d)", d->I);
  if ((long long)d->T * d->top_k > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "T * top_k too large");
  // whole-array buffers are addressed with 32-bit byte offsets; the staging
  // rows (T*top_k rows of H rounded up to 256, BF16) and the intermediate
  // rows (T*top_k*I, at most 2 bytes each) are the largest of them
  const long long hpad = (d->H + 255LL) / 256 * 256;
  if ((long long)d->T * d->top_k * (hpad > d->I ? hpad : d->I) * 2 > 0xFFFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED,
                "T * top_k * max(H rounded up to 256, I) * 2 must be below 4 GiB (got T=%d, top_k=%d, H=%d, I=%d)",
                d->T, d->top_k, d->H, d->I);
  const bool wq = d->weight_dtype == MOE_DTYPE_FP8_E4M3 || d->weight_dtype == MOE_DTYPE_FP4_E2M1;
  const bool pair_ok = (d->act_dtype == MOE_DTYPE_BF16 && (d->weight_dtype == MOE_DTYPE_BF16 || wq)) ||
                       (d->act_dtype == MOE_DTYPE_FP8_E4M3 && wq);
  if (!pair_ok)
    return fail(MOE_ERR_UNSUPPORTED,
                "unsupported dtype pair act=%d weight=%d (supported: bf16xbf16, fp8xfp8, fp8xfp4, bf16xfp8, bf16xfp4)",
                d->act_dtype, d->weight_dtype);
  if (d->mode != MOE_MODE_MEGA && d->mode != MOE_MODE_SEPARATE)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown mode %d", d->mode);
  if (d->flags & ~(MOE_FLAG_ROUTING_GIVEN | MOE_FLAG_TRACE))
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", d->flags);
  if (d->weight_layout != MOE_LAYOUT_ROW_MAJOR && d->weight_layout != MOE_LAYOUT_TILED)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown weight_layout %d", d->weight_layout);
  if (d->inter_scale != MOE_INTER_SCALE_F32 && d->inter_scale != MOE_INTER_SCALE_POW2)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown inter_scale %d", d->inter_scale);
  if (d->weight_scale != MOE_WSCALE_BLOCK && d->weight_scale != MOE_WSCALE_CHANNEL)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown weight_scale %d", d->weight_scale);
  if (d->weight_scale == MOE_WSCALE_CHANNEL && d->weight_dtype != MOE_DTYPE_FP8_E4M3)
    return fail(MOE_ERR_UNSUPPORTED, "per-channel weight scales need FP8 weights (weight_dtype=%d)", d->weight_dtype);
  return MOE_OK;
}

moe_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", name) : MOE_OK;
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define TRY(expr)                       \
  do {                                  \
    moe_status _s = (expr);             \
    if (_s != MOE_OK) return _s;        \
  } while (0)

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t _e = (expr);                                                              \
    if (_e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

struct DevInfo {
  int checked = 0, ok = 0, cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

moe_status device_info(DevInfo* out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& di = g_dev[dev];
  if (!di.checked) {
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, dev));
    di.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    di.cus = prop.multiProcessorCount;
    di.checked = 1;
  }
  if (!di.ok) return fail(MOE_ERR_UNSUPPORTED, "this library is built for gfx950 (MI355X) only");
  *out = di;
  return MOE_OK;
}

// The workspace of moe_forward_static: a file-scope device array, one copy
// per GPU.  In host code `scratch` names a host-side stand-in, not device
// memory; its device address on the current GPU is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever passed to kernels.
static __device__ __align__(256) char scratch[MOE_STATIC_WORKSPACE_BYTES];
void* g_scratch_ptr[64];

moe_status static_workspace(void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress returned a null address for the static workspace");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

moe_status fill_plan(const moe_desc* d, const Layout& L, char* ws, Plan* P) {
  Plan& p = *P;
  memset(&p, 0, sizeof p);
  p.T = d->T; p.H = d->H; p.E = d->E; p.I = d->I; p.k = d->top_k;
  p.quant_in = d->act_dtype == MOE_DTYPE_BF16 && d->weight_dtype != MOE_DTYPE_BF16;
  p.act_fp8 = d->act_dtype == MOE_DTYPE_FP8_E4M3 || p.quant_in;
  p.pow2 = d->inter_scale == MOE_INTER_SCALE_POW2;
  p.wchan = d->weight_scale == MOE_WSCALE_CHANNEL;
  p.wdt = d->weight_dtype == MOE_DTYPE_FP8_E4M3 ? W_FP8 : d->weight_dtype == MOE_DTYPE_FP4_E2M1 ? W_FP4 : W_BF16;
  p.routing_given = (d->flags & MOE_FLAG_ROUTING_GIVEN) != 0;
  p.nblk = L.nblk; p.nTR = L.nTR; p.nER = L.nER; p.nKS = L.nKS; p.max_tiles = L.max_tiles;
  p.tile_rows = p.act_fp8 ? GemmLds<ACT_FP8>::kRows : GemmLds<ACT_BF16>::kRows;
  p.nnb1 = L.nnb1; p.nnb2 = L.nnb2;
  p.comb_tokens = kCombineTokens;
  p.nCT = (d->T + kCombineTokens - 1) / kCombineTokens;
  p.err = reinterpret_cast<int32_t*>(ws + L.err);
  p.ctr = reinterpret_cast<int32_t*>(ws + L.ctr);
  p.rdone = reinterpret_cast<int32_t*>(ws + L.rdone);
  p.rtile = reinterpret_cast<int32_t*>(ws + L.rtile);
  p.tkdone = reinterpret_cast<int32_t*>(ws + L.tkdone);
  p.done1 = reinterpret_cast<int32_t*>(ws + L.done1);
  p.done2 = reinterpret_cast<int32_t*>(ws + L.done2);
  p.zero_bytes = L.zero_end - L.zero_begin;
  p.logits = reinterpret_cast<float*>(ws + L.logits);
  p.blockcnt = reinterpret_cast<int32_t*>(ws + L.blockcnt);
  p.base = reinterpret_cast<int32_t*>(ws + L.base);
  p.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  p.perm = reinterpret_cast<int32_t*>(ws + L.perm);
  p.row_of = reinterpret_cast<int32_t*>(ws + L.row_of);
  p.tiles = reinterpret_cast<Tile*>(ws + L.tiles);
  p.meta = reinterpret_cast<int32_t*>(ws + L.meta);
  p.aq = reinterpret_cast<uint8_t*>(ws + L.aq);
  p.sa = reinterpret_cast<float*>(ws + L.sa);
  // permuted activation scales when there are several 256-token blocks (for
  // a single block the extra step costs more than it saves)
  p.sxp = (p.act_fp8 && L.nblk > 1) ? reinterpret_cast<float*>(ws + L.sxp) : nullptr;
  p.staging = reinterpret_cast<uint16_t*>(ws + L.staging);
  p.trace = (d->flags & MOE_FLAG_TRACE) ? reinterpret_cast<uint64_t*>(ws + L.trace) : nullptr;
  if (p.quant_in) {          // the experts read the layer's own quantisation of x
    p.x = reinterpret_cast<const uint8_t*>(ws + L.xq);
    p.x_scales = reinterpret_cast<const float*>(ws + L.xs);
  }
  return MOE_OK;
}

enum { WS_LAYER, WS_ROUTE, WS_PERMUTE };

size_t workspace_need(const moe_desc* d, int what) {
  const Layout L = make_layout(d);
  return what == WS_ROUTE ? L.blockcnt : what == WS_PERMUTE ? L.aq : L.total;
}

moe_status check_workspace(const moe_desc* d, const void* ws, size_t bytes, int what = WS_LAYER) {
  TRY(check_ptr(ws, "workspace"));
  const size_t need = workspace_need(d, what);
  if (bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", bytes, need);
  return MOE_OK;
}

template <typename K>
moe_status set_lds_limit(K kernel, int bytes) {
  if (bytes > 64 * 1024) HIP_TRY(hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
  return MOE_OK;
}

int gemm_lds(int act_fp8) { return act_fp8 ? GemmLds<ACT_FP8>::kBytes : GemmLds<ACT_BF16>::kBytes; }

int mega_lds(const Plan& p) {
  int b = gemm_lds(p.act_fp8);
  b = b > kRouterLds ? b : kRouterLds;
  const int scat = 4 * p.E * 8 + (2 * p.E + kXcds * ((p.E + kXcds - 1) / kXcds) + 64) * 4;   // scan and scatter
  b = b > scat ? b : scat;
  return b;
}

// nks: K slices (partials at logits + ks*T*E, summed into slice 0 by the
// last slice of each tile).
moe_status launch_route(const Plan& p, float* logits, int nks, hipStream_t st) {
  RouterArgs ra{p.x, p.x_scales, p.wr, p.bias, logits, p.T, p.H, p.E, p.act_fp8};
  if (p.quant_in) ra = RouterArgs{reinterpret_cast<const uint8_t*>(p.xb), nullptr, p.wr, p.bias, logits, p.T, p.H,
                                  p.E, 0};
  const int wide_tiles = p.nTR * ((p.E + kRouterExpertsWide - 1) / kRouterExpertsWide);
  if (ra.act_fp8 && nks == 1 && p.E >= 512 && wide_tiles >= 1024) {
    // wide tiles (128 experts): half the router weight bytes per flop, where
    // they are still several per CU
    TRY(set_lds_limit(k_router<ACT_FP8, kRouterExpertsWide>, kRouterLds));
    hipLaunchKernelGGL((k_router<ACT_FP8, kRouterExpertsWide>),
                       dim3((p.E + kRouterExpertsWide - 1) / kRouterExpertsWide, p.nTR, 1), dim3(256), kRouterLds, st, ra,
                       1, p.rtile);
  } else if (ra.act_fp8) {
    TRY(set_lds_limit(k_router<ACT_FP8>, kRouterLds));
    hipLaunchKernelGGL(k_router<ACT_FP8>, dim3(p.nER, p.nTR, nks), dim3(256), kRouterLds, st, ra, nks, p.rtile);
  } else {
    TRY(set_lds_limit(k_router<ACT_BF16>, kRouterLds));
    hipLaunchKernelGGL(k_router<ACT_BF16>, dim3(p.nER, p.nTR, nks), dim3(256), kRouterLds, st, ra, nks, p.rtile);
  }
  HIP_TRY(hipGetLastError());
  const int tpb = p.E <= 256 ? kTopkTokens : 4;
  hipLaunchKernelGGL(k_topk, dim3((p.T + tpb - 1) / tpb), dim3(256), 0, st, logits, p.T, p.E, p.k, p.ids, p.wts, tpb);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

moe_status launch_permute(const Plan& p, int32_t* row_of, hipStream_t st) {
  hipLaunchKernelGGL(k_count, dim3(p.nblk), dim3(256), p.E * 4, st, p.ids, p.T, p.k, p.E, p.blockcnt);
  HIP_TRY(hipGetLastError());
  const int scan_threads = std::min(1024, std::max(256, (p.E + 63) / 64 * 64));
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(scan_threads), (2 * p.E + 72) * 4, st, p.blockcnt, p.nblk, p.E,
                     p.tile_rows, p.base, p.offsets, p.tiles, p.meta);
  HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_scatter, dim3(p.nblk), dim3(256), 4 * p.E * 8, st, p.ids, p.T, p.k, p.E, p.base, p.perm, row_of);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

template <int AF, int WF>
moe_status launch_layer(const Plan& p, const DevInfo& di, int mode, hipStream_t st) {
  const size_t zero_ints = (p.zero_bytes + 256) / 4;   // error word region + counters
  hipLaunchKernelGGL(k_zero, dim3(16), dim3(256), 0, st, p.err, zero_ints);
  HIP_TRY(hipGetLastError());
  // The persistent kernel's head (routing and permutation) runs at one
  // workgroup per CU; from kMegaHeadSplitBlocks 256-token blocks on, the
  // separate kernels (several workgroups per CU) do it faster, and the
  // persistent kernel then starts at the GEMM items.
  const bool split_head = mode != MOE_MODE_SEPARATE && p.nblk >= kMegaHeadSplitBlocks;
  if (mode == MOE_MODE_SEPARATE || split_head) {
    if (p.quant_in) {
      const int nb = p.T * (p.H / 128);
      hipLaunchKernelGGL(k_quant<QIN_BF16>, dim3((nb + 63) / 64), dim3(256), 0, st, (const void*)p.xb, p.T, p.H,
                         p.pow2, const_cast<uint8_t*>(p.x), const_cast<float*>(p.x_scales));
      HIP_TRY(hipGetLastError());
    }
    if (!p.routing_given) TRY(launch_route(p, p.logits, p.nKS, st));
    TRY(launch_permute(p, p.row_of, st));
    if (p.sxp) {
      hipLaunchKernelGGL(k_permute_scales, dim3((p.T * p.k + 255) / 256), dim3(256), 0, st, p.perm, p.x_scales, p.T,
                         p.k, p.H / 128, p.sxp);
      HIP_TRY(hipGetLastError());
    }
  }
  if (mode == MOE_MODE_SEPARATE) {
    const GemmArgs g = gemm_args(p);
    const int lds = gemm_lds(AF == ACT_FP8);
    TRY(set_lds_limit(k_gemm<AF, WF, 1>, lds));
    TRY(set_lds_limit(k_gemm<AF, WF, 2>, lds));
    const int grid = di.cus;
    hipLaunchKernelGGL((k_gemm<AF, WF, 1>), dim3(grid), dim3(256), lds, st, g, p.tiles, p.meta, p.nnb1,
                       p.ctr + CTR_Q1);
    HIP_TRY(hipGetLastError());
    hipLaunchKernelGGL((k_gemm<AF, WF, 2>), dim3(grid), dim3(256), lds, st, g, p.tiles, p.meta, p.nnb2,
                       p.ctr + CTR_Q2);
    HIP_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_combine, dim3((p.T + kCombineKernelTokens - 1) / kCombineKernelTokens, p.nnb2), dim3(256), 0,
                       st, p.staging, p.y, p.T, p.H, p.k);
    HIP_TRY(hipGetLastError());
  } else {
    const int lds = mega_lds(p);
    TRY(set_lds_limit(k_mega<AF, WF>, lds));
    int occ = 0;
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_mega<AF, WF>, 256, lds));
    if (occ < 1) occ = 1;
    Plan pm = p;
    pm.head_given = split_head ? 1 : 0;
    // combine items: at least two per workgroup where the token count allows
    // (a decode batch has one 256-token chunk per N block: too few items for
    // the grid, and the combine tail is then latency-bound)
    const int nnb = (p.H + 255) / 256;
    while (pm.comb_tokens > 16 && (long)((p.T + pm.comb_tokens - 1) / pm.comb_tokens) * nnb < 2L * di.cus * occ)
      pm.comb_tokens /= 2;
    pm.nCT = (p.T + pm.comb_tokens - 1) / pm.comb_tokens;
    hipLaunchKernelGGL((k_mega<AF, WF>), dim3(di.cus * occ), dim3(256), lds, st, pm);
    HIP_TRY(hipGetLastError());
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- backward
// Workspace of the backward pass: the permutation's regions of the forward
// layout, then the backward's own buffers (P = T*k permuted rows).
struct BwdLayout {
  size_t gu, dau, dgu, dgu_lo, aw, aw_lo, dws, dxr_rows, dl, dl_lo, dxr, xp, dyp, total;
};

BwdLayout bwd_layout(const moe_desc* d) {
  const Layout L = make_layout(d);
  const size_t T = d->T, H = d->H, E = d->E, I = d->I, P = (size_t)d->T * d->top_k;
  BwdLayout B{};
  size_t o = align256(L.aq);                       // the forward layout up to the intermediate
  B.gu = o; o = align256(o + P * 2 * I * 4);
  B.dau = o; o = align256(o + P * I * 4);
  B.dgu = o; o = align256(o + P * 2 * I * 2);     // hi part, then the lo part
  B.dgu_lo = o; o = align256(o + P * 2 * I * 2);
  B.aw = o; o = align256(o + P * I * 2);
  B.aw_lo = o; o = align256(o + P * I * 2);
  B.dws = o; o = align256(o + P * 4);
  B.dxr_rows = o; o = align256(o + P * H * 4);
  B.dl = o; o = align256(o + T * E * 2);
  B.dl_lo = o; o = align256(o + T * E * 2);
  B.dxr = o; o = align256(o + T * H * 4);
  B.xp = o; o = align256(o + P * H * 2);
  B.dyp = o; o = align256(o + P * H * 2);
  B.total = o;
  return B;
}

moe_status check_bwd_desc(const moe_desc* d) {
  TRY(check_desc(d));
  if (d->act_dtype != MOE_DTYPE_BF16 || d->weight_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the backward pass supports BF16 layers only (act=%d weight=%d)", d->act_dtype,
                d->weight_dtype);
  if (d->weight_layout != MOE_LAYOUT_ROW_MAJOR)
    return fail(MOE_ERR_INVALID_ARGUMENT, "the backward pass reads row-major weights (weight_layout=%d)",
                d->weight_layout);
  return MOE_OK;
}

// grid: gx x gy x gz logical tiles (BwdGemm), launched as one dimension;
// A split into hi / lo parts when g.a.p_lo is set.  The grouped-row product
// of two K-contiguous BF16 operands with whole column tiles runs the
// direct-load kernel (when its buffers fit 32-bit offsets); the others run
// the register-staged kernel.
moe_status launch_bwd_gemm(BwdGemm g, unsigned gx, unsigned gy, unsigned gz, hipStream_t st) {
  g.gx = (int)gx;
  g.gy = (int)gy;
  g.gz = (int)gz;
  size_t units = 1, gyb = gy;
  if (g.group == BWD_GROUP_ROWS) g.gx = (int)(gx + 15) / 16 * 16;       // whole pairs, a multiple of 8 of them
  if (g.group == BWD_GROUP_K) {
    units = (gz + 7) / 8 * 8;
    gyb = (gy + kBwdTpb - 1) / kBwdTpb;
  }
  const dim3 grid((unsigned)((size_t)g.gx * gyb * units));
  const bool split = g.a.p_lo != nullptr;
  const long lim = 1L << 31;
  if ((g.a.trans && g.a.map) || (!g.b.trans && g.b.map))
    return fail(MOE_ERR_INVALID_ARGUMENT, "internal: a transposed backward operand has a row map");
  if (g.group == BWD_GROUP_ROWS && !split && !g.c_trans && !g.a.trans && g.b.trans && g.N % kBwdBN == 0 &&
      g.K % kBwdBK == 0 && g.a.ld % 8 == 0 && g.b.ld % 8 == 0 && g.a_bytes < lim && g.b_bytes < lim) {
    TRY(set_lds_limit(k_bwd_gemm_dma, kBwdDmaLds));
    hipLaunchKernelGGL(k_bwd_gemm_dma, grid, dim3(256), kBwdDmaLds, st, g);
    HIP_TRY(hipGetLastError());
    return MOE_OK;
  }
  if (split && g.c_trans)
    hipLaunchKernelGGL((k_bwd_gemm<1, 1>), grid, dim3(256), bwd_lds_bytes<1>(), st, g);
  else if (split)
    hipLaunchKernelGGL((k_bwd_gemm<1, 0>), grid, dim3(256), bwd_lds_bytes<1>(), st, g);
  else if (g.c_trans)
    hipLaunchKernelGGL((k_bwd_gemm<0, 1>), grid, dim3(256), bwd_lds_bytes<0>(), st, g);
  else
    hipLaunchKernelGGL((k_bwd_gemm<0, 0>), grid, dim3(256), bwd_lds_bytes<0>(), st, g);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

BwdOperand bwd_op(const void* p, long ld, int trans, const int32_t* map = nullptr, int div = 1, long gstride = 0) {
  return BwdOperand{p, nullptr, ld, trans, map, div, gstride};
}
// an fp32 operand held as hi / lo BF16 parts
BwdOperand bwd_op2(const void* hi, const void* lo, long ld, int trans) {
  return BwdOperand{hi, lo, ld, trans, nullptr, 1, 0};
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

size_t moe_workspace_size(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return workspace_need(d, WS_LAYER);
}

size_t moe_route_workspace_size(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return workspace_need(d, WS_ROUTE);
}

size_t moe_permute_workspace_size(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return workspace_need(d, WS_PERMUTE);
}

moe_status moe_get_workspace_regions(const moe_desc* d, moe_workspace_regions* out) {
  TRY(check_desc(d));
  if (!out) return fail(MOE_ERR_INVALID_ARGUMENT, "out is NULL");
  const Layout L = make_layout(d);
  out->logits = L.logits;
  out->perm = L.perm;
  out->row_of = L.row_of;
  out->offsets = L.offsets;
  out->inter = L.aq;
  out->inter_scales = L.sa;
  out->staging = L.staging;
  out->trace = L.trace;
  out->total = L.total;
  return MOE_OK;
}

moe_status moe_validate(const moe_desc* d, const void* x, const float* x_scales, const void* router_w,
                        const float* router_bias, const void* w_gate_up, const void* w_gate_up_scales,
                        const void* w_down, const void* w_down_scales, const void* y, const int32_t* topk_ids,
                        const float* topk_weights, const void* workspace, size_t workspace_bytes) {
  TRY(check_desc(d));
  if (d->weight_layout != MOE_LAYOUT_TILED)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "the expert weights must be in the MFMA-tiled layout: convert them with moe_pack_weights and set "
                "weight_layout = MOE_LAYOUT_TILED");
  const bool given = (d->flags & MOE_FLAG_ROUTING_GIVEN) != 0;
  TRY(check_ptr(x, "x", !given));
  TRY(check_ptr(x_scales, "x_scales", d->act_dtype == MOE_DTYPE_FP8_E4M3 && !given));
  if (d->act_dtype == MOE_DTYPE_BF16 && d->weight_dtype != MOE_DTYPE_BF16 && x_scales)
    return fail(MOE_ERR_INVALID_ARGUMENT, "x_scales must be NULL when the layer quantises its BF16 input");
  TRY(check_ptr(router_w, "router_w", !given));
  TRY(check_ptr(router_bias, "router_bias", false));
  TRY(check_ptr(w_gate_up, "w_gate_up"));
  TRY(check_ptr(w_gate_up_scales, "w_gate_up_scales", d->weight_dtype != MOE_DTYPE_BF16));
  TRY(check_ptr(w_down, "w_down"));
  TRY(check_ptr(w_down_scales, "w_down_scales", d->weight_dtype != MOE_DTYPE_BF16));
  TRY(check_ptr(y, "y"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_weights, "topk_weights"));
  if (given && !x) return fail(MOE_ERR_INVALID_ARGUMENT, "x is NULL");
  if (given && d->act_dtype == MOE_DTYPE_FP8_E4M3 && !x_scales) return fail(MOE_ERR_INVALID_ARGUMENT, "x_scales is NULL");
  TRY(check_workspace(d, workspace, workspace_bytes));
  return MOE_OK;
}

moe_status moe_forward(const moe_desc* d, const void* x, const float* x_scales, const void* router_w,
                       const float* router_bias, const void* w_gate_up, const void* w_gate_up_scales,
                       const void* w_down, const void* w_down_scales, void* y, int32_t* topk_ids,
                       float* topk_weights, int32_t* expert_offsets, int32_t* perm, void* workspace,
                       size_t workspace_bytes, moe_stream_t stream) {
  TRY(moe_validate(d, x, x_scales, router_w, router_bias, w_gate_up, w_gate_up_scales, w_down, w_down_scales, y,
                   topk_ids, topk_weights, workspace, workspace_bytes));
  TRY(check_ptr(expert_offsets, "expert_offsets", false));
  TRY(check_ptr(perm, "perm", false));
  DevInfo di;
  TRY(device_info(&di));
  const Layout L = make_layout(d);
  Plan p;
  TRY(fill_plan(d, L, static_cast<char*>(workspace), &p));
  if (p.quant_in) {
    p.xb = static_cast<const uint16_t*>(x);
  } else {
    p.x = static_cast<const uint8_t*>(x);
    p.x_scales = x_scales;
  }
  p.wr = static_cast<const uint16_t*>(router_w); p.bias = router_bias;
  p.w_gu = static_cast<const uint8_t*>(w_gate_up); p.w_gu_scales = w_gate_up_scales;
  p.w_d = static_cast<const uint8_t*>(w_down); p.w_d_scales = w_down_scales;
  p.y = static_cast<uint16_t*>(y); p.ids = topk_ids; p.wts = topk_weights;
  if (expert_offsets) p.offsets = expert_offsets;
  if (perm) p.perm = perm;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.act_fp8 && p.wdt == W_FP8) return launch_layer<ACT_FP8, W_FP8>(p, di, d->mode, st);
  if (p.act_fp8 && p.wdt == W_FP4) return launch_layer<ACT_FP8, W_FP4>(p, di, d->mode, st);
  return launch_layer<ACT_BF16, W_BF16>(p, di, d->mode, st);
}

moe_status moe_quantize_input(int32_t T, int32_t H, int32_t in_dtype, int32_t scale_mode, const void* x, uint8_t* xq,
                              float* x_scales, moe_stream_t stream) {
  if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 1 (got %d)", T);
  if (H < 128 || H % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (got %d)", H);
  if ((long long)T * H >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T * H must be below 2^31");
  if (in_dtype != MOE_DTYPE_BF16 && in_dtype != MOE_DTYPE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "in_dtype must be MOE_DTYPE_BF16 or MOE_DTYPE_F32 (got %d)", in_dtype);
  if (scale_mode != MOE_INTER_SCALE_F32 && scale_mode != MOE_INTER_SCALE_POW2)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown scale_mode %d", scale_mode);
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(xq, "xq"));
  TRY(check_ptr(x_scales, "x_scales"));
  DevInfo di;
  TRY(device_info(&di));
  const int nb = T * (H / 128);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int pow2 = scale_mode == MOE_INTER_SCALE_POW2;
  if (in_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(k_quant<QIN_BF16>, dim3((nb + 63) / 64), dim3(256), 0, st, x, T, H, pow2, xq, x_scales);
  else
    hipLaunchKernelGGL(k_quant<QIN_F32>, dim3((nb + 63) / 64), dim3(256), 0, st, x, T, H, pow2, xq, x_scales);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

moe_status moe_quantize_e5m6(int32_t T, int32_t H, int32_t in_dtype, int32_t scale_mode, const void* x, uint8_t* xq,
                             float* x_scales, moe_stream_t stream) {
  if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 1 (got %d)", T);
  if (H < 128 || H % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (got %d)", H);
  if ((long long)T * H >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T * H must be below 2^31");
  if (in_dtype != MOE_DTYPE_BF16 && in_dtype != MOE_DTYPE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "in_dtype must be MOE_DTYPE_BF16 or MOE_DTYPE_F32 (got %d)", in_dtype);
  if (scale_mode != MOE_INTER_SCALE_F32 && scale_mode != MOE_INTER_SCALE_POW2)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown scale_mode %d", scale_mode);
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(xq, "xq"));
  TRY(check_ptr(x_scales, "x_scales"));
  const int nb = T * (H / 128);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int pow2 = scale_mode == MOE_INTER_SCALE_POW2;
  if (in_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(k_quant_e5m6<QIN_BF16>, dim3((nb + 63) / 64), dim3(256), 0, st, x, T, H, pow2, xq, x_scales);
  else
    hipLaunchKernelGGL(k_quant_e5m6<QIN_F32>, dim3((nb + 63) / 64), dim3(256), 0, st, x, T, H, pow2, xq, x_scales);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

moe_status moe_dequantize_e5m6(int32_t T, int32_t H, const uint8_t* xq, const float* x_scales, float* out,
                               moe_stream_t stream) {
  if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 1 (got %d)", T);
  if (H < 128 || H % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (got %d)", H);
  if ((long long)T * H >= (1LL << 31)) return fail(MOE_ERR_UNSUPPORTED, "T * H must be below 2^31");
  TRY(check_ptr(xq, "xq"));
  TRY(check_ptr(x_scales, "x_scales"));
  TRY(check_ptr(out, "out"));
  const long n8 = (long)T * H / 8;
  hipLaunchKernelGGL(k_dequant_e5m6, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     xq, x_scales, T, H, out);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

moe_status moe_forward_static(const moe_desc* d, const void* x, const float* x_scales, const void* router_w,
                              const float* router_bias, const void* w_gate_up, const void* w_gate_up_scales,
                              const void* w_down, const void* w_down_scales, void* y, int32_t* topk_ids,
                              float* topk_weights, int32_t* expert_offsets, int32_t* perm, moe_stream_t stream) {
  TRY(check_desc(d));
  const size_t need = workspace_need(d, WS_LAYER);
  if (need > MOE_STATIC_WORKSPACE_BYTES)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "this layer needs %zu bytes of workspace; moe_forward_static has %zu (pass a workspace to moe_forward)",
                need, (size_t)MOE_STATIC_WORKSPACE_BYTES);
  void* ws = nullptr;
  TRY(static_workspace(&ws));
  return moe_forward(d, x, x_scales, router_w, router_bias, w_gate_up, w_gate_up_scales, w_down, w_down_scales, y,
                     topk_ids, topk_weights, expert_offsets, perm, ws, MOE_STATIC_WORKSPACE_BYTES, stream);
}

moe_status moe_route(const moe_desc* d, const void* x, const float* x_scales, const void* router_w,
                     const float* router_bias, float* logits, int32_t* topk_ids, float* topk_weights,
                     void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  TRY(check_desc(d));
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(x_scales, "x_scales", d->act_dtype == MOE_DTYPE_FP8_E4M3));
  TRY(check_ptr(router_w, "router_w"));
  TRY(check_ptr(router_bias, "router_bias", false));
  TRY(check_ptr(logits, "logits", false));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_weights, "topk_weights"));
  TRY(check_workspace(d, workspace, workspace_bytes, WS_ROUTE));
  DevInfo di;
  TRY(device_info(&di));
  const Layout L = make_layout(d);
  Plan p;
  TRY(fill_plan(d, L, static_cast<char*>(workspace), &p));
  // the router reads x as the descriptor's activation dtype says (BF16 input
  // is read as BF16 whatever the weights are)
  p.quant_in = 0;
  p.act_fp8 = d->act_dtype == MOE_DTYPE_FP8_E4M3;
  p.x = static_cast<const uint8_t*>(x); p.x_scales = x_scales;
  p.wr = static_cast<const uint16_t*>(router_w); p.bias = router_bias;
  p.ids = topk_ids; p.wts = topk_weights;
  return launch_route(p, logits ? logits : p.logits, 1, static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_desc* d, const int32_t* topk_ids, int32_t* expert_offsets, int32_t* perm,
                       int32_t* row_of, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  TRY(check_desc(d));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(expert_offsets, "expert_offsets"));
  TRY(check_ptr(perm, "perm"));
  TRY(check_ptr(row_of, "row_of", false));
  TRY(check_workspace(d, workspace, workspace_bytes, WS_PERMUTE));
  DevInfo di;
  TRY(device_info(&di));
  const Layout L = make_layout(d);
  Plan p;
  TRY(fill_plan(d, L, static_cast<char*>(workspace), &p));
  p.ids = const_cast<int32_t*>(topk_ids);
  p.offsets = expert_offsets;
  p.perm = perm;
  return launch_permute(p, row_of, static_cast<hipStream_t>(stream));
}

moe_status moe_pack_weights(const moe_desc* d, int32_t which, const void* src, const void* src_scales, void* dst,
                            void* dst_scales, moe_stream_t stream) {
  TRY(check_desc(d));
  if (which != MOE_WEIGHTS_GATE_UP && which != MOE_WEIGHTS_DOWN)
    return fail(MOE_ERR_INVALID_ARGUMENT, "which must be MOE_WEIGHTS_GATE_UP or MOE_WEIGHTS_DOWN (got %d)", which);
  TRY(check_ptr(src, "src"));
  TRY(check_ptr(dst, "dst"));
  const bool fp4 = d->weight_dtype == MOE_DTYPE_FP4_E2M1;
  if (fp4) {
    TRY(check_ptr(src_scales, "src_scales"));
    TRY(check_ptr(dst_scales, "dst_scales"));
  } else if (src_scales || dst_scales) {
    return fail(MOE_ERR_INVALID_ARGUMENT, "scale pointers must be NULL unless the weights are FP4");
  }
  const size_t N = which == MOE_WEIGHTS_GATE_UP ? 2 * (size_t)d->I : (size_t)d->H;
  const int K = which == MOE_WEIGHTS_GATE_UP ? d->H : d->I;
  const int bs = d->weight_dtype == MOE_DTYPE_BF16 ? 256 : fp4 ? 64 : 128;
  const size_t rows = (size_t)d->E * N, bytes = rows * (size_t)(K / 128) * bs;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "dst overlaps src");
  DevInfo di;
  TRY(device_info(&di));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int grid = di.cus * 8;
  hipLaunchKernelGGL(k_pack_weights, dim3(grid), dim3(256), 0, st, static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst), rows, (int)N, K / 128, bs);
  HIP_TRY(hipGetLastError());
  if (fp4) {
    hipLaunchKernelGGL(k_pack_e8m0, dim3(grid), dim3(256), 0, st, static_cast<const uint8_t*>(src_scales),
                       static_cast<uint8_t*>(dst_scales), rows, (int)N, K / 128, which == MOE_WEIGHTS_GATE_UP ? 1 : 0);
    HIP_TRY(hipGetLastError());
  }
  return MOE_OK;
}

size_t moe_backward_workspace_size(const moe_desc* d) {
  if (check_bwd_desc(d) != MOE_OK) return 0;
  return bwd_layout(d).total;
}

moe_status moe_backward(const moe_desc* d, const void* x, const void* router_w, const void* w_gate_up,
                        const void* w_down, const int32_t* topk_ids, const float* topk_weights, const void* dy,
                        float* dx, float* dw_gate_up, float* dw_down, float* dw_router, float* dbias,
                        void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  TRY(check_bwd_desc(d));
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(router_w, "router_w"));
  TRY(check_ptr(w_gate_up, "w_gate_up"));
  TRY(check_ptr(w_down, "w_down"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_weights, "topk_weights"));
  TRY(check_ptr(dy, "dy"));
  TRY(check_ptr(dx, "dx"));
  TRY(check_ptr(dw_gate_up, "dw_gate_up"));
  TRY(check_ptr(dw_down, "dw_down"));
  TRY(check_ptr(dw_router, "dw_router"));
  TRY(check_ptr(dbias, "dbias", false));
  TRY(check_ptr(workspace, "workspace"));
  const BwdLayout B = bwd_layout(d);
  if (workspace_bytes < B.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, B.total);
  DevInfo di;
  TRY(device_info(&di));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = make_layout(d);
  char* ws = static_cast<char*>(workspace);
  Plan p;
  TRY(fill_plan(d, L, ws, &p));
  p.ids = const_cast<int32_t*>(topk_ids);
  const int T = d->T, H = d->H, E = d->E, I = d->I, k = d->top_k, P = T * k;
  float* GU = reinterpret_cast<float*>(ws + B.gu);
  float* dAu = reinterpret_cast<float*>(ws + B.dau);
  uint16_t* dgu_hi = reinterpret_cast<uint16_t*>(ws + B.dgu);
  uint16_t* dgu_lo = reinterpret_cast<uint16_t*>(ws + B.dgu_lo);
  uint16_t* aw_hi = reinterpret_cast<uint16_t*>(ws + B.aw);
  uint16_t* aw_lo = reinterpret_cast<uint16_t*>(ws + B.aw_lo);
  float* dws = reinterpret_cast<float*>(ws + B.dws);
  float* dXr = reinterpret_cast<float*>(ws + B.dxr_rows);
  uint16_t* dl_hi = reinterpret_cast<uint16_t*>(ws + B.dl);
  uint16_t* dl_lo = reinterpret_cast<uint16_t*>(ws + B.dl_lo);
  float* dxr = reinterpret_cast<float*>(ws + B.dxr);

  // counters, then the dense logit gradients (only the selected entries are written)
  hipLaunchKernelGGL(k_zero, dim3(16), dim3(256), 0, st, p.err, (p.zero_bytes + 256) / 4);
  HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_bwd_zero, dim3(di.cus * 4), dim3(256), 0, st, reinterpret_cast<uint32_t*>(dl_hi),
                     (B.dxr - B.dl) / 4);        // both parts
  HIP_TRY(hipGetLastError());
  p.tile_rows = kBwdBM;
  TRY(launch_permute(p, p.row_of, st));          // perm, offsets, row_of, row tiles of at most kBwdBM

  const auto up = [](long a, long b) { return (unsigned)((a + b - 1) / b); };
  const unsigned pairs = (unsigned)p.max_tiles;     // row-tile slots (launch_bwd_gemm pads them)
  const long H2 = 2L * I;
  BwdGemm g{};
  g.tiles = p.tiles;
  g.ntiles = p.meta;
  g.offsets = p.offsets;
  const long Pl = P;
  // x and dy in permuted row order (the weight-gradient products' B)
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws + B.xp);
  uint16_t* dyp = reinterpret_cast<uint16_t*>(ws + B.dyp);
  hipLaunchKernelGGL(k_bwd_gather, dim3(di.cus * 8), dim3(256), 0, st, static_cast<const uint16_t*>(x), p.perm, k, H,
                     Pl, xp);
  HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(k_bwd_gather, dim3(di.cus * 8), dim3(256), 0, st, static_cast<const uint16_t*>(dy), p.perm, k,
                     H, Pl, dyp);
  HIP_TRY(hipGetLastError());
  // GU = x[tok] W_gu[e]^T
  g.a = bwd_op(x, H, 0, p.perm, k);
  g.b = bwd_op(w_gate_up, H, 1, nullptr, 1, H2 * H);
  g.a_bytes = (long)T * H * 2; g.b_bytes = H2 * H * 2;
  g.c = GU; g.ldc = H2; g.N = (int)H2; g.K = H; g.group = BWD_GROUP_ROWS;
  TRY(launch_bwd_gemm(g, pairs, up(H2, kBwdBN), 1, st));
  // dAu = dy[tok] W_d[e]
  g.a = bwd_op(dy, H, 0, p.perm, k);
  g.b = bwd_op(w_down, I, 0, nullptr, 1, (long)H * I);
  g.a_bytes = (long)T * H * 2; g.b_bytes = (long)H * I * 2;
  g.c = dAu; g.ldc = I; g.N = I; g.K = H;
  TRY(launch_bwd_gemm(g, pairs, up(I, kBwdBN), 1, st));
  // rows: dw, dG|dU, w a
  hipLaunchKernelGGL(k_bwd_rows, dim3(P), dim3(256), 0, st, GU, dAu, p.perm, topk_weights, I, P, dgu_hi, dgu_lo,
                     aw_hi, aw_lo, dws);
  HIP_TRY(hipGetLastError());
  // dXr = [dG|dU] W_gu[e]
  g.a = bwd_op2(dgu_hi, dgu_lo, H2, 0);
  g.b = bwd_op(w_gate_up, H, 0, nullptr, 1, H2 * H);
  g.a_bytes = Pl * H2 * 2; g.b_bytes = H2 * H * 2;
  g.c = dXr; g.ldc = H; g.N = H; g.K = (int)H2;
  TRY(launch_bwd_gemm(g, pairs, up(H, kBwdBN), 1, st));
  // dW_gu[e] = sum_p [dG|dU]_p^T x[tok(p)] (x in permuted order)
  g.a = bwd_op2(dgu_hi, dgu_lo, H2, 1);
  g.b = bwd_op(xp, H, 0);
  g.a_bytes = Pl * H2 * 2; g.b_bytes = Pl * H * 2;
  g.c = dw_gate_up; g.ldc = H; g.c_gstride = H2 * H; g.M = (int)H2; g.N = H; g.group = BWD_GROUP_K;
  TRY(launch_bwd_gemm(g, up(H2, kBwdBM), up(H, kBwdBN), E, st));
  // dW_d[e] = sum_p dy[tok(p)]^T (w a)_p, formed as its transpose
  // sum_p (w a)_p^T dy[tok(p)] (the split operand as A) and stored transposed
  g.a = bwd_op2(aw_hi, aw_lo, I, 1);
  g.b = bwd_op(dyp, H, 0);
  g.a_bytes = Pl * I * 2; g.b_bytes = Pl * H * 2;
  g.c = dw_down; g.ldc = I; g.c_trans = 1; g.c_gstride = (long)H * I; g.M = I; g.N = H;
  TRY(launch_bwd_gemm(g, up(I, kBwdBM), up(H, kBwdBN), E, st));
  g.c_trans = 0;
  // router: logit gradients, bias, W_r and the router's share of dx
  hipLaunchKernelGGL(k_bwd_router, dim3(up(T, 256)), dim3(256), 0, st, topk_ids, topk_weights, dws, T, E, k, dl_hi,
                     dl_lo);
  HIP_TRY(hipGetLastError());
  if (dbias) {
    hipLaunchKernelGGL(k_bwd_dbias, dim3(E), dim3(256), 0, st, dl_hi, dl_lo, T, E, dbias);
    HIP_TRY(hipGetLastError());
  }
  g.a = bwd_op2(dl_hi, dl_lo, E, 1);
  g.b = bwd_op(x, H, 0);
  g.c = dw_router; g.ldc = H; g.c_gstride = 0; g.M = E; g.N = H; g.K = T; g.group = BWD_GROUP_NONE;
  TRY(launch_bwd_gemm(g, up(E, kBwdBM), up(H, kBwdBN), 1, st));
  g.a = bwd_op2(dl_hi, dl_lo, E, 0);
  g.b = bwd_op(router_w, H, 0);
  g.c = dxr; g.ldc = H; g.M = T; g.N = H; g.K = E;
  TRY(launch_bwd_gemm(g, up(T, kBwdBM), up(H, kBwdBN), 1, st));
  // dx = sum_j dXr[row(t, j)] + dxr
  hipLaunchKernelGGL(k_bwd_dx, dim3(up((long)T * (H / 4), 256)), dim3(256), 0, st, dXr, p.row_of, dxr, T, H, k, dx);
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
