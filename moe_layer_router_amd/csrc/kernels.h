// Kernel entry points and the workspace plan shared by the host code.
#pragma once
#include "device_common.h"
#include "expert_gemm.h"
#include "permute.h"
#include "quant.h"
#include "router.h"

namespace moe {

// Counters at the start of the zeroed workspace region.
enum {
  CTR_QUEUE = 0,      // persistent-kernel work queue head
  CTR_COUNT_DONE,     // histogram items finished
  CTR_SCATTER_DONE,   // scan-and-scatter items finished
  CTR_G1_DONE,        // gate|up items finished
  CTR_QUEUE2,         // persistent kernel: queue head after the gate|up items
  CTR_SXP_DONE,       // permuted activation-scale items finished
  CTR_QUANT_DONE,     // input quantisation items finished
  CTR_Q1 = 8,         // [kXcds] gate|up item queues, one per expert class
  CTR_Q2 = 16,        // [kXcds] down item queues (separate kernels)
  CTR_NUM = 32
};

// Everything a kernel needs: shapes, caller buffers and workspace regions.
struct Plan {
  int T, H, E, I, k;
  int act_fp8, wdt;            // ACT_*, W_* (act_fp8: the expert GEMMs read FP8 activations)
  int quant_in;                // BF16 input quantised in the layer: router reads xb, experts x
  int pow2;                    // power-of-two scales for the layer's own quantisations
  int wchan;                   // FP8 weights with one scale per output channel
  int routing_given;
  int head_given;              // persistent kernel: routing and permutation already done by the
                               // separate kernels in the same stream (its head queue is empty)
  int nblk;                    // 256-token blocks
  int nTR, nER;                // router tiles (kRouterTokens x kRouterExperts)
  int nKS;                     // router K slices (partial logits summed by the top-k)
  int max_tiles;
  int tile_rows;               // rows of a full GEMM tile
  int nnb1, nnb2;              // N blocks of gate|up (128 channels) and down (256 columns)
  int nCT;                     // combine token chunks per N block
  int comb_tokens;             // tokens per combine item (kCombineTokens, fewer for small T)
  // caller buffers
  const uint8_t* x; const float* x_scales; const uint16_t* wr; const float* bias;
  const uint16_t* xb;          // BF16 input (quant_in), the router's input
  const uint8_t* w_gu; const void* w_gu_scales; const uint8_t* w_d; const void* w_d_scales;
  uint16_t* y; int32_t* ids; float* wts; int32_t* offsets; int32_t* perm;
  // workspace
  int32_t* err;                // device error word (byte offset 0)
  int32_t* ctr;                // [CTR_NUM]
  int32_t* rdone;              // [nTR]    router items finished per token tile
  int32_t* rtile;              // [nTR*nER] K slices finished per router tile (separate router kernel)
  int32_t* tkdone;             // [nblk]   top-k items finished per 256-token block
  int32_t* done1;              // [max_tiles] gate|up items finished per tile
  int32_t* done2;              // [nnb2]   down items finished per N block
  size_t zero_bytes;           // bytes to clear from ctr up to the end of done2
  float* logits; int32_t* blockcnt; int32_t* base; int32_t* row_of;
  Tile* tiles; int32_t* meta;
  uint8_t* aq; float* sa; uint16_t* staging;
  float* sxp;                  // [H/128][T*k] activation scales, permuted rows, or NULL
  uint64_t* trace;             // [MOE_TRACE_GROUPS][MOE_TRACE_FIELDS] phase stamps, or NULL
};

constexpr int kTraceGroups = 1024;
constexpr int kTraceFields = 8;
// Phase stamp i of the calling workgroup (thread 0; the constant-rate clock).
DEV void trace_stamp(uint64_t* trace, int i) {
  if (trace && threadIdx.x == 0 && blockIdx.x < kTraceGroups)
    trace[blockIdx.x * kTraceFields + i] = __builtin_amdgcn_s_memrealtime();
}
DEV void trace_count(uint64_t* trace, int i, uint64_t n) {
  if (trace && threadIdx.x == 0 && blockIdx.x < kTraceGroups) trace[blockIdx.x * kTraceFields + i] = n;
}

constexpr int kCombineTokens = 256;

// Per-class work queues over (tile, N block) items.  A workgroup on XCD x
// takes items of class x (tiles first[x] .. first[x+1], a copy of meta[1..]
// in LDS) and, once those are all claimed, moves on to the following
// classes.  Returns the global item index, or -1 when every class is
// exhausted.  `cls` is the workgroup's current class (start: its XCD),
// advanced as classes run dry.  Called by one thread.
DEV int pop_class_item(int32_t* queues, const int* first, int nnb, int* cls) {
  for (int n = 0; n < kXcds; ++n) {
    const int x = *cls;
    const int lo = first[x] * nnb, cnt = first[x + 1] * nnb - lo;
    if (cnt > 0) {
      const int j = __hip_atomic_fetch_add(&queues[x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (j < cnt) return lo + j;
    }
    *cls = (x + 1) % kXcds;
  }
  return -1;
}

__host__ __device__ inline GemmArgs gemm_args(const Plan& p) {
  GemmArgs g;
  g.x = p.x; g.x_scales = p.x_scales; g.perm = p.perm; g.topk_w = p.wts;
  g.w_gu = p.w_gu; g.w_gu_scales = p.w_gu_scales; g.w_d = p.w_d; g.w_d_scales = p.w_d_scales;
  g.aq = p.aq; g.sa = p.sa; g.staging = p.staging; g.sxp = p.sxp;
  g.T = p.T; g.H = p.H; g.E = p.E; g.I = p.I; g.k = p.k;
  g.pow2 = p.pow2;
  g.wchan = p.wchan;
  g.pow2_x = p.pow2 && p.quant_in;
  return g;
}

}  // namespace moe
