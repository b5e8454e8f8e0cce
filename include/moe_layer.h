/*
 * moe_layer.h — C ABI of the fused Mixture-of-Experts layer forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  One MoE layer, as described on 机器之心, "DeepSeek悄悄更新：
 * Mega MoE、FP4 Indexer来了", section "Mega MoE 是什么？": every token is
 * dispatched to its experts, goes through a linear map, SwiGLU and a second
 * linear map, and the expert outputs are combined back per token; the whole
 * block runs as one fused kernel.  Gating, routing and quantisation follow
 * youleyou, "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性", section
 * "Tile Kernels" (top-k selection and scoring; token-to-expert mapping with
 * fused expand/reduce and weight normalisation; per-token / per-block FP8 and
 * FP4 quantisation fused with SwiGLU).  Concretely, for token t:
 *
 *   l[e]     = sum_h xhat[t,h] * Wr[e,h] + bias[e]              (fp32 accumulate)
 *   ids      = the top_k experts by l, descending, ties to the lower index
 *   w[j]     = exp(l[ids[j]] - l[ids[0]]) / sum_i exp(l[ids[i]] - l[ids[0]])
 *   g|u      = xhat[t,:] @ W_gate_up[e]^T     (gate = channels 0..I-1, up = I..2I-1)
 *   a        = g / (1 + exp(-g)) * u
 *   ahat     = FP8 E4M3 re-quantisation of a per 128 channels, scale amax/448
 *              (all-BF16 layers round a to BF16 instead)
 *   o_j      = ahat @ W_down[e]^T
 *   y[t,:]   = BF16( sum_j w[j] * o_j )     (fp32 sum in ascending j)
 *
 * Layouts (row-major unless stated, contiguous, caller-owned device memory):
 *   x                 [T][H]    BF16, or FP8 E4M3 bytes with
 *   x_scales          [T][H/128] fp32 (one scale per token per 128 channels)
 *   router_w          [E][H]    BF16
 *   router_bias       [E]       fp32, optional (NULL = no bias)
 *   w_gate_up         [E][2I][H]   BF16 or FP8 E4M3 bytes;
 *                     [E][2I][H/2] FP4 E2M1, two per byte, even K in the low nibble
 *                     -- passed to moe_forward in the MFMA-tiled layout below
 *   w_gate_up_scales  [E][2I/128][H/128] fp32 (FP8, one per 128x128 block)
 *                     [E][2I][H/32]      E8M0 bytes (FP4, one per 32 along K;
 *                                        MFMA-tiled for moe_forward)
 *                     NULL for BF16
 *   w_down            [E][H][I] (BF16 / FP8) or [E][H][I/2] (FP4), MFMA-tiled
 *   w_down_scales     [E][H/128][I/128] fp32 (FP8) or [E][H][I/32] E8M0 (FP4,
 *                     MFMA-tiled)
 *   y                 [T][H]    BF16 (output)
 *   topk_ids          [T][top_k] int32 (output; input with MOE_FLAG_ROUTING_GIVEN)
 *   topk_weights      [T][top_k] fp32  (output; input with MOE_FLAG_ROUTING_GIVEN)
 *   expert_offsets    [E+1] int32, optional output: first permuted row of each expert
 *   perm              [T*top_k] int32, optional output: flat index t*top_k+j held by
 *                     each permuted row (rows grouped by expert, ascending token)
 *
 * MFMA-tiled weight layout.  The expert GEMMs stream weights straight from
 * HBM into matrix-core operand registers; a wave's operand load is 1 KB, and
 * it is contiguous only if the weights are stored in operand order.  For an
 * expert matrix with N rows and K columns (N = 2I, K = H for w_gate_up;
 * N = H, K = I for w_down), let BS be the bytes of one row per 128 columns
 * (BF16 256, FP8 128, FP4 64) and nsteps = K/128.  The tiled matrix of
 * expert e (same size and position as the row-major one) is the sequence of
 * blocks (s, t), s = 0 .. nsteps-1, t = 0 .. N/16-1, block (s, t) at byte
 * (s*(N/16) + t)*16*BS, each made of BS/64 pieces of 1024 bytes: byte
 * 16*l + j of piece p (l = 0..63, j = 0..15) is byte BS*s + 64*p + 16*(l/16)
 * + j of row 16*t + l%16 of the row-major matrix.  (K step major, so that
 * the blocks one K step of a GEMM item reads are adjacent and spread over
 * the memory channels.)  FP4 E8M0 scales: block (s, t) is 64 bytes at
 * (s*(N/16) + t)*64, byte l holding the scale of row 16*t + l%16 for K group
 * 4*s + l/16.  FP8 fp32 block scales stay row-major.
 * moe_pack_weights converts row-major weights into this layout.
 *
 * Supported dtype pairs (act x weight): BF16 x BF16, FP8 x FP8, FP8 x FP4.
 * Limits: T >= 1; H and I multiples of 128 (H <= 16384, I <= 16384);
 * 1 <= top_k <= E; E <= 1024; top_k <= 16; T * top_k * max(H, I) * 2 < 4 GiB
 * (the staging and intermediate rows are addressed with 32-bit offsets).
 * Pointers must be 16-byte aligned.
 *
 * Ownership and asynchrony.  The library never allocates device memory in
 * moe_forward / moe_route / moe_permute: every buffer, including the
 * workspace, belongs to the caller.  Calls enqueue work on `stream` (a
 * hipStream_t; NULL = the default stream) and return; outputs are valid once
 * the stream reaches that point.  Calls on different streams are independent
 * when each has its own workspace.
 *
 * Errors.  Host-detectable problems return a status and never abort; the
 * thread-local string from moe_last_error() describes the last failure.
 * Device-side waits inside the persistent kernel are bounded: if one ever
 * times out the kernel abandons its work and writes a nonzero word at byte
 * offset 0 of the workspace (read it after synchronising the stream).
 *
 * Determinism.  Identical inputs and descriptor on the same device give
 * bitwise-identical outputs; the persistent (MOE_MODE_MEGA) and separate-
 * kernel (MOE_MODE_SEPARATE) modes give bitwise-identical outputs.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2   /* 2: packed weight blocks ordered K step major */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad shape, misalignment      */
  MOE_ERR_UNSUPPORTED = 2,        /* dtype pair, limit or device not supported  */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP runtime call failed (see last error) */
} moe_status;

typedef enum moe_dtype {
  MOE_DTYPE_BF16 = 0,
  MOE_DTYPE_FP8_E4M3 = 1,         /* OCP E4M3 "fn": bias 7, max 448, no inf     */
  MOE_DTYPE_FP4_E2M1 = 2          /* OCP MX E2M1 with E8M0 scales per 32        */
} moe_dtype;

typedef enum moe_mode {
  MOE_MODE_MEGA = 0,              /* one persistent work-queue kernel (default) */
  MOE_MODE_SEPARATE = 1           /* one kernel per step, in stream order       */
} moe_mode;

/* moe_desc.flags */
#define MOE_FLAG_ROUTING_GIVEN 1  /* topk_ids / topk_weights are inputs: skip the router */

typedef struct moe_desc {
  int32_t T;             /* tokens                                   */
  int32_t H;             /* hidden size (K of linear 1, N of linear 2) */
  int32_t E;             /* experts                                  */
  int32_t I;             /* expert intermediate size                 */
  int32_t top_k;         /* experts per token                        */
  int32_t act_dtype;     /* moe_dtype of x: BF16 or FP8_E4M3         */
  int32_t weight_dtype;  /* moe_dtype of expert weights              */
  int32_t mode;          /* moe_mode                                 */
  int32_t flags;         /* MOE_FLAG_*                               */
} moe_desc;

typedef void* moe_stream_t;   /* hipStream_t */

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int32_t moe_abi_version(void);

/* Bytes of device workspace moe_forward needs for this descriptor
 * (0 if the descriptor is invalid).  Host-only; no device call. */
size_t moe_workspace_size(const moe_desc* d);

/* Workspace bytes moe_route and moe_permute need (a prefix of the layer's
 * workspace layout; never more than moe_workspace_size).  0 if invalid. */
size_t moe_route_workspace_size(const moe_desc* d);
size_t moe_permute_workspace_size(const moe_desc* d);

/* Byte offsets, inside the moe_forward workspace, of the layer's internal
 * buffers, for inspection after the call has completed on its stream:
 *   logits        [T][E] fp32 router logits (bias included); when T is small
 *                 the region also holds the router's partial sums over
 *                 slices of H, of which the logits are the first [T][E]
 *   perm, row_of  [T*top_k] int32 (used only when the caller passes no perm)
 *   offsets       [E+1] int32 (used only when the caller passes none)
 *   inter         [T*top_k][I] intermediate activations in permuted row
 *                 order: E4M3 codes (FP8 layers) or BF16 (BF16 layers)
 *   inter_scales  [I/128][T*top_k] fp32 re-quantisation scales (FP8 layers),
 *                 K block major: block c of permuted row r at c*T*top_k + r
 *   staging       [T*top_k][H] BF16 weighted expert outputs, row t*top_k+j
 * Returns MOE_OK, or the status of an invalid descriptor. */
typedef struct moe_workspace_regions {
  size_t logits, perm, row_of, offsets, inter, inter_scales, staging, total;
} moe_workspace_regions;
moe_status moe_get_workspace_regions(const moe_desc* d, moe_workspace_regions* out);

/* Check a descriptor and the pointers of a moe_forward call without touching
 * the device: returns MOE_OK or the status moe_forward would return. */
moe_status moe_validate(const moe_desc* d,
                        const void* x, const float* x_scales,
                        const void* router_w, const float* router_bias,
                        const void* w_gate_up, const void* w_gate_up_scales,
                        const void* w_down, const void* w_down_scales,
                        const void* y, const int32_t* topk_ids, const float* topk_weights,
                        const void* workspace, size_t workspace_bytes);

/* The whole layer (router, top-k, permutation, gate|up GEMM + SwiGLU + FP8
 * requant, down GEMM, weighted combine).  expert_offsets and perm may be
 * NULL.  Layouts and errors: see the top of this file. */
moe_status moe_forward(const moe_desc* d,
                       const void* x, const float* x_scales,
                       const void* router_w, const float* router_bias,
                       const void* w_gate_up, const void* w_gate_up_scales,
                       const void* w_down, const void* w_down_scales,
                       void* y, int32_t* topk_ids, float* topk_weights,
                       int32_t* expert_offsets, int32_t* perm,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Gating only: router logits (optional output, [T][E] fp32, bias included),
 * top-k ids and renormalised softmax weights.  Same layouts as moe_forward;
 * needs moe_route_workspace_size(d) bytes of workspace.  d->I and the
 * weight dtype are not used beyond validation. */
moe_status moe_route(const moe_desc* d,
                     const void* x, const float* x_scales,
                     const void* router_w, const float* router_bias,
                     float* logits, int32_t* topk_ids, float* topk_weights,
                     void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Dispatch as a local permutation: from topk_ids [T][top_k] build
 * expert_offsets [E+1], perm [T*top_k] and (optional) row_of [T*top_k], the
 * inverse of perm.  Rows are grouped by expert in ascending token order.
 * Needs moe_permute_workspace_size(d) bytes of workspace. */
moe_status moe_permute(const moe_desc* d, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* perm, int32_t* row_of,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* moe_pack_weights `which` */
#define MOE_WEIGHTS_GATE_UP 0     /* N = 2I rows, K = H columns per expert */
#define MOE_WEIGHTS_DOWN 1        /* N = H rows,  K = I columns per expert */

/* Convert one expert weight tensor from the row-major layout to the
 * MFMA-tiled layout that moe_forward reads (see the top of this file):
 * src -> dst, both [E] experts of N x K elements of d->weight_dtype.  For
 * FP4 weights the E8M0 scales are converted too (src_scales -> dst_scales,
 * both required); for BF16 / FP8 weights the scale pointers must be NULL
 * (FP8 block scales are used as they are).  Out of place: dst must not
 * overlap src.  A pure byte permutation, enqueued on `stream`; run it once
 * when the weights are loaded. */
moe_status moe_pack_weights(const moe_desc* d, int32_t which, const void* src, const void* src_scales,
                            void* dst, void* dst_scales, moe_stream_t stream);

/* Human-readable name of a status, and the calling thread's last error text. */
const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */
