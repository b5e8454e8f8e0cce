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
 *                     [E][2I]            fp32 (FP8 with MOE_WSCALE_CHANNEL:
 *                                        one per output channel, all of K)
 *                     [E][2I][H/32]      E8M0 bytes (FP4, one per 32 along K;
 *                                        MFMA-tiled for moe_forward)
 *                     NULL for BF16
 *   w_down            [E][H][I] (BF16 / FP8) or [E][H][I/2] (FP4), MFMA-tiled
 *   w_down_scales     [E][H/128][I/128] fp32 (FP8), [E][H] fp32 (FP8 with
 *                     MOE_WSCALE_CHANNEL) or [E][H][I/32] E8M0 (FP4,
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
 * the memory channels.)  FP4 E8M0 scales: per K step s and quad q (q =
 * 0 .. N/64-1) 256 bytes at (s*(N/64) + q)*256; byte 4*l + c (l = 0..63,
 * c = 0..3) holds the scale of row 16*t + l%16 for K group 4*s + l/16, where
 * t is the quad's c-th 16-row tile: for the gate|up matrix t = 2q + c (c < 2,
 * gate rows) or N/32 + 2q + c - 2 (c >= 2, the matching up rows), for the
 * down matrix t = 4q + c.  (The four column tiles a wave of a GEMM item
 * multiplies are one quad: their scales are one 4-byte load per lane.)
 * FP8 fp32 block scales stay row-major.
 * moe_pack_weights converts row-major weights into this layout.
 *
 * Supported dtype pairs (act x weight): BF16 x BF16, FP8 x FP8, FP8 x FP4,
 * and BF16 x FP8 / BF16 x FP4: BF16 activations that the layer quantises
 * itself (moe_quantize_input's per-token FP8 quantisation, into the
 * workspace) for the expert GEMMs, while the router reads the BF16 input;
 * x_scales must then be NULL.
 * Limits: T >= 1; H and I multiples of 128 (H <= 16384, I <= 16384);
 * 1 <= top_k <= E; E <= 1024; top_k <= 16; T * top_k * max(Hp, I) * 2 < 4 GiB
 * with Hp = H rounded up to a multiple of 256 (the staging and intermediate
 * rows are addressed with 32-bit offsets).
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

#define MOE_ABI_VERSION 6   /* 3: moe_desc.weight_layout and moe_desc.inter_scale;
                               4: moe_desc.weight_scale;
                               5: moe_quantize_e5m6, moe_dequantize_e5m6;
                               6: FP4 E8M0 scales packed in quads (weights packed
                                  by an earlier version must be packed again),
                                  staging region N-block major */

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
  MOE_DTYPE_FP4_E2M1 = 2,         /* OCP MX E2M1 with E8M0 scales per 32        */
  MOE_DTYPE_F32 = 3               /* IEEE binary32 (moe_quantize_input only)    */
} moe_dtype;

typedef enum moe_mode {
  MOE_MODE_MEGA = 0,              /* one persistent work-queue kernel (default) */
  MOE_MODE_SEPARATE = 1           /* one kernel per step, in stream order       */
} moe_mode;

/* moe_desc.flags */
#define MOE_FLAG_ROUTING_GIVEN 1  /* topk_ids / topk_weights are inputs: skip the router */
#define MOE_FLAG_TRACE 2          /* persistent kernel: per-workgroup phase timestamps in the
                                     workspace's trace region (see moe_get_workspace_regions) */

/* Layout of the expert weights (and FP4 E8M0 scales) a call receives.
 * moe_forward reads only the MFMA-tiled layout that moe_pack_weights
 * writes; a descriptor that says row-major is rejected there, so weights
 * that were never packed cannot be read as if they were. */
typedef enum moe_weight_layout {
  MOE_LAYOUT_ROW_MAJOR = 0,       /* [E][N][K] as generated / loaded          */
  MOE_LAYOUT_TILED = 1            /* moe_pack_weights output                  */
} moe_weight_layout;

/* Scale of the FP8 re-quantisation of the intermediate activation (FP8
 * activation layers; ignored for BF16 layers).  The quantisation options of
 * youleyou, "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性", section
 * "Tile Kernels" (per-token / per-block FP8 scaling). */
typedef enum moe_inter_scale {
  MOE_INTER_SCALE_F32 = 0,        /* s = fl32(amax / 448) per row per 128 channels   */
  MOE_INTER_SCALE_POW2 = 1        /* s = the smallest power of two >= amax / 448      */
} moe_inter_scale;

/* Granularity of FP8 weight scales (FP8 weights only; FP4 weights always
 * carry E8M0 scales per 32 along K, BF16 none).  The per-block and
 * per-channel options of youleyou, "DeepSeek 模型更新解读 Tile Kernels 与
 * DeepEP V2 新特性", section "Tile Kernels", quantisation bullet.  Channel
 * scales are applied once to each output after its K sum, block scales to
 * each 128-wide K block's partial sum. */
typedef enum moe_weight_scale {
  MOE_WSCALE_BLOCK = 0,           /* fp32 per 128 x 128 block of [N][K]        */
  MOE_WSCALE_CHANNEL = 1          /* fp32 per output channel (row n of [N][K]) */
} moe_weight_scale;

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
  int32_t weight_layout; /* moe_weight_layout of the expert weights  */
  int32_t inter_scale;   /* moe_inter_scale                          */
  int32_t weight_scale;  /* moe_weight_scale (FP8 weights)           */
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
 *   staging       [Hp/256][T*top_k][256] BF16 weighted expert outputs:
 *                 columns 256b .. 256b+255 of row t*top_k+j at
 *                 (b*T*top_k + t*top_k + j)*256 (Hp = H rounded up to 256)
 *   trace         with MOE_FLAG_TRACE (persistent kernel): [1024][8] uint64,
 *                 row b for workgroup b < 1024: the device's constant 100 MHz
 *                 clock at 0 kernel entry, 1 the end of its routing phase
 *                 (no routing item left to claim), 2 the start of its
 *                 gate|up phase (routing done), 3 its last gate|up item
 *                 done, 4 its last down item done, 5 its exit; then
 *                 6 the number of gate|up items and 7 of down items it ran.
 *                 Without the flag the region is empty (offset = total).
 * Returns MOE_OK, or the status of an invalid descriptor. */
#define MOE_TRACE_GROUPS 1024
#define MOE_TRACE_FIELDS 8
typedef struct moe_workspace_regions {
  size_t logits, perm, row_of, offsets, inter, inter_scales, staging, trace, total;
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
 * NULL.  Layouts and errors: see the top of this file.  The weights must
 * be in the MFMA-tiled layout (d->weight_layout == MOE_LAYOUT_TILED; a
 * row-major descriptor returns MOE_ERR_INVALID_ARGUMENT).
 * d->inter_scale selects the scale rule of the layer's own FP8
 * quantisations: the intermediate's re-quantisation and, for BF16 input
 * with FP8 / FP4 weights, the input quantisation (ignored by all-BF16
 * layers).  With MOE_INTER_SCALE_POW2 and FP4 weights those products carry
 * only power-of-two scales, which the matrix-core instruction applies
 * itself (no fp32 promotion). */
moe_status moe_forward(const moe_desc* d,
                       const void* x, const float* x_scales,
                       const void* router_w, const float* router_bias,
                       const void* w_gate_up, const void* w_gate_up_scales,
                       const void* w_down, const void* w_down_scales,
                       void* y, int32_t* topk_ids, float* topk_weights,
                       int32_t* expert_offsets, int32_t* perm,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Per-token FP8 quantisation of activations, the step in front of the
 * router (youleyou, "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性",
 * section "Tile Kernels", quantisation bullet: per-token FP8 quantisation).
 * For each token t and 128-channel block c of x [T][H] (in_dtype
 * MOE_DTYPE_BF16 or MOE_DTYPE_F32, finite values): amax = max |x|;
 * scale_mode MOE_INTER_SCALE_F32: s = fl32(amax / 448), codes = E4M3
 * round-to-nearest-even, saturating to +-448, of fl32(x * fl32(1 / s));
 * MOE_INTER_SCALE_POW2: s = the smallest power of two with 448 s >= amax
 * (clamped to 2^-127 .. 2^127) and codes of x / s (exact scaling); a block
 * of zeros gets s = 1.  (In F32 mode, blocks whose maximum is below
 * 448 * 2^-127 are out of contract: 1/s overflows.)  Outputs xq [T][H] E4M3
 * bytes and x_scales [T][H/128] fp32, the layout moe_forward takes.  1 <= T,
 * H a multiple of 128, T * H < 2^31; pointers 16-byte aligned.  Enqueued
 * on `stream`; errors as moe_forward. */
moe_status moe_quantize_input(int32_t T, int32_t H, int32_t in_dtype, int32_t scale_mode, const void* x,
                              uint8_t* xq, float* x_scales, moe_stream_t stream);

/* Per-token E5M6 quantisation, the third format of the same quantisation
 * bullet (youleyou, "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性",
 * section "Tile Kernels": per-token / per-block / per-channel FP8 / FP4 /
 * E5M6 quantisation).  The pages do not define E5M6; it is read as the
 * IEEE-754-style binary format with 1 sign, 5 exponent (bias 15) and 6
 * fraction bits: subnormals at exponent 0, exponent 31 reserved for
 * infinities and NaN, largest finite 65024.  No matrix-core instruction
 * takes it; it is a storage format (each value is exactly a BF16 number).
 * For each token t and 128-channel block c of x [T][H] (in_dtype
 * MOE_DTYPE_BF16 or MOE_DTYPE_F32, finite values): amax = max |x|;
 * scale_mode MOE_INTER_SCALE_F32: s = fl32(amax / 65024), codes = E5M6
 * round-to-nearest-even, saturating to +-65024, of fl32(x * fl32(1 / s));
 * MOE_INTER_SCALE_POW2: s = the smallest power of two with 65024 s >= amax
 * (clamped to 2^-127 .. 2^127) and codes of x / s; a block of zeros gets
 * s = 1.  Outputs xq [T][3H/2] bytes: the 12-bit codes (sign in bit 11) of
 * a row, two to three bytes, little-endian (byte 0 = the first code's low 8
 * bits, byte 1 = its high 4 bits | the second code's low 4 bits << 4, byte
 * 2 = the second code's high 8 bits), and x_scales [T][H/128] fp32.  1 <= T,
 * H a multiple of 128, T * H < 2^31; pointers 16-byte aligned.  Enqueued on
 * `stream`; errors as moe_quantize_input. */
moe_status moe_quantize_e5m6(int32_t T, int32_t H, int32_t in_dtype, int32_t scale_mode, const void* x,
                             uint8_t* xq, float* x_scales, moe_stream_t stream);

/* Inverse of moe_quantize_e5m6: out [T][H] fp32 = fl32(value(code) * s)
 * for the codes xq [T][3H/2] and scales x_scales [T][H/128] (same layout
 * and limits).  Enqueued on `stream`. */
moe_status moe_dequantize_e5m6(int32_t T, int32_t H, const uint8_t* xq, const float* x_scales, float* out,
                               moe_stream_t stream);

/* Bytes of the library's own device workspace used by moe_forward_static. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same layer and arguments, with the workspace taken from
 * a static device array of MOE_STATIC_WORKSPACE_BYTES (64 MiB) that the
 * library holds on every GPU it runs on until the process ends (decode-sized
 * batches fit: T = 256, H = 7168, E = 256, top-8, I = 2048 needs 34 MiB).
 * The call allocates and frees nothing.  Layers whose moe_workspace_size
 * exceeds the array return MOE_ERR_WORKSPACE_TOO_SMALL.  Every call on one
 * GPU uses that GPU's array, which keeps the last call's contents (each call
 * clears what must start at zero); calls that overlap on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller.
 * The array's intermediate buffers are not readable through the ABI. */
moe_status moe_forward_static(const moe_desc* d,
                              const void* x, const float* x_scales,
                              const void* router_w, const float* router_bias,
                              const void* w_gate_up, const void* w_gate_up_scales,
                              const void* w_down, const void* w_down_scales,
                              void* y, int32_t* topk_ids, float* topk_weights,
                              int32_t* expert_offsets, int32_t* perm, moe_stream_t stream);

/* Gating only (youleyou, "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2
 * 新特性", section "Tile Kernels", gating bullet: top-k expert selection and
 * scoring): router logits l = xhat Wr^T + bias (optional output, [T][E]
 * fp32), the top_k experts per token by logit, descending, ties to the
 * lower index, and their weights, the softmax over the selected logits.
 * Same layouts and error behaviour as moe_forward; needs
 * moe_route_workspace_size(d) bytes of workspace.  d->I, the weight dtype
 * and layout are not used beyond validation. */
moe_status moe_route(const moe_desc* d,
                     const void* x, const float* x_scales,
                     const void* router_w, const float* router_bias,
                     float* logits, int32_t* topk_ids, float* topk_weights,
                     void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Dispatch as a local permutation (机器之心, "DeepSeek悄悄更新：Mega MoE、FP4
 * Indexer来了", section "Mega MoE 是什么？": tokens are dispatched to their
 * experts; youleyou, section "Tile Kernels", MoE routing bullet: the
 * token-to-expert mapping): from topk_ids [T][top_k] (every id in [0, E);
 * ids out of range are clamped) build expert_offsets [E+1], perm
 * [T*top_k] (the flat index t*top_k + j held by each permuted row) and
 * (optional) row_of [T*top_k], the inverse of perm.  Rows are grouped by
 * expert in ascending token order (a stable sort of the flat index by
 * expert).  Needs moe_permute_workspace_size(d) bytes of workspace; errors
 * as moe_forward. */
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
 * when the weights are loaded.  src is row-major whatever d->weight_layout
 * says; pass dst to moe_forward with weight_layout = MOE_LAYOUT_TILED. */
moe_status moe_pack_weights(const moe_desc* d, int32_t which, const void* src, const void* src_scales,
                            void* dst, void* dst_scales, moe_stream_t stream);

/* Human-readable name of a status, and the calling thread's last error text. */
/* Backward pass of the layer: the gradients of sum(dy * y) with the routing
 * of the forward call (topk_ids, topk_weights) held fixed, the layer being a
 * trainable layer as in the model-layer bullet of youleyou, "DeepSeek 模型更新
 * 解读 Tile Kernels 与 DeepEP V2 新特性", section "Tile Kernels".  With
 * e = topk_ids[t][j], w = topk_weights, g|u = x[t] W_gu[e]^T, a = SwiGLU(g, u):
 *   dW_down[e]    += w[t][j] dy[t]^T a
 *   dW_gate_up[e] += [dg | du]^T x[t],  dg = w dy[t] W_d[e] * u * SiLU'(g),
 *                                       du = w dy[t] W_d[e] * SiLU(g)
 *   dl[t][j]       = w[t][j] (dw[t][j] - sum_i w[t][i] dw[t][i]),  dw[t][j] = <dy[t], a W_d[e]^T>
 *   dW_router[e]  += dl[t][j] x[t],  dbias[e] += dl[t][j]
 *   dx[t]          = sum_j [dg | du] W_gu[e] + sum_j dl[t][j] W_router[e]
 * (the forward pass's rounding of the intermediate is passed straight
 * through).  BF16 layers only (act_dtype = weight_dtype = BF16, else
 * MOE_ERR_UNSUPPORTED); weights in the row-major layout the forward call's
 * caller loaded (weight_layout = ROW_MAJOR, else MOE_ERR_INVALID_ARGUMENT).
 * Inputs: x [T][H], router_w [E][H], w_gate_up [E][2I][H], w_down [E][H][I],
 * dy [T][H] (BF16); topk_ids [T][top_k] int32 and topk_weights fp32 as the
 * forward call returned them.  Outputs (fp32, overwritten): dx [T][H],
 * dw_gate_up [E][2I][H], dw_down [E][H][I], dw_router [E][H], dbias [E]
 * (optional, NULL = not computed).  Sums are fp32; the inputs and weights
 * enter the matrix cores as BF16 (exact), the fp32 intermediates (dg|du, w*a,
 * the logit gradients) as two BF16 parts each (hi + lo, within 2^-17 of the
 * fp32 value).  Asynchronous on `stream`; workspace of
 * moe_backward_workspace_size(d) bytes (0 for an invalid descriptor). */
size_t moe_backward_workspace_size(const moe_desc* d);
moe_status moe_backward(const moe_desc* d, const void* x, const void* router_w, const void* w_gate_up,
                        const void* w_down, const int32_t* topk_ids, const float* topk_weights, const void* dy,
                        float* dx, float* dw_gate_up, float* dw_down, float* dw_router, float* dbias,
                        void* workspace, size_t workspace_bytes, moe_stream_t stream);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */
