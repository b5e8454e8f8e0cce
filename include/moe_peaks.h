/*
 * moe_peaks.h — measured machine peaks for the roofline of the MoE layer
 * (AMD Instinct MI355X, gfx950).
 *
 * The layer's kernels are judged against the matrix-core issue rate of the
 * operand formats they use (FP8 x FP8, FP8 x FP4, BF16) and against the HBM
 * read bandwidth, the two bounds of a MoE layer that streams block-scaled
 * expert weights (机器之心, "DeepSeek悄悄更新：Mega MoE、FP4 Indexer来了",
 * section "Mega MoE 是什么？", names the FP8 x FP4 operator; youleyou,
 * "DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性", section "Tile
 * Kernels", states the goal of approaching the hardware limits).  These
 * kernels measure those rates on the device at hand, so that nominal peaks
 * can be checked rather than assumed.  They touch only the caller's buffers.
 *
 * Errors and ownership follow moe_layer.h: every pointer is caller-owned
 * device memory, calls enqueue on `stream` and return a moe_status.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#include "moe_layer.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core instruction whose issue rate moe_peak_mfma measures. */
typedef enum moe_peak_kind {
  MOE_PEAK_MFMA16_FP8_FP8 = 0,   /* v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3            */
  MOE_PEAK_MFMA16_FP4_FP8 = 1,   /* the same, E2M1 (A, with E8M0 scales) x E4M3 (B)          */
  MOE_PEAK_MFMA16_FP4_FP4 = 2,   /* the same, E2M1 x E2M1                                    */
  MOE_PEAK_MFMA16_BF16 = 3,      /* v_mfma_f32_16x16x32_bf16                                  */
  MOE_PEAK_MFMA32_FP8_FP8 = 4,   /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3            */
  MOE_PEAK_MFMA32_FP4_FP8 = 5,   /* the same, E2M1 x E4M3                                    */
  MOE_PEAK_NUM = 6
} moe_peak_kind;

/* Floating-point operations (2 per multiply-add) of one moe_peak_mfma launch
 * with these arguments; 0 for an invalid kind. */
double moe_peak_mfma_flops(int32_t kind, int32_t iters, int32_t blocks);

/* `blocks` workgroups of 256 threads (one wave per SIMD of a CU), each wave
 * issuing iters x 8 independent instructions of `kind` on its registers.
 * sink [blocks * 256] fp32 receives a value that depends on every result
 * (so that no work is dropped); cycles [blocks * 4] uint64 receives, per
 * wave, the shader clock cycles its loop took.  1 <= iters <= 1<<20,
 * 1 <= blocks <= 1<<16. */
moe_status moe_peak_mfma(int32_t kind, int32_t iters, int32_t blocks, float* sink, uint64_t* cycles,
                         moe_stream_t stream);

/* Read `bytes` (a multiple of 16, at most 2^40) of device memory at `buf`
 * (16-byte aligned) with 16-byte loads, spread over `blocks` workgroups of
 * 256 threads in 64 KB chunks; sink [blocks * 256] uint32 receives an XOR of
 * what each thread read. */
moe_status moe_peak_hbm_read(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PEAKS_H */
