// Microbenchmarks of the machine peaks the layer is measured against
// (matrix-core issue rate per operand format, HBM read bandwidth).  See
// include/moe_peaks.h for the interface.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_peaks.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;        // independent accumulators per wave

template <int KIND>
__device__ __forceinline__ void step(v4f (&c)[kChains], v16f (&d)[kChains], const v8i& a, const v8i& b) {
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    if (KIND == MOE_PEAK_MFMA16_FP8_FP8)
      c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 0, 0, 0, 127, 0, 127);
    else if (KIND == MOE_PEAK_MFMA16_FP4_FP8)
      c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 4, 0, 0, 127, 0, 127);
    else if (KIND == MOE_PEAK_MFMA16_FP4_FP4)
      c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 4, 4, 0, 127, 0, 127);
    else if (KIND == MOE_PEAK_MFMA16_BF16)
      c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, v4i{a[0], a[1], a[2], a[3]}),
                                                     __builtin_bit_cast(v8bf, v4i{b[0], b[1], b[2], b[3]}), c[i],
                                                     0, 0, 0);
    else if (KIND == MOE_PEAK_MFMA32_FP8_FP8)
      d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d[i], 0, 0, 0, 127, 0, 127);
    else
      d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, d[i], 4, 0, 0, 127, 0, 127);
  }
}

template <int KIND>
__global__ void __launch_bounds__(256) k_peak_mfma(int iters, float* sink, uint64_t* cycles) {
  const int tid = threadIdx.x;
  // small finite operands in every format (no NaN codes): bytes 0x11..0x3F
  const int base = 0x11111111 + (tid & 31) * 0x01010101;
  const v8i a = {base, base + 1, base + 2, base + 3, base ^ 4, base ^ 5, base ^ 6, base ^ 7};
  const v8i b = {base + 8, base + 9, base ^ 2, base ^ 3, base + 5, base + 4, base ^ 1, base};
  v4f c[kChains];
  v16f d[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    c[i] = v4f{0.f, 0.f, 0.f, 0.f};
    d[i] = v16f{};
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) step<KIND>(c, d, a, b);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += c[i][0] + c[i][3] + d[i][0] + d[i][15];
  sink[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) cycles[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

__global__ void __launch_bounds__(256) k_peak_read(const v4i* buf, uint64_t n16, uint32_t* sink) {
  // 64 KB chunks (4096 pieces of 16 bytes), 16 pieces per thread per chunk,
  // consecutive lanes on consecutive pieces
  constexpr uint64_t kChunk = 4096;
  uint32_t x = 0;
  const uint64_t nchunks = (n16 + kChunk - 1) / kChunk;
  for (uint64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const uint64_t b0 = ch * kChunk;
    v4i v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint64_t i = b0 + (uint64_t)j * 256 + threadIdx.x;
      v[j] = (i < n16) ? __builtin_nontemporal_load(buf + i) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) x ^= (uint32_t)(v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3]);
  }
  sink[blockIdx.x * 256 + threadIdx.x] = x;
}

double flops_per_instr(int kind) {
  switch (kind) {
    case MOE_PEAK_MFMA16_FP8_FP8:
    case MOE_PEAK_MFMA16_FP4_FP8:
    case MOE_PEAK_MFMA16_FP4_FP4: return 2.0 * 16 * 16 * 128;
    case MOE_PEAK_MFMA16_BF16: return 2.0 * 16 * 16 * 32;
    case MOE_PEAK_MFMA32_FP8_FP8:
    case MOE_PEAK_MFMA32_FP4_FP8: return 2.0 * 32 * 32 * 64;
  }
  return 0.0;
}

template <int KIND>
hipError_t launch(int iters, int blocks, float* sink, uint64_t* cycles, hipStream_t st) {
  hipLaunchKernelGGL(k_peak_mfma<KIND>, dim3(blocks), dim3(256), 0, st, iters, sink, cycles);
  return hipGetLastError();
}

}  // namespace

extern "C" {

double moe_peak_mfma_flops(int32_t kind, int32_t iters, int32_t blocks) {
  return flops_per_instr(kind) * kChains * (double)iters * 4.0 * (double)blocks;
}

moe_status moe_peak_mfma(int32_t kind, int32_t iters, int32_t blocks, float* sink, uint64_t* cycles,
                         moe_stream_t stream) {
  if (kind < 0 || kind >= MOE_PEAK_NUM || iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > (1 << 16) ||
      !sink || !cycles)
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  switch (kind) {
    case MOE_PEAK_MFMA16_FP8_FP8: e = launch<MOE_PEAK_MFMA16_FP8_FP8>(iters, blocks, sink, cycles, st); break;
    case MOE_PEAK_MFMA16_FP4_FP8: e = launch<MOE_PEAK_MFMA16_FP4_FP8>(iters, blocks, sink, cycles, st); break;
    case MOE_PEAK_MFMA16_FP4_FP4: e = launch<MOE_PEAK_MFMA16_FP4_FP4>(iters, blocks, sink, cycles, st); break;
    case MOE_PEAK_MFMA16_BF16: e = launch<MOE_PEAK_MFMA16_BF16>(iters, blocks, sink, cycles, st); break;
    case MOE_PEAK_MFMA32_FP8_FP8: e = launch<MOE_PEAK_MFMA32_FP8_FP8>(iters, blocks, sink, cycles, st); break;
    default: e = launch<MOE_PEAK_MFMA32_FP4_FP8>(iters, blocks, sink, cycles, st); break;
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_peak_hbm_read(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink, moe_stream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15) || bytes > (1ull << 40) ||
      blocks < 1 || blocks > (1 << 16))
    return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(k_peak_read, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(buf), (uint64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
