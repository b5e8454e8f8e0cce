// Device helpers shared by the MoE layer kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DEV __device__ __forceinline__

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------ conversions
// fp32 -> BF16 bits, round to nearest even (finite inputs), with the gfx950
// conversion instruction (v_cvt_pk_bf16_f32; equal to the integer rounding
// u + 0x7FFF + lsb on 8.4M checked pairs, ties and denormals included).
DEV uint32_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two values packed, lo in the low half (one conversion instruction).
DEV uint32_t bf16x2_rne(float lo, float hi) {
  const v2bf v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

DEV float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> E4M3 byte with the hardware converter (round to nearest even);
// the input is clamped to +-448 first, so the result saturates.
DEV uint32_t f32_to_e4m3(float v) {
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}
// Four E4M3 codes packed little-endian (v0 in the low byte), as above.
DEV uint32_t f32x4_to_e4m3x4(float v0, float v1, float v2, float v3) {
  v0 = fminf(fmaxf(v0, -448.0f), 448.0f);
  v1 = fminf(fmaxf(v1, -448.0f), 448.0f);
  v2 = fminf(fmaxf(v2, -448.0f), 448.0f);
  v3 = fminf(fmaxf(v3, -448.0f), 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true);
}

// Monotone map of fp32 onto uint32 (larger float -> larger key); -0 and +0
// map to the same key.
DEV uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV float f32_from_order_key(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------- MFMA
// 16x16x128 block-scaled MFMA (gfx950).  Lane l holds row (A) / column (B)
// l%16.  8-bit operands: lane group g = l/16 holds K 16g..16g+15 (bytes
// 0..15) and K 64+16g..64+16g+15 (bytes 16..31).  4-bit operands: lane group
// g holds K 32g..32g+31, two per byte, even K in the low nibble, in the low
// 16 bytes.  The E8M0 scale supplied by lane l applies to row/column l%16 and
// K 32g..32g+31.  Result: lane l, element v is row 4g+v, column l%16.
DEV v4f mfma_fp8_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// 4-bit A (E2M1, with its E8M0 scales) times 8-bit B (E4M3, with E8M0
// scales, 127 = 1).
DEV v4f mfma_fp4_fp8(const v8i& a, const v8i& b, const v4f& c, int ascale, int bscale = 127) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, ascale, 0, bscale);
}
// E8M0 code of a positive power of two held in fp32 (2^-127, the subnormal
// 0x00400000, gives 0 = 2^-127 as well): its biased exponent field.
DEV int e8m0_of_pow2(float s) { return (int)(__float_as_uint(s) >> 23); }
// 16x16x32 BF16 MFMA: lane l holds row/column l%16, 8 K of group l/16.
DEV v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

DEV v8bf as_v8bf(const v4i& v) { return __builtin_bit_cast(v8bf, v); }

// -------------------------------------------------------- wave reductions
// Max over the 16 lanes of a DPP row (the lanes sharing l/16), returned to
// every lane of the row.  Four DPP moves (swap neighbours, swap pairs, mirror
// halves of 8, mirror the row) instead of cross-lane LDS permutes.
template <int CTRL>
DEV float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
DEV float row_max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));   // row_mirror
  return v;
}

// Max over the four lanes l % 16 + 16 g (g = 0..3), returned to each of
// them: swap neighbouring rows of 16 lanes, then the two halves of the wave.
DEV float max_row_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t h = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(h, h, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Inclusive prefix sum over a workgroup of `nthreads` (multiple of 64) ints.
// `scratch` needs nthreads/64 ints of LDS.  Returns the inclusive sum of the
// thread's value; *total receives the workgroup total.
DEV int block_inclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) scratch[wv] = v;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int s = scratch[i];
    if (i < wv) pre += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return v + pre;
}

// ----------------------------------------------------- memory helpers
// Hide the known bits of a per-lane offset from the optimiser.  LDS
// addresses are then formed as (opaque base + compile-time constant), which
// folds into the DS instruction's immediate offset instead of being
// materialised (and kept live) as one register per constant.
DEV uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
template <typename T>
DEV T lds_ld(const char* lds, uint32_t off) { return *reinterpret_cast<const T*>(lds + off); }
template <typename T>
DEV void lds_st(char* lds, uint32_t off, const T& v) { *reinterpret_cast<T*>(lds + off) = v; }

// ------------------------------------------------------- buffer loads
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
// Raw buffer over [base, base + bytes): 32-bit offsets, and loads past the
// end return zero instead of faulting.  Word 3 = 0x00020000 (CDNA raw
// buffer, 32-bit data format).
DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// A buffer's base, size and scalar offset are wave-uniform by contract (the
// instruction takes them from scalar registers).  Non-inlined device
// functions receive their arguments in vector registers, so the compiler
// cannot see that and would wrap each access in a loop over the distinct
// values; reading the first lane states the uniformity.  Code that runs in
// such functions builds its buffers with make_rsrc_u and passes scalar
// offsets through uni().
DEV uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
DEV rsrc_t make_rsrc_u(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)uni((uint32_t)(b >> 32)) << 32) | uni((uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), 0, (int)uni(bytes), 0x00020000);
}
// Device-coherent scalar accesses (relaxed, device scope): the store writes
// through to memory and the load does not take a line that another XCD's
// L2 may hold stale.  For data that one workgroup hands to another inside a
// kernel, ordered by a relaxed counter after the producer's stores have
// completed (no device-wide fence).
template <typename T>
DEV T ld_coh(const T* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
DEV void st_coh(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Wait until this wave's stores have completed.
DEV void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cache policy of a buffer access (the instruction's cache-coherence bits):
// 0 = default; kCoherent (sc1) = device-scope coherent.  The L2 of each XCD
// is not coherent with the others: data that one workgroup writes and a
// workgroup on another XCD reads inside the same kernel is written with
// kCoherent (stores write through) and read with kCoherent (loads do not use
// L2 lines) unless no L2 can hold an older copy of it, so that no
// device-wide fence (which would write back or invalidate the whole L2) is
// needed between them.
constexpr int kCoherent = 16;

template <int AUX = 0>
DEV v4i buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
template <int AUX = 0>
DEV float buf_ldf(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, AUX));
}
template <int AUX = 0>
DEV void buf_st16(rsrc_t r, uint32_t voff, const v4i& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, 0, AUX);
}
template <int AUX = 0>
DEV void buf_st8(rsrc_t r, uint32_t voff, const v2u& v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, 0, AUX);
}
template <int AUX = 0>
DEV void buf_stf(rsrc_t r, uint32_t voff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, (int)voff, 0, AUX);
}
// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land
// at lds_base + 16*l (lds_base is wave-uniform).
template <int AUX = 0>
DEV void buf_ld16_lds(rsrc_t r, void* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, (int)voff, (int)soff, 0, AUX);
}
// 4 bytes per lane from the buffer straight into LDS: lane l's word lands
// at lds_base + 4*l (lds_base is wave-uniform).
template <int AUX = 0>
DEV void buf_ld4_lds(rsrc_t r, void* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, (int)voff, (int)soff, 0, AUX);
}
// Wait until at most n vector-memory operations of this wave are in flight
// (other counters untouched).  Inline asm, like barrier_vmcnt below, so that
// the compiler cannot drop it when the loads it waits for write LDS.
template <int n>
DEV void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// Workgroup barrier that first waits for this wave's LDS operations and for
// all but its n most recent vector-memory operations.  Unlike
// __syncthreads() it does not wait for every direct-to-LDS load in flight,
// so loads issued for later pipeline stages stay outstanding.  The memory
// clobber keeps the compiler from moving memory accesses across it.  (It
// is inline asm on purpose: the compiler does not know that other waves
// read the LDS that direct loads write, and may relax an s_waitcnt builtin
// that it considers unneeded.)
template <int n>
DEV void barrier_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

DEV v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
DEV void st16(void* p, const v4i& v) { *reinterpret_cast<v4i*>(p) = v; }

}  // namespace moe
