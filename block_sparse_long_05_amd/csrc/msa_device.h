// Device helpers shared by the MSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// s_waitcnt vmcnt(n) with the other counters at their maximum (gfx9 encoding): waits until
// at most n of this wave's vector-memory operations are outstanding.
#define MSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)
// The same, and also until every LDS read of this wave has returned (lgkmcnt(0)).
#define MSA_WAIT_VMCNT_LDS(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0070)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache policy of direct global->LDS loads of data that is read once (a decode step streams
// the whole index-key cache and each kept K/V block once): non-temporal (gfx950 "nt"), so the
// stream does not evict reusable lines. Measured on the 8 x 1M decode scan: 311 us instead of
// 361 us for the same 2.15 GB.
constexpr int kLoadOnce = 2;

constexpr int kBlock = 128;
constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- bf16 storage is raw uint16_t --------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Round to nearest even with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// Buffer views (raw buffer loads: 32-bit byte offsets from a base, bounded by a byte count):
// word 3 of a gfx9 buffer descriptor selects 32-bit data and raw access; a load at or past
// the bound returns zeros without touching memory.
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufWord3);
}
constexpr uint32_t kBufNone = 0x80000000u;  // an offset past every view's bound (< 2^31)

// 2^x with the hardware v_exp_f32 (2^-inf = 0; results below 2^-126 flush to 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- element traits -----------------------------------------------------------------
// Operand of one MFMA k-step per lane: 8 bf16 (16 B) or 1 fp32.
struct BF16 {
  typedef uint16_t elem;
  static constexpr int kPerLane = 8;       // elements per lane per MFMA k-step
  static constexpr bool is_bf16 = true;
};
struct F32 {
  typedef float elem;
  static constexpr int kPerLane = 1;
  static constexpr bool is_bf16 = false;
};


// ---- MFMA wrappers --------------------------------------------------------------------
// 32x32 output tile. Lane l holds column l % 32 and rows 8*(r/4) + 4*(l/32) + r%4, r < 16.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// 16x16 output tile. Lane l holds column l % 16 and rows 4*(l/16) + r, r < 4.
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- ordered keys for top-k -------------------------------------------------------------
// Monotone map of finite floats to uint32 (a < b  <=>  key(a) < key(b)); -0.0 == +0.0.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


__device__ __forceinline__ float wave_max_xor(float x, int from_mask) {
  // Max over lanes that differ only in bits >= from_mask (from_mask a power of two).
  for (int m = from_mask; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum_xor(float x, int from_mask) {
  for (int m = from_mask; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace msa
