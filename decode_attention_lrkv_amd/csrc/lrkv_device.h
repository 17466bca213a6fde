// Device-side helpers shared by the gfx950 kernels of liblrkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Two float32 -> packed bfloat16 pair (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// D = A(16x32) * B(32x16) + C on the matrix cores, bf16 in, fp32 accumulate.
// Lane l supplies row (A) / column (B) l % 16 and 8 consecutive k-slots of
// group l / 16; the result's lane l holds rows 4*(l/16) .. +3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Buffer resources: loads past `bytes` read zero and stores past it are
// dropped by the hardware, so a lane that has nothing to do is given the
// offset kOob instead of a branch (which keeps the memory-instruction count of
// a loop body fixed, and the compiler's waits on earlier loads exact).
constexpr uint32_t kOob = 0x80000000u;
// cache-policy operand of the buffer intrinsics: bit 1 is nt on gfx950
constexpr int kPolicyNt = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
// Streaming load: the non-temporal cache policy (nt) for data read once, such
// as the coefficient rows of a decode.  A read probe shaped like the cache
// (two streams, 2048 waves) moves 6.9 TB/s with it against 6.1 TB/s with
// the default policy, which allocates every line in the caches on its way.
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kPolicyNt));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t voff, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, 0, 0);
}
__device__ __forceinline__ void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, 0, 0);
}
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, (int)voff, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace lrkv
