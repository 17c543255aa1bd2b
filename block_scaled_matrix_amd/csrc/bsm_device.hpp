// bsm_device.hpp - device-side helpers shared by the gfx950 kernels of libbsm.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BSM_LDS __attribute__((address_space(3)))

namespace bsm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Byte permutation of a swizzled shared image (modes 1/2/3 = 32/64/128-byte
// swizzle): the 16-byte chunk index (bits 4..) is XORed with the 128-byte row
// index (bits 7..) over log2(period/128) bits. Mode 3 is the 128-byte form
// offset ^ ((offset >> 3) & 112) of "Explicit CUDA tile patterns", Shared matrix
// descriptors.
__device__ __forceinline__ uint32_t image_swizzle(uint32_t off, int mode) {
  const uint32_t mask = 16u * ((1u << mode) - 1u);
  return off ^ ((off >> 3) & mask);
}

// Wave-wide direct global->LDS copy of 16 bytes per lane: lane l's 16 bytes land at
// lds_base + 16*l (lds_base must be wave-uniform).
__device__ __forceinline__ void load_lds_16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (BSM_LDS void*)lds_base, 16, 0, 0);
}

// The silu_affine scalar epilogue in float32 ("Explicit CUDA tile patterns", Scalar
// compositions): y = x / (1 + exp(-x)), then y * scale + bias.
// exp(z) is taken as 2^(z log2 e) on the hardware base-2 exponential (v_exp_f32). The
// product p = z log2 e is rounded; its remainder r = z log2 e - p (exact fma against the
// float part of log2 e, plus z times the rest of it) enters as the first-order factor
// 2^r = 1 + r ln 2, so exp keeps a few-ulp relative error at every |z| instead of the
// |z| 2^-24 that the rounded product alone would leave. Outside |x| < 88 (exp(-x) beyond
// float range or below half an ulp of 1, and for infinities and NaN, where r is not finite)
// the factor is skipped. The quotient is x times the hardware reciprocal (1 ulp) of 1 + e.
// So a large negative x gives y = -0 once e overflows, x = -inf gives NaN (-inf * 0), and
// NaN stays NaN.
__device__ __forceinline__ float silu_affine(float x, float scale, float bias) {
  constexpr float kLog2e = 0x1.715476p+0f;      // log2(e) rounded to float
  constexpr float kLog2eRest = 0x1.4ae0cp-26f;  // log2(e) - kLog2e, to float
  constexpr float kLn2 = 0x1.62e43p-1f;
  const float z = -x;
  const float p = z * kLog2e;
  const float r = __builtin_fmaf(z, kLog2eRest, __builtin_fmaf(z, kLog2e, -p));
  const float e0 = __builtin_amdgcn_exp2f(p);
  const float e = __builtin_fabsf(x) < 88.0f ? __builtin_fmaf(e0, r * kLn2, e0) : e0;
  const float y = x * __builtin_amdgcn_rcpf(1.0f + e);
  return __builtin_fmaf(y, scale, bias);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_read_b128(const void* p) {
  const u32x4 v = *(const BSM_LDS u32x4*)(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void lds_write_b128(void* p, uint4 v) {
  u32x4 x = {v.x, v.y, v.z, v.w};
  *(BSM_LDS u32x4*)(p) = x;
}

// Transposing LDS read: within each 16-lane group, result lane i element e is the
// 16-bit value i%4 of the 8 bytes addressed by lane 4e + i/4.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSM_LDS i16x4*)(p));
}

// Round-to-nearest-even float -> 16-bit formats, and the exact widening back.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 b = (_Float16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

}  // namespace bsm
