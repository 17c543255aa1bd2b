// k_diag.hip - diagnostic kernels that measure the two ceilings the hot path runs against on
// this chip, with nothing of the path around them:
//  - k_stream_mix_bf16: the box copy's HBM traffic mix on flat buffers (read src, write dst,
//    read add, write add + src rounded to bf16), 16-byte non-temporal accesses, no boxes and
//    no edges: the stream rate that mix can sustain;
//  - k_mfma_loop: back-to-back MFMAs of the GEMMs' instruction and accumulator layout (16
//    independent 32x32 accumulators per wave, 256 AGPRs) on random register operands, with no
//    loads, stores or LDS traffic: the matrix-pipe rate the chip holds under that load (its
//    clock falls under sustained MFMA work with random data).
#include "bsm_device.hpp"
#include "bsm_internal.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int kMixChunks = 4;   // 16-byte chunks per lane

__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_store(uint4* p, uint4 x) {
  const u32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, (u32x4*)p);
}

// Two bf16 lanes of a word added in float32, each rounded back to bf16 (RNE).
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  const uint16_t lo = f32_to_bf16_bits(bf16_bits_to_f32((uint16_t)a) + bf16_bits_to_f32((uint16_t)b));
  const uint16_t hi = f32_to_bf16_bits(bf16_bits_to_f32((uint16_t)(a >> 16)) + bf16_bits_to_f32((uint16_t)(b >> 16)));
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Lane l of workgroup w moves chunks (w * kMixChunks + c) * 256 + l, c < kMixChunks, all loads
// issued before the first store; chunks at or past n16 are skipped.
__global__ __launch_bounds__(256) void k_stream_mix_bf16(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        uint4* __restrict__ add, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kMixChunks * 256 + threadIdx.x;
  uint4 s[kMixChunks], a[kMixChunks];
#pragma unroll
  for (int c = 0; c < kMixChunks; c++) {
    const int64_t i = base + 256 * c;
    if (i < n16) {
      s[c] = nt_load(src + i);
      a[c] = nt_load(add + i);
    }
  }
#pragma unroll
  for (int c = 0; c < kMixChunks; c++) {
    const int64_t i = base + 256 * c;
    if (i < n16) {
      nt_store(dst + i, s[c]);
      nt_store(add + i, make_uint4(add_bf16x2(a[c].x, s[c].x), add_bf16x2(a[c].y, s[c].y), add_bf16x2(a[c].z, s[c].z),
                                   add_bf16x2(a[c].w, s[c].w)));
    }
  }
}

// A per-lane pseudo-random word (an integer hash of the lane's global index, the dword and
// the seed): operand bits only, no arithmetic of the path.
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// Operand dword d of fragment f: bf16 pairs with random sign and mantissa and exponents of
// +-[2^-8, 2) (finite, no subnormals); E4M3 bytes with the two NaN codes moved to their
// neighbours; E2M1 nibbles as they come (every code is a value).
template <int KIND>
__device__ __forceinline__ uint32_t operand_word(uint32_t seed, uint32_t t, int f, int d) {
  const uint32_t r = hash32(seed ^ hash32(t * 64u + (uint32_t)(8 * f + d)));
  if (KIND == BSM_BF16) {
    const uint32_t lo = (r & 0x807Fu) | ((119u + ((r >> 7) & 7u)) << 7);
    const uint32_t h = r >> 16;
    const uint32_t hi = (h & 0x807Fu) | ((119u + ((h >> 7) & 7u)) << 7);
    return lo | (hi << 16);
  } else if (KIND == BSM_E4M3) {
    uint32_t w = r;
#pragma unroll
    for (int b = 0; b < 4; b++)
      if (((w >> (8 * b)) & 0x7Fu) == 0x7Fu) w ^= 1u << (8 * b);
    return w;
  }
  return r;
}

// 16 accumulators per wave, each MFMA k of iteration it taking A fragment k / 4 and B fragment
// k % 4 (the GEMMs' 4 x 4 accumulator blocks); the result sum goes to out[t] so nothing is dead.
template <int KIND>
__global__ __launch_bounds__(256, 1) void k_mfma_loop(uint32_t seed, int iters, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  i32x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; f++)
#pragma unroll
    for (int d = 0; d < 8; d++) {
      a[f][d] = (int)operand_word<KIND>(seed, t, f, d);
      b[f][d] = (int)operand_word<KIND>(seed, t, 4 + f, d);
      if (KIND == BSM_E2M1 && d >= 4) a[f][d] = b[f][d] = 0;
    }
  f32x16 acc[16];
#pragma unroll
  for (int k = 0; k < 16; k++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[k][r] = 0.0f;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int k = 0; k < 16; k++) {
      const int fa = k >> 2, fb = k & 3;
      if constexpr (KIND == BSM_BF16) {
        const u32x4 x = {(uint32_t)a[fa][0], (uint32_t)a[fa][1], (uint32_t)a[fa][2], (uint32_t)a[fa][3]};
        const u32x4 y = {(uint32_t)b[fb][0], (uint32_t)b[fb][1], (uint32_t)b[fb][2], (uint32_t)b[fb][3]};
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, y), __builtin_bit_cast(bf16x8, x),
                                                         acc[k], 0, 0, 0);
      } else {
        constexpr int code = KIND == BSM_E4M3 ? 0 : 4;
        acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[fb], a[fa], acc[k], code, code, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k++)
#pragma unroll
    for (int r = 0; r < 16; r++) s += acc[k][r];
  out[t] = s;
}

}  // namespace

hipError_t launch_stream_mix_bf16(const void* src, void* dst, void* add, int64_t n, hipStream_t st) {
  const int64_t n16 = n / 8;
  const int64_t wgs = (n16 + kMixChunks * 256 - 1) / (kMixChunks * 256);
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_mix_bf16, dim3((unsigned)wgs), dim3(256), 0, st, (const uint4*)src, (uint4*)dst,
                     (uint4*)add, n16);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int kind, int64_t workgroups, int iters, float* out, hipStream_t st) {
  const uint32_t seed = 0x5EEDu;
  if (kind == BSM_BF16)
    hipLaunchKernelGGL(k_mfma_loop<BSM_BF16>, dim3((unsigned)workgroups), dim3(256), 0, st, seed, iters, out);
  else if (kind == BSM_E4M3)
    hipLaunchKernelGGL(k_mfma_loop<BSM_E4M3>, dim3((unsigned)workgroups), dim3(256), 0, st, seed, iters, out);
  else
    hipLaunchKernelGGL(k_mfma_loop<BSM_E2M1>, dim3((unsigned)workgroups), dim3(256), 0, st, seed, iters, out);
  return hipGetLastError();
}

}  // namespace bsm
