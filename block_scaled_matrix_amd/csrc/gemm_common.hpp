// gemm_common.hpp - pieces shared by the dense and block-scaled GEMM kernels.
#pragma once
#include "bsm_device.hpp"
#include "bsm_internal.hpp"

namespace bsm {
namespace gemm {

// Direct HBM -> LDS copy of 16 bytes per lane: lane l copies base + voff (its own
// 32-bit byte offset from the wave-uniform base) to LDS byte lds_addr + 16 * l
// (lds_addr wave-uniform). Issued through inline assembly so that the compiler does
// not serialise it against LDS reads of the other pipeline stage: the kernels wait for
// these copies themselves (wait_dma) before the stage barrier.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = (uint64_t)base;
  // readfirstlane yields a signed int: widen through uint32_t so that the low word is
  // zero-extended (sign extension would corrupt the high half of the address).
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(a) : "memory", "m0");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(BSM_LDS const void*)p;
}

// Workgroup -> output tile. The dispatcher sends workgroup p to XCD p % 8; when the
// tile count divides by 8 the ids are renumbered so that each XCD owns one contiguous
// range of tiles, then walked in groups of GROUP_M tile rows (column-major inside a
// group) so that the workgroups resident on one XCD share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 4;
  const int total = tiles_m * tiles_n;
  int lid = pid;
  if ((total & 7) == 0) lid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int g = lid / per_group;
  const int first = g * GROUP_M;
  const int gsize = min(tiles_m - first, GROUP_M);
  const int in = lid - g * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

// D = s * acc (+ D) for a 128 x 128 wave sub-tile held as 4 x 4 blocks of
// v_mfma 32x32 accumulators: register r of block (mt, nt) is row
// 32mt + 8(r/4) + 4(l/32) + r%4, column 32nt + l%32.
__device__ __forceinline__ void store_tile(float* __restrict__ D, int64_t ldd, int64_t M, int64_t N, int64_t row0,
                                           int64_t col0, int lane, float sgn, int accum, const f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      const int64_t col = col0 + 32 * nt + (lane & 31);
      const bool cok = col < N;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = row0 + 32 * mt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (cok && row < M) {
          float* d = D + row * ldd + col;
          const float v = sgn * acc[mt][nt][r];
          *d = accum ? *d + v : v;
        }
      }
    }
  }
}

}  // namespace gemm
}  // namespace bsm
