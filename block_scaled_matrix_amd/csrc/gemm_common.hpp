// gemm_common.hpp - pieces shared by the dense and block-scaled GEMM kernels.
#pragma once
#include "bsm_device.hpp"
#include "bsm_internal.hpp"

namespace bsm {
namespace gemm {

// Direct HBM -> LDS copy of 16 bytes per lane: lane l copies base + voff (its own
// 32-bit byte offset from the wave-uniform base) to LDS byte lds_addr + 16 * l (lds_addr
// wave-uniform). Issued through inline assembly so that the compiler does not serialise it
// against LDS reads of the other pipeline stage: the kernels wait for these copies themselves
// (wait_dma, stage barriers) before reading what they brought. The LDS address goes to M0 as
// an operand bound to that register, so the compiler knows M0's contents at every point (a
// clobber of M0, a reserved register, is not guaranteed to be honoured).
// Hazards: the compiler pads its own instructions for the wait states the hardware needs
// but cannot see inside inline assembly, so the copies pad for themselves. A vector-memory
// instruction that reads an SGPR written by the VALU needs 5 wait states after that write:
// the base reaches its SGPRs through v_readfirstlane, followed by an s_nop 4 that claims to
// rewrite them (sgpr_base); that asm is not volatile, so the copies of one tile with the same
// base share one (a schedule that left no wait state between the readfirstlane of a tile base
// and its copy gave intermittent wrong values in a ragged MN-major dense GEMM). An SALU write
// of M0 needs 1 wait state before an LDS-DMA instruction reads it: the s_nop 0 in the copy.
// The SGPRs must not be spilled between the two (a restore is a VALU write): the build
// checks that no kernel spills SGPRs.
__device__ __forceinline__ uint64_t sgpr_base(const void* p) {
  const uint64_t b = (uint64_t)p;
  // readfirstlane yields a signed int: widen through uint32_t so that the low word is
  // zero-extended (sign extension would corrupt the high half of the address).
  uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  asm("s_nop 4" : "+s"(lo), "+s"(hi));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
// Two bases pinned with one s_nop 4 (the A and B tiles of one K tile).
__device__ __forceinline__ void sgpr_base2(const void* p, const void* q, uint64_t& sp, uint64_t& sq) {
  const uint64_t bp = (uint64_t)p, bq = (uint64_t)q;
  uint32_t plo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp);
  uint32_t phi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32));
  uint32_t qlo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bq);
  uint32_t qhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bq >> 32));
  asm("s_nop 4" : "+s"(plo), "+s"(phi), "+s"(qlo), "+s"(qhi));
  sp = ((uint64_t)phi << 32) | (uint64_t)plo;
  sq = ((uint64_t)qhi << 32) | (uint64_t)qlo;
}
// The copy from a base that sgpr_base / sgpr_base2 produced (or SALU arithmetic on one).
__device__ __forceinline__ void dma16u(uint64_t sb, uint32_t voff, uint32_t lds_addr) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "{m0}"(a) : "memory");
}
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  dma16u(sgpr_base(base), voff, lds_addr);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order), i.e. every copy issued before the last N has landed.
#define BSM_WAIT_VMCNT(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

// Direct HBM -> LDS copy of 4 bytes per lane (lane l lands at lds_addr + 4 * l), the same
// way as dma16s.
__device__ __forceinline__ void dma4u(uint64_t sb, uint32_t voff, uint32_t lds_addr) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sb), "{m0}"(a) : "memory");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t voff, uint32_t lds_addr) {
  dma4u(sgpr_base(base), voff, lds_addr);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(BSM_LDS const void*)p;
}

// Workgroup -> output tile. The dispatcher sends workgroup p to XCD p % 8; when the
// tile count divides by 8 the ids are renumbered so that each XCD owns one contiguous
// range of tiles, then walked in groups of GROUP_M tile rows (column-major inside a
// group) so that the workgroups resident on one XCD share A and B panels in its L2.
// GROUP_M 4 measured best against 2, 8 and 16 on the 8192- and 16384-wide block-scaled and
// bf16 GEMMs (BSM_GROUP_M overrides it at build time for such sweeps).
#ifndef BSM_GROUP_M
#define BSM_GROUP_M 4
#endif
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = BSM_GROUP_M;
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

// Waits until at most N of this wave's vector-memory operations are outstanding (they
// complete in issue order) and all of its LDS operations are done, then joins the
// workgroup barrier. The compiler does not count the inline-assembly copies, so the
// kernels place these waits themselves.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Instruction-order fences. The MFMA builtins are pure, so instruction selection may
// place them on either side of the scheduling fences and barriers; an empty volatile asm
// that claims to rewrite a value pins the computations around it: pin_acc after MFMAs
// that must issue before a barrier, pin_frag on the operands of MFMAs that must issue
// after the LDS reads that precede them.
__device__ __forceinline__ void pin_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) asm volatile("" : "+a"(acc[i][j])::"memory");
}
__device__ __forceinline__ void pin_frag(uint4& x) {
  u32x4 v = {x.x, x.y, x.z, x.w};
  asm volatile("" : "+v"(v)::"memory");
  x = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void pin_word(uint32_t& x) { asm volatile("" : "+v"(x)::"memory"); }

// Joins the workgroup barrier once this wave's LDS operations are done (its vector-memory
// copies may still be in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- K-major operand tiles: 256 rows x 128 bytes of K, 32 KiB per tile -------------
// Whole 128-byte cache lines per row: the copy path sustains far more bandwidth with
// full-line requests than with half lines. The 16-byte chunk c of LDS row r is stored
// at physical chunk c ^ ((r >> 1) & 7): the 16 rows that one 16-lane group of a 16-byte
// LDS read touches then cover all 64 banks (2 rows per 256-byte bank window, 8 distinct
// chunks per row parity).
constexpr int kKRowBytes = 128;
constexpr int kKTileBytes = 256 * kKRowBytes;

// Per-lane offsets (bytes, relative to the tile's first row at the tile's first K byte)
// of the 8 direct LDS copies a wave issues per tile. Copy j of wave w fills LDS bytes
// [1024 (w + 4j), +1024), i.e. rows 8 (w + 4j) .. +7: lane l writes row 8 (w + 4j) + l/8,
// physical chunk l%8, which holds logical chunk (l%8) ^ ((row >> 1) & 7). Rows past the
// operand's last row re-read the last row (their results are not stored).
__device__ __forceinline__ void kmajor_dma_offsets(int64_t ld_bytes, int64_t row0, int64_t rows, int w, int lane,
                                                   uint32_t (&off)[8]) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int r = 8 * (w + 4 * j) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t rg = min(row0 + r, rows - 1);
    off[j] = (uint32_t)((rg - row0) * ld_bytes + 16 * c);
  }
}

__device__ __forceinline__ void issue_tile8(const void* base, const uint32_t (&off)[8], uint32_t lds_tile, int w) {
#pragma unroll
  for (int j = 0; j < 8; j++) dma16s(base, off[j], lds_tile + 1024 * (w + 4 * j));
}

// Byte offset inside a K-major tile of logical chunk `chunk` of the row that lane l
// reads for a 32-row fragment block (block and wave offsets are multiples of 16 rows,
// so they add to this without changing the swizzle).
__device__ __forceinline__ uint32_t kmajor_frag_base(int lane, int chunk) {
  const int r = lane & 31;
  return (uint32_t)(r * kKRowBytes + ((chunk ^ ((r >> 1) & 7)) << 4));
}

// The same tile for a partial last K tile, through registers: bytes at or past kb_end
// (relative to the row start) are zero. Same row / chunk assignment as the copies.
__device__ __forceinline__ void kmajor_fill_masked(const uint8_t* __restrict__ p, int64_t ld_bytes, int64_t row0,
                                                   int64_t rows, int64_t kb0, int64_t kb_end, uint8_t* tile,
                                                   int w, int lane) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int i = w + 4 * j;
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t rg = min(row0 + r, rows - 1);
    const int64_t kb = kb0 + 16 * c;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kb < kb_end) {
      v = *(const uint4*)(p + rg * ld_bytes + kb);
      const int64_t valid = kb_end - kb;  // bytes kept
      uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const int64_t nb = valid - 4 * d;
        wd[d] &= nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : (1u << (8 * nb)) - 1u);
      }
      v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    lds_write_b128(tile + 1024 * i + 16 * lane, v);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][nt][r] = 0.0f;
}

// Whole 512-byte row pieces of one 64-row half (rows rowh + r, r < 64, of region), lane
// l moving the 16 bytes at column col of rows 2j + l/32: D = f(x (+ D)), f = silu_affine
// when EW. Eight LDS reads and D loads are in flight ahead of their stores.
typedef __attribute__((address_space(1))) u32x4 global_u32x4;
typedef __attribute__((address_space(1))) float global_f32;
template <bool EW>
__device__ __forceinline__ void store_half_whole(float* __restrict__ D, int64_t ldd, int64_t rowh, int64_t col,
                                                 int lane, int c, const uint8_t* region, bool add, float es,
                                                 float eb) {
#pragma unroll
  for (int j0 = 0; j0 < 32; j0 += 8) {
    uint4 x[8];
    u32x4 y[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int r = 2 * (j0 + j) + (lane >> 5);
      x[j] = lds_read_b128(region + 512 * r + 16 * (c ^ (r & 15)));
      if (add) y[j] = *(global_u32x4*)(D + (rowh + r) * ldd + col);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int r = 2 * (j0 + j) + (lane >> 5);
      u32x4 o = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float v = __uint_as_float(o[e]);
        if (add) v += __uint_as_float(y[j][e]);
        if (EW) v = silu_affine(v, es, eb);
        o[e] = __float_as_uint(v);
      }
      *(global_u32x4*)(D + (rowh + r) * ldd + col) = o;
    }
  }
}

// D = f(s * acc (+ D when `add`)) for a 128 x 128 wave sub-tile held as 4 x 4 blocks of
// v_mfma 32x32 accumulators computed with the operands swapped (the MFMA row index runs over
// N): register 4q + e of block (mt, nt) is output row 32mt + l%32, column
// 32nt + 8q + 4(l/32) + e. f is the scalar epilogue (ew_op 0: identity, 1: silu_affine
// with es, eb), applied in registers to each float32 value just before its store. The
// accumulators pass through this wave's
// 32 KiB region `region` in two halves of 64 rows and leave as stores of two 512-byte row
// pieces per instruction (whole 128-byte lines), instead of 32 rows x 32 bytes per
// instruction, which the memory path takes about twice as long to accept; with `add`, D
// arrives in the same whole-line pieces, eight loads in flight. Region row r (512 bytes)
// keeps its 16-byte chunk c at c ^ (r & 15): the 16 rows written by one 16-lane group then
// cover all 64 banks, and so does a read of 16 consecutive chunks of one row. D is
// addressed as global memory so that the compiler may keep several LDS reads and D loads
// in flight ahead of the stores. A sub-tile that crosses the edge of D touches the
// in-range elements only. The caller has synchronised the workgroup so that nobody still
// reads the region's bytes. (s * acc + D rounds once, as an accumulating MFMA chain started
// from D would round the same terms in another order.)
__device__ __forceinline__ void store_tile_lines(float* __restrict__ D, int64_t ldd, int64_t M, int64_t N, int64_t row0,
                                                 int64_t col0, int lane, float sgn, const f32x16 (&acc)[4][4],
                                                 uint8_t* region, bool add, int ew_op, float es, float eb) {
  const bool whole = row0 + 128 <= M && col0 + 128 <= N;  // wave-uniform
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int m2 = 0; m2 < 2; m2++) {
      const int r = 32 * m2 + (lane & 31);
#pragma unroll
      for (int nt = 0; nt < 4; nt++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int c = 8 * nt + 2 * q + (lane >> 5);
          const f32x16& v = acc[2 * half + m2][nt];
          const uint4 x = make_uint4(__float_as_uint(sgn * v[4 * q]), __float_as_uint(sgn * v[4 * q + 1]),
                                     __float_as_uint(sgn * v[4 * q + 2]), __float_as_uint(sgn * v[4 * q + 3]));
          lds_write_b128(region + 512 * r + 16 * (c ^ (r & 15)), x);
        }
    }
    const int c = lane & 31;
    const int64_t col = col0 + 4 * c;
    if (whole) {
      if (ew_op) store_half_whole<true>(D, ldd, row0 + 64 * half, col, lane, c, region, add, es, eb);
      else store_half_whole<false>(D, ldd, row0 + 64 * half, col, lane, c, region, add, es, eb);
    } else {
      for (int j = 0; j < 32; j++) {
        const int r = 2 * j + (lane >> 5);
        const uint4 x = lds_read_b128(region + 512 * r + 16 * (c ^ (r & 15)));
        const int64_t row = row0 + 64 * half + r;
        if (row < M) {
          global_f32* p = (global_f32*)(D + row * ldd + col);
          const float xv[4] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (col + e < N) {
              float v = add ? xv[e] + p[e] : xv[e];
              if (ew_op) v = silu_affine(v, es, eb);
              p[e] = v;
            }
        }
      }
    }
  }
}

}  // namespace gemm
}  // namespace bsm
