// k_gemm_mx.hip - block-scaled GEMM (MXFP8 E4M3 / MXFP4 E2M1 with E8M0 scales per 32
// K elements) D = s * A * B^T (+ D) on gfx950 v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Semantics ("tcgen05.mma": Weight-stationary and block scaling, Call parameters;
// "Explicit CUDA tile patterns": tcgen05 MMA): operand value = element * 2^(scale-127)
// with one scale per 32 consecutive K elements of a row, float32 accumulation.
//
// gfx950 design (operand layouts probed on the device):
//  - the scaled MFMA takes per lane one 32-bit register of scales and selects a byte
//    with op_sel; for K = 64 per instruction the scale of row i, block b (32 K) is
//    taken from lane i + 32*b;
//  - fp8 operand (32 bytes per lane): lane l holds row l%32 with k in
//    [16(l/32), +16) and [32 + 16(l/32), +16) of the 64-K step;
//  - fp4 operand (16 bytes per lane, two elements per byte, low nibble first): lane l
//    holds row l%32 with k in [32(l/32), +32);
//  - the MFMA is issued with the operands swapped (B first, with B's scales), so a lane
//    holds four consecutive output columns per register group (16-byte epilogue);
//  - workgroup tile 256 x 256 x (128 bytes of K per row), four wave64s with 128 x 128
//    sub-tiles (4 x 4 accumulators of 16 fp32 in AGPRs); operand tiles (whole 128-byte
//    lines per row, the 128-byte-row XOR swizzle shared with the dense kernel) and the
//    scale words of each row stream HBM -> LDS with global_load_lds_dwordx4 / _dword
//    into two stages;
//  - each wave reads a tile's fragments into registers early, so a stage is released
//    after the first 64-K step and the copy of tile kt+2 starts while tile kt is still
//    being multiplied: two K tiles stay in flight. fp8 tiles have two 64-K steps (the
//    barrier for the next tile sits inside the second), fp4 tiles four.
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int ROWB = 128;                  // bytes of K per row per K tile
constexpr int TILE_BYTES = 256 * ROWB;     // 32 KiB per operand tile
static_assert(TILE_BYTES == gemm::kKTileBytes, "K-major tile geometry");

template <int FMT>
struct Fmt {
  static constexpr int KT = FMT == 4 ? 256 : 128;  // K elements per K tile
  static constexpr int STEPS = FMT == 4 ? 4 : 2;   // 64-K MFMA steps per K tile
  static constexpr int EPB = FMT == 4 ? 2 : 1;     // elements per byte
  static constexpr int SFW = FMT == 4 ? 2 : 1;     // scale words per row per K tile
  static constexpr int SF_BYTES = 256 * 4 * SFW;   // scale words of one operand tile
  // stage: A tile, B tile, A scales, B scales (scale word q of row r at 1024 q + 4 r)
  static constexpr int STAGE = 2 * TILE_BYTES + 2 * SF_BYTES;
  static constexpr int DMA_PER_TILE = 16 + 2 * SFW;  // copies per wave per K tile
};

struct Ops {
  const uint8_t* A; int64_t lda_b; uint32_t aoff[8];
  const uint8_t* B; int64_t ldb_b; uint32_t boff[8];
  const uint8_t* SFA; uint32_t sfa_off;
  const uint8_t* SFB; uint32_t sfb_off;
};

// Copies of K tile kt: operand rows from the tile's first row; scale word q of rows
// 64w + l (each wave one 64-row quarter) into LDS word-major order.
template <int FMT>
__device__ __forceinline__ void issue_stage(const Ops& o, int kt, uint32_t stage, int w) {
  typedef Fmt<FMT> F;
  const int64_t kb = (int64_t)kt * ROWB;
  gemm::issue_tile8(o.A + kb, o.aoff, stage, w);
  gemm::issue_tile8(o.B + kb, o.boff, stage + TILE_BYTES, w);
#pragma unroll
  for (int q = 0; q < F::SFW; q++) {
    const int64_t word = 4 * ((int64_t)kt * F::SFW + q);
    gemm::dma4s(o.SFA + word, o.sfa_off, stage + 2 * TILE_BYTES + 1024 * q + 256 * w);
    gemm::dma4s(o.SFB + word, o.sfb_off, stage + 2 * TILE_BYTES + F::SF_BYTES + 1024 * q + 256 * w);
  }
}

// Fragments of one 64-K step for one wave: af/bf[t][0..1] are the 16-byte chunks of
// 32-row block t (fp4 uses [t][0] only).
struct Frags {
  uint4 af[4][2], bf[4][2];
};

// Reads the fragments of 64-K step s of the stage at `st` for this wave. The lane's row
// within a 32-row block is l%32; fp8 step s covers bytes 64s.. of the row: logical chunks
// 4s + l/32 (k 16(l/32)..) and 4s + 2 + l/32 (k 32 + 16(l/32)..); fp4 step s covers bytes
// 32s..: logical chunk 2s + l/32.
template <int FMT>
__device__ __forceinline__ void read_frags(const uint8_t* st, int s, int wa, int wb, int lane, Frags& f) {
  const int h = lane >> 5;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint8_t* pa = st + wa * ROWB + 4096 * t;
    const uint8_t* pb = st + TILE_BYTES + wb * ROWB + 4096 * t;
    if (FMT == 4) {
      const uint32_t o = gemm::kmajor_frag_base(lane, 2 * s + h);
      f.af[t][0] = lds_read_b128(pa + o);
      f.bf[t][0] = lds_read_b128(pb + o);
    } else {
      const uint32_t o0 = gemm::kmajor_frag_base(lane, 4 * s + h), o1 = gemm::kmajor_frag_base(lane, 4 * s + 2 + h);
      f.af[t][0] = lds_read_b128(pa + o0);
      f.af[t][1] = lds_read_b128(pa + o1);
      f.bf[t][0] = lds_read_b128(pb + o0);
      f.bf[t][1] = lds_read_b128(pb + o1);
    }
  }
}

// Raw scale words q of this lane's rows (wave base + 32t + l%32).
template <int FMT>
__device__ __forceinline__ void read_scales(const uint8_t* st, int wa, int wb, int lane, uint32_t (&sa)[4][2],
                                            uint32_t (&sb)[4][2]) {
  typedef Fmt<FMT> F;
  const uint8_t* pa = st + 2 * TILE_BYTES;
  const uint8_t* pb = pa + F::SF_BYTES;
#pragma unroll
  for (int q = 0; q < F::SFW; q++)
#pragma unroll
    for (int t = 0; t < 4; t++) {
      sa[t][q] = *(const BSM_LDS uint32_t*)(pa + 1024 * q + 4 * (wa + 32 * t + (lane & 31)));
      sb[t][q] = *(const BSM_LDS uint32_t*)(pb + 1024 * q + 4 * (wb + 32 * t + (lane & 31)));
    }
}

template <int FMT, int SEL>
__device__ __forceinline__ f32x16 mfma_sc(const uint4 (&b)[2], const uint4 (&a)[2], f32x16 c, uint32_t sb,
                                          uint32_t sa) {
  i32x8 av, bv;
  bv[0] = b[0].x; bv[1] = b[0].y; bv[2] = b[0].z; bv[3] = b[0].w;
  av[0] = a[0].x; av[1] = a[0].y; av[2] = a[0].z; av[3] = a[0].w;
  if (FMT == 4) {
    av[4] = av[5] = av[6] = av[7] = 0;
    bv[4] = bv[5] = bv[6] = bv[7] = 0;
  } else {
    bv[4] = b[1].x; bv[5] = b[1].y; bv[6] = b[1].z; bv[7] = b[1].w;
    av[4] = a[1].x; av[5] = a[1].y; av[6] = a[1].z; av[7] = a[1].w;
  }
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, c, FMT, FMT, SEL, (int)sb, SEL, (int)sa);
}

template <int FMT, int MT0, int MT1>
__device__ __forceinline__ void pin_frags(Frags& f) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    if (t >= MT0 && t < MT1) {
      gemm::pin_frag(f.af[t][0]);
      if (FMT != 4) gemm::pin_frag(f.af[t][1]);
    }
    gemm::pin_frag(f.bf[t][0]);
    if (FMT != 4) gemm::pin_frag(f.bf[t][1]);
  }
}

// MFMAs of accumulator rows mt in [MT0, MT1) for 64-K step s of the tile: scale word
// s / 2 of each row (after the per-lane shift), byte 2 (s & 1) (op_sel).
template <int FMT, int S, int MT0, int MT1>
__device__ __forceinline__ void mfma_rows(const Frags& f, const uint32_t (&sa)[4][2], const uint32_t (&sb)[4][2],
                                          f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = MT0; mt < MT1; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
      acc[mt][nt] = mfma_sc<FMT, 2 * (S & 1)>(f.bf[nt], f.af[mt], acc[mt][nt], sb[nt][S >> 1], sa[mt][S >> 1]);
}

// Right-shift by 8 (l/32): lanes 32..63 carry the second 32-K block of each 64-K step,
// so bytes 0 and 2 become the blocks of the word's two steps for this lane.
template <int FMT>
__device__ __forceinline__ void shift_scales(const uint32_t (&ra)[4][2], const uint32_t (&rb)[4][2], int sh,
                                             uint32_t (&sa)[4][2], uint32_t (&sb)[4][2]) {
#pragma unroll
  for (int q = 0; q < Fmt<FMT>::SFW; q++)
#pragma unroll
    for (int t = 0; t < 4; t++) {
      sa[t][q] = ra[t][q] >> sh;
      sb[t][q] = rb[t][q] >> sh;
    }
}

template <int FMT, bool ACC>
__global__ __launch_bounds__(256, 1) void k_gemm_mx(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Fmt<FMT> F;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * F::STAGE];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nblk = a.K / 32;
  const int wa = 128 * wm, wb = 128 * wn;
  const float sgn = a.negate ? -1.0f : 1.0f;

  // accumulators start from s * D (or zero); D is read here, before the operand copies
  f32x16 acc[4][4];
  if (ACC) gemm::load_acc(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc);
  else gemm::zero_acc(acc);

  Ops o;
  o.lda_b = a.lda / F::EPB;
  o.ldb_b = a.ldb / F::EPB;
  o.A = (const uint8_t*)a.A + m0 * o.lda_b;
  o.B = (const uint8_t*)a.B + n0 * o.ldb_b;
  o.SFA = a.SFA + m0 * a.ld_sfa;
  o.SFB = a.SFB + n0 * a.ld_sfb;
  gemm::kmajor_dma_offsets(o.lda_b, m0, a.M, w, lane, o.aoff);
  gemm::kmajor_dma_offsets(o.ldb_b, n0, a.N, w, lane, o.boff);
  // scale row 64w + l of the tile (clamped to the last row), relative to the first row
  o.sfa_off = (uint32_t)((min(m0 + 64 * w + lane, a.M - 1) - m0) * a.ld_sfa);
  o.sfb_off = (uint32_t)((min(n0 + 64 * w + lane, a.N - 1) - n0) * a.ld_sfb);

  const int nfull = (int)(a.K / F::KT);
  const int tail = (int)(a.K % F::KT);
  const uint32_t lds0 = gemm::lds_addr(lds);
  const int h8 = 8 * (lane >> 5);
  Frags f0, f1, f2, f3;
  uint32_t sa[4][2], sb[4][2], ra[4][2], rb[4][2];
  if (nfull > 0) {
    issue_stage<FMT>(o, 0, lds0, w);
    issue_stage<FMT>(o, min(1, nfull - 1), lds0 + F::STAGE, w);
    gemm::stage_barrier<F::DMA_PER_TILE>();
    read_frags<FMT>(lds, 0, wa, wb, lane, f0);
    read_scales<FMT>(lds, wa, wb, lane, ra, rb);
    shift_scales<FMT>(ra, rb, h8, sa, sb);
  }
  // K tile kt lives in stage kt & 1. The loop body is branch-free so that the scheduling
  // fences hold: past the last tile the copies re-read the last tile (clamped index)
  // into a stage nobody reads again.
  for (int kt = 0; kt < nfull; kt++) {
    const uint8_t* st = lds + (kt & 1) * F::STAGE;
    const uint8_t* nst = lds + ((kt + 1) & 1) * F::STAGE;
    const uint32_t stage = lds0 + (kt & 1) * F::STAGE;
    const int kn = min(kt + 2, nfull - 1);
    if constexpr (FMT == 4) {
      // read steps 1..3; MFMAs of step 0; barrier (stage free); copy tile kt + 2;
      // MFMAs of steps 1, 2; barrier (tile kt + 1 landed); read step 0 and the scales of
      // tile kt + 1; MFMAs of step 3; shift the new scales into place
      read_frags<4>(st, 1, wa, wb, lane, f1);
      read_frags<4>(st, 2, wa, wb, lane, f2);
      read_frags<4>(st, 3, wa, wb, lane, f3);
      pin_frags<4, 0, 4>(f0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<4, 0, 0, 4>(f0, sa, sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      gemm::lds_barrier();
      issue_stage<4>(o, kn, stage, w);
      pin_frags<4, 0, 4>(f1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<4, 1, 0, 4>(f1, sa, sb, acc);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<4, 2, 0, 4>(f2, sa, sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      gemm::stage_barrier<F::DMA_PER_TILE>();
      read_frags<4>(nst, 0, wa, wb, lane, f0);
      read_scales<4>(nst, wa, wb, lane, ra, rb);
      pin_frags<4, 0, 4>(f3);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<4, 3, 0, 4>(f3, sa, sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      shift_scales<4>(ra, rb, h8, sa, sb);
    } else {
      // read step 1; MFMAs of step 0; barrier (stage free); copy tile kt + 2; MFMAs of
      // rows 0-1 of step 1; barrier (tile kt + 1 landed); read step 0 and the scales of
      // tile kt + 1; MFMAs of rows 2-3 of step 1; shift the new scales into place
      read_frags<0>(st, 1, wa, wb, lane, f1);
      pin_frags<0, 0, 4>(f0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<0, 0, 0, 4>(f0, sa, sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      gemm::lds_barrier();
      issue_stage<0>(o, kn, stage, w);
      pin_frags<0, 0, 2>(f1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<0, 1, 0, 2>(f1, sa, sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      gemm::stage_barrier<F::DMA_PER_TILE>();
      read_frags<0>(nst, 0, wa, wb, lane, f0);
      read_scales<0>(nst, wa, wb, lane, ra, rb);
      pin_frags<0, 2, 4>(f1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<0, 1, 2, 4>(f1, sa, sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      shift_scales<0>(ra, rb, h8, sa, sb);
    }
  }
  // Every copy has landed and every wave is done with LDS before stage 0 is refilled
  // (and before the workgroup can end with copies in flight).
  gemm::stage_barrier<0>();
  if (tail) {
    const int64_t kb0 = (int64_t)nfull * ROWB;
    const int64_t kb_end = a.K / F::EPB;
    gemm::kmajor_fill_masked((const uint8_t*)a.A, o.lda_b, m0, a.M, kb0, kb_end, lds, w, lane);
    gemm::kmajor_fill_masked((const uint8_t*)a.B, o.ldb_b, n0, a.N, kb0, kb_end, lds + TILE_BYTES, w, lane);
#pragma unroll
    for (int q = 0; q < F::SFW; q++) {
      // scale word q of the partial tile; blocks at or past nblk (beyond K) become 127
      // (2^0): their operand bytes are zero, and a NaN code in the row padding must not
      // poison them. A word wholly past the row's blocks is not read.
      const int64_t blk = ((int64_t)nfull * F::SFW + q) * 4;
      const int64_t valid = nblk - blk;
      const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : (1u << (8 * valid)) - 1u);
      uint32_t wa_ = 0x7F7F7F7Fu, wb_ = 0x7F7F7F7Fu;
      if (valid > 0) {
        wa_ = (*(const uint32_t*)(o.SFA + o.sfa_off + blk) & keep) | (0x7F7F7F7Fu & ~keep);
        wb_ = (*(const uint32_t*)(o.SFB + o.sfb_off + blk) & keep) | (0x7F7F7F7Fu & ~keep);
      }
      *(BSM_LDS uint32_t*)(lds + 2 * TILE_BYTES + 1024 * q + 256 * w + 4 * lane) = wa_;
      *(BSM_LDS uint32_t*)(lds + 2 * TILE_BYTES + F::SF_BYTES + 1024 * q + 256 * w + 4 * lane) = wb_;
    }
    __syncthreads();
    // 64-K steps of the partial tile: steps past K see zero operands (and unit scales)
    // and add exact zeros. A counted loop keeps the accumulators in place across the
    // optional work.
    const int steps = (tail + 63) / 64;
    for (int s = 0; s < steps; s++) {
      read_frags<FMT>(lds, s, wa, wb, lane, f0);
      read_scales<FMT>(lds, wa, wb, lane, ra, rb);
      const int sh = h8 + 16 * (s & 1);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        sa[t][0] = __builtin_amdgcn_readfirstlane(s >> 1) ? ra[t][1] >> sh : ra[t][0] >> sh;
        sb[t][0] = __builtin_amdgcn_readfirstlane(s >> 1) ? rb[t][1] >> sh : rb[t][0] >> sh;
      }
      mfma_rows<FMT, 0, 0, 4>(f0, sa, sb, acc);
    }
  }
  gemm::store_tile_t(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc);
}

}  // namespace

hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t st) {
  if (a.K == 0) {
    if (a.accum) return hipSuccess;
    return launch_zero_f32_2d(a.D, a.ldd, a.M, a.N, st);
  }
  const int64_t tm64 = (a.M + BM - 1) / BM, tn64 = (a.N + BN - 1) / BN;
  if (tm64 * tn64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = (int)tm64, tiles_n = (int)tn64;
  const dim3 grid(tiles_m * tiles_n);
  if (a.dtype == BSM_E2M1) {
    if (a.accum) hipLaunchKernelGGL((k_gemm_mx<4, true>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);
    else hipLaunchKernelGGL((k_gemm_mx<4, false>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);
  } else {
    if (a.accum) hipLaunchKernelGGL((k_gemm_mx<0, true>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);
    else hipLaunchKernelGGL((k_gemm_mx<0, false>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace bsm
