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
//  - workgroup tile 256 x 256 x (64 bytes of K per row), four wave64s with 128 x 128
//    sub-tiles (4 x 4 accumulators of 16 fp32 in AGPRs); operand tiles and the scale
//    word of each row stream HBM -> LDS with global_load_lds_dwordx4 / _dword into four
//    stages (64-byte-row XOR swizzle shared with the dense kernel), three K tiles ahead
//    of the one consumed; one barrier per K tile waits only for the next tile;
//  - fp4 (two 64-K steps per tile): the MFMAs of one step overlap the LDS reads of the
//    other; fp8 (one step per tile): the barrier sits after the first 8 MFMAs of a tile
//    and the next tile's fragments are read while the last 8 run (two register sets).
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int ROWB = 64;                                    // bytes of K per row per K tile
constexpr int TILE_BYTES = 256 * ROWB;                      // 16 KiB per operand tile
constexpr int SF_BYTES = 256 * 4;                           // one scale word per row
constexpr int STAGE_BYTES = 2 * TILE_BYTES + 2 * SF_BYTES;  // A, B, SFA, SFB
constexpr int NST = 4;                                      // LDS stages
constexpr int PF = NST - 1;                                 // K tiles in flight ahead
constexpr int DMA_PER_TILE = 10;                            // per wave: 4 A + 4 B + 1 + 1 scale
static_assert(TILE_BYTES == gemm::kKTileBytes, "K-major tile geometry");

template <int FMT>
struct Fmt {
  static constexpr int KT = FMT == 4 ? 128 : 64;  // K elements per K tile
  static constexpr int STEPS = FMT == 4 ? 2 : 1;  // 64-K MFMA steps per K tile
  static constexpr int EPB = FMT == 4 ? 2 : 1;    // elements per byte
  static constexpr int BPT = KT / 32;             // scale blocks per K tile
};

// Byte offset inside a scale row of the aligned 32-bit word holding the first block of
// K tile kt (fp4: the tile's 4 blocks; fp8: a pair of tiles, this one at byte 2 (kt&1)).
template <int FMT>
__device__ __forceinline__ int64_t sf_word(int kt) {
  return FMT == 4 ? 4 * (int64_t)kt : 4 * (int64_t)(kt >> 1);
}

struct Ops {
  const uint8_t* A; int64_t lda_b; uint32_t aoff[4];
  const uint8_t* B; int64_t ldb_b; uint32_t boff[4];
  const uint8_t* SFA; int64_t ld_sfa; uint32_t sfa_off;
  const uint8_t* SFB; int64_t ld_sfb; uint32_t sfb_off;
};

// Copies of K tile kt (operand rows from the tile's first row, scale rows 64w + l).
template <int FMT>
__device__ __forceinline__ void issue_stage(const Ops& o, int kt, uint32_t stage, int w) {
  const int64_t kb = (int64_t)kt * ROWB;
  gemm::issue_tile4(o.A + kb, o.aoff, stage, w);
  gemm::issue_tile4(o.B + kb, o.boff, stage + TILE_BYTES, w);
  gemm::dma4s(o.SFA + sf_word<FMT>(kt), o.sfa_off, stage + 2 * TILE_BYTES + 256 * w);
  gemm::dma4s(o.SFB + sf_word<FMT>(kt), o.sfb_off, stage + 2 * TILE_BYTES + SF_BYTES + 256 * w);
}

// Fragments (and raw scale words) of one K tile for one wave: af/bf[t][0..1] are the
// 16-byte chunks of 32-row block t, sa/sb[t] the scale word of the lane's row.
template <int FMT>
struct Set {
  uint4 af[4][2], bf[4][2];
  uint32_t sa[4], sb[4];
};

// LDS offsets of the fragment chunks: logical chunk 2q + l/32 of the lane's row. fp8
// uses q = 0, 1 (k 16(l/32).. and 32 + 16(l/32)..) of its single step; fp4 uses q = s.
__device__ __forceinline__ void frag_bases(int lane, uint32_t (&base)[2]) {
#pragma unroll
  for (int q = 0; q < 2; q++) base[q] = gemm::kmajor_frag_base(lane, 2 * q + (lane >> 5));
}

// Reads the fragments of 64-K step s of the stage at `st` (fp8: s = 0) for this wave.
template <int FMT>
__device__ __forceinline__ void read_frags(const uint8_t* st, int s, int wa, int wb, const uint32_t (&base)[2],
                                           uint4 (&af)[4][2], uint4 (&bf)[4][2]) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint8_t* pa = st + wa * 64 + 2048 * t;
    const uint8_t* pb = st + TILE_BYTES + wb * 64 + 2048 * t;
    if (FMT == 4) {
      const uint32_t bs = s ? base[1] : base[0];
      af[t][0] = lds_read_b128(pa + bs);
      bf[t][0] = lds_read_b128(pb + bs);
    } else {
      af[t][0] = lds_read_b128(pa + base[0]);
      af[t][1] = lds_read_b128(pa + base[1]);
      bf[t][0] = lds_read_b128(pb + base[0]);
      bf[t][1] = lds_read_b128(pb + base[1]);
    }
  }
}

__device__ __forceinline__ void read_scales(const uint8_t* st, int wa, int wb, int lane, uint32_t (&sa)[4],
                                            uint32_t (&sb)[4]) {
  const uint8_t* pa = st + 2 * TILE_BYTES;
  const uint8_t* pb = pa + SF_BYTES;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    sa[t] = *(const BSM_LDS uint32_t*)(pa + 4 * (wa + 32 * t + (lane & 31)));
    sb[t] = *(const BSM_LDS uint32_t*)(pb + 4 * (wb + 32 * t + (lane & 31)));
  }
}

// Right-shift so that byte 0 (and byte 2 for fp4's second step) holds the block this
// lane feeds: lanes 32..63 carry the second 32-K block of each 64-K step.
__device__ __forceinline__ void shift_scales(uint32_t (&sa)[4], uint32_t (&sb)[4], int sh) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    sa[t] >>= sh;
    sb[t] >>= sh;
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
__device__ __forceinline__ void pin_set(uint4 (&af)[4][2], uint4 (&bf)[4][2], uint32_t (&sa)[4], uint32_t (&sb)[4]) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    if (t >= MT0 && t < MT1) {
      gemm::pin_frag(af[t][0]);
      if (FMT != 4) gemm::pin_frag(af[t][1]);
      gemm::pin_word(sa[t]);
    }
    gemm::pin_frag(bf[t][0]);
    if (FMT != 4) gemm::pin_frag(bf[t][1]);
    gemm::pin_word(sb[t]);
  }
}

// MFMAs of accumulator rows mt in [MT0, MT1) for one 64-K step.
template <int FMT, int SEL, int MT0, int MT1>
__device__ __forceinline__ void mfma_rows(const uint4 (&af)[4][2], const uint4 (&bf)[4][2], const uint32_t (&sa)[4],
                                          const uint32_t (&sb)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = MT0; mt < MT1; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++) acc[mt][nt] = mfma_sc<FMT, SEL>(bf[nt], af[mt], acc[mt][nt], sb[nt], sa[mt]);
}

// One fp8 K tile kt from register set X (fragments + shifted scales of tile kt) while
// set Y receives tile kt + 1.
__device__ __forceinline__ void fp8_tile(const Ops& o, int kt, int nfull, const uint8_t* lds, uint32_t lds0, int w,
                                         int lane, int wa, int wb, const uint32_t (&base)[2], Set<0>& X, Set<0>& Y,
                                         f32x16 (&acc)[4][4]) {
  issue_stage<0>(o, min(kt + PF, nfull - 1), lds0 + ((kt + PF) % NST) * STAGE_BYTES, w);
  pin_set<0, 0, 2>(X.af, X.bf, X.sa, X.sb);
  __builtin_amdgcn_sched_barrier(0);
  mfma_rows<0, 0, 0, 2>(X.af, X.bf, X.sa, X.sb, acc);
  gemm::pin_acc(acc);
  __builtin_amdgcn_sched_barrier(0);
  gemm::stage_barrier<(PF - 1) * DMA_PER_TILE>();
  const uint8_t* nst = lds + ((kt + 1) % NST) * STAGE_BYTES;
  read_frags<0>(nst, 0, wa, wb, base, Y.af, Y.bf);
  read_scales(nst, wa, wb, lane, Y.sa, Y.sb);
  pin_set<0, 2, 4>(X.af, X.bf, X.sa, X.sb);
  __builtin_amdgcn_sched_barrier(0);
  mfma_rows<0, 0, 2, 4>(X.af, X.bf, X.sa, X.sb, acc);
  gemm::pin_acc(acc);
  __builtin_amdgcn_sched_barrier(0);
  shift_scales(Y.sa, Y.sb, 8 * (lane >> 5) + 16 * ((kt + 1) & 1));
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_gemm_mx(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Fmt<FMT> F;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nblk = a.K / 32;
  const int wa = 128 * wm, wb = 128 * wn;

  f32x16 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][nt][r] = 0.0f;

  Ops o;
  o.lda_b = a.lda / F::EPB;
  o.ldb_b = a.ldb / F::EPB;
  o.A = (const uint8_t*)a.A + m0 * o.lda_b;
  o.B = (const uint8_t*)a.B + n0 * o.ldb_b;
  o.SFA = a.SFA + m0 * a.ld_sfa;
  o.SFB = a.SFB + n0 * a.ld_sfb;
  o.ld_sfa = a.ld_sfa;
  o.ld_sfb = a.ld_sfb;
  gemm::kmajor_dma_offsets(o.lda_b, m0, a.M, w, lane, o.aoff);
  gemm::kmajor_dma_offsets(o.ldb_b, n0, a.N, w, lane, o.boff);
  // scale row 64w + l of the tile (clamped to the last row), relative to the first row
  o.sfa_off = (uint32_t)((min(m0 + 64 * w + lane, a.M - 1) - m0) * a.ld_sfa);
  o.sfb_off = (uint32_t)((min(n0 + 64 * w + lane, a.N - 1) - n0) * a.ld_sfb);
  uint32_t base[2];
  frag_bases(lane, base);

  const int nfull = (int)(a.K / F::KT);
  const int tail = (int)(a.K % F::KT);
  const uint32_t lds0 = gemm::lds_addr(lds);
  const int h8 = 8 * (lane >> 5);
  Set<FMT> X, Y;
  if (nfull > 0) {
#pragma unroll
    for (int p = 0; p < PF; p++) issue_stage<FMT>(o, min(p, nfull - 1), lds0 + p * STAGE_BYTES, w);
    gemm::stage_barrier<(PF - 1) * DMA_PER_TILE>();
    read_frags<FMT>(lds, 0, wa, wb, base, X.af, X.bf);
    read_scales(lds, wa, wb, lane, X.sa, X.sb);
    shift_scales(X.sa, X.sb, h8);
  }
  if constexpr (FMT == 4) {
    // Iteration kt: read step 1 of tile kt, start the copy of tile kt + PF into the
    // stage tile kt - 1 used, MFMAs of step 0, barrier (tile kt + 1 landed), read step 0
    // and the scales of tile kt + 1, MFMAs of step 1, then shift the new scales.
    // Branch-free: past the last tile the copies re-read it into unused stages.
    for (int kt = 0; kt < nfull; kt++) {
      const uint8_t* st = lds + (kt % NST) * STAGE_BYTES;
      const uint8_t* nst = lds + ((kt + 1) % NST) * STAGE_BYTES;
      read_frags<4>(st, 1, wa, wb, base, Y.af, Y.bf);
      issue_stage<4>(o, min(kt + PF, nfull - 1), lds0 + ((kt + PF) % NST) * STAGE_BYTES, w);
      pin_set<4, 0, 4>(X.af, X.bf, X.sa, X.sb);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<4, 0, 0, 4>(X.af, X.bf, X.sa, X.sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
      gemm::stage_barrier<(PF - 1) * DMA_PER_TILE>();
      read_frags<4>(nst, 0, wa, wb, base, X.af, X.bf);
      read_scales(nst, wa, wb, lane, Y.sa, Y.sb);
      pin_set<4, 0, 4>(Y.af, Y.bf, X.sa, X.sb);
      __builtin_amdgcn_sched_barrier(0);
      mfma_rows<4, 2, 0, 4>(Y.af, Y.bf, X.sa, X.sb, acc);
      gemm::pin_acc(acc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        X.sa[t] = Y.sa[t] >> h8;
        X.sb[t] = Y.sb[t] >> h8;
      }
    }
  } else {
    // Two register sets alternate between consecutive K tiles.
    int kt = 0;
    for (; kt + 2 <= nfull; kt += 2) {
      fp8_tile(o, kt, nfull, lds, lds0, w, lane, wa, wb, base, X, Y, acc);
      fp8_tile(o, kt + 1, nfull, lds, lds0, w, lane, wa, wb, base, Y, X, acc);
    }
    if (kt < nfull) {
      fp8_tile(o, kt, nfull, lds, lds0, w, lane, wa, wb, base, X, Y, acc);
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
    {
      // scale words of the partial tile; blocks at or past nblk (beyond K) become 127
      // (2^0): their operand bytes are zero, and a NaN code in the row padding must not
      // poison them
      const int64_t word = sf_word<FMT>(nfull);
      const int64_t valid = nblk - word;  // >= 1: the partial tile's first block exists
      const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : (1u << (8 * valid)) - 1u;
      const uint32_t ra = *(const uint32_t*)(o.SFA + o.sfa_off + word);
      const uint32_t rb = *(const uint32_t*)(o.SFB + o.sfb_off + word);
      *(BSM_LDS uint32_t*)(lds + 2 * TILE_BYTES + 256 * w + 4 * lane) = (ra & keep) | (0x7F7F7F7Fu & ~keep);
      *(BSM_LDS uint32_t*)(lds + 2 * TILE_BYTES + SF_BYTES + 256 * w + 4 * lane) = (rb & keep) | (0x7F7F7F7Fu & ~keep);
    }
    __syncthreads();
    // 64-K steps of the partial tile (fp4: one or two); the second one takes its scale
    // bytes from a 16-bit further shift, so every step uses op_sel 0. A counted loop keeps
    // the accumulators in place across the optional work.
    const int steps = (tail + 63) / 64;
    for (int s = 0; s < steps; s++) {
      read_scales(lds, wa, wb, lane, X.sa, X.sb);
      shift_scales(X.sa, X.sb, FMT == 4 ? h8 + 16 * s : h8 + 16 * (nfull & 1));
      read_frags<FMT>(lds, s, wa, wb, base, X.af, X.bf);
      mfma_rows<FMT, 0, 0, 4>(X.af, X.bf, X.sa, X.sb, acc);
    }
  }
  gemm::store_tile_t(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, a.negate ? -1.0f : 1.0f, a.accum, acc);
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
  if (a.dtype == BSM_E2M1)
    hipLaunchKernelGGL(k_gemm_mx<4>, dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(k_gemm_mx<0>, dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bsm
