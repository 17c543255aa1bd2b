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
//  - workgroup tile 256 x 256 x (128 bytes of K per row), four wave64s with 128 x 128
//    sub-tiles (4 x 4 accumulators of 16 fp32 in AGPRs); operand tiles HBM -> LDS with
//    global_load_lds_dwordx4 into two stages (same 128-byte-row XOR swizzle as the
//    dense kernel); scales go straight to registers one K tile ahead as dword loads;
//  - the MFMAs of one 64-K step overlap the LDS reads of the next step and the DMA of
//    the next K tile; the stage barrier sits before the MFMAs of the last step.
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int ROWB = 128;                  // bytes of K per row per K tile
constexpr int TILE_BYTES = 256 * ROWB;     // 32 KiB per operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;

template <int FMT>
struct Fmt {
  static constexpr int KT = FMT == 4 ? 256 : 128;  // K elements per K tile
  static constexpr int STEPS = FMT == 4 ? 4 : 2;    // 64-K MFMA steps per K tile
  static constexpr int SFW = FMT == 4 ? 2 : 1;      // scale dwords per row per K tile
  static constexpr int EPB = FMT == 4 ? 2 : 1;      // elements per byte
};

// Per-lane byte offsets of the 8 direct LDS copies of one operand tile (relative to the
// tile's global base): LDS row r = 8(w+4j) + l/8 holds global row row0 + r (clamped),
// physical chunk l%8 holds logical chunk (l%8) ^ ((r >> 1) & 7).
__device__ __forceinline__ void dma_offsets(int64_t ldb, int64_t row0, int64_t rows, int w, int lane,
                                            uint32_t (&off)[8]) {
  const int c = (lane & 7) ^ (((8 * w + (lane >> 3)) >> 1) & 7);
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int64_t rg = min(row0 + 8 * w + 32 * j + (lane >> 3), rows - 1);
    off[j] = (uint32_t)((rg - row0) * ldb + 16 * c);
  }
}

__device__ __forceinline__ void issue_tile(const uint8_t* base, const uint32_t (&off)[8], uint32_t lds_tile, int w) {
#pragma unroll
  for (int j = 0; j < 8; j++) gemm::dma16s(base, off[j], lds_tile + 1024 * (w + 4 * j));
}

// Partial last K tile: chunks at or past kb_end (bytes) are zero.
__device__ __forceinline__ void fill_tile_masked(const uint8_t* __restrict__ p, int64_t ldb, int64_t row0,
                                                 int64_t rows, int64_t kb0, int64_t kb_end, uint8_t* tile, int w,
                                                 int lane) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int i = w + 4 * j;
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t rg = min(row0 + r, rows - 1);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kb0 + 16 * c < kb_end) v = *(const uint4*)(p + rg * ldb + kb0 + 16 * c);
    lds_write_b128(tile + 1024 * i + 16 * lane, v);
  }
}

// LDS address bases of the operand fragments (row wbase + 32t + l%32): the 16-byte
// chunk of the fragment of step s sits at 128 wbase + 4096t + base[.].
//  fp8: chunks 4s + l/32 (k 16(l/32)..) and 4s + 2 + l/32 (k 32 + 16(l/32)..) -> base[2s + h];
//  fp4: chunk 2s + l/32 -> base[s].
template <int FMT>
__device__ __forceinline__ void frag_bases(int lane, uint32_t (&base)[4]) {
  const int r = lane & 31, sw = (r >> 1) & 7, hi = lane >> 5;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int chunk = FMT == 4 ? 2 * q + hi : 4 * (q >> 1) + 2 * (q & 1) + hi;
    base[q] = (uint32_t)(r * 128 + ((chunk ^ sw) << 4));
  }
}

template <int FMT>
__device__ __forceinline__ void read_frag(const uint8_t* tile, int wbase, const uint32_t (&base)[4], int s, int t,
                                          uint4 (&f)[2]) {
  const uint8_t* p = tile + wbase * 128 + 4096 * t;
  if (FMT == 4) {
    f[0] = lds_read_b128(p + base[s]);
  } else {
    f[0] = lds_read_b128(p + base[2 * s]);
    f[1] = lds_read_b128(p + base[2 * s + 1]);
  }
}

template <int FMT>
__device__ __forceinline__ void read_step(const uint8_t* ta, const uint8_t* tb, int s, int wa, int wb,
                                          const uint32_t (&ab)[4], const uint32_t (&bb)[4], uint4 (&af)[4][2],
                                          uint4 (&bf)[4][2]) {
#pragma unroll
  for (int t = 0; t < 4; t++) read_frag<FMT>(ta, wa, ab, s, t, af[t]);
#pragma unroll
  for (int t = 0; t < 4; t++) read_frag<FMT>(tb, wb, bb, s, t, bf[t]);
}

template <int FMT, int SEL>
__device__ __forceinline__ f32x16 mfma_sc(const uint4 (&a)[2], const uint4 (&b)[2], f32x16 c, uint32_t sa,
                                          uint32_t sb) {
  i32x8 av, bv;
  av[0] = a[0].x; av[1] = a[0].y; av[2] = a[0].z; av[3] = a[0].w;
  bv[0] = b[0].x; bv[1] = b[0].y; bv[2] = b[0].z; bv[3] = b[0].w;
  if (FMT == 4) {
    av[4] = av[5] = av[6] = av[7] = 0;
    bv[4] = bv[5] = bv[6] = bv[7] = 0;
  } else {
    av[4] = a[1].x; av[5] = a[1].y; av[6] = a[1].z; av[7] = a[1].w;
    bv[4] = b[1].x; bv[5] = b[1].y; bv[6] = b[1].z; bv[7] = b[1].w;
  }
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, FMT, FMT, SEL, (int)sa, SEL, (int)sb);
}

// 16 MFMAs of 64-K step s. Scale word s/2 of each row block holds, after the per-lane
// shift, the block of step 2q in byte 0 and of step 2q+1 in byte 2 (op_sel 0 / 2).
template <int FMT>
__device__ __forceinline__ void mfma_step(const uint4 (&af)[4][2], const uint4 (&bf)[4][2], int s,
                                          const uint32_t (&sa)[4][2], const uint32_t (&sb)[4][2],
                                          f32x16 (&acc)[4][4]) {
  const int q = s >> 1;
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      if (s & 1) acc[mt][nt] = mfma_sc<FMT, 2>(af[mt], bf[nt], acc[mt][nt], sa[mt][q], sb[nt][q]);
      else acc[mt][nt] = mfma_sc<FMT, 0>(af[mt], bf[nt], acc[mt][nt], sa[mt][q], sb[nt][q]);
    }
}

// Scale words of one K tile for this lane's 4 row blocks: word q holds the scales of
// blocks blk0 + 4q .. +3 of each row (rows start 4-byte aligned). A word that would lie
// wholly past the last block (nblk) is not read: its slot re-reads word 0 and
// prep_scales replaces its bytes. Loaded one K tile ahead and only consumed after the
// next stage barrier (prep_scales), so the loads never stall.
template <int FMT>
__device__ __forceinline__ void load_scales(const uint8_t* __restrict__ sf_rows, const uint32_t (&roff)[4],
                                            int64_t blk0, int64_t nblk, uint32_t (&raw)[4][2]) {
#pragma unroll
  for (int q = 0; q < Fmt<FMT>::SFW; q++) {
    const int64_t blk = blk0 + 4 * q < nblk ? blk0 + 4 * q : blk0;
#pragma unroll
    for (int t = 0; t < 4; t++) raw[t][q] = *(const uint32_t*)(sf_rows + roff[t] + blk);
  }
}

// Shift right by 8 * (l/32) so that bytes 0 and 2 are the blocks this lane feeds to
// steps 2q and 2q+1. Blocks at or past nblk (beyond K) read as 127 (2^0): the matching
// operand bytes are zero, and a NaN scale code in the row padding must not poison them.
template <int FMT>
__device__ __forceinline__ void prep_scales(const uint32_t (&raw)[4][2], int64_t blk0, int64_t nblk, int lane,
                                            uint32_t (&out)[4][2]) {
  const int sh = 8 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < Fmt<FMT>::SFW; q++) {
    const int64_t valid = nblk - blk0 - 4 * q;
    const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : (1u << (8 * valid)) - 1u);
#pragma unroll
    for (int t = 0; t < 4; t++) out[t][q] = ((raw[t][q] & keep) | (0x7F7F7F7Fu & ~keep)) >> sh;
  }
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_gemm_mx(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Fmt<FMT> F;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const uint8_t* A = (const uint8_t*)a.A;
  const uint8_t* B = (const uint8_t*)a.B;
  const int64_t lda_b = a.lda / F::EPB, ldb_b = a.ldb / F::EPB;
  const int64_t nblk = a.K / 32;
  const int wa = 128 * wm, wb = 128 * wn;

  f32x16 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][nt][r] = 0.0f;

  uint32_t aoff[8], boff[8], abase[4], bbase[4], sfa_off[4], sfb_off[4];
  dma_offsets(lda_b, m0, a.M, w, lane, aoff);
  dma_offsets(ldb_b, n0, a.N, w, lane, boff);
  frag_bases<FMT>(lane, abase);
  frag_bases<FMT>(lane, bbase);
  // scale rows of this lane: wave base + 32t + l%32, clamped to the last row, as byte
  // offsets from the tile's first row (never negative: the tile's first row exists)
  const uint8_t* sfa0 = a.SFA + m0 * a.ld_sfa;
  const uint8_t* sfb0 = a.SFB + n0 * a.ld_sfb;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    sfa_off[t] = (uint32_t)((min(m0 + wa + 32 * t + (lane & 31), a.M - 1) - m0) * a.ld_sfa);
    sfb_off[t] = (uint32_t)((min(n0 + wb + 32 * t + (lane & 31), a.N - 1) - n0) * a.ld_sfb);
  }
  const int bpt = F::KT / 32;  // scale blocks per K tile

  const int nfull = (int)(a.K / F::KT);
  const int tail = (int)(a.K % F::KT);
  const uint32_t lds0 = gemm::lds_addr(lds);
  uint4 af[2][4][2], bf[2][4][2];
  uint32_t sa[4][2], sb[4][2], na[4][2], nb[4][2];
  load_scales<FMT>(sfa0, sfa_off, 0, nblk, na);
  load_scales<FMT>(sfb0, sfb_off, 0, nblk, nb);
  prep_scales<FMT>(na, 0, nblk, lane, sa);
  prep_scales<FMT>(nb, 0, nblk, lane, sb);
  if (nfull > 0) {
    issue_tile(A + m0 * lda_b, aoff, lds0, w);
    issue_tile(B + n0 * ldb_b, boff, lds0 + TILE_BYTES, w);
    gemm::wait_dma();
    __syncthreads();
    read_step<FMT>(lds, lds + TILE_BYTES, 0, wa, wb, abase, bbase, af[0], bf[0]);
  }
  // The loop body is branch-free so that the scheduling fences hold: on the last K tile
  // the prefetch re-reads the last tile (clamped index) into the stage nobody reads again.
  for (int kt = 0; kt < nfull; kt++) {
    const int cur = kt & 1;
    const uint8_t* ta = lds + cur * STAGE_BYTES;
    const uint8_t* tb = ta + TILE_BYTES;
    const uint8_t* nta = lds + (cur ^ 1) * STAGE_BYTES;
    const int kn = min(kt + 1, nfull - 1);
    read_step<FMT>(ta, tb, 1, wa, wb, abase, bbase, af[1], bf[1]);
    {
      const uint32_t nxt = lds0 + (cur ^ 1) * STAGE_BYTES;
      const int64_t kb1 = (int64_t)kn * ROWB;
      issue_tile(A + m0 * lda_b + kb1, aoff, nxt, w);
      issue_tile(B + n0 * ldb_b + kb1, boff, nxt + TILE_BYTES, w);
    }
    // scales of K tile kt+1 (it exists when kt+1 < nfull or a partial tile follows)
    const int64_t blk1 = (kt + 1 < nfull || tail) ? (int64_t)(kt + 1) * bpt : (int64_t)kt * bpt;
    load_scales<FMT>(sfa0, sfa_off, blk1, nblk, na);
    load_scales<FMT>(sfb0, sfb_off, blk1, nblk, nb);
#pragma unroll
    for (int s = 0; s < F::STEPS; s++) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_step<FMT>(af[s & 1], bf[s & 1], s, sa, sb, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 2 < F::STEPS) {
        read_step<FMT>(ta, tb, s + 2, wa, wb, abase, bbase, af[s & 1], bf[s & 1]);
      } else if (s + 2 == F::STEPS) {
        gemm::wait_dma();
        __syncthreads();
        read_step<FMT>(nta, nta + TILE_BYTES, 0, wa, wb, abase, bbase, af[s & 1], bf[s & 1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    prep_scales<FMT>(na, blk1, nblk, lane, sa);
    prep_scales<FMT>(nb, blk1, nblk, lane, sb);
  }
  if (tail) {
    uint8_t* st = lds + (nfull & 1) * STAGE_BYTES;
    const int64_t kb0 = (int64_t)nfull * ROWB;
    const int64_t kb_end = a.K / F::EPB;
    fill_tile_masked(A, lda_b, m0, a.M, kb0, kb_end, st, w, lane);
    fill_tile_masked(B, ldb_b, n0, a.N, kb0, kb_end, st + TILE_BYTES, w, lane);
    __syncthreads();
    const int steps = (tail + 63) / 64;
#pragma unroll
    for (int s = 0; s < F::STEPS; s++) {
      if (s < steps) {
        read_step<FMT>(st, st + TILE_BYTES, s, wa, wb, abase, bbase, af[0], bf[0]);
        mfma_step<FMT>(af[0], bf[0], s, sa, sb, acc);
      }
    }
  }
  gemm::store_tile(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, a.negate ? -1.0f : 1.0f, a.accum, acc);
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
