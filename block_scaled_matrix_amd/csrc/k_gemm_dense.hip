// k_gemm_dense.hip - fp16/bf16 GEMM D = s * A * B^T (+ D) on gfx950 MFMA.
//
// Semantics ("tcgen05.mma": Call parameters, Operand specification, Code generation,
// Example: four K16 issues; "Explicit CUDA tile patterns": Warp MMA): B is the
// (N,K) operand, the product is A times B transposed, float32 accumulation; the
// first K step starts from D when accumulating and from zero otherwise.
//
// gfx950 design:
//  - workgroup tile 256 x 256, K tile 64, four wave64s in a 2 x 2 grid, each owning a
//    128 x 128 sub-tile as 4 x 4 v_mfma_f32_32x32x16 accumulators (256 fp32 per lane,
//    held in AGPRs). The MFMA is issued with the operands swapped (B fragment first), so
//    a lane ends up holding four consecutive output columns per register group and the
//    epilogue moves D in 16-byte pieces;
//  - operand tiles stream HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging) in whole 128-byte lines: an SGPR tile base plus per-lane 32-bit offsets
//    that stay fixed over the whole K loop; two LDS stages of 64 KiB;
//  - each wave reads all four K steps of a tile's fragments into registers early, so a
//    stage is released after the first K step and the copy of tile kt+2 starts while
//    tile kt is still being multiplied: two K tiles stay in flight;
//  - LDS reads and copies are interleaved one by one with the MFMAs, so they issue while
//    the matrix pipe is busy rather than in bursts that stall it;
//  - K-major tiles: 128-byte rows, 16-byte chunk c of row r stored at chunk
//    c ^ ((r >> 1) & 7), so the 16 rows one 16-lane group reads with ds_read_b128
//    cover all 64 LDS banks;
//  - MN-major tiles (the transposed storage): 512-byte k-rows, chunk c of k-row kr
//    stored at c ^ (4 * (kr & 3)); fragments come from ds_read_b64_tr_b16, the LDS
//    transpose read (the analog of ldmatrix .trans in "ldmatrix / stmatrix",
//    Transpose and stores), whose 32-lane groups again cover all banks;
//  - M/N edges clamp the rows that are loaded and mask the stores; a ragged last K
//    tile is loaded through registers with the elements past K zeroed.
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE_BYTES = 256 * BK * 2;  // one operand tile: 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int DMA_PER_TILE = 16;          // copies per wave per K tile (8 A + 8 B)
static_assert(TILE_BYTES == gemm::kKTileBytes, "K-major tile geometry");

// Per-lane byte offsets (relative to the tile's global base) of the 8 direct LDS copies
// a wave issues for one operand tile; copy j of wave w fills LDS bytes
// [1024 (w + 4j), +1024).
//  K-major: the shared 128-byte-row layout (gemm::kmajor_dma_offsets);
//  MN-major: LDS k-row kr = 2(w+4j) + l/32 holds global k-row k0 + kr, its physical
//           chunk l%32 holds logical chunk (l%32) ^ (4 (kr & 3)) (columns clamped to
//           the last 8-aligned chunk).
template <bool KMAJ>
__device__ __forceinline__ void dma_offsets(int64_t ld, int64_t row0, int64_t rows, int w, int lane,
                                            uint32_t (&off)[8]) {
  if (KMAJ) {
    gemm::kmajor_dma_offsets(2 * ld, row0, rows, w, lane, off);
  } else {
    const int kr0 = 2 * w + (lane >> 5);
    const int c = (lane & 31) ^ ((kr0 & 3) << 2);
    const int64_t col = min(row0 + 8 * c, (rows - 1) & ~int64_t(7));
#pragma unroll
    for (int j = 0; j < 8; j++) off[j] = (uint32_t)(((kr0 + 8 * j) * ld + (col - row0)) * 2);
  }
}

// Global base (wave-uniform) of the operand tile whose K range starts at k0.
template <bool KMAJ>
__device__ __forceinline__ const uint16_t* tile_base(const uint16_t* p, int64_t ld, int64_t row0, int64_t k0) {
  return KMAJ ? p + row0 * ld + k0 : p + k0 * ld + row0;
}

// The same tile for a partial K tile: through registers, elements with k >= K zeroed.
template <bool KMAJ>
__device__ __forceinline__ void fill_tile_masked(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                                 int64_t rows, int64_t k0, int64_t K, uint8_t* tile, int w, int lane) {
  if (KMAJ) {
    gemm::kmajor_fill_masked((const uint8_t*)p, 2 * ld, row0, rows, 2 * k0, 2 * K, tile, w, lane);
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int i = w + 4 * j;
    const int kr = 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ ((kr & 3) << 2);
    const int64_t col = min(row0 + 8 * c, (rows - 1) & ~int64_t(7));
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k0 + kr < K) v = *(const uint4*)(p + (k0 + kr) * ld + col);
    lds_write_b128(tile + 1024 * i + 16 * lane, v);
  }
}

template <int DT>
struct Frag;
template <>
struct Frag<BSM_BF16> { typedef bf16x8 T; };
template <>
struct Frag<BSM_F16> { typedef f16x8 T; };

// LDS read addresses of the v_mfma_f32_32x32x16 operand fragments. Lane l must hold
// operand (row wbase + 32t + l%32, k 16ks + 8(l/32) + e), e = 0..7.
//  K-major: one ds_read_b128 at 128 wbase + 4096t + base[ks] (logical chunk 2ks + l/32);
//  MN-major: two ds_read_b64_tr_b16 (h = 0, 1) at 2 wbase + base[t] + 8192ks + 2048h,
//   where within each 16-lane group (i = l%16, G = l/16) lane i provides k-row
//   16ks + 8(G/2) + 4h + i/4 and columns 16(G%2) + 4(i%4)..+3, and receives the
//   transposed 4 x 16 block as column 16(G%2) + i, k-rows +0..3. The 32-column block t
//   enters the swizzled address as an XOR of bits 6..7 (chunk bits 2..3).
template <bool KMAJ>
__device__ __forceinline__ void frag_bases(int lane, uint32_t (&base)[4]) {
  if (KMAJ) {
#pragma unroll
    for (int ks = 0; ks < 4; ks++) base[ks] = gemm::kmajor_frag_base(lane, 2 * ks + (lane >> 5));
  } else {
    const int i = lane & 15, G = lane >> 4;
    const uint32_t L = (uint32_t)((8 * (G >> 1) + (i >> 2)) * 512 + 16 * (2 * (G & 1) + ((i & 3) >> 1)) + 8 * (i & 1) +
                                  64 * ((i >> 2) & 3));
#pragma unroll
    for (int t = 0; t < 4; t++) base[t] = L ^ (uint32_t)(t << 6);
  }
}

template <bool KMAJ>
__device__ __forceinline__ uint4 read_frag(const uint8_t* tile, int wbase, const uint32_t (&base)[4], int ks, int t) {
  if (KMAJ) {
    return lds_read_b128(tile + wbase * 128 + 4096 * t + base[ks]);
  } else {
    const uint8_t* p = tile + 2 * wbase + base[t] + 8192 * ks;
    const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(p));
    const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(p + 2048));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// One 32x32x16 MFMA with the B fragment as the first source: the result block is
// indexed [n][m], so lane l holds output row m = l%32 and, in registers 4q..4q+3,
// columns n = 8q + 4(l/32) + 0..3.
template <int DT>
__device__ __forceinline__ f32x16 mfma(uint4 b, uint4 a, f32x16 c) {
  typedef typename Frag<DT>::T T;
  const T bv = __builtin_bit_cast(T, b), av = __builtin_bit_cast(T, a);
  if constexpr (DT == BSM_BF16) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, av, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, av, c, 0, 0, 0);
}

template <bool AK, bool BKM>
__device__ __forceinline__ void read_step(const uint8_t* ta, const uint8_t* tb, int ks, int wa, int wb,
                                          const uint32_t (&ab)[4], const uint32_t (&bb)[4], uint4 (&af)[4],
                                          uint4 (&bf)[4]) {
#pragma unroll
  for (int t = 0; t < 4; t++) af[t] = read_frag<AK>(ta, wa, ab, ks, t);
#pragma unroll
  for (int t = 0; t < 4; t++) bf[t] = read_frag<BKM>(tb, wb, bb, ks, t);
}

template <int DT>
__device__ __forceinline__ void mfma_step(const uint4 (&af)[4], const uint4 (&bf)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++) acc[mt][nt] = mfma<DT>(bf[nt], af[mt], acc[mt][nt]);
}

__device__ __forceinline__ void pin_step(uint4 (&af)[4], uint4 (&bf)[4]) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    gemm::pin_frag(af[t]);
    gemm::pin_frag(bf[t]);
  }
}


// One K step of 16 MFMAs with side work interleaved: side(i) runs after MFMA i, so that
// LDS reads and copies issue while the matrix pipe is busy instead of in bursts. Empty asm
// "rewrites" of each accumulator before and after its MFMA fix the order of the MFMAs and
// the side operations (all volatile) without any hardware wait.
template <int DT, typename Side>
__device__ __forceinline__ void mfma_step_il(const uint4 (&af)[4], const uint4 (&bf)[4], f32x16 (&acc)[4][4],
                                             Side side) {
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int mt = i >> 2, nt = i & 3;
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    acc[mt][nt] = mfma<DT>(bf[nt], af[mt], acc[mt][nt]);
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    side(i);
  }
}

template <bool AK, bool BKM>
__device__ __forceinline__ void issue_stage(const uint16_t* A, int64_t lda, int64_t m0, const uint16_t* B,
                                            int64_t ldb, int64_t n0, int kt, const uint32_t (&aoff)[8],
                                            const uint32_t (&boff)[8], uint32_t stage, int w) {
  const int64_t k0 = (int64_t)kt * BK;
  gemm::issue_tile8(tile_base<AK>(A, lda, m0, k0), aoff, stage, w);
  gemm::issue_tile8(tile_base<BKM>(B, ldb, n0, k0), boff, stage + TILE_BYTES, w);
}

template <int DT, bool AK, bool BKM, bool ACC>
__global__ __launch_bounds__(256, 1) void k_gemm_dense(GemmArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* B = (const uint16_t*)a.B;
  const int wa = 128 * wm, wb = 128 * wn;
  const float sgn = a.negate ? -1.0f : 1.0f;

  // accumulators start from zero; the epilogue adds D when accumulating
  f32x16 acc[4][4];
  gemm::zero_acc(acc);

  uint32_t aoff[8], boff[8], abase[4], bbase[4];
  dma_offsets<AK>(a.lda, m0, a.M, w, lane, aoff);
  dma_offsets<BKM>(a.ldb, n0, a.N, w, lane, boff);
  frag_bases<AK>(lane, abase);
  frag_bases<BKM>(lane, bbase);

  const int nfull = (int)(a.K / BK);
  const int tail = (int)(a.K % BK);
  const uint32_t lds0 = gemm::lds_addr(lds);
  // fragments of the four K steps of the current tile
  uint4 a0[4], b0[4], a1[4], b1[4], a2[4], b2[4], a3[4], b3[4];
  if (nfull > 0) {
    issue_stage<AK, BKM>(A, a.lda, m0, B, a.ldb, n0, 0, aoff, boff, lds0, w);
    issue_stage<AK, BKM>(A, a.lda, m0, B, a.ldb, n0, min(1, nfull - 1), aoff, boff, lds0 + STAGE_BYTES, w);
    gemm::stage_barrier<DMA_PER_TILE>();
    read_step<AK, BKM>(lds, lds + TILE_BYTES, 0, wa, wb, abase, bbase, a0, b0);
  }
  // K tile kt lives in stage kt & 1. Iteration kt: MFMAs of step 0 with the fragment reads
  // of steps 1..3 spread over its first 12 MFMAs; barrier once every wave's reads of the
  // stage are done; MFMAs of steps 1 and 2 with the 16 copies of tile kt + 2 into the
  // stage, one after every second MFMA (the four waves' copies then keep the shared copy
  // path busy without blocking their issue); barrier once this wave's copies of tile
  // kt + 1 have landed; MFMAs of step 3 with the step-0 fragment reads of tile kt + 1. The body is
  // branch-free: past the last tile the copies re-read the last tile (clamped index) into
  // a stage nobody reads again.
  for (int kt = 0; kt < nfull; kt++) {
    const uint8_t* ta = lds + (kt & 1) * STAGE_BYTES;
    const uint8_t* tb = ta + TILE_BYTES;
    const uint8_t* na = lds + ((kt + 1) & 1) * STAGE_BYTES;
    const uint32_t stage = lds0 + (kt & 1) * STAGE_BYTES;
    const int64_t k2 = (int64_t)min(kt + 2, nfull - 1) * BK;
    const uint16_t* ga = tile_base<AK>(A, a.lda, m0, k2);
    const uint16_t* gb = tile_base<BKM>(B, a.ldb, n0, k2);
    pin_step(a0, b0);
    mfma_step_il<DT>(a0, b0, acc, [&](int i) {
      if (i < 12) {
#pragma unroll
        for (int rr = 0; rr < 2; rr++) {
          const int r = 2 * i + rr;  // read r: step 1 + r / 8, operand (r / 4) & 1, block r & 3
          const int st = 1 + r / 8, op = (r / 4) & 1, t = r & 3;
          uint4& dst = st == 1 ? (op ? b1[t] : a1[t]) : st == 2 ? (op ? b2[t] : a2[t]) : (op ? b3[t] : a3[t]);
          dst = op ? read_frag<BKM>(tb, wb, bbase, st, t) : read_frag<AK>(ta, wa, abase, st, t);
        }
      }
    });
    gemm::lds_barrier();
    pin_step(a1, b1);
    mfma_step_il<DT>(a1, b1, acc, [&](int i) {
      if ((i & 1) == 0) gemm::dma16s(ga, aoff[i >> 1], stage + 1024 * (w + 4 * (i >> 1)));
    });
    pin_step(a2, b2);
    mfma_step_il<DT>(a2, b2, acc, [&](int i) {
      if ((i & 1) == 0) gemm::dma16s(gb, boff[i >> 1], stage + TILE_BYTES + 1024 * (w + 4 * (i >> 1)));
    });
    gemm::stage_barrier<DMA_PER_TILE>();
    pin_step(a3, b3);
    mfma_step_il<DT>(a3, b3, acc, [&](int i) {
      if (i < 4) a0[i] = read_frag<AK>(na, wa, abase, 0, i);
      else if (i < 8) b0[i - 4] = read_frag<BKM>(na + TILE_BYTES, wb, bbase, 0, i - 4);
    });
  }
  // Every copy has landed and every wave is done with LDS before the stage is refilled
  // (and before the workgroup can end with copies in flight).
  gemm::stage_barrier<0>();
  if (tail) {
    const int64_t k0 = (int64_t)nfull * BK;
    fill_tile_masked<AK>(A, a.lda, m0, a.M, k0, a.K, lds, w, lane);
    fill_tile_masked<BKM>(B, a.ldb, n0, a.N, k0, a.K, lds + TILE_BYTES, w, lane);
    __syncthreads();
    for (int ks = 0; ks < (tail + 15) / 16; ks++) {
      read_step<AK, BKM>(lds, lds + TILE_BYTES, ks, wa, wb, abase, bbase, a0, b0);
      mfma_step<DT>(a0, b0, acc);
    }
  }
  // every wave is done with LDS before the accumulators pass through it
  __syncthreads();
  gemm::store_tile_lines(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc, lds + 32768 * w, ACC, a.ew_op,
                         a.ew_scale, a.ew_bias);
}

template <int DT, bool AK, bool BKM>
hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  const int64_t tm64 = (a.M + BM - 1) / BM, tn64 = (a.N + BN - 1) / BN;
  if (tm64 * tn64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = (int)tm64, tiles_n = (int)tn64;
  if (a.accum)
    hipLaunchKernelGGL((k_gemm_dense<DT, AK, BKM, true>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_dense<DT, AK, BKM, false>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs& a, hipStream_t st) {
  if (a.a_kmajor && a.b_kmajor) return launch_one<DT, true, true>(a, st);
  if (a.a_kmajor) return launch_one<DT, true, false>(a, st);
  if (a.b_kmajor) return launch_one<DT, false, true>(a, st);
  return launch_one<DT, false, false>(a, st);
}

// Debug: one operand tile through the GEMM's loader and fragment reads.
template <bool KMAJ>
__global__ __launch_bounds__(256) void k_debug_fragments(const uint16_t* __restrict__ src, uint16_t* dump) {
  __shared__ __attribute__((aligned(1024))) uint8_t tile[TILE_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t off[8], base[4];
  dma_offsets<KMAJ>(KMAJ ? BK : BM, 0, BM, w, lane, off);
  gemm::issue_tile8(src, off, gemm::lds_addr(tile), w);
  gemm::stage_barrier<0>();
  frag_bases<KMAJ>(lane, base);
  for (int mb = 2 * w; mb < 2 * w + 2; mb++) {
    for (int ks = 0; ks < BK / 16; ks++) {
      // rows 32 mb ..: wave base 128 (mb / 4), 32-row block mb % 4
      const uint4 v = read_frag<KMAJ>(tile, 128 * (mb >> 2), base, ks, mb & 3);
      *(uint4*)(dump + ((mb * (BK / 16) + ks) * 64 + lane) * 8) = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t st) {
  // Empty sum: D = f(accum ? D : 0) (the sign of an empty sum is irrelevant).
  if (a.K == 0) return launch_empty_gemm(a.D, a.ldd, a.M, a.N, a.accum, a.ew_op, a.ew_scale, a.ew_bias, st);
  return a.dtype == BSM_BF16 ? launch_dt<BSM_BF16>(a, st) : launch_dt<BSM_F16>(a, st);
}

hipError_t launch_debug_fragments(const uint16_t* src, int kmajor, uint16_t* dump, hipStream_t st) {
  if (kmajor) hipLaunchKernelGGL(k_debug_fragments<true>, dim3(1), dim3(256), 0, st, src, dump);
  else hipLaunchKernelGGL(k_debug_fragments<false>, dim3(1), dim3(256), 0, st, src, dump);
  return hipGetLastError();
}

}  // namespace bsm
