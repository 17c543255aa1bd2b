// k_gemm_dense.hip - fp16/bf16 GEMM D = s * A * B^T (+ D) on gfx950 MFMA.
//
// Semantics ("tcgen05.mma": Call parameters, Operand specification, Code generation,
// Example: four K16 issues; "Explicit CUDA tile patterns": Warp MMA): B is the
// (N,K) operand, the product is A times B transposed, float32 accumulation; the
// first K step starts from D when accumulating and from zero otherwise.
//
// gfx950 design:
//  - workgroup tile 256 x 256, K tile 64, four wave64s in a 2 x 2 grid, each owning a
//    128 x 128 sub-tile as 8 x 8 v_mfma_f32_16x16x32 accumulators (256 fp32 per lane,
//    held in AGPRs). Under sustained load the chip's power limit sets the clock, and the
//    16x16x32 shape moves fewer accumulator bytes per product than 32x32x16 (4 registers
//    read and written per 8192 products instead of 16 per 16384): a pure MFMA loop of it
//    sustains about 7% more than the 32x32x16 loop, and this kernel runs 4-6% faster with
//    it. The MFMA is issued with the operands swapped (B fragment first), so a lane ends up
//    holding four consecutive output columns per block and the epilogue moves D in 16-byte
//    pieces;
//  - operand tiles stream HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging) in whole 128-byte lines: an SGPR tile base plus per-lane 32-bit offsets
//    that stay fixed over the whole K loop; two LDS stages of 64 KiB;
//  - a K tile is two 32-K steps of 64 MFMAs; each wave reads step 1's fragments during
//    step 0, so the stage is released in the middle of step 0 and the copy of tile kt+2
//    starts while tile kt is still being multiplied: two K tiles stay in flight;
//  - LDS reads and copies are interleaved one by one with the MFMAs (a copy every fifth
//    16-cycle MFMA: denser copies held the issuing waves behind the shared copy path), so
//    they issue while the matrix pipe is busy rather than in bursts that stall it;
//  - K-major tiles: 128-byte rows, 16-byte chunk c of row r stored at chunk
//    c ^ ((r >> 1) & 7), so the 16 rows one 16-lane group reads with ds_read_b128
//    cover all 64 LDS banks;
//  - MN-major tiles (the transposed storage): 512-byte k-rows, chunk c of k-row kr
//    stored at c ^ 4(kr & 3) ^ 2((kr >> 3) & 1); fragments come from ds_read_b64_tr_b16,
//    the LDS transpose read (the analog of ldmatrix .trans in "ldmatrix / stmatrix",
//    Transpose and stores): the two 16-lane groups of a half-wave read k-rows 8 apart, and
//    the swizzle puts their eight 32-byte row pieces in distinct banks (checked on the CPU);
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

template <int DT>
struct Frag;
template <>
struct Frag<BSM_BF16> { typedef bf16x8 T; };
template <>
struct Frag<BSM_F16> { typedef f16x8 T; };

constexpr int STEPS = 2;     // 32-K MFMA steps per K tile

// MN-major tiles: 16-byte chunk c of k-row kr stored at c ^ mn_swz(kr).
__device__ __forceinline__ uint32_t mn_swz(int kr) { return (uint32_t)(4 * (kr & 3) ^ 2 * ((kr >> 3) & 1)); }

// LDS read addresses of the v_mfma_f32_16x16x32 operand fragments. Lane l (G = l/16, i = l%16)
// must hold operand (row wbase + 16t + i, k 32s + 8G + e), e = 0..7.
//  K-major: one ds_read_b128 of row wbase + 16t + i, logical chunk 4s + G;
//  MN-major: two ds_read_b64_tr_b16 (h = 0, 1): lane i of group G addresses k-row
//   32s + 8G + 4h + i/4, columns 16t + 4(i%4)..+3, and receives column i, k-rows +0..3.
template <bool KMAJ>
__device__ __forceinline__ uint32_t frag_addr(int lane, int wbase, int s, int t, int h) {
  const int G = lane >> 4, i = lane & 15;
  if (KMAJ) {
    const int r = wbase + 16 * t + i;
    const int c = 4 * s + G;
    return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
  } else {
    const int kr = 32 * s + 8 * G + 4 * h + (i >> 2);
    const int colb = 2 * wbase + 32 * t + 8 * (i & 3);
    const int c = colb >> 4;
    return (uint32_t)(kr * 512 + ((c ^ mn_swz(kr)) << 4) + (colb & 15));
  }
}

template <bool KMAJ>
__device__ __forceinline__ uint4 read_frag(const uint8_t* tile, int lane, int wbase, int s, int t) {
  if (KMAJ) {
    return lds_read_b128(tile + frag_addr<true>(lane, wbase, s, t, 0));
  } else {
    const uint2 lo = __builtin_bit_cast(uint2, lds_read_tr16(tile + frag_addr<false>(lane, wbase, s, t, 0)));
    const uint2 hi = __builtin_bit_cast(uint2, lds_read_tr16(tile + frag_addr<false>(lane, wbase, s, t, 1)));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// One 16x16x32 MFMA with the B fragment as the first source: lane l holds output row
// m = l%16 and, in registers 0..3, columns n = 4(l/16) + 0..3 of the block.
template <int DT>
__device__ __forceinline__ f32x4 mfma(uint4 b, uint4 a, f32x4 c) {
  typedef typename Frag<DT>::T T;
  const T bv = __builtin_bit_cast(T, b), av = __builtin_bit_cast(T, a);
  if constexpr (DT == BSM_BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, av, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_f16(bv, av, c, 0, 0, 0);
}

struct Frags { uint4 a[8], b[8]; };

__device__ __forceinline__ void pin_frags(Frags& f) {
#pragma unroll
  for (int t = 0; t < 8; t++) {
    gemm::pin_frag(f.a[t]);
    gemm::pin_frag(f.b[t]);
  }
}

// Read r (0..15) of a step's fragments, in the order the step's MFMAs (row-block-major) first
// need them: A block 0, B blocks 0..7, A blocks 1..7.
template <bool AK, bool BKM>
__device__ __forceinline__ void read_one(const uint8_t* ta, const uint8_t* tb, int lane, int wa, int wb, int s, int r,
                                         Frags& f) {
  if (r >= 1 && r <= 8) f.b[r - 1] = read_frag<BKM>(tb, lane, wb, s, r - 1);
  else {
    const int t = r == 0 ? 0 : r - 8;
    f.a[t] = read_frag<AK>(ta, lane, wa, s, t);
  }
}

// The 64 MFMAs of one 32-K step, row-block-major; side(i) runs after MFMA i, so that LDS
// reads, copies and barriers issue while the matrix pipe is busy. Empty asm "rewrites" of
// each accumulator before and after its MFMA fix the order of the MFMAs and the side
// operations (all volatile) without any hardware wait.
template <int DT, typename Side>
__device__ __forceinline__ void mfma_step_il(const Frags& f, f32x4 (&acc)[8][8], Side side) {
#pragma unroll
  for (int i = 0; i < 64; i++) {
    const int mt = i >> 3, nt = i & 7;
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    acc[mt][nt] = mfma<DT>(f.b[nt], f.a[mt], acc[mt][nt]);
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    side(i);
  }
}

// Per-lane byte offsets (relative to the tile's global base) of the 8 direct LDS copies
// a wave issues for one operand tile; copy j of wave w fills LDS bytes
// [1024 (w + 4j), +1024).
//  K-major: the shared 128-byte-row layout (gemm::kmajor_dma_offsets);
//  MN-major: LDS k-row kr = 2(w+4j) + l/32 holds global k-row k0 + kr, its physical
//           chunk l%32 holds logical chunk (l%32) ^ mn_swz(kr) (columns clamped to
//           the last 8-aligned chunk).
template <bool KMAJ>
__device__ __forceinline__ void dma_offsets(int64_t ld, int64_t row0, int64_t rows, int w, int lane,
                                            uint32_t (&off)[8]) {
  if (KMAJ) {
    gemm::kmajor_dma_offsets(2 * ld, row0, rows, w, lane, off);
  } else {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int kr = 2 * (w + 4 * j) + (lane >> 5);
      const int c = (lane & 31) ^ (int)mn_swz(kr);
      const int64_t col = min(row0 + 8 * c, (rows - 1) & ~int64_t(7));
      off[j] = (uint32_t)((kr * ld + (col - row0)) * 2);
    }
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
    const int c = (lane & 31) ^ (int)mn_swz(kr);
    const int64_t col = min(row0 + 8 * c, (rows - 1) & ~int64_t(7));
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k0 + kr < K) v = *(const uint4*)(p + (k0 + kr) * ld + col);
    lds_write_b128(tile + 1024 * i + 16 * lane, v);
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

// D = f(s * acc (+ D)) for a 128 x 128 wave sub-tile held as 8 x 8 blocks of 16x16
// accumulators (register e of block (mt, nt) is output row 16mt + l%16, column
// 16nt + 4(l/16) + e), staged through the wave's 32 KiB LDS region in two halves of 64 rows
// (region row r keeps its 16-byte chunk c at c ^ (r & 15)) and stored as whole lines.
__device__ __forceinline__ void store_tile16(float* __restrict__ D, int64_t ldd, int64_t M, int64_t N, int64_t row0,
                                             int64_t col0, int lane, float sgn, const f32x4 (&acc)[8][8],
                                             uint8_t* region, bool add, int ew_op, float es, float eb) {
  const bool whole = row0 + 128 <= M && col0 + 128 <= N;
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int m4 = 0; m4 < 4; m4++) {
      const int r = 16 * m4 + (lane & 15);
#pragma unroll
      for (int nt = 0; nt < 8; nt++) {
        const int c = 4 * nt + (lane >> 4);
        const f32x4& v = acc[4 * half + m4][nt];
        const uint4 x = make_uint4(__float_as_uint(sgn * v[0]), __float_as_uint(sgn * v[1]),
                                   __float_as_uint(sgn * v[2]), __float_as_uint(sgn * v[3]));
        lds_write_b128(region + 512 * r + 16 * (c ^ (r & 15)), x);
      }
    }
    const int c = lane & 31;
    const int64_t col = col0 + 4 * c;
    if (whole) {
      if (ew_op) gemm::store_half_whole<true>(D, ldd, row0 + 64 * half, col, lane, c, region, add, es, eb);
      else gemm::store_half_whole<false>(D, ldd, row0 + 64 * half, col, lane, c, region, add, es, eb);
    } else {
      for (int j = 0; j < 32; j++) {
        const int r = 2 * j + (lane >> 5);
        const uint4 x = lds_read_b128(region + 512 * r + 16 * (c ^ (r & 15)));
        const int64_t row = row0 + 64 * half + r;
        if (row < M) {
          gemm::global_f32* p = (gemm::global_f32*)(D + row * ldd + col);
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

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t aoff[8], boff[8];
  dma_offsets<AK>(a.lda, m0, a.M, w, lane, aoff);
  dma_offsets<BKM>(a.ldb, n0, a.N, w, lane, boff);

  const int nfull = (int)(a.K / BK);
  const int tail = (int)(a.K % BK);
  const uint32_t lds0 = gemm::lds_addr(lds);
  Frags f0, f1;
  if (nfull > 0) {
    issue_stage<AK, BKM>(A, a.lda, m0, B, a.ldb, n0, 0, aoff, boff, lds0, w);
    issue_stage<AK, BKM>(A, a.lda, m0, B, a.ldb, n0, min(1, nfull - 1), aoff, boff, lds0 + STAGE_BYTES, w);
    gemm::stage_barrier<DMA_PER_TILE>();
#pragma unroll
    for (int r = 0; r < 16; r++) read_one<AK, BKM>(lds, lds + TILE_BYTES, lane, wa, wb, 0, r, f0);
  }
  // K tile kt lives in stage kt & 1; f0 holds its step-0 fragments when iteration kt starts.
  for (int kt = 0; kt < nfull; kt++) {
    const uint8_t* ta = lds + (kt & 1) * STAGE_BYTES;
    const uint8_t* tb = ta + TILE_BYTES;
    const uint8_t* na = lds + ((kt + 1) & 1) * STAGE_BYTES;
    const uint32_t stage = lds0 + (kt & 1) * STAGE_BYTES;
    const int64_t k2 = (int64_t)min(kt + 2, nfull - 1) * BK;
    uint64_t ga, gb;
    gemm::sgpr_base2(tile_base<AK>(A, a.lda, m0, k2), tile_base<BKM>(B, a.ldb, n0, k2), ga, gb);
    auto copy = [&](int d) {
      if (d < 8) gemm::dma16u(ga, aoff[d], stage + 1024 * (w + 4 * d));
      else gemm::dma16u(gb, boff[d - 8], stage + TILE_BYTES + 1024 * (w + 4 * (d - 8)));
    };
    // Side work by MFMA slot g (0..63 step 0, 64..127 step 1): step 1's 16 fragment reads at
    // every second slot from 0; barrier once every wave has read the stage; the 16 copies of
    // tile kt + 2, one every fifth slot; barrier once this wave's copies of tile kt + 1 have
    // landed; the next tile's step-0 reads in step 1's last slots.
    constexpr int R1S = 2, CPS = 5;
    constexpr int C0 = 16 * R1S, B2 = C0 + 15 * CPS, G2 = B2 + 1 > 64 ? B2 + 1 : 64, RS2 = (128 - G2) / 16;
    static_assert(RS2 >= 1 && G2 >= 64 && C0 <= 64, "side-work schedule");
    auto side = [&](int g) {
      if (g < C0 && g % R1S == 0) read_one<AK, BKM>(ta, tb, lane, wa, wb, 1, g / R1S, f1);
      if (g == C0 - 1) gemm::lds_barrier();
      if (g >= C0 && g <= B2 && (g - C0) % CPS == 0) copy((g - C0) / CPS);
      if (g == B2) gemm::stage_barrier<DMA_PER_TILE>();
      if (g >= G2 && (g - G2) % RS2 == 0 && (g - G2) / RS2 < 16)
        read_one<AK, BKM>(na, na + TILE_BYTES, lane, wa, wb, 0, (g - G2) / RS2, f0);
    };
    pin_frags(f0);
    mfma_step_il<DT>(f0, acc, [&](int i) { side(i); });
    pin_frags(f1);
    mfma_step_il<DT>(f1, acc, [&](int i) { side(64 + i); });
  }
  // Every copy has landed and every wave is done with LDS before the stage is refilled
  // (and before the workgroup can end with copies in flight).
  gemm::stage_barrier<0>();
  if (tail) {
    const int64_t k0 = (int64_t)nfull * BK;
    fill_tile_masked<AK>(A, a.lda, m0, a.M, k0, a.K, lds, w, lane);
    fill_tile_masked<BKM>(B, a.ldb, n0, a.N, k0, a.K, lds + TILE_BYTES, w, lane);
    __syncthreads();
    for (int s = 0; s < (tail + 31) / 32; s++) {
#pragma unroll
      for (int r = 0; r < 16; r++) read_one<AK, BKM>(lds, lds + TILE_BYTES, lane, wa, wb, s, r, f0);
      mfma_step_il<DT>(f0, acc, [](int) {});
    }
  }
  __syncthreads();
  store_tile16(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc, lds + 32768 * w, ACC, a.ew_op, a.ew_scale,
               a.ew_bias);
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

// Debug: one operand tile through the GEMM's loader and fragment reads. The dump holds, for
// 16-row block b (0..15) and 32-K step s (0..1), each lane's 8 elements: dump[((b * 2 + s) * 64
// + lane) * 8 + e] = operand (16b + lane % 16, 32s + 8 (lane / 16) + e).
template <bool KMAJ>
__global__ __launch_bounds__(256) void k_debug_fragments(const uint16_t* __restrict__ src, uint16_t* dump) {
  __shared__ __attribute__((aligned(1024))) uint8_t tile[TILE_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t off[8];
  dma_offsets<KMAJ>(KMAJ ? BK : BM, 0, BM, w, lane, off);
  gemm::issue_tile8(src, off, gemm::lds_addr(tile), w);
  gemm::stage_barrier<0>();
  for (int b = 4 * w; b < 4 * w + 4; b++) {
    for (int s = 0; s < STEPS; s++) {
      // rows 16b ..: wave base 128 (b / 8), 16-row block b % 8
      const uint4 v = read_frag<KMAJ>(tile, lane, 128 * (b >> 3), s, b & 7);
      *(uint4*)(dump + ((b * STEPS + s) * 64 + lane) * 8) = v;
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
