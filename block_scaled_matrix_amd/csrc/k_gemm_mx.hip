// k_gemm_mx.hip - block-scaled GEMM (MXFP8 E4M3 / MXFP4 E2M1 with E8M0 scales per 32
// K elements) D = s * A * B^T (+ D) on gfx950 v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Semantics ("tcgen05.mma": Weight-stationary and block scaling, Call parameters;
// "Explicit CUDA tile patterns": tcgen05 MMA): operand value = element * 2^(scale-127)
// with one scale per 32 consecutive K elements of a row, float32 accumulation.
//
// gfx950 design (probed on the device):
//  - the scaled MFMA takes per lane one 32-bit register of scales and selects a byte
//    with op_sel; for K = 64 per instruction the scale of row i, block b (32 K) is
//    taken from lane i + 32*b;
//  - fp8 operand (32 bytes per lane): lane l holds row l%32 with k in
//    [16(l/32), +16) and [32 + 16(l/32), +16) of the 64-K step;
//  - fp4 operand (16 bytes per lane, two elements per byte, low nibble first): lane l
//    holds row l%32 with k in [32(l/32), +32);
//  - workgroup tile 256 x 256 x (128 bytes of K per row), four wave64s with 128 x 128
//    sub-tiles (4 x 4 accumulators of 16 fp32), operand tiles HBM -> LDS with
//    global_load_lds_dwordx4 into two stages, the same 128-byte-row swizzle as the
//    dense kernel; scales go to registers one K tile ahead.
#include "bsm_device.hpp"
#include "bsm_internal.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int ROWB = 128;                  // bytes of K per row per K tile
constexpr int TILE_BYTES = 256 * ROWB;     // 32 KiB per operand tile

__device__ __forceinline__ uint32_t kmaj_off(int r, int c) { return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4)); }

template <int FMT>
struct Fmt {
  static constexpr int KT = FMT == 4 ? 256 : 128;  // K elements per K tile
  static constexpr int STEPS = FMT == 4 ? 4 : 2;    // 64-K MFMA steps per K tile
  static constexpr int SFW = FMT == 4 ? 2 : 1;      // scale dwords per row per K tile
  static constexpr int EPB = FMT == 4 ? 2 : 1;      // elements per byte
};

// HBM -> LDS, one 256-row x 128-byte operand tile; rows past `rows` clamped.
__device__ __forceinline__ void issue_tile(const uint8_t* __restrict__ p, int64_t ldb_bytes, int64_t row0,
                                           int64_t rows, int64_t kb0, uint8_t* tile, int w, int lane) {
  const int c = (lane & 7) ^ (((8 * w + (lane >> 3)) >> 1) & 7);
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int i = w + 4 * j;
    const int64_t rg = min(row0 + 8 * i + (lane >> 3), rows - 1);
    load_lds_16(p + rg * ldb_bytes + kb0 + 16 * c, tile + 1024 * i);
  }
}

// Partial last K tile: chunks at or past kb_end (bytes) are zero.
__device__ __forceinline__ void fill_tile_masked(const uint8_t* __restrict__ p, int64_t ldb_bytes, int64_t row0,
                                                 int64_t rows, int64_t kb0, int64_t kb_end, uint8_t* tile, int w,
                                                 int lane) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int i = w + 4 * j;
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t rg = min(row0 + r, rows - 1);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kb0 + 16 * c < kb_end) v = *(const uint4*)(p + rg * ldb_bytes + kb0 + 16 * c);
    lds_write_b128(tile + 1024 * i + 16 * lane, v);
  }
}

// Scale dwords of one K tile for this lane's rows (4 row blocks of 32): word q holds
// the scales of blocks 4q..4q+3 of the tile, pre-shifted so that byte 0 / byte 2 are
// the blocks of K steps 2q / 2q+1 this lane feeds (block parity = l/32). Blocks at or
// past nblk (the end of K) read as 127 (2^0) so that zero padding stays zero.
template <int FMT>
__device__ __forceinline__ void load_scales(const uint8_t* __restrict__ sf, int64_t ld_sf, int64_t row0, int64_t rows,
                                            int64_t blk0, int64_t nblk, int lane, uint32_t (&out)[4][2]) {
  const int sh = 8 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int64_t rg = min(row0 + 32 * t + (lane & 31), rows - 1);
    const uint8_t* p = sf + rg * ld_sf + blk0;
#pragma unroll
    for (int q = 0; q < Fmt<FMT>::SFW; q++) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const int64_t blk = blk0 + 4 * q + b;
        const uint32_t s = blk < nblk ? p[4 * q + b] : 127u;
        v |= s << (8 * b);
      }
      out[t][q] = v >> sh;
    }
  }
}

template <int FMT>
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int rbase, int s, int lane) {
  const int r = rbase + (lane & 31);
  i32x8 f;
  if (FMT == 4) {
    const uint4 v = lds_read_b128(tile + kmaj_off(r, 2 * s + (lane >> 5)));
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; f[4] = 0; f[5] = 0; f[6] = 0; f[7] = 0;
  } else {
    const uint4 v0 = lds_read_b128(tile + kmaj_off(r, 4 * s + (lane >> 5)));
    const uint4 v1 = lds_read_b128(tile + kmaj_off(r, 4 * s + 2 + (lane >> 5)));
    f[0] = v0.x; f[1] = v0.y; f[2] = v0.z; f[3] = v0.w; f[4] = v1.x; f[5] = v1.y; f[6] = v1.z; f[7] = v1.w;
  }
  return f;
}

template <int FMT, int SEL>
__device__ __forceinline__ f32x16 mfma_sc(i32x8 a, i32x8 b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, SEL, (int)sa, SEL, (int)sb);
}

template <int FMT>
__device__ __forceinline__ void compute_step(const uint8_t* ta, const uint8_t* tb, int s, int wm, int wn, int lane,
                                             const uint32_t (&sa)[4][2], const uint32_t (&sb)[4][2],
                                             f32x16 (&acc)[4][4]) {
  i32x8 af[4], bf[4];
#pragma unroll
  for (int t = 0; t < 4; t++) af[t] = read_frag<FMT>(ta, 128 * wm + 32 * t, s, lane);
#pragma unroll
  for (int t = 0; t < 4; t++) bf[t] = read_frag<FMT>(tb, 128 * wn + 32 * t, s, lane);
  const int q = s >> 1;
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      if (s & 1) acc[mt][nt] = mfma_sc<FMT, 2>(af[mt], bf[nt], acc[mt][nt], sa[mt][q], sb[nt][q]);
      else acc[mt][nt] = mfma_sc<FMT, 0>(af[mt], bf[nt], acc[mt][nt], sa[mt][q], sb[nt][q]);
    }
}

__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = pid / per_group;
  const int first = g * GROUP;
  const int gsize = min(tiles_m - first, GROUP);
  const int in = pid - g * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void k_gemm_mx(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Fmt<FMT> F;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][TILE_BYTES];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const uint8_t* A = (const uint8_t*)a.A;
  const uint8_t* B = (const uint8_t*)a.B;
  const int64_t lda_b = a.lda / F::EPB, ldb_b = a.ldb / F::EPB;
  const int64_t nblk = a.K / 32;

  f32x16 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][nt][r] = 0.0f;

  const int nfull = (int)(a.K / F::KT);
  const int tail = (int)(a.K % F::KT);
  const int bpt = F::KT / 32;  // scale blocks per K tile
  uint32_t sa[4][2], sb[4][2], na[4][2], nb[4][2];
  if (nfull > 0) {
    issue_tile(A, lda_b, m0, a.M, 0, lds[0][0], w, lane);
    issue_tile(B, ldb_b, n0, a.N, 0, lds[0][1], w, lane);
  }
  load_scales<FMT>(a.SFA, a.ld_sfa, m0 + 128 * wm, a.M, 0, nblk, lane, sa);
  load_scales<FMT>(a.SFB, a.ld_sfb, n0 + 128 * wn, a.N, 0, nblk, lane, sb);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < nfull; kt++) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nfull || tail;
    if (kt + 1 < nfull) {
      issue_tile(A, lda_b, m0, a.M, (int64_t)(kt + 1) * ROWB, lds[cur ^ 1][0], w, lane);
      issue_tile(B, ldb_b, n0, a.N, (int64_t)(kt + 1) * ROWB, lds[cur ^ 1][1], w, lane);
    }
    if (more) {
      load_scales<FMT>(a.SFA, a.ld_sfa, m0 + 128 * wm, a.M, (int64_t)(kt + 1) * bpt, nblk, lane, na);
      load_scales<FMT>(a.SFB, a.ld_sfb, n0 + 128 * wn, a.N, (int64_t)(kt + 1) * bpt, nblk, lane, nb);
    }
#pragma unroll
    for (int s = 0; s < F::STEPS; s++) compute_step<FMT>(lds[cur][0], lds[cur][1], s, wm, wn, lane, sa, sb, acc);
    wait_vmem();
    __syncthreads();
    if (more) {
#pragma unroll
      for (int t = 0; t < 4; t++)
#pragma unroll
        for (int q = 0; q < 2; q++) { sa[t][q] = na[t][q]; sb[t][q] = nb[t][q]; }
    }
  }
  if (tail) {
    const int st = nfull & 1;
    const int64_t kb0 = (int64_t)nfull * ROWB;
    const int64_t kb_end = a.K / F::EPB;
    fill_tile_masked(A, lda_b, m0, a.M, kb0, kb_end, lds[st][0], w, lane);
    fill_tile_masked(B, ldb_b, n0, a.N, kb0, kb_end, lds[st][1], w, lane);
    __syncthreads();
    const int steps = (tail + 63) / 64;
    for (int s = 0; s < steps; s++) {
      if (s == 0) compute_step<FMT>(lds[st][0], lds[st][1], 0, wm, wn, lane, sa, sb, acc);
      else if (s == 1) compute_step<FMT>(lds[st][0], lds[st][1], 1, wm, wn, lane, sa, sb, acc);
      else if (s == 2) compute_step<FMT>(lds[st][0], lds[st][1], 2, wm, wn, lane, sa, sb, acc);
      else compute_step<FMT>(lds[st][0], lds[st][1], 3, wm, wn, lane, sa, sb, acc);
    }
  }

  const float sgn = a.negate ? -1.0f : 1.0f;
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      const int64_t col = n0 + 128 * wn + 32 * nt + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = m0 + 128 * wm + 32 * mt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.M && col < a.N) {
          float* d = a.D + row * a.ldd + col;
          const float v = sgn * acc[mt][nt][r];
          *d = a.accum ? *d + v : v;
        }
      }
    }
  }
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
