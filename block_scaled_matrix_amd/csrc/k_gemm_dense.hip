// k_gemm_dense.hip - fp16/bf16 GEMM D = s * A * B^T (+ D) on gfx950 MFMA.
//
// Semantics ("tcgen05.mma": Call parameters, Operand specification, Code generation,
// Example: four K16 issues; "Explicit CUDA tile patterns": Warp MMA): B is the
// (N,K) operand, the product is A times B transposed, float32 accumulation; the
// first K step starts from D when accumulating and from zero otherwise.
//
// gfx950 design:
//  - workgroup tile 256 x 256, K tile 64, four wave64s in a 2 x 2 grid, each owning a
//    128 x 128 sub-tile as 4 x 4 v_mfma_f32_32x32x16 accumulators (256 fp32 per lane);
//  - operand tiles stream HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging), two LDS stages (2 x 64 KiB), one barrier per K tile;
//  - K-major tiles: 128-byte rows, 16-byte chunk c of row r stored at chunk
//    c ^ ((r >> 1) & 7), so the 16 rows one 16-lane group reads with ds_read_b128
//    cover all 64 LDS banks;
//  - MN-major tiles (the transposed storage): 512-byte k-rows, chunk c of k-row kr
//    stored at c ^ (4 * (kr & 3)); fragments come from ds_read_b64_tr_b16, the LDS
//    transpose read (the analog of ldmatrix .trans in "ldmatrix / stmatrix",
//    Transpose and stores), whose 32-lane groups again cover all banks;
//  - M/N edges clamp the rows that are loaded and mask the stores; a ragged last K
//    tile is loaded through registers with the elements past K zeroed.
#include "bsm_device.hpp"
#include "bsm_internal.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE_BYTES = 256 * BK * 2;  // one operand tile: 32 KiB

__device__ __forceinline__ uint32_t kmaj_off(int r, int c) { return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4)); }
__device__ __forceinline__ uint32_t mnmaj_off(int kr, int c) { return (uint32_t)(kr * 512 + ((c ^ ((kr & 3) << 2)) << 4)); }

// Direct HBM -> LDS copy of one 256-row x 64-k operand tile (32 wave instructions of
// 1 KiB; wave w issues instructions w, w+4, ..., w+28). Rows past `rows` are clamped.
template <bool KMAJ>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ p, int64_t ld, int64_t row0, int64_t rows,
                                           int64_t k0, uint8_t* tile, int w, int lane) {
  if (KMAJ) {
    const int c = (lane & 7) ^ (((8 * w + (lane >> 3)) >> 1) & 7);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int i = w + 4 * j;
      const int64_t rg = min(row0 + 8 * i + (lane >> 3), rows - 1);
      load_lds_16(p + rg * ld + k0 + 8 * c, tile + 1024 * i);
    }
  } else {
    const int kr0 = 2 * w + (lane >> 5);
    const int c = (lane & 31) ^ ((kr0 & 3) << 2);
    const int64_t col = min(row0 + 8 * c, (rows - 1) & ~int64_t(7));
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int i = w + 4 * j;
      load_lds_16(p + (k0 + kr0 + 8 * j) * ld + col, tile + 1024 * i);
    }
  }
}

// The same tile for a partial K tile: through registers, elements with k >= K zeroed.
template <bool KMAJ>
__device__ __forceinline__ void fill_tile_masked(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                                 int64_t rows, int64_t k0, int64_t K, uint8_t* tile, int w, int lane) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int i = w + 4 * j;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (KMAJ) {
      const int r = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int64_t rg = min(row0 + r, rows - 1);
      const int64_t k = k0 + 8 * c;
      if (k < K) {
        v = *(const uint4*)(p + rg * ld + k);
        const int64_t valid = K - k;  // elements k..k+7 kept while < K
        uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; e++)
          if (e >= valid) wd[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    } else {
      const int kr = 2 * i + (lane >> 5);
      const int c = (lane & 31) ^ ((kr & 3) << 2);
      const int64_t col = min(row0 + 8 * c, (rows - 1) & ~int64_t(7));
      if (k0 + kr < K) v = *(const uint4*)(p + (k0 + kr) * ld + col);
    }
    lds_write_b128(tile + 1024 * i + 16 * lane, v);
  }
}

template <int DT>
struct Frag;
template <>
struct Frag<BSM_BF16> { typedef bf16x8 T; };
template <>
struct Frag<BSM_F16> { typedef f16x8 T; };

// Operand fragment of v_mfma_f32_32x32x16: lane l holds (row rbase + l%32,
// k 16*ks + 8*(l/32) + e), e = 0..7.
template <bool KMAJ>
__device__ __forceinline__ uint4 read_frag(const uint8_t* tile, int rbase, int ks, int lane) {
  if (KMAJ) {
    return lds_read_b128(tile + kmaj_off(rbase + (lane & 31), 2 * ks + (lane >> 5)));
  } else {
    const int i = lane & 15, G = lane >> 4;
    const int kb = 16 * ks + 8 * (G >> 1) + (i >> 2);
    const int n = rbase + 16 * (G & 1) + 4 * (i & 3);
    const i16x4 lo = lds_read_tr16(tile + mnmaj_off(kb, n >> 3) + (n & 7) * 2);
    const i16x4 hi = lds_read_tr16(tile + mnmaj_off(kb + 4, n >> 3) + (n & 7) * 2);
    uint4 v;
    v.x = (uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    v.y = (uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    v.z = (uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    v.w = (uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return v;
  }
}

template <int DT>
__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
  typedef typename Frag<DT>::T T;
  const T av = __builtin_bit_cast(T, a), bv = __builtin_bit_cast(T, b);
  if constexpr (DT == BSM_BF16) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
}

template <int DT, bool AK, bool BKM>
__device__ __forceinline__ void compute_tile(const uint8_t* ta, const uint8_t* tb, int nsteps, int wm, int wn,
                                             int lane, f32x16 (&acc)[4][4]) {
  for (int ks = 0; ks < nsteps; ks++) {
    uint4 af[4], bf[4];
#pragma unroll
    for (int t = 0; t < 4; t++) af[t] = read_frag<AK>(ta, 128 * wm + 32 * t, ks, lane);
#pragma unroll
    for (int t = 0; t < 4; t++) bf[t] = read_frag<BKM>(tb, 128 * wn + 32 * t, ks, lane);
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int nt = 0; nt < 4; nt++) acc[mt][nt] = mfma<DT>(af[mt], bf[nt], acc[mt][nt]);
  }
}

// Tile order: consecutive workgroup ids walk a column of GROUP tile rows so that
// workgroups running together share A row panels and B column panels in L2.
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

template <int DT, bool AK, bool BKM>
__global__ __launch_bounds__(256, 1) void k_gemm_dense(GemmArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][TILE_BYTES];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* B = (const uint16_t*)a.B;

  f32x16 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][nt][r] = 0.0f;

  const int nfull = (int)(a.K / BK);
  const int tail = (int)(a.K % BK);
  if (nfull > 0) {
    issue_tile<AK>(A, a.lda, m0, a.M, 0, lds[0][0], w, lane);
    issue_tile<BKM>(B, a.ldb, n0, a.N, 0, lds[0][1], w, lane);
  }
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < nfull; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nfull) {
      issue_tile<AK>(A, a.lda, m0, a.M, (int64_t)(kt + 1) * BK, lds[cur ^ 1][0], w, lane);
      issue_tile<BKM>(B, a.ldb, n0, a.N, (int64_t)(kt + 1) * BK, lds[cur ^ 1][1], w, lane);
    }
    compute_tile<DT, AK, BKM>(lds[cur][0], lds[cur][1], BK / 16, wm, wn, lane, acc);
    wait_vmem();
    __syncthreads();
  }
  if (tail) {
    const int st = nfull & 1;
    const int64_t k0 = (int64_t)nfull * BK;
    fill_tile_masked<AK>(A, a.lda, m0, a.M, k0, a.K, lds[st][0], w, lane);
    fill_tile_masked<BKM>(B, a.ldb, n0, a.N, k0, a.K, lds[st][1], w, lane);
    __syncthreads();
    compute_tile<DT, AK, BKM>(lds[st][0], lds[st][1], (tail + 15) / 16, wm, wn, lane, acc);
  }

  // Epilogue: D = s * acc (+ D). Accumulator register r of a 32x32 block holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
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

template <int DT, bool AK, bool BKM>
hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  const int64_t tm64 = (a.M + BM - 1) / BM, tn64 = (a.N + BN - 1) / BN;
  if (tm64 * tn64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = (int)tm64, tiles_n = (int)tn64;
  hipLaunchKernelGGL((k_gemm_dense<DT, AK, BKM>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m, tiles_n);
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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  issue_tile<KMAJ>(src, KMAJ ? BK : BM, 0, BM, 0, tile, w, lane);
  wait_vmem();
  __syncthreads();
  for (int mb = 2 * w; mb < 2 * w + 2; mb++) {
    for (int ks = 0; ks < BK / 16; ks++) {
      const uint4 v = read_frag<KMAJ>(tile, 32 * mb, ks, lane);
      *(uint4*)(dump + ((mb * (BK / 16) + ks) * 64 + lane) * 8) = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t st) {
  if (a.K == 0) {
    // Empty sum: D = accum ? D : 0 (the sign of an empty sum is irrelevant).
    if (a.accum) return hipSuccess;
    return launch_zero_f32_2d(a.D, a.ldd, a.M, a.N, st);
  }
  return a.dtype == BSM_BF16 ? launch_dt<BSM_BF16>(a, st) : launch_dt<BSM_F16>(a, st);
}

hipError_t launch_debug_fragments(const uint16_t* src, int kmajor, uint16_t* dump, hipStream_t st) {
  if (kmajor) hipLaunchKernelGGL(k_debug_fragments<true>, dim3(1), dim3(256), 0, st, src, dump);
  else hipLaunchKernelGGL(k_debug_fragments<false>, dim3(1), dim3(256), 0, st, src, dump);
  return hipGetLastError();
}

}  // namespace bsm
