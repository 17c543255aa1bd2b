// k_gemm_mx_any.hip - block-scaled GEMM for any pairing of the f8f6f4 element formats
// (E4M3, E5M2, E2M3, E3M2, E2M1) on gfx950 v_mfma_scale_f32_32x32x64_f8f6f4: the 6-bit
// formats and operands of different widths (say E4M3 x E2M1). Pairs of equal width that
// the tuned kernel of k_gemm_mx.hip covers (8-bit x 8-bit, E2M1 x E2M1) do not come here.
//
// Semantics as there ("tcgen05.mma": Weight-stationary and block scaling; "Explicit CUDA
// tile patterns": tcgen05 MMA): value = element * 2^(scale - 127), one scale per 32 K of a
// row, float32 accumulation, D = s * A * B^T (+ D), then the scalar epilogue.
//
// Operand registers (probed on the device; each operand follows its own format's layout,
// so mixed pairs need no conversion):
//  - 8-bit: lane l holds row l%32, k in [16(l/32), +16) and [32 + 16(l/32), +16) of the
//    64-K step (two 16-byte groups);
//  - 6-bit: lane l holds row l%32, k in [32(l/32), +32): 24 bytes, element i at bits
//    6i .. 6i+5 (the same little-endian packing as in memory);
//  - 4-bit: lane l holds row l%32, k in [32(l/32), +32): 16 bytes, low nibble first.
//
// Design (a general path, not the tuned pipeline): workgroup tile 256 x 256, K tiles of
// 128 elements (128, 96 or 64 bytes of a row), four waves with 128 x 128 sub-tiles.
// Operand tiles go HBM -> registers -> LDS, one K tile ahead (the loads of tile kt + 2
// are issued after tile kt + 1 is written to LDS, so they land during tile kt + 1's
// multiplies). LDS rows are padded by 16 bytes, so the 16 rows read at one offset by a
// 16-lane group fall in distinct banks for every row width. Scales go straight from HBM
// to registers (one 32-bit word per row per K tile: the four 32-K blocks). A partial last
// K tile reads zero elements and unit scales past K.
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256, KT = 128;

__host__ __device__ constexpr int fmt_bits(int c) { return c <= 1 ? 8 : (c <= 3 ? 6 : 4); }

template <int C>
struct Op {
  static constexpr int BITS = fmt_bits(C);
  static constexpr int ROW = 16 * BITS;   // bytes of a row per K tile: 128, 96, 64
  static constexpr int PITCH = ROW + 16;  // LDS row pitch
  static constexpr int TILE = 256 * PITCH;
  static constexpr int CPR = ROW / 16;    // 16-byte chunks per row per K tile (and per lane)
};

template <int CA, int CB>
struct Lay {
  static constexpr int STAGE = Op<CA>::TILE + Op<CB>::TILE;
  static constexpr int BYTES = 2 * STAGE > 131072 ? 2 * STAGE : 131072;  // the epilogue uses 128 KiB
};

__device__ __forceinline__ uint2 lds_read_b64(const void* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *(const BSM_LDS u32x2*)(p);
  return make_uint2(v[0], v[1]);
}

// Byte offsets (from the tile's first row) of the rows of this lane's CPR chunks, rows past
// the operand clamped to its last row (the host keeps 256 rows of a leading dimension below
// 2^31 bytes).
template <int C>
__device__ __forceinline__ void row_offsets(int64_t ld_bytes, int64_t rows, int q, uint32_t (&ro)[Op<C>::CPR]) {
  typedef Op<C> P;
#pragma unroll
  for (int i = 0; i < P::CPR; i++) {
    const int c = q + 256 * i, r = c / P::CPR;
    ro[i] = (uint32_t)(min((int64_t)r, rows - 1) * ld_bytes);
  }
}

// Chunk i (of CPR) of this lane in K tile kt of one operand: bytes [16 cc, +16) of the
// tile's row piece of row ro[i]; bytes at or past `kbytes` (the row's K extent) read as zero.
template <int C>
__device__ __forceinline__ void load_chunks(const uint8_t* base, const uint32_t (&ro)[Op<C>::CPR], int kt,
                                            int64_t kbytes, int q, uint4 (&v)[Op<C>::CPR]) {
  typedef Op<C> P;
#pragma unroll
  for (int i = 0; i < P::CPR; i++) {
    const int c = q + 256 * i, r = c / P::CPR, cc = c - r * P::CPR;
    const int64_t off = (int64_t)kt * P::ROW + 16 * cc;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (off < kbytes) {
      x = *(const uint4*)(base + ro[i] + off);   // inside the row: rows are whole 16-byte chunks
      const int64_t valid = kbytes - off;
      if (valid < 16) {
        uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const int64_t nb = valid - 4 * d;
          wd[d] &= nb >= 4 ? 0xFFFFFFFFu : (nb <= 0 ? 0u : (1u << (8 * nb)) - 1u);
        }
        x = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
    v[i] = x;
  }
}

template <int C>
__device__ __forceinline__ void store_chunks(uint8_t* tile, int q, const uint4 (&v)[Op<C>::CPR]) {
  typedef Op<C> P;
#pragma unroll
  for (int i = 0; i < P::CPR; i++) {
    const int c = q + 256 * i, r = c / P::CPR, cc = c - r * P::CPR;
    lds_write_b128(tile + r * P::PITCH + 16 * cc, v[i]);
  }
}

// Scale words of K tile kt for this lane's four rows (row0 + base + 32t + l%32); the bytes
// of blocks at or past nblk (K / 32) become 127 (unit scale on zero elements).
__device__ __forceinline__ void load_scales(const uint8_t* sf, int64_t ld_sf, int64_t row0, int64_t rows, int base,
                                            int lane, int kt, int64_t nblk, uint32_t (&s)[4]) {
  const int64_t b0 = 4 * (int64_t)kt;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int64_t grow = min(row0 + base + 32 * t + (lane & 31), rows - 1);
    uint32_t x = *(const uint32_t*)(sf + grow * ld_sf + b0);
    if (b0 + 4 > nblk) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (b0 + j >= nblk) x = (x & ~(0xFFu << (8 * j))) | (127u << (8 * j));
    }
    s[t] = x;
  }
}

// Operand registers of 64-K step s for the lane's row of 32-row block t.
template <int C>
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int base, int t, int s, int lane) {
  typedef Op<C> P;
  const int h = lane >> 5;
  const uint8_t* row = tile + (base + 32 * t + (lane & 31)) * P::PITCH;
  i32x8 v;
  if (P::BITS == 8) {
    const uint4 x = lds_read_b128(row + 64 * s + 16 * h), y = lds_read_b128(row + 64 * s + 32 + 16 * h);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else if (P::BITS == 6) {
    const uint8_t* p = row + 48 * s + 24 * h;
    const uint2 x = lds_read_b64(p), y = lds_read_b64(p + 8), z = lds_read_b64(p + 16);
    v[0] = x.x; v[1] = x.y; v[2] = y.x; v[3] = y.y; v[4] = z.x; v[5] = z.y;
    v[6] = v[7] = 0;
  } else {
    const uint4 x = lds_read_b128(row + 32 * s + 16 * h);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = v[5] = v[6] = v[7] = 0;
  }
  return v;
}

// The 16 MFMAs of 64-K step S (fragments read first). The MFMA takes B first (its format
// code and scales as src0); after the per-lane shift by 8 (l/32), op_sel byte 2S holds the
// scale of the lane's 32-K block of this step.
template <int CA, int CB, int S>
__device__ __forceinline__ void mx_step(const uint8_t* ta, const uint8_t* tb, int wa, int wb, int lane, int sh,
                                        const uint32_t (&sa)[4], const uint32_t (&sb)[4], f32x16 (&acc)[4][4]) {
  i32x8 fa[4], fb[4];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    fa[t] = read_frag<CA>(ta, wa, t, S, lane);
    fb[t] = read_frag<CB>(tb, wb, t, S, lane);
  }
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
    {
      asm volatile("" : "+a"(acc[mt][nt]));   // keep the accumulators in AGPRs
      acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[nt], fa[mt], acc[mt][nt], CB, CA, 2 * S,
                                                                     (int)(sb[nt] >> sh), 2 * S, (int)(sa[mt] >> sh));
      asm volatile("" : "+a"(acc[mt][nt]));
    }
}

template <int CA, int CB>
__global__ __launch_bounds__(256, 1) void k_gemm_mx_any(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Op<CA> PA;
  typedef Op<CB> PB;
  typedef Lay<CA, CB> L;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
  const int q = threadIdx.x, lane = q & 63, w = __builtin_amdgcn_readfirstlane(q >> 6);
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wa = 128 * (w >> 1), wb = 128 * (w & 1);
  const float sgn = a.negate ? -1.0f : 1.0f;
  const int64_t nblk = a.K / 32;
  const int nkt = (int)((a.K + KT - 1) / KT);
  const int64_t lda_b = a.lda * PA::BITS / 8, ldb_b = a.ldb * PB::BITS / 8;
  const int64_t ka = a.K * PA::BITS / 8, kb = a.K * PB::BITS / 8;   // a row's K extent in bytes
  const uint8_t* A = (const uint8_t*)a.A + m0 * lda_b;
  const uint8_t* B = (const uint8_t*)a.B + n0 * ldb_b;
  const int64_t rows_a = a.M - m0, rows_b = a.N - n0;
  const int sh = 8 * (lane >> 5);

  f32x16 acc[4][4];
  gemm::zero_acc(acc);
  uint4 va[PA::CPR], vb[PB::CPR];
  uint32_t sa[4], sb[4], na[4], nb[4], roa[PA::CPR], rob[PB::CPR];
  row_offsets<CA>(lda_b, rows_a, q, roa);
  row_offsets<CB>(ldb_b, rows_b, q, rob);

  load_chunks<CA>(A, roa, 0, ka, q, va);
  load_chunks<CB>(B, rob, 0, kb, q, vb);
  load_scales(a.SFA, a.ld_sfa, m0, a.M, wa, lane, 0, nblk, sa);
  load_scales(a.SFB, a.ld_sfb, n0, a.N, wb, lane, 0, nblk, sb);
  store_chunks<CA>(lds, q, va);
  store_chunks<CB>(lds + PA::TILE, q, vb);
  if (nkt > 1) {
    load_chunks<CA>(A, roa, 1, ka, q, va);
    load_chunks<CB>(B, rob, 1, kb, q, vb);
    load_scales(a.SFA, a.ld_sfa, m0, a.M, wa, lane, 1, nblk, na);
    load_scales(a.SFB, a.ld_sfb, n0, a.N, wb, lane, 1, nblk, nb);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; kt++) {
    const uint8_t* ta = lds + (kt & 1) * L::STAGE;
    const uint8_t* tb = ta + PA::TILE;
    mx_step<CA, CB, 0>(ta, tb, wa, wb, lane, sh, sa, sb, acc);
    mx_step<CA, CB, 1>(ta, tb, wa, wb, lane, sh, sa, sb, acc);
    if (kt + 1 < nkt) {
      uint8_t* na_t = lds + ((kt + 1) & 1) * L::STAGE;
      store_chunks<CA>(na_t, q, va);
      store_chunks<CB>(na_t + PA::TILE, q, vb);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        sa[t] = na[t];
        sb[t] = nb[t];
      }
      if (kt + 2 < nkt) {
        load_chunks<CA>(A, roa, kt + 2, ka, q, va);
        load_chunks<CB>(B, rob, kt + 2, kb, q, vb);
        load_scales(a.SFA, a.ld_sfa, m0, a.M, wa, lane, kt + 2, nblk, na);
        load_scales(a.SFB, a.ld_sfb, n0, a.N, wb, lane, kt + 2, nblk, nb);
      }
    }
    __syncthreads();
  }
  gemm::store_tile_lines(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc, lds + 32768 * w, a.accum != 0,
                         a.ew_op, a.ew_scale, a.ew_bias);
}

// Pairs of equal width (8-bit x 8-bit, E2M1 x E2M1) belong to the tuned kernel.
template <int CA, int CB>
hipError_t launch_pair(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t st) {
  if constexpr ((fmt_bits(CA) == 8 && fmt_bits(CB) == 8) || (CA == 4 && CB == 4)) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((k_gemm_mx_any<CA, CB>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m, tiles_n);
    return hipGetLastError();
  }
}

template <int CA>
hipError_t launch_b(int cb, const GemmArgs& a, int tm, int tn, hipStream_t st) {
  switch (cb) {
    case 0: return launch_pair<CA, 0>(a, tm, tn, st);
    case 1: return launch_pair<CA, 1>(a, tm, tn, st);
    case 2: return launch_pair<CA, 2>(a, tm, tn, st);
    case 3: return launch_pair<CA, 3>(a, tm, tn, st);
    default: return launch_pair<CA, 4>(a, tm, tn, st);
  }
}

// bsm_dtype -> MFMA format code
int mfma_code(int32_t dt) {
  switch (dt) {
    case BSM_E4M3: return 0;
    case BSM_E5M2: return 1;
    case BSM_E2M3: return 2;
    case BSM_E3M2: return 3;
    default: return 4;  // BSM_E2M1
  }
}

}  // namespace

hipError_t launch_gemm_mx_any(const GemmArgs& a, hipStream_t st) {
  const int64_t tm64 = (a.M + BM - 1) / BM, tn64 = (a.N + BN - 1) / BN;
  if (tm64 * tn64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tm = (int)tm64, tn = (int)tn64;
  const int ca = mfma_code(a.dtype), cb = mfma_code(a.dtype_b);
  switch (ca) {
    case 0: return launch_b<0>(cb, a, tm, tn, st);
    case 1: return launch_b<1>(cb, a, tm, tn, st);
    case 2: return launch_b<2>(cb, a, tm, tn, st);
    case 3: return launch_b<3>(cb, a, tm, tn, st);
    default: return launch_b<4>(cb, a, tm, tn, st);
  }
}

}  // namespace bsm
