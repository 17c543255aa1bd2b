// gemm_mx_any.hpp - the general block-scaled GEMM kernel: any pairing of the f8f6f4 element formats
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
// Design: workgroup tile 256 x 256, K
// tiles of 128 elements (128, 96 or 64 bytes of a row), four waves with 128 x 128
// sub-tiles. Whole K tiles stream HBM -> LDS with direct copies (global_load_lds, 1 KiB of
// LDS per copy) into three stages (two when an 8-bit operand meets a 6-bit one: three do
// not fit), the copy of tile kt + NST issued as soon as every wave is done reading tile kt,
// so the copies have NST - 1 K tiles of multiplies to land in (one K tile of 6- or 4-bit
// operands is only 1024 MFMA cycles); on the scaled-MFMA route with three stages half of
// them wait for the next step, which spreads the copies over the whole K tile. Each row's 16-byte chunks are permuted (by the
// copies' global addresses) so that the 16 rows one 16-lane group reads at one offset fall
// in distinct banks: chunk c of row r sits at c ^ ((r >> 1) & 7) for 128-byte rows,
// (c + ((r >> 3) & 1)) % 6 for 96-byte rows and c ^ ((r >> 2) & 3) for 64-byte rows. The
// scale words (one 32-bit word per row and K tile: its four 32-K blocks) come through a
// ring of two buffers, each holding a group of four K tiles (16 bytes per row), a quarter
// of a group copied with every K tile's data as 16-row copies of 4 bytes per lane: a copy
// whose 64 lanes touch 64 rows, one word per row and K tile, held the shared copy path
// four times as long. One barrier per K tile, at the start of its step 1; step 1's
// fragment reads go out between step 0's MFMAs, the next tile's scales and step-0
// fragments between step 1's, so no K tile starts by waiting for the LDS. A partial last
// K tile goes through registers with zero elements and unit scales past K, multiplied
// before the whole tiles (its sum is added first).
//
// Two ways to multiply a step's fragments (template parameter BF):
//  - the scaled f8f6f4 MFMA (BF false). It sums the products of one 32-K scale block on a grid
//    of 2^-13 times the block's largest |product| (measured on the device), which is exact only
//    when every product of the pair's formats is a multiple of that grid (E2M1 x E2M1, E2M3 x
//    E2M3, E2M1 x E2M3, E2M1 x E3M2);
//  - exact products (BF true), for every pairing with a wider product range: each operand
//    element times its block scale is converted to bf16 in registers (exact: 2 to 4 significant
//    bits and an exponent inside bf16's range), and the products are summed by the bf16
//    32x32x16 MFMA, which keeps every product bit down to about 2^-24 of the largest term of
//    each instruction (measured on the device). The conversion reads the scale as E8M0 from the
//    exponent field of a float (code << 23; code 255 gives NaN), so it applies the scale exactly.
//    Every format is then read so that lane half h holds the contiguous k in [32h, +32) of the
//    64-K step, element 8j + e feeding the bf16 MFMA j of the step at k 8h + e, for both
//    operands alike; one step is four bf16 MFMAs per accumulator, at half the 8-bit MFMA rate.
//
// MN-major operands (K rows with M or N contiguous; 8-bit and E2M1 elements): the tile is
// 128 k-rows of the workgroup's 256 M/N elements, copied as they are, and the fragments
// come from gfx950's transposing LDS reads (probed on the device): within a 16-lane group
// ds_read_b64_tr_b8 hands lane i column i of an 8 (k) x 16 (m) byte block whose k-row e
// the lanes 2e and 2e + 1 address (8 bytes each), and ds_read_b64_tr_b4 column i of a
// 16 x 16 nibble block whose k-row e lane e addresses, k in register order either way.
// Chunk c of k-row r sits at c ^ (r & 7) ^ 8 (c & 1) (256-byte k-rows: a group's eight
// k-rows in distinct banks, the even and odd chunks the two groups of a half-wave read in
// opposite halves of the row) or c ^ ((r >> 1) & 7) (128-byte k-rows: sixteen k-rows in
// distinct (row parity, chunk) pairs), so no two lanes of a half-wave share a bank.
#pragma once
#include <type_traits>
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace mxany {

constexpr int BM = 256, BN = 256, KT = 128;

__host__ __device__ constexpr int fmt_bits(int c) { return c <= 1 ? 8 : (c <= 3 ? 6 : 4); }

// True when some product of the two formats is not a multiple of 2^-13 times the largest
// product the formats can form, so the scaled MFMA's block sum may drop bits: any 8-bit
// operand, and E3M2 with E3M2 or E2M3 (E3M2 values are multiples of 2^-4 up to 28).
__host__ __device__ constexpr bool wide_products(int ca, int cb) {
  return fmt_bits(ca) == 8 || fmt_bits(cb) == 8 || (ca == 3 && cb != 4) || (cb == 3 && ca != 4);
}

// bsm_dtype -> MFMA format code
inline int mfma_code(int32_t dt) {
  switch (dt) {
    case BSM_E4M3: return 0;
    case BSM_E5M2: return 1;
    case BSM_E2M3: return 2;
    case BSM_E3M2: return 3;
    default: return 4;  // BSM_E2M1
  }
}

// An operand's K tile in LDS: K-major, 256 rows (M or N) of 128 K elements; MN-major, 128
// k-rows of the tile's 256 M or N elements. The same bytes either way (4096 x bits).
template <int C, bool MN>
struct Op {
  static constexpr int BITS = fmt_bits(C);
  static constexpr int ROWS = MN ? 128 : 256;
  static constexpr int ROW = MN ? 32 * BITS : 16 * BITS;  // bytes of an LDS row
  static constexpr int TILE = ROWS * ROW;
  static constexpr int CPR = ROW / 16;                    // 16-byte chunks per LDS row
  static constexpr int LPC = TILE / 16 / 256;             // chunks per lane per tile
  static_assert(!MN || BITS != 6, "MN-major operands are 8-bit or E2M1");
  // physical chunk of logical chunk c in row r, and back
  __device__ static int phys(int c, int r) {
    if (MN) return CPR == 16 ? c ^ (r & 7) ^ ((c & 1) << 3) : c ^ ((r >> 1) & 7);
    return CPR == 8 ? c ^ ((r >> 1) & 7) : (CPR == 6 ? (c + ((r >> 3) & 1)) % 6 : c ^ ((r >> 2) & 3));
  }
  __device__ static int logical(int pc, int r) {
    if (MN) return CPR == 16 ? (pc ^ (r & 7)) ^ (((pc ^ r) & 1) << 3) : pc ^ ((r >> 1) & 7);
    return CPR == 8 ? pc ^ ((r >> 1) & 7) : (CPR == 6 ? (pc + 6 - ((r >> 3) & 1)) % 6 : pc ^ ((r >> 2) & 3));
  }
};

// A stage: A tile, B tile. NST stages, then the scale ring: two buffers of one group of
// four K tiles each, A's 256 rows then B's, 16 bytes per row (the row's scale words of the
// group's tiles), all within the 160 KiB of LDS.
template <int CA, int CB>
struct Lay {
  static constexpr int STAGE = Op<CA, false>::TILE + Op<CB, false>::TILE;
  static constexpr int RING_BUF = 2 * 256 * 16;
  static constexpr int NST = 3 * STAGE + 2 * RING_BUF <= 163840 ? 3 : 2;
  static constexpr int RING = NST * STAGE;
  static constexpr int END = RING + 2 * RING_BUF;
  static constexpr int BYTES = END > 131072 ? END : 131072;  // the epilogue uses 128 KiB
};

// Scale ring: word q (K tile 4g + q) of row R of a group buffer sits at physical word
// q ^ ((R >> 4) & 3) ^ ((R >> 6) & 1), XOR 2 in B's half: the 32 consecutive rows one read
// instruction touches fall in 32 distinct banks, and so do the words of rows 32, 64 or 96
// apart (blocks t and t + 1 .. 3, multiples of 512 bytes apart), which the compiler may
// fetch with one two-address read.
__device__ __forceinline__ uint32_t ring_word_offset(int op, int R, int q) {
  return (uint32_t)(16 * R + 4 * (q ^ ((R >> 4) & 3) ^ ((R >> 6) & 1) ^ (op ? 2 : 0)));
}

// This lane's scale words of K tile kt for its four rows (base + 32t + l%32) from the ring
// buffer of kt's group (operand op's half).
__device__ __forceinline__ void read_scales_ring(const uint8_t* half, int op, int kt, int base, int lane,
                                                 uint32_t (&s)[4]) {
#pragma unroll
  for (int t = 0; t < 4; t++) s[t] = *(const BSM_LDS uint32_t*)(half + ring_word_offset(op, base + 32 * t + (lane & 31), kt & 3));
}

__device__ __forceinline__ uint2 lds_read_b64(const void* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = *(const BSM_LDS u32x2*)(p);
  return make_uint2(v[0], v[1]);
}

// Byte offsets (from the tile's first row) of the rows of this lane's CPR chunks, rows past
// the operand clamped to its last row (the host keeps 256 rows of a leading dimension below
// 2^31 bytes).
template <int C>
__device__ __forceinline__ void row_offsets(int64_t ld_bytes, int64_t rows, int q, uint32_t (&ro)[Op<C, false>::LPC]) {
  typedef Op<C, false> P;
#pragma unroll
  for (int i = 0; i < P::LPC; i++) {
    const int c = q + 256 * i, r = c / P::CPR;
    ro[i] = (uint32_t)(min((int64_t)r, rows - 1) * ld_bytes);
  }
}

// This lane's CPR chunks of the partial last K tile kt of one operand (bytes [16 cc, +16)
// of the tile's row piece of row ro[i]): bytes at or past `kbytes` (the row's K extent)
// read as zero (rows are whole 16-byte chunks, so a chunk that starts inside the K extent
// lies inside the row).
template <int C>
__device__ __forceinline__ void load_chunks_tail(const uint8_t* base, const uint32_t (&ro)[Op<C, false>::LPC], int kt,
                                                 int64_t kbytes, int q, uint4 (&v)[Op<C, false>::LPC]) {
  typedef Op<C, false> P;
#pragma unroll
  for (int i = 0; i < P::LPC; i++) {
    const int c = q + 256 * i, r = c / P::CPR, cc = c - r * P::CPR;
    const int64_t off = (int64_t)kt * P::ROW + 16 * cc;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (off < kbytes) {
      x = *(const uint4*)(base + ro[i] + off);
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

// MN-major partial last K tile: k-rows at or past K read as zero; chunks past the row's
// leading dimension (M or N elements beyond the operand) are clamped to its last chunk
// (their outputs are never stored).
template <int C>
__device__ __forceinline__ void load_chunks_tail_mn(const uint8_t* base, int64_t ld_bytes, uint32_t mlim, int kt,
                                                    int64_t K, int q, uint4 (&v)[Op<C, true>::LPC]) {
  typedef Op<C, true> P;
#pragma unroll
  for (int i = 0; i < P::LPC; i++) {
    const int c = q + 256 * i, r = c / P::CPR, cc = c - r * P::CPR;
    const int64_t k = (int64_t)kt * 128 + r;
    v[i] = k < K ? *(const uint4*)(base + k * ld_bytes + min((uint32_t)(16 * cc), mlim)) : make_uint4(0, 0, 0, 0);
  }
}

template <int C, bool MN>
__device__ __forceinline__ void store_chunks(uint8_t* tile, int q, const uint4 (&v)[Op<C, MN>::LPC]) {
  typedef Op<C, MN> P;
#pragma unroll
  for (int i = 0; i < P::LPC; i++) {
    const int c = q + 256 * i, r = c / P::CPR, cc = c - r * P::CPR;
    lds_write_b128(tile + r * P::ROW + 16 * P::phys(cc, r), v[i]);
  }
}

// Thread q's scale word of K tile kt: row q of the tile (clamped to the operand), the four
// 32-K blocks of the tile. In a partial last tile the bytes of blocks at or past nblk
// (K / 32) become 127 (unit scale on zero elements).
__device__ __forceinline__ uint32_t load_scale_word(const uint8_t* sf, int64_t ld_sf, int64_t row0, int64_t rows,
                                                    int q, int kt) {
  const int64_t grow = min(row0 + q, rows - 1);
  return *(const uint32_t*)(sf + grow * ld_sf + 4 * (int64_t)kt);
}

__device__ __forceinline__ uint32_t mask_scale_word(uint32_t x, int kt, int64_t nblk) {
  const int64_t b0 = 4 * (int64_t)kt;
#pragma unroll
  for (int j = 0; j < 4; j++)
    if (b0 + j >= nblk) x = (x & ~(0xFFu << (8 * j))) | (127u << (8 * j));
  return x;
}

// This lane's scale words for its four rows (base + 32t + l%32) from a stage's scale area.
__device__ __forceinline__ void read_scales(const uint8_t* area, int base, int lane, uint32_t (&s)[4]) {
#pragma unroll
  for (int t = 0; t < 4; t++) s[t] = *(const BSM_LDS uint32_t*)(area + 4 * (base + 32 * t + (lane & 31)));
}

// Operand registers of 64-K step s for the lane's row of 32-row block t. With BF (the exact-
// products route) an 8-bit operand is read with the contiguous k in [32h, +32) of the step in
// lane half h, the order of the 6- and 4-bit formats.
template <int C, bool MN, bool BF = false>
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int base, int t, int s, int lane) {
  typedef Op<C, MN> P;
  const int h = lane >> 5;
  i32x8 v;
  if (MN) {
    // the lane's row m = base + 32t + l%32 is column i of its 16-lane group's block
    const int i = lane & 15, m0 = base + 32 * t + 16 * ((lane >> 4) & 1);
    typedef int v2i __attribute__((ext_vector_type(2)));
    auto at = [&](int kr, int o) { return tile + kr * P::ROW + 16 * P::phys(o >> 4, kr) + (o & 15); };
    if (P::BITS == 8) {
#pragma unroll
      for (int r = 0; r < 4; r++) {   // k 16h + 8r' (r' = r & 1) and 32 + ..., eight k-rows each
        const int kb = BF ? 64 * s + 32 * h + 8 * r : 64 * s + 16 * h + 8 * (r & 1) + 32 * (r >> 1);
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((BSM_LDS v2i*)at(kb + (i >> 1), m0 + 8 * (i & 1)));
        v[2 * r] = x[0];
        v[2 * r + 1] = x[1];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 2; r++) {   // k 32h + 16r .. +15, sixteen k-rows each
        const int kb = 64 * s + 32 * h + 16 * r;
        const v2i x = __builtin_amdgcn_ds_read_tr4_b64_v2i32((BSM_LDS v2i*)at(kb + i, m0 >> 1));
        v[2 * r] = x[0];
        v[2 * r + 1] = x[1];
      }
      v[4] = v[5] = v[6] = v[7] = 0;
    }
    return v;
  }
  const int r = base + 32 * t + (lane & 31);
  const uint8_t* row = tile + r * P::ROW;
  // logical byte offset o of the row -> its place in the permuted row
  auto at = [&](int o) { return row + 16 * P::phys(o >> 4, r) + (o & 15); };
  if (P::BITS == 8) {
    const int o0 = BF ? 64 * s + 32 * h : 64 * s + 16 * h, o1 = BF ? o0 + 16 : o0 + 32;
    const uint4 x = lds_read_b128(at(o0)), y = lds_read_b128(at(o1));
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else if (P::BITS == 6) {
    const int o = 48 * s + 24 * h;
    const uint2 x = lds_read_b64(at(o)), y = lds_read_b64(at(o + 8)), z = lds_read_b64(at(o + 16));
    v[0] = x.x; v[1] = x.y; v[2] = y.x; v[3] = y.y; v[4] = z.x; v[5] = z.y;
    v[6] = v[7] = 0;
  } else {
    const uint4 x = lds_read_b128(at(32 * s + 16 * h));
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = v[5] = v[6] = v[7] = 0;
  }
  return v;
}

// Operand registers of 64-K step S for the wave: A blocks t = 0..3 (rows wa + 32t + l%32),
// B blocks (rows wb + ...).
template <int CA, int CB, bool AMN, bool BMN, bool BF, int S>
__device__ __forceinline__ void read_frags(const uint8_t* ta, const uint8_t* tb, int wa, int wb, int lane,
                                           i32x8 (&fa)[4], i32x8 (&fb)[4]) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    fa[t] = read_frag<CA, AMN, BF>(ta, wa, t, S, lane);
    fb[t] = read_frag<CB, BMN, BF>(tb, wb, t, S, lane);
  }
}

// ---- exact-products route: operand elements times their scale as bf16 ----------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x6_t __attribute__((ext_vector_type(6)));
typedef unsigned u32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t bits2(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Elements 8j .. 8j + 7 of the lane's 32 (8-bit: dwords 2j, 2j + 1; 4-bit: dword j, low
// nibble first) times 2^(code - 127), as 8 bf16 (the operand of bf16 MFMA j). `sbits` is
// code << 23: the conversions take the scale from a float's exponent field.
template <int C, int J>
__device__ __forceinline__ uint4 cvt_part(const i32x8& v, uint32_t sbits) {
  const float s = __uint_as_float(sbits);
  if constexpr (C == 0) {
    const uint32_t w0 = (uint32_t)v[2 * J], w1 = (uint32_t)v[2 * J + 1];
    return make_uint4(bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true)));
  } else if constexpr (C == 1) {
    const uint32_t w0 = (uint32_t)v[2 * J], w1 = (uint32_t)v[2 * J + 1];
    return make_uint4(bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, s, false)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, s, true)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, s, false)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, s, true)));
  } else {
    static_assert(C == 4, "6-bit operands convert all 32 elements at once (cvt_all6)");
    const uint32_t w = (uint32_t)v[J];
    return make_uint4(bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                      bits2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3)));
  }
}

// All 32 elements of a 6-bit operand (dwords 0..5, element i at bits 6i..6i+5) times
// 2^(code - 127) as bf16, o[j] = elements 8j .. 8j + 7. Written as inline assembly with an
// early-clobber 16-register result: the compiler's builtin for these conversions let the
// result overlap live registers. The compiler does not know the assembly is a VALU write, so
// it ends with the 2 wait states an MFMA needs before reading VGPRs a VALU instruction wrote.
template <int C>
__device__ __forceinline__ void cvt_all6(const i32x8& v, uint32_t sbits, uint4 (&o)[4]) {
  const u32x6_t in = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3], (uint32_t)v[4], (uint32_t)v[5]};
  const float s = __uint_as_float(sbits);
  u32x16_t r;
  if constexpr (C == 2) asm volatile("v_cvt_scalef32_pk32_bf16_fp6 %0, %1, %2\n\ts_nop 1" : "=&v"(r) : "v"(in), "v"(s));
  else asm volatile("v_cvt_scalef32_pk32_bf16_bf6 %0, %1, %2\n\ts_nop 1" : "=&v"(r) : "v"(in), "v"(s));
#pragma unroll
  for (int j = 0; j < 4; j++) o[j] = make_uint4(r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]);
}

// One operand's converted fragments for the bf16 MFMAs. 8- and 4-bit operands convert one
// part j (elements 8j .. 8j + 7 of every block) at a time into buffer j & 1, ahead of its MFMAs,
// and part 0 of the next step during part 3 of the current one (PREFETCH); 6-bit operands
// convert whole blocks (all four parts) at the start of the step. The dwords a conversion
// reads are pinned in place first (an empty asm that claims to rewrite them), so it issues
// where it is written, between two MFMAs, rather than in a burst ahead of the step.
template <int C>
struct Conv {
  static constexpr bool WHOLE = fmt_bits(C) == 6;
  static constexpr bool PREFETCH = !WHOLE;
  uint4 p[WHOLE ? 4 : 2][WHOLE ? 4 : 1][4];   // WHOLE: [t][0][j]; else [j & 1][0][t]
  template <int J>
  __device__ __forceinline__ void prepare(i32x8 (&f)[4], const uint32_t (&sb)[4], int t) {
    if constexpr (WHOLE) {
      if (J == 0) cvt_all6<C>(f[t], sb[t], p[t][0]);
    } else {
      constexpr int D = C == 4 ? J : 2 * J;
      asm volatile("" : "+v"(f[t][D])::"memory");
      if constexpr (C != 4) asm volatile("" : "+v"(f[t][D + 1])::"memory");
      p[J & 1][0][t] = cvt_part<C, J>(f[t], sb[t]);
      gemm::pin_frag(p[J & 1][0][t]);
    }
  }
  template <int J>
  __device__ __forceinline__ const uint4& get(int t) const {
    if constexpr (WHOLE) return p[t][0][J];
    else return p[J & 1][0][t];
  }
};

// Scale operand of this lane's 32-K block in step S: byte 2S + h of the tile's word rotated into
// bits 23..30, a float's exponent field (rotate right by 8 (2S + h) + 9 = 16S + sh + 9, mod 32).
// The 2-element conversions read only that field (probed: sign and mantissa bits are ignored),
// so one rotate is the whole operand; the 32-element 6-bit conversions get the field alone.
template <int C, int S>
__device__ __forceinline__ void scale_bits(const uint32_t (&s)[4], int sh, uint32_t (&o)[4]) {
  const uint32_t r = (uint32_t)(16 * S + 9 + sh) & 31u;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint32_t x = __builtin_amdgcn_alignbit(s[t], s[t], r);
    o[t] = fmt_bits(C) == 6 ? (x & 0x7F800000u) : x;
  }
}

__device__ __forceinline__ f32x16 mfma_bf16(const uint4& b, const uint4& a, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a), c, 0, 0,
                                                 0);
}

// The scale operands of a step (xa, xb) and part 0 of its fragments for both operands (the
// prefetching formats), from raw fragments and the scale words of the step's tile.
template <int CA, int CB, int S>
__device__ __forceinline__ void prepare_first(Conv<CA>& ca, Conv<CB>& cb, i32x8 (&fa)[4], i32x8 (&fb)[4],
                                              const uint32_t (&sa)[4], const uint32_t (&sb)[4], int sh,
                                              uint32_t (&xa)[4], uint32_t (&xb)[4]) {
  scale_bits<CA, S>(sa, sh, xa);
  scale_bits<CB, S>(sb, sh, xb);
#pragma unroll
  for (int t = 0; t < 4; t++) {
    if constexpr (Conv<CA>::PREFETCH) ca.template prepare<0>(fa, xa, t);
    if constexpr (Conv<CB>::PREFETCH) cb.template prepare<0>(fb, xb, t);
  }
}

// The 64 bf16 MFMAs of 64-K step S (MFMA j of each accumulator covers elements 8j..8j+7 of
// the lanes' 32), j-major so that the conversions of part j + 1 go out between part j's
// MFMAs. The step's scale operands are in xa / xb and part 0 of its fragments in ca / cb
// (prefetching formats). With NEXT, part 3 replaces xa / xb with the next step's (step index
// SN of the tile whose scale words are nsa / nsb) and converts that step's part 0 (raw
// fragments nfa / nfb) between its MFMAs; nfa, nfb, nsa and nsb are read only then, so side
// work of this step may still be filling them. side(i) (i = 0..15) runs after every fourth
// MFMA, as mfma16 runs it after every one.
template <int CA, int CB, int S, bool NEXT, int SN, typename Side>
__device__ __forceinline__ void mfma64_bf(Conv<CA>& ca, Conv<CB>& cb, i32x8 (&fa)[4], i32x8 (&fb)[4],
                                          uint32_t (&xa)[4], uint32_t (&xb)[4], i32x8 (&nfa)[4], i32x8 (&nfb)[4],
                                          const uint32_t (&nsa)[4], const uint32_t (&nsb)[4], int sh,
                                          f32x16 (&acc)[4][4], Side side) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    if constexpr (!Conv<CA>::PREFETCH) ca.template prepare<0>(fa, xa, t);
    if constexpr (!Conv<CB>::PREFETCH) cb.template prepare<0>(fb, xb, t);
  }
  auto part = [&](auto jc) {
    constexpr int J = decltype(jc)::value;
    if constexpr (J == 3 && NEXT) {
      scale_bits<CA, SN>(nsa, sh, xa);
      scale_bits<CB, SN>(nsb, sh, xb);
    }
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int mt = i >> 2, nt = i & 3;
      asm volatile("" : "+a"(acc[mt][nt])::"memory");
      acc[mt][nt] = mfma_bf16(cb.template get<J>(nt), ca.template get<J>(mt), acc[mt][nt]);
      asm volatile("" : "+a"(acc[mt][nt])::"memory");
      if (i < 8) {
        if constexpr (J < 3) {
          if (i & 1) cb.template prepare<J + 1>(fb, xb, i >> 1);
          else ca.template prepare<J + 1>(fa, xa, i >> 1);
        } else if constexpr (NEXT) {
          if (i & 1) {
            if constexpr (Conv<CB>::PREFETCH) cb.template prepare<0>(nfb, xb, i >> 1);
          } else {
            if constexpr (Conv<CA>::PREFETCH) ca.template prepare<0>(nfa, xa, i >> 1);
          }
        }
      }
      if ((i & 3) == 3) side(4 * J + (i >> 2));
    }
  };
  part(std::integral_constant<int, 0>{});
  part(std::integral_constant<int, 1>{});
  part(std::integral_constant<int, 2>{});
  part(std::integral_constant<int, 3>{});
}

// All four parts (elements 8j .. 8j + 7, j < 4) of one fragment as bf16 times its scale.
template <int C>
__device__ __forceinline__ void cvt_whole(const i32x8& v, uint32_t sbits, uint4 (&o)[4]) {
  if constexpr (fmt_bits(C) == 6) {
    cvt_all6<C>(v, sbits, o);
  } else {
    o[0] = cvt_part<C, 0>(v, sbits);
    o[1] = cvt_part<C, 1>(v, sbits);
    o[2] = cvt_part<C, 2>(v, sbits);
    o[3] = cvt_part<C, 3>(v, sbits);
  }
}

// 64-K step S of the exact-products route with nothing in flight beside it, for the partial
// last K tile: each A fragment converted once, each B fragment once per A fragment, the four
// bf16 MFMAs of an accumulator in part order j = 0..3 as in mfma64_bf. Few registers live at
// once, so this code, which runs once per tile, does not raise the whole kernel's register
// pressure.
template <int CA, int CB, int S>
__device__ __forceinline__ void step_bf_plain(const i32x8 (&fa)[4], const i32x8 (&fb)[4], const uint32_t (&sa)[4],
                                              const uint32_t (&sb)[4], int sh, f32x16 (&acc)[4][4]) {
  uint32_t xa[4], xb[4];
  scale_bits<CA, S>(sa, sh, xa);
  scale_bits<CB, S>(sb, sh, xb);
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    uint4 pa[4];
    cvt_whole<CA>(fa[mt], xa[mt], pa);
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      uint4 pb[4];
      cvt_whole<CB>(fb[nt], xb[nt], pb);
#pragma unroll
      for (int j = 0; j < 4; j++) acc[mt][nt] = mfma_bf16(pb[j], pa[j], acc[mt][nt]);
    }
  }
}

// The 16 MFMAs of 64-K step S (accumulator rows mt-major). The MFMA takes B first (its
// format code and scales as src0); after the per-lane shift by 8 (l/32), op_sel byte 2S
// holds the scale of the lane's 32-K block of this step. side(i) runs after MFMA i: the
// empty asm statements around each MFMA (accumulators kept in AGPRs, memory clobbered)
// keep the side work - LDS reads and writes - between the MFMAs, where it overlaps the
// matrix pipe instead of waiting for it.
template <int CA, int CB, int S, typename Side>
__device__ __forceinline__ void mfma16(const i32x8 (&fa)[4], const i32x8 (&fb)[4], const uint32_t (&sa)[4],
                                       const uint32_t (&sb)[4], int sh, f32x16 (&acc)[4][4], Side side) {
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int mt = i >> 2, nt = i & 3;
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[nt], fa[mt], acc[mt][nt], CB, CA, 2 * S,
                                                                   (int)(sb[nt] >> sh), 2 * S, (int)(sa[mt] >> sh));
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    side(i);
  }
}

template <int CA, int CB, bool AMN, bool BMN, bool BF>
__global__ __launch_bounds__(256, 1) void k_gemm_mx_any(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Op<CA, AMN> PA;
  typedef Op<CB, BMN> PB;
  typedef Lay<CA, CB> L;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
  const int q = threadIdx.x, lane = q & 63, w = __builtin_amdgcn_readfirstlane(q >> 6);
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wa = 128 * (w >> 1), wb = 128 * (w & 1);
  const float sgn = a.negate ? -1.0f : 1.0f;
  const int64_t nblk = a.K / 32;
  const int64_t lda_b = a.lda * PA::BITS / 8, ldb_b = a.ldb * PB::BITS / 8;
  const int64_t ka = a.K * PA::BITS / 8, kb = a.K * PB::BITS / 8;   // a row's K extent in bytes
  // operand bases: the tile's first row (K-major) or its first M / N element (MN-major)
  const uint8_t* A = (const uint8_t*)a.A + (AMN ? m0 * PA::BITS / 8 : m0 * lda_b);
  const uint8_t* B = (const uint8_t*)a.B + (BMN ? n0 * PB::BITS / 8 : n0 * ldb_b);
  // bytes from one K tile to the next; the last chunk start inside an MN-major k-row
  const int64_t stepa = AMN ? 128 * lda_b : PA::ROW, stepb = BMN ? 128 * ldb_b : PB::ROW;
  const uint32_t mlima = (uint32_t)(lda_b - 16 - (AMN ? m0 * PA::BITS / 8 : 0));
  const uint32_t mlimb = (uint32_t)(ldb_b - 16 - (BMN ? n0 * PB::BITS / 8 : 0));
  const int64_t rows_a = a.M - m0, rows_b = a.N - n0;
  const int sh = 8 * (lane >> 5);

  f32x16 acc[4][4];
  gemm::zero_acc(acc);
  // Direct copies of one stage: NA (NB) 1 KiB copies for the A (B) tile, copy j going to
  // wave j % 4. A batch of copies (one per K tile) also carries a quarter of a scale group:
  // two 256-byte copies per wave, each 16 rows x 16 bytes.
  constexpr int NA = PA::TILE / 1024, NB = PB::TILE / 1024;
  constexpr int DA = NA / 4, DB = NB / 4, DD = DA + DB, DPW = DD + 2, NST = L::NST;
  uint32_t oa[DA], ob[DB];
  {
    // lane l of copy j lands at LDS chunk 64 (w + 4j) + l of the tile: row p / CPR, physical
    // chunk p % CPR, which holds the row's logical chunk `logical(...)`. K-major rows past
    // the operand re-read its last row; MN-major chunks past the row's end re-read its
    // last chunk.
    auto offs = [&](auto P, int64_t ld_bytes, int64_t rows, uint32_t mlim, int j) -> uint32_t {
      typedef decltype(P) PP;
      const int p = 64 * (w + 4 * j) + lane;
      const int r = p / PP::CPR, c = PP::logical(p - r * PP::CPR, r);
      if (PP::ROWS == 128) return (uint32_t)(r * ld_bytes) + min((uint32_t)(16 * c), mlim);
      return (uint32_t)(min((int64_t)r, rows - 1) * ld_bytes + 16 * c);
    };
#pragma unroll
    for (int j = 0; j < DA; j++) oa[j] = offs(PA{}, lda_b, rows_a, mlima, j);
#pragma unroll
    for (int j = 0; j < DB; j++) ob[j] = offs(PB{}, ldb_b, rows_b, mlimb, j);
  }
  const uint8_t* SA = a.SFA + m0 * a.ld_sfa;
  const uint8_t* SB = a.SFB + n0 * a.ld_sfb;
  uint64_t sSA, sSB;                       // the scale bases pinned once for the slice copies
  gemm::sgpr_base2(SA, SB, sSA, sSB);
  const uint32_t lds0 = gemm::lds_addr(lds);
  const int nfull = (int)(a.K / KT);
  // Data copy d (of DD) of tile kt into stage `stage`.
  auto copy = [&](int kt, int stage, int d) {
    const uint32_t st = lds0 + stage * L::STAGE;
    if (d < DA) gemm::dma16s(A + kt * stepa, oa[d], st + 1024 * (w + 4 * d));
    else gemm::dma16s(B + kt * stepb, ob[d - DA], st + PA::TILE + 1024 * (w + 4 * (d - DA)));
  };
  // Copy c (0, 1) of this wave for quarter j of scale group g (K tiles 4g .. 4g + 3):
  // rows 64j + 16p .. +15 of operand op (k = 2w + c: op = k / 4, p = k % 4), lane l moving
  // physical word l % 4 of row 64j + 16p + l / 4. Words of tiles past the last whole
  // tile re-read the last one, and rows past the operand its last row (unused values).
  auto slice = [&](int g, int j, int c) {
    const int k = 2 * w + c, op = k >> 2, R = 64 * j + 16 * (k & 3) + (lane >> 2);
    const int qw = (lane & 3) ^ ((R >> 4) & 3) ^ ((R >> 6) & 1) ^ (op ? 2 : 0);
    const int64_t rows = op ? rows_b : rows_a;
    const uint32_t off = (uint32_t)(min((int64_t)R, rows - 1) * (op ? a.ld_sfb : a.ld_sfa)) +
                         4u * (uint32_t)min(4 * g + qw, nfull - 1);
    gemm::dma4u(op ? sSB : sSA, off, lds0 + L::RING + (g & 1) * L::RING_BUF + op * 4096 + 16 * (64 * j + 16 * (k & 3)));
  };
  // Batch b (issued once tile b's stage has been read): quarter (b + 5) % 4 of scale group
  // (b + 5) / 4, then the data of tile kb into stage `stage`. Group g's buffer is free once
  // every wave has read the scales of tile 4g - 5 (before batch 4g - 5), and its quarters are
  // all in batches 4g - 5 .. 4g - 2, which have landed when tile 4g's scales are read.
  auto batch_copy = [&](int b, int kb, int stage, int d) {
    if (d < 2) slice((b + 5) >> 2, (b + 5) & 3, d);
    else copy(kb, stage, d - 2);
  };
  static_assert(DPW <= 32, "at most two copies per MFMA slot of step 1");
  // With three stages on the scaled-MFMA route a batch goes out in two halves: its scale
  // copies and the first DH data copies at every other MFMA slot of step 1 of iteration b,
  // the other DD - DH at every other slot of step 0 of iteration b + 1 (its stage is still
  // free then), so that the four waves' copies reach the shared copy path about one per 16
  // cycles instead of all within one step (measured: 6-bit pairs 4-8% faster). With two
  // stages the whole batch goes out in step 1 (a K tile would otherwise have only half a
  // tile of lead), and so it does on the exact-products route, whose K tiles last twice as
  // long (the split made it 1.5% slower).
  constexpr bool SPLIT = NST >= 3 && !BF;
  constexpr int DH = SPLIT ? DD / 2 : DD;
  static_assert(!SPLIT || (2 + DH <= 8 && DD - DH <= 8), "one copy per two MFMA slots");
  // Converted fragments and scale operands of the exact-products route (unused on the other).
  Conv<CA> cva;
  Conv<CB> cvb;
  uint32_t xsa[4], xsb[4];
  // Multiply the partial K tile, held in stage st with its scale words (one per row, A's then
  // B's) at `scales`, one step at a time with only that step's fragments live (the pipelined
  // form of the loop, with two steps' fragments and the conversion buffers live at once, made
  // the compiler spill accumulators around it).
  auto multiply = [&](const uint8_t* st, const uint8_t* scales) {
    uint32_t sa[4], sb[4];
    read_scales(scales, wa, lane, sa);
    read_scales(scales + 1024, wb, lane, sb);
    {
      i32x8 fa[4], fb[4];
      read_frags<CA, CB, AMN, BMN, BF, 0>(st, st + PA::TILE, wa, wb, lane, fa, fb);
      if constexpr (BF) step_bf_plain<CA, CB, 0>(fa, fb, sa, sb, sh, acc);
      else mfma16<CA, CB, 0>(fa, fb, sa, sb, sh, acc, [](int) {});
    }
    {
      i32x8 fa[4], fb[4];
      read_frags<CA, CB, AMN, BMN, BF, 1>(st, st + PA::TILE, wa, wb, lane, fa, fb);
      if constexpr (BF) step_bf_plain<CA, CB, 1>(fa, fb, sa, sb, sh, acc);
      else mfma16<CA, CB, 1>(fa, fb, sa, sb, sh, acc, [](int) {});
    }
  };

  // The partial K tile past the whole ones (K not a multiple of 128), loaded with zeros past
  // K, goes first, into the zeroed accumulators. Multiplied after the loop, it joined the
  // no-tail path just before the epilogue, and the compiler kept the accumulators in scratch
  // across that join on every tile, tail or not (for an 8192 x 8192 fp32 D, 144 MiB more
  // written per launch than D itself, and read back).
  if (a.K % KT) {
    uint4 va[PA::LPC], vb[PB::LPC];
    uint8_t* st = lds;
    if constexpr (AMN) {
      load_chunks_tail_mn<CA>(A, lda_b, mlima, nfull, a.K, q, va);
    } else {
      uint32_t roa[PA::LPC];
      row_offsets<CA>(lda_b, rows_a, q, roa);
      load_chunks_tail<CA>(A, roa, nfull, ka, q, va);
    }
    if constexpr (BMN) {
      load_chunks_tail_mn<CB>(B, ldb_b, mlimb, nfull, a.K, q, vb);
    } else {
      uint32_t rob[PB::LPC];
      row_offsets<CB>(ldb_b, rows_b, q, rob);
      load_chunks_tail<CB>(B, rob, nfull, kb, q, vb);
    }
    const uint32_t wsa = mask_scale_word(load_scale_word(a.SFA, a.ld_sfa, m0, a.M, q, nfull), nfull, nblk);
    const uint32_t wsb = mask_scale_word(load_scale_word(a.SFB, a.ld_sfb, n0, a.N, q, nfull), nfull, nblk);
    store_chunks<CA, AMN>(st, q, va);
    store_chunks<CB, BMN>(st + PA::TILE, q, vb);
    uint8_t* scales = lds + L::RING;          // one word per row: A's 256, then B's
    *(BSM_LDS uint32_t*)(scales + 4 * q) = wsa;
    *(BSM_LDS uint32_t*)(scales + 1024 + 4 * q) = wsb;
    __syncthreads();
    multiply(st, scales);
    __syncthreads();
  }
  // Whole K tiles; tile kt lives in stage kt % NST. One barrier per tile, at the start of
  // its step 1: every wave has then read the stage's step-1 fragments (issued between the
  // step-0 MFMAs) and the copies of tile kt + 1 have landed, so the copies of tile kt + NST
  // go into the stage just read and the scales and step-0 fragments of tile kt + 1 are read
  // between the step-1 MFMAs, ahead of their use. Past the last tile the copies re-read
  // the last tile into the stage just released (nobody reads it again), so every iteration
  // issues the same copies and the wait counts stay fixed; the last iteration's reads of
  // the next stage and ring buffer fetch values nobody uses.
  if (nfull > 0) {
    uint32_t sa[4], sb[4], na[4], nb[4];
    i32x8 fa0[4], fb0[4], fa1[4], fb1[4];
    // scale group 0 and the first quarter of group 1 (batches -5 .. -1), then the data of
    // tiles 0 .. NST - 1
#pragma unroll
    for (int j = 0; j < 4; j++) {
      slice(0, j, 0);
      slice(0, j, 1);
    }
    slice(1, 0, 0);
    slice(1, 0, 1);
#pragma unroll
    for (int i = 0; i < NST; i++)
#pragma unroll
      for (int d = 0; d < (i == NST - 1 ? DH : DD); d++) copy(min(i, nfull - 1), i, d);
    // the scales and tile 0 have landed (tiles 1 .. NST - 2 and the first DH copies of tile
    // NST - 1 may still fly; the rest of that tile goes out in iteration 0, as in every one)
    gemm::stage_barrier<(NST - 2) * DD + DH>();
    read_scales_ring(lds + L::RING, 0, 0, wa, lane, sa);
    read_scales_ring(lds + L::RING + 4096, 1, 0, wb, lane, sb);
    read_frags<CA, CB, AMN, BMN, BF, 0>(lds, lds + PA::TILE, wa, wb, lane, fa0, fb0);
    if constexpr (BF) prepare_first<CA, CB, 0>(cva, cvb, fa0, fb0, sa, sb, sh, xsa, xsb);
    int cur = 0;                             // kt % NST
    for (int kt = 0; kt < nfull; kt++) {
      const uint8_t* st = lds + cur * L::STAGE;
      const int nxt = cur + 1 == NST ? 0 : cur + 1;
      const uint8_t* nst = lds + nxt * L::STAGE;
      const int knext = min(kt + NST, nfull - 1);
      // the second half of the previous iteration's batch: tile kt - 1 + NST into its stage
      const int kprev = min(kt - 1 + NST, nfull - 1), prv = cur == 0 ? NST - 1 : cur - 1;
      auto side0 = [&](int i) {
        if (i < 8) {
          if (i & 1) fb1[i >> 1] = read_frag<CB, BMN, BF>(st + PA::TILE, wb, i >> 1, 1, lane);
          else fa1[i >> 1] = read_frag<CA, AMN, BF>(st, wa, i >> 1, 1, lane);
        }
        if constexpr (SPLIT) {
          if ((i & 1) && (i >> 1) < DD - DH) copy(kprev, prv, DH + (i >> 1));
        }
      };
      auto side1 = [&](int i) {
        if (i == 0) {
          // only the data copies of the batches after tile kt + 1's (tiles kt + 2 ..
          // kt + NST - 1) may still fly: every scale quarter issued so far has landed
          gemm::stage_barrier<(NST - 2) * DD>();
          const uint8_t* ring = lds + L::RING + (((kt + 1) >> 2) & 1) * L::RING_BUF;
          read_scales_ring(ring, 0, kt + 1, wa, lane, na);
          read_scales_ring(ring + 4096, 1, kt + 1, wb, lane, nb);
        }
        if (i < 8) {
          if (i & 1) fb0[i >> 1] = read_frag<CB, BMN, BF>(nst + PA::TILE, wb, i >> 1, 0, lane);
          else fa0[i >> 1] = read_frag<CA, AMN, BF>(nst, wa, i >> 1, 0, lane);
        }
        if constexpr (SPLIT) {
          if (!(i & 1) && (i >> 1) < 2 + DH) batch_copy(kt, knext, cur, i >> 1);
        } else {
          if (i < DPW) batch_copy(kt, knext, cur, i);
          if (i + 16 < DPW) batch_copy(kt, knext, cur, i + 16);   // two 8-bit operands: 18 copies
        }
      };
      if constexpr (BF) {
        // step 0 converts step 1's first part from fa1 / fb1 (read by side0), step 1 the next
        // tile's from fa0 / fb0 and its scale words na / nb (read by side1)
        mfma64_bf<CA, CB, 0, true, 1>(cva, cvb, fa0, fb0, xsa, xsb, fa1, fb1, sa, sb, sh, acc, side0);
        mfma64_bf<CA, CB, 1, true, 0>(cva, cvb, fa1, fb1, xsa, xsb, fa0, fb0, na, nb, sh, acc, side1);
      } else {
        mfma16<CA, CB, 0>(fa0, fb0, sa, sb, sh, acc, side0);
        mfma16<CA, CB, 1>(fa1, fb1, sa, sb, sh, acc, side1);
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        sa[t] = na[t];
        sb[t] = nb[t];
      }
      cur = nxt;
    }
  }
  gemm::wait_dma();                          // the repeated copies too, before LDS is reused
  __syncthreads();
  // (accumulation as a constant in each branch: the fresh-D path then holds no registers for
  // D's values, which made the compiler spill accumulators here)
  if (a.accum)
    gemm::store_tile_lines(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc, lds + 32768 * w, true, a.ew_op,
                           a.ew_scale, a.ew_bias);
  else
    gemm::store_tile_lines(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc, lds + 32768 * w, false, a.ew_op,
                           a.ew_scale, a.ew_bias);
}

// Launch of one (A format, B format, major orders) instance on the route the call asks for:
// exact products where the pairing needs them (wide_products), or the scaled MFMA when the
// call takes its accumulation window (a.mx_window, K-major operands only). Instances the tuned
// kernels of k_gemm_mx.hip cover (K-major E2M1 x E2M1, and K-major 8-bit x 8-bit on the
// scaled MFMA) and 6-bit MN-major operands are never compiled here: they report an invalid
// launch.
template <int CA, int CB, bool AMN, bool BMN, bool BF>
hipError_t launch_route(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t st) {
  constexpr bool tuned = !AMN && !BMN && ((CA == 4 && CB == 4) || (!BF && fmt_bits(CA) == 8 && fmt_bits(CB) == 8));
  constexpr bool fp6_mn = (AMN && fmt_bits(CA) == 6) || (BMN && fmt_bits(CB) == 6);
  if constexpr (tuned || fp6_mn) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((k_gemm_mx_any<CA, CB, AMN, BMN, BF>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_m,
                       tiles_n);
    return hipGetLastError();
  }
}

template <int CA, int CB, bool AMN, bool BMN>
hipError_t launch_pair(const GemmArgs& a, int tiles_m, int tiles_n, hipStream_t st) {
  constexpr bool wide = wide_products(CA, CB);
  if constexpr (!wide || AMN || BMN) {
    // one route: the scaled MFMA is exact for these formats, or the operands are MN-major
    // (the window route takes K-major operands only)
    if (a.mx_window && (AMN || BMN)) return hipErrorInvalidValue;
    return launch_route<CA, CB, AMN, BMN, wide>(a, tiles_m, tiles_n, st);
  } else {
    if (a.mx_window) return launch_route<CA, CB, AMN, BMN, false>(a, tiles_m, tiles_n, st);
    return launch_route<CA, CB, AMN, BMN, true>(a, tiles_m, tiles_n, st);
  }
}

// Every format pairing for fixed major orders.
template <bool AMN, bool BMN>
hipError_t launch_formats(const GemmArgs& a, hipStream_t st) {
  const int64_t tm64 = (a.M + BM - 1) / BM, tn64 = (a.N + BN - 1) / BN;
  if (tm64 * tn64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tm = (int)tm64, tn = (int)tn64;
  auto with_b = [&](auto ca) -> hipError_t {
    constexpr int CA = decltype(ca)::value;
    switch (mfma_code(a.dtype_b)) {
      case 0: return launch_pair<CA, 0, AMN, BMN>(a, tm, tn, st);
      case 1: return launch_pair<CA, 1, AMN, BMN>(a, tm, tn, st);
      case 2: return launch_pair<CA, 2, AMN, BMN>(a, tm, tn, st);
      case 3: return launch_pair<CA, 3, AMN, BMN>(a, tm, tn, st);
      default: return launch_pair<CA, 4, AMN, BMN>(a, tm, tn, st);
    }
  };
  switch (mfma_code(a.dtype)) {
    case 0: return with_b(std::integral_constant<int, 0>{});
    case 1: return with_b(std::integral_constant<int, 1>{});
    case 2: return with_b(std::integral_constant<int, 2>{});
    case 3: return with_b(std::integral_constant<int, 3>{});
    default: return with_b(std::integral_constant<int, 4>{});
  }
}

}  // namespace mxany
}  // namespace bsm
