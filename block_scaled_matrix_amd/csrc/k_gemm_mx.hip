// k_gemm_mx.hip - block-scaled GEMM (MXFP8 E4M3 or E5M2 / MXFP4 E2M1 with E8M0 scales per 32
// K elements) D = s * A * B^T (+ D) on gfx950 v_mfma_scale_f32_32x32x64_f8f6f4, K-major
// operands. The other pairings (6-bit formats, mixed widths) and MN-major operands go to
// the general kernel (gemm_mx_any.hpp; k_gemm_mx_any.hip, k_gemm_mx_mn_*.hip).
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
//    lines per row, the 128-byte-row XOR swizzle shared with the dense kernel) stream
//    HBM -> LDS with global_load_lds_dwordx4 into two stages;
//  - scale words reach LDS through a ring of two groups of 32 bytes per row (8 K tiles
//    of fp8, 4 of fp4), copied a slice per K tile with 8 rows per 4-byte-per-lane copy:
//    measured on the device, a copy whose 64 lanes touch 64 rows occupies the copy path
//    four times as long as a 1 KiB operand copy, one touching 8 rows 0.6 times as long;
//  - each wave reads a tile's fragments into registers early, so a stage is released
//    during the tile's first 64-K step and the copy of tile kt+2 starts while tile kt is
//    still being multiplied: two K tiles stay in flight;
//  - fragment reads, copies and barriers are placed one by one between the MFMAs: four
//    wave bursts of copies would block the issuing waves behind the shared copy path
//    while the matrix pipe idles, whereas one copy per 64-cycle fp8 MFMA (per two 32-cycle
//    fp4 MFMAs) keeps it fed in the background.
#include "gemm_common.hpp"
#include "../../include/bsm.h"

namespace bsm {
namespace {

constexpr int BM = 256, BN = 256;
constexpr int ROWB = 128;                  // bytes of K per row per K tile
constexpr int TILE_BYTES = 256 * ROWB;     // 32 KiB per operand tile
constexpr int STAGE = 2 * TILE_BYTES;      // A tile, B tile
static_assert(TILE_BYTES == gemm::kKTileBytes, "K-major tile geometry");
// Scale ring: two group buffers (A, B) of 256 rows x 32 bytes after the two stages.
constexpr int RING = 2 * STAGE;
constexpr int RING_OP = 256 * 32;
constexpr int RING_GROUP = 2 * RING_OP;
constexpr int LDS_BYTES = RING + 2 * RING_GROUP;  // 160 KiB

template <int FMT>
struct Fmt {
  static constexpr int KT = FMT == 4 ? 256 : 128;  // K elements per K tile
  static constexpr int STEPS = FMT == 4 ? 4 : 2;   // 64-K MFMA steps per K tile
  static constexpr int EPB = FMT == 4 ? 2 : 1;     // elements per byte
  static constexpr int SFW = FMT == 4 ? 2 : 1;     // scale words per row per K tile
  static constexpr int G = 8 / SFW;                // K tiles per scale group (32 bytes of a row)
  static constexpr int SLICE_ROWS = 256 / G;       // rows of each operand's group copied per K tile
  static constexpr int SLICE_COPIES = 2 * SLICE_ROWS / 8 / 4;  // per wave per K tile (8 rows a copy)
  static constexpr int DMA_PER_TILE = 16 + SLICE_COPIES;
};

struct Ops {
  const uint8_t* A; uint32_t aoff[8];
  const uint8_t* B; uint32_t boff[8];
  const uint8_t* SFA; uint32_t ld_sfa; int lim_a;  // lim: last valid tile row (<= 255)
  const uint8_t* SFB; uint32_t ld_sfb; int lim_b;
  uint64_t sfa, sfb;                               // SFA, SFB as pinned copy bases (gemm::sgpr_base2)
  int ldw;                                         // scale words per row that may be read
};

// Copy d of the 16 operand copies of one K tile (8 of A, then 8 of B) into `stage`, from the
// tile's A and B bases pinned together (gemm::sgpr_base2).
__device__ __forceinline__ void issue_data(const Ops& o, uint64_t ga, uint64_t gb, int d, uint32_t stage, int w) {
  if (d < 8) gemm::dma16u(ga, o.aoff[d], stage + 1024 * (w + 4 * d));
  else gemm::dma16u(gb, o.boff[d - 8], stage + TILE_BYTES + 1024 * (w + 4 * (d - 8)));
}

// Scale ring. Row R of an operand's group buffer holds the 8 scale words of K tiles
// G g .. G g + G - 1 (SFW words per tile) as four 8-byte pairs, read with one 64-bit read
// each: pair P (words 2P, 2P + 1: an E2M1 tile's two words, or the words of two
// consecutive 8-bit tiles) at physical pair P ^ s2(R), s2(R) = ((R >> 3) & 3) ^ 2 ((R >> 6)
// & 1), so the 32 rows one wave reads per block land in distinct bank pairs, and so do the
// pairs of rows 64 apart (blocks t and t + 2, 2 KiB apart), which the compiler may fetch
// with one two-address read.
__device__ __forceinline__ int ring_s2(int R) { return ((R >> 3) & 3) ^ (((R >> 6) & 1) << 1); }
// Group g lives in buffer g & 1 and is copied in G slices of SLICE_ROWS rows per
// operand, one slice per K tile while group g - 1 is in use. Copy c of this wave for
// slice j of group g: 8 rows, lane l -> row 8 (l / 8) + ..., physical word l % 8.
template <int FMT>
__device__ __forceinline__ void issue_slice(const Ops& o, int g, int j, int c, uint32_t ring, int w, int lane) {
  typedef Fmt<FMT> F;
  constexpr int PER_OP = F::SLICE_ROWS / 8;
  const int k = w * F::SLICE_COPIES + c;
  const int op = k / PER_OP, ii = k % PER_OP;
  const int R = j * F::SLICE_ROWS + 8 * ii + (lane >> 3);
  const int p = lane & 7;  // physical word
  const int q = 2 * ((p >> 1) ^ ring_s2(R)) + (p & 1);
  const uint32_t word = (uint32_t)min(8 * g + q, o.ldw - 1);
  const uint64_t base = op ? o.sfb : o.sfa;
  const uint32_t off = (uint32_t)min(R, op ? o.lim_b : o.lim_a) * (op ? o.ld_sfb : o.ld_sfa) + 4 * word;
  gemm::dma4u(base, off, ring + (g & 1) * RING_GROUP + op * RING_OP + 32 * (j * F::SLICE_ROWS + 8 * ii));
}

// Raw scale words for this lane's rows (wave base + 32t + l%32): the pair holding K tile kt's
// words, [t][0] and [t][1]: for E2M1 the tile's two words, for 8-bit operands (kt even) the
// words of tiles kt and kt + 1.
template <int FMT>
__device__ __forceinline__ void read_scales(const uint8_t* lds, int kt, int wa, int wb, int lane, uint32_t (&sa)[4][2],
                                            uint32_t (&sb)[4][2]) {
  typedef Fmt<FMT> F;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const uint8_t* buf = lds + RING + ((kt / F::G) & 1) * RING_GROUP;
  const int r = lane & 31;
  const int P = FMT == 4 ? kt % F::G : (kt % F::G) >> 1;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    // s2(R) for rows R = wave base (0 or 128) + 32t + r
    const int s2 = ((r >> 3) & 3) ^ (((t >> 1) & 1) << 1);
    const uint32_t o = 32 * (32 * t + r) + 8 * (P ^ s2);
    const u32x2 x = *(const BSM_LDS u32x2*)(buf + 32 * wa + o);
    const u32x2 y = *(const BSM_LDS u32x2*)(buf + RING_OP + 32 * wb + o);
    sa[t][0] = x[0]; sa[t][1] = x[1];
    sb[t][0] = y[0]; sb[t][1] = y[1];
  }
}

// Scale words of a partial last K tile, word-major at `area` (word q of row r at 1024q + 4r,
// B after SFW KiB).
template <int FMT>
__device__ __forceinline__ void read_scales_wm(const uint8_t* area, int wa, int wb, int lane, uint32_t (&sa)[4][2],
                                               uint32_t (&sb)[4][2]) {
  typedef Fmt<FMT> F;
#pragma unroll
  for (int q = 0; q < F::SFW; q++)
#pragma unroll
    for (int t = 0; t < 4; t++) {
      sa[t][q] = *(const BSM_LDS uint32_t*)(area + 1024 * q + 4 * (wa + 32 * t + (lane & 31)));
      sb[t][q] = *(const BSM_LDS uint32_t*)(area + 1024 * F::SFW + 1024 * q + 4 * (wb + 32 * t + (lane & 31)));
    }
}

// Fragments of one 64-K step for one wave: af/bf[t][0..1] are the 16-byte chunks of
// 32-row block t (fp4 uses [t][0] only).
struct Frags {
  uint4 af[4][2], bf[4][2];
};

// LDS read r of the fragments of 64-K step s of the tile at `st`: fp8 has 16 reads per step
// (r: operand r / 8, block (r / 2) % 4, chunk r % 2), fp4 8 (operand r / 4, block r % 4).
// The lane's row within a 32-row block is l%32; fp8 step s covers bytes 64s.. of the row:
// logical chunks 4s + l/32 (k 16(l/32)..) and 4s + 2 + l/32 (k 32 + 16(l/32)..); fp4 step
// s covers bytes 32s..: logical chunk 2s + l/32.
template <int FMT>
__device__ __forceinline__ void read_frag(const uint8_t* st, int s, int r, int wa, int wb, int lane, Frags& f) {
  const int h = lane >> 5;
  if (FMT == 4) {
    const int op = r >> 2, t = r & 3;
    const uint8_t* p = st + op * TILE_BYTES + (op ? wb : wa) * ROWB + 4096 * t;
    const uint4 v = lds_read_b128(p + gemm::kmajor_frag_base(lane, 2 * s + h));
    if (op) f.bf[t][0] = v; else f.af[t][0] = v;
  } else {
    const int op = r >> 3, t = (r >> 1) & 3, c = r & 1;
    const uint8_t* p = st + op * TILE_BYTES + (op ? wb : wa) * ROWB + 4096 * t;
    const uint4 v = lds_read_b128(p + gemm::kmajor_frag_base(lane, 4 * s + 2 * c + h));
    if (op) f.bf[t][c] = v; else f.af[t][c] = v;
  }
}

template <int FMT>
__device__ __forceinline__ void read_frags(const uint8_t* st, int s, int wa, int wb, int lane, Frags& f) {
#pragma unroll
  for (int r = 0; r < (FMT == 4 ? 8 : 16); r++) read_frag<FMT>(st, s, r, wa, wb, lane, f);
}

// FMT: the operand layout (0: one byte per element, 4: fp4); CA, CB: the MFMA format codes
// of A and B (0 E4M3, 1 E5M2, 4 E2M1). The MFMA takes B first (cbsz = B's code).
template <int FMT, int CA, int CB, int SEL>
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
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, c, CB, CA, SEL, (int)sb, SEL, (int)sa);
}

template <int FMT>
__device__ __forceinline__ void pin_frags(Frags& f) {
#pragma unroll
  for (int t = 0; t < 4; t++) {
    gemm::pin_frag(f.af[t][0]);
    gemm::pin_frag(f.bf[t][0]);
    if (FMT != 4) {
      gemm::pin_frag(f.af[t][1]);
      gemm::pin_frag(f.bf[t][1]);
    }
  }
}

// The 16 MFMAs of 64-K step S (accumulator rows mt-major), scale word S / 2 of each row
// (after the per-lane shift), byte 2 (S & 1) (op_sel); side(i) runs after MFMA i, so that
// LDS reads, copies and barriers issue while the matrix pipe is busy. Empty asm
// "rewrites" of each accumulator before and after its MFMA fix the order of the MFMAs and
// the side operations (all volatile) without any hardware wait.
template <int FMT, int CA, int CB, int S, typename Side>
__device__ __forceinline__ void mfma_step_il(const Frags& f, const uint32_t (&sa)[4][2], const uint32_t (&sb)[4][2],
                                             f32x16 (&acc)[4][4], Side side) {
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int mt = i >> 2, nt = i & 3;
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    acc[mt][nt] = mfma_sc<FMT, CA, CB, 2 * (S & 1)>(f.bf[nt], f.af[mt], acc[mt][nt], sb[nt][S >> 1], sa[mt][S >> 1]);
    asm volatile("" : "+a"(acc[mt][nt])::"memory");
    side(i);
  }
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

template <int FMT, int CA, int CB, bool ACC>
__global__ __launch_bounds__(256, 1) void k_gemm_mx(GemmArgs a, int tiles_m, int tiles_n) {
  typedef Fmt<FMT> F;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  gemm::tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nblk = a.K / 32;
  const int wa = 128 * wm, wb = 128 * wn;
  const float sgn = a.negate ? -1.0f : 1.0f;

  // accumulators start from zero; the epilogue adds D when accumulating
  f32x16 acc[4][4];
  gemm::zero_acc(acc);

  Ops o;
  const int64_t lda_b = a.lda / F::EPB, ldb_b = a.ldb / F::EPB;
  o.A = (const uint8_t*)a.A + m0 * lda_b;
  o.B = (const uint8_t*)a.B + n0 * ldb_b;
  gemm::kmajor_dma_offsets(lda_b, m0, a.M, w, lane, o.aoff);
  gemm::kmajor_dma_offsets(ldb_b, n0, a.N, w, lane, o.boff);
  o.SFA = a.SFA + m0 * a.ld_sfa;
  o.SFB = a.SFB + n0 * a.ld_sfb;
  o.ld_sfa = (uint32_t)a.ld_sfa;
  o.ld_sfb = (uint32_t)a.ld_sfb;
  o.lim_a = (int)min(a.M - 1 - m0, (int64_t)255);
  o.lim_b = (int)min(a.N - 1 - n0, (int64_t)255);
  o.ldw = (int)(min(a.ld_sfa, a.ld_sfb) / 4);
  gemm::sgpr_base2(o.SFA, o.SFB, o.sfa, o.sfb);

  const int nfull = (int)(a.K / F::KT);
  const int tail = (int)(a.K % F::KT);
  const uint32_t lds0 = gemm::lds_addr(lds);
  const uint32_t ring = lds0 + RING;
  const int h8 = 8 * (lane >> 5);
  Frags f0, f1, f2, f3;
  uint32_t sa[4][2], sb[4][2], ra[4][2], rb[4][2];
  if (nfull > 0) {
    // scale group 0 whole and slice 0 of group 1, then K tiles 0 and 1
#pragma unroll
    for (int j = 0; j < F::G; j++)
#pragma unroll
      for (int c = 0; c < F::SLICE_COPIES; c++) issue_slice<FMT>(o, 0, j, c, ring, w, lane);
#pragma unroll
    for (int c = 0; c < F::SLICE_COPIES; c++) issue_slice<FMT>(o, 1, 0, c, ring, w, lane);
    const int k1 = min(1, nfull - 1);
    uint64_t sa0, sb0, sa1, sb1;
    gemm::sgpr_base2(o.A, o.B, sa0, sb0);
#pragma unroll
    for (int d = 0; d < 16; d++) issue_data(o, sa0, sb0, d, lds0, w);
    gemm::sgpr_base2(o.A + k1 * ROWB, o.B + k1 * ROWB, sa1, sb1);
#pragma unroll
    for (int d = 0; d < 16; d++) issue_data(o, sa1, sb1, d, lds0 + STAGE, w);
    gemm::stage_barrier<16>();
    read_frags<FMT>(lds, 0, wa, wb, lane, f0);
    read_scales<FMT>(lds, 0, wa, wb, lane, ra, rb);
    shift_scales<FMT>(ra, rb, h8, sa, sb);
  }
  // K tile kt lives in stage kt & 1; f0 holds its first 64-K step and sa/sb its scales
  // when iteration kt starts. Each iteration: the fragment reads of the tile's other steps
  // go out over the first MFMAs; one barrier once every wave's reads of the stage are done
  // (then it takes the copies of tile kt + 2 and its share of the next scale group,
  // spread one per MFMA slot or two); a second barrier once this wave's copies of tile
  // kt + 1 have landed (then the step-0 fragments and the scales of tile kt + 1 are read).
  // The body is branch-free: past the last tile the copies re-read the last tile (clamped
  // index) into a stage nobody reads again, and the scale copies re-read the last words.
  for (int kt = 0; kt < nfull; kt++) {
    const uint8_t* st = lds + (kt & 1) * STAGE;
    const uint8_t* nst = lds + ((kt + 1) & 1) * STAGE;
    const uint32_t stage = lds0 + (kt & 1) * STAGE;
    const int64_t k2 = (int64_t)min(kt + 2, nfull - 1) * ROWB;
    uint64_t ga, gb;
    gemm::sgpr_base2(o.A + k2, o.B + k2, ga, gb);
    const int sg = (kt + 1) / F::G + 1, sj = (kt + 1) % F::G;
    // copy d of this iteration: operand copies 0..15, then the scale slice copies
    auto copy = [&](int d) {
      if (d < 16) issue_data(o, ga, gb, d, stage, w);
      else issue_slice<FMT>(o, sg, sj, d - 16, ring, w, lane);
    };
    if constexpr (FMT == 4) {
      // 64 MFMA slots of 32 cycles: step 0 (slots 0..15) reads steps 1..3 (two a slot);
      // barrier at slot 24, once the LDS has served those reads; copies at even slots
      // 24..62; barrier at slot 48 (12 copies issued); the next tile's step-0 fragments
      // and scales at slots 48..55
      pin_frags<4>(f0);
      mfma_step_il<4, CA, CB, 0>(f0, sa, sb, acc, [&](int i) {
        if (i < 12) {
#pragma unroll
          for (int rr = 0; rr < 2; rr++) {
            const int r = 2 * i + rr;  // step 1 + r / 8, read r % 8
            Frags& dst = r < 8 ? f1 : (r < 16 ? f2 : f3);
            read_frag<4>(st, 1 + r / 8, r & 7, wa, wb, lane, dst);
          }
        }
      });
      pin_frags<4>(f1);
      mfma_step_il<4, CA, CB, 1>(f1, sa, sb, acc, [&](int i) {
        if (i == 7) gemm::lds_barrier();
        if (i >= 8 && (i & 1) == 0) copy((i - 8) >> 1);
      });
      pin_frags<4>(f2);
      mfma_step_il<4, CA, CB, 2>(f2, sa, sb, acc, [&](int i) {
        if ((i & 1) == 0) copy(4 + (i >> 1));
      });
      pin_frags<4>(f3);
      mfma_step_il<4, CA, CB, 3>(f3, sa, sb, acc, [&](int i) {
        if (i == 0) gemm::stage_barrier<12>();
        if ((i & 1) == 0) copy(12 + (i >> 1));
        if (i == 0) read_scales<4>(lds, kt + 1, wa, wb, lane, ra, rb);
        if (i < 8) read_frag<4>(nst, 0, i, wa, wb, lane, f0);
      });
      shift_scales<4>(ra, rb, h8, sa, sb);
    } else {
      // 32 MFMA slots of 64 cycles: step 0 reads step 1 at slots 0..3 (four a slot);
      // barrier after slot 9; copies at slots 10..27; barrier at slot 20 (10 copies
      // issued); the next tile's step-0 fragments and scales at slots 20..27
      pin_frags<0>(f0);
      mfma_step_il<0, CA, CB, 0>(f0, sa, sb, acc, [&](int i) {
        if (i < 4) {
#pragma unroll
          for (int rr = 0; rr < 4; rr++) read_frag<0>(st, 1, 4 * i + rr, wa, wb, lane, f1);
        }
        if (i == 9) gemm::lds_barrier();
        if (i >= 10) copy(i - 10);
      });
      pin_frags<0>(f1);
      mfma_step_il<0, CA, CB, 1>(f1, sa, sb, acc, [&](int i) {
        if (i == 4) gemm::stage_barrier<10>();
        if (i < 12) copy(6 + i);
        // tile kt + 1's words: one pair read serves tiles kt + 1 (even) and kt + 2
        if (i == 4) {
          if (((kt + 1) & 1) == 0) {
            read_scales<0>(lds, kt + 1, wa, wb, lane, ra, rb);
          } else {
#pragma unroll
            for (int t = 0; t < 4; t++) {
              ra[t][0] = ra[t][1];
              rb[t][0] = rb[t][1];
            }
          }
        }
        if (i >= 4 && i < 12) {
          read_frag<0>(nst, 0, 2 * (i - 4), wa, wb, lane, f0);
          read_frag<0>(nst, 0, 2 * (i - 4) + 1, wa, wb, lane, f0);
        }
      });
      shift_scales<0>(ra, rb, h8, sa, sb);
    }
  }
  // Every copy has landed and every wave is done with LDS before stage 0 is refilled
  // (and before the workgroup can end with copies in flight).
  gemm::stage_barrier<0>();
  if (tail) {
    const int64_t kb0 = (int64_t)nfull * ROWB;
    const int64_t kb_end = a.K / F::EPB;
    gemm::kmajor_fill_masked((const uint8_t*)a.A, lda_b, m0, a.M, kb0, kb_end, lds, w, lane);
    gemm::kmajor_fill_masked((const uint8_t*)a.B, ldb_b, n0, a.N, kb0, kb_end, lds + TILE_BYTES, w, lane);
    uint8_t* area = lds + STAGE;
#pragma unroll
    for (int q = 0; q < F::SFW; q++) {
      // scale word q of the partial tile; blocks at or past nblk (beyond K) become 127
      // (2^0): their operand bytes are zero, and a NaN code in the row padding must not
      // poison them. A word wholly past the row's blocks is not read.
      const int64_t blk = ((int64_t)nfull * F::SFW + q) * 4;
      const int64_t valid = nblk - blk;
      const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : (1u << (8 * valid)) - 1u);
      const int ra_row = min(64 * w + lane, o.lim_a), rb_row = min(64 * w + lane, o.lim_b);
      uint32_t wa_ = 0x7F7F7F7Fu, wb_ = 0x7F7F7F7Fu;
      if (valid > 0) {
        wa_ = (*(const uint32_t*)(o.SFA + (int64_t)ra_row * a.ld_sfa + blk) & keep) | (0x7F7F7F7Fu & ~keep);
        wb_ = (*(const uint32_t*)(o.SFB + (int64_t)rb_row * a.ld_sfb + blk) & keep) | (0x7F7F7F7Fu & ~keep);
      }
      *(BSM_LDS uint32_t*)(area + 1024 * q + 256 * w + 4 * lane) = wa_;
      *(BSM_LDS uint32_t*)(area + 1024 * F::SFW + 1024 * q + 256 * w + 4 * lane) = wb_;
    }
    __syncthreads();
    // 64-K steps of the partial tile: steps past K see zero operands (and unit scales)
    // and add exact zeros. A counted loop keeps the accumulators in place across the
    // optional work.
    const int steps = (tail + 63) / 64;
    for (int s = 0; s < steps; s++) {
      read_frags<FMT>(lds, s, wa, wb, lane, f0);
      read_scales_wm<FMT>(area, wa, wb, lane, ra, rb);
      const int sh = h8 + 16 * (s & 1);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        sa[t][0] = __builtin_amdgcn_readfirstlane(s >> 1) ? ra[t][1] >> sh : ra[t][0] >> sh;
        sb[t][0] = __builtin_amdgcn_readfirstlane(s >> 1) ? rb[t][1] >> sh : rb[t][0] >> sh;
      }
      mfma_step_il<FMT, CA, CB, 0>(f0, sa, sb, acc, [](int) {});
    }
  }
  // every wave is done with LDS before the accumulators pass through it
  __syncthreads();
  gemm::store_tile_lines(a.D, a.ldd, a.M, a.N, m0 + wa, n0 + wb, lane, sgn, acc, lds + 32768 * w, ACC, a.ew_op,
                         a.ew_scale, a.ew_bias);
}

}  // namespace

hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t st) {
  if (a.K == 0) return launch_empty_gemm(a.D, a.ldd, a.M, a.N, a.accum, a.ew_op, a.ew_scale, a.ew_bias, st);
  const bool byte_a = a.dtype == BSM_E4M3 || a.dtype == BSM_E5M2, byte_b = a.dtype_b == BSM_E4M3 || a.dtype_b == BSM_E5M2;
  if (!a.a_kmajor && !a.b_kmajor) return launch_gemm_mx_mn_ab(a, st);
  if (!a.a_kmajor) return launch_gemm_mx_mn_a(a, st);
  if (!a.b_kmajor) return launch_gemm_mx_mn_b(a, st);
  if (!(byte_a && byte_b) && !(a.dtype == BSM_E2M1 && a.dtype_b == BSM_E2M1)) return launch_gemm_mx_any(a, st);
  // 8-bit pairs sum exactly only through the general kernel's bf16 route; this kernel's
  // scaled fp8 MFMA serves calls that take its accumulation window
  if (byte_a && byte_b && !a.mx_window) return launch_gemm_mx_any(a, st);
  const int64_t tm64 = (a.M + BM - 1) / BM, tn64 = (a.N + BN - 1) / BN;
  if (tm64 * tn64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int tiles_m = (int)tm64, tiles_n = (int)tn64;
  const dim3 grid(tiles_m * tiles_n);
  // MFMA format codes: E4M3 0, E5M2 1, E2M1 4 (fp4 pairs only with fp4)
#define BSM_MX_LAUNCH(FMT, CA, CB)                                                                              \
  do {                                                                                                            \
    if (a.accum) hipLaunchKernelGGL((k_gemm_mx<FMT, CA, CB, true>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);  \
    else hipLaunchKernelGGL((k_gemm_mx<FMT, CA, CB, false>), grid, dim3(256), 0, st, a, tiles_m, tiles_n);         \
  } while (0)
  const bool a5 = a.dtype == BSM_E5M2, b5 = a.dtype_b == BSM_E5M2;
  if (a.dtype == BSM_E2M1) BSM_MX_LAUNCH(4, 4, 4);
  else if (!a5 && !b5) BSM_MX_LAUNCH(0, 0, 0);
  else if (a5 && b5) BSM_MX_LAUNCH(0, 1, 1);
  else if (a5) BSM_MX_LAUNCH(0, 1, 0);
  else BSM_MX_LAUNCH(0, 0, 1);
#undef BSM_MX_LAUNCH
  return hipGetLastError();
}

}  // namespace bsm
