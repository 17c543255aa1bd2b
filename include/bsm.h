/* bsm.h - block-scaled tile-matrix kernels for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsm.so. Every entry point:
 *   - takes plain host structs, plain device pointers and sizes (no framework types);
 *   - checks the whole call contract on the host first; on a violation it returns a
 *     negative bsm_status, records a message for bsm_last_error() and launches nothing;
 *   - otherwise enqueues its kernels on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and returns BSM_OK without synchronising;
 *   - never allocates, frees or keeps a pointer after it returns (other than in
 *     the enqueued work). The caller owns every buffer, keeps it alive until the
 *     stream work completes, and owns all synchronisation;
 *   - enqueues kernels only (no memory copy, memset or host synchronisation), so a
 *     sequence of calls may be captured into a HIP graph on a capturing stream and
 *     replayed; the first box-copy call on a device must run outside a capture (it
 *     sets a kernel attribute once per device).
 * Device faults surface asynchronously at the caller's next synchronisation.
 *
 * Pages cited (web documentation of Apache TVM "TIRx"):
 *   [TP]  "Explicit CUDA tile patterns"
 *   [TMA] "cp.async.bulk.tensor / cp.reduce.async.bulk.tensor"
 *   [LDM] "ldmatrix / stmatrix"
 *   [TOE] "Tile Operands and Execution"
 *   [MMA] "tcgen05.mma"
 * Storage formats follow the OCP Microscaling Formats (MX) v1.0 specification.
 */
#ifndef BSM_H
#define BSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element storage formats. */
typedef enum bsm_dtype {
  BSM_U8 = 0, BSM_U16 = 1, BSM_U32 = 2,
  BSM_F16 = 3,   /* IEEE binary16 */
  BSM_BF16 = 4,  /* bfloat16 */
  BSM_F32 = 5,   /* IEEE binary32 */
  BSM_E4M3 = 6,  /* OCP fp8 E4M3 ("fn": no infinities, 0x7F/0xFF NaN, max 448) */
  BSM_E2M1 = 7,  /* OCP fp4 E2M1, two per byte, even element in the low nibble */
  BSM_E8M0 = 8,  /* OCP 8-bit power-of-two scale: 2^(code-127), 0xFF NaN */
  BSM_E5M2 = 9,  /* OCP fp8 E5M2 (IEEE-like: infinities, NaNs; max 57344) */
  BSM_E2M3 = 10, /* OCP fp6 E2M3 (max 7.5), packed: element i at bits 6i..6i+5, little-endian */
  BSM_E3M2 = 11  /* OCP fp6 E3M2 (max 28), packed like E2M3 */
} bsm_dtype;

/* Status codes: one per violated rule. */
typedef enum bsm_status {
  BSM_OK = 0,
  BSM_E_NULL = -1,     /* a required pointer is NULL */
  BSM_E_RANK = -2,     /* rank not in 1..5, or box rank != tensor rank */
  BSM_E_BOX = -3,      /* a box extent not in 1..256, or an image larger than 160 KiB */
  BSM_E_ESTRIDE = -4,  /* an element stride not in 1..8, or the inner one != 1 */
  BSM_E_ALIGN = -5,    /* base / stride / leading-dimension / image alignment */
  BSM_E_SWIZZLE = -6,  /* swizzle not in 0..3, or inner image row not allowed for it */
  BSM_E_FILL = -7,     /* oob_fill not 0/1, or NaN fill on a format without NaN */
  BSM_E_DTYPE = -8,    /* storage format not supported by this call */
  BSM_E_SHAPE = -9,    /* negative size, dimension out of range, K not a block multiple */
  BSM_E_MAJOR = -10,   /* major-order selector not recognised */
  BSM_E_ALIAS = -11,   /* an output overlaps an input it must not overlap */
  BSM_E_HIP = -12,     /* the HIP runtime reported an error at launch */
  BSM_E_ARG = -13      /* any other out-of-contract argument (flags not 0/1, ...) */
} bsm_status;

/* A rectangular global tensor view ([TMA] "Operand specification": rank, shape and
 * outer byte strides of the global operand, unit innermost stride).
 *   base:    device pointer, 16-byte aligned;
 *   dtype:   a bsm_dtype of whole bytes (E2M1 data is viewed as U8);
 *   rank:    1..5;
 *   dims:    extents, outer to inner, each 1..2^31-1;
 *   strides: byte strides, outer to inner; strides[rank-1] == element size; every
 *            outer stride a positive multiple of 16.
 * Element (g_0..g_{r-1}) lives at base + sum_i g_i * strides[i]. */
typedef struct bsm_tensor {
  void* base;
  int32_t dtype;
  int32_t rank;
  int64_t dims[5];
  int64_t strides[5];
} bsm_tensor;

/* A box and its shared-memory image ([TMA] "Call parameters", "Data representation";
 * [TP] "TMA").
 *   box:             extents outer to inner, each 1..256;
 *   element_strides: sampling steps outer to inner, each 1..8, the inner one 1;
 *   swizzle:         0/1/2/3 = none / 32 B / 64 B / 128 B;
 *   oob_fill:        0 = zero, 1 = canonical NaN (F32, F16, BF16, E4M3, E5M2 only; the
 *                    E5M2 NaN is 0x7E, the top byte of binary16's 0x7E00).
 * The image has extents n_i = ceil(box_i / element_strides_i), is compact row-major
 * (outer to inner) before swizzling, and image element j holds global coordinate
 * coords + j * element_strides (the fill value if any coordinate is outside
 * [0, dims)). Byte offset o of the compact image is stored at swizzle(o), where
 * swizzle(o) = o ^ ((o >> 3) & m) with m = 0, 16, 48, 112 for modes 0..3 ([TP]
 * "Shared matrix descriptors" gives mode 3; modes 1 and 2 take the same form over
 * their 256- and 512-byte periods). The inner image row (n_inner * element size)
 * must be a multiple of 16 bytes and, when swizzled, at most 16 << swizzle bytes;
 * the whole image must fit in 160 KiB (one workgroup's LDS). */
typedef struct bsm_box {
  int32_t rank;
  int32_t box[5];
  int32_t element_strides[5];
  int32_t swizzle;
  int32_t oob_fill;
} bsm_box;

/* Bytes one image occupies in an image buffer: the compact image rounded up to
 * 128 bytes ([TMA] "Operand specification": every atom origin is 128-byte aligned)
 * or, when swizzled, to the whole period 2^(7+swizzle). Returns a negative status
 * for an invalid box or dtype. */
int64_t bsm_image_stride(const bsm_box* box, int32_t dtype);

/* Box load, global -> image ([TMA] "Call parameters", "Operand specification",
 * "Example: two explicit 8x16 boxes").
 *   src:        the global tensor;
 *   coords_dev: DEVICE array of n_boxes * rank int32 starting coordinates, box t's
 *               coordinates at [t*rank .. t*rank+rank), outer to inner; any value,
 *               out-of-range elements take the fill;
 *   images:     DEVICE buffer, n_boxes * bsm_image_stride() bytes, aligned to 128
 *               bytes (to the swizzle period when swizzled); image t at
 *               t * bsm_image_stride(); padding bytes between images are not written.
 * n_boxes == 0 is a no-op. images must not overlap src's byte range. */
int bsm_tile_box_load(const bsm_tensor* src, const bsm_box* box, const int32_t* coords_dev,
                      int64_t n_boxes, void* images, void* stream);

/* Box store or add-reduction, image -> global ([TMA] "Stores, reductions, and
 * completion").  Same box, coordinate and image contract as bsm_tile_box_load.
 * Elements whose coordinate is out of range are not written. reduce_add = 1 adds
 * each image element into the destination, dst <- round_to_nearest_even(dst + x) in
 * the destination format (F32, F16, BF16); the destination holds its starting value.
 * Boxes that overlap in global memory race (store) or are summed in an unspecified
 * order (reduce). images must not overlap dst's byte range. */
int bsm_tile_box_store(const bsm_tensor* dst, const bsm_box* box, const int32_t* coords_dev,
                       int64_t n_boxes, const void* images, int reduce_add, void* stream);

/* Box load and store / add-reduction with repeat axes ([TMA] "Call parameters": coords
 * plus coord_steps, one increment vector per repeat axis; "Code generation": one box per
 * repeat coordinate, in row-major repeat order; "Example: two explicit 8x16 boxes" is
 * coords (0, 0), coord_steps ((8, 0),) over one repeat axis of 2):
 *   coords:  HOST array of rank int64 starting coordinates, outer to inner;
 *   n_axes:  number of repeat axes, 0..4 (0: one box at coords);
 *   repeats: HOST array of n_axes extents, each >= 1, their product <= 2^31 - 1;
 *   steps:   HOST array of n_axes * rank int64 increments, axis a's vector at
 *            [a * rank, a * rank + rank);
 * box t, t = row-major index of (j_0, .., j_{n_axes-1}), has coordinates
 * coords + sum_a j_a * steps[a] and its image sits at t * bsm_image_stride(). The host
 * arrays are read during the call only. Every generated coordinate must fit in 32 bits
 * (BSM_E_SHAPE otherwise); n_axes outside 0..4 -> BSM_E_ARG; coords, or repeats / steps
 * with n_axes > 0, NULL -> BSM_E_NULL. Everything else as for bsm_tile_box_load /
 * bsm_tile_box_store (the coordinates need no device array). */
int bsm_tile_box_load_steps(const bsm_tensor* src, const bsm_box* box, const int64_t* coords, int32_t n_axes,
                            const int32_t* repeats, const int64_t* steps, void* images, void* stream);
int bsm_tile_box_store_steps(const bsm_tensor* dst, const bsm_box* box, const int64_t* coords, int32_t n_axes,
                             const int32_t* repeats, const int64_t* steps, const void* images, int reduce_add,
                             void* stream);

/* Four-row gather, global -> image ([TMA] "Gather4 and scatter4"; [TP] "TMA"): a
 * rank-2 tensor, a box of one row (box->box = {1, width}, element strides {1, 1}) and,
 * per issue, four explicit row coordinates that need not be consecutive or distinct.
 *   src:        the global tensor (rank 2, as for bsm_tile_box_load);
 *   coords_dev: DEVICE array of n_issues * 5 int32: issue t's column start c at [5t]
 *               and its rows r0..r3 at [5t+1 .. 5t+4]; any values (the row component of
 *               the box coordinates is replaced by the four rows);
 *   images:     DEVICE buffer of n_issues images of shape (4, width): image row i,
 *               element j = src[r_i, c + j], or the fill when r_i or c + j is out of
 *               range; compact row-major and swizzled as one (4, width) box image (the
 *               inner row rules of bsm_box apply to width); image t at t * S, where S =
 *               bsm_image_stride of the box {4, width} with the same swizzle; aligned
 *               like a box-load image buffer. Padding bytes between images are not written.
 * 0 <= n_issues <= 2^33 (0 is a no-op). images must not overlap src's byte range.
 * Rank, box, stride, swizzle and fill errors as for bsm_tile_box_load. */
int bsm_tile_gather4(const bsm_tensor* src, const bsm_box* box, const int32_t* coords_dev,
                     int64_t n_issues, void* images, void* stream);

/* Four-row scatter, image -> global ([TMA] "Gather4 and scatter4": the store form, the
 * global tensor first). Same box, coordinate and image contract as bsm_tile_gather4:
 * image row i is written to dst row r_i from column c; elements whose row or column is
 * out of range are not written (oob_fill is validated but unused). Rows repeated within
 * or across issues race (one of the writes survives). images must not overlap dst. */
int bsm_tile_scatter4(const bsm_tensor* dst, const bsm_box* box, const int32_t* coords_dev,
                      int64_t n_issues, const void* images, void* stream);

/* Grid round trip through LDS: for every tile coordinate t*box (t over
 * ceil(dims/box) per axis) the box of `src` is loaded into a swizzled LDS image,
 * which is then stored to `dst` and/or add-reduced into `dst_add` at the same
 * coordinates ([TMA] "Operand specification" and "Stores, reductions, and
 * completion"). dst or dst_add may be NULL, not both. All three tensors share
 * dtype, rank and dims (strides may differ) and must not overlap one another.
 * The boxes do not overlap, so the result is unique. */
int bsm_tile_box_copy(const bsm_tensor* src, const bsm_tensor* dst, const bsm_tensor* dst_add,
                      const bsm_box* box, void* stream);

/* Dense GEMM ([MMA] "Call parameters", "Operand specification", "Code generation",
 * "Example: four K16 issues"; [TP] "Warp MMA", "tcgen05 MMA"):
 *   D[m,n] = (accum ? D[m,n] : 0) + s * sum_k A(m,k) * B(n,k),  s = (-1)^(neg_a+neg_b),
 * products and sums in float32, D float32 row-major (D[m*ldd + n]).
 *   ab:      BSM_F16 or BSM_BF16 (both operands);
 *   a_major: 'k': A(m,k) = A[m*lda + k] (lda >= K);  'm': A(m,k) = A[k*lda + m] (lda >= M);
 *   b_major: 'k': B(n,k) = B[n*ldb + k] (ldb >= K);  'n': B(n,k) = B[k*ldb + n] (ldb >= N);
 *   A, B 16-byte aligned, lda and ldb multiples of 8 and at most 2^22; each operand
 *   buffer spans whole rows (rows * ld elements: the kernels read 16-byte chunks up to
 *   the row's padded end); D 16-byte aligned, ldd >= N and a multiple of 4;
 *   M, N, K >= 0 (M or N == 0: no-op; K == 0: D = accum ? D : 0);
 *   neg_a, neg_b, accum in {0, 1}. With accum == 0, D is never read. A and B must
 *   not overlap D. */
int bsm_gemm(int64_t M, int64_t N, int64_t K, int32_t ab,
             const void* A, int64_t lda, char a_major,
             const void* B, int64_t ldb, char b_major,
             float* D, int64_t ldd, int neg_a, int neg_b, int accum, void* stream);

/* Block-scaled GEMM ([MMA] "Weight-stationary and block scaling", "Call parameters";
 * [TP] "tcgen05 MMA"), both operands K-major:
 *   A(m,k) = dec(A[m*lda + k]) * 2^(SFA[m*ld_sfa + k/32] - 127),
 *   B(n,k) = dec(B[n*ldb + k]) * 2^(SFB[n*ld_sfb + k/32] - 127),
 *   D[m,n] = (accum ? D[m,n] : 0) + s * sum_k A(m,k) * B(n,k), float32 accumulation.
 * One E8M0 scale per 32 consecutive K elements (OCP MX block size 32); a scale code
 * of 0xFF (NaN) makes every product of its block NaN.
 *   a_fmt, b_fmt: any of BSM_E4M3, BSM_E5M2, BSM_E2M3, BSM_E3M2, BSM_E2M1, in any pairing
 *            ([MMA] "Weight-stationary and block scaling": the block-scaled kinds; the
 *            8-bit pairs and E2M1 x E2M1 run the tuned kernels, the other pairings a
 *            general one);
 *   lda, ldb in elements; E2M1 element index i is the (i & 1) nibble of byte i/2
 *   (low nibble first); E2M3 / E3M2 element i is bits 6i..6i+5 of the operand's bytes
 *   read as one little-endian bit string; rows 16-byte aligned (lda * bits and
 *   ldb * bits multiples of 128, e.g. lda a multiple of 64 for the 6-bit formats);
 *   K a multiple of 32; ld_sfa >= K/32, ld_sfb >= K/32, both multiples of 4, SFA and
 *   SFB 4-byte aligned (scale rows are read as 32-bit words); every buffer spans whole
 *   rows (rows * ld); D as for bsm_gemm. A, B, SFA, SFB must not overlap D.
 * Precision: every product of decoded, scaled values is formed exactly and the sums
 * keep |D - ref| within 1e-5 * sum_k |A(m,k) B(n,k)| (plus half an ulp of the float32
 * result): pairings whose products are all multiples of 2^-13 times the largest product
 * the two formats can form (E2M1 x E2M1, E2M3 x E2M3, E2M1 x E2M3, E2M1 x E3M2, in either
 * order) run the scaled f8f6f4 MFMA, whose block sums are then exact; every other pairing
 * (any 8-bit operand, E3M2 with E3M2 or E2M3) converts each element times its scale to
 * bf16 in registers (exact) and sums the products with the bf16 MFMA, which keeps every
 * product bit down to about 2^-24 of the largest term of each 16-product instruction,
 * at half the 8-bit MFMA rate. Scaled values must lie inside bf16's range on that route
 * (2^-133 up to about 3.4e38, i.e. scale codes that keep |element| * 2^(code - 127)
 * there); beyond it they round to bf16 subnormals, zero or infinity. */
int bsm_gemm_block_scale(int64_t M, int64_t N, int64_t K,
                         int32_t a_fmt, const void* A, int64_t lda, const uint8_t* SFA, int64_t ld_sfa,
                         int32_t b_fmt, const void* B, int64_t ldb, const uint8_t* SFB, int64_t ld_sfb,
                         float* D, int64_t ldd, int neg_a, int neg_b, int accum, void* stream);

/* Scalar epilogue f applied to every GEMM output element in registers, just before its
 * store ([TP] "Scalar compositions": a typed float32 scalar function inlined at each
 * register store, with scalar constants broadcast; the pages' example is silu followed
 * by an affine map, called with scale 2 and bias 1):
 *   BSM_EW_NONE:        f(x) = x;
 *   BSM_EW_SILU_AFFINE: f(x) = y * scale + bias,  y = x / (1 + exp(-x)),
 * evaluated in float32: exp(-x) within a few ulp (the hardware base-2 exponential with
 * the rounding of -x log2(e) carried as a correction), then x times the hardware
 * reciprocal of 1 + exp(-x), so y is within about 4 ulp of silu(x) for every float x
 * (results below 2^-112 may flush to zero). */
typedef enum bsm_ewise_op { BSM_EW_NONE = 0, BSM_EW_SILU_AFFINE = 1 } bsm_ewise_op;
typedef struct bsm_ewise {
  int32_t op;   /* bsm_ewise_op */
  float scale;  /* silu_affine: multiplier of silu(x) */
  float bias;   /* silu_affine: added last */
} bsm_ewise;

/* bsm_gemm and bsm_gemm_block_scale with the epilogue fused into the output store:
 *   D[m,n] = f(x),  x = (accum ? D[m,n] : 0) + s * sum_k A(m,k) * B(n,k),
 * where x is the float32 value the plain call would have stored (same kernels, same
 * rounding) and f is given by *ew (a host struct, read during the call only). K == 0
 * gives D = f(accum ? D : 0). Every other argument and rule is that of the plain call;
 * ew == NULL -> BSM_E_NULL, ew->op not a bsm_ewise_op -> BSM_E_ARG. With BSM_EW_NONE
 * the result is bit-identical to the plain call's. */
int bsm_gemm_ewise(int64_t M, int64_t N, int64_t K, int32_t ab,
                   const void* A, int64_t lda, char a_major,
                   const void* B, int64_t ldb, char b_major,
                   float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                   const bsm_ewise* ew, void* stream);
int bsm_gemm_block_scale_ewise(int64_t M, int64_t N, int64_t K,
                               int32_t a_fmt, const void* A, int64_t lda, const uint8_t* SFA, int64_t ld_sfa,
                               int32_t b_fmt, const void* B, int64_t ldb, const uint8_t* SFB, int64_t ld_sfb,
                               float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                               const bsm_ewise* ew, void* stream);

/* Block-scaled GEMM with the major order of each operand chosen ([MMA] "Shared
 * descriptors are byte-stride contracts": a_major / b_major are "k" or "mn", MN-major rows
 * enumerate K; "Weight-stationary and block scaling"; [TP] "tcgen05 MMA"):
 *   a_major 'k': A(m,k) = dec(A[m*lda + k]),  lda >= K;
 *           'm': A(m,k) = dec(A[k*lda + m]),  lda >= M   (K rows of M contiguous elements);
 *   b_major 'k': B(n,k) = dec(B[n*ldb + k]),  ldb >= K;
 *           'n': B(n,k) = dec(B[k*ldb + n]),  ldb >= N;
 * element index i of a row read as for bsm_gemm_block_scale (E2M1 low nibble first). The
 * scales keep their layout whatever the major order: SFA[m*ld_sfa + k/32],
 * SFB[n*ld_sfb + k/32]. An MN-major operand is BSM_E4M3, BSM_E5M2 or BSM_E2M1 (6-bit
 * MN-major operands -> BSM_E_MAJOR); the other operand may be any format and either
 * order. ew as for bsm_gemm_block_scale_ewise, or NULL for no epilogue. A major order
 * other than 'k' / 'm' ('k' / 'n' for B) -> BSM_E_MAJOR. Every other argument, rule and
 * the precision are those of bsm_gemm_block_scale: rows (K-major: M or N of them, MN-major:
 * K) 16-byte aligned (ld * bits a multiple of 128), every buffer spans whole rows
 * (rows * ld elements), ld * bits / 8 at most 2^23 bytes. With both orders 'k' the call
 * is bsm_gemm_block_scale_ewise (bit-identical results). MN-major operands run the
 * general kernel, which reads them through the gfx950 transposing LDS reads. */
int bsm_gemm_block_scale_major(int64_t M, int64_t N, int64_t K,
                               int32_t a_fmt, const void* A, int64_t lda, char a_major,
                               const uint8_t* SFA, int64_t ld_sfa,
                               int32_t b_fmt, const void* B, int64_t ldb, char b_major,
                               const uint8_t* SFB, int64_t ld_sfb,
                               float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                               const bsm_ewise* ew, void* stream);

/* bsm_gemm_block_scale_ewise with every pairing on gfx950's scaled f8f6f4 MFMA: the
 * fast-accumulation form, at the full 8-bit (and 4/6-bit) MFMA rate, for callers that
 * accept its block sums. Same arguments, layouts and errors (K-major operands only; ew may
 * be NULL for no epilogue). Precision: products are exact, but the instruction sums the 32
 * products of one scale block on a fixed grid of 2^-13 times the block's largest |product|
 * (measured on the device: a product 2^-13 below the block maximum is kept, one 2^-14
 * below is dropped), so each block may lose up to sum_k min(|p_k|, grid) beyond float32
 * rounding; the block sums are then accumulated in float32. For pairings whose products
 * all lie on that grid (see bsm_gemm_block_scale) the result equals bsm_gemm_block_scale's
 * bound; for wide-range 8-bit operands it does not meet 1e-5 * sum|ab|. */
int bsm_gemm_block_scale_fastacc(int64_t M, int64_t N, int64_t K,
                                 int32_t a_fmt, const void* A, int64_t lda, const uint8_t* SFA, int64_t ld_sfa,
                                 int32_t b_fmt, const void* B, int64_t ldb, const uint8_t* SFB, int64_t ld_sfb,
                                 float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                                 const bsm_ewise* ew, void* stream);

/* Element-wise scalar add on float32 ([TOE] "A Load, Compute, and Store Example"
 * adds one to a (2,32,3,4) tile; [TP] "Scalar compositions"): dst[i] = src[i] + s,
 * i < n, each lane moving 16-byte vectors. src, dst 16-byte aligned; they may be
 * equal (in place) but must not otherwise overlap. n >= 0. */
int bsm_tile_add_scalar_f32(const float* src, float* dst, int64_t n, float s, void* stream);

/* Diagnostic: the LDS -> register fragment load of the dense GEMM ([LDM]
 * "Address providers and result owners", "Transpose and stores"; [TP] "ldmatrix
 * with interleaved rows and separated registers"). One operand tile of
 * bsm_debug_fragment_shape() rows x kdim 16-bit elements is read from `src`
 * (major 'k': src[r*kdim + k]; major 'm': src[k*rows + r]), staged into LDS with
 * the GEMM's own loader and swizzle, and read back with the GEMM's own fragment
 * reads (16-byte reads for 'k', transposing 16-bit reads for 'm'). For every
 * 16-row block b, 32-wide K step s, lane l and element e, the value the lane holds
 * for operand (row 16b + l%16, k 32s + 8(l/16) + e) is written to
 * dump[((b * (kdim/32) + s) * 64 + l) * 8 + e] (the operand layout of the GEMM's
 * 16x16x32 MFMA). rows/kdim must equal the shape returned by
 * bsm_debug_fragment_shape. */
int bsm_debug_fragments(const uint16_t* src, int64_t rows, int64_t kdim, char major,
                        uint16_t* dump, void* stream);
void bsm_debug_fragment_shape(int64_t* rows, int64_t* kdim);

/* Diagnostic: the box copy's HBM traffic mix on flat buffers, with no boxes and no edges:
 * dst[i] = src[i] and add[i] = RNE_bf16(add[i] + src[i]) for i < n bf16 elements (4 * 2 * n
 * bytes moved, as bsm_tile_box_copy moves per element), 16-byte non-temporal accesses. It
 * measures the stream rate this read/write mix sustains on the device, the ceiling of the
 * box copy ([TMA] "Stores, reductions, and completion"). n a multiple of 8 (n == 0: no-op);
 * src, dst, add 16-byte aligned and pairwise non-overlapping. */
int bsm_debug_stream_mix_bf16(const void* src, void* dst, void* add, int64_t n, void* stream);

/* Diagnostic: workgroups x 256 lanes of back-to-back MFMAs on random register operands,
 * 16 independent 32x32 accumulators per wave (the block-scaled GEMMs' layout; the dense GEMM
 * runs 16x16x32 blocks, which hold a slightly higher clock), iters x 16 MFMAs per wave,
 * no memory or LDS traffic: the matrix-pipe rate the device holds under that load ([MMA]
 * "Example: four K16 issues": the MMA issue stream alone). kind: BSM_BF16 (v_mfma_f32_32x32x16_bf16,
 * 32768 FLOP each), BSM_E4M3 or BSM_E2M1 (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales,
 * 131072 FLOP each); so 4 * 16 * iters * workgroups MFMAs per launch. out receives one float
 * per lane (workgroups * 256, the lane's accumulator sum, so that no MFMA is dead code);
 * 4-byte aligned. workgroups and iters in 1 .. 2^20. */
int bsm_debug_mfma_loop(int32_t kind, int64_t workgroups, int32_t iters, float* out, void* stream);

/* Message describing the last nonzero status returned on this thread. */
const char* bsm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BSM_H */
