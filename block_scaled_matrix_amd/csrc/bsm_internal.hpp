// bsm_internal.hpp - launch interface between the validated C ABI (bsm_api.hip) and
// the kernels. Arguments reaching these functions have passed every contract check.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsm {

// Geometry of one box over one global tensor, as the kernels consume it.
struct BoxGeom {
  int32_t rank;
  int32_t esize;        // element bytes: 1, 2 or 4
  int32_t dtype;        // bsm_dtype
  int32_t swizzle;      // 0..3
  int32_t fill;         // 0 zero, 1 NaN
  uint32_t fill_bits;   // the fill element's bit pattern
  int32_t row_bytes;    // inner image row: ext[rank-1] * esize (multiple of 16)
  int32_t nrows;        // product of the outer image extents
  int64_t image_bytes;  // compact image bytes = nrows * row_bytes
  int64_t image_stride; // bytes between consecutive images in an image buffer
  int64_t dims[5];
  int64_t strides[5];   // bytes
  int32_t box[5];
  int32_t estr[5];
  int32_t ext[5];       // image extents ceil(box / estr)
};

// D[m*ldd + n] = 0 for m < M, n < N (a kernel, so the call can be graph-captured).
hipError_t launch_zero_f32_2d(float* D, int64_t ldd, int64_t M, int64_t N, hipStream_t st);
// The K == 0 GEMM output: D[m*ldd + n] = f(accum ? D[m*ldd + n] : 0) for m < M, n < N,
// f the epilogue (ew_op, ew_scale, ew_bias) of GemmArgs.
hipError_t launch_empty_gemm(float* D, int64_t ldd, int64_t M, int64_t N, int accum, int ew_op, float ew_scale,
                             float ew_bias, hipStream_t st);

hipError_t launch_add_scalar_f32(const float* src, float* dst, int64_t n, float s, hipStream_t st);

// Box coordinates generated on the device for a call with repeat axes: box t (row-major
// over rep[0..naxes)) starts at base + sum_a j_a * step[a]. The host has checked that every
// such coordinate fits in 32 bits.
struct BoxRepeat {
  int32_t naxes;       // 0..4
  int32_t rep[4];
  int32_t base[5];
  int32_t step[4][5];
};

// coords: DEVICE array of n_boxes * rank int32, or NULL to generate them from rp.
hipError_t launch_box_load(const BoxGeom& g, const void* src, const int32_t* coords, const BoxRepeat& rp,
                           int64_t n_boxes, void* images, hipStream_t st);
hipError_t launch_box_store(const BoxGeom& g, void* dst, const int32_t* coords, const BoxRepeat& rp, int64_t n_boxes,
                            const void* images, int reduce_add, hipStream_t st);
// Four-row gather (scatter = 0: tensor -> images) or scatter (1: images -> tensor) of
// n_issues issues; g describes the rank-2 tensor and the (4, width) image; coords holds
// 5 int32 per issue (column start, four rows).
hipError_t launch_row4(const BoxGeom& g, void* tensor, const int32_t* coords, int64_t n_issues, void* images,
                       int scatter, hipStream_t st);
// Grid round trip; dst_strides / add_strides describe dst and dst_add (NULL allowed).
hipError_t launch_box_copy(const BoxGeom& g, const void* src, void* dst, const int64_t* dst_strides,
                           void* dst_add, const int64_t* add_strides, hipStream_t st);

struct GemmArgs {
  int64_t M, N, K;
  int32_t dtype;        // BSM_F16 / BSM_BF16 (dense) or A's block-scaled format (E4M3, E5M2, E2M3, E3M2, E2M1)
  int32_t dtype_b;      // block scaled: B's format (0 for dense)
  const void* A; int64_t lda; int32_t a_kmajor;
  const void* B; int64_t ldb; int32_t b_kmajor;
  const uint8_t* SFA; int64_t ld_sfa;
  const uint8_t* SFB; int64_t ld_sfb;
  float* D; int64_t ldd;
  int32_t negate;       // neg_a xor neg_b
  int32_t accum;
  int32_t ew_op;        // bsm_ewise_op applied to each output before its store (0: none)
  float ew_scale, ew_bias;
  int32_t mx_window;    // block scaled: 1 = every pairing on the scaled f8f6f4 MFMA (its 2^-13 block
                        // window), 0 = exact products (bf16 MFMA) for the pairings that need them
};

hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t st);
// Any pairing of E4M3, E5M2, E2M3, E3M2, E2M1 except E2M1 x E2M1, and except 8-bit x 8-bit
// when mx_window is set (K > 0).
hipError_t launch_gemm_mx_any(const GemmArgs& a, hipStream_t st);
// One or both operands MN-major (A only, B only, both); an MN-major operand is E4M3, E5M2 or
// E2M1 (K > 0).
hipError_t launch_gemm_mx_mn_a(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mx_mn_b(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mx_mn_ab(const GemmArgs& a, hipStream_t st);

// Diagnostics (k_diag.hip): the box copy's traffic mix on flat bf16 buffers of n elements
// (n a multiple of 8, 16-byte aligned), and workgroups x 256 lanes of back-to-back MFMAs of
// `kind` (BSM_BF16, BSM_E4M3, BSM_E2M1), iters x 16 per wave, one float per lane to out.
hipError_t launch_stream_mix_bf16(const void* src, void* dst, void* add, int64_t n, hipStream_t st);
hipError_t launch_mfma_loop(int kind, int64_t workgroups, int iters, float* out, hipStream_t st);

// Operand-tile geometry of the dense GEMM (rows x K elements per LDS stage).
constexpr int kDenseTileRows = 256;
constexpr int kDenseTileK = 64;
hipError_t launch_debug_fragments(const uint16_t* src, int kmajor, uint16_t* dump, hipStream_t st);

}  // namespace bsm
