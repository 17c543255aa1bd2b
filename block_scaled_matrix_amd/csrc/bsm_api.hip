// bsm_api.hip - the C ABI of libbsm: host-side contract checks, then launches.
//
// Every rule checked here is stated in include/bsm.h next to the entry point it
// belongs to. Nothing is launched when a check fails; no check touches device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bsm.h"
#include "bsm_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return BSM_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BSM_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

int elem_size(int32_t dt) {
  switch (dt) {
    case BSM_U8: case BSM_E4M3: case BSM_E5M2: case BSM_E8M0: return 1;
    case BSM_U16: case BSM_F16: case BSM_BF16: return 2;
    case BSM_U32: case BSM_F32: return 4;
    default: return 0;
  }
}

bool has_nan(int32_t dt) {
  return dt == BSM_F32 || dt == BSM_F16 || dt == BSM_BF16 || dt == BSM_E4M3 || dt == BSM_E5M2;
}

uint32_t nan_bits(int32_t dt) {
  switch (dt) {
    case BSM_F32: return 0x7FC00000u;
    case BSM_F16: return 0x7E00u;
    case BSM_BF16: return 0x7FC0u;
    case BSM_E5M2: return 0x7Eu;
    default: return 0x7Fu;  // E4M3
  }
}

// Half-open byte range [lo, hi) a tensor view can touch.
struct Range { uintptr_t lo, hi; };
Range tensor_range(const bsm_tensor* t) {
  uintptr_t lo = (uintptr_t)t->base, hi = lo + (uintptr_t)elem_size(t->dtype);
  for (int i = 0; i < t->rank; i++) hi += (uintptr_t)((t->dims[i] - 1) * t->strides[i]);
  return {lo, hi};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_tensor(const bsm_tensor* t, const char* name) {
  if (!t) return fail(BSM_E_NULL, "%s: tensor descriptor is NULL", name);
  if (!t->base) return fail(BSM_E_NULL, "%s: base pointer is NULL", name);
  if (t->rank < 1 || t->rank > 5) return fail(BSM_E_RANK, "%s: rank %d not in 1..5", name, t->rank);
  const int es = elem_size(t->dtype);
  if (es == 0)
    return fail(BSM_E_DTYPE, "%s: dtype %d is not a whole-byte box format (view packed fp4 as U8)", name, t->dtype);
  if ((uintptr_t)t->base % 16) return fail(BSM_E_ALIGN, "%s: base not 16-byte aligned", name);
  for (int i = 0; i < t->rank; i++) {
    if (t->dims[i] < 1 || t->dims[i] > 0x7FFFFFFF)
      return fail(BSM_E_SHAPE, "%s: dims[%d] = %lld not in 1..2^31-1", name, i, (long long)t->dims[i]);
  }
  if (t->strides[t->rank - 1] != es)
    return fail(BSM_E_ALIGN, "%s: innermost stride %lld must equal the element size %d", name,
                (long long)t->strides[t->rank - 1], es);
  for (int i = 0; i < t->rank - 1; i++) {
    if (t->strides[i] <= 0 || t->strides[i] % 16)
      return fail(BSM_E_ALIGN, "%s: strides[%d] = %lld is not a positive multiple of 16 bytes", name, i,
                  (long long)t->strides[i]);
  }
  return BSM_OK;
}

int make_geom(const bsm_box* b, int32_t dtype, bsm::BoxGeom* g) {
  if (!b) return fail(BSM_E_NULL, "box descriptor is NULL");
  if (b->rank < 1 || b->rank > 5) return fail(BSM_E_RANK, "box rank %d not in 1..5", b->rank);
  const int es = elem_size(dtype);
  if (es == 0) return fail(BSM_E_DTYPE, "dtype %d is not a whole-byte box format", dtype);
  memset(g, 0, sizeof *g);
  g->rank = b->rank;
  g->esize = es;
  g->dtype = dtype;
  int64_t rows = 1;
  for (int i = 0; i < b->rank; i++) {
    if (b->box[i] < 1 || b->box[i] > 256) return fail(BSM_E_BOX, "box[%d] = %d not in 1..256", i, b->box[i]);
    if (b->element_strides[i] < 1 || b->element_strides[i] > 8)
      return fail(BSM_E_ESTRIDE, "element_strides[%d] = %d not in 1..8", i, b->element_strides[i]);
    g->box[i] = b->box[i];
    g->estr[i] = b->element_strides[i];
    g->ext[i] = (b->box[i] + b->element_strides[i] - 1) / b->element_strides[i];
    if (i < b->rank - 1) rows *= g->ext[i];
  }
  if (b->element_strides[b->rank - 1] != 1)
    return fail(BSM_E_ESTRIDE, "the innermost element stride must be 1 (got %d)", b->element_strides[b->rank - 1]);
  if (b->swizzle < 0 || b->swizzle > 3) return fail(BSM_E_SWIZZLE, "swizzle %d not in 0..3", b->swizzle);
  const int row_bytes = g->ext[b->rank - 1] * es;
  if (row_bytes % 16)
    return fail(BSM_E_SWIZZLE, "inner image row of %d bytes is not a multiple of 16", row_bytes);
  if (b->swizzle && row_bytes > (16 << b->swizzle))
    return fail(BSM_E_SWIZZLE, "inner image row of %d bytes exceeds the %d-byte swizzle span", row_bytes,
                16 << b->swizzle);
  if (b->oob_fill != 0 && b->oob_fill != 1) return fail(BSM_E_FILL, "oob_fill %d not 0/1", b->oob_fill);
  if (b->oob_fill == 1 && !has_nan(dtype)) return fail(BSM_E_FILL, "NaN fill on dtype %d, which has no NaN", dtype);
  g->swizzle = b->swizzle;
  g->fill = b->oob_fill;
  g->fill_bits = b->oob_fill ? nan_bits(dtype) : 0u;
  g->row_bytes = row_bytes;
  g->nrows = (int32_t)rows;
  g->image_bytes = rows * row_bytes;
  if (g->image_bytes > 163840)
    return fail(BSM_E_BOX, "image of %lld bytes exceeds 160 KiB of LDS", (long long)g->image_bytes);
  const int64_t align = b->swizzle ? (int64_t(1) << (7 + b->swizzle)) : 128;
  g->image_stride = (g->image_bytes + align - 1) / align * align;
  return BSM_OK;
}

void fill_tensor_geom(const bsm_tensor* t, bsm::BoxGeom* g) {
  for (int i = 0; i < t->rank; i++) { g->dims[i] = t->dims[i]; g->strides[i] = t->strides[i]; }
}

// A four-row gather / scatter: a rank-2 tensor and a (1, width) box with unit element
// strides; g then describes the tensor and the (4, width) image.
int row4_geom(const bsm_tensor* t, const char* name, const bsm_box* box, bsm::BoxGeom* g) {
  int rc = check_tensor(t, name);
  if (rc) return rc;
  if (!box) return fail(BSM_E_NULL, "box descriptor is NULL");
  if (t->rank != 2) return fail(BSM_E_RANK, "%s: gather4 / scatter4 take a rank-2 tensor (rank %d)", name, t->rank);
  if (box->rank != 2) return fail(BSM_E_RANK, "box rank %d: gather4 / scatter4 take a rank-2 box", box->rank);
  if (box->box[0] != 1)
    return fail(BSM_E_BOX, "box (%d, %d): gather4 / scatter4 take a box of one row", box->box[0], box->box[1]);
  if (box->element_strides[0] != 1 || box->element_strides[1] != 1)
    return fail(BSM_E_ESTRIDE, "gather4 / scatter4 take unit element strides");
  bsm_box b4 = *box;
  b4.box[0] = 4;
  if ((rc = make_geom(&b4, t->dtype, g))) return rc;
  fill_tensor_geom(t, g);
  return BSM_OK;
}

int check_flag(int v, const char* name) {
  if (v != 0 && v != 1) return fail(BSM_E_ARG, "%s = %d is not 0 or 1", name, v);
  return BSM_OK;
}

}  // namespace

extern "C" {

const char* bsm_last_error(void) { return g_err; }

int64_t bsm_image_stride(const bsm_box* box, int32_t dtype) {
  bsm::BoxGeom g;
  int rc = make_geom(box, dtype, &g);
  if (rc) return rc;
  return g.image_stride;
}

static int box_load_impl(const bsm_tensor* src, const bsm_box* box, const int32_t* coords_dev,
                         const bsm::BoxRepeat* rp, int64_t n_boxes, void* images, void* stream, const char* name) {
  int rc = check_tensor(src, "src");
  if (rc) return rc;
  bsm::BoxGeom g;
  if ((rc = make_geom(box, src->dtype, &g))) return rc;
  if (box->rank != src->rank) return fail(BSM_E_RANK, "box rank %d != tensor rank %d", box->rank, src->rank);
  if (n_boxes < 0 || n_boxes > 0x7FFFFFFF) return fail(BSM_E_SHAPE, "n_boxes %lld out of range", (long long)n_boxes);
  if (n_boxes == 0) return ok();
  if (!rp && !coords_dev) return fail(BSM_E_NULL, "coords is NULL");
  if (!images) return fail(BSM_E_NULL, "images is NULL");
  if (!rp && (uintptr_t)coords_dev % 4) return fail(BSM_E_ALIGN, "coords not 4-byte aligned");
  const uintptr_t ia = box->swizzle ? (uintptr_t(1) << (7 + box->swizzle)) : 128;
  if ((uintptr_t)images % ia) return fail(BSM_E_ALIGN, "images not %u-byte aligned", (unsigned)ia);
  Range ir{(uintptr_t)images, (uintptr_t)images + (uintptr_t)(n_boxes * g.image_stride)};
  if (overlap(ir, tensor_range(src))) return fail(BSM_E_ALIAS, "images overlap src");
  fill_tensor_geom(src, &g);
  const bsm::BoxRepeat none{};
  hipError_t e = bsm::launch_box_load(g, src->base, rp ? nullptr : coords_dev, rp ? *rp : none, n_boxes, images,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

static int box_store_impl(const bsm_tensor* dst, const bsm_box* box, const int32_t* coords_dev,
                          const bsm::BoxRepeat* rp, int64_t n_boxes, const void* images, int reduce_add, void* stream,
                          const char* name) {
  int rc = check_tensor(dst, "dst");
  if (rc) return rc;
  bsm::BoxGeom g;
  if ((rc = make_geom(box, dst->dtype, &g))) return rc;
  if (box->rank != dst->rank) return fail(BSM_E_RANK, "box rank %d != tensor rank %d", box->rank, dst->rank);
  if ((rc = check_flag(reduce_add, "reduce_add"))) return rc;
  if (reduce_add && dst->dtype != BSM_F32 && dst->dtype != BSM_F16 && dst->dtype != BSM_BF16)
    return fail(BSM_E_DTYPE, "add-reduction needs an F32, F16 or BF16 destination (got %d)", dst->dtype);
  if (n_boxes < 0 || n_boxes > 0x7FFFFFFF) return fail(BSM_E_SHAPE, "n_boxes %lld out of range", (long long)n_boxes);
  if (n_boxes == 0) return ok();
  if (!rp && !coords_dev) return fail(BSM_E_NULL, "coords is NULL");
  if (!images) return fail(BSM_E_NULL, "images is NULL");
  if (!rp && (uintptr_t)coords_dev % 4) return fail(BSM_E_ALIGN, "coords not 4-byte aligned");
  const uintptr_t ia = box->swizzle ? (uintptr_t(1) << (7 + box->swizzle)) : 128;
  if ((uintptr_t)images % ia) return fail(BSM_E_ALIGN, "images not %u-byte aligned", (unsigned)ia);
  Range ir{(uintptr_t)images, (uintptr_t)images + (uintptr_t)(n_boxes * g.image_stride)};
  if (overlap(ir, tensor_range(dst))) return fail(BSM_E_ALIAS, "images overlap dst");
  fill_tensor_geom(dst, &g);
  const bsm::BoxRepeat none{};
  hipError_t e = bsm::launch_box_store(g, dst->base, rp ? nullptr : coords_dev, rp ? *rp : none, n_boxes, images,
                                       reduce_add, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

// Repeat axes of a box call: checks them and every coordinate they generate against the
// 32-bit range the kernels use; n_boxes = product of the repeat extents.
static int make_repeat(const bsm_box* box, const int64_t* coords, int32_t n_axes, const int32_t* repeats,
                       const int64_t* steps, bsm::BoxRepeat* rp, int64_t* n_boxes) {
  if (!box) return fail(BSM_E_NULL, "box descriptor is NULL");
  if (box->rank < 1 || box->rank > 5) return fail(BSM_E_RANK, "box rank %d not in 1..5", box->rank);
  if (!coords) return fail(BSM_E_NULL, "coords is NULL");
  if (n_axes < 0 || n_axes > 4) return fail(BSM_E_ARG, "n_axes = %d not in 0..4", n_axes);
  if (n_axes > 0 && (!repeats || !steps)) return fail(BSM_E_NULL, "repeats or steps is NULL");
  memset(rp, 0, sizeof *rp);
  rp->naxes = n_axes;
  int64_t n = 1;
  for (int a = 0; a < n_axes; a++) {
    if (repeats[a] < 1) return fail(BSM_E_SHAPE, "repeats[%d] = %d is not positive", a, repeats[a]);
    n *= repeats[a];
    if (n > 0x7FFFFFFF) return fail(BSM_E_SHAPE, "more than 2^31 - 1 boxes");
    rp->rep[a] = repeats[a];
  }
  const int64_t lim = int64_t(1) << 31;
  for (int i = 0; i < box->rank; i++) {
    __int128 lo = coords[i], hi = coords[i];
    for (int a = 0; a < n_axes; a++) {
      const __int128 d = (__int128)(repeats[a] - 1) * steps[a * box->rank + i];
      if (d < 0) lo += d; else hi += d;
      if (steps[a * box->rank + i] < -lim || steps[a * box->rank + i] >= lim)
        return fail(BSM_E_SHAPE, "steps[%d][%d] outside the 32-bit range", a, i);
      rp->step[a][i] = (int32_t)steps[a * box->rank + i];
    }
    if (lo < -lim || hi >= lim) return fail(BSM_E_SHAPE, "a repeat coordinate of dimension %d leaves the 32-bit range", i);
    rp->base[i] = (int32_t)coords[i];
  }
  *n_boxes = n;
  return BSM_OK;
}

int bsm_tile_box_load(const bsm_tensor* src, const bsm_box* box, const int32_t* coords_dev, int64_t n_boxes,
                      void* images, void* stream) {
  return box_load_impl(src, box, coords_dev, nullptr, n_boxes, images, stream, "bsm_tile_box_load");
}

int bsm_tile_box_store(const bsm_tensor* dst, const bsm_box* box, const int32_t* coords_dev, int64_t n_boxes,
                       const void* images, int reduce_add, void* stream) {
  return box_store_impl(dst, box, coords_dev, nullptr, n_boxes, images, reduce_add, stream, "bsm_tile_box_store");
}

int bsm_tile_box_load_steps(const bsm_tensor* src, const bsm_box* box, const int64_t* coords, int32_t n_axes,
                            const int32_t* repeats, const int64_t* steps, void* images, void* stream) {
  bsm::BoxRepeat rp;
  int64_t n = 0;
  int rc = make_repeat(box, coords, n_axes, repeats, steps, &rp, &n);
  if (rc) return rc;
  return box_load_impl(src, box, nullptr, &rp, n, images, stream, "bsm_tile_box_load_steps");
}

int bsm_tile_box_store_steps(const bsm_tensor* dst, const bsm_box* box, const int64_t* coords, int32_t n_axes,
                             const int32_t* repeats, const int64_t* steps, const void* images, int reduce_add,
                             void* stream) {
  bsm::BoxRepeat rp;
  int64_t n = 0;
  int rc = make_repeat(box, coords, n_axes, repeats, steps, &rp, &n);
  if (rc) return rc;
  return box_store_impl(dst, box, nullptr, &rp, n, images, reduce_add, stream, "bsm_tile_box_store_steps");
}

int bsm_tile_box_copy(const bsm_tensor* src, const bsm_tensor* dst, const bsm_tensor* dst_add, const bsm_box* box,
                      void* stream) {
  int rc = check_tensor(src, "src");
  if (rc) return rc;
  if (!dst && !dst_add) return fail(BSM_E_NULL, "dst and dst_add are both NULL");
  if (dst && (rc = check_tensor(dst, "dst"))) return rc;
  if (dst_add && (rc = check_tensor(dst_add, "dst_add"))) return rc;
  bsm::BoxGeom g;
  if ((rc = make_geom(box, src->dtype, &g))) return rc;
  if (box->rank != src->rank) return fail(BSM_E_RANK, "box rank %d != tensor rank %d", box->rank, src->rank);
  for (const bsm_tensor* t : {dst, dst_add}) {
    if (!t) continue;
    if (t->dtype != src->dtype) return fail(BSM_E_DTYPE, "dst/dst_add dtype differs from src");
    if (t->rank != src->rank) return fail(BSM_E_RANK, "dst/dst_add rank differs from src");
    for (int i = 0; i < src->rank; i++)
      if (t->dims[i] != src->dims[i]) return fail(BSM_E_SHAPE, "dst/dst_add dims differ from src");
  }
  if (dst_add && src->dtype != BSM_F32 && src->dtype != BSM_F16 && src->dtype != BSM_BF16)
    return fail(BSM_E_DTYPE, "add-reduction needs F32, F16 or BF16 (got %d)", src->dtype);
  const Range rs = tensor_range(src);
  if (dst && overlap(rs, tensor_range(dst))) return fail(BSM_E_ALIAS, "dst overlaps src");
  if (dst_add && overlap(rs, tensor_range(dst_add))) return fail(BSM_E_ALIAS, "dst_add overlaps src");
  if (dst && dst_add && overlap(tensor_range(dst), tensor_range(dst_add)))
    return fail(BSM_E_ALIAS, "dst overlaps dst_add");
  fill_tensor_geom(src, &g);
  hipError_t e = bsm::launch_box_copy(g, src->base, dst ? dst->base : nullptr, dst ? dst->strides : nullptr,
                                      dst_add ? dst_add->base : nullptr, dst_add ? dst_add->strides : nullptr,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsm_tile_box_copy");
  return ok();
}

static int row4_call(const bsm_tensor* t, const bsm_box* box, const int32_t* coords_dev, int64_t n_issues,
                     const void* images, int scatter, void* stream) {
  const char* name = scatter ? "dst" : "src";
  bsm::BoxGeom g;
  int rc = row4_geom(t, name, box, &g);
  if (rc) return rc;
  if (n_issues < 0 || n_issues > (int64_t(1) << 33))
    return fail(BSM_E_SHAPE, "n_issues %lld out of range", (long long)n_issues);
  if (n_issues == 0) return ok();
  if (!coords_dev) return fail(BSM_E_NULL, "coords is NULL");
  if (!images) return fail(BSM_E_NULL, "images is NULL");
  if ((uintptr_t)coords_dev % 4) return fail(BSM_E_ALIGN, "coords not 4-byte aligned");
  const uintptr_t ia = box->swizzle ? (uintptr_t(1) << (7 + box->swizzle)) : 128;
  if ((uintptr_t)images % ia) return fail(BSM_E_ALIGN, "images not %u-byte aligned", (unsigned)ia);
  Range ir{(uintptr_t)images, (uintptr_t)images + (uintptr_t)(n_issues * g.image_stride)};
  if (overlap(ir, tensor_range(t))) return fail(BSM_E_ALIAS, "images overlap %s", name);
  hipError_t e = bsm::launch_row4(g, t->base, coords_dev, n_issues, (void*)images, scatter, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, scatter ? "bsm_tile_scatter4" : "bsm_tile_gather4");
  return ok();
}

int bsm_tile_gather4(const bsm_tensor* src, const bsm_box* box, const int32_t* coords_dev, int64_t n_issues,
                     void* images, void* stream) {
  return row4_call(src, box, coords_dev, n_issues, images, 0, stream);
}

int bsm_tile_scatter4(const bsm_tensor* dst, const bsm_box* box, const int32_t* coords_dev, int64_t n_issues,
                      const void* images, void* stream) {
  return row4_call(dst, box, coords_dev, n_issues, images, 1, stream);
}

static int check_d(float* D, int64_t M, int64_t N, int64_t ldd) {
  if (!D) return fail(BSM_E_NULL, "D is NULL");
  if ((uintptr_t)D % 16) return fail(BSM_E_ALIGN, "D not 16-byte aligned");
  if (ldd < N || ldd % 4) return fail(BSM_E_ALIGN, "ldd = %lld must be >= N and a multiple of 4", (long long)ldd);
  (void)M;
  return BSM_OK;
}

static int gemm_dense(int64_t M, int64_t N, int64_t K, int32_t ab, const void* A, int64_t lda, char a_major,
                      const void* B, int64_t ldb, char b_major, float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                      const bsm_ewise& ew, void* stream, const char* name) {
  int rc;
  if ((rc = check_flag(neg_a, "neg_a")) || (rc = check_flag(neg_b, "neg_b")) || (rc = check_flag(accum, "accum")))
    return rc;
  if (ab != BSM_F16 && ab != BSM_BF16) return fail(BSM_E_DTYPE, "ab = %d: dense GEMM takes F16 or BF16", ab);
  if (M < 0 || N < 0 || K < 0 || M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF)
    return fail(BSM_E_SHAPE, "M, N, K = %lld, %lld, %lld out of range", (long long)M, (long long)N, (long long)K);
  if (a_major != 'k' && a_major != 'm') return fail(BSM_E_MAJOR, "a_major '%c' is not 'k' or 'm'", a_major);
  if (b_major != 'k' && b_major != 'n') return fail(BSM_E_MAJOR, "b_major '%c' is not 'k' or 'n'", b_major);
  if (M == 0 || N == 0) return ok();
  if ((rc = check_d(D, M, N, ldd))) return rc;
  if (K > 0) {
    if (!A || !B) return fail(BSM_E_NULL, "A or B is NULL");
    if ((uintptr_t)A % 16 || (uintptr_t)B % 16) return fail(BSM_E_ALIGN, "A and B must be 16-byte aligned");
    const int64_t amin = a_major == 'k' ? K : M, bmin = b_major == 'k' ? K : N;
    if (lda < amin || lda % 8) return fail(BSM_E_ALIGN, "lda = %lld must be >= %lld and a multiple of 8", (long long)lda, (long long)amin);
    if (ldb < bmin || ldb % 8) return fail(BSM_E_ALIGN, "ldb = %lld must be >= %lld and a multiple of 8", (long long)ldb, (long long)bmin);
    if (lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22))
      return fail(BSM_E_SHAPE, "lda, ldb must be at most 2^22 elements (32-bit in-tile offsets)");
    const Range rd{(uintptr_t)D, (uintptr_t)(D + (M - 1) * ldd + N)};
    const int64_t arows = a_major == 'k' ? M : K, brows = b_major == 'k' ? N : K;
    const Range ra{(uintptr_t)A, (uintptr_t)A + (uintptr_t)(((arows - 1) * lda + amin) * 2)};
    const Range rb{(uintptr_t)B, (uintptr_t)B + (uintptr_t)(((brows - 1) * ldb + bmin) * 2)};
    if (overlap(rd, ra) || overlap(rd, rb)) return fail(BSM_E_ALIAS, "A or B overlaps D");
  }
  bsm::GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.dtype = ab;
  g.A = A; g.lda = lda; g.a_kmajor = a_major == 'k';
  g.B = B; g.ldb = ldb; g.b_kmajor = b_major == 'k';
  g.D = D; g.ldd = ldd; g.negate = neg_a ^ neg_b; g.accum = accum;
  g.ew_op = ew.op; g.ew_scale = ew.scale; g.ew_bias = ew.bias;
  hipError_t e = bsm::launch_gemm_dense(g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

static int check_ewise(const bsm_ewise* ew) {
  if (!ew) return fail(BSM_E_NULL, "ew is NULL");
  if (ew->op != BSM_EW_NONE && ew->op != BSM_EW_SILU_AFFINE) return fail(BSM_E_ARG, "ew->op = %d is not a bsm_ewise_op", ew->op);
  return BSM_OK;
}

int bsm_gemm(int64_t M, int64_t N, int64_t K, int32_t ab, const void* A, int64_t lda, char a_major, const void* B,
             int64_t ldb, char b_major, float* D, int64_t ldd, int neg_a, int neg_b, int accum, void* stream) {
  return gemm_dense(M, N, K, ab, A, lda, a_major, B, ldb, b_major, D, ldd, neg_a, neg_b, accum,
                    bsm_ewise{BSM_EW_NONE, 1.0f, 0.0f}, stream, "bsm_gemm");
}

int bsm_gemm_ewise(int64_t M, int64_t N, int64_t K, int32_t ab, const void* A, int64_t lda, char a_major,
                   const void* B, int64_t ldb, char b_major, float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                   const bsm_ewise* ew, void* stream) {
  int rc;
  if ((rc = check_ewise(ew))) return rc;
  return gemm_dense(M, N, K, ab, A, lda, a_major, B, ldb, b_major, D, ldd, neg_a, neg_b, accum, *ew, stream,
                    "bsm_gemm_ewise");
}

static int gemm_block_scale(int64_t M, int64_t N, int64_t K, int32_t a_fmt, const void* A, int64_t lda,
                            char a_major, const uint8_t* SFA, int64_t ld_sfa, int32_t b_fmt, const void* B,
                            int64_t ldb, char b_major, const uint8_t* SFB, int64_t ld_sfb, float* D, int64_t ldd,
                            int neg_a, int neg_b, int accum, const bsm_ewise& ew, void* stream, const char* name,
                            int window = 0) {
  int rc;
  if ((rc = check_flag(neg_a, "neg_a")) || (rc = check_flag(neg_b, "neg_b")) || (rc = check_flag(accum, "accum")))
    return rc;
  auto bits = [](int32_t f) {
    return f == BSM_E4M3 || f == BSM_E5M2 ? 8 : (f == BSM_E2M3 || f == BSM_E3M2 ? 6 : (f == BSM_E2M1 ? 4 : 0));
  };
  const int ba = bits(a_fmt), bb = bits(b_fmt);
  if (!ba || !bb)
    return fail(BSM_E_DTYPE, "a_fmt %d / b_fmt %d: block-scaled GEMM takes E4M3, E5M2, E2M3, E3M2 or E2M1", a_fmt,
                b_fmt);
  if (a_major != 'k' && a_major != 'm') return fail(BSM_E_MAJOR, "a_major '%c' is not 'k' or 'm'", a_major);
  if (b_major != 'k' && b_major != 'n') return fail(BSM_E_MAJOR, "b_major '%c' is not 'k' or 'n'", b_major);
  if ((a_major == 'm' && ba == 6) || (b_major == 'n' && bb == 6))
    return fail(BSM_E_MAJOR, "MN-major block-scaled operands are E4M3, E5M2 or E2M1 (not the 6-bit formats)");
  if (M < 0 || N < 0 || K < 0 || M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF)
    return fail(BSM_E_SHAPE, "M, N, K = %lld, %lld, %lld out of range", (long long)M, (long long)N, (long long)K);
  if (K % 32) return fail(BSM_E_SHAPE, "K = %lld is not a multiple of the 32-element scale block", (long long)K);
  if (M == 0 || N == 0) return ok();
  if ((rc = check_d(D, M, N, ldd))) return rc;
  if (K > 0) {
    if (!A || !B || !SFA || !SFB) return fail(BSM_E_NULL, "A, B, SFA or SFB is NULL");
    if ((uintptr_t)A % 16 || (uintptr_t)B % 16) return fail(BSM_E_ALIGN, "A and B must be 16-byte aligned");
    // (rows, row length) of each operand's storage
    const int64_t arows = a_major == 'k' ? M : K, alen = a_major == 'k' ? K : M;
    const int64_t brows = b_major == 'k' ? N : K, blen = b_major == 'k' ? K : N;
    if (lda < alen) return fail(BSM_E_ALIGN, "lda = %lld must be >= %lld", (long long)lda, (long long)alen);
    if (ldb < blen) return fail(BSM_E_ALIGN, "ldb = %lld must be >= %lld", (long long)ldb, (long long)blen);
    if ((lda * ba) % 128 || (ldb * bb) % 128)
      return fail(BSM_E_ALIGN, "lda = %lld, ldb = %lld: rows must start 16-byte aligned", (long long)lda, (long long)ldb);
    if (ld_sfa < K / 32 || ld_sfb < K / 32) return fail(BSM_E_ALIGN, "ld_sfa, ld_sfb must be >= K/32");
    if (ld_sfa % 4 || ld_sfb % 4 || (uintptr_t)SFA % 4 || (uintptr_t)SFB % 4)
      return fail(BSM_E_ALIGN, "scale rows must start 4-byte aligned (SFA, SFB 4-byte aligned, ld_sfa, ld_sfb multiples of 4)");
    if (lda * ba / 8 > (int64_t(1) << 23) || ldb * bb / 8 > (int64_t(1) << 23) || ld_sfa > (int64_t(1) << 24) ||
        ld_sfb > (int64_t(1) << 24))
      return fail(BSM_E_SHAPE, "leading dimensions too large for 32-bit in-tile offsets");
    const Range rd{(uintptr_t)D, (uintptr_t)(D + (M - 1) * ldd + N)};
    const Range ra{(uintptr_t)A, (uintptr_t)A + (uintptr_t)(((arows - 1) * lda + alen) * ba / 8)};
    const Range rb{(uintptr_t)B, (uintptr_t)B + (uintptr_t)(((brows - 1) * ldb + blen) * bb / 8)};
    const Range rsa{(uintptr_t)SFA, (uintptr_t)SFA + (uintptr_t)(M * ld_sfa)};
    const Range rsb{(uintptr_t)SFB, (uintptr_t)SFB + (uintptr_t)(N * ld_sfb)};
    if (overlap(rd, ra) || overlap(rd, rb) || overlap(rd, rsa) || overlap(rd, rsb))
      return fail(BSM_E_ALIAS, "an operand or scale tensor overlaps D");
  }
  bsm::GemmArgs g{};
  g.M = M; g.N = N; g.K = K; g.dtype = a_fmt; g.dtype_b = b_fmt;
  g.A = A; g.lda = lda; g.a_kmajor = a_major == 'k';
  g.B = B; g.ldb = ldb; g.b_kmajor = b_major == 'k';
  g.SFA = SFA; g.ld_sfa = ld_sfa; g.SFB = SFB; g.ld_sfb = ld_sfb;
  g.D = D; g.ldd = ldd; g.negate = neg_a ^ neg_b; g.accum = accum;
  g.ew_op = ew.op; g.ew_scale = ew.scale; g.ew_bias = ew.bias;
  g.mx_window = window;
  hipError_t e = bsm::launch_gemm_mx(g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, name);
  return ok();
}

int bsm_gemm_block_scale(int64_t M, int64_t N, int64_t K, int32_t a_fmt, const void* A, int64_t lda,
                         const uint8_t* SFA, int64_t ld_sfa, int32_t b_fmt, const void* B, int64_t ldb,
                         const uint8_t* SFB, int64_t ld_sfb, float* D, int64_t ldd, int neg_a, int neg_b, int accum,
                         void* stream) {
  return gemm_block_scale(M, N, K, a_fmt, A, lda, 'k', SFA, ld_sfa, b_fmt, B, ldb, 'k', SFB, ld_sfb, D, ldd, neg_a,
                          neg_b, accum, bsm_ewise{BSM_EW_NONE, 1.0f, 0.0f}, stream, "bsm_gemm_block_scale");
}

int bsm_gemm_block_scale_ewise(int64_t M, int64_t N, int64_t K, int32_t a_fmt, const void* A, int64_t lda,
                               const uint8_t* SFA, int64_t ld_sfa, int32_t b_fmt, const void* B, int64_t ldb,
                               const uint8_t* SFB, int64_t ld_sfb, float* D, int64_t ldd, int neg_a, int neg_b,
                               int accum, const bsm_ewise* ew, void* stream) {
  int rc;
  if ((rc = check_ewise(ew))) return rc;
  return gemm_block_scale(M, N, K, a_fmt, A, lda, 'k', SFA, ld_sfa, b_fmt, B, ldb, 'k', SFB, ld_sfb, D, ldd, neg_a,
                          neg_b, accum, *ew, stream, "bsm_gemm_block_scale_ewise");
}

int bsm_gemm_block_scale_major(int64_t M, int64_t N, int64_t K, int32_t a_fmt, const void* A, int64_t lda,
                               char a_major, const uint8_t* SFA, int64_t ld_sfa, int32_t b_fmt, const void* B,
                               int64_t ldb, char b_major, const uint8_t* SFB, int64_t ld_sfb, float* D, int64_t ldd,
                               int neg_a, int neg_b, int accum, const bsm_ewise* ew, void* stream) {
  int rc;
  if (ew && (rc = check_ewise(ew))) return rc;
  return gemm_block_scale(M, N, K, a_fmt, A, lda, a_major, SFA, ld_sfa, b_fmt, B, ldb, b_major, SFB, ld_sfb, D, ldd,
                          neg_a, neg_b, accum, ew ? *ew : bsm_ewise{BSM_EW_NONE, 1.0f, 0.0f}, stream,
                          "bsm_gemm_block_scale_major");
}

int bsm_gemm_block_scale_fastacc(int64_t M, int64_t N, int64_t K, int32_t a_fmt, const void* A, int64_t lda,
                                 const uint8_t* SFA, int64_t ld_sfa, int32_t b_fmt, const void* B, int64_t ldb,
                                 const uint8_t* SFB, int64_t ld_sfb, float* D, int64_t ldd, int neg_a, int neg_b,
                                 int accum, const bsm_ewise* ew, void* stream) {
  int rc;
  if (ew && (rc = check_ewise(ew))) return rc;
  return gemm_block_scale(M, N, K, a_fmt, A, lda, 'k', SFA, ld_sfa, b_fmt, B, ldb, 'k', SFB, ld_sfb, D, ldd, neg_a,
                          neg_b, accum, ew ? *ew : bsm_ewise{BSM_EW_NONE, 1.0f, 0.0f}, stream,
                          "bsm_gemm_block_scale_fastacc", 1);
}

int bsm_tile_add_scalar_f32(const float* src, float* dst, int64_t n, float s, void* stream) {
  if (n < 0) return fail(BSM_E_SHAPE, "n = %lld is negative", (long long)n);
  if (n == 0) return ok();
  if (!src || !dst) return fail(BSM_E_NULL, "src or dst is NULL");
  if ((uintptr_t)src % 16 || (uintptr_t)dst % 16) return fail(BSM_E_ALIGN, "src and dst must be 16-byte aligned");
  const Range a{(uintptr_t)src, (uintptr_t)(src + n)}, b{(uintptr_t)dst, (uintptr_t)(dst + n)};
  if (src != dst && overlap(a, b)) return fail(BSM_E_ALIAS, "src and dst overlap without being equal");
  hipError_t e = bsm::launch_add_scalar_f32(src, dst, n, s, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsm_tile_add_scalar_f32");
  return ok();
}

int bsm_debug_stream_mix_bf16(const void* src, void* dst, void* add, int64_t n, void* stream) {
  if (n < 0 || n % 8) return fail(BSM_E_SHAPE, "n = %lld must be a non-negative multiple of 8", (long long)n);
  if (n == 0) return ok();
  if (!src || !dst || !add) return fail(BSM_E_NULL, "src, dst or add is NULL");
  if ((uintptr_t)src % 16 || (uintptr_t)dst % 16 || (uintptr_t)add % 16)
    return fail(BSM_E_ALIGN, "src, dst and add must be 16-byte aligned");
  const uintptr_t nb = (uintptr_t)n * 2;
  const Range a{(uintptr_t)src, (uintptr_t)src + nb}, b{(uintptr_t)dst, (uintptr_t)dst + nb},
      c{(uintptr_t)add, (uintptr_t)add + nb};
  if (overlap(a, b) || overlap(a, c) || overlap(b, c)) return fail(BSM_E_ALIAS, "src, dst and add must not overlap");
  hipError_t e = bsm::launch_stream_mix_bf16(src, dst, add, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsm_debug_stream_mix_bf16");
  return ok();
}

int bsm_debug_mfma_loop(int32_t kind, int64_t workgroups, int32_t iters, float* out, void* stream) {
  if (kind != BSM_BF16 && kind != BSM_E4M3 && kind != BSM_E2M1)
    return fail(BSM_E_DTYPE, "kind %d: the MFMA loop takes BSM_BF16, BSM_E4M3 or BSM_E2M1", kind);
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20))
    return fail(BSM_E_SHAPE, "workgroups = %lld and iters = %d must lie in 1 .. 2^20", (long long)workgroups, iters);
  if (!out) return fail(BSM_E_NULL, "out is NULL");
  if ((uintptr_t)out % 4) return fail(BSM_E_ALIGN, "out must be 4-byte aligned");
  hipError_t e = bsm::launch_mfma_loop(kind, workgroups, iters, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsm_debug_mfma_loop");
  return ok();
}

void bsm_debug_fragment_shape(int64_t* rows, int64_t* kdim) {
  if (rows) *rows = bsm::kDenseTileRows;
  if (kdim) *kdim = bsm::kDenseTileK;
}

int bsm_debug_fragments(const uint16_t* src, int64_t rows, int64_t kdim, char major, uint16_t* dump, void* stream) {
  if (!src || !dump) return fail(BSM_E_NULL, "src or dump is NULL");
  if (rows != bsm::kDenseTileRows || kdim != bsm::kDenseTileK)
    return fail(BSM_E_SHAPE, "tile must be %d x %d (got %lld x %lld)", bsm::kDenseTileRows, bsm::kDenseTileK,
                (long long)rows, (long long)kdim);
  if (major != 'k' && major != 'm') return fail(BSM_E_MAJOR, "major '%c' is not 'k' or 'm'", major);
  if ((uintptr_t)src % 16 || (uintptr_t)dump % 16) return fail(BSM_E_ALIGN, "src and dump must be 16-byte aligned");
  hipError_t e = bsm::launch_debug_fragments(src, major == 'k', dump, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsm_debug_fragments");
  return ok();
}

}  // extern "C"
