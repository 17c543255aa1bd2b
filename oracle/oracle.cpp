// oracle.cpp - reference CPU implementation of the block-scaled tile-matrix hot path.
//
// TEST INFRASTRUCTURE ONLY. This file is the reference the HIP library is compared
// against. Only the test-suite, the smoke check and the CPU-baseline leg of the
// benchmark may load it. It shares no code, header, table or constant with the
// library under block_scaled_matrix_amd/: it is plain, slow, serial-per-output C++
// that computes every floating-point result in double precision and decodes every
// storage format bit by bit.
//
// Pages cited (web documentation of Apache TVM "TIRx"):
//   [TP]  "Explicit CUDA tile patterns"
//   [TMA] "cp.async.bulk.tensor / cp.reduce.async.bulk.tensor"
//   [LDM] "ldmatrix / stmatrix"
//   [TOE] "Tile Operands and Execution"
//   [MMA] "tcgen05.mma"
// Storage formats the pages only name (e4m3, e5m2, the 6-bit e2m3 / e3m2, e2m1, the 8-bit
// scale) follow the public OCP Microscaling Formats (MX) v1.0 specification, section 5.
//
// Every function returns 0 on success and a negative value on an argument it
// cannot interpret; it never guesses.
//
// Parity status of each function (what pins it is in tests/test_oracle_*.py):
//   decoders (fp6 included), encoders, swizzle, box load/store/reduce, gather4/scatter4, grid copy,
//   add_scalar, ldmatrix image, dense GEMM, block-scaled GEMM, silu_affine epilogue:
//   all pinned (none unpinned).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

// Storage-format codes of this oracle (its own numbering; the Python wrapper maps names).
enum OracleDtype {
  OD_U8 = 0, OD_U16 = 1, OD_U32 = 2, OD_F16 = 3, OD_BF16 = 4, OD_F32 = 5,
  OD_E4M3 = 6, OD_E2M1 = 7, OD_E8M0 = 8, OD_E5M2 = 9, OD_E2M3 = 10, OD_E3M2 = 11
};

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// ---------------------------------------------------------------------------
// C1. Decoders: storage bits -> exact double.
// ---------------------------------------------------------------------------

// IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double oracle_dec_f16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = std::ldexp((double)m, -24);
  else v = std::ldexp(1024.0 + m, e - 25);
  return s ? -v : v;
}

// bfloat16: the top half of an IEEE binary32 (8 exponent bits, bias 127, 7 fraction bits).
double oracle_dec_bf16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 7) & 255, m = h & 127;
  double v;
  if (e == 255) v = m ? NAN : INFINITY;
  else if (e == 0) v = std::ldexp((double)m, -133);
  else v = std::ldexp(128.0 + m, e - 134);
  return s ? -v : v;
}

// IEEE binary32.
double oracle_dec_f32(uint32_t u) {
  int s = (u >> 31) & 1, e = (u >> 23) & 255;
  uint32_t m = u & 0x7FFFFFu;
  double v;
  if (e == 255) v = m ? NAN : INFINITY;
  else if (e == 0) v = std::ldexp((double)m, -149);
  else v = std::ldexp(8388608.0 + m, e - 150);
  return s ? -v : v;
}

// OCP E4M3 ("fn" variant): s.eeee.mmm, bias 7, no infinities, S.1111.111 is NaN,
// subnormals m * 2^-9, largest finite 448 (OCP MX v1.0, section 5.3).
double oracle_dec_e4m3(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = std::ldexp((double)m, -9);
  else v = std::ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

// OCP E5M2: s.eeeee.mm, bias 15, IEEE-like: exponent 31 is infinity (m == 0) or NaN,
// subnormals m * 2^-16, largest finite 57344 (OCP MX v1.0, section 5.3).
double oracle_dec_e5m2(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 2) & 31, m = c & 3;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = std::ldexp((double)m, -16);
  else v = std::ldexp(4.0 + m, e - 17);
  return s ? -v : v;
}

// OCP E2M1: s.ee.m, bias 1, no infinities or NaN; subnormal m * 2^-1
// (OCP MX v1.0, section 5.3.3). Only the low 4 bits of `nib` are used.
double oracle_dec_e2m1(uint8_t nib) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double v;
  if (e == 0) v = 0.5 * m;
  else v = std::ldexp(2.0 + m, e - 2);
  return s ? -v : v;
}

// OCP E2M3 (FP6): s.ee.mmm, bias 1, no infinities or NaN; subnormals m * 2^-3,
// largest 7.5 (OCP MX v1.0, section 5.3.2). Only the low 6 bits of `c` are used.
double oracle_dec_e2m3(uint8_t c) {
  int s = (c >> 5) & 1, e = (c >> 3) & 3, m = c & 7;
  double v = e == 0 ? std::ldexp((double)m, -3) : std::ldexp(8.0 + m, e - 4);
  return s ? -v : v;
}

// OCP E3M2 (FP6): s.eee.mm, bias 3, no infinities or NaN; subnormals m * 2^-4,
// largest 28 (OCP MX v1.0, section 5.3.2). Only the low 6 bits of `c` are used.
double oracle_dec_e3m2(uint8_t c) {
  int s = (c >> 5) & 1, e = (c >> 2) & 7, m = c & 3;
  double v = e == 0 ? std::ldexp((double)m, -4) : std::ldexp(4.0 + m, e - 5);
  return s ? -v : v;
}

// Packed 6-bit storage (a reading: the pages name the 6-bit kinds but no memory layout):
// element i of a row is bits 6i .. 6i+5 of the row's bytes read as one little-endian bit
// string, so four elements fill three bytes.
static uint8_t fp6_code(const uint8_t* row, int64_t i) {
  const int64_t bit = 6 * i;
  const unsigned lo = row[bit >> 3];
  const unsigned hi = ((bit & 7) > 2) ? row[(bit >> 3) + 1] : 0u;
  return (uint8_t)(((lo | (hi << 8)) >> (bit & 7)) & 63);
}

// OCP E8M0 scale: an unsigned biased exponent, value 2^(c-127); 0xFF is NaN
// (OCP MX v1.0, section 5.4.1).
double oracle_dec_e8m0(uint8_t c) {
  if (c == 255) return NAN;
  return std::ldexp(1.0, (int)c - 127);
}

// ---------------------------------------------------------------------------
// Encoders: double -> storage bits, round-to-nearest-even, IEEE overflow to
// infinity and gradual underflow. Written as the textbook definition: pick the
// binade of |x|, express |x| in units of that binade's spacing, round that
// quotient to the nearest integer (ties to even), renormalise on carry.
// ---------------------------------------------------------------------------
static uint32_t enc_ieee(double x, int ebits, int mbits) {
  const int bias = (1 << (ebits - 1)) - 1;
  const int emin = 1 - bias, emax = bias;
  const uint32_t sign = std::signbit(x) ? (1u << (ebits + mbits)) : 0u;
  const uint32_t expmask = (1u << ebits) - 1;
  if (std::isnan(x)) return (expmask << mbits) | (1u << (mbits - 1));  // canonical quiet NaN
  double a = std::fabs(x);
  if (std::isinf(a)) return sign | (expmask << mbits);
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);          // a = f * 2^e2, f in [0.5, 1)
  int E = e2 - 1;              // exponent of the leading bit
  if (E < emin) E = emin;      // subnormal range shares emin's spacing
  double q = std::ldexp(a, mbits - E);  // |x| in units of 2^(E - mbits); exact
  double n = std::nearbyint(q);         // default rounding mode: to nearest, ties to even
  if (n >= std::ldexp(1.0, mbits + 1)) { n = std::ldexp(n, -1); E += 1; }  // carry into next binade
  if (E > emax) return sign | (expmask << mbits);                         // overflow -> inf
  uint32_t ni = (uint32_t)n;
  if (ni < (1u << mbits)) return sign | ni;                               // subnormal (E == emin)
  return sign | ((uint32_t)(E + bias) << mbits) | (ni - (1u << mbits));
}
uint16_t oracle_enc_f16(double x) { return (uint16_t)enc_ieee(x, 5, 10); }
uint16_t oracle_enc_bf16(double x) { return (uint16_t)enc_ieee(x, 8, 7); }
uint32_t oracle_enc_f32(double x) { return enc_ieee(x, 8, 23); }

// Bulk helpers (tests decode whole arrays through these).
int oracle_decode_array(int dtype, const void* src, int64_t n, double* out) {
  const uint8_t* b = (const uint8_t*)src;
  for (int64_t i = 0; i < n; i++) {
    switch (dtype) {
      case OD_U8: out[i] = b[i]; break;
      case OD_U16: { uint16_t v; std::memcpy(&v, b + 2 * i, 2); out[i] = v; break; }
      case OD_U32: { uint32_t v; std::memcpy(&v, b + 4 * i, 4); out[i] = v; break; }
      case OD_F16: { uint16_t v; std::memcpy(&v, b + 2 * i, 2); out[i] = oracle_dec_f16(v); break; }
      case OD_BF16: { uint16_t v; std::memcpy(&v, b + 2 * i, 2); out[i] = oracle_dec_bf16(v); break; }
      case OD_F32: { uint32_t v; std::memcpy(&v, b + 4 * i, 4); out[i] = oracle_dec_f32(v); break; }
      case OD_E4M3: out[i] = oracle_dec_e4m3(b[i]); break;
      case OD_E5M2: out[i] = oracle_dec_e5m2(b[i]); break;
      case OD_E2M1: out[i] = oracle_dec_e2m1((b[i / 2] >> (4 * (i & 1))) & 15); break;
      case OD_E8M0: out[i] = oracle_dec_e8m0(b[i]); break;
      case OD_E2M3: out[i] = oracle_dec_e2m3(fp6_code(b, i)); break;
      case OD_E3M2: out[i] = oracle_dec_e3m2(fp6_code(b, i)); break;
      default: return -1;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Swizzle of a shared box image ([TP] "TMA" and "Shared matrix descriptors";
// [TMA] "Call parameters": swizzle 0/1/2/3 = none/32B/64B/128B).
// The pages give mode 3 as offset ^ ((offset >> 3) & 112) with a 1024-byte
// period and list periods 256/512/1024 for modes 1/2/3. Reading for modes 1
// and 2: the same XOR of bits 7.. into the 16-byte chunk index, restricted to
// log2(period/128) bits, i.e. masks 16 and 48.
// ---------------------------------------------------------------------------
int64_t oracle_swizzle(int64_t off, int mode) {
  if (mode == 0) return off;
  int64_t mask = 16 * ((1 << mode) - 1);  // 16, 48, 112
  return off ^ ((off >> 3) & mask);
}

static int elem_size(int dtype) {
  switch (dtype) {
    case OD_U8: case OD_E4M3: case OD_E5M2: case OD_E8M0: return 1;
    case OD_U16: case OD_F16: case OD_BF16: return 2;
    case OD_U32: case OD_F32: return 4;
    default: return 0;  // E2M1 is sub-byte: box copies treat packed fp4 as U8
  }
}

// Canonical NaN used for oob_fill = 1 (the pages say only "NaN for supported
// floating-point formats"; this oracle takes the canonical quiet NaN of each format).
static int nan_bits(int dtype, uint8_t* out) {
  switch (dtype) {
    case OD_F32: { uint32_t v = 0x7FC00000u; std::memcpy(out, &v, 4); return 0; }
    case OD_F16: { uint16_t v = 0x7E00; std::memcpy(out, &v, 2); return 0; }
    case OD_BF16: { uint16_t v = 0x7FC0; std::memcpy(out, &v, 2); return 0; }
    case OD_E4M3: out[0] = 0x7F; return 0;
    case OD_E5M2: out[0] = 0x7E; return 0;  // exponent 31, quiet-NaN mantissa (the f16 0x7E00 top byte)
    default: return -1;
  }
}

static int64_t image_elems(int rank, const int32_t* box, const int32_t* estr, int64_t* ext) {
  int64_t n = 1;
  for (int i = 0; i < rank; i++) {
    ext[i] = (box[i] + estr[i] - 1) / estr[i];  // ceil(box / element_stride)
    n *= ext[i];
  }
  return n;
}

// ---------------------------------------------------------------------------
// C2. Box load ([TMA] "Call parameters", "Data representation", "Operand
// specification"; [TP] "TMA"). Image element j (row-major over extents
// ceil(box/element_strides), outer to inner) reads global coordinate
// g = coords + j * element_strides; any coordinate outside [0, dims) yields the
// fill value (0: zero bytes, 1: NaN). The compact byte offset linear(j)*esize
// is then permuted by the swizzle.
// Global layout: element g lives at base + sum_i g_i * strides[i] (bytes).
// ---------------------------------------------------------------------------
int oracle_box_load(const void* base, int dtype, int rank, const int64_t* dims,
                    const int64_t* strides, const int32_t* box, const int32_t* estr,
                    const int64_t* coords, int swizzle, int fill, void* image) {
  const int es = elem_size(dtype);
  if (es == 0 || rank < 1 || rank > 5 || swizzle < 0 || swizzle > 3) return -1;
  uint8_t fillv[4] = {0, 0, 0, 0};
  if (fill == 1 && nan_bits(dtype, fillv) != 0) return -2;
  if (fill != 0 && fill != 1) return -2;
  int64_t ext[5];
  const int64_t n = image_elems(rank, box, estr, ext);
  const uint8_t* src = (const uint8_t*)base;
  uint8_t* img = (uint8_t*)image;
  for (int64_t lin = 0; lin < n; lin++) {
    int64_t rem = lin, off = 0;
    bool inb = true;
    for (int i = rank - 1; i >= 0; i--) {
      int64_t j = rem % ext[i];
      rem /= ext[i];
      int64_t g = coords[i] + j * estr[i];
      if (g < 0 || g >= dims[i]) inb = false;
      else off += g * strides[i];
    }
    for (int b = 0; b < es; b++) {
      uint8_t v = inb ? src[off + b] : fillv[b];
      img[oracle_swizzle(lin * es + b, swizzle)] = v;
    }
  }
  return 0;
}

static void reduce_add_elem(int dtype, uint8_t* dst, const uint8_t* val) {
  // dst <- round(dst + val), the exact sum rounded once to the destination format.
  if (dtype == OD_F32) {
    uint32_t a, b; std::memcpy(&a, dst, 4); std::memcpy(&b, val, 4);
    uint32_t r = oracle_enc_f32(oracle_dec_f32(a) + oracle_dec_f32(b));
    std::memcpy(dst, &r, 4);
  } else if (dtype == OD_F16) {
    uint16_t a, b; std::memcpy(&a, dst, 2); std::memcpy(&b, val, 2);
    uint16_t r = oracle_enc_f16(oracle_dec_f16(a) + oracle_dec_f16(b));
    std::memcpy(dst, &r, 2);
  } else {  // OD_BF16
    uint16_t a, b; std::memcpy(&a, dst, 2); std::memcpy(&b, val, 2);
    uint16_t r = oracle_enc_bf16(oracle_dec_bf16(a) + oracle_dec_bf16(b));
    std::memcpy(dst, &r, 2);
  }
}

// ---------------------------------------------------------------------------
// C3. Box store / add-reduction ([TMA] "Stores, reductions, and completion":
// same box/coordinate contract with the global operand as destination; the
// reduction destination holds its starting value). Reading where the pages are
// silent: image elements whose global coordinate is out of bounds are not
// written. The add is the exact sum rounded once (round-to-nearest-even) to the
// destination format; it is defined for f32, f16 and bf16.
// ---------------------------------------------------------------------------
int oracle_box_store(void* base, int dtype, int rank, const int64_t* dims,
                     const int64_t* strides, const int32_t* box, const int32_t* estr,
                     const int64_t* coords, int swizzle, const void* image, int reduce_add) {
  const int es = elem_size(dtype);
  if (es == 0 || rank < 1 || rank > 5 || swizzle < 0 || swizzle > 3) return -1;
  if (reduce_add && dtype != OD_F32 && dtype != OD_F16 && dtype != OD_BF16) return -3;
  int64_t ext[5];
  const int64_t n = image_elems(rank, box, estr, ext);
  uint8_t* dst = (uint8_t*)base;
  const uint8_t* img = (const uint8_t*)image;
  for (int64_t lin = 0; lin < n; lin++) {
    int64_t rem = lin, off = 0;
    bool inb = true;
    for (int i = rank - 1; i >= 0; i--) {
      int64_t j = rem % ext[i];
      rem /= ext[i];
      int64_t g = coords[i] + j * estr[i];
      if (g < 0 || g >= dims[i]) inb = false;
      else off += g * strides[i];
    }
    if (!inb) continue;
    uint8_t v[4];
    for (int b = 0; b < es; b++) v[b] = img[oracle_swizzle(lin * es + b, swizzle)];
    if (reduce_add) reduce_add_elem(dtype, dst + off, v);
    else std::memcpy(dst + off, v, es);
  }
  return 0;
}

// ---------------------------------------------------------------------------
// C3b. Row gather and scatter of four rows ([TMA] "Gather4 and scatter4": a 2-D
// global operand, a box of one row by `width` elements, a shared image of four such
// rows, and four explicit row coordinates that need not be consecutive). Reading:
// the column start `col` is the inner coordinate of the box; image row i holds
// tensor row rows[i], elements col .. col + width - 1. The image is the compact
// row-major (4, width) array, permuted by the swizzle as one image. Gather: an
// element whose row or column is out of range reads the fill. Scatter: such elements
// are not written; rows are written in the order i = 0..3, so a repeated row keeps
// the last one.
// ---------------------------------------------------------------------------
int oracle_gather4(const void* base, int dtype, const int64_t* dims, const int64_t* strides, int32_t width,
                   int64_t col, const int64_t* rows, int swizzle, int fill, void* image) {
  const int es = elem_size(dtype);
  if (es == 0 || width < 1 || swizzle < 0 || swizzle > 3) return -1;
  if (fill != 0 && fill != 1) return -2;
  uint8_t fillv[4] = {0, 0, 0, 0};
  if (fill == 1 && nan_bits(dtype, fillv) != 0) return -2;
  const uint8_t* src = (const uint8_t*)base;
  uint8_t* img = (uint8_t*)image;
  for (int i = 0; i < 4; i++) {
    for (int64_t j = 0; j < width; j++) {
      const int64_t r = rows[i], c = col + j;
      const bool inb = r >= 0 && r < dims[0] && c >= 0 && c < dims[1];
      const int64_t lin = (int64_t)i * width + j;
      for (int b = 0; b < es; b++)
        img[oracle_swizzle(lin * es + b, swizzle)] = inb ? src[r * strides[0] + c * strides[1] + b] : fillv[b];
    }
  }
  return 0;
}

int oracle_scatter4(void* base, int dtype, const int64_t* dims, const int64_t* strides, int32_t width,
                    int64_t col, const int64_t* rows, int swizzle, const void* image) {
  const int es = elem_size(dtype);
  if (es == 0 || width < 1 || swizzle < 0 || swizzle > 3) return -1;
  uint8_t* dst = (uint8_t*)base;
  const uint8_t* img = (const uint8_t*)image;
  for (int i = 0; i < 4; i++) {
    for (int64_t j = 0; j < width; j++) {
      const int64_t r = rows[i], c = col + j;
      if (r < 0 || r >= dims[0] || c < 0 || c >= dims[1]) continue;
      const int64_t lin = (int64_t)i * width + j;
      for (int b = 0; b < es; b++) dst[r * strides[0] + c * strides[1] + b] = img[oracle_swizzle(lin * es + b, swizzle)];
    }
  }
  return 0;
}

// Bytes one image occupies in an image buffer: the compact image rounded up to
// 128 bytes (every atom origin is 128-byte aligned, [TMA] "Operand
// specification") or, when swizzled, to the whole swizzle period 2^(7+mode).
int64_t oracle_image_stride(int dtype, int rank, const int32_t* box, const int32_t* estr, int swizzle) {
  int64_t ext[5];
  int64_t bytes = image_elems(rank, box, estr, ext) * elem_size(dtype);
  int64_t align = swizzle ? (int64_t(1) << (7 + swizzle)) : 128;
  return (bytes + align - 1) / align * align;
}

// Grid round trip: one box at every tile coordinate t * box (t over
// ceil(dims/box) per axis), loaded into an image, then stored to `dst`
// and/or add-reduced into `dst_add` at the same coordinates. The boxes do not
// overlap, so the result is independent of their order. Any of dst/dst_add
// may be NULL (not both). All three tensors share dims, strides and dtype.
int oracle_box_copy_grid(const void* src, void* dst, void* dst_add, int dtype, int rank,
                         const int64_t* dims, const int64_t* strides, const int32_t* box,
                         const int32_t* estr, int swizzle, int fill) {
  if (!dst && !dst_add) return -4;
  if (rank < 1 || rank > 5) return -1;
  int64_t tiles[5], ntiles = 1;
  for (int i = 0; i < rank; i++) { tiles[i] = (dims[i] + box[i] - 1) / box[i]; ntiles *= tiles[i]; }
  const int64_t stride = oracle_image_stride(dtype, rank, box, estr, swizzle);
  std::vector<uint8_t> img((size_t)stride);
  for (int64_t t = 0; t < ntiles; t++) {
    int64_t rem = t, coords[5];
    for (int i = rank - 1; i >= 0; i--) { coords[i] = (rem % tiles[i]) * box[i]; rem /= tiles[i]; }
    int rc = oracle_box_load(src, dtype, rank, dims, strides, box, estr, coords, swizzle, fill, img.data());
    if (rc) return rc;
    if (dst) { rc = oracle_box_store(dst, dtype, rank, dims, strides, box, estr, coords, swizzle, img.data(), 0); if (rc) return rc; }
    if (dst_add) { rc = oracle_box_store(dst_add, dtype, rank, dims, strides, box, estr, coords, swizzle, img.data(), 1); if (rc) return rc; }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// C4. Add a scalar to every float32 element ([TOE] "A Load, Compute, and Store
// Example": every value of the tile plus one; [TP] "Scalar compositions").
// The float32 sum is the exact sum rounded once to float32.
// ---------------------------------------------------------------------------
int oracle_add_scalar_f32(const float* src, float* dst, int64_t n, float s) {
  for (int64_t i = 0; i < n; i++) {
    uint32_t a, b; std::memcpy(&a, &src[i], 4); std::memcpy(&b, &s, 4);
    uint32_t r = oracle_enc_f32(oracle_dec_f32(a) + oracle_dec_f32(b));
    std::memcpy(&dst[i], &r, 4);
  }
  return 0;
}

// ---------------------------------------------------------------------------
// C5. ldmatrix register image ([LDM] "Address providers and result owners",
// "Parameterized layouts", "Code generation", "Transpose and stores"; [TP]
// "ldmatrix with interleaved rows and separated registers").
// One warp instruction over N in {1,2,4} 8x8 matrices of 16-bit elements.
// Matrix i, row j starts at byte offset row_offsets[8*i + j] of `shared` (its
// address is what lane 8*i+j provides; 16-byte aligned, four 32-bit words).
// Result word (matrix i, row j, word w) is owned by lane 4*j + w and holds
// image[i][j][2w] (low 16 bits) and image[i][j][2w+1] (high 16 bits), where
// image[i][j][c] = S_i[j][c] without transpose and S_i[c][j] with transpose
// (S_i[r][c] = 16-bit element c of row r of matrix i).
// Output: regs[lane * N + i] for lanes 0..31.
// ---------------------------------------------------------------------------
int oracle_ldmatrix(const void* shared, const int64_t* row_offsets, int nmat, int trans,
                    uint32_t* regs) {
  if (nmat != 1 && nmat != 2 && nmat != 4) return -1;
  for (int r = 0; r < 8 * nmat; r++) if (row_offsets[r] % 16 != 0) return -2;
  const uint8_t* sm = (const uint8_t*)shared;
  auto S = [&](int i, int r, int c) -> uint16_t {
    uint16_t v;
    std::memcpy(&v, sm + row_offsets[8 * i + r] + 2 * c, 2);
    return v;
  };
  for (int lane = 0; lane < 32; lane++) {
    int j = lane / 4, w = lane % 4;  // the word this lane owns in every matrix
    for (int i = 0; i < nmat; i++) {
      uint16_t lo = trans ? S(i, 2 * w, j) : S(i, j, 2 * w);
      uint16_t hi = trans ? S(i, 2 * w + 1, j) : S(i, j, 2 * w + 1);
      regs[lane * nmat + i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// C6/C7. GEMM. D[m,n] = (accum ? D0[m,n] : 0) + sigma * sum_k A(m,k) * B(n,k),
// sigma = (neg_a ? -1 : 1) * (neg_b ? -1 : 1).
//  - Orientation: B is the (N,K) operand and the product is A times B
//    transposed ([MMA] "Operand specification" canonical shapes and
//    "Example: four K16 issues", checked against a @ b.T; [TP] "Warp MMA").
//  - Major order ([MMA] "Shared descriptors are byte-stride contracts": K-major
//    rows enumerate M/N, MN-major rows enumerate K): a_major 'k' stores A(m,k)
//    at A[m*lda + k]; 'm' stores it at A[k*lda + m]. b_major 'k': B(n,k) at
//    B[n*ldb + k]; 'n': at B[k*ldb + n].
//  - accum ([MMA] "Call parameters" and "Code generation"): the first K step
//    uses the existing D iff accum; every later step accumulates.
//  - neg_a/neg_b ([MMA] "Call parameters"): negate the operand.
// Also returns bound[m,n] = sum_k |A(m,k) * B(n,k)| (the error scale).
// Rows [m_begin, m_end) are computed; ref/bound are (m_end-m_begin) x N, row-major.
// ---------------------------------------------------------------------------
static double load_op_dense(int dtype, const uint8_t* p, int64_t idx) {
  uint16_t v;
  std::memcpy(&v, p + 2 * idx, 2);
  return dtype == OD_F16 ? oracle_dec_f16(v) : oracle_dec_bf16(v);
}

int oracle_gemm(int64_t M, int64_t N, int64_t K, int dtype,
                const void* A, int64_t lda, int a_major, const void* B, int64_t ldb, int b_major,
                const float* D0, int64_t ldd, int neg_a, int neg_b, int accum,
                int64_t m_begin, int64_t m_end, double* ref, double* bound) {
  if (dtype != OD_F16 && dtype != OD_BF16) return -1;
  if (M < 0 || N < 0 || K < 0 || m_begin < 0 || m_end > M || m_begin > m_end) return -2;
  if ((a_major != 'k' && a_major != 'm') || (b_major != 'k' && b_major != 'n')) return -3;
  if (accum && !D0) return -4;
  const uint8_t* pa = (const uint8_t*)A;
  const uint8_t* pb = (const uint8_t*)B;
  const double sigma = (neg_a ? -1.0 : 1.0) * (neg_b ? -1.0 : 1.0);
#pragma omp parallel for schedule(dynamic)
  for (int64_t m = m_begin; m < m_end; m++) {
    for (int64_t n = 0; n < N; n++) {
      double s = 0.0, b = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double a = load_op_dense(dtype, pa, a_major == 'k' ? m * lda + k : k * lda + m);
        double bb = load_op_dense(dtype, pb, b_major == 'k' ? n * ldb + k : k * ldb + n);
        s += a * bb;
        b += std::fabs(a * bb);
      }
      double d0 = accum ? (double)D0[m * ldd + n] : 0.0;
      ref[(m - m_begin) * N + n] = d0 + sigma * s;
      bound[(m - m_begin) * N + n] = b;
    }
  }
  return 0;
}

// Same as oracle_gemm but for an explicit list of output points (m[i], n[i]).
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, int dtype,
                       const void* A, int64_t lda, int a_major, const void* B, int64_t ldb, int b_major,
                       const float* D0, int64_t ldd, int neg_a, int neg_b, int accum,
                       const int64_t* pm, const int64_t* pn, int64_t npts, double* ref, double* bound) {
  if (dtype != OD_F16 && dtype != OD_BF16) return -1;
  if ((a_major != 'k' && a_major != 'm') || (b_major != 'k' && b_major != 'n')) return -3;
  if (accum && !D0) return -4;
  const uint8_t* pa = (const uint8_t*)A;
  const uint8_t* pb = (const uint8_t*)B;
  const double sigma = (neg_a ? -1.0 : 1.0) * (neg_b ? -1.0 : 1.0);
  for (int64_t i = 0; i < npts; i++) if (pm[i] < 0 || pm[i] >= M || pn[i] < 0 || pn[i] >= N) return -2;
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < npts; i++) {
    const int64_t m = pm[i], n = pn[i];
    double s = 0.0, b = 0.0;
    for (int64_t k = 0; k < K; k++) {
      double a = load_op_dense(dtype, pa, a_major == 'k' ? m * lda + k : k * lda + m);
      double bb = load_op_dense(dtype, pb, b_major == 'k' ? n * ldb + k : k * ldb + n);
      s += a * bb;
      b += std::fabs(a * bb);
    }
    double d0 = accum ? (double)D0[m * ldd + n] : 0.0;
    ref[i] = d0 + sigma * s;
    bound[i] = b;
  }
  return 0;
}

// Block-scaled operand value ([MMA] "Weight-stationary and block scaling":
// block-scaled kinds carry 8-bit scale factors per K group; [TP] "tcgen05 MMA").
// Reading (OCP MX v1.0, section 5): one E8M0 scale per 32 consecutive K
// elements starting at k = 0; the operand value is decode(element) * 2^(s-127).
// Storage ([MMA] "Call parameters": a_major / b_major select "k" or "mn"): K-major
// element (r,k) at index r*ld + k, MN-major (K rows, M or N contiguous) at k*ld + r; for
// packed E2M1 the index selects byte idx/2 and the low nibble for even idx; for the 6-bit
// formats, bits 6 idx .. 6 idx + 5 of the operand's little-endian bit string (ld * 6 is a
// multiple of 8, so every row starts on a byte). Scales stay per (r, k/32) either way.
static bool mx_fmt(int f) {
  return f == OD_E4M3 || f == OD_E5M2 || f == OD_E2M1 || f == OD_E2M3 || f == OD_E3M2;
}

static double load_op_scaled(int fmt, const uint8_t* p, int64_t ld, int mn, const uint8_t* sf,
                             int64_t ld_sf, int64_t r, int64_t k) {
  int64_t idx = mn ? k * ld + r : r * ld + k;
  double v;
  if (fmt == OD_E4M3) v = oracle_dec_e4m3(p[idx]);
  else if (fmt == OD_E5M2) v = oracle_dec_e5m2(p[idx]);
  else if (fmt == OD_E2M3) v = oracle_dec_e2m3(fp6_code(p, idx));
  else if (fmt == OD_E3M2) v = oracle_dec_e3m2(fp6_code(p, idx));
  else v = oracle_dec_e2m1((p[idx >> 1] >> (4 * (idx & 1))) & 15);
  return v * oracle_dec_e8m0(sf[r * ld_sf + k / 32]);
}

int oracle_gemm_block_scale(int64_t M, int64_t N, int64_t K,
                            int a_fmt, const void* A, int64_t lda, const uint8_t* SFA, int64_t ld_sfa,
                            int b_fmt, const void* B, int64_t ldb, const uint8_t* SFB, int64_t ld_sfb,
                            const float* D0, int64_t ldd, int neg_a, int neg_b, int accum,
                            int64_t m_begin, int64_t m_end, double* ref, double* bound, int a_mn, int b_mn) {
  if (!mx_fmt(a_fmt) || !mx_fmt(b_fmt)) return -1;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || m_begin < 0 || m_end > M || m_begin > m_end) return -2;
  if (accum && !D0) return -4;
  const uint8_t* pa = (const uint8_t*)A;
  const uint8_t* pb = (const uint8_t*)B;
  const double sigma = (neg_a ? -1.0 : 1.0) * (neg_b ? -1.0 : 1.0);
#pragma omp parallel for schedule(dynamic)
  for (int64_t m = m_begin; m < m_end; m++) {
    for (int64_t n = 0; n < N; n++) {
      double s = 0.0, b = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double a = load_op_scaled(a_fmt, pa, lda, a_mn, SFA, ld_sfa, m, k);
        double bb = load_op_scaled(b_fmt, pb, ldb, b_mn, SFB, ld_sfb, n, k);
        s += a * bb;
        b += std::fabs(a * bb);
      }
      double d0 = accum ? (double)D0[m * ldd + n] : 0.0;
      ref[(m - m_begin) * N + n] = d0 + sigma * s;
      bound[(m - m_begin) * N + n] = b;
    }
  }
  return 0;
}

int oracle_gemm_block_scale_points(int64_t M, int64_t N, int64_t K,
                                   int a_fmt, const void* A, int64_t lda, const uint8_t* SFA, int64_t ld_sfa,
                                   int b_fmt, const void* B, int64_t ldb, const uint8_t* SFB, int64_t ld_sfb,
                                   const float* D0, int64_t ldd, int neg_a, int neg_b, int accum,
                                   const int64_t* pm, const int64_t* pn, int64_t npts,
                                   double* ref, double* bound, int a_mn, int b_mn) {
  if (!mx_fmt(a_fmt) || !mx_fmt(b_fmt)) return -1;
  if (K % 32 != 0) return -2;
  if (accum && !D0) return -4;
  for (int64_t i = 0; i < npts; i++) if (pm[i] < 0 || pm[i] >= M || pn[i] < 0 || pn[i] >= N) return -2;
  const uint8_t* pa = (const uint8_t*)A;
  const uint8_t* pb = (const uint8_t*)B;
  const double sigma = (neg_a ? -1.0 : 1.0) * (neg_b ? -1.0 : 1.0);
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < npts; i++) {
    const int64_t m = pm[i], n = pn[i];
    double s = 0.0, b = 0.0;
    for (int64_t k = 0; k < K; k++) {
      double a = load_op_scaled(a_fmt, pa, lda, a_mn, SFA, ld_sfa, m, k);
      double bb = load_op_scaled(b_fmt, pb, ldb, b_mn, SFB, ld_sfb, n, k);
      s += a * bb;
      b += std::fabs(a * bb);
    }
    double d0 = accum ? (double)D0[m * ldd + n] : 0.0;
    ref[i] = d0 + sigma * s;
    bound[i] = b;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Scalar epilogue ([TP] "Scalar compositions": a typed scalar function applied to every
// element; the pages' example is silu_affine with scalar scale and bias). In fp64:
//   out = x / (1 + exp(-x)) * scale + bias
// ---------------------------------------------------------------------------
int oracle_ewise_silu_affine(const double* x, int64_t n, double scale, double bias, double* out) {
  if (n < 0) return -2;
  for (int64_t i = 0; i < n; i++) out[i] = x[i] / (1.0 + std::exp(-x[i])) * scale + bias;
  return 0;
}

// ---------------------------------------------------------------------------
// C8. Comparison: |D - ref| <= tol * bound + 2^-24 * |ref| (the second term is
// the half-ulp of the float32 result), exact equality where bound == 0 and the
// reference is finite; NaN matches NaN. Returns the number of violations, the
// first violating index and the largest |D-ref| / bound.
// ---------------------------------------------------------------------------
int64_t oracle_check_gemm(const float* D, int64_t rows, int64_t cols, int64_t ldd,
                          const double* ref, const double* bound, double tol,
                          int64_t* first_bad, double* max_ratio) {
  int64_t bad = 0;
  double worst = 0.0;
  *first_bad = -1;
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t c = 0; c < cols; c++) {
      double d = (double)D[r * ldd + c], e = ref[r * cols + c], b = bound[r * cols + c];
      bool ok;
      if (std::isnan(e) || std::isnan(d)) ok = std::isnan(e) && std::isnan(d);
      else if (std::isinf(e) || std::isinf(d)) ok = d == e;   // an infinity matches only itself
      else {
        double err = std::fabs(d - e);
        ok = err <= tol * b + std::ldexp(std::fabs(e), -24);
        if (b > 0) { double q = err / b; if (q > worst) worst = q; }
      }
      if (!ok) { if (bad == 0) *first_bad = r * cols + c; bad++; }
    }
  }
  *max_ratio = worst;
  return bad;
}

}  // extern "C"
