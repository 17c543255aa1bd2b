// k_tile.hip - element-wise tile kernel and the box load / store / reduce-add kernels.
//
// Box semantics ("cp.async.bulk.tensor / cp.reduce.async.bulk.tensor", Call
// parameters, Data representation, Operand specification, Stores, reductions and
// completion): image element j holds global coordinate coords + j*element_strides,
// out-of-range coordinates read the fill value and are never written; the image is
// compact row-major before a 16-byte-chunk XOR swizzle.
//
// Work mapping: one workgroup (256 lanes) per box; the image is cut into 16-byte
// chunks (an image row is a whole number of them). General boxes: lane i moves chunks
// i, i+256, ...; a chunk whose 16 global bytes are in range and 16-byte aligned moves
// with one 128-bit access, any other chunk element by element. Rank-2 boxes with unit
// element strides (the common case, chosen on the host) use a dedicated kernel that
// issues every HBM read of the workgroup before its first use, uses streaming accesses
// and handles ragged edges without per-element loads.
#include <atomic>

#include "bsm_device.hpp"
#include "bsm_internal.hpp"
#include "../../include/bsm.h"

namespace bsm {

// ------------------------------------------------------------------ add scalar
// "Tile Operands and Execution", A Load, Compute, and Store Example: 64 lanes,
// each with three 4-word loads, twelve scalar adds and three 4-word stores.
// One wave64 covers a (2,32,3,4) float32 tile. Lane t owns the float4 groups at 4t,
// 256 + 4t and 512 + 4t (rather than 12 consecutive floats), so that every 16-byte
// access of the wave covers 1 KiB contiguous; the element-wise map is unchanged.
__global__ __launch_bounds__(64) void k_add_scalar_f32(const float* __restrict__ src, float* dst, int64_t n, float s) {
  const int64_t base = (int64_t)blockIdx.x * 768 + 4 * threadIdx.x;
#pragma unroll
  for (int r = 0; r < 3; r++) {
    const int64_t i = base + 256 * r;
    if (i + 4 <= n) {
      float4 v = *(const float4*)(src + i);
      v.x += s; v.y += s; v.z += s; v.w += s;
      *(float4*)(dst + i) = v;
    } else {
      for (int64_t e = i; e < n && e < i + 4; e++) dst[e] = src[e] + s;
    }
  }
}

hipError_t launch_add_scalar_f32(const float* src, float* dst, int64_t n, float s, hipStream_t st) {
  const int64_t blocks = (n + 767) / 768;
  hipLaunchKernelGGL(k_add_scalar_f32, dim3((unsigned)blocks), dim3(64), 0, st, src, dst, n, s);
  return hipGetLastError();
}

// Grid-stride over (row, 256-column block) pairs.
__global__ __launch_bounds__(256) void k_zero_f32_2d(float* D, int64_t ldd, int64_t M, int64_t N) {
  const int64_t cb = (N + 255) / 256;
  for (int64_t b = blockIdx.x; b < M * cb; b += gridDim.x) {
    const int64_t row = b / cb, col = (b - row * cb) * 256 + threadIdx.x;
    if (col < N) D[row * ldd + col] = 0.0f;
  }
}

hipError_t launch_zero_f32_2d(float* D, int64_t ldd, int64_t M, int64_t N, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int64_t blocks = M * ((N + 255) / 256);
  const unsigned g = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_zero_f32_2d, dim3(g), dim3(256), 0, st, D, ldd, M, N);
  return hipGetLastError();
}

// The empty-sum GEMM output with its epilogue, in place: D = f(accum ? D : 0), grid-stride
// over (row, 256-column block) pairs like k_zero_f32_2d.
__global__ __launch_bounds__(256) void k_empty_gemm_f32_2d(float* D, int64_t ldd, int64_t M, int64_t N, int accum,
                                                           float es, float eb) {
  const int64_t cb = (N + 255) / 256;
  for (int64_t b = blockIdx.x; b < M * cb; b += gridDim.x) {
    const int64_t row = b / cb, col = (b - row * cb) * 256 + threadIdx.x;
    if (col < N) {
      float* p = D + row * ldd + col;
      *p = silu_affine(accum ? *p : 0.0f, es, eb);
    }
  }
}

hipError_t launch_empty_gemm(float* D, int64_t ldd, int64_t M, int64_t N, int accum, int ew_op, float es, float eb,
                             hipStream_t st) {
  if (ew_op == 0) return accum ? hipSuccess : launch_zero_f32_2d(D, ldd, M, N, st);
  if (M <= 0 || N <= 0) return hipSuccess;
  const int64_t blocks = M * ((N + 255) / 256);
  const unsigned g = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_empty_gemm_f32_2d, dim3(g), dim3(256), 0, st, D, ldd, M, N, accum, es, eb);
  return hipGetLastError();
}

// ------------------------------------------------------------------ box helpers
struct RowPos {
  bool ok;       // every outer coordinate in range
  int64_t off;   // byte offset of the row's outer coordinates (valid when ok)
};

// Outer coordinates of image row r: unravel r over ext[0..rank-2] (row-major),
// g_i = c_i + j_i * estr_i.
__device__ __forceinline__ RowPos row_pos(const BoxGeom& g, const int32_t* c, const int64_t* strides, int r) {
  RowPos p{true, 0};
  const int in = g.rank - 1;
  int rem = r;
#pragma unroll
  for (int i = 3; i >= 0; i--) {
    if (i < in) {
      const int j = rem % g.ext[i];
      rem /= g.ext[i];
      const int64_t gi = (int64_t)c[i] + (int64_t)j * g.estr[i];
      if (gi < 0 || gi >= g.dims[i]) p.ok = false;
      else p.off += gi * strides[i];
    }
  }
  return p;
}

__device__ __forceinline__ uint32_t load_elem(const uint8_t* p, int esize) {
  if (esize == 1) return *p;
  if (esize == 2) return *(const uint16_t*)p;
  return *(const uint32_t*)p;
}

__device__ __forceinline__ void store_elem(uint8_t* p, int esize, uint32_t v) {
  if (esize == 1) *p = (uint8_t)v;
  else if (esize == 2) *(uint16_t*)p = (uint16_t)v;
  else *(uint32_t*)p = v;
}

// Word i of a 16-byte chunk, and its replacement, as register selects (no local arrays,
// which the compiler would place in scratch memory once indexed at run time).
__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ void set_word(uint4& v, int i, uint32_t x) {
  v.x = i == 0 ? x : v.x;
  v.y = i == 1 ? x : v.y;
  v.z = i == 2 ? x : v.z;
  v.w = i == 3 ? x : v.w;
}
__device__ __forceinline__ uint4 select4(bool c, const uint4& a, const uint4& b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

__device__ __forceinline__ uint32_t get_elem(const uint4& v, int esize, int e) {
  const int bit = e * esize * 8;
  const uint32_t word = word_of(v, bit >> 5);
  if (esize == 4) return word;
  const uint32_t mask = esize == 2 ? 0xFFFFu : 0xFFu;
  return (word >> (bit & 31)) & mask;
}

__device__ __forceinline__ void put_elem(uint4& v, int esize, int e, uint32_t x) {
  const int bit = e * esize * 8;
  if (esize == 4) {
    set_word(v, bit >> 5, x);
  } else {
    const uint32_t mask = (esize == 2 ? 0xFFFFu : 0xFFu) << (bit & 31);
    const uint32_t w = word_of(v, bit >> 5);
    set_word(v, bit >> 5, (w & ~mask) | ((x << (bit & 31)) & mask));
  }
}

// Element-wise add of two elements of a float format, rounded once (RNE) to the format.
__device__ __forceinline__ uint32_t add_elem(int dtype, uint32_t a, uint32_t b) {
  if (dtype == BSM_F32) return __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
  if (dtype == BSM_BF16) return f32_to_bf16_bits(bf16_bits_to_f32((uint16_t)a) + bf16_bits_to_f32((uint16_t)b));
  return f32_to_f16_bits(f16_bits_to_f32((uint16_t)a) + f16_bits_to_f32((uint16_t)b));
}

__device__ __forceinline__ uint4 add_chunk(int dtype, uint4 a, uint4 b) {
  if (dtype == BSM_F32) {
    return make_uint4(add_elem(dtype, a.x, b.x), add_elem(dtype, a.y, b.y), add_elem(dtype, a.z, b.z),
                      add_elem(dtype, a.w, b.w));
  }
  uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w}, wr[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t lo = add_elem(dtype, wa[i] & 0xFFFFu, wb[i] & 0xFFFFu);
    const uint32_t hi = add_elem(dtype, wa[i] >> 16, wb[i] >> 16);
    wr[i] = lo | (hi << 16);
  }
  return make_uint4(wr[0], wr[1], wr[2], wr[3]);
}

// Global -> 16-byte image chunk (row r, chunk cc of the row).
__device__ __forceinline__ uint4 gather_chunk(const BoxGeom& g, const uint8_t* src, const int32_t* c, int r, int cc) {
  const RowPos rp = row_pos(g, c, g.strides, r);
  const int in = g.rank - 1;
  const int epc = 16 / g.esize;
  const int64_t g0 = (int64_t)c[in] + (int64_t)cc * epc;
  const uint8_t* p = src + rp.off + g0 * g.esize;
  if (rp.ok && g0 >= 0 && g0 + epc <= g.dims[in] && (((uintptr_t)p) & 15) == 0) return *(const uint4*)p;
  uint4 v = make_uint4(0, 0, 0, 0);
  for (int e = 0; e < epc; e++) {
    const int64_t gi = g0 + e;
    const bool ok = rp.ok && gi >= 0 && gi < g.dims[in];
    put_elem(v, g.esize, e, ok ? load_elem(src + rp.off + gi * g.esize, g.esize) : g.fill_bits);
  }
  return v;
}

// 16-byte image chunk -> global (store or add-reduce), in-range elements only.
__device__ __forceinline__ void scatter_chunk(const BoxGeom& g, uint8_t* dst, const int64_t* strides, const int32_t* c,
                                              int r, int cc, uint4 v, bool reduce) {
  const RowPos rp = row_pos(g, c, strides, r);
  if (!rp.ok) return;
  const int in = g.rank - 1;
  const int epc = 16 / g.esize;
  const int64_t g0 = (int64_t)c[in] + (int64_t)cc * epc;
  uint8_t* p = dst + rp.off + g0 * g.esize;
  if (g0 >= 0 && g0 + epc <= g.dims[in] && (((uintptr_t)p) & 15) == 0) {
    if (reduce) v = add_chunk(g.dtype, *(const uint4*)p, v);
    *(uint4*)p = v;
    return;
  }
  for (int e = 0; e < epc; e++) {
    const int64_t gi = g0 + e;
    if (gi < 0 || gi >= g.dims[in]) continue;
    uint8_t* q = dst + rp.off + gi * g.esize;
    uint32_t x = get_elem(v, g.esize, e);
    if (reduce) x = add_elem(g.dtype, load_elem(q, g.esize), x);
    store_elem(q, g.esize, x);
  }
}

// ------------------------------------------------------------------ box load / store
// Coordinates of box t: from the device array, or generated from the repeat axes
// ("cp.async.bulk.tensor", Call parameters: coord_steps; one box per repeat coordinate in
// row-major repeat order).
__device__ __forceinline__ void box_coords(const BoxGeom& g, const int32_t* coords, const BoxRepeat& rp, uint32_t t,
                                           int32_t (&c)[5]) {
  if (coords) {
#pragma unroll
    for (int i = 0; i < 5; i++) c[i] = i < g.rank ? coords[(int64_t)t * g.rank + i] : 0;
    return;
  }
#pragma unroll
  for (int i = 0; i < 5; i++) c[i] = i < g.rank ? rp.base[i] : 0;
#pragma unroll
  for (int a = 3; a >= 0; a--) {
    if (a < rp.naxes) {
      const uint32_t j = t % (uint32_t)rp.rep[a];
      t /= (uint32_t)rp.rep[a];
#pragma unroll
      for (int i = 0; i < 5; i++) c[i] += (int32_t)j * rp.step[a][i];
    }
  }
}

__global__ __launch_bounds__(256) void k_box_load(BoxGeom g, const uint8_t* __restrict__ src,
                                                  const int32_t* __restrict__ coords, BoxRepeat rp,
                                                  uint8_t* __restrict__ images) {
  const int64_t t = blockIdx.x;
  int32_t c[5];
  box_coords(g, coords, rp, (uint32_t)t, c);
  uint8_t* img = images + t * g.image_stride;
  const int cpr = g.row_bytes >> 4;
  const int nchunks = g.nrows * cpr;
  for (int q = threadIdx.x; q < nchunks; q += 256) {
    const int r = q / cpr, cc = q - r * cpr;
    const uint4 v = gather_chunk(g, src, c, r, cc);
    *(uint4*)(img + image_swizzle((uint32_t)(r * g.row_bytes + cc * 16), g.swizzle)) = v;
  }
}

__global__ __launch_bounds__(256) void k_box_store(BoxGeom g, uint8_t* dst, const int32_t* __restrict__ coords,
                                                   BoxRepeat rp, const uint8_t* __restrict__ images, int reduce) {
  const int64_t t = blockIdx.x;
  int32_t c[5];
  box_coords(g, coords, rp, (uint32_t)t, c);
  const uint8_t* img = images + t * g.image_stride;
  const int cpr = g.row_bytes >> 4;
  const int nchunks = g.nrows * cpr;
  for (int q = threadIdx.x; q < nchunks; q += 256) {
    const int r = q / cpr, cc = q - r * cpr;
    const uint4 v = *(const uint4*)(img + image_swizzle((uint32_t)(r * g.row_bytes + cc * 16), g.swizzle));
    scatter_chunk(g, dst, g.strides, c, r, cc, v, reduce != 0);
  }
}

hipError_t launch_box_load(const BoxGeom& g, const void* src, const int32_t* coords, const BoxRepeat& rp,
                           int64_t n_boxes, void* images, hipStream_t st) {
  hipLaunchKernelGGL(k_box_load, dim3((unsigned)n_boxes), dim3(256), 0, st, g, (const uint8_t*)src, coords, rp,
                     (uint8_t*)images);
  return hipGetLastError();
}

hipError_t launch_box_store(const BoxGeom& g, void* dst, const int32_t* coords, const BoxRepeat& rp, int64_t n_boxes,
                            const void* images, int reduce_add, hipStream_t st) {
  hipLaunchKernelGGL(k_box_store, dim3((unsigned)n_boxes), dim3(256), 0, st, g, (uint8_t*)dst, coords, rp,
                     (const uint8_t*)images, reduce_add);
  return hipGetLastError();
}

// Non-temporal 16-byte global accesses for data touched exactly once.
__device__ __forceinline__ uint4 stream_load16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void stream_store16(uint8_t* p, uint4 x) {
  const u32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, (u32x4*)p);
}

// The first nb bytes (0 < nb < 16) of a 16-byte chunk to a 16-byte aligned address, as at
// most four naturally aligned stores of 8, 4, 2 and 1 bytes: element-wise sub-dword stores
// of a chunk's tail cost the memory path far more than these.
__device__ __forceinline__ void store_head16(uint8_t* p, uint4 x, int nb) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  int o = 0;
  if (nb & 8) {
    *(uint2*)p = make_uint2(x.x, x.y);
    o = 8;
  }
  if (nb & 4) {
    *(uint32_t*)(p + o) = o ? x.z : x.x;
    o += 4;
  }
  const uint32_t wo = o == 0 ? w[0] : (o == 4 ? w[1] : (o == 8 ? w[2] : w[3]));
  if (nb & 2) *(uint16_t*)(p + o) = (uint16_t)wo;
  if (nb & 1) *(p + o + (nb & 2)) = (uint8_t)(wo >> (8 * (nb & 2)));
}

// ------------------------------------------------------------------ grid round trip
struct CopyOut {
  int64_t dst_strides[5];
  int64_t add_strides[5];
  uint32_t tiles[5];  // boxes per axis, ceil(dims / box)
};

// One workgroup per tile coordinate t*box: global -> swizzled LDS image -> dst / dst_add.
__global__ __launch_bounds__(256) void k_box_copy(BoxGeom g, CopyOut o, const uint8_t* __restrict__ src,
                                                  uint8_t* __restrict__ dst, uint8_t* __restrict__ dst_add) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t image[];
  // Box coordinates: blockIdx unravelled over the per-axis tile counts, innermost fastest
  // (the host guarantees fewer than 2^31 boxes, so 32-bit arithmetic suffices).
  int32_t c[5];
  uint32_t rem = blockIdx.x;
#pragma unroll
  for (int i = 4; i >= 0; i--) {
    c[i] = 0;
    if (i < g.rank) {
      c[i] = (int32_t)((rem % o.tiles[i]) * (uint32_t)g.box[i]);
      rem /= o.tiles[i];
    }
  }
  const int cpr = g.row_bytes >> 4;
  const int nchunks = g.nrows * cpr;
  for (int q = threadIdx.x; q < nchunks; q += 256) {
    const int r = q / cpr, cc = q - r * cpr;
    const uint4 v = gather_chunk(g, src, c, r, cc);
    lds_write_b128(image + image_swizzle((uint32_t)(r * g.row_bytes + cc * 16), g.swizzle), v);
  }
  __syncthreads();
  for (int q = threadIdx.x; q < nchunks; q += 256) {
    const int r = q / cpr, cc = q - r * cpr;
    const uint4 v = lds_read_b128(image + image_swizzle((uint32_t)(r * g.row_bytes + cc * 16), g.swizzle));
    if (dst) scatter_chunk(g, dst, o.dst_strides, c, r, cc, v, false);
    if (dst_add) scatter_chunk(g, dst_add, o.add_strides, c, r, cc, v, true);
  }
}


// Rank-2 grid round trip with unit element strides, an image of at most 1024 16-byte chunks
// with a power-of-two number of chunks per row, and rows of at least one whole chunk (the
// host checks all of this): a small kernel with only the arguments this case needs.
struct Copy2D {
  const uint8_t* src; uint8_t* dst; uint8_t* add;
  int64_t dims0, dims1;                 // rows, columns (elements)
  int64_t s_src, s_dst, s_add;          // row strides (bytes)
  uint32_t tiles1;                      // boxes per row of boxes
  uint32_t groups1;                     // workgroups per row of boxes: ceil(tiles1 / 2^lg_nb)
  uint32_t slices;                      // row slices per box: ceil(box0 / (kCopyPasses * rows per pass))
  int32_t box0, box1;                   // box extents (rows, elements)
  int32_t esize, dtype, swizzle, lg_cpr, lg_nb, row_bytes;
  uint32_t fill_word;                   // the fill element replicated over 32 bits
};

// Rows of a slice each lane moves (one 16-byte chunk per row): two keep 8 KiB of every
// tensor per workgroup, which measured faster on HBM than four (the grid doubles, and
// each workgroup's accesses are all in flight at once).
constexpr int kCopyPasses = 2;

// A workgroup moves one row slice of 2^lg_nb horizontally adjacent boxes (the bf16 (128,
// 64) box: 8 rows x 8 boxes, i.e. rows of 1 KiB contiguous bytes, which HBM serves
// markedly faster than the 128-byte rows of a single box at a power-of-two row pitch).
// Lane l takes chunk column l % (nb cpr) (box (l % (nb cpr)) / cpr) of slice rows
// l / (nb cpr) + k * rstep, k < kCopyPasses. Each box keeps its own image region in LDS: the slice's
// rows sit there at the swizzled offsets they have in the full box image (a slice spans a
// whole number of swizzle periods, so the pattern is the same). All source and
// reduce-add chunks are fetched first with 128-bit streaming loads, so every HBM read of the
// workgroup is in flight at once. A chunk that straddles the last column is read whole as
// well (its 16 bytes lie inside the tensor's extent on every row but the last) and its
// elements past the last column are replaced by the fill; on the tensor's last row it is
// gathered element by element. Rows past the last row and chunks past the last column
// take the fill. Whole chunks are stored with 128-bit streaming stores, the straddling
// chunk's in-range head with at most four aligned stores. Boxes past the end of a row of boxes (when
// the workgroup's group is incomplete) do nothing.
// ADDT: 0 for a plain copy, else the reduce-add element type (BSM_F32, BSM_BF16, BSM_F16),
// fixed at compile time so that the add is straight-line code: a run-time type switch
// between the stores makes the compiler wait for every outstanding store before each add.
// DST: whether the image is also stored to dst (a reduce-add alone passes no dst), likewise
// a compile-time choice, so that each of the three forms is its own kernel.
template <int ADDT, bool DST>
__global__ __launch_bounds__(256) void k_box_copy2d(Copy2D a) {
  constexpr bool ADD = ADDT != 0;
  static_assert(ADD || DST, "a copy stores, reduce-adds, or both");
  extern __shared__ __attribute__((aligned(1024))) uint8_t image[];
  const uint32_t g1 = blockIdx.x % a.groups1, rest = blockIdx.x / a.groups1;
  const uint32_t sl = rest % a.slices, t0 = rest / a.slices;
  const int lg_row = a.lg_cpr + a.lg_nb;                  // log2 chunks per slice row
  const int cpr = 1 << a.lg_cpr;
  const int call = threadIdx.x & ((1 << lg_row) - 1);
  const int bx = call >> a.lg_cpr, cc = call & (cpr - 1);
  const int rr0 = threadIdx.x >> lg_row, rstep = 256 >> lg_row;
  const int rs = kCopyPasses * rstep;                     // rows per slice
  const uint32_t t1 = (g1 << a.lg_nb) + bx;
  const bool boxok = t1 < a.tiles1;
  const int64_t c0 = (int64_t)t0 * a.box0, c1 = (int64_t)t1 * a.box1;
  const int epc = 16 / a.esize;
  const int64_t k0 = c1 + (int64_t)cc * epc;           // first element of the lane's chunk
  const bool whole = k0 + epc <= a.dims1;              // chunk wholly in range
  const bool part = !whole && k0 < a.dims1;            // chunk straddles the last column
  const int64_t kc = whole || part ? k0 : ((a.dims1 / epc) - 1) * epc;  // a whole chunk stands in
  const uint4 fill4 = make_uint4(a.fill_word, a.fill_word, a.fill_word, a.fill_word);
  uint8_t* region = image + bx * rs * a.row_bytes;      // this box's slice of its image
  uint4 v[kCopyPasses], d[kCopyPasses];
  bool rin[kCopyPasses], last[kCopyPasses];
#pragma unroll
  for (int k = 0; k < kCopyPasses; k++) {
    const int r = (int)sl * rs + rr0 + k * rstep;        // row within the box
    const int64_t row = c0 + r;
    rin[k] = boxok && r < a.box0 && row < a.dims0;
    const int64_t rowc = min(row, a.dims0 - 1);          // rows past the end re-read the last row
    last[k] = part && rowc == a.dims0 - 1;               // no 16-byte read past the tensor's end
    const int64_t col = (last[k] ? ((a.dims1 / epc) - 1) * epc : kc) * a.esize;
    v[k] = stream_load16(a.src + rowc * a.s_src + col);
    if (ADD) d[k] = stream_load16(a.add + rowc * a.s_add + col);
  }
#pragma unroll
  for (int k = 0; k < kCopyPasses; k++) {
    v[k] = select4(rin[k] && (whole || part), v[k], fill4);
    if (part) {
      for (int e = 0; e < epc; e++)
        if (k0 + e >= a.dims1) put_elem(v[k], a.esize, e, a.fill_word);
    }
  }
  if (__builtin_expect(part && a.dims0 - 1 < c0 + a.box0, 0)) {
    // the straddling chunk of the tensor's last row, element by element
#pragma unroll
    for (int k = 0; k < kCopyPasses; k++) {
      if (!rin[k] || !last[k]) continue;
      const uint8_t* row = a.src + (c0 + (int)sl * rs + rr0 + k * rstep) * a.s_src;
      for (int e = 0; e < epc; e++)
        if (k0 + e < a.dims1) put_elem(v[k], a.esize, e, load_elem(row + (k0 + e) * a.esize, a.esize));
    }
  }
#pragma unroll
  for (int k = 0; k < kCopyPasses; k++) {
    const int rr = rr0 + k * rstep;
    if ((int)sl * rs + rr < a.box0)
      lds_write_b128(region + image_swizzle((uint32_t)(rr * a.row_bytes + cc * 16), a.swizzle), v[k]);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kCopyPasses; k++) {
    const int rr = rr0 + k * rstep;
    const int64_t row = c0 + (int)sl * rs + rr;
    if (!rin[k] || !(whole || part)) continue;
    const uint4 x = lds_read_b128(region + image_swizzle((uint32_t)(rr * a.row_bytes + cc * 16), a.swizzle));
    if (__builtin_expect(whole, 1)) {
      if (DST) stream_store16(a.dst + row * a.s_dst + k0 * a.esize, x);
      if (ADD) stream_store16(a.add + row * a.s_add + k0 * a.esize, add_chunk(ADDT, d[k], x));
    } else {
      // the straddling chunk: its in-range head only
      const int nb = (int)(a.dims1 - k0) * a.esize;
      if (DST) store_head16(a.dst + row * a.s_dst + k0 * a.esize, x, nb);
      if (ADD) {
        uint8_t* q = a.add + row * a.s_add + k0 * a.esize;
        if (!last[k]) {
          store_head16(q, add_chunk(ADDT, d[k], x), nb);  // d[k] holds this chunk
        } else {
          // the tensor's last row: d[k] holds another chunk, the addends come element-wise
          for (int e = 0; e < epc; e++)
            if (k0 + e < a.dims1)
              store_elem(q + e * a.esize, a.esize, add_elem(ADDT, load_elem(q + e * a.esize, a.esize), get_elem(x, a.esize, e)));
        }
      }
    }
  }
}

hipError_t launch_box_copy(const BoxGeom& g, const void* src, void* dst, const int64_t* dst_strides, void* dst_add,
                           const int64_t* add_strides, hipStream_t st) {
  // The general kernel's image may take up to 160 KiB of dynamic LDS: raise the kernel's limit
  // once per device (a bit per device id; concurrent first calls may both set it, which is
  // harmless).
  static std::atomic<uint64_t> attr_devices{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (!(attr_devices.load(std::memory_order_acquire) & bit) || !bit) {
    e = hipFuncSetAttribute((const void*)k_box_copy, hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
    if (e != hipSuccess) return e;
    attr_devices.fetch_or(bit, std::memory_order_release);
  }
  CopyOut o{};
  for (int i = 0; i < g.rank; i++) {
    o.dst_strides[i] = dst_strides ? dst_strides[i] : 0;
    o.add_strides[i] = add_strides ? add_strides[i] : 0;
  }
  int64_t tiles = 1;
  for (int i = 0; i < g.rank; i++) {
    const int64_t t = (g.dims[i] + g.box[i] - 1) / g.box[i];
    o.tiles[i] = (uint32_t)t;
    tiles *= t;
  }
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // LDS holds the whole swizzle period: a swizzled offset of the image can land past
  // image_bytes (up to image_stride).
  const int cpr = g.row_bytes >> 4;
  if (g.rank == 2 && g.estr[0] == 1 && g.nrows * cpr <= 1024 && (cpr & (cpr - 1)) == 0 && g.dims[1] * g.esize >= 16) {
    Copy2D a;
    a.src = (const uint8_t*)src; a.dst = (uint8_t*)dst; a.add = (uint8_t*)dst_add;
    a.dims0 = g.dims[0]; a.dims1 = g.dims[1];
    a.s_src = g.strides[0]; a.s_dst = o.dst_strides[0]; a.s_add = o.add_strides[0];
    a.tiles1 = o.tiles[1];
    a.box0 = g.box[0]; a.box1 = g.box[1];
    a.esize = g.esize; a.dtype = g.dtype; a.swizzle = g.swizzle; a.row_bytes = g.row_bytes;
    a.lg_cpr = 0;
    while ((1 << a.lg_cpr) < cpr) a.lg_cpr++;
    // up to 8 boxes side by side per workgroup while a slice row stays within 128 chunks
    // (at least 2 rows per pass) and the row of boxes has that many boxes
    a.lg_nb = 0;
    while (a.lg_nb < 3 && (2 * cpr << a.lg_nb) <= 128 && (int64_t(2) << a.lg_nb) <= (int64_t)o.tiles[1]) a.lg_nb++;
    const int rs = kCopyPasses * (256 >> (a.lg_cpr + a.lg_nb));  // rows per slice
    a.groups1 = (uint32_t)((o.tiles[1] + (1u << a.lg_nb) - 1) >> a.lg_nb);
    a.slices = (uint32_t)((g.box[0] + rs - 1) / rs);
    a.fill_word = g.esize == 1 ? g.fill_bits * 0x01010101u : (g.esize == 2 ? g.fill_bits * 0x00010001u : g.fill_bits);
    const int64_t wgs = (int64_t)o.tiles[0] * a.slices * a.groups1;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    // every box's slice region is rs * row_bytes = 8 KiB / 2^lg_nb >= 1 KiB, a whole number
    // of swizzle periods (the swizzle stays inside aligned 2^(7 + mode)-byte windows)
    const size_t lds_bytes = (size_t)kCopyPasses * 256 * 16;
    const dim3 grid((unsigned)wgs);
#define BSM_COPY2D(ADDT)                                                                        \
  do {                                                                                          \
    if (dst) hipLaunchKernelGGL((k_box_copy2d<ADDT, true>), grid, dim3(256), lds_bytes, st, a);  \
    else hipLaunchKernelGGL((k_box_copy2d<ADDT, false>), grid, dim3(256), lds_bytes, st, a);     \
  } while (0)
    if (!dst_add) {
      if (!dst) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_box_copy2d<0, true>), grid, dim3(256), lds_bytes, st, a);
    } else if (g.dtype == BSM_F32) {
      BSM_COPY2D(BSM_F32);
    } else if (g.dtype == BSM_BF16) {
      BSM_COPY2D(BSM_BF16);
    } else if (g.dtype == BSM_F16) {
      BSM_COPY2D(BSM_F16);
    } else {
      return hipErrorInvalidValue;
    }
#undef BSM_COPY2D
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_box_copy, dim3((unsigned)tiles), dim3(256), (size_t)g.image_stride, st, g, o,
                     (const uint8_t*)src, (uint8_t*)dst, (uint8_t*)dst_add);
  return hipGetLastError();
}

// ------------------------------------------------------------------ four-row gather / scatter
// "cp.async.bulk.tensor / cp.reduce.async.bulk.tensor", Gather4 and scatter4: issue t names
// a column start and four rows (coords[5t .. 5t+4]) of a rank-2 tensor; its (4, width)
// image holds those rows' `width` elements from the column start, swizzled as one image.
// Each lane moves one 16-byte image chunk per issue; a workgroup pass covers
// ipw = 256 / (4 * chunks per row) issues and a workgroup makes kRow4Passes passes over
// consecutive issues, both loads before both stores. Whole chunks move with non-temporal
// loads and stores (each byte is touched once). Measured on the 65536 x 4096 bf16
// permutation workload: 2 passes beat 1, 4 and 8, and the non-temporal accesses gain
// 10-15% over plain ones.
constexpr int kRow4Passes = 2;

// Chunk cc of tensor row `row` from column `col` (the fill outside the tensor).
__device__ __forceinline__ uint4 row_chunk_load(const BoxGeom& g, const uint8_t* src, int64_t row, int64_t col,
                                                int cc) {
  const int epc = 16 / g.esize;
  const int64_t g0 = col + (int64_t)cc * epc;
  const bool rok = row >= 0 && row < g.dims[0];
  if (rok && g0 >= 0 && g0 + epc <= g.dims[1]) {
    const uint8_t* p = src + row * g.strides[0] + g0 * g.esize;
    if ((((uintptr_t)p) & 15) == 0) return stream_load16(p);
  }
  uint4 v = make_uint4(0, 0, 0, 0);
  for (int e = 0; e < epc; e++) {
    const int64_t gi = g0 + e;
    const bool ok = rok && gi >= 0 && gi < g.dims[1];
    put_elem(v, g.esize, e, ok ? load_elem(src + row * g.strides[0] + gi * g.esize, g.esize) : g.fill_bits);
  }
  return v;
}

// Chunk cc of tensor row `row` from column `col`, in-range elements only.
__device__ __forceinline__ void row_chunk_store(const BoxGeom& g, uint8_t* dst, int64_t row, int64_t col, int cc,
                                                uint4 v) {
  if (row < 0 || row >= g.dims[0]) return;
  const int epc = 16 / g.esize;
  const int64_t g0 = col + (int64_t)cc * epc;
  uint8_t* p = dst + row * g.strides[0] + g0 * g.esize;
  if (g0 >= 0 && g0 + epc <= g.dims[1] && (((uintptr_t)p) & 15) == 0) {
    stream_store16(p, v);
    return;
  }
  for (int e = 0; e < epc; e++) {
    const int64_t gi = g0 + e;
    if (gi >= 0 && gi < g.dims[1]) store_elem(dst + row * g.strides[0] + gi * g.esize, g.esize, get_elem(v, g.esize, e));
  }
}

template <bool SCATTER>
__global__ __launch_bounds__(256) void k_row4(BoxGeom g, uint8_t* tensor, const int32_t* __restrict__ coords,
                                              uint8_t* images, int64_t n, int ipw) {
  const int cpr = g.row_bytes >> 4, cpi = 4 * cpr;
  const int slot = threadIdx.x / cpi, w = threadIdx.x - slot * cpi;
  if (slot >= ipw) return;  // lanes past the last whole issue of a pass (no barrier follows)
  const int r = w / cpr, cc = w - r * cpr;
  const uint32_t ioff = image_swizzle((uint32_t)(r * g.row_bytes + cc * 16), g.swizzle);
  int64_t t[kRow4Passes];
  uint4 v[kRow4Passes];
#pragma unroll
  for (int p = 0; p < kRow4Passes; p++) t[p] = ((int64_t)blockIdx.x * kRow4Passes + p) * ipw + slot;
#pragma unroll
  for (int p = 0; p < kRow4Passes; p++) {
    if (t[p] < n) {
      if (SCATTER) v[p] = stream_load16(images + t[p] * g.image_stride + ioff);
      else v[p] = row_chunk_load(g, tensor, coords[5 * t[p] + 1 + r], coords[5 * t[p]], cc);
    }
  }
#pragma unroll
  for (int p = 0; p < kRow4Passes; p++) {
    if (t[p] < n) {
      if (SCATTER) row_chunk_store(g, tensor, coords[5 * t[p] + 1 + r], coords[5 * t[p]], cc, v[p]);
      else stream_store16(images + t[p] * g.image_stride + ioff, v[p]);
    }
  }
}

hipError_t launch_row4(const BoxGeom& g, void* tensor, const int32_t* coords, int64_t n_issues, void* images,
                       int scatter, hipStream_t st) {
  const int cpi = 4 * (g.row_bytes >> 4);  // 4..256 chunks per issue
  const int ipw = cpi >= 256 ? 1 : 256 / cpi;
  const int64_t per_block = (int64_t)ipw * kRow4Passes;
  const int64_t blocks = (n_issues + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (scatter)
    hipLaunchKernelGGL(k_row4<true>, dim3((unsigned)blocks), dim3(256), 0, st, g, (uint8_t*)tensor, coords,
                       (uint8_t*)images, n_issues, ipw);
  else
    hipLaunchKernelGGL(k_row4<false>, dim3((unsigned)blocks), dim3(256), 0, st, g, (uint8_t*)tensor, coords,
                       (uint8_t*)images, n_issues, ipw);
  return hipGetLastError();
}

}  // namespace bsm
