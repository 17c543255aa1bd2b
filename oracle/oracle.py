"""Python wrapper of the CPU oracle (``liboracle.so``, built from ``oracle.cpp``).

Test infrastructure only: the test-suite, the smoke check and the CPU-baseline leg
of the benchmark use it to compute expected results. The HIP library never imports
it and nothing in it is shared with the library. All arrays are numpy, on the host.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

# The oracle's own storage-format codes (see OracleDtype in oracle.cpp).
DT = {"u8": 0, "u16": 1, "u32": 2, "f16": 3, "bf16": 4, "f32": 5, "e4m3": 6, "e2m1": 7, "e8m0": 8, "e5m2": 9,
      "e2m3": 10, "e3m2": 11}
BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}   # block-scaled element widths
ESIZE = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4, "e4m3": 1, "e8m0": 1, "e5m2": 1}


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)   # missing, or older than its source
        L = C.CDLL(_LIB)
        P, I64, I32, D = C.c_void_p, C.c_int64, C.c_int, C.c_double
        L.oracle_num_threads.restype = I32
        for n in ("f16", "bf16", "e4m3", "e5m2", "e2m1", "e8m0", "e2m3", "e3m2"):
            f = getattr(L, "oracle_dec_" + n)
            f.restype = D
            f.argtypes = [C.c_uint16 if n in ("f16", "bf16") else C.c_uint8]
        L.oracle_dec_f32.restype = D
        L.oracle_dec_f32.argtypes = [C.c_uint32]
        L.oracle_enc_f16.restype = C.c_uint16
        L.oracle_enc_bf16.restype = C.c_uint16
        L.oracle_enc_f32.restype = C.c_uint32
        for n in ("f16", "bf16", "f32"):
            getattr(L, "oracle_enc_" + n).argtypes = [D]
        L.oracle_decode_array.argtypes = [I32, P, I64, P]
        L.oracle_swizzle.restype = I64
        L.oracle_swizzle.argtypes = [I64, I32]
        L.oracle_box_load.argtypes = [P, I32, I32, P, P, P, P, P, I32, I32, P]
        L.oracle_box_store.argtypes = [P, I32, I32, P, P, P, P, P, I32, P, I32]
        L.oracle_image_stride.restype = I64
        L.oracle_image_stride.argtypes = [I32, I32, P, P, I32]
        L.oracle_gather4.argtypes = [P, I32, P, P, I32, I64, P, I32, I32, P]
        L.oracle_scatter4.argtypes = [P, I32, P, P, I32, I64, P, I32, P]
        L.oracle_box_copy_grid.argtypes = [P, P, P, I32, I32, P, P, P, P, I32, I32]
        L.oracle_add_scalar_f32.argtypes = [P, P, I64, C.c_float]
        L.oracle_ldmatrix.argtypes = [P, P, I32, I32, P]
        L.oracle_gemm.argtypes = [I64, I64, I64, I32, P, I64, I32, P, I64, I32, P, I64,
                                  I32, I32, I32, I64, I64, P, P]
        L.oracle_gemm_points.argtypes = [I64, I64, I64, I32, P, I64, I32, P, I64, I32, P, I64,
                                         I32, I32, I32, P, P, I64, P, P]
        L.oracle_gemm_block_scale.argtypes = [I64, I64, I64, I32, P, I64, P, I64, I32, P, I64, P, I64,
                                              P, I64, I32, I32, I32, I64, I64, P, P, I32, I32]
        L.oracle_gemm_block_scale_points.argtypes = [I64, I64, I64, I32, P, I64, P, I64, I32, P, I64,
                                                     P, I64, P, I64, I32, I32, I32, P, P, I64, P, P, I32, I32]
        L.oracle_check_gemm.restype = I64
        L.oracle_check_gemm.argtypes = [P, I64, I64, I64, P, P, D, P, P]
        L.oracle_ewise_silu_affine.argtypes = [P, I64, D, D, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _i64(xs):
    return np.ascontiguousarray(np.asarray(xs, dtype=np.int64))


def _i32(xs):
    return np.ascontiguousarray(np.asarray(xs, dtype=np.int32))


def num_threads() -> int:
    return lib().oracle_num_threads()


def decode(dtype: str, raw: np.ndarray, n: int | None = None) -> np.ndarray:
    """Decode storage bits to float64. ``raw`` is the backing array; for the packed formats
    (e2m1, e2m3, e3m2), n = element count (default: every element the bytes hold)."""
    raw = np.ascontiguousarray(raw)
    if n is None:
        n = raw.nbytes * 8 // BITS[dtype] if dtype in ("e2m1", "e2m3", "e3m2") else raw.nbytes // ESIZE[dtype]
    out = np.empty(n, dtype=np.float64)
    rc = lib().oracle_decode_array(DT[dtype], _p(raw), n, _p(out))
    assert rc == 0
    return out


def enc(dtype: str, x) -> np.ndarray:
    f = getattr(lib(), "oracle_enc_" + dtype)
    vals = np.asarray(x, dtype=np.float64).ravel()
    out = np.array([f(float(v)) for v in vals], dtype=np.uint32 if dtype == "f32" else np.uint16)
    return out.reshape(np.shape(x))


def swizzle(off: int, mode: int) -> int:
    return lib().oracle_swizzle(int(off), int(mode))


def image_extents(box, estr):
    return tuple((b + e - 1) // e for b, e in zip(box, estr))


def image_stride(dtype: str, box, estr, swz: int) -> int:
    b, e = _i32(box), _i32(estr)
    return lib().oracle_image_stride(DT[dtype], len(box), _p(b), _p(e), swz)


def box_load(mem: np.ndarray, dtype: str, dims, strides, box, estr, coords, swz=0, fill=0) -> np.ndarray:
    """Image bytes of one box (length = image_stride)."""
    mem = np.ascontiguousarray(mem)
    img = np.zeros(image_stride(dtype, box, estr, swz), dtype=np.uint8)
    d, s, b, e, c = _i64(dims), _i64(strides), _i32(box), _i32(estr), _i64(coords)
    rc = lib().oracle_box_load(_p(mem), DT[dtype], len(dims), _p(d), _p(s), _p(b), _p(e), _p(c), swz, fill, _p(img))
    if rc:
        raise ValueError(f"oracle_box_load rc={rc}")
    return img


def box_store(mem: np.ndarray, dtype: str, dims, strides, box, estr, coords, image, swz=0, reduce_add=0):
    """In place on ``mem`` (a contiguous numpy array of the tensor's backing bytes)."""
    assert mem.flags.c_contiguous
    image = np.ascontiguousarray(image)
    d, s, b, e, c = _i64(dims), _i64(strides), _i32(box), _i32(estr), _i64(coords)
    rc = lib().oracle_box_store(_p(mem), DT[dtype], len(dims), _p(d), _p(s), _p(b), _p(e), _p(c), swz,
                                _p(image), int(reduce_add))
    if rc:
        raise ValueError(f"oracle_box_store rc={rc}")


def repeat_coords(coords, repeats, steps) -> np.ndarray:
    """Box coordinates of a call with repeat axes ("cp.async.bulk.tensor", Call parameters:
    coord_steps holds one increment vector per repeat axis; Code generation: one box per
    repeat coordinate, row-major over the repeat axes): box t = (j_0, .., j_{n-1}) in
    row-major order starts at coords + sum_a j_a * steps[a]. Shape (prod(repeats), rank)."""
    coords = np.asarray(coords, np.int64)
    out = []
    for js in np.ndindex(*repeats) if len(repeats) else [()]:
        c = coords.copy()
        for a, j in enumerate(js):
            c = c + j * np.asarray(steps[a], np.int64)
        out.append(c)
    return np.array(out, np.int64).reshape(-1, coords.size)


def box_load_steps(mem, dtype, dims, strides, box, estr, coords, repeats, steps, swz=0, fill=0) -> np.ndarray:
    """Images of every repeat coordinate, concatenated (each image_stride bytes)."""
    return np.concatenate([box_load(mem, dtype, dims, strides, box, estr, c, swz, fill)
                           for c in repeat_coords(coords, repeats, steps)])


def box_store_steps(mem, dtype, dims, strides, box, estr, coords, repeats, steps, images, swz=0, reduce_add=0):
    """In place on ``mem``: image t (of image_stride bytes) to repeat coordinate t, in order."""
    st = image_stride(dtype, box, estr, swz)
    images = np.ascontiguousarray(images).reshape(-1)
    for t, c in enumerate(repeat_coords(coords, repeats, steps)):
        box_store(mem, dtype, dims, strides, box, estr, c, images[t * st:(t + 1) * st], swz, reduce_add)


def gather4(mem: np.ndarray, dtype: str, dims, strides, width: int, col: int, rows, swz=0, fill=0) -> np.ndarray:
    """Image bytes of one four-row gather: a (4, width) image, length = the image stride of
    a (4, width) box."""
    mem = np.ascontiguousarray(mem)
    img = np.zeros(image_stride(dtype, (4, width), (1, 1), swz), dtype=np.uint8)
    d, s, r = _i64(dims), _i64(strides), _i64(rows)
    assert len(r) == 4
    rc = lib().oracle_gather4(_p(mem), DT[dtype], _p(d), _p(s), int(width), int(col), _p(r), swz, fill, _p(img))
    if rc:
        raise ValueError(f"oracle_gather4 rc={rc}")
    return img


def scatter4(mem: np.ndarray, dtype: str, dims, strides, width: int, col: int, rows, image, swz=0):
    """In place on ``mem`` (a contiguous numpy array of the tensor's backing bytes)."""
    assert mem.flags.c_contiguous
    image = np.ascontiguousarray(image)
    d, s, r = _i64(dims), _i64(strides), _i64(rows)
    assert len(r) == 4
    rc = lib().oracle_scatter4(_p(mem), DT[dtype], _p(d), _p(s), int(width), int(col), _p(r), swz, _p(image))
    if rc:
        raise ValueError(f"oracle_scatter4 rc={rc}")


def box_copy_grid(src, dst, dst_add, dtype, dims, strides, box, estr, swz=0, fill=0):
    """In place on dst / dst_add (either may be None)."""
    for a in (src, dst, dst_add):
        assert a is None or a.flags.c_contiguous
    d, s, b, e = _i64(dims), _i64(strides), _i32(box), _i32(estr)
    rc = lib().oracle_box_copy_grid(_p(src), _p(dst), _p(dst_add), DT[dtype], len(dims), _p(d), _p(s),
                                    _p(b), _p(e), swz, fill)
    if rc:
        raise ValueError(f"oracle_box_copy_grid rc={rc}")


def add_scalar_f32(x: np.ndarray, s: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().oracle_add_scalar_f32(_p(x), _p(out), x.size, C.c_float(s))
    return out


def ldmatrix(shared: np.ndarray, row_offsets, nmat: int, trans: int) -> np.ndarray:
    """(32, nmat) uint32 register image; row_offsets are byte offsets into ``shared``."""
    shared = np.ascontiguousarray(shared)
    ro = _i64(row_offsets)
    out = np.zeros((32, nmat), dtype=np.uint32)
    rc = lib().oracle_ldmatrix(_p(shared), _p(ro), nmat, trans, _p(out))
    if rc:
        raise ValueError(f"oracle_ldmatrix rc={rc}")
    return out


def gemm(M, N, K, dtype, A, lda, a_major, B, ldb, b_major, D0=None, ldd=0, neg_a=0, neg_b=0, accum=0,
         m_begin=0, m_end=None):
    """(ref, bound) as float64 arrays of shape (m_end-m_begin, N)."""
    m_end = M if m_end is None else m_end
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    D0 = None if D0 is None else np.ascontiguousarray(D0, dtype=np.float32)
    ref = np.empty((m_end - m_begin, N), dtype=np.float64)
    bound = np.empty_like(ref)
    rc = lib().oracle_gemm(M, N, K, DT[dtype], _p(A), lda, ord(a_major), _p(B), ldb, ord(b_major),
                           _p(D0), ldd, neg_a, neg_b, accum, m_begin, m_end, _p(ref), _p(bound))
    if rc:
        raise ValueError(f"oracle_gemm rc={rc}")
    return ref, bound


def gemm_points(M, N, K, dtype, A, lda, a_major, B, ldb, b_major, D0, ldd, neg_a, neg_b, accum, pm, pn):
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    D0 = None if D0 is None else np.ascontiguousarray(D0, dtype=np.float32)
    pm, pn = _i64(pm), _i64(pn)
    ref = np.empty(pm.size, dtype=np.float64)
    bound = np.empty_like(ref)
    rc = lib().oracle_gemm_points(M, N, K, DT[dtype], _p(A), lda, ord(a_major), _p(B), ldb, ord(b_major),
                                  _p(D0), ldd, neg_a, neg_b, accum, _p(pm), _p(pn), pm.size, _p(ref), _p(bound))
    if rc:
        raise ValueError(f"oracle_gemm_points rc={rc}")
    return ref, bound


def gemm_block_scale(M, N, K, a_fmt, A, lda, SFA, ld_sfa, b_fmt, B, ldb, SFB, ld_sfb, D0=None, ldd=0,
                     neg_a=0, neg_b=0, accum=0, m_begin=0, m_end=None, a_major="k", b_major="k"):
    """a_major 'k' or 'm', b_major 'k' or 'n': MN-major operands store (K rows, M or N contiguous)."""
    m_end = M if m_end is None else m_end
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    SFA, SFB = np.ascontiguousarray(SFA, dtype=np.uint8), np.ascontiguousarray(SFB, dtype=np.uint8)
    D0 = None if D0 is None else np.ascontiguousarray(D0, dtype=np.float32)
    ref = np.empty((m_end - m_begin, N), dtype=np.float64)
    bound = np.empty_like(ref)
    rc = lib().oracle_gemm_block_scale(M, N, K, DT[a_fmt], _p(A), lda, _p(SFA), ld_sfa, DT[b_fmt], _p(B), ldb,
                                       _p(SFB), ld_sfb, _p(D0), ldd, neg_a, neg_b, accum, m_begin, m_end,
                                       _p(ref), _p(bound), int(a_major != "k"), int(b_major != "k"))
    if rc:
        raise ValueError(f"oracle_gemm_block_scale rc={rc}")
    return ref, bound


def gemm_block_scale_points(M, N, K, a_fmt, A, lda, SFA, ld_sfa, b_fmt, B, ldb, SFB, ld_sfb, D0, ldd,
                            neg_a, neg_b, accum, pm, pn, a_major="k", b_major="k"):
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    SFA, SFB = np.ascontiguousarray(SFA, dtype=np.uint8), np.ascontiguousarray(SFB, dtype=np.uint8)
    D0 = None if D0 is None else np.ascontiguousarray(D0, dtype=np.float32)
    pm, pn = _i64(pm), _i64(pn)
    ref = np.empty(pm.size, dtype=np.float64)
    bound = np.empty_like(ref)
    rc = lib().oracle_gemm_block_scale_points(M, N, K, DT[a_fmt], _p(A), lda, _p(SFA), ld_sfa, DT[b_fmt], _p(B),
                                              ldb, _p(SFB), ld_sfb, _p(D0), ldd, neg_a, neg_b, accum,
                                              _p(pm), _p(pn), pm.size, _p(ref), _p(bound), int(a_major != "k"),
                                              int(b_major != "k"))
    if rc:
        raise ValueError(f"oracle_gemm_block_scale_points rc={rc}")
    return ref, bound


def ewise_silu_affine(x, scale: float, bias: float) -> np.ndarray:
    """x / (1 + exp(-x)) * scale + bias in float64, elementwise (same shape as x)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    rc = lib().oracle_ewise_silu_affine(_p(x), x.size, float(scale), float(bias), _p(out))
    if rc:
        raise ValueError(f"oracle_ewise_silu_affine rc={rc}")
    return out


def check_gemm(D: np.ndarray, ref: np.ndarray, bound: np.ndarray, tol: float):
    """(n_bad, first_bad_flat_index, max |D-ref|/bound). D is (rows, cols) float32."""
    D = np.ascontiguousarray(D, dtype=np.float32)
    ref, bound = np.ascontiguousarray(ref), np.ascontiguousarray(bound)
    rows, cols = ref.shape
    fb = C.c_int64(0)
    mr = C.c_double(0)
    nb = lib().oracle_check_gemm(_p(D), rows, cols, D.shape[1], _p(ref), _p(bound), tol, C.byref(fb), C.byref(mr))
    return int(nb), int(fb.value), float(mr.value)
