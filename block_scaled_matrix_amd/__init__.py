"""block_scaled_matrix_amd - Python binding of libbsm, the gfx950 HIP library.

Argument marshalling only: every entry point forwards to the C function of the same
name in libbsm.so (declared in include/bsm.h) and raises BsmError on a negative
status. Device buffers are torch tensors (or raw device addresses); the stream is
torch's current HIP stream unless one is given. There is no other implementation of
these operations: if libbsm.so has not been built, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsm.so")

DTYPE = {"u8": 0, "u16": 1, "u32": 2, "f16": 3, "bf16": 4, "f32": 5, "e4m3": 6, "e2m1": 7, "e8m0": 8, "e5m2": 9,
         "e2m3": 10, "e3m2": 11}
ESIZE = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4, "e4m3": 1, "e8m0": 1, "e5m2": 1}
STATUS = {0: "BSM_OK", -1: "BSM_E_NULL", -2: "BSM_E_RANK", -3: "BSM_E_BOX", -4: "BSM_E_ESTRIDE",
          -5: "BSM_E_ALIGN", -6: "BSM_E_SWIZZLE", -7: "BSM_E_FILL", -8: "BSM_E_DTYPE", -9: "BSM_E_SHAPE",
          -10: "BSM_E_MAJOR", -11: "BSM_E_ALIAS", -12: "BSM_E_HIP", -13: "BSM_E_ARG"}
EWISE = {"none": 0, "silu_affine": 1}
EXPORTS = ("bsm_image_stride", "bsm_tile_box_load", "bsm_tile_box_store", "bsm_tile_box_copy",
           "bsm_tile_box_load_steps", "bsm_tile_box_store_steps", "bsm_tile_gather4", "bsm_tile_scatter4", "bsm_gemm",
           "bsm_gemm_block_scale", "bsm_gemm_ewise", "bsm_gemm_block_scale_ewise", "bsm_gemm_block_scale_major",
           "bsm_gemm_block_scale_fastacc", "bsm_debug_stream_mix_bf16", "bsm_debug_mfma_loop", "bsm_tile_add_scalar_f32", "bsm_debug_fragments", "bsm_debug_fragment_shape", "bsm_last_error")


class BsmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class bsm_tensor(C.Structure):
    _fields_ = [("base", C.c_void_p), ("dtype", C.c_int32), ("rank", C.c_int32),
                ("dims", C.c_int64 * 5), ("strides", C.c_int64 * 5)]


class bsm_box(C.Structure):
    _fields_ = [("rank", C.c_int32), ("box", C.c_int32 * 5), ("element_strides", C.c_int32 * 5),
                ("swizzle", C.c_int32), ("oob_fill", C.c_int32)]


class bsm_ewise(C.Structure):
    _fields_ = [("op", C.c_int32), ("scale", C.c_float), ("bias", C.c_float)]


_lib = None


def lib():
    """The loaded libbsm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python block_scaled_matrix_amd/_build.py)")
        L = C.CDLL(LIB_PATH)
        P, I64, I32 = C.c_void_p, C.c_int64, C.c_int32
        L.bsm_last_error.restype = C.c_char_p
        L.bsm_image_stride.restype = I64
        L.bsm_image_stride.argtypes = [C.POINTER(bsm_box), I32]
        L.bsm_tile_box_load.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_box), P, I64, P, P]
        L.bsm_tile_box_store.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_box), P, I64, P, C.c_int, P]
        L.bsm_tile_box_copy.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_tensor), C.POINTER(bsm_tensor),
                                        C.POINTER(bsm_box), P]
        L.bsm_tile_box_load_steps.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_box), P, I32, P, P, P, P]
        L.bsm_tile_box_store_steps.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_box), P, I32, P, P, P, C.c_int, P]
        L.bsm_tile_gather4.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_box), P, I64, P, P]
        L.bsm_tile_scatter4.argtypes = [C.POINTER(bsm_tensor), C.POINTER(bsm_box), P, I64, P, P]
        L.bsm_gemm.argtypes = [I64, I64, I64, I32, P, I64, C.c_char, P, I64, C.c_char, P, I64, C.c_int, C.c_int,
                               C.c_int, P]
        L.bsm_gemm_block_scale.argtypes = [I64, I64, I64, I32, P, I64, P, I64, I32, P, I64, P, I64, P, I64,
                                           C.c_int, C.c_int, C.c_int, P]
        L.bsm_gemm_ewise.argtypes = L.bsm_gemm.argtypes[:-1] + [C.POINTER(bsm_ewise), P]
        L.bsm_gemm_block_scale_ewise.argtypes = L.bsm_gemm_block_scale.argtypes[:-1] + [C.POINTER(bsm_ewise), P]
        L.bsm_gemm_block_scale_major.argtypes = [I64, I64, I64, I32, P, I64, C.c_char, P, I64, I32, P, I64, C.c_char,
                                                 P, I64, P, I64, C.c_int, C.c_int, C.c_int, C.POINTER(bsm_ewise), P]
        L.bsm_gemm_block_scale_fastacc.argtypes = L.bsm_gemm_block_scale_ewise.argtypes
        L.bsm_tile_add_scalar_f32.argtypes = [P, P, I64, C.c_float, P]
        L.bsm_debug_stream_mix_bf16.argtypes = [P, P, P, I64, P]
        L.bsm_debug_mfma_loop.argtypes = [I32, I64, I32, P, P]
        L.bsm_debug_fragments.argtypes = [P, I64, I64, C.c_char, P, P]
        L.bsm_debug_fragment_shape.restype = None
        L.bsm_debug_fragment_shape.argtypes = [C.POINTER(I64), C.POINTER(I64)]
        for rc_fn in ("bsm_tile_box_load", "bsm_tile_box_store", "bsm_tile_box_copy", "bsm_tile_box_load_steps",
                      "bsm_tile_box_store_steps", "bsm_tile_gather4",
                      "bsm_tile_scatter4", "bsm_gemm",
                      "bsm_gemm_block_scale", "bsm_gemm_ewise", "bsm_gemm_block_scale_ewise",
                      "bsm_gemm_block_scale_major", "bsm_gemm_block_scale_fastacc", "bsm_tile_add_scalar_f32",
                      "bsm_debug_fragments", "bsm_debug_stream_mix_bf16", "bsm_debug_mfma_loop"):
            getattr(L, rc_fn).restype = C.c_int
        _lib = L
    return _lib


def _ptr(x):
    """Device address of a torch tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc < 0:
        raise BsmError(rc, bsm_last_error())
    return rc


def bsm_last_error() -> str:
    return lib().bsm_last_error().decode()


def tensor_desc(base, dtype: str, dims, strides_bytes) -> bsm_tensor:
    """A bsm_tensor view: dims and byte strides outer to inner."""
    t = bsm_tensor()
    t.base = _ptr(base)
    t.dtype = DTYPE[dtype]
    t.rank = len(dims)
    for i, (d, s) in enumerate(zip(dims, strides_bytes)):
        t.dims[i] = int(d)
        t.strides[i] = int(s)
    return t


def box_desc(box, element_strides=None, swizzle: int = 0, oob_fill: int = 0) -> bsm_box:
    b = bsm_box()
    b.rank = len(box)
    es = element_strides or (1,) * len(box)
    for i, (x, e) in enumerate(zip(box, es)):
        b.box[i] = int(x)
        b.element_strides[i] = int(e)
    b.swizzle = swizzle
    b.oob_fill = oob_fill
    return b


def bsm_image_stride(box: bsm_box, dtype: str) -> int:
    return _check(lib().bsm_image_stride(C.byref(box), DTYPE[dtype]))


def bsm_tile_box_load(src: bsm_tensor, box: bsm_box, coords, n_boxes: int, images, stream=None):
    _check(lib().bsm_tile_box_load(C.byref(src), C.byref(box), _ptr(coords), n_boxes, _ptr(images),
                                   _stream(stream)))


def bsm_tile_box_store(dst: bsm_tensor, box: bsm_box, coords, n_boxes: int, images, reduce_add: int = 0,
                       stream=None):
    _check(lib().bsm_tile_box_store(C.byref(dst), C.byref(box), _ptr(coords), n_boxes, _ptr(images),
                                    reduce_add, _stream(stream)))


def bsm_tile_box_copy(src: bsm_tensor, dst: bsm_tensor | None, dst_add: bsm_tensor | None, box: bsm_box,
                      stream=None):
    _check(lib().bsm_tile_box_copy(C.byref(src), C.byref(dst) if dst is not None else None,
                                   C.byref(dst_add) if dst_add is not None else None, C.byref(box),
                                   _stream(stream)))


def _host_i64(xs):
    a = (C.c_int64 * max(len(xs), 1))(*[int(x) for x in xs])
    return a


def _repeat_args(coords, repeats, steps):
    rank = len(coords)
    flat = [int(v) for st in steps for v in st]
    assert len(flat) == rank * len(repeats)
    return (_host_i64(coords), len(repeats), (C.c_int32 * max(len(repeats), 1))(*[int(r) for r in repeats]),
            _host_i64(flat))


def bsm_tile_box_load_steps(src: bsm_tensor, box: bsm_box, coords, repeats, steps, images, stream=None):
    """coords: rank ints; repeats: one extent per repeat axis; steps: one rank-length vector per axis."""
    c, n, r, s = _repeat_args(coords, repeats, steps)
    _check(lib().bsm_tile_box_load_steps(C.byref(src), C.byref(box), c, n, r, s, _ptr(images), _stream(stream)))


def bsm_tile_box_store_steps(dst: bsm_tensor, box: bsm_box, coords, repeats, steps, images, reduce_add: int = 0,
                             stream=None):
    c, n, r, s = _repeat_args(coords, repeats, steps)
    _check(lib().bsm_tile_box_store_steps(C.byref(dst), C.byref(box), c, n, r, s, _ptr(images), reduce_add,
                                          _stream(stream)))


def bsm_tile_gather4(src: bsm_tensor, box: bsm_box, coords, n_issues: int, images, stream=None):
    _check(lib().bsm_tile_gather4(C.byref(src), C.byref(box), _ptr(coords), n_issues, _ptr(images), _stream(stream)))


def bsm_tile_scatter4(dst: bsm_tensor, box: bsm_box, coords, n_issues: int, images, stream=None):
    _check(lib().bsm_tile_scatter4(C.byref(dst), C.byref(box), _ptr(coords), n_issues, _ptr(images),
                                   _stream(stream)))


def bsm_gemm(M, N, K, ab: str, A, lda, a_major: str, B, ldb, b_major: str, D, ldd, neg_a=0, neg_b=0,
             accum=0, stream=None):
    _check(lib().bsm_gemm(M, N, K, DTYPE[ab], _ptr(A), lda, a_major.encode(), _ptr(B), ldb, b_major.encode(),
                          _ptr(D), ldd, neg_a, neg_b, accum, _stream(stream)))


def bsm_gemm_block_scale(M, N, K, a_fmt: str, A, lda, SFA, ld_sfa, b_fmt: str, B, ldb, SFB, ld_sfb, D, ldd,
                         neg_a=0, neg_b=0, accum=0, stream=None):
    _check(lib().bsm_gemm_block_scale(M, N, K, DTYPE[a_fmt], _ptr(A), lda, _ptr(SFA), ld_sfa, DTYPE[b_fmt],
                                      _ptr(B), ldb, _ptr(SFB), ld_sfb, _ptr(D), ldd, neg_a, neg_b, accum,
                                      _stream(stream)))


def ewise_desc(op: str = "silu_affine", scale: float = 1.0, bias: float = 0.0) -> bsm_ewise:
    """A bsm_ewise epilogue: op "none" or "silu_affine" (y = x / (1 + exp(-x)); y * scale + bias)."""
    return bsm_ewise(EWISE[op] if isinstance(op, str) else int(op), scale, bias)


def bsm_gemm_ewise(M, N, K, ab: str, A, lda, a_major: str, B, ldb, b_major: str, D, ldd, neg_a=0, neg_b=0,
                   accum=0, ew: bsm_ewise | None = None, stream=None):
    _check(lib().bsm_gemm_ewise(M, N, K, DTYPE[ab], _ptr(A), lda, a_major.encode(), _ptr(B), ldb,
                                b_major.encode(), _ptr(D), ldd, neg_a, neg_b, accum,
                                C.byref(ew) if ew is not None else None, _stream(stream)))


def bsm_gemm_block_scale_ewise(M, N, K, a_fmt: str, A, lda, SFA, ld_sfa, b_fmt: str, B, ldb, SFB, ld_sfb, D, ldd,
                               neg_a=0, neg_b=0, accum=0, ew: bsm_ewise | None = None, stream=None):
    _check(lib().bsm_gemm_block_scale_ewise(M, N, K, DTYPE[a_fmt], _ptr(A), lda, _ptr(SFA), ld_sfa, DTYPE[b_fmt],
                                            _ptr(B), ldb, _ptr(SFB), ld_sfb, _ptr(D), ldd, neg_a, neg_b, accum,
                                            C.byref(ew) if ew is not None else None, _stream(stream)))


def bsm_gemm_block_scale_major(M, N, K, a_fmt: str, A, lda, a_major: str, SFA, ld_sfa, b_fmt: str, B, ldb,
                               b_major: str, SFB, ld_sfb, D, ldd, neg_a=0, neg_b=0, accum=0,
                               ew: bsm_ewise | None = None, stream=None):
    _check(lib().bsm_gemm_block_scale_major(M, N, K, DTYPE[a_fmt], _ptr(A), lda, a_major.encode(), _ptr(SFA), ld_sfa,
                                            DTYPE[b_fmt], _ptr(B), ldb, b_major.encode(), _ptr(SFB), ld_sfb, _ptr(D),
                                            ldd, neg_a, neg_b, accum, C.byref(ew) if ew is not None else None,
                                            _stream(stream)))


def bsm_gemm_block_scale_fastacc(M, N, K, a_fmt: str, A, lda, SFA, ld_sfa, b_fmt: str, B, ldb, SFB, ld_sfb, D, ldd,
                                 neg_a=0, neg_b=0, accum=0, ew: bsm_ewise | None = None, stream=None):
    _check(lib().bsm_gemm_block_scale_fastacc(M, N, K, DTYPE[a_fmt], _ptr(A), lda, _ptr(SFA), ld_sfa, DTYPE[b_fmt],
                                              _ptr(B), ldb, _ptr(SFB), ld_sfb, _ptr(D), ldd, neg_a, neg_b, accum,
                                              C.byref(ew) if ew is not None else None, _stream(stream)))


def bsm_tile_add_scalar_f32(src, dst, n: int, s: float, stream=None):
    _check(lib().bsm_tile_add_scalar_f32(_ptr(src), _ptr(dst), n, s, _stream(stream)))


def bsm_debug_fragment_shape():
    r, k = C.c_int64(0), C.c_int64(0)
    lib().bsm_debug_fragment_shape(C.byref(r), C.byref(k))
    return r.value, k.value


def bsm_debug_fragments(src, rows: int, kdim: int, major: str, dump, stream=None):
    _check(lib().bsm_debug_fragments(_ptr(src), rows, kdim, major.encode(), _ptr(dump), _stream(stream)))


def bsm_debug_stream_mix_bf16(src, dst, add, n: int, stream=None):
    _check(lib().bsm_debug_stream_mix_bf16(_ptr(src), _ptr(dst), _ptr(add), n, _stream(stream)))


def bsm_debug_mfma_loop(kind: str, workgroups: int, iters: int, out, stream=None):
    _check(lib().bsm_debug_mfma_loop(DTYPE[kind], workgroups, iters, _ptr(out), _stream(stream)))
