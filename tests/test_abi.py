"""CPU tests of the C ABI: libbsm.so loads, exports every function include/bsm.h declares,
and rejects each kind of contract violation on the host with its status code (no call
here reaches the GPU: validation runs before any HIP call)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import block_scaled_matrix_amd as bsm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsm.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsm.LIB_PATH):
        from block_scaled_matrix_amd import _build
        _build.build()
    return bsm.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert set(decl) == set(bsm.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", bsm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (bsm_\w+)", out))
    assert set(decl) <= exported, set(decl) - exported
    for name in decl:
        assert hasattr(L, name)


FAKE = 1 << 40          # a 1 TiB-aligned fake device address: never dereferenced (checks fail first)


def tensor(dtype="bf16", dims=(64, 64), strides=None, base=FAKE):
    es = bsm.ESIZE.get(dtype, 1)
    strides = strides or tuple([dims[-1] * es * 1] * (len(dims) - 1) + [es])
    return bsm.tensor_desc(base, dtype, dims, strides)


def expect(code, fn, *args):
    with pytest.raises(bsm.BsmError) as e:
        fn(*args)
    assert e.value.status == code, (e.value.status, str(e.value))
    assert bsm.bsm_last_error()


def test_box_contract_violations(L):
    b = bsm.box_desc((16, 64), (1, 1), 3, 0)
    load = lambda t, bx, co=FAKE, n=1, img=FAKE + (1 << 30): bsm.bsm_tile_box_load(t, bx, co, n, img, 0)
    expect("BSM_E_NULL", load, tensor(base=0), b)
    expect("BSM_E_RANK", load, bsm.tensor_desc(FAKE, "bf16", (), ()), b)
    expect("BSM_E_RANK", load, tensor(dims=(4, 64, 64)), b)
    expect("BSM_E_BOX", load, tensor(), bsm.box_desc((300, 64)))
    expect("BSM_E_BOX", load, tensor(), bsm.box_desc((0, 64)))
    expect("BSM_E_ESTRIDE", load, tensor(), bsm.box_desc((16, 64), (9, 1)))
    expect("BSM_E_ESTRIDE", load, tensor(), bsm.box_desc((16, 64), (1, 2)))
    expect("BSM_E_ALIGN", load, tensor(base=FAKE + 8), b)
    expect("BSM_E_ALIGN", load, tensor(strides=(120, 2)), b)
    expect("BSM_E_ALIGN", load, tensor(strides=(128, 4)), b)
    expect("BSM_E_SWIZZLE", load, tensor(), bsm.box_desc((16, 64), (1, 1), 4))
    expect("BSM_E_SWIZZLE", load, tensor(), bsm.box_desc((16, 64), (1, 1), 2))   # 128-byte row > 64-byte span
    expect("BSM_E_SWIZZLE", load, tensor(), bsm.box_desc((16, 12)))              # 24-byte rows
    expect("BSM_E_FILL", load, tensor("u16"), bsm.box_desc((16, 64), (1, 1), 0, 1))
    expect("BSM_E_FILL", load, tensor(), bsm.box_desc((16, 64), (1, 1), 0, 2))
    expect("BSM_E_DTYPE", load, bsm.tensor_desc(FAKE, "e2m1", (64, 64), (64, 1)), b)
    expect("BSM_E_BOX", load, tensor("f32", dims=(4, 256, 64)), bsm.box_desc((4, 256, 64)))  # 256 KiB image
    expect("BSM_E_ALIGN", load, tensor(), b, FAKE, 1, FAKE + (1 << 30) + 512)             # image not 1024-aligned
    expect("BSM_E_ALIAS", load, tensor(), b, FAKE, 1, FAKE + 1024)                       # image inside src
    expect("BSM_E_SHAPE", load, tensor(), b, FAKE, -1)
    expect("BSM_E_SHAPE", load, tensor(dims=(0, 64)), b)
    bsm.bsm_tile_box_load(tensor(), b, 0, 0, 0, 0)        # n_boxes == 0: no-op, pointers unused
    st = lambda t, red: bsm.bsm_tile_box_store(t, b, FAKE, 1, FAKE + (1 << 30), red, 0)
    expect("BSM_E_DTYPE", st, tensor("u16"), 1)
    expect("BSM_E_ARG", st, tensor(), 2)
    cp = bsm.bsm_tile_box_copy
    src = tensor()
    expect("BSM_E_NULL", cp, src, None, None, b, 0)
    expect("BSM_E_ALIAS", cp, src, tensor(base=FAKE + 4096), None, b, 0)
    expect("BSM_E_SHAPE", cp, src, tensor(dims=(64, 32), base=FAKE + (1 << 30)), None, b, 0)
    expect("BSM_E_DTYPE", cp, src, tensor("f16", base=FAKE + (1 << 30)), None, b, 0)
    expect("BSM_E_DTYPE", cp, tensor("u16"), None, tensor("u16", base=FAKE + (1 << 30)), b, 0)
    sl = lambda *a: bsm.bsm_tile_box_load_steps(*a, stream=0)
    expect("BSM_E_ARG", sl, tensor(), b, (0, 0), (1, 1, 1, 1, 1), [(0, 0)] * 5, FAKE + (1 << 30))  # 5 axes
    expect("BSM_E_SHAPE", sl, tensor(), b, (0, 0), (0,), [(8, 0)], FAKE + (1 << 30))              # empty axis
    expect("BSM_E_SHAPE", sl, tensor(), b, (0, 0), (3,), [(1 << 30, 0)], FAKE + (1 << 30))        # 2^31 reached
    expect("BSM_E_SHAPE", sl, tensor(), b, (0, -(1 << 31)), (2,), [(0, -1)], FAKE + (1 << 30))    # below -2^31
    expect("BSM_E_SHAPE", sl, tensor(), b, (0, 0), (1 << 16, 1 << 16), [(0, 0), (0, 0)], FAKE + (1 << 30))
    expect("BSM_E_RANK", sl, tensor(), bsm.box_desc((16, 64, 8)), (0, 0, 0), (), [], FAKE + (1 << 30))
    expect("BSM_E_NULL", sl, tensor(), b, (0, 0), (2,), [(8, 0)], 0)                              # images NULL
    expect("BSM_E_ALIAS", sl, tensor(), b, (0, 0), (2,), [(8, 0)], FAKE + 1024)
    expect("BSM_E_NULL", lambda: bsm._check(L.bsm_tile_box_load_steps(C.byref(tensor()), C.byref(b), None, 0, None,
                                                                      None, C.c_void_p(FAKE + (1 << 30)), None)))
    ss = lambda *a: bsm.bsm_tile_box_store_steps(*a, stream=0)
    expect("BSM_E_DTYPE", ss, tensor("u16"), b, (0, 0), (2,), [(8, 0)], FAKE + (1 << 30), 1)
    expect("BSM_E_ARG", ss, tensor(), b, (0, 0), (2,), [(8, 0)], FAKE + (1 << 30), 2)
    g4 = bsm.box_desc((1, 64), (1, 1), 3)
    for fn in (bsm.bsm_tile_gather4, bsm.bsm_tile_scatter4):
        call = lambda t, bx, co=FAKE, n=1, img=FAKE + (1 << 30), fn=fn: fn(t, bx, co, n, img, 0)
        expect("BSM_E_NULL", call, tensor(base=0), g4)
        expect("BSM_E_RANK", call, tensor(dims=(4, 64, 64)), bsm.box_desc((1, 1, 64)))
        expect("BSM_E_RANK", call, tensor(), bsm.box_desc((1, 1, 64)))
        expect("BSM_E_BOX", call, tensor(), bsm.box_desc((4, 64)))              # a box of one row only
        expect("BSM_E_BOX", call, tensor(), bsm.box_desc((1, 300)))
        expect("BSM_E_ESTRIDE", call, tensor(), bsm.box_desc((1, 64), (2, 1)))
        expect("BSM_E_SWIZZLE", call, tensor(), bsm.box_desc((1, 12)))          # 24-byte rows
        expect("BSM_E_SWIZZLE", call, tensor(), bsm.box_desc((1, 128), (1, 1), 3))  # 256-byte row > 128
        expect("BSM_E_FILL", call, tensor("u16"), bsm.box_desc((1, 64), (1, 1), 0, 1))
        expect("BSM_E_SHAPE", call, tensor(), g4, FAKE, -1)
        expect("BSM_E_SHAPE", call, tensor(), g4, FAKE, (1 << 33) + 1)
        expect("BSM_E_NULL", call, tensor(), g4, 0)
        expect("BSM_E_ALIGN", call, tensor(), g4, FAKE + 2)
        expect("BSM_E_ALIGN", call, tensor(), g4, FAKE, 1, FAKE + (1 << 30) + 512)    # images not 1024-aligned
        expect("BSM_E_ALIAS", call, tensor(), g4, FAKE, 1, FAKE + 1024)
        fn(tensor(), g4, 0, 0, 0, 0)                      # n_issues == 0: no-op
    assert bsm.bsm_image_stride(bsm.box_desc((128, 64), (1, 1), 3), "bf16") == 16384
    assert bsm.bsm_image_stride(bsm.box_desc((8, 16)), "u32") == 512
    assert bsm.bsm_image_stride(bsm.box_desc((3, 8), (1, 1), 2), "bf16") == 512
    assert bsm.bsm_image_stride(bsm.box_desc((5, 16), (2, 1), 0), "u8") == 128


def test_gemm_contract_violations(L):
    A, B, D = FAKE, FAKE + (1 << 32), FAKE + (2 << 32)
    g = lambda *a: bsm.bsm_gemm(*a, stream=0)
    expect("BSM_E_DTYPE", g, 64, 64, 64, "f32", A, 64, "k", B, 64, "k", D, 64)
    expect("BSM_E_MAJOR", g, 64, 64, 64, "bf16", A, 64, "n", B, 64, "k", D, 64)
    expect("BSM_E_MAJOR", g, 64, 64, 64, "bf16", A, 64, "k", B, 64, "m", D, 64)
    expect("BSM_E_SHAPE", g, -1, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 64)
    expect("BSM_E_ALIGN", g, 64, 64, 64, "bf16", A, 60, "k", B, 64, "k", D, 64)     # lda < K
    expect("BSM_E_ALIGN", g, 64, 64, 60, "bf16", A, 60, "k", B, 64, "k", D, 64)     # lda % 8
    expect("BSM_E_ALIGN", g, 64, 64, 64, "bf16", A + 2, 64, "k", B, 64, "k", D, 64)
    expect("BSM_E_ALIGN", g, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 62)     # ldd < N
    expect("BSM_E_ALIGN", g, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D + 4, 64)
    expect("BSM_E_NULL", g, 64, 64, 64, "bf16", 0, 64, "k", B, 64, "k", D, 64)
    expect("BSM_E_NULL", g, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", 0, 64)
    expect("BSM_E_ALIAS", g, 64, 64, 64, "bf16", D + 1024, 64, "k", B, 64, "k", D, 64)
    expect("BSM_E_ARG", g, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 64, 2)
    expect("BSM_E_SHAPE", g, 64, 64, 64, "bf16", A, 1 << 23, "k", B, 64, "k", D, 64)    # 32-bit tile offsets
    expect("BSM_E_ARG", g, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 64, 0, 0, 3)
    bsm.bsm_gemm(0, 64, 64, "bf16", 0, 0, "k", 0, 0, "k", 0, 0, stream=0)      # M == 0: no-op
    s = lambda *a: bsm.bsm_gemm_block_scale(*a, stream=0)
    SA, SB = FAKE + (3 << 32), FAKE + (4 << 32)
    expect("BSM_E_DTYPE", s, 64, 64, 64, "bf16", A, 64, SA, 4, "bf16", B, 64, SB, 4, D, 64)
    expect("BSM_E_DTYPE", s, 64, 64, 64, "e4m3", A, 64, SA, 4, "f16", B, 64, SB, 4, D, 64)
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e2m3", A, 96, SA, 4, "e4m3", B, 64, SB, 4, D, 64)   # 72-byte fp6 rows
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e4m3", A, 64, SA, 4, "e3m2", B, 32, SB, 4, D, 64)   # ldb < K
    expect("BSM_E_SHAPE", s, 64, 64, 48, "e4m3", A, 64, SA, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e4m3", A, 72, SA, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e2m1", A, 80, SA, 4, "e2m1", B, 64, SB, 4, D, 64)   # 40-byte rows
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e4m3", A, 64, SA, 1, "e4m3", B, 64, SB, 4, D, 64)   # ld_sfa < K/32
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e4m3", A, 64, SA, 2, "e4m3", B, 64, SB, 4, D, 64)   # ld_sfa % 4
    expect("BSM_E_ALIGN", s, 64, 64, 64, "e4m3", A, 64, SA + 2, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_NULL", s, 64, 64, 64, "e4m3", A, 64, 0, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_ALIAS", s, 64, 64, 64, "e4m3", A, 64, D + 64, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_SHAPE", s, 64, 64, 64, "e4m3", A, 1 << 24, SA, 4, "e4m3", B, 64, SB, 4, D, 64)
    ew = bsm.ewise_desc("silu_affine", 2.0, 1.0)
    ge = lambda *a, ew=ew: bsm.bsm_gemm_ewise(*a[:15], ew=a[15] if len(a) > 15 else ew, stream=0)
    expect("BSM_E_NULL", lambda: bsm.bsm_gemm_ewise(64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 64, stream=0))
    expect("BSM_E_ARG", ge, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 64, 0, 0, 0, bsm.ewise_desc(2))
    expect("BSM_E_ARG", ge, 64, 64, 64, "bf16", A, 64, "k", B, 64, "k", D, 64, 0, 0, 0, bsm.ewise_desc(-1))
    expect("BSM_E_DTYPE", ge, 64, 64, 64, "f32", A, 64, "k", B, 64, "k", D, 64)     # plain-call rules hold
    expect("BSM_E_ALIAS", ge, 64, 64, 64, "bf16", D + 1024, 64, "k", B, 64, "k", D, 64)
    bsm.bsm_gemm_ewise(64, 0, 64, "bf16", 0, 0, "k", 0, 0, "k", 0, 0, ew=ew, stream=0)   # N == 0: no-op
    se = lambda *a: bsm.bsm_gemm_block_scale_ewise(*a[:18], ew=a[18] if len(a) > 18 else ew, stream=0)
    expect("BSM_E_NULL", lambda: bsm.bsm_gemm_block_scale_ewise(64, 64, 64, "e4m3", A, 64, SA, 4, "e4m3", B, 64, SB,
                                                                4, D, 64, stream=0))
    expect("BSM_E_ARG", se, 64, 64, 64, "e4m3", A, 64, SA, 4, "e4m3", B, 64, SB, 4, D, 64, 0, 0, 0,
           bsm.ewise_desc(7))
    expect("BSM_E_SHAPE", se, 64, 64, 48, "e4m3", A, 64, SA, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_DTYPE", se, 64, 64, 64, "e4m3", A, 64, SA, 4, "bf16", B, 64, SB, 4, D, 64)
    sm = lambda *a, ew=None: bsm.bsm_gemm_block_scale_major(*a, ew=ew, stream=0)
    expect("BSM_E_MAJOR", sm, 64, 64, 64, "e4m3", A, 64, "n", SA, 4, "e4m3", B, 64, "k", SB, 4, D, 64)
    expect("BSM_E_MAJOR", sm, 64, 64, 64, "e4m3", A, 64, "k", SA, 4, "e4m3", B, 64, "m", SB, 4, D, 64)
    expect("BSM_E_MAJOR", sm, 64, 64, 64, "e2m3", A, 64, "m", SA, 4, "e4m3", B, 64, "k", SB, 4, D, 64)  # fp6 MN
    expect("BSM_E_MAJOR", sm, 64, 64, 64, "e4m3", A, 64, "k", SA, 4, "e3m2", B, 64, "n", SB, 4, D, 64)
    expect("BSM_E_ALIGN", sm, 96, 64, 64, "e4m3", A, 64, "m", SA, 4, "e4m3", B, 64, "k", SB, 4, D, 64)  # lda < M
    expect("BSM_E_ALIGN", sm, 64, 96, 64, "e4m3", A, 64, "k", SA, 4, "e2m1", B, 64, "n", SB, 4, D, 64)  # ldb < N
    expect("BSM_E_ALIGN", sm, 64, 64, 64, "e2m1", A, 72, "m", SA, 4, "e4m3", B, 64, "k", SB, 4, D, 64)  # 36-byte rows
    expect("BSM_E_SHAPE", sm, 64, 64, 48, "e4m3", A, 64, "m", SA, 4, "e4m3", B, 64, "n", SB, 4, D, 64)
    expect("BSM_E_SHAPE", sm, 64, 64, 64, "e4m3", A, 1 << 24, "m", SA, 4, "e4m3", B, 64, "n", SB, 4, D, 64)
    expect("BSM_E_ARG", lambda: sm(64, 64, 64, "e4m3", A, 64, "m", SA, 4, "e4m3", B, 64, "n", SB, 4, D, 64,
                                   ew=bsm.ewise_desc(5)))
    # an MN-major A spans K = 128 rows of lda = 64 bytes (8 KiB, where M rows of it would span 4 KiB)
    expect("BSM_E_ALIAS", sm, 64, 64, 128, "e4m3", A, 64, "m", SA, 4, "e4m3", B, 128, "k", SB, 4, A + 4096, 64)
    bsm.bsm_gemm_block_scale_major(64, 0, 64, "e4m3", 0, 0, "m", 0, 0, "e4m3", 0, 0, "n", 0, 0, 0, 0, stream=0)
    # the fast-accumulation call keeps every rule of the plain call; ew may be NULL
    sf = lambda *a, ew=None: bsm.bsm_gemm_block_scale_fastacc(*a, ew=ew, stream=0)
    expect("BSM_E_SHAPE", sf, 64, 64, 48, "e4m3", A, 64, SA, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_DTYPE", sf, 64, 64, 64, "e4m3", A, 64, SA, 4, "bf16", B, 64, SB, 4, D, 64)
    expect("BSM_E_ALIGN", sf, 64, 64, 64, "e4m3", A, 72, SA, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_ALIAS", sf, 64, 64, 64, "e4m3", A, 64, D + 64, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_NULL", sf, 64, 64, 64, "e4m3", A, 64, 0, 4, "e4m3", B, 64, SB, 4, D, 64)
    expect("BSM_E_ARG", lambda: sf(64, 64, 64, "e4m3", A, 64, SA, 4, "e4m3", B, 64, SB, 4, D, 64,
                                   ew=bsm.ewise_desc(9)))
    bsm.bsm_gemm_block_scale_fastacc(0, 64, 64, "e4m3", 0, 0, 0, 0, "e4m3", 0, 0, 0, 0, 0, 0, stream=0)
    a = lambda *x: bsm.bsm_tile_add_scalar_f32(*x, stream=0)
    expect("BSM_E_SHAPE", a, A, B, -1, 1.0)
    expect("BSM_E_ALIGN", a, A + 4, B, 8, 1.0)
    expect("BSM_E_ALIAS", a, A, A + 16, 8, 1.0)
    expect("BSM_E_NULL", a, 0, B, 8, 1.0)
    mix = lambda *x: bsm.bsm_debug_stream_mix_bf16(*x, stream=0)
    expect("BSM_E_SHAPE", mix, A, B, D, 12)                      # not a multiple of 8
    expect("BSM_E_SHAPE", mix, A, B, D, -8)
    expect("BSM_E_NULL", mix, A, 0, D, 8)
    expect("BSM_E_ALIGN", mix, A + 8, B, D, 8)
    expect("BSM_E_ALIAS", mix, A, A + 16, D, 64)
    bsm.bsm_debug_stream_mix_bf16(0, 0, 0, 0, stream=0)           # n == 0: no-op
    loop = lambda *x: bsm.bsm_debug_mfma_loop(*x, stream=0)
    expect("BSM_E_DTYPE", loop, "f16", 4, 4, D)
    expect("BSM_E_SHAPE", loop, "bf16", 0, 4, D)
    expect("BSM_E_SHAPE", loop, "e4m3", 4, (1 << 20) + 1, D)
    expect("BSM_E_NULL", loop, "e2m1", 4, 4, 0)
    expect("BSM_E_ALIGN", loop, "bf16", 4, 4, D + 2)
    rows, kdim = bsm.bsm_debug_fragment_shape()
    expect("BSM_E_SHAPE", bsm.bsm_debug_fragments, A, rows, kdim + 16, "k", B, 0)
    expect("BSM_E_MAJOR", bsm.bsm_debug_fragments, A, rows, kdim, "n", B, 0)


def test_error_state_is_per_call(L):
    expect("BSM_E_DTYPE", lambda: bsm.bsm_gemm(1, 1, 1, "f32", FAKE, 8, "k", FAKE, 8, "k", FAKE + 4096, 4, stream=0))
    bsm.bsm_gemm(0, 1, 1, "bf16", 0, 0, "k", 0, 0, "k", 0, 0, stream=0)
    assert bsm.bsm_last_error() == ""
