"""GPU parity: dense fp16/bf16 GEMM, block-scaled MXFP8/MXFP4 GEMM and the fragment loads.

Tolerances (the stated bound of the method, written out):
  dense:        |D - ref| <= 2e-3 * sum_k |a_mk b_nk|  (+ half an ulp of the float32 result)
  block scaled: |D - ref| <= 1e-5 * sum_k |a_mk b_nk|  (+ half an ulp; mx_check.check_strict)
Inputs whose every partial sum is exact in float32 must match bit for bit. Only the
fast-accumulation call (bsm_gemm_block_scale_fastacc) is checked with the scaled MFMA's
block-window allowance (mx_check.check_window).
"""
import numpy as np
import pytest
import torch

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_f32, host, say
from mx_check import TOL_MX, check_strict, check_window, note, pad_cols, pad_scales, pair_case

pytestmark = pytest.mark.gpu

TOL_DENSE = 2e-3


def run_dense(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, D0=None, neg_a=0, neg_b=0, accum=0, ldd=None):
    ldd = ldd or ((N + 3) // 4 * 4)
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    bsm.bsm_gemm(M, N, K, dt, dev(A), lda, amaj, dev(B), ldb, bmaj, dD, ldd, neg_a, neg_b, accum)
    return dD.cpu().numpy()


def dense_case(rng, M, N, K, dt, amaj, bmaj, exact=False):
    if exact:
        a = (rng.integers(-4, 5, (M, K)) / 4).astype(np.float32)
        b = (rng.integers(-4, 5, (N, K)) / 4).astype(np.float32)
    else:
        a = rng.standard_normal((M, K)).astype(np.float32)
        b = rng.standard_normal((N, K)).astype(np.float32)
    a, b = W.to_half_bits(a, dt), W.to_half_bits(b, dt)
    if amaj == "k":
        lda = (K + 7) // 8 * 8
        A = pad_cols(a, lda)
    else:
        lda = (M + 7) // 8 * 8
        A = pad_cols(np.ascontiguousarray(a.T), lda)
    if bmaj == "k":
        ldb = (K + 7) // 8 * 8
        B = pad_cols(b, ldb)
    else:
        ldb = (N + 7) // 8 * 8
        B = pad_cols(np.ascontiguousarray(b.T), ldb)
    return A, lda, B, ldb


def test_pages_tcgen05_example_bit_exact(O):
    """The example GEMM of "tcgen05.mma" (Example: four K16 issues): M = 128, N = K = 64, fp16
    operands on the quarter grid from seed 0. Every sum is exact in float32, so the result must
    equal the oracle's bit for bit (the page itself checks to 2e-4, relative and absolute)."""
    a, b = W.quarter_grid_f16(0)
    say("gemm pages example")
    D = run_dense(128, 64, 64, "f16", a, 64, "k", b, 64, "k")[:, :64]
    ref, _ = O.gemm(128, 64, 64, "f16", a, 64, "k", b, 64, "k")
    assert np.array_equal(D, ref.astype(np.float32))
    want = a.view(np.float16).astype(np.float64) @ b.view(np.float16).astype(np.float64).T
    assert (np.abs(D - want) <= 2e-4 * (1.0 + np.abs(want))).all()


def test_gemm_f16_128_workload(O):
    w = W.gemm_f16_128()
    say("gemm f16 128x128x64")
    D = run_dense(128, 128, 64, "f16", w["A"], 64, "k", w["B"], 64, "k")
    assert not np.isnan(D).any()
    ref, bound = O.gemm(128, 128, 64, "f16", w["A"], 64, "k", w["B"], 64, "k")
    nb, first, worst = O.check_gemm(D, ref, bound, TOL_DENSE)
    assert nb == 0, (first, worst)


SHAPES = [(1, 1, 1), (7, 9, 5), (17, 33, 9), (64, 64, 64), (255, 257, 130), (300, 520, 200), (513, 130, 64),
          (96, 272, 1000), (33, 40, 31), (40, 33, 33), (64, 64, 96), (256, 256, 33), (64, 72, 128)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("amaj,bmaj", [("k", "k"), ("k", "n"), ("m", "k"), ("m", "n")])
def test_dense_vs_oracle(O, dt, amaj, bmaj):
    rng = np.random.default_rng([ord(c) for c in dt + amaj + bmaj])
    for i, (M, N, K) in enumerate(SHAPES):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        A, lda, B, ldb = dense_case(rng, M, N, K, dt, amaj, bmaj)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        say("dense", dt, amaj, bmaj, M, N, K, neg_a, neg_b, accum)
        D = run_dense(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = O.gemm(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, d0, N, neg_a, neg_b, accum)
        nb, first, worst = O.check_gemm(D, ref, bound, TOL_DENSE)
        assert nb == 0, (M, N, K, first, worst)
        assert np.isnan(D[:, N:]).all()  # columns past N of the padded D are never written


@pytest.mark.parametrize("amaj,bmaj", [("k", "k"), ("k", "n"), ("m", "n")])
def test_dense_exact_sums_bit_exact(O, amaj, bmaj):
    rng = np.random.default_rng(5)
    for M, N, K in [(256, 256, 64), (130, 300, 96), (512, 256, 200)]:
        A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", amaj, bmaj, exact=True)
        say("dense exact", amaj, bmaj, M, N, K)
        D = run_dense(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj)
        ref, _ = O.gemm(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj)
        assert np.array_equal(D[:, :N], ref.astype(np.float32))


def test_dense_accum_zero_A_and_determinism(O):
    rng = np.random.default_rng(6)
    M, N, K = 300, 260, 128
    A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", "k", "n")
    d0 = rng.standard_normal((M, N)).astype(np.float32)
    say("dense accum with A = 0")
    D = run_dense(M, N, K, "bf16", np.zeros_like(A), lda, "k", B, ldb, "n", d0, 1, 0, 1)
    assert np.array_equal(D[:, :N], d0)
    say("dense determinism")
    D1 = run_dense(M, N, K, "bf16", A, lda, "k", B, ldb, "n", d0, 0, 0, 1)
    D2 = run_dense(M, N, K, "bf16", A, lda, "k", B, ldb, "n", d0, 0, 0, 1)
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32))
    Dn = run_dense(M, N, K, "bf16", A, lda, "k", B, ldb, "n", None, 1, 0, 0)
    Dp = run_dense(M, N, K, "bf16", A, lda, "k", B, ldb, "n", None, 0, 0, 0)
    assert np.array_equal(Dn[:, :N], -Dp[:, :N])


@pytest.mark.parametrize("amaj,bmaj", [("k", "k"), ("k", "n"), ("m", "k"), ("m", "n")])
def test_dense_accum_long_k(O, amaj, bmaj):
    """Accumulation after a long K loop (32 or more whole K tiles of 64; the epilogue adds D to
    the sum once): ragged M and N edges, a ragged K tail, both signs; then A = 0, where D must
    come back bit for bit under either sign."""
    rng = np.random.default_rng([7, ord(amaj), ord(bmaj)])
    for i, (M, N, K) in enumerate([(300, 260, 2088), (256, 512, 2048), (130, 300, 4112)]):
        A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", amaj, bmaj)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        neg_a, neg_b = i & 1, (i >> 1) & 1
        say("dense accum long K", amaj, bmaj, M, N, K, neg_a, neg_b)
        D = run_dense(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj, d0, neg_a, neg_b, 1)
        ref, bound = O.gemm(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj, d0, N, neg_a, neg_b, 1)
        nb, first, worst = O.check_gemm(D, ref, bound, TOL_DENSE)
        assert nb == 0, (M, N, K, first, worst)
        assert np.isnan(D[:, N:]).all()
    M, N, K = 300, 260, 2048
    A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", amaj, bmaj)
    d0 = rng.standard_normal((M, N)).astype(np.float32)
    for neg_a in (0, 1):
        say("dense accum long K with A = 0", amaj, bmaj, neg_a)
        D = run_dense(M, N, K, "bf16", np.zeros_like(A), lda, amaj, B, ldb, bmaj, d0, neg_a, 0, 1)
        assert np.array_equal(D[:, :N], d0)


@pytest.mark.parametrize("amaj,bmaj", [("m", "n"), ("k", "n")])
def test_dense_ragged_copies_repeated(O, amaj, bmaj):
    """Regression for the copies' hardware wait states (the 5 a vector-memory read of a
    VALU-written SGPR base needs, which inline assembly must pad for itself): without them,
    ragged MN-major accumulating GEMMs came out wrong on some runs and right on others. Each
    case runs five times; every run must meet the bound and match the first bit for bit."""
    rng = np.random.default_rng([11, ord(amaj), ord(bmaj)])
    for M, N, K in [(300, 520, 200), (96, 272, 1000), (513, 130, 456)]:
        A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", amaj, bmaj)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        ref, bound = O.gemm(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj, d0, N, 1, 0, 1)
        first_run = None
        for rep in range(5):
            say("dense ragged repeated", amaj, bmaj, M, N, K, "run", rep)
            D = run_dense(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj, d0, 1, 0, 1)
            nb, first, worst = O.check_gemm(D, ref, bound, TOL_DENSE)
            assert nb == 0, (M, N, K, rep, first, worst)
            if first_run is None:
                first_run = D
            assert np.array_equal(D.view(np.uint32), first_run.view(np.uint32)), (M, N, K, rep)


@pytest.mark.parametrize("M,N,K,amaj,bmaj", [(1, 300, 131112, "k", "n"), (300, 1, 131072, "m", "k"),
                                             (3, 5, 262144, "k", "k")])
def test_dense_long_k_thin(O, M, N, K, amaj, bmaj):
    """Degenerate widths (one row or column: every workgroup but one masked away) with K in the
    hundreds of thousands (2048 to 4096 K tiles, one with a ragged tail), accumulating."""
    rng = np.random.default_rng(K + M)
    A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", amaj, bmaj)
    d0 = rng.standard_normal((M, N)).astype(np.float32)
    say("dense long K thin", M, N, K, amaj, bmaj)
    D = run_dense(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj, d0, 1, 0, 1)
    ref, bound = O.gemm(M, N, K, "bf16", A, lda, amaj, B, ldb, bmaj, d0, N, 1, 0, 1)
    nb, first, worst = O.check_gemm(D, ref, bound, TOL_DENSE)
    assert nb == 0, (first, worst)
    assert np.isnan(D[:, N:]).all()


def test_dense_k_zero():
    say("dense K = 0")
    D = run_dense(5, 6, 0, "bf16", np.zeros((5, 8), np.uint16), 8, "k", np.zeros((6, 8), np.uint16), 8, "k")
    assert (D[:, :6] == 0).all()
    d0 = np.arange(30, dtype=np.float32).reshape(5, 6)
    D = run_dense(5, 6, 0, "bf16", np.zeros((5, 8), np.uint16), 8, "k", np.zeros((6, 8), np.uint16), 8, "k", d0,
                  accum=1)
    assert np.array_equal(D[:, :6], d0)


def test_gemm_bf16_8192_sampled(O):
    """M = N = K = 8192 bf16, A K-major, B MN-major, accumulate onto D0: sampled outputs."""
    w = W.gemm_bf16()
    M, N, K = w["M"], w["N"], w["K"]
    say("gemm bf16 8192 full")
    dA, dB = dev(w["A"]), dev(w["B"])
    dD = dev_f32(w["D0"])
    bsm.bsm_gemm(M, N, K, "bf16", dA, K, "k", dB, N, "n", dD, N, 0, 0, 1)
    D = dD.cpu().numpy()
    pm, pn = W.sample_points(M, N, 2000)
    ref, bound = O.gemm_points(M, N, K, "bf16", w["A"], K, "k", w["B"], N, "n", w["D0"], N, 0, 0, 1, pm, pn)
    nb, first, worst = O.check_gemm(D[pm, pn].reshape(1, -1), ref.reshape(1, -1), bound.reshape(1, -1), TOL_DENSE)
    assert nb == 0, (first, worst)
    assert np.isfinite(D).all()


# ----------------------------------------------------------------------------- fragments
@pytest.mark.parametrize("major", ["k", "m"])
def test_fragment_loads_vs_oracle_ldmatrix_image(O, major):
    """The dense kernel's LDS->register fragment reads, mapped back through the MFMA
    operand lane map, equal the oracle's 8x8 b16 matrix images (transposed for the
    MN-major storage: the .trans image rule)."""
    rows, kdim = bsm.bsm_debug_fragment_shape()
    rng = np.random.default_rng(3)
    op = rng.integers(0, 2 ** 16, (rows, kdim), dtype=np.uint64).astype(np.uint16)   # logical operand (row, k)
    stored = op if major == "k" else np.ascontiguousarray(op.T)                     # storage order
    dump = torch.zeros((rows // 16) * (kdim // 32) * 64 * 8, dtype=torch.int16, device="cuda")
    say("fragments", major)
    bsm.bsm_debug_fragments(dev(stored), rows, kdim, major, dump)
    got = host(dump, np.uint16).reshape(rows // 16, kdim // 32, 64, 8)
    # oracle: 8x8 matrices of the stored array; with transpose for MN-major storage
    sb = stored.view(np.uint8).reshape(-1)
    row_pitch = stored.shape[1] * 2
    for b in range(rows // 16):
        for s in range(kdim // 32):
            for lane in range(64):
                # the 16x16x32 MFMA operand: lane l holds row l%16 of the block, k 8(l/16)..+7 of the step
                r, kb = 16 * b + lane % 16, 32 * s + 8 * (lane // 16)
                if major == "k":   # matrix rows are operand rows r8..r8+7, columns k8..k8+7
                    r8, k8 = r - r % 8, kb
                    offs = [(r8 + j) * row_pitch + k8 * 2 for j in range(8)]
                    regs = O.ldmatrix(sb, offs, 1, 0)
                else:              # stored rows are k: matrix rows k8.., columns r8..; transpose
                    r8, k8 = r - r % 8, kb
                    offs = [(k8 + j) * row_pitch + r8 * 2 for j in range(8)]
                    regs = O.ldmatrix(sb, offs, 1, 1)
                j = r % 8       # image row j (operand row r) owned by lanes 4j..4j+3
                vals = []
                for w in range(4):
                    word = int(regs[4 * j + w, 0])
                    vals += [word & 0xFFFF, word >> 16]
                assert list(got[b, s, lane]) == vals, (b, s, lane)
                assert vals == list(op[r, kb:kb + 8])


# ----------------------------------------------------------------------------- block scaled
def run_mx(M, N, K, fmt, g, D0=None, neg_a=0, neg_b=0, accum=0, b_fmt=None):
    ldd = (N + 3) // 4 * 4
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    bsm.bsm_gemm_block_scale(M, N, K, fmt, dev(g["A"]), g["lda"], dev(g["SFA"]), g["ld_sfa"], b_fmt or fmt, dev(g["B"]),
                             g["ldb"], dev(g["SFB"]), g["ld_sfb"], dD, ldd, neg_a, neg_b, accum)
    return dD.cpu().numpy()


def mx_case(fmt, seed, M, N, K, exp_range=4, ld_pad=0, b_fmt=None):
    if fmt == "e2m1":
        g = W.mxfp4(seed=seed, M=M, N=N, K=K, exp_range=exp_range)
    else:
        g = W.mxfp8(seed=seed, M=M, N=N, K=K, exp_range=exp_range, a_fmt=fmt, b_fmt=b_fmt or fmt)
    if ld_pad:
        epb = 2 if fmt == "e2m1" else 1
        lda = K + ld_pad
        g["A"] = pad_cols(g["A"].reshape(M, -1), lda // epb)
        g["B"] = pad_cols(g["B"].reshape(N, -1), lda // epb)
        g["lda"] = g["ldb"] = lda
    ld_sf = (K // 32 + 3) // 4 * 4 + (4 if ld_pad else 0)    # scale rows start 4-byte aligned
    g["SFA"], g["SFB"] = pad_scales(g["SFA"], ld_sf), pad_scales(g["SFB"], ld_sf)
    g["ld_sfa"] = g["ld_sfb"] = ld_sf
    return g


MX_SHAPES = [(1, 1, 32), (9, 17, 64), (33, 40, 96), (256, 256, 128), (300, 260, 288), (130, 513, 512),
             (64, 96, 1056), (64, 64, 160), (64, 64, 224), (40, 40, 192)]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_block_scale_vs_oracle(O, fmt):
    for i, (M, N, K) in enumerate(MX_SHAPES):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        g = mx_case(fmt, 10 + i, M, N, K, ld_pad=64 if i % 3 == 2 else 0)
        rng = np.random.default_rng(i)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        say("mx", fmt, M, N, K, neg_a, neg_b, accum)
        D = run_mx(M, N, K, fmt, g, d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = O.gemm_block_scale(M, N, K, fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], fmt, g["B"], g["ldb"],
                                        g["SFB"], g["ld_sfb"], d0, N, neg_a, neg_b, accum)
        nb, worst = check_strict(O, D, ref, bound, name=f"{fmt} x {fmt} shapes")
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()


# A larger grid (33 x 9 = 297 output tiles, more than one wave of workgroups) with a ragged
# K tail after the full K tiles, checked element by element on one tile row (rows 256..511).
LARGE_SHAPE = (8448, 2304, 2112)


@pytest.mark.parametrize("fmt,neg_a,accum", [("e4m3", 0, 1), ("e2m1", 1, 0), ("e2m1", 0, 1), ("e5m2", 1, 1)])
def test_block_scale_large_grid_vs_oracle(O, fmt, neg_a, accum):
    M, N, K = LARGE_SHAPE
    g = mx_case(fmt, 77, M, N, K)
    d0 = np.random.default_rng(5).standard_normal((M, N)).astype(np.float32)
    say("mx large", fmt, M, N, K, neg_a, accum)
    D = run_mx(M, N, K, fmt, g, d0 if accum else None, neg_a, 0, accum)
    ref, bound = O.gemm_block_scale(M, N, K, fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], fmt, g["B"], g["ldb"],
                                    g["SFB"], g["ld_sfb"], d0, N, neg_a, 0, accum, 256, 512)
    nb, worst = check_strict(O, D[256:512], ref, bound, name=f"{fmt} x {fmt} 8448x2304x2112 rows 256..511")
    assert nb == 0, worst
    assert np.isfinite(D[:, :N]).all()


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_block_scale_e5m2_vs_oracle(O, a_fmt, b_fmt):
    """E5M2 operands, alone and paired with E4M3 (the MFMA takes a format code per operand)."""
    for i, (M, N, K) in enumerate([(9, 17, 64), (300, 260, 288), (130, 513, 512), (64, 96, 1056), (256, 256, 128)]):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        g = mx_case(a_fmt, 50 + i, M, N, K, ld_pad=64 if i % 3 == 2 else 0, b_fmt=b_fmt)
        d0 = np.random.default_rng(i).standard_normal((M, N)).astype(np.float32)
        say("mx e5m2", a_fmt, b_fmt, M, N, K, neg_a, neg_b, accum)
        D = run_mx(M, N, K, a_fmt, g, d0 if accum else None, neg_a, neg_b, accum, b_fmt=b_fmt)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"],
                                        g["ldb"], g["SFB"], g["ld_sfb"], d0, N, neg_a, neg_b, accum)
        nb, worst = check_strict(O, D, ref, bound, name=f"{a_fmt} x {b_fmt} shapes")
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()


def test_block_scale_e5m2_infinities(O):
    """An E5M2 infinity in row 3 of A makes row 3 of D infinite with the sign of each product
    (every B element of that K column is a nonzero finite value), as in the oracle."""
    M, N, K = 8, 24, 64
    g = mx_case("e5m2", 61, M, N, K)
    A = g["A"].reshape(M, -1)
    A[3, 5] = 0x7C                                           # +inf
    B = g["B"].reshape(N, -1)
    B[:, 5] = np.where((B[:, 5] & 0x7F) == 0, 0x3C, B[:, 5])  # no zero (or -0) in column 5
    D = run_mx(M, N, K, "e5m2", g)
    ref, _ = O.gemm_block_scale(M, N, K, "e5m2", g["A"], g["lda"], g["SFA"], g["ld_sfa"], "e5m2", g["B"], g["ldb"],
                                g["SFB"], g["ld_sfb"])
    assert np.isinf(ref[3]).all()
    assert np.array_equal(D[3, :N], ref[3].astype(np.float32))
    assert np.isfinite(np.delete(D[:, :N], 3, 0)).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_block_scale_exact_sums_bit_exact(O, fmt):
    # narrow scales and small codes: every partial sum is exact in float32
    for M, N, K in [(256, 256, 128), (300, 200, 256)]:
        g = mx_case(fmt, 3, M, N, K, exp_range=2)
        if fmt == "e4m3":   # codes of +-{0, 0.5, 1, 1.5, 2}
            pick = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0xB0, 0xB8, 0xBC, 0xC0], np.uint8)
            rng = np.random.default_rng(1)
            g["A"] = pick[rng.integers(0, 9, g["A"].shape)]
            g["B"] = pick[rng.integers(0, 9, g["B"].shape)]
        say("mx exact", fmt, M, N, K)
        D = run_mx(M, N, K, fmt, g)
        ref, _ = O.gemm_block_scale(M, N, K, fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], fmt, g["B"], g["ldb"],
                                    g["SFB"], g["ld_sfb"])
        assert np.array_equal(D[:, :N], ref.astype(np.float32))


# Scale codes bounding the range in which every scaled 8-bit element is exact in bf16, its
# subnormals included (the exact-products route forms element * 2^(code - 127) in bf16).
SCALE_EDGES = {"e4m3": (3, 246), "e5m2": (10, 239)}


@pytest.mark.parametrize("a_fmt,b_fmt", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2")])
def test_block_scale_scale_range_edges(O, a_fmt, b_fmt):
    """Every A block at the top scale code of its format and every B block at the bottom one,
    then the reverse: the largest and the smallest (subnormal) scaled elements the route
    claims to form exactly, with products inside float32's range. Strict bound against the
    oracle, ragged K included."""
    for i, (M, N, K) in enumerate([(300, 260, 288), (256, 256, 1056)]):
        for top_a in (True, False):
            g = mx_case(a_fmt, 90 + i, M, N, K, b_fmt=b_fmt)
            (alo, ahi), (blo, bhi) = SCALE_EDGES[a_fmt], SCALE_EDGES[b_fmt]
            g["SFA"][:] = ahi if top_a else alo
            g["SFB"][:] = blo if top_a else bhi
            say("mx scale edges", a_fmt, b_fmt, M, N, K, "A top" if top_a else "B top")
            D = run_mx(M, N, K, a_fmt, g, b_fmt=b_fmt)
            ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"],
                                            g["ldb"], g["SFB"], g["ld_sfb"])
            assert np.isfinite(ref).all() and (bound > 0).any()
            nb, worst = check_strict(O, D, ref, bound, name=f"{a_fmt} x {b_fmt} scale-range edges")
            assert nb == 0, (M, N, K, top_a, worst)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_block_scale_nan_scale_poisons_row(O, fmt):
    M, N, K = 64, 64, 128
    g = mx_case(fmt, 4, M, N, K)
    g["SFA"][5, 2] = 255
    say("mx nan scale", fmt)
    D = run_mx(M, N, K, fmt, g)
    assert np.isnan(D[5, :N]).all()
    assert np.isfinite(np.delete(D[:, :N], 5, 0)).all()


def test_mxfp8_full_size_sampled(O):
    """The MXFP8 workload (8192 x 8192 x 16384, E4M3 codes uniform over the finite values,
    scales 127 +- 4): 1000 sampled outputs within the stated bound, with no allowance for the
    scaled fp8 MFMA's block window (the call sums exact products with the bf16 MFMA)."""
    g = W.mxfp8()
    M, N, K = g["M"], g["N"], g["K"]
    say("mxfp8 full", M, N, K)
    D = run_mx(M, N, K, "e4m3", g)
    pm, pn = W.sample_points(M, N, 1000)
    ref, bound = O.gemm_block_scale_points(M, N, K, "e4m3", g["A"], K, g["SFA"], K // 32, "e4m3", g["B"], K,
                                           g["SFB"], K // 32, None, 0, 0, 0, 0, pm, pn)
    nb, worst = check_strict(O, D, ref, bound, pm, pn, name="mxfp8 8192x8192x16384 (1000 points)")
    assert nb == 0, worst
    assert np.isfinite(D[:, :N]).all()


def test_mxfp4_full_size_sampled(O):
    g = W.mxfp4()
    M, N, K = g["M"], g["N"], g["K"]
    say("mxfp4 full", M, N, K)
    D = run_mx(M, N, K, "e2m1", g, neg_a=1)
    pm, pn = W.sample_points(M, N, 1000)
    ref, bound = O.gemm_block_scale_points(M, N, K, "e2m1", g["A"], K, g["SFA"], K // 32, "e2m1", g["B"], K,
                                           g["SFB"], K // 32, None, 0, 1, 0, 0, pm, pn)
    nb, worst = check_strict(O, D, ref, bound, pm, pn, name="mxfp4 16384x8192x8192 (1000 points)")
    assert nb == 0, worst
    assert np.isfinite(D[:, :N]).all()


def _window_pair(O, run, small_a, small_b):
    """One 32-element block with products 256 * 256 = 2^16 and small_a * small_b (E4M3 codes)."""
    A = np.zeros((1, 32), np.uint8)
    B = np.zeros((1, 32), np.uint8)
    A[0, 0] = B[0, 0] = 0x78          # 256 * 256 = 2^16
    A[0, 1], B[0, 1] = small_a, small_b
    sf = np.full((1, 4), 127, np.uint8)
    g = {"A": A, "B": B, "SFA": sf, "SFB": sf, "lda": 32, "ldb": 32, "ld_sfa": 4, "ld_sfb": 4}
    D = run(1, 1, 32, "e4m3", g)
    ref, _ = O.gemm_block_scale(1, 1, 32, "e4m3", A, 32, sf, 4, "e4m3", B, 32, sf, 4)
    return float(D[0, 0]), float(ref[0, 0])


@pytest.mark.parametrize("fmt,M,N,K", [("e4m3", 1, 257, 131072), ("e2m1", 257, 1, 131104), ("e4m3", 2, 3, 262144)])
def test_block_scale_long_k_thin(O, fmt, M, N, K):
    """One row or column of output with 4096 to 8192 scale blocks per row (a ragged K tail for
    E2M1): the exact-products route and the scaled MFMA over the longest K the tests run."""
    g = mx_case(fmt, 31, M, N, K)
    say("mx long K thin", fmt, M, N, K)
    D = run_mx(M, N, K, fmt, g)
    ref, bound = O.gemm_block_scale(M, N, K, fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], fmt, g["B"], g["ldb"],
                                    g["SFB"], g["ld_sfb"])
    nb, worst = check_strict(O, D, ref, bound, name=f"{fmt} x {fmt} long K, one row or column")
    assert nb == 0, worst
    assert np.isnan(D[:, N:]).all()


def test_e4m3_block_window_characterization(O):
    """The device fact behind the two routes: inside one 32-element scale block the scaled fp8
    MFMA (the fast-accumulation call) keeps a product 2^-13 below the block's largest product
    and drops one 2^-14 below (2^16 + 2^3 is exact, 2^16 + 2^2 returns 2^16); the plain call
    keeps products down to 2^-24 of the largest (2^16 + 2^2 and 2^16 + 2^-2 exact), smaller
    ones costing at most that much."""
    say("e4m3 window")
    got, ref = _window_pair(O, run_mx_fast, 0x48, 0x40)     # 4 * 2 = 2^3 -> kept
    assert got == ref == 65536.0 + 8.0
    got, ref = _window_pair(O, run_mx_fast, 0x40, 0x40)     # 2 * 2 = 2^2 -> dropped
    assert ref == 65536.0 + 4.0 and got == 65536.0
    for small in (0x40, 0x30):                               # 2^2, 2^-2 (0.5^2): kept exactly
        got, ref = _window_pair(O, run_mx, small, small)
        assert got == ref, (small, got, ref)
    for small in (0x08, 0x01):                               # 2^-12, 2^-18: below the bf16 MFMA's
        got, ref = _window_pair(O, run_mx, small, small)     # 2^-24 window, within the bound
        assert abs(got - ref) <= np.ldexp(65536.0, -24), (small, got, ref)


def test_bf16_mfma_accumulation_characterization(O):
    """The device fact the exact-products route rests on, through the dense bf16 GEMM: one
    32x32x16 bf16 MFMA keeps product bits down to 2^-24 of its largest term (1 + 2^-20 and
    1 + 2^-12 + ... + 2^-16 are exact) and drops terms far below it (2^30 + 1 - 2^30 gives 0);
    products below the window therefore cost at most about 2^-24 of the instruction's
    largest term each."""
    def one(vals):
        a = np.zeros((1, 16), np.float32)
        a[0, :len(vals)] = vals
        A = W.to_half_bits(a, "bf16")
        B = W.to_half_bits(np.ones((1, 16), np.float32), "bf16")
        return float(run_dense(1, 1, 16, "bf16", A, 16, "k", B, 16, "k")[0, 0])
    say("bf16 mfma window")
    assert one([1.0, 2.0 ** -20]) == 1.0 + 2.0 ** -20
    assert one([1.0, 2.0 ** -12, 2.0 ** -13, 2.0 ** -14, 2.0 ** -15, 2.0 ** -16]) == \
        1.0 + 2.0 ** -12 + 2.0 ** -13 + 2.0 ** -14 + 2.0 ** -15 + 2.0 ** -16
    assert one([2.0 ** 16, 2.0 ** 2]) == 65540.0
    assert one([2.0 ** 30, 1.0, -2.0 ** 30]) == 0.0


def run_mx_fast(M, N, K, fmt, g, D0=None, neg_a=0, neg_b=0, accum=0, b_fmt=None, ew=None):
    ldd = (N + 3) // 4 * 4
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    bsm.bsm_gemm_block_scale_fastacc(M, N, K, fmt, dev(g["A"]), g["lda"], dev(g["SFA"]), g["ld_sfa"], b_fmt or fmt,
                                     dev(g["B"]), g["ldb"], dev(g["SFB"]), g["ld_sfb"], dD, ldd, neg_a, neg_b, accum,
                                     ew=ew)
    return dD.cpu().numpy()


@pytest.mark.parametrize("a_fmt,b_fmt", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e2m1"), ("e3m2", "e3m2")])
def test_fastacc_within_window(O, a_fmt, b_fmt):
    """The fast-accumulation call on pairings with wide product ranges: within the stated
    bound plus the scaled MFMA's block-window allowance, over ragged shapes, negation and
    accumulation."""
    for i, (M, N, K) in enumerate([(9, 17, 64), (300, 260, 288), (130, 513, 512), (256, 256, 1056)]):
        neg_a, accum = i & 1, (i >> 1) & 1
        g = pair_case(a_fmt, b_fmt, 90 + i, M, N, K, ld_pad=64 if i == 2 else 0)
        d0 = np.random.default_rng(i).standard_normal((M, N)).astype(np.float32)
        say("mx fastacc", a_fmt, b_fmt, M, N, K, neg_a, accum)
        D = run_mx_fast(M, N, K, a_fmt, g, d0 if accum else None, neg_a, 0, accum, b_fmt=b_fmt)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"],
                                        g["ldb"], g["SFB"], g["ld_sfb"], d0, N, neg_a, 0, accum)
        nb, worst = check_window(O, g, a_fmt, b_fmt, K, D, ref, bound)
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()


@pytest.mark.parametrize("a_fmt,b_fmt", [("e2m1", "e2m1"), ("e2m3", "e2m3"), ("e2m1", "e3m2")])
def test_fastacc_equals_plain_call_for_exact_pairs(O, a_fmt, b_fmt):
    """For pairings whose products lie on the scaled MFMA's grid both calls run the same kernel:
    bit-identical results."""
    M, N, K = 300, 260, 1056
    g = pair_case(a_fmt, b_fmt, 95, M, N, K)
    say("mx fastacc vs plain", a_fmt, b_fmt)
    D1 = run_mx_fast(M, N, K, a_fmt, g, b_fmt=b_fmt)
    D2 = run_mx(M, N, K, a_fmt, g, b_fmt=b_fmt)
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32))


def test_mxfp8_fastacc_full_size_margin(O):
    """The MXFP8 workload through the fast-accumulation call: within the window allowance; the
    measured margin against the stated bound is recorded (it exceeds 1e-5 on this data, which
    is why the plain call takes the exact-products route)."""
    g = W.mxfp8()
    M, N, K = g["M"], g["N"], g["K"]
    say("mxfp8 fastacc full", M, N, K)
    D = run_mx_fast(M, N, K, "e4m3", g)
    pm, pn = W.sample_points(M, N, 300)
    ref, bound = O.gemm_block_scale_points(M, N, K, "e4m3", g["A"], K, g["SFA"], K // 32, "e4m3", g["B"], K,
                                           g["SFB"], K // 32, None, 0, 0, 0, 0, pm, pn)
    nb, worst = check_window(O, g, "e4m3", "e4m3", K, D, ref, bound, pm, pn)
    note("mxfp8 8192x8192x16384 fast accumulation (300 points)", worst)
    assert nb == 0, worst
