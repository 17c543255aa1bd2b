"""Pins of the oracle's dense and block-scaled GEMM.

Independent references: numpy float64 matmul on operands decoded by numpy/torch
(not by the oracle), the pages' 128x64x64 fp16 example (whose sums are exact),
closed forms (identity B, K = 1 outer product, scale doubling) and the sign /
accumulate invariants. Each would fail on a dropped term, a transposed operand, a
wrong major-order index, a wrong sign or a misplaced scale.
"""
import numpy as np
import pytest
import torch

from block_scaled_matrix_amd import workloads as W


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def half_vals(bits, dt):
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_pages_tcgen05_example_exact(O):
    """The example GEMM of "tcgen05.mma" (Example: four K16 issues): M = 128, N = K = 64, fp16
    operands on the quarter grid from seed 0, D = A B^T; against numpy float64."""
    ab, bb = W.quarter_grid_f16(0)
    a, b = ab.view(np.float16), bb.view(np.float16)
    ref, bound = O.gemm(128, 64, 64, "f16", ab, 64, "k", bb, 64, "k")
    exp = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.array_equal(ref, exp)
    assert np.array_equal(bound, np.abs(a.astype(np.float64)) @ np.abs(b.astype(np.float64)).T)
    # every product is a multiple of 1/16 and |sum| <= 64, so float32 holds it exactly
    assert np.array_equal(exp.astype(np.float32).astype(np.float64), exp)


SIZES = [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("amaj,bmaj", [("k", "k"), ("k", "n"), ("m", "k"), ("m", "n")])
def test_dense_vs_numpy_brute_force(O, dt, amaj, bmaj):
    rng = np.random.default_rng([ord(c) for c in dt + amaj + bmaj])
    for trial in range(12):
        M, N, K = (int(rng.choice(SIZES)) for _ in range(3))
        neg_a, neg_b, accum = (int(v) for v in rng.integers(0, 2, 3))
        a = W.to_half_bits(rng.standard_normal((M, K)).astype(np.float32), dt)
        b = W.to_half_bits(rng.standard_normal((N, K)).astype(np.float32), dt)
        A = a if amaj == "k" else np.ascontiguousarray(a.T)
        B = b if bmaj == "k" else np.ascontiguousarray(b.T)
        lda = K if amaj == "k" else M
        ldb = K if bmaj == "k" else N
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        ref, bound = O.gemm(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, d0, N, neg_a, neg_b, accum)
        av, bv = half_vals(a, dt), half_vals(b, dt)
        sig = (-1.0) ** (neg_a + neg_b)
        exp = (d0.astype(np.float64) if accum else 0.0) + sig * (av @ bv.T)
        np.testing.assert_allclose(ref, exp, rtol=0, atol=1e-12 * (1 + np.abs(av) @ np.abs(bv).T).max())
        np.testing.assert_allclose(bound, np.abs(av) @ np.abs(bv).T, rtol=1e-12)


def test_dense_closed_forms(O):
    rng = np.random.default_rng(1)
    M, K = 24, 16
    a = f16_bits(rng.standard_normal((M, K)))
    eye = f16_bits(np.eye(K))
    ref, _ = O.gemm(M, K, K, "f16", a, K, "k", eye, K, "k")
    assert np.array_equal(ref, a.view(np.float16).astype(np.float64))           # B = I -> A
    u, v = f16_bits(rng.standard_normal((M, 1))), f16_bits(rng.standard_normal((9, 1)))
    ref, _ = O.gemm(M, 9, 1, "f16", u, 1, "k", v, 1, "k")
    assert np.array_equal(ref, u.view(np.float16).astype(np.float64) @ v.view(np.float16).astype(np.float64).T)
    b = f16_bits(rng.standard_normal((13, K)))
    d0 = rng.standard_normal((M, 13)).astype(np.float32)
    base, _ = O.gemm(M, 13, K, "f16", a, K, "k", b, K, "k")
    na, _ = O.gemm(M, 13, K, "f16", a, K, "k", b, K, "k", neg_a=1)
    nab, _ = O.gemm(M, 13, K, "f16", a, K, "k", b, K, "k", neg_a=1, neg_b=1)
    assert np.array_equal(na, -base) and np.array_equal(nab, base)
    z = np.zeros_like(a)
    acc, bnd = O.gemm(M, 13, K, "f16", z, K, "k", b, K, "k", d0, 13, 0, 0, 1)
    assert np.array_equal(acc, d0.astype(np.float64)) and not bnd.any()
    ka, _ = O.gemm(M, 13, 0, "f16", a, K, "k", b, K, "k", d0, 13, 1, 0, 1)   # K = 0: D unchanged
    assert np.array_equal(ka, d0.astype(np.float64))


def test_dense_major_orders_agree(O):
    rng = np.random.default_rng(2)
    M, N, K = 19, 23, 29
    a = W.to_half_bits(rng.standard_normal((M, K)).astype(np.float32), "bf16")
    b = W.to_half_bits(rng.standard_normal((N, K)).astype(np.float32), "bf16")
    r_kk, _ = O.gemm(M, N, K, "bf16", a, K, "k", b, K, "k")
    r_mn, _ = O.gemm(M, N, K, "bf16", np.ascontiguousarray(a.T), M, "m", np.ascontiguousarray(b.T), N, "n")
    assert np.array_equal(r_kk, r_mn)
    # padded leading dimensions
    ap = np.zeros((M, 40), np.uint16)
    ap[:, :K] = a
    r_pad, _ = O.gemm(M, N, K, "bf16", ap, 40, "k", b, K, "k")
    assert np.array_equal(r_kk, r_pad)


def test_dense_points_match_full(O):
    g = W.gemm_bf16(seed=3, M=96, N=80, K=72)
    ref, bound = O.gemm(96, 80, 72, "bf16", g["A"], 72, "k", g["B"], 80, "n", g["D0"], 80, 0, 1, 1)
    pm, pn = W.sample_points(96, 80, 40)
    pr, pb = O.gemm_points(96, 80, 72, "bf16", g["A"], 72, "k", g["B"], 80, "n", g["D0"], 80, 0, 1, 1, pm, pn)
    assert np.array_equal(pr, ref[pm, pn]) and np.array_equal(pb, bound[pm, pn])


# ----------------------------------------------------------------------------- block scaled
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def mx_vals(raw, fmt, rows, K):
    """Decoded element values via torch (e4m3, e5m2) or the OCP table (e2m1), low nibble first."""
    if fmt in ("e4m3", "e5m2"):
        t = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
        return torch.from_numpy(raw.reshape(rows, K)).view(t).to(torch.float64).numpy()
    r = raw.reshape(rows, K // 2)
    out = np.empty((rows, K))
    out[:, 0::2] = E2M1[r & 15]
    out[:, 1::2] = E2M1[r >> 4]
    return out


def fp6_vals(raw, fmt, rows, K):
    """6-bit elements: codes extracted with numpy's unpackbits (little-endian bit string per
    row), values from the OCP table of the format (codes 0..31 positive, bit 5 the sign)."""
    bits = np.unpackbits(raw.reshape(rows, -1), axis=1, bitorder="little")[:, :6 * K].reshape(rows, K, 6)
    codes = (bits * (1 << np.arange(6))).sum(axis=2)
    if fmt == "e2m3":   # subnormals m/8; normals (1 + m/8) 2^(e-1)
        pos = [m / 8 for m in range(8)] + [(1 + m / 8) * 2.0 ** (e - 1) for e in range(1, 4) for m in range(8)]
    else:               # subnormals m/16; normals (1 + m/4) 2^(e-3)
        pos = [m / 16 for m in range(4)] + [(1 + m / 4) * 2.0 ** (e - 3) for e in range(1, 8) for m in range(4)]
    table = np.array(pos + [-v for v in pos])
    return table[codes]


def any_vals(raw, fmt, rows, K):
    return fp6_vals(raw, fmt, rows, K) if fmt in ("e2m3", "e3m2") else mx_vals(raw, fmt, rows, K)


def scaled(vals, sf):
    return vals * np.repeat(np.exp2(sf.astype(np.float64) - 127), 32, axis=1)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_block_scale_vs_numpy_brute_force(O, fmt):
    rng = np.random.default_rng(7 if fmt == "e4m3" else 8)
    for trial in range(10):
        M, N = int(rng.choice(SIZES)), int(rng.choice(SIZES))
        K = int(rng.choice([32, 64, 96, 160]))
        neg_a, neg_b, accum = (int(v) for v in rng.integers(0, 2, 3))
        g = (W.mxfp8 if fmt == "e4m3" else W.mxfp4)(seed=trial, M=M, N=N, K=K)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        ref, bound = O.gemm_block_scale(M, N, K, fmt, g["A"], K, g["SFA"], K // 32, fmt, g["B"], K, g["SFB"],
                                        K // 32, d0, N, neg_a, neg_b, accum)
        av = scaled(mx_vals(g["A"], fmt, M, K), g["SFA"])
        bv = scaled(mx_vals(g["B"], fmt, N, K), g["SFB"])
        exp = (d0.astype(np.float64) if accum else 0.0) + (-1.0) ** (neg_a + neg_b) * (av @ bv.T)
        np.testing.assert_allclose(ref, exp, rtol=0, atol=1e-12 * (1 + (np.abs(av) @ np.abs(bv).T).max()))
        np.testing.assert_allclose(bound, np.abs(av) @ np.abs(bv).T, rtol=1e-12)


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_block_scale_e5m2_vs_numpy_brute_force(O, a_fmt, b_fmt):
    """E5M2 operands, alone and mixed with E4M3 (8-bit operands of either kind pair up)."""
    rng = np.random.default_rng(17)
    for trial in range(6):
        M, N = int(rng.choice(SIZES)), int(rng.choice(SIZES))
        K = int(rng.choice([32, 64, 96, 160]))
        neg_a, neg_b, accum = (int(v) for v in rng.integers(0, 2, 3))
        g = W.mxfp8(seed=40 + trial, M=M, N=N, K=K, a_fmt=a_fmt, b_fmt=b_fmt)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], K, g["SFA"], K // 32, b_fmt, g["B"], K, g["SFB"],
                                        K // 32, d0, N, neg_a, neg_b, accum)
        av = scaled(mx_vals(g["A"], a_fmt, M, K), g["SFA"])
        bv = scaled(mx_vals(g["B"], b_fmt, N, K), g["SFB"])
        exp = (d0.astype(np.float64) if accum else 0.0) + (-1.0) ** (neg_a + neg_b) * (av @ bv.T)
        np.testing.assert_allclose(ref, exp, rtol=0, atol=1e-12 * (1 + (np.abs(av) @ np.abs(bv).T).max()))
        np.testing.assert_allclose(bound, np.abs(av) @ np.abs(bv).T, rtol=1e-12)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_block_scale_unit_scales_equal_dense_values(O, fmt):
    M, N, K = 9, 11, 64
    g = (W.mxfp8 if fmt == "e4m3" else W.mxfp4)(seed=3, M=M, N=N, K=K)
    one = np.full((M, K // 32), 127, np.uint8)
    oneb = np.full((N, K // 32), 127, np.uint8)
    ref, _ = O.gemm_block_scale(M, N, K, fmt, g["A"], K, one, 2, fmt, g["B"], K, oneb, 2)
    assert np.array_equal(ref, mx_vals(g["A"], fmt, M, K) @ mx_vals(g["B"], fmt, N, K).T)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_block_scale_row_doubling_and_nan_scale(O, fmt):
    M, N, K = 6, 5, 96
    g = (W.mxfp8 if fmt == "e4m3" else W.mxfp4)(seed=4, M=M, N=N, K=K)
    base, _ = O.gemm_block_scale(M, N, K, fmt, g["A"], K, g["SFA"], 3, fmt, g["B"], K, g["SFB"], 3)
    sfa = g["SFA"].copy()
    sfa[2] += 1
    dbl, _ = O.gemm_block_scale(M, N, K, fmt, g["A"], K, sfa, 3, fmt, g["B"], K, g["SFB"], 3)
    exp = base.copy()
    exp[2] *= 2
    assert np.array_equal(dbl, exp)
    # a NaN scale poisons exactly the products of its block: row 4 -> NaN, others unchanged
    sfa = g["SFA"].copy()
    sfa[4, 1] = 255
    nan, _ = O.gemm_block_scale(M, N, K, fmt, g["A"], K, sfa, 3, fmt, g["B"], K, g["SFB"], 3)
    assert np.isnan(nan[4]).all() and np.array_equal(np.delete(nan, 4, 0), np.delete(base, 4, 0))
    # the block size is 32: changing the scale of block 1 leaves k < 32 and k >= 64 alone
    a2 = g["A"].copy()
    sf1 = g["SFA"].copy()
    sf1[:, 1] = 127 - 60   # block 1 almost vanishes
    tiny, _ = O.gemm_block_scale(M, N, K, fmt, a2, K, sf1, 3, fmt, g["B"], K, g["SFB"], 3)
    av = scaled(mx_vals(g["A"], fmt, M, K), g["SFA"])
    bv = scaled(mx_vals(g["B"], fmt, N, K), g["SFB"])
    keep = np.r_[0:32, 64:96]
    np.testing.assert_allclose(tiny, av[:, keep] @ bv[:, keep].T, rtol=1e-12, atol=1e-12)


def test_block_scale_e2m1_nibble_placement(O):
    # element 1 of row 0 is the high nibble of byte 0; element 0 the low nibble
    A = np.zeros((1, 16), np.uint8)
    A[0, 0] = 0x20          # element1 = code 2 = 1.0, element0 = 0
    B = np.zeros((1, 16), np.uint8)
    B[0, 0] = 0x40          # element1 = code 4 = 2.0
    sf = np.full((1, 1), 127, np.uint8)
    ref, _ = O.gemm_block_scale(1, 1, 32, "e2m1", A, 32, sf, 1, "e2m1", B, 32, sf, 1)
    assert ref[0, 0] == 2.0
    B[0, 0] = 0x04          # now element0 = 2.0, element1 = 0 -> product vanishes
    ref, _ = O.gemm_block_scale(1, 1, 32, "e2m1", A, 32, sf, 1, "e2m1", B, 32, sf, 1)
    assert ref[0, 0] == 0.0


def test_block_scale_points_match_full(O):
    g = W.mxfp4(seed=5, M=64, N=48, K=128)
    ref, bound = O.gemm_block_scale(64, 48, 128, "e2m1", g["A"], 128, g["SFA"], 4, "e2m1", g["B"], 128, g["SFB"],
                                    4, None, 0, 1, 0, 0)
    pm, pn = W.sample_points(64, 48, 30)
    pr, pb = O.gemm_block_scale_points(64, 48, 128, "e2m1", g["A"], 128, g["SFA"], 4, "e2m1", g["B"], 128,
                                       g["SFB"], 4, None, 0, 1, 0, 0, pm, pn)
    assert np.array_equal(pr, ref[pm, pn]) and np.array_equal(pb, bound[pm, pn])


# ----------------------------------------------------------------------------- comparison (check_gemm)
def test_check_gemm_flags_planted_errors(O):
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((8, 8))
    bound = np.abs(ref) + 1.0
    D = ref.astype(np.float32)
    assert O.check_gemm(D, ref, bound, 2e-3)[0] == 0
    D2 = D.copy()
    D2[3, 4] += np.float32(3e-3 * bound[3, 4])
    nb, first, _ = O.check_gemm(D2, ref, bound, 2e-3)
    assert nb == 1 and first == 3 * 8 + 4
    D3 = D.copy()
    D3[0, 0] = np.nan
    assert O.check_gemm(D3, ref, bound, 2e-3)[0] == 1
    z = np.zeros((2, 2))
    assert O.check_gemm(np.array([[0, -0.0], [1e-30, 0]], np.float32), z, z, 2e-3)[0] == 1  # exact where bound 0


def test_check_gemm_infinities(O):
    """An infinite reference (an E5M2 infinity times a nonzero finite value) matches exactly the
    same infinity: +inf = +inf and -inf = -inf pass; the other sign, a finite value or NaN fail."""
    inf = np.inf
    ref = np.array([[inf, -inf, inf, -inf, inf, 1.0]])
    bound = np.array([[inf, inf, inf, inf, inf, 1.0]])
    D = np.array([[inf, -inf, inf, -inf, inf, 1.0]], np.float32)
    assert O.check_gemm(D, ref, bound, 1e-5)[0] == 0
    for j, wrong in [(0, -inf), (1, inf), (2, 3.0e38), (3, np.nan), (5, inf)]:
        D2 = D.copy()
        D2[0, j] = wrong
        nb, first, _ = O.check_gemm(D2, ref, bound, 1e-5)
        assert nb == 1 and first == j, (j, wrong)


PAIRS = [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e4m3", "e2m1"), ("e2m1", "e5m2"), ("e2m3", "e4m3"), ("e2m1", "e3m2"),
         ("e3m2", "e2m3")]


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
def test_block_scale_any_pair_vs_numpy_brute_force(O, a_fmt, b_fmt):
    """Every pairing of the block-scaled formats (the 6-bit ones and mixed widths), against
    numpy matmul of operands decoded independently (unpackbits and the OCP tables for the
    6-bit formats, torch for 8-bit, the OCP table for E2M1)."""
    rng = np.random.default_rng([19, len(a_fmt + b_fmt), ord(a_fmt[1]), ord(b_fmt[3])])
    for trial in range(5):
        M, N = int(rng.choice(SIZES)), int(rng.choice(SIZES))
        K = int(rng.choice([32, 64, 128, 192]))
        neg_a, neg_b, accum = (int(v) for v in rng.integers(0, 2, 3))
        g = W.mx_pair(60 + trial, M, N, K, a_fmt, b_fmt)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], K, g["SFA"], K // 32, b_fmt, g["B"], K, g["SFB"],
                                        K // 32, d0, N, neg_a, neg_b, accum)
        av = scaled(any_vals(g["A"], a_fmt, M, K), g["SFA"])
        bv = scaled(any_vals(g["B"], b_fmt, N, K), g["SFB"])
        exp = (d0.astype(np.float64) if accum else 0.0) + (-1.0) ** (neg_a + neg_b) * (av @ bv.T)
        np.testing.assert_allclose(ref, exp, rtol=0, atol=1e-12 * (1 + (np.abs(av) @ np.abs(bv).T).max()))
        np.testing.assert_allclose(bound, np.abs(av) @ np.abs(bv).T, rtol=1e-12)


def transpose_codes(raw, fmt, rows, K):
    """K-major packed codes (rows, K) -> MN-major packed codes (K, rows), by numpy: unpack the
    elements (bytes, nibbles low first, or 6-bit fields), transpose, repack."""
    bits = W.BITS[fmt]
    r = np.ascontiguousarray(raw).reshape(rows, -1)
    if bits == 8:
        return np.ascontiguousarray(r[:, :K].T)
    if bits == 4:
        codes = np.stack([r & 15, r >> 4], axis=2).reshape(rows, -1)[:, :K].T
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    bs = np.unpackbits(r, axis=1, bitorder="little")[:, :6 * K].reshape(rows, K, 6)
    codes = (bs * (1 << np.arange(6))).sum(axis=2).T
    return W.pack_fp6(np.ascontiguousarray(codes))


@pytest.mark.parametrize("a_fmt,b_fmt,amaj,bmaj", [("e4m3", "e4m3", "m", "k"), ("e2m1", "e2m1", "k", "n"),
                                                   ("e5m2", "e2m1", "m", "n"), ("e2m3", "e4m3", "m", "k")])
def test_block_scale_mn_major_vs_numpy(O, a_fmt, b_fmt, amaj, bmaj):
    """MN-major operands (K rows, M or N contiguous): the oracle on storage transposed by numpy
    against numpy matmul of the values decoded from the original K-major codes."""
    rng = np.random.default_rng(23)
    for trial in range(4):
        M, N = int(rng.choice(SIZES)) * 4, int(rng.choice(SIZES)) * 4     # whole bytes of packed elements
        K = int(rng.choice([32, 64, 96]))
        g = W.mx_pair(80 + trial, M, N, K, a_fmt, b_fmt)
        A = transpose_codes(g["A"], a_fmt, M, K) if amaj == "m" else g["A"]
        B = transpose_codes(g["B"], b_fmt, N, K) if bmaj == "n" else g["B"]
        lda, ldb = (M if amaj == "m" else K), (N if bmaj == "n" else K)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, A, lda, g["SFA"], K // 32, b_fmt, B, ldb, g["SFB"], K // 32,
                                        a_major=amaj, b_major=bmaj)
        av = scaled(any_vals(g["A"], a_fmt, M, K), g["SFA"])
        bv = scaled(any_vals(g["B"], b_fmt, N, K), g["SFB"])
        np.testing.assert_allclose(ref, av @ bv.T, rtol=0, atol=1e-12 * (1 + (np.abs(av) @ np.abs(bv).T).max()))
        np.testing.assert_allclose(bound, np.abs(av) @ np.abs(bv).T, rtol=1e-12)
