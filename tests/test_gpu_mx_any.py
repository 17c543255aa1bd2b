"""GPU parity: block-scaled GEMM over the other pairings of the f8f6f4 formats (the 6-bit
E2M3 / E3M2 and operands of different widths, run by the general kernel) against the oracle.

Tolerance: the stated bound, 1e-5 * sum|ab| + half an ulp of the float32 result
(mx_check.check_strict), for every pairing. Pairings whose products all lie on the scaled
MFMA's grid sum exactly there (checked bit for bit by the exact-sum cases); the others run the
exact-products route.
"""
import numpy as np
import pytest
import torch

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_f32, say
from mx_check import TOL_MX, check_strict, pair_case

pytestmark = pytest.mark.gpu

BITS = W.BITS
PAIRS = [("e4m3", "e2m1"), ("e2m1", "e4m3"), ("e5m2", "e2m1"), ("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"),
         ("e2m3", "e4m3"), ("e3m2", "e2m1"), ("e2m1", "e2m3"), ("e5m2", "e3m2")]
case = pair_case


def run(g, M, N, K, a_fmt, b_fmt, D0=None, neg_a=0, neg_b=0, accum=0, ew=None):
    ldd = (N + 3) // 4 * 4
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    args = (M, N, K, a_fmt, dev(g["A"]), g["lda"], dev(g["SFA"]), g["ld_sfa"], b_fmt, dev(g["B"]), g["ldb"],
            dev(g["SFB"]), g["ld_sfb"], dD, ldd, neg_a, neg_b, accum)
    if ew is None:
        bsm.bsm_gemm_block_scale(*args)
    else:
        bsm.bsm_gemm_block_scale_ewise(*args, ew=ew)
    return dD.cpu().numpy()


def check(O, g, a_fmt, b_fmt, K, D, ref, bound, pm=None, pn=None, name=None):
    return check_strict(O, D, ref, bound, pm, pn, name=name)


SHAPES = [(1, 1, 32), (9, 17, 64), (300, 260, 288), (130, 513, 512), (256, 256, 128), (64, 96, 1056), (33, 40, 96)]


@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
def test_mx_any_pair_vs_oracle(O, a_fmt, b_fmt):
    for i, (M, N, K) in enumerate(SHAPES):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        g = case(a_fmt, b_fmt, 70 + i, M, N, K, ld_pad=64 if i % 3 == 2 else 0)
        d0 = np.random.default_rng(i).standard_normal((M, N)).astype(np.float32)
        say("mx any", a_fmt, b_fmt, M, N, K, neg_a, neg_b, accum)
        D = run(g, M, N, K, a_fmt, b_fmt, d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"],
                                        g["ldb"], g["SFB"], g["ld_sfb"], d0, N, neg_a, neg_b, accum)
        nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, name=f"{a_fmt} x {b_fmt} shapes")
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()


@pytest.mark.parametrize("a_fmt,b_fmt", [("e2m3", "e2m3"), ("e2m1", "e2m3"), ("e2m3", "e2m1"), ("e2m1", "e3m2")])
def test_mx_any_exact_pairs_bit_exact(O, a_fmt, b_fmt):
    """Products of these pairs all lie on the scaled MFMA's grid and unit-range scales keep
    every partial sum exact in float32: the result must equal the oracle's bit for bit, also
    over K of several scale-ring groups (K = 1408: eleven K tiles, three groups)."""
    for M, N, K in [(256, 256, 128), (300, 200, 352), (264, 136, 1408)]:
        g = case(a_fmt, b_fmt, 5, M, N, K, exp_range=1)
        say("mx any exact", a_fmt, b_fmt, M, N, K)
        D = run(g, M, N, K, a_fmt, b_fmt)
        ref, _ = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"], g["ldb"],
                                    g["SFB"], g["ld_sfb"])
        assert np.array_equal(D[:, :N], ref.astype(np.float32))


@pytest.mark.parametrize("a_fmt,b_fmt", [("e2m3", "e3m2"), ("e4m3", "e2m1")])
def test_mx_any_nan_scale_poisons_row(O, a_fmt, b_fmt):
    M, N, K = 64, 64, 256
    g = case(a_fmt, b_fmt, 4, M, N, K)
    g["SFA"][5, 6] = 255
    say("mx any nan scale", a_fmt, b_fmt)
    D = run(g, M, N, K, a_fmt, b_fmt)
    assert np.isnan(D[5, :N]).all()
    assert np.isfinite(np.delete(D[:, :N], 5, 0)).all()


def test_mx_any_with_epilogue(O):
    M, N, K = 300, 260, 288
    g = case("e4m3", "e2m1", 9, M, N, K)
    say("mx any silu_affine")
    D = run(g, M, N, K, "e4m3", "e2m1", ew=bsm.ewise_desc("silu_affine", 2.0, 1.0))
    ref, bound = O.gemm_block_scale(M, N, K, "e4m3", g["A"], g["lda"], g["SFA"], g["ld_sfa"], "e2m1", g["B"],
                                    g["ldb"], g["SFB"], g["ld_sfb"])
    t_x = (TOL_MX * bound + np.ldexp(np.abs(ref), -24)).reshape(-1)
    f = O.ewise_silu_affine(ref, 2.0, 1.0).reshape(-1)
    silu = O.ewise_silu_affine(ref, 1.0, 0.0).reshape(-1)
    tol = 1.1 * 2.0 * t_x + np.ldexp(2.0 * np.abs(silu), -20) + np.ldexp(np.abs(f), -23) + np.ldexp(3.0, -112)
    assert (np.abs(D[:, :N].reshape(-1).astype(np.float64) - f) <= tol).all()


@pytest.mark.parametrize("a_fmt,b_fmt", [("e4m3", "e2m1"), ("e2m3", "e2m3")])
def test_mx_any_full_size_sampled(O, a_fmt, b_fmt):
    """The timed workloads (M = N = 8192, K = 16384): sampled outputs against the oracle."""
    M, N, K = 8192, 8192, 16384
    g = W.mx_pair(21 if a_fmt == "e4m3" else 22, M, N, K, a_fmt, b_fmt)
    say("mx any full", a_fmt, b_fmt, M, N, K)
    D = run(g, M, N, K, a_fmt, b_fmt)
    pm, pn = W.sample_points(M, N, 600)
    ref, bound = O.gemm_block_scale_points(M, N, K, a_fmt, g["A"], K, g["SFA"], K // 32, b_fmt, g["B"], K, g["SFB"],
                                           K // 32, None, 0, 0, 0, 0, pm, pn)
    nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, pm, pn, name=f"{a_fmt} x {b_fmt} 8192x8192x16384 (600 points)")
    assert nb == 0, worst
    assert np.isfinite(D[:, :N]).all()


@pytest.mark.parametrize("a_fmt,b_fmt", [("e2m3", "e2m3"), ("e4m3", "e2m3"), ("e2m1", "e3m2")])
def test_mx_any_scale_groups(O, a_fmt, b_fmt):
    """K tile counts around the scale ring's four-tile groups (5, 6, 7, 9 and 13 whole tiles,
    with and without a partial last tile): groups the last tile leaves partly unused, a last
    tile that ends its group, and both pipeline depths (three stages for 6-bit x 6-bit, two
    for 8-bit x 6-bit)."""
    for i, K in enumerate([640, 768, 896, 1184, 1664, 1696]):
        M, N = 300, 260
        accum = i & 1
        g = case(a_fmt, b_fmt, 130 + i, M, N, K, ld_pad=64 if i % 2 else 0)
        d0 = np.random.default_rng(40 + i).standard_normal((M, N)).astype(np.float32)
        say("mx any scale groups", a_fmt, b_fmt, M, N, K, accum)
        D = run(g, M, N, K, a_fmt, b_fmt, d0 if accum else None, 0, 0, accum)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"],
                                        g["ldb"], g["SFB"], g["ld_sfb"], d0, N, 0, 0, accum)
        nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, name=f"{a_fmt} x {b_fmt} scale groups")
        assert nb == 0, (K, worst)
