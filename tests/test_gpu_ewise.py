"""GPU parity: GEMMs with the fused silu_affine scalar epilogue (bsm_gemm_ewise,
bsm_gemm_block_scale_ewise) against the oracle's fp64 GEMM followed by its fp64 silu_affine.

Tolerance, derived from the arithmetic ("Explicit CUDA tile patterns", Scalar compositions:
f(x) = y * scale + bias, y = x / (1 + exp(-x)), typed float32):
  the kernel applies f in float32 to its float32 GEMM value x_d, which lies within T_x of the
  exact x (T_x: the plain GEMM's tolerance at that element). silu is 1.0999-Lipschitz (its
  derivative peaks near x = 2.4), so exact f moves by at most 1.1 |scale| T_x. Evaluating f
  in float32 adds: exp(-x) within 2 ulp (2^-22), 1 + e rounded (2^-24), the reciprocal
  within 1 ulp (2^-23) and the product rounded (2^-24), so |y| is off by at most 2^-21
  relatively; then y * scale + bias rounds once (2^-24 |f|). Allowed, with a factor 2
  margin on the rounding terms:
    |D - f(ref)| <= 1.1 |scale| T_x + 2^-20 |scale| |silu(ref)| + 2^-23 |f(ref)| + 2^-112 (1 + |scale|),
  the last term covering float32 results that underflow (|y| < |x| 2^-126, |x| < 104, once
  1 + exp(-x) passes 2^126).
"""
import numpy as np
import pytest

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_f32, say
from test_gpu_gemm import (TOL_DENSE, TOL_MX, dense_case, mx_case)

pytestmark = pytest.mark.gpu

# (scale, bias): the pages' example call (2, 1), a negative scale and a zero bias
PARAMS = [(2.0, 1.0), (-0.75, 0.5), (3.0, 0.0)]


def ewise_tol(O, ref, t_x, scale, bias):
    silu = O.ewise_silu_affine(ref, 1.0, 0.0)
    f = O.ewise_silu_affine(ref, scale, bias)
    tol = (1.1 * abs(scale) * t_x + np.ldexp(abs(scale) * np.abs(silu), -20) + np.ldexp(np.abs(f), -23)
           + np.ldexp(1.0 + abs(scale), -112))
    return f, tol


def compare(D, f, tol):
    """Number of elements outside tol (NaN must meet NaN), and the worst err / tol."""
    d = D.astype(np.float64)
    nan_ok = np.isnan(d) & np.isnan(f)
    with np.errstate(invalid="ignore"):
        err = np.abs(d - f)
        same_inf = np.isinf(d) & (d == f)
        ok = (err <= tol) | nan_ok | same_inf
        worst = float(np.nanmax(np.where(ok & ~nan_ok & ~same_inf, err / np.maximum(tol, 1e-300), 0.0)))
    return int((~ok).sum()), worst


def run_dense_ew(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, ew, D0=None, neg_a=0, neg_b=0, accum=0):
    ldd = (N + 3) // 4 * 4
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    bsm.bsm_gemm_ewise(M, N, K, dt, dev(A), lda, amaj, dev(B), ldb, bmaj, dD, ldd, neg_a, neg_b, accum, ew=ew)
    return dD.cpu().numpy()


def run_mx_ew(M, N, K, a_fmt, b_fmt, g, ew, D0=None, neg_a=0, neg_b=0, accum=0):
    ldd = (N + 3) // 4 * 4
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    bsm.bsm_gemm_block_scale_ewise(M, N, K, a_fmt, dev(g["A"]), g["lda"], dev(g["SFA"]), g["ld_sfa"], b_fmt,
                                   dev(g["B"]), g["ldb"], dev(g["SFB"]), g["ld_sfb"], dD, ldd, neg_a, neg_b, accum,
                                   ew=ew)
    return dD.cpu().numpy()


# several 256 x 256 workgroup tiles, ragged edges in M, N and K, and one-element cases
DENSE_SHAPES = [(1, 1, 1), (17, 33, 9), (255, 257, 130), (300, 520, 200), (513, 130, 64), (96, 272, 1000),
                (512, 512, 128)]


@pytest.mark.parametrize("dt,amaj,bmaj", [("bf16", "k", "n"), ("f16", "m", "k"), ("bf16", "k", "k")])
def test_dense_ewise_vs_oracle(O, dt, amaj, bmaj):
    rng = np.random.default_rng([7, ord(dt[0]), ord(amaj), ord(bmaj)])
    for i, (M, N, K) in enumerate(DENSE_SHAPES):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        scale, bias = PARAMS[i % len(PARAMS)]
        A, lda, B, ldb = dense_case(rng, M, N, K, dt, amaj, bmaj)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        say("dense ewise", dt, amaj, bmaj, M, N, K, neg_a, neg_b, accum, scale, bias)
        D = run_dense_ew(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, bsm.ewise_desc("silu_affine", scale, bias),
                         d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = O.gemm(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, d0, N, neg_a, neg_b, accum)
        f, tol = ewise_tol(O, ref, TOL_DENSE * bound + np.ldexp(np.abs(ref), -24), scale, bias)
        nb, worst = compare(D[:, :N], f, tol)
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()   # padding columns are never written


MX_CASES = [("e4m3", "e4m3"), ("e2m1", "e2m1"), ("e4m3", "e5m2")]


@pytest.mark.parametrize("a_fmt,b_fmt", MX_CASES)
def test_block_scale_ewise_vs_oracle(O, a_fmt, b_fmt):
    for i, (M, N, K) in enumerate([(9, 17, 64), (300, 260, 288), (130, 513, 512), (256, 256, 128),
                                   (64, 96, 1056)]):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        scale, bias = PARAMS[i % len(PARAMS)]
        g = mx_case(a_fmt, 90 + i, M, N, K, ld_pad=64 if i == 2 else 0, b_fmt=b_fmt)
        d0 = np.random.default_rng(i).standard_normal((M, N)).astype(np.float32)
        say("mx ewise", a_fmt, b_fmt, M, N, K, neg_a, neg_b, accum, scale, bias)
        D = run_mx_ew(M, N, K, a_fmt, b_fmt, g, bsm.ewise_desc("silu_affine", scale, bias), d0 if accum else None,
                      neg_a, neg_b, accum)
        ref, bound = O.gemm_block_scale(M, N, K, a_fmt, g["A"], g["lda"], g["SFA"], g["ld_sfa"], b_fmt, g["B"],
                                        g["ldb"], g["SFB"], g["ld_sfb"], d0, N, neg_a, neg_b, accum)
        t_x = TOL_MX * bound + np.ldexp(np.abs(ref), -24)
        f, tol = ewise_tol(O, ref, t_x, scale, bias)
        nb, worst = compare(D[:, :N], f, tol)
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()


def test_ewise_exact_sums_tight(O):
    """Where every partial sum is exact in float32 the kernel's x equals the oracle's, so only
    the float32 evaluation of f remains: T_x = 0. Magnitudes up to about 2^7 reach the regions
    where silu saturates (y = x) and where exp(-x) overflows (y = -0, f = bias)."""
    rng = np.random.default_rng(11)
    M, N, K = 300, 260, 64
    for amp in (0.25, 4.0, 64.0):
        a = (rng.integers(-4, 5, (M, K)) * amp / 4).astype(np.float32)
        b = (rng.integers(-4, 5, (N, K)) / 4).astype(np.float32)
        A, B = W.to_half_bits(a, "bf16"), W.to_half_bits(b, "bf16")
        for scale, bias in PARAMS:
            say("ewise exact", amp, scale, bias)
            D = run_dense_ew(M, N, K, "bf16", A, K, "k", B, K, "k", bsm.ewise_desc("silu_affine", scale, bias))
            ref, _ = O.gemm(M, N, K, "bf16", A, K, "k", B, K, "k")
            f, tol = ewise_tol(O, ref, 0.0, scale, bias)
            nb, worst = compare(D[:, :N], f, tol)
            assert nb == 0, (amp, scale, bias, worst)
    assert (np.abs(ref) > 100).any()   # the last case reaches |x| > 100


def test_ewise_none_matches_plain_call():
    """op NONE through the epilogue entry points is bit-identical to the plain calls."""
    rng = np.random.default_rng(12)
    M, N, K = 300, 260, 200
    A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", "k", "n")
    d0 = rng.standard_normal((M, N)).astype(np.float32)
    say("ewise none dense")
    ldd = (N + 3) // 4 * 4
    outs = []
    for use_ew in (0, 1):
        d = np.full((M, ldd), np.nan, np.float32)
        d[:, :N] = d0
        dD = dev_f32(d)
        args = (M, N, K, "bf16", dev(A), lda, "k", dev(B), ldb, "n", dD, ldd, 1, 0, 1)
        if use_ew:
            bsm.bsm_gemm_ewise(*args, ew=bsm.ewise_desc("none", 5.0, 7.0))
        else:
            bsm.bsm_gemm(*args)
        outs.append(dD.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    g = mx_case("e2m1", 13, 130, 513, 256)
    say("ewise none mx")
    outs = []
    for use_ew in (0, 1):
        dD = dev_f32(np.zeros((130, 516), np.float32))
        args = (130, 513, 256, "e2m1", dev(g["A"]), g["lda"], dev(g["SFA"]), g["ld_sfa"], "e2m1", dev(g["B"]),
                g["ldb"], dev(g["SFB"]), g["ld_sfb"], dD, 516, 0, 1, 0)
        if use_ew:
            bsm.bsm_gemm_block_scale_ewise(*args, ew=bsm.ewise_desc("none"))
        else:
            bsm.bsm_gemm_block_scale(*args)
        outs.append(dD.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_ewise_k_zero(O):
    """K = 0: the sum is empty, D = f(accum ? D : 0)."""
    M, N = 37, 300
    z8 = np.zeros((M, 8), np.uint16)
    for scale, bias in PARAMS:
        ew = bsm.ewise_desc("silu_affine", scale, bias)
        say("ewise K = 0", scale, bias)
        D = run_dense_ew(M, N, 0, "bf16", z8, 8, "k", np.zeros((N, 8), np.uint16), 8, "k", ew)
        assert (D[:, :N] == np.float32(bias)).all()    # silu(0) = 0 exactly
        d0 = np.random.default_rng(14).standard_normal((M, N)).astype(np.float32) * 8
        D = run_dense_ew(M, N, 0, "bf16", z8, 8, "k", np.zeros((N, 8), np.uint16), 8, "k", ew, d0, accum=1)
        f, tol = ewise_tol(O, d0.astype(np.float64), 0.0, scale, bias)
        assert compare(D[:, :N], f, tol)[0] == 0
        g = {"A": np.zeros((M, 16), np.uint8), "B": np.zeros((N, 16), np.uint8), "lda": 32, "ldb": 32,
             "SFA": np.zeros((M, 4), np.uint8), "SFB": np.zeros((N, 4), np.uint8), "ld_sfa": 4, "ld_sfb": 4}
        D = run_mx_ew(M, N, 0, "e2m1", "e2m1", g, ew, d0, accum=1)
        assert compare(D[:, :N], f, tol)[0] == 0


def test_ewise_infinities(O):
    """E5M2 infinities reach the epilogue: f(+inf) = +inf * scale + bias, f(-inf) = -inf / inf
    = NaN, in the kernel as in the oracle."""
    M, N, K = 8, 24, 64
    g = mx_case("e5m2", 61, M, N, K)
    A = g["A"].reshape(M, -1)
    A[3, 5] = 0x7C                                           # +inf
    B = g["B"].reshape(N, -1)
    B[:, 5] = np.where((B[:, 5] & 0x7F) == 0, 0x3C, B[:, 5])  # no zero (or -0) in column 5
    say("ewise infinities")
    D = run_mx_ew(M, N, K, "e5m2", "e5m2", g, bsm.ewise_desc("silu_affine", 2.0, 1.0))
    ref, _ = O.gemm_block_scale(M, N, K, "e5m2", g["A"], g["lda"], g["SFA"], g["ld_sfa"], "e5m2", g["B"], g["ldb"],
                                g["SFB"], g["ld_sfb"])
    f = O.ewise_silu_affine(ref, 2.0, 1.0)
    assert np.isinf(f[3]).any() and np.isnan(f[3]).any()
    assert np.array_equal(np.isnan(D[3, :N]), np.isnan(f[3]))
    assert np.array_equal(D[3, :N][np.isinf(f[3])], f[3][np.isinf(f[3])].astype(np.float32))


def test_gemm_bf16_8192_ewise_sampled(O):
    """The 8192^3 bf16 workload (A K-major, B MN-major, accumulating onto D0) with the pages'
    silu_affine(scale 2, bias 1) epilogue, as timed: sampled outputs against the oracle."""
    w = W.gemm_bf16()
    M, N, K = w["M"], w["N"], w["K"]
    say("gemm bf16 8192 ewise")
    dD = dev_f32(w["D0"])
    bsm.bsm_gemm_ewise(M, N, K, "bf16", dev(w["A"]), K, "k", dev(w["B"]), N, "n", dD, N, 0, 0, 1,
                       ew=bsm.ewise_desc("silu_affine", 2.0, 1.0))
    D = dD.cpu().numpy()
    pm, pn = W.sample_points(M, N, 2000)
    ref, bound = O.gemm_points(M, N, K, "bf16", w["A"], K, "k", w["B"], N, "n", w["D0"], N, 0, 0, 1, pm, pn)
    f, tol = ewise_tol(O, ref, TOL_DENSE * bound + np.ldexp(np.abs(ref), -24), 2.0, 1.0)
    nb, worst = compare(D[pm, pn], f, tol)
    assert nb == 0, worst
    assert np.isfinite(D).all()
