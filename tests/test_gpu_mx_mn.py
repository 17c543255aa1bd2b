"""GPU parity: block-scaled GEMM with MN-major operands (K rows, M or N contiguous;
bsm_gemm_block_scale_major) against the oracle on the same MN-major storage.

Tolerance as for the K-major pairs (test_gpu_mx_any): the stated bound, 1e-5 * sum|ab| +
half an ulp of the float32 result. MN-major and K-major operands of a pair the general kernel
runs in both orders go through the same MFMA sequence, so those results must also agree bit
for bit.
"""
import numpy as np
import pytest

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_f32, say
from test_gpu_gemm import pad_cols, pad_scales
from test_gpu_mx_any import check

pytestmark = pytest.mark.gpu

BITS = W.BITS


def ld_for(n, fmt, pad=0):
    """Smallest leading dimension >= n + pad whose rows are 16-byte aligned."""
    q = {8: 16, 6: 64, 4: 32}[BITS[fmt]]
    return (n + pad + q - 1) // q * q


def case(a_fmt, b_fmt, amaj, bmaj, seed, M, N, K, exp_range=4, pad=0):
    """W.mx_pair operands; g["A"] / g["B"] keep the K-major codes (the slack and the
    K-major comparison use them), g["As"] / g["Bs"] the storage passed to the call."""
    g = W.mx_pair(seed, M, N, K, a_fmt, b_fmt, exp_range)
    ldk_a, ldk_b = ld_for(K, a_fmt, pad), ld_for(K, b_fmt, pad)
    g["A"] = pad_cols(g["A"].reshape(M, -1), ldk_a * BITS[a_fmt] // 8)
    g["B"] = pad_cols(g["B"].reshape(N, -1), ldk_b * BITS[b_fmt] // 8)
    g["lda"], g["ldb"] = ldk_a, ldk_b
    if amaj == "m":
        g["lda_s"] = ld_for(M, a_fmt, pad)
        g["As"] = W.mn_major(g["A"], a_fmt, M, K, g["lda_s"], seed=seed + 1000)
    else:
        g["lda_s"], g["As"] = ldk_a, g["A"]
    if bmaj == "n":
        g["ldb_s"] = ld_for(N, b_fmt, pad)
        g["Bs"] = W.mn_major(g["B"], b_fmt, N, K, g["ldb_s"], seed=seed + 2000)
    else:
        g["ldb_s"], g["Bs"] = ldk_b, g["B"]
    ld_sf = (K // 32 + 3) // 4 * 4 + (4 if pad else 0)
    g["SFA"], g["SFB"] = pad_scales(g["SFA"], ld_sf), pad_scales(g["SFB"], ld_sf)
    g["ld_sfa"] = g["ld_sfb"] = ld_sf
    return g


def run(g, M, N, K, a_fmt, b_fmt, amaj, bmaj, D0=None, neg_a=0, neg_b=0, accum=0, ew=None):
    ldd = (N + 3) // 4 * 4
    d = np.full((M, ldd), np.nan, np.float32)
    if D0 is not None:
        d[:, :N] = D0
    dD = dev_f32(d)
    bsm.bsm_gemm_block_scale_major(M, N, K, a_fmt, dev(g["As"]), g["lda_s"], amaj, dev(g["SFA"]), g["ld_sfa"], b_fmt,
                                   dev(g["Bs"]), g["ldb_s"], bmaj, dev(g["SFB"]), g["ld_sfb"], dD, ldd, neg_a, neg_b,
                                   accum, ew=ew)
    return dD.cpu().numpy()


def oracle(O, g, M, N, K, a_fmt, b_fmt, amaj, bmaj, D0=None, neg_a=0, neg_b=0, accum=0):
    return O.gemm_block_scale(M, N, K, a_fmt, g["As"], g["lda_s"], g["SFA"], g["ld_sfa"], b_fmt, g["Bs"], g["ldb_s"],
                              g["SFB"], g["ld_sfb"], D0, N, neg_a, neg_b, accum, a_major=amaj, b_major=bmaj)


PAIRS = [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m1", "e2m1"), ("e4m3", "e2m1"), ("e2m1", "e5m2")]
MAJORS = [("m", "k"), ("k", "n"), ("m", "n")]
SHAPES = [(1, 1, 32), (9, 17, 64), (300, 260, 288), (130, 513, 512), (256, 256, 128), (64, 96, 1056), (33, 40, 96)]


@pytest.mark.parametrize("amaj,bmaj", MAJORS)
@pytest.mark.parametrize("a_fmt,b_fmt", PAIRS)
def test_mx_mn_vs_oracle(O, a_fmt, b_fmt, amaj, bmaj):
    for i, (M, N, K) in enumerate(SHAPES):
        neg_a, neg_b, accum = i & 1, (i >> 1) & 1, (i >> 2) & 1
        g = case(a_fmt, b_fmt, amaj, bmaj, 90 + i, M, N, K, pad=64 if i % 3 == 2 else 0)
        d0 = np.random.default_rng(i).standard_normal((M, N)).astype(np.float32)
        say("mx mn", a_fmt, b_fmt, amaj, bmaj, M, N, K, neg_a, neg_b, accum)
        D = run(g, M, N, K, a_fmt, b_fmt, amaj, bmaj, d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = oracle(O, g, M, N, K, a_fmt, b_fmt, amaj, bmaj, d0, neg_a, neg_b, accum)
        nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, name=f"{a_fmt} x {b_fmt} {amaj}{bmaj}-major shapes")
        assert nb == 0, (M, N, K, worst)
        assert np.isnan(D[:, N:]).all()


@pytest.mark.parametrize("a_fmt,b_fmt,amaj,bmaj", [("e4m3", "e4m3", "m", "n"), ("e2m1", "e4m3", "k", "n"),
                                                   ("e2m1", "e2m1", "m", "k")])
def test_mx_mn_scale_groups(O, a_fmt, b_fmt, amaj, bmaj):
    """MN-major storage at K tile counts around the scale ring's four-tile groups (5, 7 and 13
    whole tiles, one with a partial last tile), both pipeline depths (two stages for two
    8-bit MN-major operands, three otherwise)."""
    for i, K in enumerate([640, 896, 1696]):
        M, N = 260, 300
        g = case(a_fmt, b_fmt, amaj, bmaj, 150 + i, M, N, K)
        say("mx mn scale groups", a_fmt, b_fmt, amaj, bmaj, M, N, K)
        D = run(g, M, N, K, a_fmt, b_fmt, amaj, bmaj)
        ref, bound = oracle(O, g, M, N, K, a_fmt, b_fmt, amaj, bmaj)
        nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, name=f"{a_fmt} x {b_fmt} {amaj}{bmaj}-major scale groups")
        assert nb == 0, (K, worst)


@pytest.mark.parametrize("a_fmt,b_fmt,amaj,bmaj", [("e2m3", "e4m3", "k", "n"), ("e4m3", "e3m2", "m", "k"),
                                                   ("e2m1", "e2m3", "m", "k"), ("e3m2", "e2m1", "k", "n")])
def test_mx_mn_with_6bit_kmajor_operand(O, a_fmt, b_fmt, amaj, bmaj):
    """An MN-major 8- or 4-bit operand against a K-major 6-bit one."""
    for i, (M, N, K) in enumerate([(300, 260, 288), (64, 96, 1056), (33, 40, 96)]):
        g = case(a_fmt, b_fmt, amaj, bmaj, 110 + i, M, N, K)
        say("mx mn 6-bit partner", a_fmt, b_fmt, amaj, bmaj, M, N, K)
        D = run(g, M, N, K, a_fmt, b_fmt, amaj, bmaj)
        ref, bound = oracle(O, g, M, N, K, a_fmt, b_fmt, amaj, bmaj)
        nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, name=f"{a_fmt} x {b_fmt} {amaj}{bmaj}-major 6-bit partner")
        assert nb == 0, (M, N, K, worst)


@pytest.mark.parametrize("a_fmt,b_fmt", [("e4m3", "e2m1"), ("e2m1", "e5m2"), ("e2m1", "e2m3")])
def test_mx_mn_equals_kmajor_bitwise(O, a_fmt, b_fmt):
    """The general kernel on MN-major storage against the same kernel on the K-major codes."""
    M, N, K = 300, 260, 416
    for amaj, bmaj in MAJORS:
        if (amaj == "m" and BITS[a_fmt] == 6) or (bmaj == "n" and BITS[b_fmt] == 6):
            continue
        g = case(a_fmt, b_fmt, amaj, bmaj, 7, M, N, K)
        say("mx mn vs k-major", a_fmt, b_fmt, amaj, bmaj)
        D = run(g, M, N, K, a_fmt, b_fmt, amaj, bmaj)
        gk = dict(g, As=g["A"], Bs=g["B"], lda_s=g["lda"], ldb_s=g["ldb"])
        Dk = run(gk, M, N, K, a_fmt, b_fmt, "k", "k")
        assert np.array_equal(D[:, :N], Dk[:, :N]), (amaj, bmaj)


def test_mx_mn_exact_pair_bit_exact(O):
    """E2M1 x E2M1 with unit-range scales sums exactly: bit-identical to the oracle."""
    M, N, K = 300, 200, 352
    g = case("e2m1", "e2m1", "m", "n", 5, M, N, K, exp_range=1)
    say("mx mn exact e2m1")
    D = run(g, M, N, K, "e2m1", "e2m1", "m", "n")
    ref, _ = oracle(O, g, M, N, K, "e2m1", "e2m1", "m", "n")
    assert np.array_equal(D[:, :N], ref.astype(np.float32))


def test_mx_mn_nan_scale_and_epilogue(O):
    M, N, K = 200, 136, 256
    g = case("e4m3", "e2m1", "m", "n", 4, M, N, K)
    g["SFA"][5, 6] = 255
    say("mx mn nan scale")
    D = run(g, M, N, K, "e4m3", "e2m1", "m", "n")
    assert np.isnan(D[5, :N]).all()
    assert np.isfinite(np.delete(D[:, :N], 5, 0)).all()
    g["SFA"][5, 6] = 127
    say("mx mn silu_affine")
    D = run(g, M, N, K, "e4m3", "e2m1", "m", "n", ew=bsm.ewise_desc("silu_affine", 2.0, 1.0))
    ref, bound = oracle(O, g, M, N, K, "e4m3", "e2m1", "m", "n")
    pm, pn = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    t_x = (1e-5 * bound + np.ldexp(np.abs(ref), -24)).reshape(-1)
    f = O.ewise_silu_affine(ref, 2.0, 1.0).reshape(-1)
    silu = O.ewise_silu_affine(ref, 1.0, 0.0).reshape(-1)
    tol = 1.1 * 2.0 * t_x + np.ldexp(2.0 * np.abs(silu), -20) + np.ldexp(np.abs(f), -23) + np.ldexp(3.0, -112)
    assert (np.abs(D[:, :N].reshape(-1).astype(np.float64) - f) <= tol).all()


@pytest.mark.parametrize("a_fmt,b_fmt,amaj,bmaj", [("e4m3", "e4m3", "m", "n"), ("e2m1", "e2m1", "k", "n")])
def test_mx_mn_full_size_sampled(O, a_fmt, b_fmt, amaj, bmaj):
    """M = N = 8192, K = 16384 with MN-major storage: sampled outputs against the oracle."""
    M, N, K = 8192, 8192, 16384
    g = W.mx_pair(23, M, N, K, a_fmt, b_fmt)
    As = W.mn_major(g["A"], a_fmt, M, K, M) if amaj == "m" else g["A"]
    Bs = W.mn_major(g["B"], b_fmt, N, K, N) if bmaj == "n" else g["B"]
    lda, ldb = (M if amaj == "m" else K), (N if bmaj == "n" else K)
    gs = dict(g, As=As, Bs=Bs, lda_s=lda, ldb_s=ldb, lda=K, ldb=K)
    say("mx mn full", a_fmt, b_fmt, amaj, bmaj, M, N, K)
    D = run(gs, M, N, K, a_fmt, b_fmt, amaj, bmaj)
    pm, pn = W.sample_points(M, N, 600)
    ref, bound = O.gemm_block_scale_points(M, N, K, a_fmt, As, lda, g["SFA"], K // 32, b_fmt, Bs, ldb, g["SFB"],
                                           K // 32, None, 0, 0, 0, 0, pm, pn, a_major=amaj, b_major=bmaj)
    nb, worst = check(O, gs, a_fmt, b_fmt, K, D, ref, bound, pm, pn,
                      name=f"{a_fmt} x {b_fmt} {amaj}{bmaj}-major 8192x8192x16384 (600 points)")
    assert nb == 0, worst
    assert np.isfinite(D[:, :N]).all()
