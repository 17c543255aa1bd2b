"""GPU parity over seeded random configurations: dense and block-scaled GEMMs whose shapes,
majors, format pairings, negation, accumulation and leading-dimension padding are drawn from
one seeded generator, each checked against the oracle under the stated bound (dense
2e-3 * sum|ab|, block-scaled 1e-5 * sum|ab|, plus half an ulp of the float32 result), with the
columns past N left untouched. The fixed-case tests pin chosen edges; the sweep covers the
combinations between them."""
import numpy as np
import pytest

from gpu_util import say
from test_gpu_gemm import TOL_DENSE, dense_case, run_dense
from test_gpu_mx_any import check
from test_gpu_mx_mn import case, oracle, run

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"]
MN_MAJOR = {"e4m3", "e5m2", "e2m1"}     # formats that may be stored MN-major


def test_dense_random_sweep(O):
    rng = np.random.default_rng(2024)
    for c in range(24):
        M, N, K = (int(x) for x in (rng.integers(1, 600), rng.integers(1, 600), rng.integers(1, 1300)))
        dt = ("bf16", "f16")[c % 2]
        amaj, bmaj = str(rng.choice(["k", "m"])), str(rng.choice(["k", "n"]))
        neg_a, neg_b, accum = (int(x) for x in rng.integers(0, 2, 3))
        A, lda, B, ldb = dense_case(rng, M, N, K, dt, amaj, bmaj)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        say("dense sweep", c, dt, amaj, bmaj, M, N, K, neg_a, neg_b, accum)
        D = run_dense(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = O.gemm(M, N, K, dt, A, lda, amaj, B, ldb, bmaj, d0, N, neg_a, neg_b, accum)
        nb, first, worst = O.check_gemm(D, ref, bound, TOL_DENSE)
        assert nb == 0, (c, dt, amaj, bmaj, M, N, K, neg_a, neg_b, accum, first, worst)
        assert np.isnan(D[:, N:]).all()


def test_block_scaled_random_sweep(O):
    rng = np.random.default_rng(2025)
    for c in range(30):
        a_fmt, b_fmt = str(rng.choice(FMTS)), str(rng.choice(FMTS))
        amaj = "m" if a_fmt in MN_MAJOR and rng.random() < 0.3 else "k"
        bmaj = "n" if b_fmt in MN_MAJOR and rng.random() < 0.3 else "k"
        M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
        K = 32 * int(rng.integers(1, 48))
        pad = 64 if rng.random() < 0.3 else 0
        neg_a, neg_b, accum = (int(x) for x in rng.integers(0, 2, 3))
        g = case(a_fmt, b_fmt, amaj, bmaj, 500 + c, M, N, K, pad=pad)
        d0 = rng.standard_normal((M, N)).astype(np.float32)
        say("block-scaled sweep", c, a_fmt, b_fmt, amaj, bmaj, M, N, K, pad, neg_a, neg_b, accum)
        D = run(g, M, N, K, a_fmt, b_fmt, amaj, bmaj, d0 if accum else None, neg_a, neg_b, accum)
        ref, bound = oracle(O, g, M, N, K, a_fmt, b_fmt, amaj, bmaj, d0, neg_a, neg_b, accum)
        nb, worst = check(O, g, a_fmt, b_fmt, K, D, ref, bound, name="block-scaled random sweep")
        assert nb == 0, (c, a_fmt, b_fmt, amaj, bmaj, M, N, K, pad, neg_a, neg_b, accum, worst)
        assert np.isnan(D[:, N:]).all()
