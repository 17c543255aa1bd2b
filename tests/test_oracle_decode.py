"""Pins of the oracle's decoders and encoders against independent libraries and closed forms.

Decoders are checked code by code against torch's / numpy's own conversions (for
e4m3, e5m2 and e8m0: torch.float8_e4m3fn / float8_e5m2 / float8_e8m0fnu, the OCP formats;
e5m2 also against numpy's binary16, whose top byte it is), and the
e2m1 table against the value list of the OCP MX v1.0 specification (section 5.3.3).
Encoders (round to nearest even) are checked against numpy / torch float64 casts on
values chosen to hit ties, subnormals, carries and overflow.
"""
import numpy as np
import pytest
import torch

from block_scaled_matrix_amd import workloads as W


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_e4m3_all_codes_vs_torch(O):
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode("e4m3", codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(got, ref)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isfinite(got).sum() == 254


def test_e5m2_all_codes_vs_torch_and_f16_top_byte(O):
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode("e5m2", codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert _same(got, ref)
    # E5M2 is binary16 with the low 8 fraction bits dropped: code c is the half float c << 8
    half = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    assert _same(got, half)
    assert got[0x7B] == 57344.0 and got[0x01] == 2.0 ** -16 and got[0x7C] == np.inf and got[0xFC] == -np.inf
    assert np.isnan(got[0x7E]) and np.isfinite(got).sum() == 248


def test_e8m0_all_codes_vs_torch_and_closed_form(O):
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode("e8m0", codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same(got, ref)
    assert all(got[c] == 2.0 ** (c - 127) for c in range(255)) and np.isnan(got[255])


def test_e2m1_table_and_nibble_order(O):
    # OCP MX v1.0 E2M1 values for codes 0..7; bit 3 is the sign.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    packed = np.array([(2 * i + 1) << 4 | (2 * i) for i in range(8)], dtype=np.uint8)  # codes 0..15
    got = O.decode("e2m1", packed, 16)
    exp = np.array(table + [-v for v in table])
    assert _same(got, exp)
    assert np.signbit(got[8])  # code 8 is -0
    # low nibble is element 0: byte 0x2F -> element0 = code 0xF (-6), element1 = code 2 (1.0)
    assert list(O.decode("e2m1", np.array([0x2F], np.uint8), 2)) == [-6.0, 1.0]


def test_f16_bf16_f32_decoders(O):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _same(O.decode("f16", h), h.view(np.float16).astype(np.float64))
    ref_bf = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(O.decode("bf16", h), ref_bf)
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    u[:6] = [0, 0x80000000, 1, 0x7F800000, 0xFF800000, 0x007FFFFF]
    assert _same(O.decode("f32", u), u.view(np.float32).astype(np.float64))


def _encode_cases():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.integers(-150, 130, 20000)),
        np.exp2(rng.integers(-160, 140, 3000).astype(np.float64)) * (1 + rng.integers(0, 512, 3000) / 512.0),
        [0.0, -0.0, np.inf, -np.inf, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -11, 1 + 3 * 2 ** -11,
         1 + 2 ** -24, 1 + 3 * 2 ** -24, 65504.0, 65520.0, 65519.99, 2 ** -25, 2 ** -24 * 1.5, 3.4e38, 3.5e38],
    ])
    return x.astype(np.float64)


def test_enc_bf16_vs_torch(O):
    # torch rounds float64 -> bfloat16 through float32 (two roundings), so the library
    # reference is taken on float32-representable inputs, where it rounds once.
    with np.errstate(over="ignore"):
        x = _encode_cases().astype(np.float32).astype(np.float64)
    got = O.enc("bf16", x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_enc_bf16_single_rounding_exact(O):
    # Exact rational check on random doubles: the encoded value is the nearer of the
    # two bfloat16 neighbours (ties to even mantissa), never a double-rounded one.
    from fractions import Fraction
    rng = np.random.default_rng(5)
    xs = list(rng.uniform(1, 2, 300) * np.exp2(rng.integers(-120, 120, 300))) + [1.2074678329077994e-34]
    for x in xs:
        b = int(O.enc("bf16", [x])[0])
        v = Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))
        up = Fraction(float(np.array([(b + 1) << 16], np.uint32).view(np.float32)[0]))
        dn = Fraction(float(np.array([(b - 1) << 16], np.uint32).view(np.float32)[0]))
        fx = Fraction(x)
        assert abs(fx - v) <= abs(fx - up) and abs(fx - v) <= abs(fx - dn)
        if abs(fx - v) == abs(fx - up) or abs(fx - v) == abs(fx - dn):
            assert b % 2 == 0


def test_enc_f16_vs_numpy(O):
    x = _encode_cases()
    got = O.enc("f16", x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_enc_f32_vs_numpy(O):
    x = _encode_cases()
    got = O.enc("f32", x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_encode_decode_roundtrip(O, dt):
    rng = np.random.default_rng(3)
    n = 5000
    bits = rng.integers(0, 2 ** (32 if dt == "f32" else 16), n, dtype=np.uint64)
    bits = bits.astype(np.uint32 if dt == "f32" else np.uint16)
    vals = O.decode(dt, bits)
    keep = ~np.isnan(vals)
    back = O.enc(dt, vals[keep])
    assert np.array_equal(back, bits[keep])


# OCP MX v1.0, section 5.3.2 (FP6): max normal, min normal, max subnormal, min subnormal.
FP6_ANCHORS = {"e2m3": (7.5, 1.0, 0.875, 0.125, 3), "e3m2": (28.0, 0.25, 0.1875, 0.0625, 2)}


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_all_codes_vs_spec_and_fp8_grid(O, fmt):
    """All 64 codes: the specification's anchor values, bit 5 as the sign, strictly increasing
    magnitudes over codes 0..31, the subnormals evenly spaced and every binade holding 2^m
    evenly spaced values, and each value on the grid of the 8-bit format with the same
    mantissa width (E2M3 -> float8_e4m3fn, E3M2 -> float8_e5m2), via torch's round trip."""
    mx_n, mn_n, mx_s, mn_s, mbits = FP6_ANCHORS[fmt]
    codes = np.arange(64)
    got = O.decode(fmt, W.pack_fp6(codes.reshape(1, 64)), 64)
    pos, neg = got[:32], got[32:]
    assert _same(neg, -pos) and np.signbit(got[32])
    assert pos[31] == mx_n and pos[1 << mbits] == mn_n and pos[(1 << mbits) - 1] == mx_s and pos[1] == mn_s
    assert pos[0] == 0.0 and np.all(np.diff(pos) > 0)
    sub = pos[:1 << mbits]
    assert np.allclose(np.diff(sub), mn_s, rtol=0, atol=0)
    for e in range(1, 32 >> mbits):
        b = pos[e << mbits:(e + 1) << mbits]
        assert len(set(np.diff(b))) == 1 and b[0] == 2.0 ** (e - 1) * mn_n
    t = torch.float8_e4m3fn if fmt == "e2m3" else torch.float8_e5m2
    assert _same(torch.from_numpy(got).to(t).to(torch.float64).numpy(), got)


def test_fp6_packing_vs_unpackbits(O):
    """Element i of a packed row is bits 6i..6i+5 of the row's little-endian bit string:
    extracted independently with numpy's unpackbits, then decoded code by code."""
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 256, (5, 48), dtype=np.uint8)       # 5 rows of 64 elements
    bits = np.unpackbits(raw, axis=1, bitorder="little").reshape(5, 64, 6)
    codes = (bits * (1 << np.arange(6))).sum(axis=2)
    for fmt in ("e2m3", "e3m2"):
        table = O.decode(fmt, W.pack_fp6(np.arange(64).reshape(1, 64)), 64)
        got = O.decode(fmt, raw, 5 * 64).reshape(5, 64)
        assert _same(got, table[codes])
