"""Seeded synthetic inputs for the five workloads (host numpy arrays).

This module only draws random numbers and lays them out in memory; it holds none
of the arithmetic of the method. Both the HIP path (tests, benchmark) and the CPU
oracle consume exactly these arrays. Every generator is numpy's default_rng (PCG64)
with a fixed seed; tensors are drawn in the order listed. 16-bit floats are
produced from float32 draws by round-to-nearest-even (torch's CPU conversion).

Workloads (sizes are the ones the benchmark runs):
  gemm_f16_128      M=N=128, K=64 fp16, A and B (N,K) both K-major, U(-1,1), seed 0.
  add_one_tile      float32 arange(768) viewed as (2,32,3,4).
  box_copy_bf16     bf16 16381x8190 tensors in a 8192-element row pitch, (128,64)
                    boxes, 128-byte swizzle; src and the reduce-add target N(0,1),
                    seed 2; padding and the plain-store target hold a sentinel.
  gemm_bf16_8192    M=N=K=8192 bf16, A K-major, B stored (K,N) (MN-major),
                    N(0,1)/sqrt(K), accumulate onto D0 ~ N(0,1) float32, seed 3.
  mxfp8_8192_16384  M=N=8192, K=16384, E4M3 codes uniform over the 254 finite codes,
                    E8M0 scales 127+U{-4..4}, both K-major, fresh D, seed 4.
  mxfp4_16384_8192  M=16384, N=8192, K=8192, E2M1 bytes uniform (two uniform nibbles),
                    E8M0 scales 127+U{-6..6}, neg_a, fresh D, seed 5.
  box_rank3_bf16    a bf16 (64, 2048, 2048) tensor N(0,1), seed 7, read as (2, 64, 128) boxes
                    with element strides (1, 2, 1) tiling it (32 x 32 x 16 repeats).
  gather4_bf16      a bf16 65536x4096 table N(0,1), seed 6; four-row gathers with a (1,64)
                    box and 128-byte swizzle (512-byte images), rows taken four at a time
                    from a seeded permutation, every 64-column block of each row group;
                    the scatter sends image k's rows to the rows of a second permutation.
"""
from __future__ import annotations

import numpy as np

SENTINEL_BF16 = 0x7FC1  # a NaN payload no kernel produces: marks bytes that must stay untouched

# All E4M3 codes except the two NaN encodings 0x7F and 0xFF (OCP E4M3 "fn").
FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
FINITE_E5M2 = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)  # exponent field < 31


def to_half_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> raw uint16 bits of fp16/bf16 (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def gemm_f16_128(seed: int = 0, M: int = 128, N: int = 128, K: int = 64):
    rng = np.random.default_rng(seed)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (N, K)).astype(np.float32)
    return {"M": M, "N": N, "K": K, "A": to_half_bits(a, "f16"), "B": to_half_bits(b, "f16"),
            "a_major": "k", "b_major": "k", "accum": 0, "neg_a": 0, "neg_b": 0, "dtype": "f16"}


def quarter_grid_f16(seed: int = 0, shapes=((128, 64), (64, 64))):
    """fp16 bit arrays, one per shape in order from one generator, of values on the grid
    {-1, -3/4, ..., 3/4, 1} drawn uniformly (the operands of the 128x64x64 example GEMM that
    "tcgen05.mma", Example: four K16 issues, runs with seed 0). Every product is a multiple of
    1/16 and every K-sum of 64 of them is below 2^6, so each is exact in float32."""
    rng = np.random.default_rng(seed)
    quarter = np.float16(0.25)
    return [(rng.integers(low=-4, high=5, size=sh).astype(np.float16) * quarter).view(np.uint16) for sh in shapes]


def add_one_tile():
    return np.arange(768, dtype=np.float32).reshape(2, 32, 3, 4)


def box_copy_bf16(seed: int = 2, rows: int = 16381, cols: int = 8190, pitch: int = 8192):
    """Three (rows, pitch) uint16 buffers holding bf16 bits: src, dst (sentinel), dst_add."""
    rng = np.random.default_rng(seed)
    src = np.full((rows, pitch), SENTINEL_BF16, dtype=np.uint16)
    src[:, :cols] = to_half_bits(rng.standard_normal((rows, cols), dtype=np.float32), "bf16")
    add = np.full((rows, pitch), SENTINEL_BF16, dtype=np.uint16)
    add[:, :cols] = to_half_bits(rng.standard_normal((rows, cols), dtype=np.float32), "bf16")
    dst = np.full((rows, pitch), SENTINEL_BF16, dtype=np.uint16)
    return {"rows": rows, "cols": cols, "pitch": pitch, "src": src, "dst": dst, "dst_add": add,
            "box": (128, 64), "estr": (1, 1), "swizzle": 3, "fill": 0, "dtype": "bf16"}


def gemm_bf16(seed: int = 3, M: int = 8192, N: int = 8192, K: int = 8192):
    """A (M,K) K-major, B stored (K,N) (MN-major), D0 (M,N) float32, accumulate."""
    rng = np.random.default_rng(seed)
    s = np.float32(1.0 / np.sqrt(K))
    a = to_half_bits(rng.standard_normal((M, K), dtype=np.float32) * s, "bf16")
    b = to_half_bits(rng.standard_normal((K, N), dtype=np.float32) * s, "bf16")
    d0 = rng.standard_normal((M, N), dtype=np.float32)
    return {"M": M, "N": N, "K": K, "A": a, "B": b, "D0": d0, "lda": K, "ldb": N,
            "a_major": "k", "b_major": "n", "accum": 1, "neg_a": 0, "neg_b": 0, "dtype": "bf16"}


def mxfp8(seed: int = 4, M: int = 8192, N: int = 8192, K: int = 16384, exp_range: int = 4, a_fmt: str = "e4m3",
          b_fmt: str = "e4m3"):
    """Uniform random finite codes of the operand formats (E4M3 or E5M2) and scales 127 +- exp_range."""
    rng = np.random.default_rng(seed)
    codes = {"e4m3": FINITE_E4M3, "e5m2": FINITE_E5M2}
    a = codes[a_fmt][rng.integers(0, codes[a_fmt].size, (M, K), dtype=np.int16)]
    b = codes[b_fmt][rng.integers(0, codes[b_fmt].size, (N, K), dtype=np.int16)]
    sfa = (127 + rng.integers(-exp_range, exp_range + 1, (M, K // 32), dtype=np.int16)).astype(np.uint8)
    sfb = (127 + rng.integers(-exp_range, exp_range + 1, (N, K // 32), dtype=np.int16)).astype(np.uint8)
    return {"M": M, "N": N, "K": K, "A": a, "B": b, "SFA": sfa, "SFB": sfb, "lda": K, "ldb": K,
            "ld_sfa": K // 32, "ld_sfb": K // 32, "fmt": a_fmt, "b_fmt": b_fmt, "accum": 0, "neg_a": 0, "neg_b": 0}


def mxfp4(seed: int = 5, M: int = 16384, N: int = 8192, K: int = 8192, exp_range: int = 6):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sfa = (127 + rng.integers(-exp_range, exp_range + 1, (M, K // 32), dtype=np.int16)).astype(np.uint8)
    sfb = (127 + rng.integers(-exp_range, exp_range + 1, (N, K // 32), dtype=np.int16)).astype(np.uint8)
    return {"M": M, "N": N, "K": K, "A": a, "B": b, "SFA": sfa, "SFB": sfb, "lda": K, "ldb": K,
            "ld_sfa": K // 32, "ld_sfb": K // 32, "fmt": "e2m1", "accum": 0, "neg_a": 1, "neg_b": 0}


BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """(rows, K) 6-bit codes -> (rows, 3K/4) bytes: element i at bits 6i..6i+5 of the row's
    little-endian bit string (K a multiple of 4)."""
    c = codes.astype(np.uint32).reshape(codes.shape[0], -1, 4)
    w = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
    out = np.empty(w.shape + (3,), np.uint8)
    out[..., 0], out[..., 1], out[..., 2] = w & 255, (w >> 8) & 255, (w >> 16) & 255
    return out.reshape(codes.shape[0], -1)


def mx_codes(rng, fmt: str, rows: int, K: int) -> np.ndarray:
    """Uniform random element codes of a block-scaled format, packed K-major: (rows, K*bits/8)
    bytes. 8-bit formats draw from their finite codes, E2M1 draws whole bytes (two uniform
    nibbles), the 6-bit formats draw all 64 codes (all finite)."""
    if fmt == "e4m3":
        return FINITE_E4M3[rng.integers(0, FINITE_E4M3.size, (rows, K))]
    if fmt == "e5m2":
        return FINITE_E5M2[rng.integers(0, FINITE_E5M2.size, (rows, K))]
    if fmt == "e2m1":
        return rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    return pack_fp6(rng.integers(0, 64, (rows, K)))


def mx_pair(seed: int, M: int, N: int, K: int, a_fmt: str, b_fmt: str, exp_range: int = 4):
    """Block-scaled operands of any two formats: codes uniform (mx_codes), E8M0 scales
    127 + U{-exp_range..exp_range}, both K-major with lda = ldb = K."""
    rng = np.random.default_rng(seed)
    a = mx_codes(rng, a_fmt, M, K)
    b = mx_codes(rng, b_fmt, N, K)
    sfa = (127 + rng.integers(-exp_range, exp_range + 1, (M, K // 32))).astype(np.uint8)
    sfb = (127 + rng.integers(-exp_range, exp_range + 1, (N, K // 32))).astype(np.uint8)
    return {"M": M, "N": N, "K": K, "A": a, "B": b, "SFA": sfa, "SFB": sfb, "lda": K, "ldb": K,
            "ld_sfa": K // 32, "ld_sfb": K // 32, "fmt": a_fmt, "b_fmt": b_fmt, "accum": 0, "neg_a": 0, "neg_b": 0}


def unpack_codes(raw: np.ndarray, fmt: str, rows: int, K: int) -> np.ndarray:
    """Packed element codes (rows, K) (8-bit bytes; E2M1 two per byte, low nibble first; 6-bit
    fields of a little-endian bit string per row) -> one uint8 code per element."""
    bits = BITS[fmt]
    r = np.ascontiguousarray(raw).reshape(rows, -1)
    if bits == 8:
        return r[:, :K].copy()
    if bits == 4:
        return np.stack([r & 15, r >> 4], axis=2).reshape(rows, -1)[:, :K].copy()
    bs = np.unpackbits(r, axis=1, bitorder="little")[:, :6 * K].reshape(rows, K, 6)
    return (bs * (1 << np.arange(6, dtype=np.uint8))).sum(axis=2, dtype=np.uint8)


def pack_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """One code per element (rows, n) -> packed rows (the inverse of unpack_codes)."""
    bits = BITS[fmt]
    if bits == 8:
        return np.ascontiguousarray(codes, dtype=np.uint8)
    if bits == 4:
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return pack_fp6(np.ascontiguousarray(codes))


def mn_major(raw: np.ndarray, fmt: str, rows: int, K: int, ld: int, seed: int | None = None) -> np.ndarray:
    """K-major packed codes (rows, K) -> MN-major storage: K rows of ld elements, element
    (k, m) = code (m, k); the ld - rows padding elements of each row are random codes
    (seed given) or zero."""
    codes = unpack_codes(raw, fmt, rows, K).T
    out = np.zeros((K, ld), np.uint8)
    if seed is not None:
        out[:] = np.random.default_rng(seed).integers(0, 1 << BITS[fmt], (K, ld), dtype=np.uint8)
    out[:, :rows] = codes
    return pack_codes(out, fmt)


def gather4_bf16(seed: int = 6, rows: int = 65536, cols: int = 4096, width: int = 64):
    """Table (rows, cols) uint16 bf16 bits; gather and scatter coordinates (n, 5) int32, issue
    t = group * (cols / width) + block: column start block * width, then four rows."""
    rng = np.random.default_rng(seed)
    table = to_half_bits(rng.standard_normal((rows, cols), dtype=np.float32), "bf16")
    perm_g = rng.permutation(rows).astype(np.int32)
    perm_s = rng.permutation(rows).astype(np.int32)
    nb = cols // width
    col = np.tile(np.arange(nb, dtype=np.int32) * width, rows // 4)

    def coords(perm):
        c = np.empty((rows // 4 * nb, 5), np.int32)
        c[:, 0] = col
        c[:, 1:] = np.repeat(perm.reshape(-1, 4), nb, axis=0)
        return c

    return {"rows": rows, "cols": cols, "width": width, "table": table, "gather": coords(perm_g),
            "scatter": coords(perm_s), "perm_gather": perm_g, "perm_scatter": perm_s, "swizzle": 3, "fill": 0,
            "dtype": "bf16"}


def box_rank3_bf16(seed: int = 7, dims=(64, 2048, 2048)):
    """A rank-3 bf16 tensor and the repeat axes that tile it with (2, 64, 128) boxes sampled at
    element strides (1, 2, 1)."""
    rng = np.random.default_rng(seed)
    x = to_half_bits(rng.standard_normal(dims, dtype=np.float32), "bf16")
    box, estr = (2, 64, 128), (1, 2, 1)
    reps = tuple(d // b for d, b in zip(dims, box))
    steps = [tuple(box[i] if i == a else 0 for i in range(3)) for a in range(3)]
    return {"x": x, "dims": dims, "box": box, "estr": estr, "coords": (0, 0, 0), "repeats": reps, "steps": steps,
            "swizzle": 0, "fill": 0, "dtype": "bf16"}


def sample_points(M: int, N: int, n: int, seed: int = 99):
    """Output coordinates checked one by one at full size: the four corners, the last
    row and column, and uniform random points."""
    rng = np.random.default_rng(seed)
    pm = [0, 0, M - 1, M - 1] + list(rng.integers(0, M, n)) + [M - 1] * 8 + list(rng.integers(0, M, 8))
    pn = [0, N - 1, 0, N - 1] + list(rng.integers(0, N, n)) + list(rng.integers(0, N, 8)) + [N - 1] * 8
    return np.array(pm, dtype=np.int64), np.array(pn, dtype=np.int64)
