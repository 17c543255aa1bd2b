"""Pins of the oracle's box load / store / reduce-add, swizzle, add-one and ldmatrix image.

Independent references used here: the pages' worked examples (fixtures under
tests/golden/), numpy strided slicing of the same tensor (for box sampling), torch's
bfloat16/float16 addition on the CPU (for the add-reduction), and algebraic
properties of the swizzle permutation.
"""
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- swizzle
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_swizzle_is_chunk_permutation_within_period(O, mode):
    period = 128 << mode if mode else 16
    offs = np.arange(4 * 1024)
    sw = np.array([O.swizzle(int(o), mode) for o in offs])
    assert np.array_equal(np.sort(sw), offs)                      # a permutation
    assert np.array_equal(np.array([O.swizzle(int(o), mode) for o in sw]), offs)  # an involution
    assert np.array_equal(sw & 15, offs & 15)                     # 16-byte chunks move whole
    assert np.array_equal(sw // period, offs // period)           # stays inside its period
    if mode == 0:
        assert np.array_equal(sw, offs)


def test_swizzle128_rows_of_128_bytes(O):
    # A (128,64) bf16 image has 128-byte rows: the 8 chunks of logical chunk c across
    # 8 consecutive rows land on 8 different physical chunks (what the XOR is for),
    # and row r's chunk c sits at physical chunk c ^ (r % 8).
    for r in range(16):
        for c in range(8):
            phys = O.swizzle(r * 128 + c * 16, 3)
            assert phys // 128 == r and (phys % 128) // 16 == c ^ (r % 8)
    for c in range(8):
        assert len({O.swizzle(r * 128 + c * 16, 3) % 128 for r in range(8)}) == 8


# ----------------------------------------------------------------------------- box load
def test_pages_two_box_example(O):
    """cp.async.bulk.tensor, Example: two 8x16 boxes of a 16x16 uint32 arange."""
    exp = np.loadtxt(os.path.join(GOLD, "tma_two_box_expected.txt"), dtype=np.uint64).astype(np.uint32)
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    imgs = [O.box_load(x, "u32", (16, 16), (64, 4), (8, 16), (1, 1), (8 * g, 0)) for g in range(2)]
    assert all(im.size == 512 for im in imgs)            # 512 bytes per box
    out = np.concatenate([im.view(np.uint32).reshape(8, 16) for im in imgs])
    assert np.array_equal(out, exp)


def _numpy_box(x, fill, box, estr, coords):
    """Expected compact image via numpy slicing of a fill-padded copy of x."""
    # pad each axis just enough to hold the box's sampled range [c, c + (b - 1) e]
    pad = [(max(0, -c), max(0, c + (b - 1) * e + 1 - d)) for c, b, e, d in zip(coords, box, estr, x.shape)]
    xp = np.pad(x, pad, constant_values=fill)
    sl = tuple(slice(c + p[0], c + p[0] + b, e) for c, p, b, e in zip(coords, pad, box, estr))
    return xp[sl]


@pytest.mark.parametrize("dtype,npdt,esz", [("u16", np.uint16, 2), ("u32", np.uint32, 4), ("u8", np.uint8, 1)])
@pytest.mark.parametrize("rank", [1, 2, 3, 4, 5])
def test_box_load_vs_numpy_slicing(O, dtype, npdt, esz, rank):
    rng = np.random.default_rng(100 + rank * 7 + esz)
    hi_dim, hi_box = (20, 12) if rank <= 3 else (9, 5)     # ranks 4 and 5: smaller tensors and boxes
    for trial in range(40 if rank <= 3 else 12):
        dims = tuple(int(v) for v in rng.integers(1, hi_dim, rank))
        inner_box = 16 // esz * int(rng.integers(1, 4))
        box = tuple(int(v) for v in rng.integers(1, hi_box, rank - 1)) + (inner_box,)
        estr = tuple(int(v) for v in rng.integers(1, 5, rank - 1)) + (1,)
        coords = tuple(int(v) for v in rng.integers(-10, 25, rank))
        swz = int(rng.integers(0, 4))
        if swz and inner_box * esz > (16 << swz):
            swz = 0
        # pitch-padded storage: inner rows padded to a multiple of 16 bytes + extra
        pitch = ((dims[-1] * esz + 15) // 16 * 16 + 16 * int(rng.integers(0, 3))) // esz
        shape_alloc = dims[:-1] + (pitch,)
        mem = rng.integers(0, 2 ** (8 * esz), shape_alloc, dtype=np.uint64).astype(npdt)
        strides = [mem.strides[i] for i in range(rank)]
        img = O.box_load(mem, dtype, dims, strides, box, estr, coords, swz, 0)
        ext = O.image_extents(box, estr)
        nbytes = int(np.prod(ext)) * esz
        unsw = np.empty(nbytes, np.uint8)
        for o in range(nbytes):
            unsw[o] = img[O.swizzle(o, swz)]
        got = unsw.view(npdt).reshape(ext)
        view = mem[tuple(slice(0, d) for d in dims)]
        assert np.array_equal(got, _numpy_box(view, 0, box, estr, coords)), (dims, box, estr, coords, swz)
        written = np.zeros(img.size, bool)
        written[[O.swizzle(o, swz) for o in range(nbytes)]] = True
        assert not img[~written].any()  # bytes outside the swizzled image untouched (zero-initialised)


def test_box_nan_fill_and_fill_count(O):
    x = np.arange(40, dtype=np.float32).reshape(5, 8)
    img = O.box_load(x, "f32", (5, 8), (32, 4), (4, 8), (1, 1), (3, -2), 0, 1)
    v = img.view(np.float32)[:32].reshape(4, 8)
    inb = np.zeros((4, 8), bool)
    inb[:2, 2:] = True                      # rows 3,4 and cols 0..5 are inside
    assert np.isnan(v[~inb]).all() and np.array_equal(v[inb], x[3:5, 0:6].ravel())
    assert img.view(np.uint32)[:32][~inb.ravel()].tolist() == [0x7FC00000] * int((~inb).sum())
    with pytest.raises(ValueError):
        O.box_load(np.zeros(16, np.uint32), "u32", (16,), (4,), (4,), (1,), (0,), 0, 1)  # no NaN in u32


def test_box_nan_fill_e5m2_and_e4m3(O):
    """One-byte float formats: the fill byte decodes to NaN (torch's OCP decoders) and, for E5M2,
    is the top byte of binary16's canonical quiet NaN."""
    import torch
    x = np.arange(24, dtype=np.uint8).reshape(3, 8)
    for dt, tdt in (("e5m2", torch.float8_e5m2), ("e4m3", torch.float8_e4m3fn)):
        img = O.box_load(x, dt, (3, 8), (8, 1), (4, 16), (1, 1), (1, 0), 0, 1)[:64].reshape(4, 16)
        assert np.array_equal(img[:2, :8], x[1:3])                     # in range: the bytes themselves
        fill = np.concatenate([img[:2, 8:].ravel(), img[2:].ravel()])
        assert len(set(fill.tolist())) == 1
        assert torch.isnan(torch.from_numpy(fill[:1].copy()).view(tdt).to(torch.float32)).all()
    assert O.box_load(x, "e5m2", (3, 8), (8, 1), (1, 16), (1, 1), (0, 0), 0, 1)[8] == \
        (np.array([np.nan], np.float16).view(np.uint16)[0] >> 8)


# ----------------------------------------------------------------------------- store / reduce
def test_load_store_identity_and_oob_untouched(O):
    rng = np.random.default_rng(21)
    dims, pitch = (37, 45), 48
    src = rng.integers(0, 2 ** 16, (37, pitch), dtype=np.uint16)
    dst = np.full((37, pitch), 0xBEEF, np.uint16)
    st = (pitch * 2, 2)
    for coords in [(0, 0), (30, 40), (-3, -5), (36, 44), (50, 0)]:
        img = O.box_load(src, "u16", dims, st, (16, 32), (1, 1), coords, 3, 0)
        O.box_store(dst, "u16", dims, st, (16, 32), (1, 1), coords, img, 3, 0)
    exp = np.full_like(dst, 0xBEEF)
    for c0, c1 in [(0, 0), (30, 40), (-3, -5), (36, 44), (50, 0)]:
        r0, r1 = max(c0, 0), min(c0 + 16, 37)
        k0, k1 = max(c1, 0), min(c1 + 32, 45)
        if r0 < r1 and k0 < k1:
            exp[r0:r1, k0:k1] = src[r0:r1, k0:k1]
    assert np.array_equal(dst, exp)


@pytest.mark.parametrize("dt,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)])
def test_reduce_add_vs_torch(O, dt, tdt):
    rng = np.random.default_rng(5)
    esz = 4 if dt == "f32" else 2
    npdt = np.uint32 if dt == "f32" else np.uint16
    er = 8 if dt == "f16" else 20   # keep sums finite (no inf - inf NaNs, whose sign is unspecified)
    a = torch.randn(24, 64, generator=torch.Generator().manual_seed(1)) * torch.exp2(torch.randint(-er, er, (24, 64)).float())
    c = torch.randn(24, 64, generator=torch.Generator().manual_seed(2)) * torch.exp2(torch.randint(-er, er, (24, 64)).float())
    at, ct = a.to(tdt), c.to(tdt)
    ibits = torch.int32 if dt == "f32" else torch.int16
    amem = at.view(ibits).numpy().view(npdt).copy()
    cmem = ct.view(ibits).numpy().view(npdt).copy()
    dims, st = (24, 64), (64 * esz, esz)
    box = (8, 64 if dt != "f32" else 32)
    for r in range(0, 24, box[0]):
        for k in range(0, 64, box[1]):
            img = O.box_load(amem, dt, dims, st, box, (1, 1), (r, k), 0, 0)
            O.box_store(cmem, dt, dims, st, box, (1, 1), (r, k), img, 0, 1)
    exp = (ct + at).view(ibits).numpy().view(npdt)   # torch: one rounding of the exact sum
    assert np.array_equal(cmem, exp)
    _ = rng


def test_box_copy_grid_ragged(O):
    rng = np.random.default_rng(9)
    rows, cols, pitch = 45, 70, 72
    src = np.full((rows, pitch), 0x7FC1, np.uint16)
    src[:, :cols] = torch.randn(rows, cols).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    add0 = np.full((rows, pitch), 0x7FC1, np.uint16)
    add0[:, :cols] = torch.randn(rows, cols).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dst = np.full((rows, pitch), 0x7FC1, np.uint16)
    add = add0.copy()
    O.box_copy_grid(src, dst, add, "bf16", (rows, cols), (pitch * 2, 2), (16, 32), (1, 1), 3, 0)
    assert np.array_equal(dst, src)   # logical region copied, padding sentinel on both sides
    a = torch.from_numpy(src[:, :cols].view(np.int16)).view(torch.bfloat16)
    c = torch.from_numpy(add0[:, :cols].view(np.int16)).view(torch.bfloat16)
    assert np.array_equal(add[:, :cols], (a + c).view(torch.int16).numpy().view(np.uint16))
    assert (add[:, cols:] == 0x7FC1).all()
    _ = rng


# ----------------------------------------------------------------------------- add-one
def test_pages_add_one(O):
    exp = np.loadtxt(os.path.join(GOLD, "add_one_expected.txt")).astype(np.float32).reshape(2, 32, 3, 4)
    a = np.arange(768, dtype=np.float32).reshape(2, 32, 3, 4)
    assert np.array_equal(O.add_scalar_f32(a, 1.0), exp)


def test_add_scalar_rounding_vs_numpy(O):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(10000) * np.exp2(rng.integers(-30, 30, 10000))).astype(np.float32)
    for s in (1.0, 3.0e-8, -2.5, 1e30):
        assert np.array_equal(O.add_scalar_f32(x, s).view(np.uint32), (x + np.float32(s)).view(np.uint32))


# ----------------------------------------------------------------------------- ldmatrix
def test_pages_ldmatrix_x2_example(O):
    """ldmatrix / stmatrix, Example: register slots 0, 2, 8, 10 with a sentinel elsewhere."""
    exp = np.loadtxt(os.path.join(GOLD, "ldmatrix_x2_expected.txt"), dtype=np.uint64).astype(np.uint32)
    x = np.arange(128, dtype=np.uint32).reshape(16, 4, 2)
    # shared layout (16,4,2):(8,1,128) in 32-bit words
    sm = np.zeros(256, np.uint32)
    for a in range(16):
        for b in range(4):
            for c in range(2):
                sm[8 * a + b + 128 * c] = x[a, b, c]
    raw = np.full((32, 12), 4294966519, np.uint32)
    for k in range(2):  # S_std[k, m, r, w] = SM[2r+m, w, k]; registers (2,2,8,4):(8,2,4@lane,1@lane)
        offs = [4 * (8 * (2 * r + m) + 128 * k) for m in range(2) for r in range(8)]
        regs = O.ldmatrix(sm, offs, 2, 0)
        for m in range(2):
            raw[:, 8 * k + 2 * m] = regs[:, m]
    assert np.array_equal(raw, exp)


@pytest.mark.parametrize("nmat", [1, 2, 4])
def test_ldmatrix_transpose_identity(O, nmat):
    """register_image[i,j,2w+h] = shared_matrix[i,2w+h,j] for .trans, [i,j,2w+h] without."""
    rng = np.random.default_rng(nmat)
    S = rng.integers(0, 2 ** 16, (nmat, 8, 8), dtype=np.uint64).astype(np.uint16)
    sm = np.zeros(nmat * 8 * 16 + 64, np.uint16)
    perm = rng.permutation(nmat * 8 + 4)[: nmat * 8]   # rows at scattered 16-byte slots
    offs = [int(p) * 16 for p in perm]
    for i in range(nmat):
        for r in range(8):
            sm[offs[8 * i + r] // 2: offs[8 * i + r] // 2 + 8] = S[i, r]
    for trans in (0, 1):
        regs = O.ldmatrix(sm, offs, nmat, trans)
        for lane in range(32):
            j, w = lane // 4, lane % 4
            for i in range(nmat):
                lo, hi = int(regs[lane, i]) & 0xFFFF, int(regs[lane, i]) >> 16
                src = S[i].T if trans else S[i]
                assert (lo, hi) == (src[j, 2 * w], src[j, 2 * w + 1])


# ----------------------------------------------------------------------------- repeats (coord_steps)
def test_pages_two_box_example_as_coord_steps(O):
    """The same example as written on the page: coords (0,0), coord_steps ((8,0),) over a
    repeat axis of 2 -> boxes at (0,0) and (8,0), images in repeat order."""
    exp = np.loadtxt(os.path.join(GOLD, "tma_two_box_expected.txt"), dtype=np.uint64).astype(np.uint32)
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    assert O.repeat_coords((0, 0), (2,), ((8, 0),)).tolist() == [[0, 0], [8, 0]]
    imgs = O.box_load_steps(x, "u32", (16, 16), (64, 4), (8, 16), (1, 1), (0, 0), (2,), ((8, 0),))
    assert imgs.size == 1024                              # 512 bytes per box, two boxes
    assert np.array_equal(imgs.view(np.uint32).reshape(16, 16), exp)


def test_repeat_coords_row_major_and_steps_vs_numpy_slicing(O):
    """Two repeat axes (3 x 2), negative steps and out-of-range boxes: box t of the
    row-major repeat order equals numpy slicing at coords + j0 s0 + j1 s1."""
    rng = np.random.default_rng(9)
    x = rng.integers(0, 1 << 16, (20, 30, 40), dtype=np.uint64).astype(np.uint16)
    coords, reps, steps = (2, 5, -3), (3, 2), ((6, -4, 0), (0, 7, 16))
    rc = O.repeat_coords(coords, reps, steps)
    assert rc.tolist() == [[2 + 6 * a, 5 - 4 * a + 7 * b, -3 + 16 * b] for a in range(3) for b in range(2)]
    box = (4, 5, 16)
    imgs = O.box_load_steps(x, "u16", x.shape, x.strides, box, (1, 1, 1), coords, reps, steps, 0, 0)
    st = O.image_stride("u16", box, (1, 1, 1), 0)
    for t, c in enumerate(rc):
        want = _numpy_box(x, 0, box, (1, 1, 1), c)
        assert np.array_equal(imgs[t * st:t * st + want.nbytes].view(np.uint16).reshape(box), want)
    y = np.zeros_like(x)
    O.box_store_steps(y, "u16", x.shape, x.strides, box, (1, 1, 1), coords, reps, steps, imgs)
    z = np.zeros_like(x)
    for t, c in enumerate(rc):
        O.box_store(z, "u16", x.shape, x.strides, box, (1, 1, 1), c, imgs[t * st:(t + 1) * st])
    assert np.array_equal(y, z) and y.any()
