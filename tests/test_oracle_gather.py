"""Pins of the oracle's four-row gather and scatter ("cp.async.bulk.tensor /
cp.reduce.async.bulk.tensor", Gather4 and scatter4): numpy fancy indexing, the pages'
example call (uint32, a (1, 32) box, rows row, row+3, row+7, row+11: 512 bytes per issue),
and the special case of four consecutive rows, which is the oracle's (already pinned) box
load / store of a (4, width) box."""
import numpy as np
import pytest

ESZ = {"u8": 1, "u16": 2, "u32": 4, "bf16": 2, "f32": 4, "e4m3": 1}
NPT = {1: np.uint8, 2: np.uint16, 4: np.uint32}


def tensor(rng, rows, cols, dt, pitch=None):
    es = ESZ[dt]
    pitch = pitch or cols
    a = rng.integers(0, 1 << (8 * es), (rows, pitch), dtype=np.uint64).astype(NPT[es])
    return a, (rows, cols), (pitch * es, es)


def test_pages_gather4_example(O):
    """uint32, box (1, 32), rows (row, row+3, row+7, row+11): one 512-byte image holding
    those four rows."""
    x = np.arange(64 * 32, dtype=np.uint32).reshape(64, 32)
    row = 5
    rows = [row, row + 3, row + 7, row + 11]
    img = O.gather4(x, "u32", (64, 32), (128, 4), 32, 0, rows)
    assert img.nbytes == 512
    assert np.array_equal(img.view(np.uint32).reshape(4, 32), x[rows, :32])


@pytest.mark.parametrize("dt", ["u8", "bf16", "f32"])
def test_gather4_vs_numpy(O, dt):
    rng = np.random.default_rng(1)
    x, dims, st = tensor(rng, 50, 96, dt, pitch=104)
    es = ESZ[dt]
    for width, col, rows in [(16 // es * 2, 0, [3, 3, 49, 0]), (96, 0, [7, 1, 30, 12]), (16 // es, 40, [0, 2, 4, 6])]:
        img = O.gather4(x, dt, dims, st, width, col, rows)
        want = x[rows, col:col + width]
        assert np.array_equal(img.view(NPT[es])[:4 * width].reshape(4, width), want)


@pytest.mark.parametrize("fill", [0, 1])
def test_gather4_out_of_range_reads_fill(O, fill):
    rng = np.random.default_rng(2)
    x, dims, st = tensor(rng, 20, 40, "bf16", pitch=48)
    fv = np.uint16(0x7FC0 if fill else 0)
    padded = np.full((20 + 4, 40 + 64), fv, np.uint16)     # rows -1 .. 22, cols -32 .. 71
    padded[1:21, 32:72] = x[:, :40]
    for col, rows in [(-8, [-1, 0, 19, 20]), (24, [5, 22, -1, 3]), (32, [0, 1, 2, 3])]:
        img = O.gather4(x, "bf16", dims, st, 32, col, rows, fill=fill)
        want = padded[np.array(rows) + 1, col + 32:col + 64]
        assert np.array_equal(img.view(np.uint16).reshape(4, 32), want), (col, rows)


@pytest.mark.parametrize("dt,width,swz", [("bf16", 64, 3), ("u8", 64, 2), ("f32", 8, 1), ("u16", 8, 0),
                                          ("e4m3", 128, 3), ("f32", 48, 0)])
def test_gather4_consecutive_rows_is_box_load(O, dt, width, swz):
    rng = np.random.default_rng(3)
    x, dims, st = tensor(rng, 37, 300, dt, pitch=304)
    for r, c in [(0, 0), (11, 64), (34, 250), (-2, -16)]:
        a = O.gather4(x, dt, dims, st, width, c, [r, r + 1, r + 2, r + 3], swz=swz)
        b = O.box_load(x, dt, dims, st, (4, width), (1, 1), (r, c), swz=swz)
        assert np.array_equal(a, b), (r, c)


def test_scatter4_vs_numpy_and_clipping(O):
    rng = np.random.default_rng(4)
    x, dims, st = tensor(rng, 30, 64, "u16", pitch=72)
    img = rng.integers(0, 1 << 16, 4 * 32, dtype=np.uint64).astype(np.uint16)
    for col, rows in [(0, [4, 9, 2, 29]), (48, [1, 0, 30, -1]), (-8, [3, 3, 5, 7])]:
        y = x.copy()
        O.scatter4(y, "u16", dims, st, 32, col, rows, img)
        want = x.copy()
        im = img.reshape(4, 32)
        for i, r in enumerate(rows):          # later rows overwrite earlier ones
            if 0 <= r < 30:
                lo, hi = max(col, 0), min(col + 32, 64)
                want[r, lo:hi] = im[i, lo - col:hi - col]
        assert np.array_equal(y, want), (col, rows)     # pitch padding and other rows untouched


@pytest.mark.parametrize("swz,width", [(3, 64), (2, 32), (0, 100)])
def test_scatter4_consecutive_rows_is_box_store(O, swz, width):
    rng = np.random.default_rng(5)
    x, dims, st = tensor(rng, 12, 200, "bf16", pitch=208)
    img = rng.integers(0, 1 << 8, O.image_stride("bf16", (4, width), (1, 1), swz), dtype=np.uint64).astype(np.uint8)
    for r, c in [(0, 0), (9, 150), (-1, 8)]:
        a, b = x.copy(), x.copy()
        O.scatter4(a, "bf16", dims, st, width, c, [r, r + 1, r + 2, r + 3], img, swz=swz)
        O.box_store(b, "bf16", dims, st, (4, width), (1, 1), (r, c), img, swz=swz)
        assert np.array_equal(a, b), (r, c)


def test_gather_then_scatter_moves_rows(O):
    """A gather4 image scattered to other rows of a zero tensor: those rows equal the
    gathered source rows (any swizzle), the rest stays zero."""
    rng = np.random.default_rng(6)
    x, dims, st = tensor(rng, 40, 64, "bf16")
    for swz in (0, 1, 2, 3):
        w = min(64, 8 << swz) if swz else 64
        img = O.gather4(x, "bf16", dims, st, w, 0, [30, 2, 17, 5], swz=swz)
        y = np.zeros_like(x)
        O.scatter4(y, "bf16", dims, st, w, 0, [0, 39, 8, 21], img, swz=swz)
        assert np.array_equal(y[[0, 39, 8, 21], :w], x[[30, 2, 17, 5], :w])
        rest = np.ones(40, bool)
        rest[[0, 39, 8, 21]] = False
        assert not y[rest].any() and not y[:, w:].any()
