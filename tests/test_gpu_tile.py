"""GPU parity: add-scalar tile and box load / store / reduce-add / grid copy vs the oracle.

Copies and images are compared bit for bit (they are unique results); the
add-reduction is compared bit for bit too (one rounding of the exact sum).
"""
import numpy as np
import pytest
import torch

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_like, host, say

pytestmark = pytest.mark.gpu

NPDT = {"u8": np.uint8, "u16": np.uint16, "u32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "f32": np.uint32,
        "e4m3": np.uint8, "e5m2": np.uint8}


def test_add_one_pages_example(O):
    say("add_one (2,32,3,4)")
    a = W.add_one_tile()
    da = torch.from_numpy(a).cuda()
    db = torch.empty_like(da)
    bsm.bsm_tile_add_scalar_f32(da, db, a.size, 1.0)
    got = db.cpu().numpy()
    assert np.array_equal(got, O.add_scalar_f32(a, 1.0))
    assert np.array_equal(got, np.arange(1, 769, dtype=np.float32).reshape(2, 32, 3, 4))


@pytest.mark.parametrize("n", [1, 3, 4, 767, 768, 769, 1000, 12345, 1 << 20])
def test_add_scalar_ragged(O, n):
    say("add_scalar n", n)
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    dx = torch.from_numpy(x).cuda()
    out = torch.full((n + 8,), 7.0, device="cuda")
    bsm.bsm_tile_add_scalar_f32(dx, out, n, -0.75)
    got = out.cpu().numpy()
    assert np.array_equal(got[:n].view(np.uint32), O.add_scalar_f32(x, -0.75).view(np.uint32))
    assert (got[n:] == 7.0).all()
    bsm.bsm_tile_add_scalar_f32(dx, dx, n, 1.0)   # in place
    assert np.array_equal(dx.cpu().numpy(), O.add_scalar_f32(x, 1.0))


def _rand_case(rng, rank, dtype):
    esz = bsm.ESIZE[dtype]
    dims = tuple(int(v) for v in rng.integers(1, 40 if rank <= 3 else 12, rank))
    inner_box = (16 // esz) * int(rng.integers(1, 9))
    box = tuple(int(v) for v in rng.integers(1, 10 if rank <= 3 else 4, rank - 1)) + (min(inner_box, 256),)
    estr = tuple(int(v) for v in rng.integers(1, 4, rank - 1)) + (1,)
    swz = int(rng.integers(0, 4))
    if swz and box[-1] * esz > (16 << swz):
        swz = 0
    pitch_b = (dims[-1] * esz + 15) // 16 * 16 + 16 * int(rng.integers(0, 3))
    shape = dims[:-1] + (pitch_b // esz,)
    mem = rng.integers(0, 2 ** (8 * esz), shape, dtype=np.uint64).astype(NPDT[dtype])
    strides = [mem.strides[i] for i in range(rank)]
    return dims, box, estr, swz, mem, strides


@pytest.mark.parametrize("dtype", ["u8", "bf16", "f32", "e5m2", "e4m3"])
@pytest.mark.parametrize("rank", [1, 2, 3, 5])
def test_box_load_store_vs_oracle(O, dtype, rank):
    rng = np.random.default_rng(1000 * rank + bsm.DTYPE[dtype])
    for trial in range(6):
        dims, box, estr, swz, mem, strides = _rand_case(rng, rank, dtype)
        fill = int(rng.integers(0, 2)) if dtype != "u8" else 0
        nb = 7
        coords = rng.integers(-12, 45, (nb, rank)).astype(np.int32)
        if trial == 0:
            coords[:] = 0
        say("box_load", dtype, rank, dims, box, estr, swz, fill)
        stride = O.image_stride(dtype, box, estr, swz)
        dsrc = dev(mem)
        dimg = dev_like(nb * stride, 0xA5)
        dco = torch.from_numpy(coords.reshape(-1)).cuda()
        td = bsm.tensor_desc(dsrc, dtype, dims, strides)
        bd = bsm.box_desc(box, estr, swz, fill)
        assert bsm.bsm_image_stride(bd, dtype) == stride
        bsm.bsm_tile_box_load(td, bd, dco, nb, dimg)
        got = host(dimg, np.uint8).reshape(nb, stride)
        nbytes = int(np.prod(O.image_extents(box, estr))) * bsm.ESIZE[dtype]
        for t in range(nb):
            exp = O.box_load(mem, dtype, dims, strides, box, estr, coords[t], swz, fill)
            written = np.zeros(stride, bool)
            written[[O.swizzle(o, swz) for o in range(nbytes)]] = True
            assert np.array_equal(got[t][written], exp[written]), (t, coords[t])
            assert (got[t][~written] == 0xA5).all()
        # store the images back into a sentinel-filled tensor; reduce-add into a second one
        say("box_store", dtype, rank)
        sent = np.full_like(mem, 0x3C if bsm.ESIZE[dtype] == 1 else 0x3C00)
        dst = dev(sent)
        bsm.bsm_tile_box_store(bsm.tensor_desc(dst, dtype, dims, strides), bd, dco, nb, dimg, 0)
        exp = sent.copy()
        for t in range(nb):
            O.box_store(exp, dtype, dims, strides, box, estr, coords[t], got[t], swz, 0)
        assert np.array_equal(host(dst, NPDT[dtype], mem.shape), exp)


# The contract's limits: box extents up to 256, element strides up to 8 (outer dimensions),
# an inner box of 16 << s bytes when swizzled, and an unswizzled (256, 256) bf16 box whose
# 128 KiB image is the largest the general kernel stages in LDS.
LIMIT_CASES = [
    ("bf16", (1000, 300), (256, 256), (1, 1), 0),
    ("f32", (2100, 40), (256, 32), (8, 1), 3),
    ("u8", (40, 9, 600), (5, 256, 64), (8, 1, 1), 2),
    ("e4m3", (3, 4, 5, 6, 300), (2, 3, 2, 3, 256), (2, 1, 3, 1, 1), 0),
    ("f16", (7, 5, 4, 33, 70), (4, 4, 4, 8, 64), (8, 2, 8, 4, 1), 3),
]


@pytest.mark.parametrize("dtype,dims,box,estr,swz", LIMIT_CASES)
def test_box_limits_vs_oracle(O, dtype, dims, box, estr, swz):
    """Boxes at the contract's limits, loaded at coordinates inside, straddling and past the
    tensor (zero and, for float formats, NaN fill), then stored and add-reduced back."""
    rng = np.random.default_rng(sum(dims) + 7 * sum(box))
    esz = bsm.ESIZE[dtype]
    rank = len(dims)
    pitch_b = (dims[-1] * esz + 15) // 16 * 16 + 16
    mem = rng.integers(0, 2 ** (8 * esz), dims[:-1] + (pitch_b // esz,), dtype=np.uint64).astype(NPDT[dtype])
    if dtype in ("f32", "f16", "bf16"):   # finite values, so that the reduce-add sums are defined
        mem = W.to_half_bits(rng.standard_normal(mem.shape).astype(np.float32), dtype) if esz == 2 else \
            rng.standard_normal(mem.shape).astype(np.float32).view(np.uint32)
    strides = [mem.strides[i] for i in range(rank)]
    ext = O.image_extents(box, estr)
    coords = np.array([[0] * rank,
                       [d - (b - 1) * e // 2 for d, b, e in zip(dims, box, estr)],
                       [-(b - 1) * e // 2 for b, e in zip(box, estr)],
                       [d + 1 for d in dims]], np.int32)
    nb = len(coords)
    fill = 1 if dtype in ("f32", "f16", "bf16", "e4m3") else 0
    say("box limits", dtype, dims, box, estr, swz, fill, "image", int(np.prod(ext)) * esz)
    stride = O.image_stride(dtype, box, estr, swz)
    bd = bsm.box_desc(box, estr, swz, fill)
    assert bsm.bsm_image_stride(bd, dtype) == stride
    dsrc = dev(mem)
    dimg = dev_like(nb * stride, 0xA5)
    dco = torch.from_numpy(coords.reshape(-1)).cuda()
    bsm.bsm_tile_box_load(bsm.tensor_desc(dsrc, dtype, dims, strides), bd, dco, nb, dimg)
    got = host(dimg, np.uint8).reshape(nb, stride)
    nbytes = int(np.prod(ext)) * esz
    written = np.zeros(stride, bool)
    written[[O.swizzle(o, swz) for o in range(nbytes)]] = True
    for t in range(nb):
        exp = O.box_load(mem, dtype, dims, strides, box, estr, coords[t], swz, fill)
        assert np.array_equal(got[t][written], exp[written]), (t, coords[t])
        assert (got[t][~written] == 0xA5).all()
    # store every image back into a sentinel tensor (clipped; overlapping boxes carry the same
    # source values there), then reduce-add the straddling box's image into a copy of the
    # source (one box: overlapping reduce-adds would race)
    say("box limits store", dtype)
    sent = np.full_like(mem, 0x3C if esz == 1 else 0x3C00)
    dst = dev(sent)
    bsm.bsm_tile_box_store(bsm.tensor_desc(dst, dtype, dims, strides), bd, dco, nb, dimg, 0)
    exp = sent.copy()
    for t in range(nb):
        O.box_store(exp, dtype, dims, strides, box, estr, coords[t], got[t], swz, 0)
    assert np.array_equal(host(dst, NPDT[dtype], mem.shape), exp)
    if dtype in ("f32", "f16", "bf16"):
        say("box limits reduce-add", dtype)
        dacc = dev(mem)
        d1 = torch.from_numpy(coords[1].copy()).cuda()
        bsm.bsm_tile_box_store(bsm.tensor_desc(dacc, dtype, dims, strides), bd, d1, 1, dimg[stride:2 * stride], 1)
        exp = mem.copy()
        O.box_store(exp, dtype, dims, strides, box, estr, coords[1], got[1], swz, 1)
        assert np.array_equal(host(dacc, NPDT[dtype], mem.shape), exp)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_box_reduce_add_vs_oracle(O, dtype):
    rng = np.random.default_rng(77 + bsm.DTYPE[dtype])
    esz = bsm.ESIZE[dtype]
    rows, cols = 70, 100
    pitch = (cols * esz + 31) // 16 * 16 // esz
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    ib = torch.int32 if dtype == "f32" else torch.int16

    def bits(x):
        m = np.zeros((rows, pitch), NPDT[dtype])
        m[:, :cols] = torch.from_numpy(x).to(tdt).view(ib).numpy().view(NPDT[dtype])
        return m

    src = bits(rng.standard_normal((rows, cols)).astype(np.float32))
    acc = bits((rng.standard_normal((rows, cols)) * 4).astype(np.float32))
    box = (16, 128 // esz)
    coords = np.array([[r, c] for r in range(-8, rows, 16) for c in range(-24, cols, box[1])], np.int32)
    coords = coords[(coords[:, 0] % 16 == 8) & ((coords[:, 1] + 24) % box[1] == 0)]  # non-overlapping grid
    nb = len(coords)
    strides = (pitch * esz, esz)
    stride = O.image_stride(dtype, box, (1, 1), 3)
    say("reduce_add", dtype, nb)
    dsrc, dacc = dev(src), dev(acc)
    dimg = dev_like(nb * stride)
    dco = torch.from_numpy(coords.reshape(-1)).cuda()
    bd = bsm.box_desc(box, (1, 1), 3, 0)
    bsm.bsm_tile_box_load(bsm.tensor_desc(dsrc, dtype, (rows, cols), strides), bd, dco, nb, dimg)
    bsm.bsm_tile_box_store(bsm.tensor_desc(dacc, dtype, (rows, cols), strides), bd, dco, nb, dimg, 1)
    imgs = host(dimg, np.uint8).reshape(nb, stride)
    exp = acc.copy()
    for t in range(nb):
        O.box_store(exp, dtype, (rows, cols), strides, box, (1, 1), coords[t], imgs[t], 3, 1)
    assert np.array_equal(host(dacc, NPDT[dtype], acc.shape), exp)


def _copy_case(O, rows, cols, pitch, box, swz, seed):
    rng = np.random.default_rng(seed)
    src = np.full((rows, pitch), W.SENTINEL_BF16, np.uint16)
    src[:, :cols] = W.to_half_bits(rng.standard_normal((rows, cols)).astype(np.float32), "bf16")
    add = np.full((rows, pitch), W.SENTINEL_BF16, np.uint16)
    add[:, :cols] = W.to_half_bits(rng.standard_normal((rows, cols)).astype(np.float32), "bf16")
    dst = np.full((rows, pitch), W.SENTINEL_BF16, np.uint16)
    return src, dst, add


@pytest.mark.parametrize("rows,cols,pitch,box,swz", [
    (45, 70, 72, (16, 32), 2), (128, 64, 64, (128, 64), 3), (300, 190, 192, (128, 64), 3),
    (257, 8190 // 8, 1024, (128, 64), 3), (33, 17, 24, (8, 8), 0), (9, 9, 16, (4, 8), 0), (130, 196, 200, (128, 64), 3)])
def test_box_copy_grid_vs_oracle(O, rows, cols, pitch, box, swz):
    src, dst, add = _copy_case(O, rows, cols, pitch, box, swz, rows)
    say("box_copy", rows, cols, pitch, box, swz)
    ds, dd, da = dev(src), dev(dst), dev(add)
    st = (pitch * 2, 2)
    bsm.bsm_tile_box_copy(bsm.tensor_desc(ds, "bf16", (rows, cols), st), bsm.tensor_desc(dd, "bf16", (rows, cols), st),
                          bsm.tensor_desc(da, "bf16", (rows, cols), st), bsm.box_desc(box, (1, 1), swz, 0))
    O.box_copy_grid(src, dst, add, "bf16", (rows, cols), st, box, (1, 1), swz, 0)
    assert np.array_equal(host(dd, np.uint16, dst.shape), dst)
    assert np.array_equal(host(da, np.uint16, add.shape), add)


_NP = {"u8": np.uint8, "f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}


@pytest.mark.parametrize("dtype,rows,cols,pitch,box,swz,mode", [
    ("u8", 70, 77, 96, (32, 64), 0, "copy"),      # straddling tail of 13 bytes: 8 + 4 + 1
    ("u8", 40, 35, 48, (16, 32), 1, "copy"),      # 3 bytes: 2 + 1
    ("f16", 50, 91, 104, (32, 64), 3, "both"),    # 6 bytes: 4 + 2
    ("f32", 33, 45, 48, (16, 32), 3, "add"),      # 4 bytes, reduce-add only
    ("f32", 66, 43, 48, (64, 16), 2, "both"),     # 12 bytes: 8 + 4
    ("bf16", 20, 63, 64, (16, 64), 3, "copy")])   # 14 bytes: 8 + 4 + 2
def test_box_copy_grid_dtypes_vs_oracle(O, dtype, rows, cols, pitch, box, swz, mode):
    """Rank-2 grid round trips over element types and ragged rows whose last 16-byte chunk is
    cut at every width the head stores handle; the row padding holds a sentinel that must stay."""
    rng = np.random.default_rng(rows * 1000 + cols)
    t = _NP[dtype]
    es = np.dtype(t).itemsize

    def tensor(fill):
        a = np.full((rows, pitch), fill, t)
        if dtype == "u8":
            a[:, :cols] = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
        elif dtype == "f32":
            a[:, :cols] = rng.standard_normal((rows, cols)).astype(np.float32).view(np.uint32)
        else:
            a[:, :cols] = W.to_half_bits(rng.standard_normal((rows, cols)).astype(np.float32), dtype)
        return a

    sentinel = {"u8": 0xA5, "f16": 0x7E01, "bf16": W.SENTINEL_BF16, "f32": 0x7FC00123}[dtype]
    src = tensor(sentinel)
    dst = np.full((rows, pitch), sentinel, t) if mode in ("copy", "both") else None
    add = tensor(sentinel) if mode in ("add", "both") else None
    say("box_copy dtypes", dtype, rows, cols, pitch, box, swz, mode)
    st = (pitch * es, es)
    ds = dev(src)
    dd = dev(dst) if dst is not None else None
    da = dev(add) if add is not None else None
    desc = lambda x: bsm.tensor_desc(x, dtype, (rows, cols), st) if x is not None else None
    bsm.bsm_tile_box_copy(desc(ds), desc(dd), desc(da), bsm.box_desc(box, (1, 1), swz, 0))
    O.box_copy_grid(src, dst, add, dtype, (rows, cols), st, box, (1, 1), swz, 0)
    if dst is not None:
        assert np.array_equal(host(dd, t, dst.shape), dst)
    if add is not None:
        assert np.array_equal(host(da, t, add.shape), add)


@pytest.mark.parametrize("mode", ["both", "copy", "add"])
def test_box_copy_full_size_vs_oracle(O, mode):
    """The 16381 x 8190 bf16 workload (8192-element pitch, (128,64) boxes, 128-byte swizzle): the
    fused store + reduce-add call, and the store alone and the reduce-add alone (each its own
    kernel)."""
    w = W.box_copy_bf16()
    rows, cols, pitch = w["rows"], w["cols"], w["pitch"]
    say("box_copy full", rows, cols, mode)
    st = (pitch * 2, 2)
    dst = w["dst"] if mode in ("both", "copy") else None
    add = w["dst_add"] if mode in ("both", "add") else None
    ds = dev(w["src"])
    dd = dev(dst) if dst is not None else None
    da = dev(add) if add is not None else None
    desc = lambda x: bsm.tensor_desc(x, "bf16", (rows, cols), st) if x is not None else None
    bsm.bsm_tile_box_copy(desc(ds), desc(dd), desc(da), bsm.box_desc(w["box"], (1, 1), 3, 0))
    got_d = host(dd, np.uint16, (rows, pitch)) if dd is not None else None
    got_a = host(da, np.uint16, (rows, pitch)) if da is not None else None
    O.box_copy_grid(w["src"], dst, add, "bf16", (rows, cols), st, w["box"], (1, 1), 3, 0)
    if dst is not None:
        assert np.array_equal(got_d, dst)
        assert np.array_equal(got_d[:, :cols], w["src"][:, :cols]) and (got_d[:, cols:] == W.SENTINEL_BF16).all()
    if add is not None:
        assert np.array_equal(got_a, add)


# ----------------------------------------------------------------------------- repeat axes
def test_box_load_steps_pages_example(O):
    """cp.async.bulk.tensor, Example: two explicit 8x16 boxes, written as on the page: coords
    (0, 0), coord_steps ((8, 0),) over one repeat axis of 2."""
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    say("box_load_steps pages example")
    dimg = dev_like(1024, 0xA5)
    bsm.bsm_tile_box_load_steps(bsm.tensor_desc(dev(x), "u32", (16, 16), (64, 4)), bsm.box_desc((8, 16)), (0, 0), (2,),
                                [(8, 0)], dimg)
    got = host(dimg, np.uint8)
    assert np.array_equal(got, O.box_load_steps(x, "u32", (16, 16), (64, 4), (8, 16), (1, 1), (0, 0), (2,), [(8, 0)]))
    assert np.array_equal(got.view(np.uint32).reshape(16, 16), x)


@pytest.mark.parametrize("dtype,swz", [("bf16", 3), ("u8", 0), ("f32", 1), ("e4m3", 2)])
def test_box_steps_vs_oracle(O, dtype, swz):
    """Rank 3, two repeat axes (3 x 4) with negative and zero steps, boxes partly out of range:
    images against the oracle; then the images stored back with the same repeats."""
    rng = np.random.default_rng([11, bsm.DTYPE[dtype], swz])
    esz = bsm.ESIZE[dtype]
    inner = {0: 48 // esz, 1: 32 // esz, 2: 64 // esz, 3: 128 // esz}[swz]
    dims = (9, 23, 3 * inner + 5)
    pitch = (dims[2] * esz + 15) // 16 * 16 // esz + 16 // esz
    mem = rng.integers(0, 1 << (8 * esz), (dims[0], dims[1], pitch), dtype=np.uint64).astype(NPDT[dtype])
    strides = (mem.strides[0], mem.strides[1], esz)
    box, estr = (2, 5, inner), (1, 2, 1)
    coords, reps, steps = (-1, 3, inner - 3), (3, 4), [(3, -2, 0), (0, 6, inner)]
    fill = 1 if dtype in ("bf16", "f32", "e4m3") else 0
    stride = O.image_stride(dtype, box, estr, swz)
    n = 12
    say("box_load_steps", dtype, swz, dims, box, reps)
    dimg = dev_like(n * stride, 0xA5)
    td = bsm.tensor_desc(dev(mem), dtype, dims, strides)
    bd = bsm.box_desc(box, estr, swz, fill)
    bsm.bsm_tile_box_load_steps(td, bd, coords, reps, steps, dimg)
    got = host(dimg, np.uint8).reshape(n, stride)
    exp = O.box_load_steps(mem, dtype, dims, strides, box, estr, coords, reps, steps, swz, fill).reshape(n, stride)
    nbytes = int(np.prod(O.image_extents(box, estr))) * esz
    written = np.zeros(stride, bool)
    written[[O.swizzle(o, swz) for o in range(nbytes)]] = True
    assert np.array_equal(got[:, written], exp[:, written])
    assert (got[:, ~written] == 0xA5).all()
    # store back into a sentinel tensor (boxes overlap: equal bytes wherever they do, since
    # every image came from the same source)
    say("box_store_steps", dtype, swz)
    sent = np.full_like(mem, 0x3C if esz == 1 else 0x3C00)
    dd = dev(sent)
    bsm.bsm_tile_box_store_steps(bsm.tensor_desc(dd, dtype, dims, strides), bd, coords, reps, steps, dimg)
    want = sent.copy()
    O.box_store_steps(want, dtype, dims, strides, box, estr, coords, reps, steps, got, swz)
    assert np.array_equal(host(dd, NPDT[dtype], mem.shape), want)


@pytest.mark.parametrize("dtype,swz,rank", [("bf16", 3, 3), ("u8", 0, 3), ("f32", 1, 2), ("e4m3", 2, 3),
                                            ("bf16", 3, 1)])
def test_box_load_steps_adjacent_runs(O, dtype, swz, rank):
    """Repeat axes whose last axis steps by exactly the box width along the innermost
    dimension (boxes side by side, loaded in runs of up to eight per workgroup): 11 boxes per
    repeat row (a partial run), the first and last boxes partly out of range, element
    stride 2 on an outer axis; images against the oracle."""
    rng = np.random.default_rng([13, bsm.DTYPE[dtype], swz, rank])
    esz = bsm.ESIZE[dtype]
    inner = {0: 48 // esz, 1: 32 // esz, 2: 64 // esz, 3: 128 // esz}[swz]
    full = (5, 21, 10 * inner + 7)[3 - rank:]
    pitch = (full[-1] * esz + 15) // 16 * 16 // esz + 16 // esz
    mem = rng.integers(0, 1 << (8 * esz), full[:-1] + (pitch,), dtype=np.uint64).astype(NPDT[dtype])
    strides = tuple(mem.strides[:-1]) + (esz,)
    box, estr = ((2, 6, inner)[3 - rank:], (1, 2, 1)[3 - rank:])
    coords = (-1, 4, -(inner // 2))[3 - rank:]
    reps = (3, 11)[max(0, 2 - rank):] if rank > 1 else (11,)
    steps = ([(2, 0, 0), (0, 0, inner)] if rank == 3 else [(5, 0), (0, inner)]) if rank > 1 else [(inner,)]
    fill = 1 if dtype in ("bf16", "f32", "e4m3") else 0
    stride = O.image_stride(dtype, box, estr, swz)
    n = int(np.prod(reps))
    say("box_load_steps adjacent", dtype, swz, full, box, reps)
    dimg = dev_like(n * stride, 0xA5)
    bsm.bsm_tile_box_load_steps(bsm.tensor_desc(dev(mem), dtype, full, strides), bsm.box_desc(box, estr, swz, fill),
                                coords, reps, steps, dimg)
    got = host(dimg, np.uint8).reshape(n, stride)
    exp = O.box_load_steps(mem, dtype, full, strides, box, estr, coords, reps, steps, swz, fill).reshape(n, stride)
    nbytes = int(np.prod(O.image_extents(box, estr))) * esz
    written = np.zeros(stride, bool)
    written[[O.swizzle(o, swz) for o in range(nbytes)]] = True
    assert np.array_equal(got[:, written], exp[:, written])
    assert (got[:, ~written] == 0xA5).all()


def test_box_store_steps_reduce_add(O):
    """Add-reduction with repeat axes onto disjoint boxes (a 3 x 2 grid of (16, 32) bf16 boxes)."""
    rng = np.random.default_rng(12)
    dims = (48, 64)
    base = W.to_half_bits(rng.standard_normal(dims).astype(np.float32), "bf16")
    box = (16, 32)
    stride = O.image_stride("bf16", box, (1, 1), 3)
    imgs = W.to_half_bits(rng.standard_normal(6 * stride // 2).astype(np.float32), "bf16").view(np.uint8)
    say("box_store_steps reduce")
    dd = dev(base)
    dimg = dev_like(6 * stride, 0)
    dimg.copy_(torch.from_numpy(imgs.copy()))
    bsm.bsm_tile_box_store_steps(bsm.tensor_desc(dd, "bf16", dims, (128, 2)), bsm.box_desc(box, (1, 1), 3, 0), (0, 0),
                                 (3, 2), [(16, 0), (0, 32)], dimg, 1)
    want = base.copy()
    O.box_store_steps(want, "bf16", dims, (128, 2), box, (1, 1), (0, 0), (3, 2), [(16, 0), (0, 32)], imgs, 3, 1)
    assert np.array_equal(host(dd, np.uint16, dims), want)


def test_box_load_steps_rank3_full_size(O):
    """The timed rank-3 workload: a bf16 (64, 2048, 2048) tensor tiled by (2, 64, 128) boxes at
    element strides (1, 2, 1) through repeat axes (32 x 32 x 16 boxes): 256 sampled boxes
    against the oracle, every image against numpy slicing of the tensor."""
    w = W.box_rank3_bf16()
    x, dims, box, estr = w["x"], w["dims"], w["box"], w["estr"]
    strides = (dims[1] * dims[2] * 2, dims[2] * 2, 2)
    bd = bsm.box_desc(box, estr, 0, 0)
    stride = bsm.bsm_image_stride(bd, "bf16")
    reps = w["repeats"]
    n = int(np.prod(reps))
    say("box_load_steps rank3 full", dims, box, estr, n)
    dimg = dev_like(n * stride, 0)
    bsm.bsm_tile_box_load_steps(bsm.tensor_desc(dev(x), "bf16", dims, strides), bd, w["coords"], reps, w["steps"], dimg)
    got = host(dimg, np.uint8).reshape(n, stride)
    rc = O.repeat_coords(w["coords"], reps, w["steps"])
    for t in np.random.default_rng(3).integers(0, n, 256):
        assert np.array_equal(got[t], O.box_load(x, "bf16", dims, strides, box, estr, rc[t])), t
    # image (a, b, c) = x[2a:2a+2, 64b:64b+64:2, 128c:128c+128], row-major over (a, b, c)
    v = x.reshape(reps[0], 2, reps[1], 32, 2, reps[2], 128)[:, :, :, :, 0, :, :]
    want = np.ascontiguousarray(v.transpose(0, 2, 4, 1, 3, 5)).reshape(n, -1)
    assert np.array_equal(got.view(np.uint16), want)
