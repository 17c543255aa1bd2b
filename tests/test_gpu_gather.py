"""GPU parity: four-row gather and scatter (bsm_tile_gather4 / bsm_tile_scatter4) against the
oracle, bit for bit (copies are unique results)."""
import numpy as np
import pytest
import torch

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_like, host, say

pytestmark = pytest.mark.gpu

NPDT = {"u8": np.uint8, "u16": np.uint16, "u32": np.uint32, "bf16": np.uint16, "f32": np.uint32, "e4m3": np.uint8}


def written_mask(O, width, es, swz, stride):
    m = np.zeros(stride, bool)
    m[[O.swizzle(o, swz) for o in range(4 * width * es)]] = True
    return m


def aligned_copy(a: np.ndarray):
    """A device copy of a byte array in a 1024-byte aligned buffer (image alignment)."""
    d = dev_like(a.nbytes, 0)
    d.copy_(torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.uint8)))
    return d


def run_gather(O, mem, dtype, dims, strides, width, coords, swz, fill):
    n = len(coords)
    stride = O.image_stride(dtype, (4, width), (1, 1), swz)
    dimg = dev_like(max(n, 1) * stride, 0xA5)
    dsrc = dev(mem)
    dco = torch.from_numpy(np.ascontiguousarray(coords, np.int32).reshape(-1)).cuda()
    bsm.bsm_tile_gather4(bsm.tensor_desc(dsrc, dtype, dims, strides), bsm.box_desc((1, width), (1, 1), swz, fill),
                         dco, n, dimg)
    return host(dimg, np.uint8).reshape(-1, stride)[:n], stride


def test_gather4_pages_example(O):
    """uint32, box (1, 32), rows (row, row+3, row+7, row+11): one 512-byte image."""
    x = np.arange(64 * 32, dtype=np.uint32).reshape(64, 32)
    rows = [5, 8, 12, 16]
    say("gather4 pages example")
    got, stride = run_gather(O, x, "u32", (64, 32), (128, 4), 32, np.array([[0] + rows]), 0, 0)
    assert stride == 512
    assert np.array_equal(got[0], O.gather4(x, "u32", (64, 32), (128, 4), 32, 0, rows))
    assert np.array_equal(got[0].view(np.uint32).reshape(4, 32), x[rows])


# (dtype, width, swizzle): one chunk per row up to 64 chunks (1 KiB rows, one issue per pass),
# a 3-chunk row (ragged issues per pass), every swizzle mode
CASES = [("u8", 16, 0), ("bf16", 24, 0), ("bf16", 64, 3), ("f32", 8, 1), ("u16", 16, 2), ("e4m3", 128, 3),
         ("f32", 256, 0), ("u32", 32, 0), ("bf16", 8, 0)]


@pytest.mark.parametrize("dtype,width,swz", CASES)
def test_gather4_vs_oracle(O, dtype, width, swz):
    rng = np.random.default_rng([bsm.DTYPE[dtype], width, swz])
    es = bsm.ESIZE[dtype]
    rows, cols = 45, 3 * width + 5
    pitch = (cols * es + 15) // 16 * 16 // es + 16 // es
    mem = rng.integers(0, 1 << (8 * es), (rows, pitch), dtype=np.uint64).astype(NPDT[dtype])
    dims, strides = (rows, cols), (pitch * es, es)
    fill = int(rng.integers(0, 2)) if dtype in ("bf16", "f32", "e4m3") else 0
    n = 37   # not a multiple of the issues per workgroup: a ragged last workgroup
    coords = np.empty((n, 5), np.int32)
    coords[:, 0] = rng.integers(-width // 2, cols, n)
    coords[:, 0] = np.where(rng.random(n) < 0.6, coords[:, 0] // (16 // es) * (16 // es), coords[:, 0])
    coords[:, 1:] = rng.integers(-3, rows + 3, (n, 4))
    coords[0] = [0, 0, 1, 2, 3]
    coords[1] = [0, 7, 7, 7, 7]                          # repeated rows
    say("gather4", dtype, width, swz, fill)
    got, stride = run_gather(O, mem, dtype, dims, strides, width, coords, swz, fill)
    wm = written_mask(O, width, es, swz, stride)
    for t in range(n):
        exp = O.gather4(mem, dtype, dims, strides, width, coords[t, 0], coords[t, 1:], swz, fill)
        assert np.array_equal(got[t][wm], exp[wm]), (t, coords[t])
        assert (got[t][~wm] == 0xA5).all()


@pytest.mark.parametrize("dtype,width,swz", CASES)
def test_scatter4_vs_oracle(O, dtype, width, swz):
    """Issues write disjoint (row, column block) targets, so the result is unique; rows and
    columns out of range are clipped and every other byte keeps its sentinel."""
    rng = np.random.default_rng([7, bsm.DTYPE[dtype], width, swz])
    es = bsm.ESIZE[dtype]
    rows, nblk = 44, 3
    cols = nblk * width - 3 if width * es > 16 else nblk * width
    pitch = (cols * es + 15) // 16 * 16 // es + 16 // es
    dims, strides = (rows, cols), (pitch * es, es)
    perm = rng.permutation(rows + 8) - 4                  # includes rows -4..-1 and rows..rows+3
    coords = []
    for g in range((rows + 8) // 4):
        for b in range(nblk):
            coords.append([b * width - (width // 2 if b == 0 and g % 3 == 0 else 0)] + list(perm[4 * g:4 * g + 4]))
    coords = np.array(coords, np.int32)
    n = len(coords)
    stride = O.image_stride(dtype, (4, width), (1, 1), swz)
    images = rng.integers(0, 256, (n, stride), dtype=np.uint64).astype(np.uint8)
    sent = np.full((rows, pitch), 0x3C if es == 1 else 0x3C00, NPDT[dtype])
    dd = dev(sent)
    say("scatter4", dtype, width, swz, n)
    bsm.bsm_tile_scatter4(bsm.tensor_desc(dd, dtype, dims, strides), bsm.box_desc((1, width), (1, 1), swz, 0),
                          torch.from_numpy(coords.reshape(-1)).cuda(), n, aligned_copy(images))
    exp = sent.copy()
    for t in range(n):
        O.scatter4(exp, dtype, dims, strides, width, coords[t, 0], coords[t, 1:], images[t], swz)
    assert np.array_equal(host(dd, NPDT[dtype], (rows, pitch)), exp)


def test_gather4_empty_is_noop():
    x = torch.zeros(64 * 64, dtype=torch.uint8, device="cuda")
    say("gather4 n = 0")
    bsm.bsm_tile_gather4(bsm.tensor_desc(x, "u8", (64, 64), (64, 1)), bsm.box_desc((1, 64)), None, 0, None)
    bsm.bsm_tile_scatter4(bsm.tensor_desc(x, "u8", (64, 64), (64, 1)), bsm.box_desc((1, 64)), None, 0, None)
    torch.cuda.synchronize()
    assert not x.any()


def test_gather4_scatter4_full_size(O):
    """The 65536 x 4096 bf16 table, (1, 64) boxes, 128-byte swizzle, 1 048 576 issues (the
    timed workload): 4096 sampled issues against the oracle, every image against the table
    (numpy indexing), then the scatter to the rows of a second permutation, which must leave
    dst as the table with its rows permuted."""
    w = W.gather4_bf16()
    rows, cols, width, swz = w["rows"], w["cols"], w["width"], w["swizzle"]
    g, sc = w["gather"], w["scatter"]
    n = len(g)
    dims, strides = (rows, cols), (cols * 2, 2)
    stride = O.image_stride("bf16", (4, width), (1, 1), swz)
    assert stride == 1024          # the 512-byte image rounded to the 1024-byte swizzle period
    box = bsm.box_desc((1, width), (1, 1), swz, 0)
    dt = dev(w["table"])
    dimg = dev_like(n * stride, 0)
    say("gather4 full", rows, cols, n)
    bsm.bsm_tile_gather4(bsm.tensor_desc(dt, "bf16", dims, strides), box, torch.from_numpy(g.reshape(-1)).cuda(), n,
                         dimg)
    imgs = host(dimg, np.uint8).reshape(n, stride)
    for t in np.random.default_rng(8).integers(0, n, 4096):
        assert np.array_equal(imgs[t], O.gather4(w["table"], "bf16", dims, strides, width, g[t, 0], g[t, 1:], swz))
    unswz = np.array([O.swizzle(o, swz) for o in range(4 * width * 2)])   # compact byte o sits at unswz[o]
    # issue t = group * blocks + block holds rows perm[4 group + i], columns block * width + j
    compact = np.ascontiguousarray(imgs[:, unswz]).view(np.uint16).reshape(rows // 4, cols // width, 4, width)
    assert np.array_equal(compact.transpose(0, 2, 1, 3).reshape(rows, cols), w["table"][w["perm_gather"]])
    del compact
    dd = dev_like(rows * cols * 2, 0)
    say("scatter4 full", rows, cols, n)
    bsm.bsm_tile_scatter4(bsm.tensor_desc(dd, "bf16", dims, strides), box, torch.from_numpy(sc.reshape(-1)).cuda(), n,
                          dimg)
    got = host(dd, np.uint16, (rows, cols))
    exp = np.empty_like(w["table"])
    exp[w["perm_scatter"]] = w["table"][w["perm_gather"]]
    assert np.array_equal(got, exp)
