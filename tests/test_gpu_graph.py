"""GPU: the library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point only enqueues kernels on the caller's stream (no allocation, no memset, no
synchronisation), so a sequence of calls can be captured once and replayed. The test runs one
small pass of the hot path eagerly, captures the same calls, and replays the graph several
times with eager work and synchronisations between the replays (the accumulating targets are
reset and the fresh outputs poisoned with NaN or a sentinel before each replay); every replay
must reproduce the eager outputs bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import block_scaled_matrix_amd as bsm
from block_scaled_matrix_amd import workloads as W
from gpu_util import dev, dev_f32, dev_like, say
from test_gpu_gemm import dense_case, mx_case

pytestmark = pytest.mark.gpu


def _pass():
    """Device inputs and outputs for one small pass, and the list of calls making it."""
    rng = np.random.default_rng(77)
    t = {}
    # box copy: 300 x 190 bf16 (192-element pitch), (128, 64) boxes, 128-byte swizzle, store + reduce-add
    rows, cols, pitch = 300, 190, 192
    src = np.full((rows, pitch), W.SENTINEL_BF16, np.uint16)
    src[:, :cols] = W.to_half_bits(rng.standard_normal((rows, cols)).astype(np.float32), "bf16")
    add = np.full((rows, pitch), W.SENTINEL_BF16, np.uint16)
    add[:, :cols] = W.to_half_bits(rng.standard_normal((rows, cols)).astype(np.float32), "bf16")
    t["src"], t["add0"] = dev(src), dev(add)
    t["dst"], t["add"] = dev(np.full((rows, pitch), W.SENTINEL_BF16, np.uint16)), dev(add)
    st = (pitch * 2, 2)
    td = lambda x: bsm.tensor_desc(x, "bf16", (rows, cols), st)
    box = bsm.box_desc((128, 64), (1, 1), 3, 0)
    # general box load: rank 3 with an element stride, out-of-range boxes filled with NaN
    x3 = rng.standard_normal((4, 40, 64)).astype(np.float32)
    t["x3"] = dev(W.to_half_bits(x3, "bf16"))
    t3 = bsm.tensor_desc(t["x3"], "bf16", (4, 40, 64), (40 * 64 * 2, 64 * 2, 2))
    bx3 = bsm.box_desc((2, 16, 32), (1, 2, 1), 0, 1)
    coords = np.array([[0, 0, 0], [3, 32, 48], [-1, 8, 16]], np.int32)
    t["coords"] = dev(coords)
    n_img = coords.shape[0]
    istride = bsm.bsm_image_stride(bx3, "bf16")
    t["img"] = dev_like(n_img * istride, 0xA5)
    # dense bf16 GEMM, A K-major, B MN-major, accumulating onto D
    M, N, K = 384, 320, 192
    A, lda, B, ldb = dense_case(rng, M, N, K, "bf16", "k", "n")
    t["A"], t["B"] = dev(A), dev(B)
    t["D0"] = dev_f32(rng.standard_normal((M, N)).astype(np.float32))
    t["D"] = t["D0"].clone()
    # block-scaled: MXFP8 (exact-products route) and MXFP4 (scaled MFMA) with negation
    g8 = mx_case("e4m3", 78, 256, 192, 512)
    g4 = mx_case("e2m1", 79, 320, 256, 512, exp_range=6)
    for key, g in (("f8", g8), ("f4", g4)):
        for part in ("A", "B", "SFA", "SFB"):
            t[f"{key}{part}"] = dev(g[part])
    t["D8"] = torch.empty((256, 192), dtype=torch.float32, device="cuda")
    t["D4"] = torch.empty((320, 256), dtype=torch.float32, device="cuda")

    def calls():
        bsm.bsm_tile_box_copy(td(t["src"]), td(t["dst"]), td(t["add"]), box)
        bsm.bsm_tile_box_load(t3, bx3, t["coords"], n_img, t["img"])
        bsm.bsm_gemm(M, N, K, "bf16", t["A"], lda, "k", t["B"], ldb, "n", t["D"], N, 0, 0, 1)
        bsm.bsm_gemm_block_scale(256, 192, 512, "e4m3", t["f8A"], g8["lda"], t["f8SFA"], g8["ld_sfa"], "e4m3",
                                 t["f8B"], g8["ldb"], t["f8SFB"], g8["ld_sfb"], t["D8"], 192, 0, 0, 0)
        bsm.bsm_gemm_block_scale(320, 256, 512, "e2m1", t["f4A"], g4["lda"], t["f4SFA"], g4["ld_sfa"], "e2m1",
                                 t["f4B"], g4["ldb"], t["f4SFB"], g4["ld_sfb"], t["D4"], 256, 1, 0, 0)

    def reset():
        """Eager work between passes: accumulating targets back to their inputs, fresh outputs poisoned."""
        t["add"].copy_(t["add0"])
        t["D"].copy_(t["D0"])
        t["dst"].fill_(0xFF)
        t["img"].fill_(0x5A)
        t["D8"].fill_(float("nan"))
        t["D4"].fill_(float("nan"))

    outs = lambda: [t[k].clone() for k in ("dst", "add", "img", "D", "D8", "D4")]
    return calls, reset, outs


def test_graph_replays_match_eager():
    say("graph capture: box copy, box load, bf16 GEMM, MXFP8, MXFP4")
    calls, reset, outs = _pass()
    reset()
    calls()
    torch.cuda.synchronize()
    eager = outs()
    assert not any(torch.isnan(x).any() for x in eager[3:]), "eager outputs hold NaN"

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            calls()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs()
        for name, e, g in zip(("dst", "add", "img", "D", "D8", "D4"), eager, got):
            assert torch.equal(e.view(torch.uint8), g.view(torch.uint8)), f"replay {rep}: {name} differs from eager"
        # eager work between the replays, on the same buffers
        calls()
        torch.cuda.synchronize()
