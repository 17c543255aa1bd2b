"""Writes the worked-example fixtures of this directory from the values the pages state.

Each fixture evaluates an expected result that a page prints as a formula or a
statement about its example; no library code is called. Run from the repo root:
    python tests/golden/make_golden.py
"""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def fragment_words(mats, trans):
    """The register image of one ldmatrix issue over n 8x8 b16 matrices ("ldmatrix / stmatrix",
    Address providers and result owners; Transpose and stores): lane 4j + w owns word w of row
    j of each matrix, i.e. halves (2w, 2w + 1) of row j, taken from the matrix or, with .trans,
    from its transpose. Returns (32 lanes, n) uint32 words, low half first."""
    n = mats.shape[0]
    out = np.zeros((32, n), np.uint64)
    for i in range(n):
        src = mats[i].T if trans else mats[i]
        for lane in range(32):
            row, word = divmod(lane, 4)
            out[lane, i] = int(src[row, 2 * word]) | (int(src[row, 2 * word + 1]) << 16)
    return out


def ldmatrix_x2():
    # "ldmatrix / stmatrix", Examples (interleaved shared rows and register slots 0, 2, 8, 10):
    # the data are 128 consecutive uint32 values in a (16, 4, 2) shared tensor; issue k reads the
    # two matrices m = 0, 1 whose eight rows are the 16-byte rows (2r + m, :, k), and the
    # register layout (2, 2, 8, 4):(8, 2, 4@lane, 1@lane) places matrix m of issue k in slot
    # 8k + 2m. Every other slot keeps the sentinel 4294966519 (int32 -777).
    x = np.arange(128, dtype=np.uint32).reshape(16, 4, 2)
    halves = x.view(np.uint16).reshape(16, 4, 2, 2)           # [row, word, issue, half]
    slots = np.full((32, 12), 4294966519, dtype=np.uint64)
    for k in range(2):
        mats = np.stack([np.stack([halves[2 * r + m, :, k, :].reshape(8) for r in range(8)]) for m in range(2)])
        words = fragment_words(mats, trans=False)
        for m in range(2):
            slots[:, 8 * k + 2 * m] = words[:, m]
    hdr = ("ldmatrix / stmatrix -- Examples: interleaved shared rows and register slots 0, 2, 8, 10.\n"
           "Input x = arange(128, uint32).reshape(16,4,2) in shared layout (16,4,2):(8,1,128);\n"
           "two ldmatrix.x2 issues. Rows: lanes 0..31; columns: the 12 register slots.\n"
           "Sentinel 4294966519 (int32 -777) marks slots the instruction must not touch.")
    np.savetxt(os.path.join(HERE, "ldmatrix_x2_expected.txt"), slots, fmt="%d", header=hdr)


def tma_two_box():
    # "cp.async.bulk.tensor / cp.reduce.async.bulk.tensor", Example: two explicit 8x16
    # boxes at (0,0) and (8,0) of a 16x16 uint32 arange; Out equals the input, and each
    # box moves 512 bytes.
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    hdr = ("cp.async.bulk.tensor -- Example: two explicit 8x16 boxes, coords (0,0) and (8,0).\n"
           "Input x = arange(256, uint32).reshape(16,16); expected Out == x; 512 bytes per box.\n"
           "Data rows below: the expected 16x16 output.")
    np.savetxt(os.path.join(HERE, "tma_two_box_expected.txt"), x, fmt="%d", header=hdr)


def add_one():
    # "Tile Operands and Execution", A Load, Compute, and Store Example:
    # a = arange(768, float32).reshape(2,32,3,4); b == a + 1.
    b = np.arange(1, 769, dtype=np.float64).reshape(64, 12)
    hdr = ("Tile Operands and Execution -- A Load, Compute, and Store Example.\n"
           "Input a = arange(768, float32).reshape(2,32,3,4); expected b = a + 1.\n"
           "Rows below: thread t = 32*warp + lane, its twelve values (three 4-word loads).")
    np.savetxt(os.path.join(HERE, "add_one_expected.txt"), b, fmt="%d", header=hdr)


if __name__ == "__main__":
    ldmatrix_x2()
    tma_two_box()
    add_one()
