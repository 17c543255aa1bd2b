"""Writes the worked-example fixtures of this directory from the values the pages state.

Each fixture evaluates an expected result that a page prints as a formula or a
statement about its example; no library code is called. Run from the repo root:
    python tests/golden/make_golden.py
"""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def ldmatrix_x2():
    # "ldmatrix / stmatrix", Examples (interleaved shared rows and register slots
    # 0, 2, 8, 10): x = arange(128) as (16,4,2) uint32; every slot holds the sentinel
    # 4294966519 except slot 8k+2m of lane l, which holds x[2(l//4)+m, l%4, k].
    x = np.arange(128, dtype=np.uint64).reshape(16, 4, 2)
    exp = np.full((32, 12), 4294966519, dtype=np.uint64)
    for lane in range(32):
        for k in range(2):
            for m in range(2):
                exp[lane, 8 * k + 2 * m] = x[2 * (lane // 4) + m, lane % 4, k]
    hdr = ("ldmatrix / stmatrix -- Examples: interleaved shared rows and register slots 0, 2, 8, 10.\n"
           "Input x = arange(128, uint32).reshape(16,4,2) in shared layout (16,4,2):(8,1,128);\n"
           "two ldmatrix.x2 issues. Rows: lanes 0..31; columns: the 12 register slots.\n"
           "Sentinel 4294966519 (int32 -777) marks slots the instruction must not touch.")
    np.savetxt(os.path.join(HERE, "ldmatrix_x2_expected.txt"), exp, fmt="%d", header=hdr)


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
