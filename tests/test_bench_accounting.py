"""The benchmark's accounting, on hand-worked cases (no GPU): algorithmic bytes
of a matrix at prefix k (planes 0..k-1 plus the depth-k table of every block),
of a B > 1 call (every distinct expert once, to its largest prefix, one table
per distinct prefix), and the useful and issued flops of the matrix-core
tiles (16 uses per tile)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import synth  # noqa: E402

WL = synth.WORKLOADS[1]          # hidden 4096, inter 1024, group 128


def mat(r, c, kmax, ks):
    return r * c * kmax // 8 + sum(r * (c // 128) * (1 << k) * 4 for k in ks)


def test_matrix_bytes_by_k():
    # 1024 x 4096 at k = 2: 1 MiB of planes, 1024 * 32 blocks * 4 nodes * 4 B
    assert bench.matrix_bytes(1024, 4096, 128, 2) == 1048576 + 524288
    # bytes per weight at group 128 (k/8 + 2^k * 4 / 128)
    for k, bpw in zip(range(1, 9), (0.1875, 0.375, 0.625, 1.0, 1.625, 2.75, 4.875, 9.0)):
        assert bench.matrix_bytes(1024, 4096, 128, k) == int(bpw * 1024 * 4096)


def test_grouped_bytes_counts_each_expert_once():
    shapes = ((1024, 4096), (1024, 4096), (4096, 1024))
    ids = np.array([[0, 1], [0, 2]])
    k3 = np.array([[[2, 2, 2], [3, 3, 3]], [[4, 4, 4], [1, 1, 1]]])
    want = sum(mat(r, c, 4, [2, 4]) for r, c in shapes)     # expert 0: k 2 and 4
    want += sum(mat(r, c, 3, [3]) for r, c in shapes)       # expert 1
    want += sum(mat(r, c, 1, [1]) for r, c in shapes)       # expert 2
    want += 2 * 2 * 4096 * 4                                # x and y of 2 tokens
    assert bench.grouped_bytes(WL, ids, k3) == want
    # a single token is the per-token sum
    assert bench.grouped_bytes(WL, ids[:1], k3[:1]) == bench.step_bytes(WL, k3[0])


def test_mfma_flops_tiles_of_sixteen():
    W = 1024 * 4096
    ids = np.zeros((20, 1), np.int64)               # one expert, 20 uses
    k3 = np.full((20, 1, 3), 2)
    k3[:3, 0, 1] = 5                                # up: 17 at k 2, 3 at k 5
    useful, issued = bench.mfma_flops(WL, ids, k3)
    assert useful == 3 * 2 * W * 20
    # gate: 20 uses -> 2 tiles; up: 17 + 3 -> 2 + 1; down: 2
    assert issued == 2 * W * 16 * (2 + 3 + 2)


def test_cpu_sample_counts_each_matrix_by_its_own_rows():
    # 256 rows of gate and up (1024 rows each) and of down (4096 rows): one
    # expert's pass is (1/4 + 1/4 + 1/16) of three matrices' worth
    wl = synth.WORKLOADS[1]
    assert abs(3 * bench.gemv_share(wl, 256) - (0.25 + 0.25 + 0.0625)) < 1e-12
    assert bench.gemv_share(wl, 4096) == 1.0
