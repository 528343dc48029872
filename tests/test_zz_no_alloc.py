"""pm_expert_gemv_noalloc, the GEMV entry point that allocates nothing (its
slice partials in a fixed per-device array), against pm_expert_gemv through
the C ABI: bit-identical outputs (the same kernels in the same order) on two
calls in a row, the second smaller, so that it reads none of the first
call's partials, plus the direct-kernel and single-slice shapes, the size
limit, and agreement with the oracle."""
import numpy as np
import pytest
import torch

import bitplane_quantized_expert_amd as pm
import oracle
import synth

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


class Matrix:
    """One seeded matrix encoded by the library on the host, on the device."""

    def __init__(self, rows, cols, group, unit):
        self.sh = pm.mshape(rows, cols, group)
        self.cd = synth.codes(13, 0, 0, unit, 0, rows, cols)
        self.lv = synth.leaves(13, 0, 0, unit, 0, rows, cols // group)
        self.pw = rows * cols // 32
        planes = np.zeros((8, self.pw), np.uint32)
        levels = np.zeros(pm.pm_levels_floats(self.sh), np.float32)
        pm.pm_encode_matrix(self.sh, self.cd, self.lv, None, planes, self.pw, levels)
        self.dp, self.dl = dev(planes), dev(levels)

    def both(self, k, xd):
        a = torch.full((self.sh.rows,), 7.0, dtype=torch.float32, device="cuda")
        b = torch.full((self.sh.rows,), -3.0, dtype=torch.float32, device="cuda")
        pm.pm_expert_gemv(self.sh, k, self.dp, self.pw, self.dl, xd, a)
        pm.pm_expert_gemv_noalloc(self.sh, k, self.dp, self.pw, self.dl, xd, b)
        return host(a), host(b)


def test_noalloc_gemv_matches_gemv_on_two_calls():
    print("[gpu case] pm_expert_gemv_noalloc vs pm_expert_gemv: 1024x4096 then 512x2048",
          flush=True)
    big = Matrix(1024, 4096, 128, unit=1)
    small = Matrix(512, 2048, 128, unit=2)
    xb = synth.activation(13, 0, 0, 1, 4096)
    xs = synth.activation(13, 0, 0, 2, 2048)
    for k in (2, 5):
        for M, x in ((big, xb), (small, xs)):
            want, got = M.both(k, dev(x))
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (M.sh.rows, k)
            rows = np.arange(0, M.sh.rows, 97)
            ref, S = oracle.gemv(oracle.pack_planes(M.cd[rows]),
                                 oracle.tree_levels(M.lv[rows]), k, 128, x)
            assert np.all(oracle.within_tolerance(got[rows], ref, S, 1e-4, 1e-6)), (M.sh.rows, k)


@pytest.mark.parametrize("rows,cols,k", [(256, 1024, 3),    # one slice: no partials
                                         (1024, 4096, 7),   # direct kernel
                                         (100, 2048, 2)])   # rows off the LUT tiling
def test_noalloc_gemv_other_paths(rows, cols, k):
    print(f"[gpu case] pm_expert_gemv_noalloc {rows}x{cols} k={k}", flush=True)
    M = Matrix(rows, cols, 128, unit=rows + k)
    x = synth.activation(13, 0, 0, rows + k, cols)
    want, got = M.both(k, dev(x))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_noalloc_gemv_size_limit():
    print("[gpu case] pm_expert_gemv_noalloc beyond its partials limit", flush=True)
    M = Matrix(64, 1024, 128, unit=9)
    rows = pm.PM_GEMV_NOALLOC_MAX_PARTIALS // 2 + 8
    sh = pm.mshape(rows, 2048, 128)
    xd = dev(np.zeros(2048, np.float32))
    y = torch.empty(8, dtype=torch.float32, device="cuda")
    # the shape is refused before any pointer is used
    with pytest.raises(pm.PMError) as ei:
        pm.pm_expert_gemv_noalloc(sh, 3, M.dp, rows * 2048 // 32, M.dl, xd, y)
    assert ei.value.status == pm.PM_ERR_SHAPE
