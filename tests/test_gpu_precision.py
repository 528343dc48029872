"""LUT-path precision on heavy-tailed codebooks.  The LUT kernels form one
bucket of every block by subtraction: the block's activation sum minus the
other buckets' sums, scaled by a middle node.  Codebooks with far outer
leaves are where such a subtraction could lose precision.  Two kinds, at
full size (hidden 4096, inter 1024, group 128):
  - outlier: seeded leaves with the top leaf of every block moved to 10^2 to
    10^3 times the block's leaf spread above the rest (and, in half of the
    blocks, the bottom leaf as far below);
  - Student-t: K-means leaves (the library's device encoder) of weights drawn
    from a Student t with 3 degrees of freedom.
Every output against the oracle's per-output bound
|gpu - oracle| <= 1e-4 * sum|w*x| + 1e-6: pm_expert_gemv at k = 1..4 (the LUT
path) on a gate-shaped matrix, and a top-2 layer call at k = 1..5 (every
matrix on the LUT path) on experts built from these codebooks."""
import ctypes

import numpy as np
import pytest
import torch

import bitplane_quantized_expert_amd as pm
import oracle
import synth

pytestmark = pytest.mark.gpu
TOL = 1e-4
ABS = 1e-6
SEED = 77


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def report(name):
    print(f"[gpu case] {name}", flush=True)


def assert_close(got, want, scale, what=""):
    ok = oracle.within_tolerance(got, want, scale, TOL, ABS)
    if not ok.all():
        i = int(np.argmin(ok))
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs out of tolerance; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r} scale {scale[i]!r}")


def outlier_codebook(rows, cols, group, unit):
    """(leaves float32 [rows][cols/group][256] ascending, codes uint8, counts None)."""
    nb = rows * (cols // group)
    lv = synth.leaves(SEED, 0, 0, unit, 0, rows, cols // group).astype(np.float32).copy()
    cd = synth.codes(SEED, 0, 0, unit, 0, rows, cols)
    u = synth.words(SEED, synth.KIND_TRUNC, 0, 0, unit, 1, 2 * nb).reshape(rows, cols // group, 2)
    f = (100.0 * 10.0 ** (u[..., 0] / 2.0 ** 32)).astype(np.float32)    # 100 .. 1000
    spread = lv[..., -1] - lv[..., 0]
    lv[..., -1] = lv[..., -2] + f * spread
    low = (u[..., 1] & 1) == 1
    lv[..., 0] = np.where(low, lv[..., 1] - f * spread, lv[..., 0])
    assert np.all(np.diff(lv, axis=-1) >= 0)
    return lv, cd, None


def student_t_codebook(rows, cols, group, unit):
    """K-means (device encoder) of Student-t(3) weights: (leaves, codes, counts)."""
    rng = np.random.default_rng(SEED * 1000 + unit)
    z = rng.standard_normal((rows, cols))
    chi = rng.chisquare(3.0, (rows, cols))
    w = (0.02 * z / np.sqrt(chi / 3.0)).astype(np.float32)
    sh = pm.mshape(rows, cols, group)
    nb = rows * (cols // group)
    codes = torch.empty(rows * cols, dtype=torch.uint8, device="cuda")
    leaves = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    counts = torch.empty(nb * 256, dtype=torch.int32, device="cuda")
    pm.pm_kmeans_codebook_device(sh, dev(w), 25, codes, leaves, counts)
    lv = host(leaves).reshape(rows, cols // group, 256)
    cd = host(codes).reshape(rows, cols)
    ct = host(counts).view(np.uint32).reshape(rows, cols // group, 256)
    return lv, cd, ct


def encode(sh, lv, cd, ct):
    pw = sh.rows * sh.cols // 32
    planes = np.zeros((8, pw), np.uint32)
    levels = np.zeros(pm.pm_levels_floats(sh), np.float32)
    pm.pm_encode_matrix(sh, cd, lv, ct, planes, pw, levels)
    ref = {"planes": oracle.pack_planes(cd), "levels": oracle.tree_levels(lv, ct)}
    return planes, levels, ref


BUILDERS = {"outlier": outlier_codebook, "student_t": student_t_codebook}


@pytest.mark.parametrize("kind", sorted(BUILDERS))
def test_lut_gemv_heavy_tailed_every_row(kind):
    report(f"LUT GEMV 1024x4096 on {kind} codebooks, k = 1..4, every row")
    rows, cols, group = 1024, 4096, 128
    sh = pm.mshape(rows, cols, group)
    lv, cd, ct = BUILDERS[kind](rows, cols, group, 1)
    planes, levels, ref = encode(sh, lv, cd, ct)
    dp, dl = dev(planes), dev(levels)
    x = synth.activation(SEED, 0, 0, 3, cols)
    xd = dev(x)
    for k in range(1, 5):
        y = torch.full((rows,), 9.0, dtype=torch.float32, device="cuda")
        pm.pm_expert_gemv(sh, k, dp, rows * cols // 32, dl, xd, y)
        want, S = oracle.gemv(ref["planes"], ref["levels"], k, group, x)
        assert_close(host(y), want, S, f"{kind} k={k}")


def test_layer_heavy_tailed_experts_k1_to_5():
    report("layer top-2 on outlier and Student-t experts, k = 1..5, every output")
    wl = synth.WORKLOADS[1]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    st = pm.pm_store_create(e, 1, 2)
    hip = ctypes.CDLL("libamdhip64.so")
    experts = []
    for ex, kind in enumerate(("outlier", "student_t")):
        pp, lp = pm.pm_store_slot(st, 0, ex)
        ref = {"group": wl.group, "planes": [], "levels": []}
        for m in range(3):
            po, lo, sh = pm.pm_expert_matrix_offsets(e, m)
            lv, cd, ct = BUILDERS[kind](sh.rows, sh.cols, sh.group, 10 * ex + m)
            planes, levels, r = encode(sh, lv, cd, ct)
            for p in range(8):
                assert hip.hipMemcpy(ctypes.c_void_p(pp + 4 * (p * pw + po)),
                                     ctypes.c_void_p(planes[p].ctypes.data),
                                     ctypes.c_size_t(planes[p].nbytes), 1) == 0
            assert hip.hipMemcpy(ctypes.c_void_p(lp + 4 * lo), ctypes.c_void_p(levels.ctypes.data),
                                 ctypes.c_size_t(levels.nbytes), 1) == 0
            ref["planes"].append(r["planes"])
            ref["levels"].append(r["levels"])
        pm.pm_store_set_resident(st, 0, ex, 8)
        experts.append(ref)
    ids = np.array([[0, 1]], np.int32)
    w = np.array([[0.6, 0.4]], np.float32)
    x = synth.activation(SEED, 1, 0, 0, wl.hidden)
    xd = dev(x[None])
    for kk in range(1, 6):
        k = np.full((1, 2, 3), kk, np.uint8)
        y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y)
        want, S = np.zeros(wl.hidden), np.zeros(wl.hidden)
        for j in range(2):
            r = oracle.expert_ffn(experts[j], kk, kk, kk, x)
            want += float(w[0, j]) * r["y"]
            S += abs(float(w[0, j])) * r["Sy"]
        assert_close(host(y)[0], want, S, f"k={kk}")
    st.close()
