"""GPU parity of the encoder from fp32 weights (pm_kmeans_codebook_device,
then pm_encode_matrix_device with the counts) against the oracle's K-means,
sort and count-weighted tree: codes, leaves, counts, iteration counts,
planes and levels must be bit-identical."""
import numpy as np
import pytest
import torch

import bitplane_quantized_expert_amd as pm
import oracle
import synth

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def report(name):
    print(f"[gpu case] {name}", flush=True)


def weights(kind, rows, cols, seed=3):
    w = synth.weights(seed, 0, 0, 0, 0, rows, cols)
    if kind == "grid":                      # many equal weights: repeated starting centroids
        w = (np.round(w.astype(np.float64) * 150) / 150).astype(np.float32)
    elif kind == "zeros":                   # runs of zeros and of one value
        w = w.copy()
        w[:, ::3] = 0.0
        w[:, 1::7] = w[0, 1]
    return w


def run_kmeans(w, group, iters):
    rows, cols = w.shape
    s = pm.mshape(rows, cols, group)
    nb = rows * (cols // group)
    codes = torch.empty(rows * cols, dtype=torch.uint8, device="cuda")
    leaves = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
    counts = torch.empty(nb * 256, dtype=torch.int32, device="cuda")
    its = torch.empty(nb, dtype=torch.int32, device="cuda")
    dw = dev(w)
    pm.pm_kmeans_codebook_device(s, dw, iters, codes, leaves, counts, its)
    torch.cuda.synchronize()
    return (codes.cpu().numpy().reshape(rows, cols), leaves.cpu().numpy().reshape(rows, -1, 256),
            counts.cpu().numpy().view(np.uint32).reshape(rows, -1, 256),
            its.cpu().numpy().reshape(rows, -1), s, codes, leaves, counts)


def check_blocks(w, group, iters, got, blocks):
    codes, leaves, counts, its = got[:4]
    for o, g in blocks:
        lv, cd, n, it = oracle.kmeans_block(w[o, g * group:(g + 1) * group], 256, iters)
        where = f"row {o} block {g}"
        assert np.array_equal(leaves[o, g], lv), where
        assert np.array_equal(codes[o, g * group:(g + 1) * group], cd.astype(np.uint8)), where
        assert np.array_equal(counts[o, g], n.astype(np.uint32)), where
        assert its[o, g] == it, where


@pytest.mark.parametrize("rows,cols,group", [(3, 128, 128), (2, 96, 32), (3, 960, 96),
                                             (4, 1024, 256), (2, 2048, 1024), (2, 4096, 4096)])
@pytest.mark.parametrize("kind", ["normal", "grid", "zeros"])
def test_kmeans_blocks_bit_exact(rows, cols, group, kind):
    report(f"kmeans {kind} rows={rows} cols={cols} group={group}")
    w = weights(kind, rows, cols)
    for iters in (0, 1, 25):
        got = run_kmeans(w, group, iters)
        check_blocks(w, group, iters, got,
                     [(o, g) for o in range(rows) for g in range(cols // group)])


def test_encoder_end_to_end_bit_exact():
    """K-means, then the device encoder with the counts: the oracle's planes
    and count-weighted levels."""
    report("encode_weights rows=6 cols=1024 group=256")
    w = weights("normal", 6, 1024)
    got = run_kmeans(w, 256, 25)
    s, codes, leaves, counts = got[4:]
    planes = torch.empty(8 * pm.pm_plane_words(s), dtype=torch.int32, device="cuda")
    levels = torch.empty(pm.pm_levels_floats(s), dtype=torch.float32, device="cuda")
    pm.pm_encode_matrix_device(s, codes, leaves, counts, planes, pm.pm_plane_words(s), levels)
    torch.cuda.synchronize()
    enc = oracle.encode_weights(w, 256, 25)
    assert np.array_equal(planes.cpu().numpy().view(np.uint32).reshape(8, 6, 32), enc["planes"])
    lv = levels.cpu().numpy()
    for d in range(1, 9):
        off = pm.pm_level_offset(s, d)
        n = 6 * 4 * (1 << d)
        assert np.array_equal(lv[off:off + n].reshape(6, 4, 1 << d), enc["levels"][d]), d


@pytest.mark.parametrize("group", [128, 1024])
def test_kmeans_full_size_sampled(group):
    """A whole 1024 x 4096 gate matrix in one launch; sampled blocks against
    the oracle, every block's counts against its codes."""
    report(f"kmeans full gate matrix 1024x4096 group={group}")
    w = synth.weights(synth.BASE_SEED + 1, 1, 0, 7, 0, 1024, 4096)
    got = run_kmeans(w, group, 25)
    codes, leaves, counts, its = got[:4]
    nbr = 4096 // group
    rng = np.random.default_rng(group)
    picks = [(int(o), int(g)) for o, g in zip(rng.integers(0, 1024, 12), rng.integers(0, nbr, 12))]
    picks += [(0, 0), (1023, nbr - 1)]
    check_blocks(w, group, 25, got, picks)
    blocks = codes.reshape(1024, nbr, group)
    for o in range(0, 1024, 97):
        for g in range(nbr):
            assert np.array_equal(np.bincount(blocks[o, g], minlength=256), counts[o, g])
    assert np.all(np.diff(leaves, axis=-1) >= 0)
