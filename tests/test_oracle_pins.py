"""Pins of the CPU oracle against what the pages and the mathematics fix:
hand-worked fixtures (tests/golden/), closed forms, library routines and
brute force.  None of these tests touches the product library or a GPU."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def ulp_diff(a, b):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float64)
    spacing = np.spacing(np.abs(a).astype(np.float32)).astype(np.float64)
    return np.abs(a.astype(np.float64) - b) / spacing


# ---------------------------------------------------------------- fixtures
@pytest.fixture(scope="module")
def tiny_expert():
    wl = synth.WORKLOADS[0]
    li = synth.expert_inputs(wl, 0, 0)
    return wl, li, oracle.encode_expert(li, wl.group)


def golden_row():
    g = load("eight_bit_row.json")
    cols = g["cols"]
    codes = np.zeros((1, cols), dtype=np.uint8)
    for c, v in g["codes_at"].items():
        codes[0, int(c)] = v
    leaves = (np.arange(256, dtype=np.float64) - 127.5).astype(np.float32)
    leaves = np.broadcast_to(leaves, (1, cols // g["group"], 256)).copy()
    return g, codes, leaves


# ---------------------------------------------------------------- tree
def test_pages_two_bit_example():
    g = load("two_bit_tree.json")
    leaves = np.array(g["leaves"], dtype=np.float32)
    lw = oracle.tree_levels(leaves, np.array(g["counts"]), depth=2)
    lu = oracle.tree_levels(leaves, None, depth=2)
    assert lw[1].tolist() == g["expected_level1_weighted"]
    assert lu[1].tolist() == g["expected_level1_unweighted"]
    assert lw[2].tolist() == g["leaves"]
    c = g["code_01"]
    # truncating code 01 to one bit lands on its parent, at two bits on itself
    assert lw[2][c["code"]] == c["k2_value"]
    assert lw[1][c["code"] >> 1] == c["k1_value_weighted"]
    assert lu[1][c["code"] >> 1] == c["k1_value_unweighted"]
    a, b = g["shared_prefix_k1"]
    assert a >> 1 == b >> 1


def test_golden_row_levels():
    g, codes, leaves = golden_row()
    lv = oracle.tree_levels(leaves)
    assert lv[1][0, 0].tolist() == g["level1"]
    assert lv[2][0, 0].tolist() == g["level2"]
    assert lv[3][0, 0].tolist() == g["level3"]
    assert np.array_equal(lv[8], leaves)


def test_golden_row_planes():
    g, codes, _ = golden_row()
    planes = oracle.pack_planes(codes)
    want = np.array([[int(h, 16) for h in row] for row in g["planes_hex"]], dtype=np.uint32)
    assert planes.shape == (8, 1, 2)
    assert np.array_equal(planes[:, 0, :], want)


def test_golden_row_dequant_and_gemv():
    g, codes, leaves = golden_row()
    planes = oracle.pack_planes(codes)
    lv = oracle.tree_levels(leaves)
    for name, col in (("col0", 0), ("col1", 1)):
        for k, v in g["dequant"][name].items():
            w = oracle.dequant(planes, lv, int(k), g["group"])
            assert w[0, col] == v
    for k, v in g["dequant"]["zero_code"].items():
        w = oracle.dequant(planes, lv, int(k), g["group"])
        assert w[0, 10] == v
    ones = np.ones(g["cols"], dtype=np.float32)
    for k, v in g["gemv_all_ones"].items():
        y, _ = oracle.gemv(planes, lv, int(k), g["group"], ones)
        assert y[0] == v
    x = np.zeros(g["cols"], dtype=np.float32)
    x[0] = x[1] = 1
    for k, v in g["gemv_e0_plus_e1"].items():
        y, _ = oracle.gemv(planes, lv, int(k), g["group"], x)
        assert y[0] == v


def test_levels_closed_form_unweighted():
    lv = synth.leaves(7, 0, 0, 0, 0, 4, 3)           # [4][3][256]
    levels = oracle.tree_levels(lv)
    assert np.array_equal(levels[8], lv)             # k = 8 reproduces the leaves
    for d in range(1, 8):
        span = 1 << (8 - d)
        exact = lv.astype(np.float64).reshape(4, 3, 1 << d, span).mean(axis=-1)
        assert ulp_diff(levels[d], exact).max() <= 8
        assert np.all(np.diff(levels[d], axis=-1) > 0)   # each level ascending


def test_levels_closed_form_weighted():
    rng_counts = synth.words(3, synth.KIND_POISON, 0, 0, 0, 0, 4 * 3 * 256) % 7
    counts = rng_counts.reshape(4, 3, 256).astype(np.int64)
    counts[0, 0, :128] = 0                           # an empty left half-tree
    lv = synth.leaves(8, 0, 0, 0, 0, 4, 3)
    levels = oracle.tree_levels(lv, counts)
    for d in range(1, 8):
        span = 1 << (8 - d)
        n = counts.reshape(4, 3, 1 << d, span).astype(np.float64)
        L = lv.astype(np.float64).reshape(4, 3, 1 << d, span)
        tot = n.sum(-1)
        ok = tot > 0
        centroid = (n * L).sum(-1) / np.where(ok, tot, 1)
        assert ulp_diff(levels[d][ok], centroid[ok]).max() <= 16
    # the empty half-tree falls back to the plain mean
    assert levels[1][0, 0, 0] == np.float32(
        (levels[2][0, 0, 0] + levels[2][0, 0, 1]) * np.float32(0.5))


def test_leaf_counts_histogram():
    codes = synth.codes(5, 0, 0, 0, 0, 3, 128)
    c = oracle.leaf_counts(codes, 64)
    assert c.shape == (3, 2, 256)
    assert np.all(c.sum(-1) == 64)
    assert c[1, 1, codes[1, 70]] >= 1


def test_leaf_counts_hand_counted_blocks():
    g = load("leaf_counts_row.json")
    codes = np.zeros((1, g["cols"]), np.uint8)
    for a, b, v in g["runs"]:
        codes[0, a:b] = v
    c = oracle.leaf_counts(codes, g["group"])
    want = np.zeros_like(c)
    for blk, d in g["counts"].items():
        for leaf, n in d.items():
            want[0, int(blk), int(leaf)] = n
    assert np.array_equal(c, want)


# ---------------------------------------------------------------- planes / prefix
def test_prefix_is_top_bits_all_codes():
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = np.concatenate([codes, codes[:, ::-1]], axis=0)
    planes = oracle.pack_planes(codes)
    for k in range(1, 9):
        assert np.array_equal(oracle.prefix_codes(planes, k), codes.astype(np.int64) >> (8 - k))


def test_prefix_nesting_and_plane_independence():
    codes = synth.codes(9, 0, 0, 0, 0, 16, 256)
    planes = oracle.pack_planes(codes)
    for k in range(1, 9):
        pk = oracle.prefix_codes(planes, k)
        for k2 in range(k, 9):
            assert np.array_equal(oracle.prefix_codes(planes, k2) >> (k2 - k), pk)
        poisoned = planes.copy()
        poisoned[k:] = synth.words(1, synth.KIND_POISON, 0, 0, 1, 0, poisoned[k:].size).reshape(poisoned[k:].shape)
        assert np.array_equal(oracle.prefix_codes(poisoned, k), pk)


def test_pack_bit_positions():
    # a single set bit of code c at column i must land in word i//32, bit i%32
    for i in (0, 1, 31, 32, 63, 100):
        for c in (0x80, 0x01, 0x10):
            codes = np.zeros((1, 128), dtype=np.uint8)
            codes[0, i] = c
            planes = oracle.pack_planes(codes)
            p = 7 - int(np.log2(c))
            nz = np.argwhere(planes != 0)
            assert nz.tolist() == [[p, 0, i // 32]]
            assert planes[p, 0, i // 32] == np.uint32(1 << (i % 32))


# ---------------------------------------------------------------- dequant / GEMV
def test_dequant_is_subtree_mean(tiny_expert):
    wl, li, enc = tiny_expert
    for m in range(3):
        lv, cd = li[m]
        rows, cols = cd.shape
        for k in range(1, 9):
            w = oracle.dequant(enc["planes"][m], enc["levels"][m], k, wl.group)
            span = 1 << (8 - k)
            means = lv.astype(np.float64).reshape(rows, cols // wl.group, 1 << k, span).mean(-1)
            g = np.arange(cols) // wl.group
            want = means[np.arange(rows)[:, None], g[None, :], cd.astype(np.int64) >> (8 - k)]
            assert ulp_diff(w, want).max() <= 8


def test_gemv_k8_is_dense_dgemv(tiny_expert):
    wl, li, enc = tiny_expert
    x = synth.activation(wl.seed, 0, 0, 0, wl.hidden)
    lv, cd = li[0]
    rows, cols = cd.shape
    g = np.arange(cols) // wl.group
    dense = lv[np.arange(rows)[:, None], g[None, :], cd.astype(np.int64)].astype(np.float64)
    y, s = oracle.gemv(enc["planes"][0], enc["levels"][0], 8, wl.group, x)
    want = np.dot(dense, x.astype(np.float64))
    assert np.all(np.abs(y - want) <= 1e-12 * s)


def test_gemv_k1_closed_form(tiny_expert):
    wl, li, enc = tiny_expert
    x = synth.activation(wl.seed, 0, 0, 0, wl.hidden).astype(np.float64)
    lv, cd = li[1]
    rows, cols = cd.shape
    l1 = enc["levels"][1][1].astype(np.float64)       # [rows][ngroups][2]
    ng = cols // wl.group
    xg = x.reshape(ng, wl.group)
    msb = (cd >> 7).reshape(rows, ng, wl.group).astype(np.float64)
    want = (l1[:, :, 0] * xg.sum(-1)[None, :]
            + (l1[:, :, 1] - l1[:, :, 0]) * (msb * xg[None]).sum(-1)).sum(-1)
    y, s = oracle.gemv(enc["planes"][1], enc["levels"][1], 1, wl.group, x)
    assert np.all(np.abs(y - want) <= 1e-12 * s + 1e-15)


def test_gemv_onehot_and_linear(tiny_expert):
    wl, li, enc = tiny_expert
    for k in (1, 3, 8):
        w = oracle.dequant(enc["planes"][2], enc["levels"][2], k, wl.group)
        for i in (0, 5, wl.inter - 1):
            x = np.zeros(wl.inter, dtype=np.float32)
            x[i] = 1
            y, _ = oracle.gemv(enc["planes"][2], enc["levels"][2], k, wl.group, x)
            assert np.array_equal(y, w[:, i].astype(np.float64))
        x = synth.activation(1, 0, 0, 3, wl.inter)
        y1, _ = oracle.gemv(enc["planes"][2], enc["levels"][2], k, wl.group, x)
        y2, _ = oracle.gemv(enc["planes"][2], enc["levels"][2], k, wl.group, 2 * x)
        assert np.array_equal(y2, 2 * y1)
        y0, s0 = oracle.gemv(enc["planes"][2], enc["levels"][2], k, wl.group, 0 * x)
        assert np.all(y0 == 0) and np.all(s0 == 0)


def test_materialized_exact_when_fp16_representable():
    g, codes, leaves = golden_row()
    planes = oracle.pack_planes(codes)
    lv = oracle.tree_levels(leaves)
    x = synth.activation(2, 0, 0, 0, g["cols"])
    for k in (1, 4, 8):
        a, _ = oracle.gemv(planes, lv, k, g["group"], x)
        b, _ = oracle.gemv_materialized_fp16(planes, lv, k, g["group"], x)
        assert np.array_equal(a, b)


def test_materialized_fp16_rounds_to_nearest_even():
    g = load("fp16_rounding.json")
    codes = np.full((1, g["cols"]), g["other_code"], np.uint8)
    for c, v in g["codes_at"].items():
        codes[0, int(c)] = v
    leaves = np.array(g["leaves"], np.float32)
    assert np.array_equal(leaves.astype(np.float64), np.array(g["leaves"]))   # exact in fp32
    planes = oracle.pack_planes(codes)
    lv = oracle.tree_levels(leaves[None, None, :])
    k, grp = g["k"], g["group"]
    for c, e in g["fp16_of_column"].items():
        x = np.zeros(g["cols"])
        x[int(c)] = 1.0
        direct, _ = oracle.gemv(planes, lv, k, grp, x)
        mat, _ = oracle.gemv_materialized_fp16(planes, lv, k, grp, x)
        assert direct[0] == e["exact"], c
        assert mat[0] == e["fp16"], c
    x = np.zeros(g["cols"])
    x[:5] = 1.0
    mat, _ = oracle.gemv_materialized_fp16(planes, lv, k, grp, x)
    sums = g["x_ones_on_columns_0_to_4"]
    assert mat[0] == sums["fp16"]
    # skipping the rounding, truncating or rounding to bf16 give other sums
    assert len({sums["fp16"], sums["no_rounding"], sums["truncation"], sums["bf16"]}) == 4


def test_relative_weight_error_hand_worked():
    r = load("relative_error_2x32.json")
    rows, cols, grp = r["rows"], r["cols"], r["group"]
    codes = np.zeros((rows, cols), np.uint8)
    codes[0, 0] = 255
    codes[1, :] = 128
    leaves = (np.arange(256, dtype=np.float64) - 127.5).astype(np.float32)
    leaves = np.broadcast_to(leaves, (rows, 1, 256)).copy()
    planes = oracle.pack_planes(codes)
    lv = oracle.tree_levels(leaves)
    # W by hand: the k = 8 reconstruction with two entries moved
    W = np.full((rows, cols), -127.5)
    W[0, 0] = 127.5
    W[1, :] = 0.5
    for key, v in r["W_changes"].items():
        o, i = (int(t) for t in key.split(","))
        W[o, i] = v
    assert np.sum(W ** 2) == r["norm_W_sq"]
    for k in (8, 1):
        want = math.sqrt(r["err_sq"][str(k)] / r["norm_W_sq"])
        got = oracle.relative_weight_error(W, planes, lv, k, grp)
        assert math.isclose(got, want, rel_tol=1e-14), (k, got, want)
    # the squared ratio, or the norm of the reconstruction in the
    # denominator, would give other values
    got8 = oracle.relative_weight_error(W, planes, lv, 8, grp)
    assert not math.isclose(got8, r["err_sq"]["8"] / r["norm_W_sq"], rel_tol=1e-6)
    assert not math.isclose(got8, math.sqrt(r["err_sq"]["8"] / r["norm_Wk_sq_8"]), rel_tol=1e-6)


# ---------------------------------------------------------------- FFN brute force
def brute_dequant(lv, cd, group, k):
    """Pure-Python loops from codes and leaves: the depth-k node of a code is
    the mean of the leaves sharing its top k bits."""
    rows, cols = cd.shape
    out = np.zeros((rows, cols))
    span = 1 << (8 - k)
    for o in range(rows):
        for i in range(cols):
            v = int(cd[o, i]) >> (8 - k)
            blk = lv[o, i // group]
            out[o, i] = sum(float(blk[v * span + t]) for t in range(span)) / span
    return out


def test_tiny_ffn_brute_force_all_k_triples():
    wl = synth.WORKLOADS[0]
    # a reduced tiny expert (hidden 64, inter 32, group 32) keeps the loops short
    small = synth.Workload(0, "tiny", 64, 32, 32, 1, 1, 1, 1, 0.0)
    li = synth.expert_inputs(small, 0, 0)
    enc = oracle.encode_expert(li, small.group)
    x = synth.activation(wl.seed, 0, 0, 0, small.hidden).astype(np.float64)
    dq = [[None] + [brute_dequant(li[m][0], li[m][1], small.group, k) for k in range(1, 9)]
          for m in range(3)]
    # the oracle's levels are fp32 (each within 8 ulp of the exact mean, see
    # test_levels_closed_form_unweighted), so a relative level error
    # eps = 8 * 2^-24 propagates into g, u, h and y; the bound below carries it
    eps = 2 * 8 * 2.0 ** -24
    for kg, ku, kd in itertools.product(range(1, 9), repeat=3):
        g = dq[0][kg] @ x
        u = dq[1][ku] @ x
        sg = np.abs(dq[0][kg]) @ np.abs(x)
        su = np.abs(dq[1][ku]) @ np.abs(x)
        h = g * expit(g) * u
        y = dq[2][kd] @ h
        hb = 1.2 * sg * np.abs(u) + (np.abs(g) + eps * sg) * su
        bound = eps * (np.abs(dq[2][kd]) @ (np.abs(h) + hb))
        r = oracle.expert_ffn(enc, kg, ku, kd, x)
        assert np.all(np.abs(r["y"] - y) <= bound + 1e-15)


def test_silu_library():
    z = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0


# ---------------------------------------------------------------- routing
def test_route_ties_and_sort():
    ids, w = oracle.route(np.array([0.5, 2.0, 2.0, -1.0, 1.0], dtype=np.float32), 3)
    assert ids.tolist() == [1, 2, 4]
    assert w[0] == w[1]
    assert abs(float(w[2]) / float(w[0]) - math.exp(-1.0)) < 1e-6
    for t in range(5):
        lg = synth.router_logits(11, 1, 0, t, 512)
        ids, w = oracle.route(lg, 10)
        ref = np.argsort(-lg, kind="stable")[:10]
        assert ids.tolist() == ref.tolist()
        assert abs(float(w.astype(np.float64).sum()) - 1.0) < 1e-6
        assert np.all(np.diff(w) <= 0)


# ---------------------------------------------------------------- allocator
def test_allocator_golden():
    g = load("allocator_and_residency.json")
    w = np.array(g["w"], dtype=np.float32)
    err = np.array([[4.0 ** -b for b in range(1, 9)]] * 2)
    for budget, want in g["budgets"].items():
        assert oracle.allocate_bits(w, err, int(budget)).tolist() == want


def test_allocator_ties():
    g = load("allocator_and_residency.json")
    for case in g["ties"]:
        w = np.array(case["w"], dtype=np.float32)
        err = np.array([[s * 4.0 ** -b for b in range(1, 9)] for s in case["scale"]])
        assert oracle.allocate_bits(w, err, case["budget"]).tolist() == case["want"]


def test_allocator_is_bruteforce_optimum():
    for t in range(6):
        lg = synth.router_logits(21, 1, 0, t, 64)
        _, w = oracle.route(lg, 4)
        err = synth.error_profiles(21, 1, t, 4)
        wd = w.astype(np.float64) ** 2
        for budget in (4, 7, 10, 13, 20, 32):
            k = oracle.allocate_bits(w, err, budget)
            assert k.sum() == budget and k.min() >= 1 and k.max() <= 8
            got = float((wd * err[np.arange(4), k - 1]).sum())
            best = min(
                float((wd * err[np.arange(4), np.array(c) - 1]).sum())
                for c in itertools.product(range(1, 9), repeat=4) if sum(c) == budget)
            assert got <= best * (1 + 1e-12)


def test_allocator_repair():
    convex = np.array([4.0 ** -b for b in range(1, 9)])
    assert np.array_equal(oracle.repair_profile(convex), convex)
    bumpy = np.array([1.0, 0.9, 0.5, 0.45, 0.2, 0.19, 0.18, 0.1])
    rep = oracle.repair_profile(bumpy)
    gains = rep[:-1] - rep[1:]
    assert np.all(np.diff(gains) <= 1e-15)               # each bit helps less
    assert rep[0] == bumpy[0] and abs(rep[-1] - bumpy[-1]) < 1e-12   # endpoints kept
    # the fit is the least-squares one: it preserves the gain total and no
    # other non-increasing sequence on a grid is closer
    d = bumpy[:-1] - bumpy[1:]
    assert abs(gains.sum() - d.sum()) < 1e-12
    assert np.allclose(oracle.isotonic_nonincreasing([1, 3, 2]), [2, 2, 2])
    assert np.allclose(oracle.isotonic_nonincreasing([3, 1, 2]), [3, 1.5, 1.5])


def test_allocator_workload_mean():
    wl = synth.WORKLOADS[1]
    err = synth.error_profiles(wl.seed, wl.cfg, 0, wl.n_experts)
    hist = np.zeros(9, dtype=np.int64)
    for t in range(40):
        ids, w = oracle.route(synth.router_logits(wl.seed, wl.cfg, 0, 0, wl.n_experts, step=t), 10)
        k = oracle.allocate_bits(w, err[ids], wl.budget)
        assert k.sum() == 25
        hist += np.bincount(k, minlength=9)
    assert hist[2] + hist[3] > hist[1] + hist[4:].sum()     # mostly 2 and 3 bits


# ---------------------------------------------------------------- residency / MoE
def test_missing_planes_pages_examples():
    g = load("allocator_and_residency.json")
    for case in g["residency"]:
        assert oracle.missing_planes(case["resident"], case["k"]) == case["fetch"]


def test_moe_onehot_weight_is_single_expert(tiny_expert):
    wl, li, enc = tiny_expert
    x = synth.activation(wl.seed, 0, 0, 0, wl.hidden)
    experts = {0: enc, 1: enc}
    y, s = oracle.moe_forward(experts, [[0, 1]], np.array([[1.0, 0.0]], np.float32),
                              [[[2, 3, 4], [8, 8, 8]]], x[None])
    r = oracle.expert_ffn(enc, 2, 3, 4, x)
    assert np.array_equal(y[0], r["y"])
    assert np.array_equal(s[0], r["Sy"])


def test_plane_cache_pages_examples():
    """[T] c13, c35: the pages' residency examples through the cache."""
    c = oracle.PrefixPlaneCache(64)
    assert c.access(7, 3) == [1, 2, 3]
    assert c.access(7, 5) == [4, 5]          # 3 resident, 5 requested
    assert c.access(7, 3) == []              # 5 resident, 3 requested
    assert c.resident(7) == 5
    d = oracle.PrefixPlaneCache(64)
    d.access(9, 2)
    assert d.access(9, 4) == [3, 4]          # only the missing part
    o = oracle.ObjectCache(64)
    o.access(17, 2)
    assert o.access(17, 4) == [1, 2, 3, 4]   # [T] c11: 2-bit copy does not help
    assert o.access(17, 2) == []


def test_plane_cache_golden_trace():
    """A hand-worked eviction trace: deepest planes age out first."""
    g = load("plane_cache_trace.json")
    c = oracle.PrefixPlaneCache(g["capacity"])
    o = oracle.ObjectCache(g["capacity"])
    for (e, k), want, res in zip(g["trace"], g["prefix"]["reads"], g["prefix"]["resident_after"]):
        assert c.access(e, k) == want
        assert {str(x): r for x, r in c.res.items()} == res
    assert (c.planes_read, c.hits, c.partial) == (g["prefix"]["planes_read"], g["prefix"]["hits"],
                                                  g["prefix"]["partial"])
    for (e, k), want in zip(g["trace"], g["objects"]["reads"]):
        assert o.access(e, k) == want
    assert (o.planes_read, o.hits) == (g["objects"]["planes_read"], g["objects"]["hits"])


def test_plane_cache_unbounded_closed_forms():
    """With room for everything nothing is evicted: the prefix cache reads
    each expert's deepest requested prefix once, the object cache each
    distinct (expert, k) once."""
    rng = np.random.default_rng(3)
    trace = [(int(e), int(k)) for e, k in zip(rng.integers(0, 20, 400), rng.integers(1, 9, 400))]
    c = oracle.PrefixPlaneCache(10 ** 6)
    o = oracle.ObjectCache(10 ** 6)
    for e, k in trace:
        c.access(e, k)
        o.access(e, k)
    deepest = {}
    for e, k in trace:
        deepest[e] = max(deepest.get(e, 0), k)
    assert c.planes_read == sum(deepest.values())
    assert o.planes_read == sum(k for _, k in set(trace))


def test_plane_cache_invariants_small_capacity():
    """Resident sets stay prefixes within the capacity, and never does the
    prefix cache read more planes than the object cache on the same trace
    with the same capacity when every request is at one fixed width."""
    rng = np.random.default_rng(4)
    trace = [(int(e), 4) for e in rng.zipf(1.3, 600) % 40]
    c = oracle.PrefixPlaneCache(48)
    o = oracle.ObjectCache(48)
    for e, k in trace:
        c.access(e, k)
        o.access(e, k)
        assert sum(c.res.values()) == len(c.order) <= 48
        assert all(1 <= r <= 8 for r in c.res.values())
    # at one fixed width both policies hold the same whole experts in the
    # same order: identical reads
    assert c.planes_read == o.planes_read


def test_downward_cache_pages_example():
    """[T] c51: a resident higher-precision copy serves lower requests and is
    promoted (read anew in full) when a request needs more."""
    d = oracle.DownwardCache(64)
    assert d.access(17, 4) == [1, 2, 3, 4]
    assert d.access(17, 2) == []              # served from the 4-bit copy
    assert d.access(17, 6) == [1, 2, 3, 4, 5, 6]
    assert d.access(17, 3) == [] and d.resident(17) == 6 and d.used == 6


def test_downward_cache_golden_traces():
    g = load("plane_cache_downward_trace.json")
    d = oracle.DownwardCache(g["capacity"])
    for (e, k), want, wd in zip(g["trace"], g["downward"]["reads"], g["downward"]["width_after"]):
        assert d.access(e, k) == want
        assert {str(x): r for x, r in d.width.items()} == wd
    assert (d.planes_read, d.hits) == (g["downward"]["planes_read"], g["downward"]["hits"])
    c = oracle.PrefixPlaneCache(g["capacity"])
    for (e, k), want, res in zip(g["trace"], g["prefix"]["reads"], g["prefix"]["resident_after"]):
        assert c.access(e, k) == want
        assert {str(x): r for x, r in c.res.items()} == res
    assert (c.planes_read, c.hits, c.partial) == (g["prefix"]["planes_read"], g["prefix"]["hits"],
                                                  g["prefix"]["partial"])
    o = oracle.ObjectCache(g["capacity"])
    for (e, k), want in zip(g["trace"], g["objects"]["reads"]):
        assert o.access(e, k) == want
    assert (o.planes_read, o.hits) == (g["objects"]["planes_read"], g["objects"]["hits"])
    first = load("plane_cache_trace.json")
    d = oracle.DownwardCache(first["capacity"])
    for (e, k), want in zip(first["trace"], g["first_trace_downward"]["reads"]):
        assert d.access(e, k) == want
    assert d.planes_read == g["first_trace_downward"]["planes_read"]


def test_downward_cache_closed_forms_and_invariants():
    """Unbounded: an expert costs k at every access that exceeds all its
    earlier requests.  At one fixed width it is the object cache."""
    rng = np.random.default_rng(5)
    trace = [(int(e), int(k)) for e, k in zip(rng.integers(0, 20, 400), rng.integers(1, 9, 400))]
    d = oracle.DownwardCache(10 ** 6)
    for e, k in trace:
        d.access(e, k)
    best, want = {}, 0
    for e, k in trace:
        if k > best.get(e, 0):
            want += k
            best[e] = k
    assert d.planes_read == want
    fixed = [(int(e), 3) for e in rng.zipf(1.3, 600) % 40]
    d, o = oracle.DownwardCache(30), oracle.ObjectCache(30)
    for e, k in fixed:
        assert d.access(e, k) == o.access(e, k)
    small = oracle.DownwardCache(10)
    for e, k in trace:
        small.access(e, k)
        assert small.used == sum(small.width.values()) <= 10
        assert sorted(small.order) == sorted(small.width)


# ---------------------------------------------------------------------------
# Encoder from fp32 weights: K-means per block, sorted leaves, weighted tree
# ---------------------------------------------------------------------------
def test_kmeans_textbook_case():
    """Two clumps, two centroids: the clump means, whatever the order."""
    w = np.array([11.0, 1.0, 12.0, 2.0, 10.0, 3.0], np.float32)
    c, a, n, it = oracle.kmeans_block(w, 2)
    assert c.tolist() == [2.0, 11.0]
    assert a.tolist() == [1, 0, 1, 0, 1, 0] and n.tolist() == [3, 3]


def test_kmeans_init_is_the_inverted_cdf_quantile():
    rng = np.random.default_rng(11)
    for g in (6, 96, 128, 255, 256, 1000, 4096):
        w = rng.normal(0, 0.02, g).astype(np.float32)
        for n in (2, 16, 256):
            q = (2 * np.arange(n) + 1) / (2 * n)
            want = np.quantile(w, q, method="inverted_cdf").astype(np.float32)
            assert np.array_equal(oracle.kmeans_init(w, n), want)


def test_kmeans_matches_scipy_lloyd():
    """scipy.cluster.vq.kmeans2 from the same start runs the same Lloyd
    iterations (it keeps fp64 centroids; ours are rounded to fp32)."""
    import warnings
    from scipy.cluster.vq import kmeans2, vq
    rng = np.random.default_rng(12)
    for trial in range(6):
        n = (4, 16, 32)[trial % 3]
        w = rng.normal(0, 0.02, 400).astype(np.float32)
        c, a, cnt, it = oracle.kmeans_block(w, n, max_iters=40)
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            ref, _ = kmeans2(w.astype(np.float64)[:, None],
                             oracle.kmeans_init(w, n).astype(np.float64)[:, None],
                             iter=it, minit="matrix", missing="warn")
        ref = ref[:, 0]
        assert np.all(np.abs(c - ref) <= 4e-7 * np.abs(ref) + 1e-12)
        assert np.array_equal(a, vq(w.astype(np.float64)[:, None], ref[:, None])[0])


@pytest.mark.parametrize("case", ["duplicates", "coarse grid"])
def test_kmeans_fixed_point_exact_rationals(case):
    """At convergence every weight sits on a nearest leaf (exact rational
    distances, ties to the lower index), the leaves ascend and every
    occupied leaf is its members' mean to within one fp32 rounding.  The
    coarse grid (many equal weights, so the 256 starting centroids repeat)
    is the case where the per-update sort matters."""
    from fractions import Fraction
    rng = np.random.default_rng(13)
    if case == "duplicates":
        w = rng.normal(0, 0.02, 300).astype(np.float32)
        w[::7] = w[1]
        n = 16
    else:
        w = (np.round(rng.normal(0, 0.02, 600) * 150) / 150).astype(np.float32)
        n = 256
    c, a, cnt, it = oracle.kmeans_block(w, n, max_iters=500)
    assert it < 500 and np.all(np.diff(c) >= 0)
    cf = [Fraction(float(v)) for v in c]
    for x in np.unique(w):
        d = [abs(Fraction(float(x)) - v) for v in cf]
        assert np.all(a[w == x] == d.index(min(d)))
    for j in range(n):
        m = w[a == j]
        assert cnt[j] == m.size
        if m.size:
            exact = sum(Fraction(float(v)) for v in m) / m.size
            assert abs(Fraction(float(c[j])) - exact) <= Fraction(float(abs(np.spacing(c[j]))))


def test_kmeans_objective_never_increases():
    rng = np.random.default_rng(14)
    w = rng.normal(0, 0.02, 2048).astype(np.float32)
    sse = []
    for t in range(0, 12):
        if t == 0:
            c = oracle.kmeans_init(w, 256)
            a = oracle.kmeans_assign(w, c)
        else:
            c, a, _, _ = oracle.kmeans_block(w, 256, max_iters=t)
        sse.append(float(np.sum((w.astype(np.float64) - c[a].astype(np.float64)) ** 2)))
    assert all(sse[i + 1] <= sse[i] * (1 + 1e-9) for i in range(len(sse) - 1))
    assert sse[-1] < sse[0]


def test_kmeans_small_block_is_exact_and_leaves_sorted():
    """A block of at most 256 distinct weights gets one leaf per weight: the
    8-bit reconstruction is exact.  The leaves are ascending in every case."""
    rng = np.random.default_rng(15)
    for g in (32, 128, 256):
        w = rng.normal(0, 0.02, g).astype(np.float32)
        c, a, cnt, it = oracle.kmeans_block(w)
        assert np.array_equal(c[a], w) and it == 1
        assert np.all(np.diff(c) >= 0)
    for g in (512, 1024):
        w = np.round(rng.normal(0, 0.02, g) * 300).astype(np.float32) / 300   # many ties
        c, a, cnt, it = oracle.kmeans_block(w)
        assert np.all(np.diff(c) >= 0) and cnt.sum() == g


def test_encoder_nodes_are_subtree_means():
    """Whole encoder: the depth-k node of a block is the mean of the block's
    weights whose code starts with that prefix (count-weighted tree over
    K-means leaves), to within a few fp32 roundings of the members' scale;
    the error shrinks with
    k and is zero at 8 bits for blocks of at most 256 distinct weights."""
    W = synth.weights(1, 0, 0, 0, 0, 4, 512)
    enc = oracle.encode_weights(W, 256, max_iters=40)
    for k in range(1, 9):
        pre = enc["codes"].astype(np.int64) >> (8 - k)
        for o in range(4):
            for g in range(2):
                blk = W[o, g * 256:(g + 1) * 256].astype(np.float64)
                pb = pre[o, g * 256:(g + 1) * 256]
                for v in np.unique(pb):
                    got = float(enc["levels"][k][o, g, v])
                    want = blk[pb == v].mean()
                    # roundings of the fp32 leaves and parents, each at most
                    # half an ulp of a value no larger than the members' scale
                    scale = np.abs(blk[pb == v]).max()
                    assert abs(got - want) <= 16 * 2.0 ** -24 * scale
    err = [oracle.relative_weight_error(W, enc["planes"], enc["levels"], k, 256) for k in range(1, 9)]
    assert all(err[i + 1] <= err[i] + 1e-12 for i in range(7)) and err[7] == 0.0
