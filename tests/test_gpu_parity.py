"""GPU parity of libpm against the CPU oracle, through the C ABI.

Bit-exact: device-drawn inputs, device-encoded planes and levels, unpacked
prefixes, dequantised values, one-hot GEMV columns, poisoned planes/levels,
repeated runs.  Within |gpu - oracle| <= 1e-4 * sum|w*x| + 1e-6 per output:
every fp32 GEMV and MoE output, on every workload configuration (the large
ones on sampled output rows)."""
import numpy as np
import pytest
import torch

import bitplane_quantized_expert_amd as pm
import oracle
import oracle_cases as oc
import synth
from synth.device import DeviceSynth
from synth.pool import PoolFiller

pytestmark = pytest.mark.gpu
TOL = 1e-4
ABS = 1e-6


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, want, scale, what=""):
    ok = oracle.within_tolerance(got, want, scale, TOL, ABS)
    if not ok.all():
        i = int(np.argmin(ok))
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs out of tolerance; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r} scale {scale[i]!r}")


def report(name):
    print(f"[gpu case] {name}", flush=True)


# ---------------------------------------------------------------- tiny expert on device
class DevExpert:
    """An expert encoded on the device by the library's device encoder."""

    def __init__(self, wl, layer=0, expert=0, weighted=False):
        self.wl = wl
        self.e = pm.eshape(wl.hidden, wl.inter, wl.group)
        self.pw = pm.pm_expert_plane_words(self.e)
        self.planes = torch.zeros(8 * self.pw, dtype=torch.int32, device="cuda")
        self.levels = torch.zeros(pm.pm_expert_levels_floats(self.e), dtype=torch.float32,
                                  device="cuda")
        self.li = synth.expert_inputs(wl, layer, expert)
        self.shapes = []
        for m in range(3):
            po, lo, sh = pm.pm_expert_matrix_offsets(self.e, m)
            lv, cd = self.li[m]
            cnt = dev(oracle.leaf_counts(cd, wl.group).astype(np.uint32)) if weighted else None
            pm.pm_encode_matrix_device(sh, dev(cd), dev(lv), cnt,
                                       self.planes.data_ptr() + 4 * po, self.pw,
                                       self.levels.data_ptr() + 4 * lo)
            self.shapes.append((po, lo, sh))
        torch.cuda.synchronize()
        self.enc = oracle.encode_expert(self.li, wl.group, weighted=weighted)

    def mat(self, m):
        po, lo, sh = self.shapes[m]
        return sh, self.planes.data_ptr() + 4 * po, self.levels.data_ptr() + 4 * lo


@pytest.fixture(scope="module")
def tiny():
    report("tiny expert (hidden 256, inter 128, group 64)")
    return DevExpert(synth.WORKLOADS[0])


def test_device_synth_is_host_synth():
    report("device synth vs host synth")
    syn = DeviceSynth()
    for (cfg, layer, e, m, rows, cols, g, r0, n) in [(1, 0, 5, 0, 1024, 4096, 128, 0, 3),
                                                     (1, 0, 511, 2, 4096, 1024, 128, 4090, 6),
                                                     (0, 0, 0, 1, 128, 256, 64, 7, 9)]:
        wl = synth.WORKLOADS[cfg]
        buf = torch.empty(n * (cols // g) * 256, dtype=torch.float32, device="cuda")
        syn.leaves_into(buf, wl.seed, cfg, layer, e, m, cols // g, r0, n)
        want = synth.leaves(wl.seed, cfg, layer, e, m, rows, cols // g, r0, r0 + n)
        assert np.array_equal(host(buf).view(np.uint32), want.reshape(-1).view(np.uint32))
        cb = torch.empty(n * cols, dtype=torch.uint8, device="cuda")
        syn.codes_into(cb, wl.seed, cfg, layer, e, m, cols, r0, n)
        assert np.array_equal(host(cb), synth.codes(wl.seed, cfg, layer, e, m, rows, cols, r0,
                                                    r0 + n).reshape(-1))


@pytest.mark.parametrize("weighted", [False, True])
def test_device_encoder_bit_exact(weighted):
    report(f"device encoder weighted={weighted}")
    x = DevExpert(synth.WORKLOADS[0], weighted=weighted)
    planes = host(x.planes).view(np.uint32).reshape(8, x.pw)
    levels = host(x.levels)
    for m in range(3):
        po, lo, sh = x.shapes[m]
        n = pm.pm_plane_words(sh)
        assert np.array_equal(planes[:, po:po + n].reshape(8, sh.rows, sh.cols // 32),
                              x.enc["planes"][m])
        want = np.concatenate([x.enc["levels"][m][d].reshape(-1) for d in range(1, 9)])
        got = levels[lo:lo + pm.pm_levels_floats(sh)]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_unpack_and_dequant_bit_exact(tiny):
    report("unpack prefix + dequant, all k")
    for m in range(3):
        sh, pp, lp = tiny.mat(m)
        for k in range(1, 9):
            pre = torch.empty(sh.rows * sh.cols, dtype=torch.uint8, device="cuda")
            pm.pm_debug_unpack_prefix(sh, k, pp, tiny.pw, pre)
            want = oracle.prefix_codes(tiny.enc["planes"][m], k)
            assert np.array_equal(host(pre).reshape(sh.rows, sh.cols), want)
            wv = torch.empty(sh.rows * sh.cols, dtype=torch.float32, device="cuda")
            pm.pm_debug_dequant(sh, k, pp, tiny.pw, lp, wv)
            wq = oracle.dequant(tiny.enc["planes"][m], tiny.enc["levels"][m], k, tiny.wl.group)
            assert np.array_equal(host(wv).reshape(sh.rows, sh.cols).view(np.uint32),
                                  wq.view(np.uint32))
            w16 = torch.empty(sh.rows * sh.cols, dtype=torch.int16, device="cuda")
            pm.pm_materialize_fp16(sh, k, pp, tiny.pw, lp, w16)
            assert np.array_equal(host(w16).view(np.float16).reshape(sh.rows, sh.cols),
                                  wq.astype(np.float16))


def test_gemv_all_k_and_determinism(tiny):
    report("prefix GEMV, 3 matrices x 8 prefixes")
    for m in range(3):
        sh, pp, lp = tiny.mat(m)
        x = synth.activation(tiny.wl.seed, 0, 0, m, sh.cols)
        xd = dev(x)
        for k in range(1, 9):
            y = torch.empty(sh.rows, dtype=torch.float32, device="cuda")
            pm.pm_expert_gemv(sh, k, pp, tiny.pw, lp, xd, y)
            want, S = oracle.gemv(tiny.enc["planes"][m], tiny.enc["levels"][m], k, tiny.wl.group, x)
            got = host(y)
            assert_close(got, want, S, f"m={m} k={k}")
            y2 = torch.empty_like(y)
            pm.pm_expert_gemv(sh, k, pp, tiny.pw, lp, xd, y2)
            assert np.array_equal(host(y2).view(np.uint32), got.view(np.uint32))


def test_gemv_onehot_columns_bit_exact(tiny):
    report("one-hot columns")
    for m in (0, 2):
        sh, pp, lp = tiny.mat(m)
        for k in (1, 2, 3, 5, 8):
            wq = oracle.dequant(tiny.enc["planes"][m], tiny.enc["levels"][m], k, tiny.wl.group)
            for i in (0, 1, 31, 32, sh.cols - 1):
                x = np.zeros(sh.cols, np.float32)
                x[i] = 1.0
                y = torch.empty(sh.rows, dtype=torch.float32, device="cuda")
                pm.pm_expert_gemv(sh, k, pp, tiny.pw, lp, dev(x), y)
                assert np.array_equal(host(y).view(np.uint32), wq[:, i].view(np.uint32))


def test_gemv_poisoned_planes_and_levels(tiny):
    report("poison planes >= k and levels != k")
    syn = DeviceSynth()
    sh, pp, lp = tiny.mat(1)
    x = dev(synth.activation(3, 0, 0, 0, sh.cols))
    for k in range(1, 9):
        y = torch.empty(sh.rows, dtype=torch.float32, device="cuda")
        pm.pm_expert_gemv(sh, k, pp, tiny.pw, lp, x, y)
        base = host(y).copy()
        planes = tiny.planes.clone()
        levels = tiny.levels.clone()
        pv = planes.view(8, tiny.pw)
        if k < 8:
            syn.poison_into(pv[k:].reshape(-1), 99, k)
        po, lo, _ = tiny.shapes[1]
        lvv = levels[lo:lo + pm.pm_levels_floats(sh)]
        for d in range(1, 9):
            if d == k:
                continue
            a = pm.pm_level_offset(sh, d)
            n = pm.pm_levels_floats(sh) // 510 * (1 << d)
            syn.poison_into(lvv[a:a + n].view(torch.int32), 7, d)
        y2 = torch.empty_like(y)
        pm.pm_expert_gemv(sh, k, planes.data_ptr() + 4 * po, tiny.pw, levels.data_ptr() + 4 * lo,
                          x, y2)
        assert np.array_equal(host(y2).view(np.uint32), base.view(np.uint32)), f"k={k}"


@pytest.mark.parametrize("rows,cols,group", [(37, 96, 32), (1, 32, 32), (5, 4096, 128),
                                             (4096, 1024, 128), (3, 0, 64)])
def test_gemv_edge_shapes(rows, cols, group):
    report(f"edge shape {rows}x{cols} g{group}")
    sh = pm.mshape(rows, cols, group)
    lv = synth.leaves(5, 0, 0, 1, 0, rows, cols // group) if cols else np.zeros((rows, 0, 256), np.float32)
    cd = synth.codes(5, 0, 0, 1, 0, rows, cols) if cols else np.zeros((rows, 0), np.uint8)
    pw = max(1, rows * cols // 32)
    planes = np.zeros((8, pw), np.uint32)
    levels = np.zeros(max(1, pm.pm_levels_floats(sh)), np.float32)
    pm.pm_encode_matrix(sh, cd, lv, None, planes, pw, levels)
    x = synth.activation(5, 0, 0, 0, max(cols, 1))[:cols]
    dp, dl, dx = dev(planes), dev(levels), dev(np.concatenate([x, [0.0]]).astype(np.float32))
    for k in (1, 2, 3, 4, 6, 8):
        y = torch.full((rows,), 7.0, dtype=torch.float32, device="cuda")
        pm.pm_expert_gemv(sh, k, dp, pw, dl, dx, y)
        got = host(y)
        if cols == 0:
            assert np.all(got == 0)
            continue
        pl = planes[:, :rows * cols // 32].reshape(8, rows, cols // 32)
        lvd = oracle.tree_levels(lv)
        want, S = oracle.gemv(pl, lvd, k, group, x)
        assert_close(got, want, S, f"{rows}x{cols} k={k}")


# ---------------------------------------------------------------- LUT-path shapes
class DevMatrix:
    """One seeded matrix encoded on the host by the library, copied to the device."""

    def __init__(self, rows, cols, group, unit=0):
        self.sh = pm.mshape(rows, cols, group)
        self.lv = synth.leaves(11, 0, 0, unit, 0, rows, cols // group)
        self.cd = synth.codes(11, 0, 0, unit, 0, rows, cols)
        self.pw = rows * cols // 32
        planes = np.zeros((8, self.pw), np.uint32)
        levels = np.zeros(pm.pm_levels_floats(self.sh), np.float32)
        pm.pm_encode_matrix(self.sh, self.cd, self.lv, None, planes, self.pw, levels)
        self.dp, self.dl = dev(planes), dev(levels)
        self.planes = oracle.pack_planes(self.cd)
        self.levels = oracle.tree_levels(self.lv)
        self.group = group

    def gemv(self, k, x, planes=None, levels=None):
        y = torch.full((self.sh.rows,), 7.0, dtype=torch.float32, device="cuda")
        pm.pm_expert_gemv(self.sh, k, self.dp if planes is None else planes, self.pw,
                          self.dl if levels is None else levels, x, y)
        return host(y)


@pytest.mark.parametrize("rows,cols", [(64, 4096), (98, 1024), (6, 2048)])
def test_lut_gemv_all_k(rows, cols):
    report(f"LUT-path GEMV {rows}x{cols}, all k")
    M = DevMatrix(rows, cols, 128, unit=rows)
    x = synth.activation(12, 0, 0, rows, cols)
    xd = dev(x)
    for k in range(1, 9):
        got = M.gemv(k, xd)
        want, S = oracle.gemv(M.planes, M.levels, k, 128, x)
        assert_close(got, want, S, f"{rows}x{cols} k={k}")
        assert np.array_equal(M.gemv(k, xd).view(np.uint32), got.view(np.uint32))


def test_comparator_batches_match_single_calls():
    """One dequant launch and one fp16 GEMV launch over several matrices of
    different shapes, groups and prefixes give the single calls' bits."""
    report("batched materialize-fp16 and fp16 GEMV vs single calls")
    mats = [DevMatrix(64, 4096, 128, unit=41), DevMatrix(256, 1024, 128, unit=42),
            DevMatrix(40, 2048, 64, unit=43), DevMatrix(8, 512, 32, unit=44)]
    ks = [1, 3, 5, 8]
    shapes = [M.sh for M in mats]
    outs = [torch.empty(M.sh.rows * M.sh.cols, dtype=torch.int16, device="cuda") for M in mats]
    pm.pm_materialize_fp16_batch(shapes, ks, [M.dp for M in mats], [M.pw for M in mats],
                                 [M.dl for M in mats], outs)
    xs = [dev(synth.activation(14, 0, 0, i, M.sh.cols)) for i, M in enumerate(mats)]
    ys = [torch.full((M.sh.rows,), 5.0, dtype=torch.float32, device="cuda") for M in mats]
    pm.pm_gemv_fp16_batch(shapes, outs, xs, ys)
    for i, (M, k) in enumerate(zip(mats, ks)):
        one = torch.empty_like(outs[i])
        pm.pm_materialize_fp16(M.sh, k, M.dp, M.pw, M.dl, one)
        assert torch.equal(one, outs[i]), i
        y1 = torch.empty_like(ys[i])
        pm.pm_gemv_fp16(M.sh, one, xs[i], y1)
        assert np.array_equal(host(y1).view(np.uint32), host(ys[i]).view(np.uint32)), i
        # and the fp16 weights are the oracle's: the depth-k node rounded to nearest even
        rows = np.arange(0, M.sh.rows, 7)
        want = oracle.dequant(oracle.pack_planes(M.cd[rows]), oracle.tree_levels(M.lv[rows]), k,
                              M.group).astype(np.float16)
        got = host(outs[i]).view(np.float16).reshape(M.sh.rows, M.sh.cols)[rows]
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), i


def test_lut_gemv_onehot_and_poison():
    report("LUT-path one-hot columns and poisoned planes/levels")
    M = DevMatrix(40, 2048, 128, unit=3)
    syn = DeviceSynth()
    for k in range(1, 6):
        wq = oracle.dequant(M.planes, M.levels, k, 128)
        for i in (0, 7, 8, 31, 32, 1023, 1024, 1500, 2047):
            x = np.zeros(2048, np.float32)
            x[i] = 1.0
            got = M.gemv(k, dev(x))
            assert np.array_equal(got.view(np.uint32), wq[:, i].view(np.uint32)), (k, i)
        xd = dev(synth.activation(13, 0, 0, k, 2048))
        base = M.gemv(k, xd)
        planes = M.dp.clone()
        levels = M.dl.clone()
        if k < 8:
            syn.poison_into(planes.view(8, M.pw)[k:].reshape(-1).view(torch.int32), 21, k)
        for d in range(1, 9):
            if d != k:
                a = pm.pm_level_offset(M.sh, d)
                n = pm.pm_levels_floats(M.sh) // 510 * (1 << d)
                syn.poison_into(levels[a:a + n].view(torch.int32), 22, d)
        got = M.gemv(k, xd, planes, levels)
        assert np.array_equal(got.view(np.uint32), base.view(np.uint32)), k


MID = synth.Workload(9, "mid-e8-h2048-i1024-g128", 2048, 1024, 128, 8, 2, 1, 3, 2.5)


def test_forward_mixed_paths_multi_slice():
    report("forward with LUT and direct paths mixed, 2 gate/up slices, shared experts")
    wl = MID
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    ks = synth.uniform_k(wl.seed, wl.cfg, 0, 0, 18 * 12)
    rows = oc.sample_rows(wl.hidden, 20, 5)
    for case in range(12):
        # three tokens; token 2 shares its first expert with token 0
        ids = np.array([[case % 8, (case + 3) % 8], [(case + 5) % 8, (case + 6) % 8],
                        [case % 8, (case + 1) % 8]], np.int32)
        w = np.array([[0.625, 0.375], [0.5, 0.5], [0.875, 0.125]], np.float32)
        k = ks[case * 18:(case + 1) * 18].reshape(3, 2, 3)
        x = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=case) for t in range(3)])
        y = torch.empty((3, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y)
        got = host(y)
        for t in range(3):
            want, S = oc.token_layer(wl, 0, ids[t], w[t], k[t], x[t], rows)
            assert_close(got[t][rows], want, S, f"case {case} token {t} k={k[t].tolist()}")
    st.close()


WIDE = synth.Workload(10, "wide-e8-h2048-i2048-g128", 2048, 2048, 128, 8, 2, 1, 3, 2.5)


def test_forward_folded_combine_two_down_slices():
    """Every product on the LUT path (k <= 5), so the routing-weighted combine
    folds into the down launch: down matrices of 2048 columns, whose two
    slice sums both add into y, three tokens top-2 with one expert shared.
    Then the same calls in place (y is x: the separate combine runs) and with
    the fixed-order combine, all against the oracle."""
    report("combine folded into the down launch, 2 down slices; in place; fixed order")
    wl = WIDE
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    ks = (synth.uniform_k(wl.seed, wl.cfg, 0, 0, 18 * 4).astype(np.int32) - 1) % 5 + 1
    rows = oc.sample_rows(wl.hidden, 20, 6)
    for case in range(4):
        ids = np.array([[case % 8, (case + 3) % 8], [(case + 5) % 8, (case + 6) % 8],
                        [case % 8, (case + 1) % 8]], np.int32)
        w = np.array([[0.625, 0.375], [0.5, 0.5], [0.875, 0.125]], np.float32)
        k = ks[case * 18:(case + 1) * 18].reshape(3, 2, 3).astype(np.uint8)
        x = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=case)
                      for t in range(3)])
        outs = {}
        y = torch.empty((3, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y)
        outs["folded"] = host(y)
        xy = dev(x)
        pm.pm_moe_token_forward(st, 0, ids, w, k, xy, xy)
        outs["in place"] = host(xy)
        pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y, flags=pm.PM_DETERMINISTIC)
        outs["fixed order"] = host(y)
        for t in range(3):
            want, S = oc.token_layer(wl, 0, ids[t], w[t], k[t], x[t], rows)
            for name, got in outs.items():
                assert_close(got[t][rows], want, S, f"case {case} token {t} {name} k={k[t].tolist()}")
    st.close()


WIDE_H = synth.Workload(11, "wideh-e6-h5120-i1024-g128", 5120, 1024, 128, 6, 2, 1, 3, 2.5)


def test_forward_five_gate_up_slices():
    """Gate/up matrices of 5120 columns: five 1024-column slice partials per
    output, more than the four the down builders load at once, so h is summed
    over the slices in a loop.  Three tokens top-2, one expert shared; prefixes
    1..5 (every product a LUT job, the combine folded into the down launch),
    then the fixed-order combine, then prefixes 1..8 (LUT and direct kernels
    mixed), all against the oracle."""
    report("five gate/up slices: h summed over the slices in a loop")
    wl = WIDE_H
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    ks8 = synth.uniform_k(wl.seed, wl.cfg, 0, 0, 18 * 3).astype(np.int32)
    ks5 = (ks8 - 1) % 5 + 1
    rows = oc.sample_rows(wl.hidden, 20, 7)
    for case in range(3):
        ids = np.array([[case % 6, (case + 2) % 6], [(case + 3) % 6, (case + 4) % 6],
                        [case % 6, (case + 1) % 6]], np.int32)
        w = np.array([[0.625, 0.375], [0.5, 0.5], [0.875, 0.125]], np.float32)
        x = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=case)
                      for t in range(3)])
        for name, ks, flags in (("lut", ks5, 0), ("lut fixed order", ks5, pm.PM_DETERMINISTIC),
                                ("mixed", ks8, 0)):
            k = ks[case * 18:(case + 1) * 18].reshape(3, 2, 3).astype(np.uint8)
            y = torch.empty((3, wl.hidden), dtype=torch.float32, device="cuda")
            pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y, flags=flags)
            got = host(y)
            for t in range(3):
                want, S = oc.token_layer(wl, 0, ids[t], w[t], k[t], x[t], rows)
                assert_close(got[t][rows], want, S, f"case {case} token {t} {name} k={k[t].tolist()}")
    st.close()


# ---------------------------------------------------------------- MoE forward
def single_expert_store(wl, li=None):
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, 1)
    PoolFiller(wl).fill(st, 0, 0)
    return st


def test_forward_tiny_all_k_triples():
    report("forward, tiny expert, all 512 k triples")
    wl = synth.WORKLOADS[0]
    st = single_expert_store(wl)
    enc = oracle.encode_expert(synth.expert_inputs(wl, 0, 0), wl.group)
    x = synth.activation(wl.seed, 0, 0, 0, wl.hidden)
    xd = dev(x[None])
    ys = []
    triples = [(a, b, c) for a in range(1, 9) for b in range(1, 9) for c in range(1, 9)]
    for (a, b, c) in triples:
        y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, np.array([[0]]), np.array([[1.0]], np.float32),
                                np.array([[[a, b, c]]]), xd, y)
        ys.append(y)
    torch.cuda.synchronize()
    for (a, b, c), y in zip(triples, ys):
        r = oracle.expert_ffn(enc, a, b, c, x)
        assert_close(host(y)[0], r["y"], r["Sy"], f"k=({a},{b},{c})")
    st.close()


@pytest.fixture(scope="module")
def layer_store():
    """A 512-expert layer (hidden 4096, inter 1024, group 128); slots are filled on
    demand."""
    wl = synth.WORKLOADS[1]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    filled = set()

    def ensure(ids):
        for i in ids:
            if int(i) not in filled:
                filler.fill(st, 0, int(i))
                filled.add(int(i))
        torch.cuda.synchronize()

    yield wl, st, ensure
    st.close()


def test_forward_layer_full_size(layer_store):
    report("512-expert layer, one token, top-10, mean k 2.5, sampled rows")
    wl, st, ensure = layer_store
    ids, w, k = oc.route_and_bits(1, 0, step=0)
    # the product's routing and allocation agree with the oracle's
    pids, pw_ = pm.pm_route_topk(synth.router_logits(wl.seed, 1, 0, 0, wl.n_experts, step=0)[None], 10)
    assert pids[0].tolist() == ids.tolist()
    err = synth.error_profiles(wl.seed, 1, 0, wl.n_experts)
    assert pm.pm_allocate_bits(ids[None], w[None], err, wl.budget)[0].tolist() == k[:, 0].tolist()
    assert int(k[:, 0].sum()) == 25
    ensure(ids)
    x = synth.activation(wl.seed, 1, 0, 0, wl.hidden, step=0)
    y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids[None], w[None], k[None], dev(x[None]), y)
    got = host(y)[0]
    rows = oc.sample_rows(wl.hidden, 48, 1)
    want, S = oc.token_layer(1, 0, ids, w, k, x, rows)
    assert_close(got[rows], want, S, "512-expert layer, one token (combine folded into down)")
    # the separate fixed-order combine: the same bound, and a repeat gives
    # the same bits
    y2, y3 = torch.empty_like(y), torch.empty_like(y)
    for yy in (y2, y3):
        pm.pm_moe_token_forward(st, 0, ids[None], w[None], k[None], dev(x[None]), yy,
                                flags=pm.PM_DETERMINISTIC)
    assert_close(host(y2)[0][rows], want, S, "512-expert layer, one token (fixed-order combine)")
    assert np.array_equal(host(y3).view(np.uint32), host(y2).view(np.uint32))


def test_batch_of_four_matches_single_tokens(layer_store):
    """4 tokens x 10 uses in one call (two gate/up launches of LUT jobs)
    against each token alone, with the fixed-order combine
    (PM_DETERMINISTIC): every row is computed by one wave in one step
    whatever the launch, and the combine sums the uses in slot order, so a
    token whose experts no other token of the batch reads gets the same bits.
    Then eight single-token calls back to back, with no host sync between,
    repeat those bits.  The batch with the combine folded into the down
    launch (the default) against the oracle."""
    report("4-token batch vs single tokens, then 8 calls back to back")
    wl, st, ensure = layer_store
    routes = [oc.route_and_bits(1, 0, step=10 + t) for t in range(4)]
    ids = np.stack([r[0] for r in routes]).astype(np.int32)
    w = np.stack([r[1] for r in routes]).astype(np.float32)
    k = np.stack([r[2] for r in routes]).astype(np.uint8)
    ensure(np.unique(ids))
    x = np.stack([synth.activation(wl.seed, 1, 0, t, wl.hidden, step=10 + t) for t in range(4)])
    xd = dev(x)
    yb = torch.empty((4, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids, w, k, xd, yb, flags=pm.PM_DETERMINISTIC)
    batch = host(yb)
    yf = torch.empty((4, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids, w, k, xd, yf)
    folded = host(yf)
    counts = {int(i): int((ids == i).sum()) for i in np.unique(ids)}
    exact = 0
    alones = []
    for t in range(4):
        y1 = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids[t:t + 1], w[t:t + 1], k[t:t + 1], xd[t:t + 1], y1,
                                flags=pm.PM_DETERMINISTIC)
        alone = host(y1)[0]
        alones.append(alone)
        if all(counts[int(i)] == 1 for i in ids[t]):
            assert np.array_equal(alone.view(np.uint32), batch[t].view(np.uint32)), t
            exact += 1
        rows = oc.sample_rows(wl.hidden, 16, 30 + t)
        want, S = oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows)
        assert_close(alone[rows], want, S, f"token {t} alone")
        assert_close(batch[t][rows], want, S, f"token {t} in the batch")
        assert_close(folded[t][rows], want, S, f"token {t} in the batch, combine folded")
    assert exact >= 2
    ys = [torch.full((1, wl.hidden), 7.0, dtype=torch.float32, device="cuda") for _ in range(8)]
    for i in range(8):
        t = i % 4
        pm.pm_moe_token_forward(st, 0, ids[t:t + 1], w[t:t + 1], k[t:t + 1], xd[t:t + 1], ys[i],
                                flags=pm.PM_DETERMINISTIC)
    for i in range(8):
        assert np.array_equal(host(ys[i])[0].view(np.uint32), alones[i % 4].view(np.uint32)), i


@pytest.mark.parametrize("kfix", [4, 8, None])
def test_forward_uniform_precisions_and_materialize(layer_store, kfix):
    report(f"512-expert layer at k={kfix or 'mixed'}: direct and materialize-fp16")
    wl, st, ensure = layer_store
    ids, w, k = oc.route_and_bits(1, 0, step=0, kfix=kfix)
    ensure(ids)
    x = synth.activation(wl.seed, 1, 0, 0, wl.hidden, step=0)
    y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids[None], w[None], k[None], dev(x[None]), y)
    rows = oc.sample_rows(wl.hidden, 24, 2)
    want, S = oc.token_layer(1, 0, ids, w, k, x, rows)
    assert_close(host(y)[0][rows], want, S, f"direct k={kfix}")
    # the materialize-then-GEMV comparator on the first selected expert's gate
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pp, lp = pm.pm_store_slot(st, 0, int(ids[0]))
    po, lo, sh = pm.pm_expert_matrix_offsets(e, 0)
    w16 = torch.empty(sh.rows * sh.cols, dtype=torch.int16, device="cuda")
    pm.pm_materialize_fp16(sh, int(k[0][0]), pp + 4 * po, pm.pm_expert_plane_words(e),
                           lp + 4 * lo, w16)
    yg = torch.empty(sh.rows, dtype=torch.float32, device="cuda")
    pm.pm_gemv_fp16(sh, w16, dev(x), yg)
    (pg, lg), _ = oc.gate_up(1, 0, int(ids[0]))
    wg, sg = oracle.gemv_materialized_fp16(pg, lg, int(k[0][0]), wl.group, x)
    assert_close(host(yg), wg, sg, "materialized gate")


def test_forward_sixty_layers():
    report("60 layers x top-10, sampled rows on 2 layers")
    wl = synth.WORKLOADS[2]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, wl.n_layers, wl.n_experts)
    filler = PoolFiller(wl)
    plan = []
    for layer in range(wl.n_layers):
        ids, w, k = oc.route_and_bits(2, layer, step=0)
        for i in ids:
            filler.fill(st, layer, int(i))
        plan.append((ids, w, k))
    torch.cuda.synchronize()
    xs = [synth.activation(wl.seed, 2, layer, 0, wl.hidden) for layer in range(wl.n_layers)]
    ys = []
    for layer, (ids, w, k) in enumerate(plan):
        y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, layer, ids[None], w[None], k[None], dev(xs[layer][None]), y)
        ys.append(y)
    torch.cuda.synchronize()
    for layer in (0, 59):
        ids, w, k = plan[layer]
        rows = oc.sample_rows(wl.hidden, 16, 3 + layer)
        want, S = oc.token_layer(2, layer, ids, w, k, xs[layer], rows)
        assert_close(host(ys[layer])[0][rows], want, S, f"layer {layer}")
    st.close()


def test_forward_batch8_grouped_with_topup():
    report("B=8 grouped, 20% of experts topped up from pinned host")
    wl = synth.WORKLOADS[4]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    B = wl.n_tokens
    routes = [oc.route_and_bits(4, 0, step=0, token=t) for t in range(B)]
    ids = np.stack([r[0] for r in routes])
    w = np.stack([r[1] for r in routes])
    k = np.stack([r[2] for r in routes])
    distinct = sorted(set(int(i) for i in ids.reshape(-1)))
    for i in distinct:
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    kmax = {i: int(k[ids == i].max()) for i in distinct}
    cand = [i for i in distinct if kmax[i] >= 2]
    pick = synth.words(wl.seed, synth.KIND_TRUNC, 4, 0, 0, 0, len(cand)).argsort()
    n_short = int(np.ceil(0.2 * len(distinct)))
    short = [cand[int(j)] for j in pick[:n_short]]
    sources = {}
    expected_planes = 0
    syn = DeviceSynth()
    for j, i in enumerate(short):
        pp, lp = pm.pm_store_slot(st, 0, i)
        # keep a pinned host source of the full expert
        torch.cuda.synchronize()
        src_p = torch.empty(8 * pw, dtype=torch.int32, pin_memory=True)
        src_l = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        assert hip.hipMemcpy(ctypes.c_void_p(src_p.data_ptr()), ctypes.c_void_p(pp),
                             ctypes.c_size_t(8 * pw * 4), 2) == 0
        assert hip.hipMemcpy(ctypes.c_void_p(src_l.data_ptr()), ctypes.c_void_p(lp),
                             ctypes.c_size_t(src_l.numel() * 4), 2) == 0
        sources[i] = (src_p, src_l)
        pm.pm_store_attach_host(st, 0, i, src_p.data_ptr(), src_l.data_ptr())
        r = 1 + int(synth.words(wl.seed, synth.KIND_TRUNC, 4, 0, 1, j, 1)[0] % (kmax[i] - 1))
        pm.pm_store_truncate(st, 0, i, r)
        # truncation released the chunks past r; the slot's address for
        # direct writes holds all 8 again (r resident), and the rest is
        # poisoned: a top-up that copied too little would read it
        pp, _ = pm.pm_store_slot(st, 0, i)
        n_poison = (8 - r) * pw
        tmp = torch.empty(n_poison, dtype=torch.int32, device="cuda")
        syn.poison_into(tmp, 5, j)
        assert hip.hipMemcpy(ctypes.c_void_p(pp + 4 * r * pw), ctypes.c_void_p(tmp.data_ptr()),
                             ctypes.c_size_t(n_poison * 4), 3) == 0
        expected_planes += kmax[i] - r
    x = np.stack([synth.activation(wl.seed, 4, 0, t, wl.hidden) for t in range(B)])
    xd = dev(x)
    y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y)
    assert ei.value.status == pm.PM_ERR_NOT_RESIDENT
    _, _, planes_before, _ = pm.pm_store_copy_stats(st)
    pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y, flags=pm.PM_AUTO_TOPUP | pm.PM_DETERMINISTIC)
    got = host(y)
    _, _, planes_after, _ = pm.pm_store_copy_stats(st)
    assert planes_after - planes_before == expected_planes
    for i in short:
        assert pm.pm_store_resident(st, 0, i) == kmax[i]
    # each token of the batch equals that token run alone (fixed-order
    # combine): bit for bit when none of its experts is shared (same kernels,
    # same order); otherwise
    # (a shared expert's uses grouped) both within the oracle's per-output
    # bound
    counts = {i: int((ids == i).sum()) for i in distinct}
    rows = oc.sample_rows(wl.hidden, 8, 10)
    for t in range(B):
        y1 = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids[t:t + 1], w[t:t + 1], k[t:t + 1], xd[t:t + 1], y1,
                                flags=pm.PM_DETERMINISTIC)
        alone = host(y1)[0]
        if all(counts[int(i)] == 1 for i in ids[t]):
            assert np.array_equal(alone.view(np.uint32), got[t].view(np.uint32)), t
        want, S = oc.token_layer(4, 0, ids[t], w[t], k[t], x[t], rows)
        assert_close(got[t][rows], want, S, f"token {t} in the batch")
        assert_close(alone[rows], want, S, f"token {t} alone")
    st.close()


def test_read_once_matches_default():
    """PM_READ_ONCE (an expert shared by several tokens read once, by the
    direct kernels) against the default path (a LUT job per use) on a B = 8
    step: both against the oracle, and, with the fixed-order combine, bit for
    bit on the tokens none of whose experts is shared (their jobs are the
    same in both)."""
    report("B=8 routing, all resident: PM_READ_ONCE vs default")
    wl = synth.WORKLOADS[4]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    B = wl.n_tokens
    routes = [oc.route_and_bits(4, 0, step=5, token=t) for t in range(B)]
    ids = np.stack([r[0] for r in routes])
    w = np.stack([r[1] for r in routes])
    k = np.stack([r[2] for r in routes])
    for i in sorted(set(int(i) for i in ids.reshape(-1))):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    counts = {int(i): int((ids == i).sum()) for i in np.unique(ids)}
    assert max(counts.values()) >= 2, "the step should share an expert"
    x = np.stack([synth.activation(wl.seed, 4, 0, t, wl.hidden, step=5) for t in range(B)])
    xd = dev(x)
    out = {}
    for name, flags in (("default", 0), ("read_once", pm.PM_READ_ONCE),
                        ("default_fixed", pm.PM_DETERMINISTIC),
                        ("read_once_fixed", pm.PM_READ_ONCE | pm.PM_DETERMINISTIC)):
        y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y, flags=flags)
        out[name] = host(y)
    rows = oc.sample_rows(wl.hidden, 8, 30)
    for t in range(B):
        a, b = out["default_fixed"][t], out["read_once_fixed"][t]
        if all(counts[int(i)] == 1 for i in ids[t]):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), t
        want, S = oc.token_layer(4, 0, ids[t], w[t], k[t], x[t], rows)
        for name in out:
            assert_close(out[name][t][rows], want, S, f"{name}, token {t}")
    st.close()


@pytest.mark.parametrize("attach_first", [True, False])
def test_topup_waits_for_an_earlier_reader(attach_first):
    """A top-up must not overwrite planes that an earlier forward, still
    queued or running, reads.  The slot's host source holds another expert's
    planes, so a copy that ran too early would change the first result.
    Attached after the first forward, the source finds that forward's end
    unrecorded (a store without sources records none)."""
    report(f"top-up ordering (source attached {'before' if attach_first else 'after'} "
           "the first forward): forward, truncate, forward with top-up, no sync between")
    wl = synth.WORKLOADS[0]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    st = pm.pm_store_create(e, 1, 2)
    filler = PoolFiller(wl)
    filler.fill(st, 0, 0)
    filler.fill(st, 0, 1)
    torch.cuda.synchronize()
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    pp1, _ = pm.pm_store_slot(st, 0, 1)
    _, lp0 = pm.pm_store_slot(st, 0, 0)
    src_p = torch.empty(8 * pw, dtype=torch.int32, pin_memory=True)
    src_l = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
    assert hip.hipMemcpy(ctypes.c_void_p(src_p.data_ptr()), ctypes.c_void_p(pp1),
                         ctypes.c_size_t(8 * pw * 4), 2) == 0
    assert hip.hipMemcpy(ctypes.c_void_p(src_l.data_ptr()), ctypes.c_void_p(lp0),
                         ctypes.c_size_t(src_l.numel() * 4), 2) == 0
    if attach_first:
        pm.pm_store_attach_host(st, 0, 0, src_p.data_ptr(), src_l.data_ptr())
    A = oracle.encode_expert(synth.expert_inputs(wl, 0, 0), wl.group)
    B = oracle.encode_expert(synth.expert_inputs(wl, 0, 1), wl.group)
    mixed = {"group": wl.group, "levels": A["levels"],
             "planes": [np.concatenate([A["planes"][m][:1], B["planes"][m][1:]]) for m in range(3)]}
    xs = [synth.activation(wl.seed, 0, 0, 0, wl.hidden, step=s) for s in range(2)]
    ys = [torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda") for _ in range(2)]
    # inputs on the device beforehand: a copy inside the loop would wait for
    # the first forward and close the window this test is about
    xd = [dev(x[None]) for x in xs]
    torch.cuda.synchronize()
    ids = np.array([[0]], np.int32)
    w = np.array([[1.0]], np.float32)
    k = np.array([[[4, 4, 4]]], np.uint8)
    # a few milliseconds of queued work ahead of the first forward: a copy
    # that did not wait for it would land before it reads the planes
    busy = torch.randn(4096, 4096, device="cuda")
    for rep in range(4):
        for _ in range(4):
            busy = busy @ busy
            busy = busy / busy.abs().max()
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd[0], ys[0],
                                torch.cuda.current_stream())
        if rep == 0 and not attach_first:
            pm.pm_store_attach_host(st, 0, 0, src_p.data_ptr(), src_l.data_ptr())
        pm.pm_store_truncate(st, 0, 0, 1)
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd[1], ys[1], torch.cuda.current_stream(),
                                flags=pm.PM_AUTO_TOPUP)
        torch.cuda.synchronize()
        first = oracle.expert_ffn(A if rep == 0 else mixed, 4, 4, 4, xs[0])
        second = oracle.expert_ffn(mixed, 4, 4, 4, xs[1])
        assert_close(host(ys[0])[0], first["y"], first["Sy"], f"rep {rep}: earlier forward")
        assert_close(host(ys[1])[0], second["y"], second["Sy"], f"rep {rep}: after top-up")
    st.close()


@pytest.mark.parametrize("mfma", [False, True])
def test_topup_into_an_unallocated_slot(mfma):
    """Slots that hold no memory yet, with only a host source attached: the
    forward allocates them before it takes their addresses, then tops them
    up.  Expert 0 is read by all 8 tokens: gate at one prefix (a group of 8,
    matrix-core tiles), up at eight prefixes (LUT jobs at k <= 5, the direct
    kernels above), down at k = 2 by six tokens (tiles) and k = 7 by two
    (direct).  Expert 1 has three uses, experts 2..6 one each."""
    report(f"top-up into never-allocated slots ({'PM_BATCH_MFMA' if mfma else 'default'} path)")
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    wl = synth.WORKLOADS[1]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    n_exp = 7
    donor = pm.pm_store_create(e, 1, n_exp)
    filler = PoolFiller(wl)
    srcs = []
    for i in range(n_exp):
        filler.fill(donor, 0, i)
        torch.cuda.synchronize()
        pp, lp = pm.pm_store_slot(donor, 0, i)
        sp = torch.empty(8 * pw, dtype=torch.int32, pin_memory=True)
        sl = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
        assert hip.hipMemcpy(ctypes.c_void_p(sp.data_ptr()), ctypes.c_void_p(pp),
                             ctypes.c_size_t(8 * pw * 4), 2) == 0
        assert hip.hipMemcpy(ctypes.c_void_p(sl.data_ptr()), ctypes.c_void_p(lp),
                             ctypes.c_size_t(sl.numel() * 4), 2) == 0
        srcs.append((sp, sl))
    st = pm.pm_store_create(e, 1, n_exp)
    for i in range(n_exp):
        pm.pm_store_attach_host(st, 0, i, srcs[i][0].data_ptr(), srcs[i][1].data_ptr())
    B = 8
    ids = np.array([[0, o] for o in (1, 1, 1, 2, 3, 4, 5, 6)], np.int32)
    w = np.array([[0.5 + 0.05 * t, 0.5 - 0.05 * t] for t in range(B)], np.float32)
    k = np.zeros((B, 2, 3), np.uint8)
    for t in range(B):
        k[t, 0] = [3, t + 1, 2 if t < 6 else 7]
        k[t, 1] = [(3 * t) % 8 + 1, (5 * t + 2) % 8 + 1, (t + 4) % 8 + 1]
    x = np.stack([synth.activation(wl.seed, 1, 0, t, wl.hidden, step=21) for t in range(B)])
    xd = dev(x)
    flags = pm.PM_AUTO_TOPUP | pm.PM_DETERMINISTIC | (pm.PM_BATCH_MFMA if mfma else 0)
    y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y, flags=flags)
    got = host(y)
    want_res = [int(k[ids == i].max()) for i in range(n_exp)]
    assert want_res[0] == 8
    assert [pm.pm_store_resident(st, 0, i) for i in range(n_exp)] == want_res
    # the donor store holds the same planes: the same launches, the same bits
    y_ref = torch.empty_like(y)
    pm.pm_moe_token_forward(donor, 0, ids, w, k, xd, y_ref, flags=flags & ~pm.PM_AUTO_TOPUP)
    ref = host(y_ref)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    rows = oc.sample_rows(wl.hidden, 12, 21)
    for t in range(B):
        want, S = oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows)
        assert_close(got[t][rows], want, S, f"token {t}")
    st.close()
    donor.close()


def test_forward_topup_waits_for_a_pending_explicit_topup():
    """An explicit top-up still queued on the caller's stream, then a forward
    that needs a deeper prefix of the same slot: the forward's own copy goes
    to a store side stream, and the forward must still wait for both copies.
    The planes the first copy brings are poisoned beforehand, and the first
    copy is held back behind queued work, so a forward that waited only for
    its own copy would read the poison."""
    report("forward top-up after a pending explicit top-up on another stream")
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    wl = synth.WORKLOADS[0]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    st = pm.pm_store_create(e, 1, 1)
    PoolFiller(wl).fill(st, 0, 0)
    torch.cuda.synchronize()
    pp, lp = pm.pm_store_slot(st, 0, 0)
    src_p = torch.empty(8 * pw, dtype=torch.int32, pin_memory=True)
    src_l = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
    assert hip.hipMemcpy(ctypes.c_void_p(src_p.data_ptr()), ctypes.c_void_p(pp),
                         ctypes.c_size_t(8 * pw * 4), 2) == 0
    assert hip.hipMemcpy(ctypes.c_void_p(src_l.data_ptr()), ctypes.c_void_p(lp),
                         ctypes.c_size_t(src_l.numel() * 4), 2) == 0
    pm.pm_store_attach_host(st, 0, 0, src_p.data_ptr(), src_l.data_ptr())
    A = oracle.encode_expert(synth.expert_inputs(wl, 0, 0), wl.group)
    x = synth.activation(wl.seed, 0, 0, 0, wl.hidden, step=4)
    xd = dev(x[None])
    ids = np.array([[0]], np.int32)
    w = np.array([[1.0]], np.float32)
    k = np.array([[[5, 5, 5]]], np.uint8)
    want = oracle.expert_ffn(A, 5, 5, 5, x)
    side = torch.cuda.Stream()
    poison = torch.empty(7 * pw, dtype=torch.int32, device="cuda")
    DeviceSynth().poison_into(poison, 9, 0)
    busy = torch.randn(4096, 4096, device="cuda")
    for rep in range(3):
        pm.pm_store_truncate(st, 0, 0, 1)
        torch.cuda.synchronize()
        # the slot again holds all 8 chunks (plane 0 resident): the explicit
        # top-up and the forward's copy then write in place
        pp, _ = pm.pm_store_slot(st, 0, 0)
        assert hip.hipMemcpy(ctypes.c_void_p(pp + 4 * pw), ctypes.c_void_p(poison.data_ptr()),
                             ctypes.c_size_t(7 * pw * 4), 3) == 0
        with torch.cuda.stream(side):
            for _ in range(4):
                busy = busy @ busy
                busy = busy / busy.abs().max()
        pm.pm_store_topup(st, 0, 0, 3, side)
        y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y, torch.cuda.current_stream(),
                                flags=pm.PM_AUTO_TOPUP)
        torch.cuda.synchronize()
        assert pm.pm_store_resident(st, 0, 0) == 5
        assert_close(host(y)[0], want["y"], want["Sy"], f"rep {rep}")
    st.close()
