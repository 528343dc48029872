"""Layer calls captured into a HIP graph (torch.cuda.graph on a side stream)
and replayed: every replay, with eager calls and host synchronisations
between the replays, against the eager results of the same calls.  With the
fixed-order combine (PM_DETERMINISTIC) the replays give the same bits; with
the combine folded into the down launch (the default), the same bound
against the oracle.  Through the C ABI."""
import numpy as np
import pytest
import torch

import bitplane_quantized_expert_amd as pm
import oracle
import oracle_cases as oc
import synth
from synth.pool import PoolFiller

pytestmark = pytest.mark.gpu
TOL = 1e-4
ABS = 1e-6
WL = synth.Workload(10, "wide-e8-h2048-i2048-g128", 2048, 2048, 128, 8, 2, 1, 3, 2.5)


def report(name):
    print(f"[gpu case] {name}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("flags", [pm.PM_DETERMINISTIC, 0])
def test_captured_layer_calls_replay_like_eager(flags):
    report(f"HIP graph of 3 layer calls, replayed 3 times (flags {flags})")
    wl = WL
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    ks = (synth.uniform_k(wl.seed, wl.cfg, 0, 3, 18).astype(np.int32) - 1) % 5 + 1
    calls = []
    for c in range(3):
        ids = np.array([[c % 8, (c + 3) % 8], [(c + 5) % 8, (c + 6) % 8], [c % 8, (c + 1) % 8]],
                       np.int32)
        w = np.array([[0.625, 0.375], [0.5, 0.5], [0.875, 0.125]], np.float32)
        k = np.roll(ks, 6 * c).reshape(3, 2, 3).astype(np.uint8)
        x = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=60 + c)
                      for t in range(3)])
        calls.append((ids, w, k, x, dev(x), torch.empty((3, wl.hidden), device="cuda")))
    cap = torch.cuda.Stream()

    def run_all(strm):
        for ids, w, k, _, xd, y in calls:
            pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y, strm, flags=flags)

    with torch.cuda.stream(cap):
        run_all(cap)
    torch.cuda.synchronize()
    eager = [y.cpu().numpy().copy() for *_, y in calls]
    rows = oc.sample_rows(wl.hidden, 16, 7)
    want = [[oc.token_layer(wl, 0, ids[t], w[t], k[t], x[t], rows) for t in range(3)]
            for ids, w, k, x, _, _ in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run_all(cap)
    other = torch.empty((3, wl.hidden), device="cuda")
    for rep in range(3):
        for *_, y in calls:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for c, (ids, w, k, x, xd, y) in enumerate(calls):
            got = y.cpu().numpy()
            if flags & pm.PM_DETERMINISTIC:
                assert np.array_equal(got.view(np.uint32), eager[c].view(np.uint32)), (rep, c)
            for t in range(3):
                yw, S = want[c][t]
                ok = oracle.within_tolerance(got[t][rows], yw, S, TOL, ABS)
                assert ok.all(), (rep, c, t)
        # eager work between the replays, on the default stream
        ids, w, k, _, xd, _ = calls[rep]
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd, other, flags=flags)
        torch.cuda.synchronize()
    st.close()


def test_capture_refuses_direct_path_and_topups():
    """Under stream capture a call that needs the direct kernels (a prefix
    above 5) or a top-up is refused with PM_ERR_STATE before it issues
    anything; the same call runs eagerly afterwards."""
    report("stream capture refuses direct-path and top-up calls")
    wl = WL
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    ids = np.array([[0, 1]], np.int32)
    w = np.array([[0.5, 0.5]], np.float32)
    x = dev(synth.activation(wl.seed, wl.cfg, 0, 0, wl.hidden, step=70)[None])
    y = torch.empty((1, wl.hidden), device="cuda")
    cap = torch.cuda.Stream()
    k_direct = np.array([[[2, 6, 3], [1, 1, 1]]], np.uint8)
    with torch.cuda.stream(cap):
        pm.pm_moe_token_forward(st, 0, ids, w, np.ones((1, 2, 3), np.uint8), x, y, cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(pm.PMError) as ei:
        with torch.cuda.graph(g, stream=cap):
            pm.pm_moe_token_forward(st, 0, ids, w, k_direct, x, y, cap)
    assert ei.value.status == pm.PM_ERR_STATE
    # a short slot with a host source: the top-up is refused as well
    pw = pm.pm_expert_plane_words(e)
    src = torch.zeros(8 * pw, dtype=torch.int32, pin_memory=True)
    lv = torch.zeros(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
    pm.pm_store_attach_host(st, 0, 2, src.data_ptr(), lv.data_ptr())
    pm.pm_store_truncate(st, 0, 2, 1)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(pm.PMError) as ei:
        with torch.cuda.graph(g2, stream=cap):
            pm.pm_moe_token_forward(st, 0, np.array([[2, 3]], np.int32), w,
                                    np.full((1, 2, 3), 3, np.uint8), x, y, cap,
                                    flags=pm.PM_AUTO_TOPUP)
    assert ei.value.status == pm.PM_ERR_STATE
    assert pm.pm_store_resident(st, 0, 2) == 1
    # eagerly, both run
    pm.pm_moe_token_forward(st, 0, ids, w, k_direct, x, y, cap)
    pm.pm_moe_token_forward(st, 0, np.array([[2, 3]], np.int32), w,
                            np.full((1, 2, 3), 3, np.uint8), x, y, cap, flags=pm.PM_AUTO_TOPUP)
    torch.cuda.synchronize()
    assert pm.pm_store_resident(st, 0, 2) == 3
    st.close()
