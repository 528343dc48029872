"""GPU parity of the matrix-core batch path (PM_BATCH_MFMA) against the CPU
oracle, through the C ABI: a batch crowded onto few experts (tiles split by
prefix and by 16 uses, every k from 1 to 8, gate, up and down at different
prefixes), a full-size 512-expert batch, agreement with the single-use path,
top-ups, and the shape check."""
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


def check_tokens(outs, ids, w, k, x, tokens, rows):
    """Every listed token of every output (name -> [B][hidden]) within the
    oracle's per-output bound on the sampled rows."""
    for t in tokens:
        want, S = oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows)
        for name, got in outs.items():
            assert_close(got[t][rows], want, S, f"{name}, token {t}")


def layer_batch(wl, n_tokens, top_k, n_exp, step):
    """Routing of n_tokens fresh tokens restricted to the first n_exp experts."""
    lg = np.stack([synth.router_logits(wl.seed, wl.cfg, 0, t, wl.n_experts, step=step)
                   for t in range(n_tokens)])
    lg[:, n_exp:] = -np.inf
    ids, w = pm.pm_route_topk(lg, top_k)
    x = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=step)
                  for t in range(n_tokens)])
    return ids, w, x


@pytest.fixture(scope="module")
def store512():
    wl = synth.WORKLOADS[1]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    filled = set()

    def ensure(ids):
        for i in np.unique(ids):
            if int(i) not in filled:
                filler.fill(st, 0, int(i))
                filled.add(int(i))
        torch.cuda.synchronize()

    yield wl, st, ensure
    st.close()


def test_mfma_crowded_batch_all_k(store512):
    """48 tokens on 8 experts, top-4: about 24 uses per expert, so tiles split
    by prefix and by 16; every k from 1 to 8, and gate, up and down of one use
    at different prefixes."""
    report("PM_BATCH_MFMA: 48 tokens x top-4 on 8 experts, k 1..8 per matrix")
    wl, st, ensure = store512
    B, top_k = 48, 4
    ids, w, x = layer_batch(wl, B, top_k, 8, step=7)
    ensure(ids)
    k = np.zeros((B, top_k, 3), np.uint8)
    for t in range(B):
        for j in range(top_k):
            k[t, j] = [(t + j) % 8 + 1, (t + 2 * j + 3) % 8 + 1, (3 * t + j + 5) % 8 + 1]
    y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y, flags=pm.PM_BATCH_MFMA)
    got = host(y)
    rows = oc.sample_rows(wl.hidden, 24, 5)
    for t in (0, 19, 47):
        want, S = oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows)
        assert_close(got[t][rows], want, S, f"token {t} k={k[t].tolist()}")
    # the same call through the default path (these experts carry enough
    # uses for its tiles): every token of both against the oracle's
    # per-output bound on sampled rows, and a repeat gives the same bits
    y1 = torch.empty_like(y)
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y1, flags=0)
    ref = host(y1)
    rows8 = oc.sample_rows(wl.hidden, 8, 15)
    check_tokens({"mfma": got, "default": ref}, ids, w, k, x, range(B), rows8)
    y2 = torch.empty_like(y)
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y2,
                            flags=pm.PM_BATCH_MFMA | pm.PM_DETERMINISTIC)
    assert np.array_equal(host(y2).view(np.uint32), got.view(np.uint32))
    y3 = torch.empty_like(y)
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y3, flags=pm.PM_DETERMINISTIC)
    assert np.array_equal(host(y3).view(np.uint32), ref.view(np.uint32))


def test_mfma_full_layer_batch(store512):
    """64 tokens, top-10 of 512 experts, allocator prefixes (mean 2.5)."""
    report("PM_BATCH_MFMA: 64 tokens x top-10 of 512 experts, mean k 2.5")
    wl, st, ensure = store512
    B = 64
    ids, w, x = layer_batch(wl, B, wl.top_k, wl.n_experts, step=11)
    ensure(ids)
    err = synth.error_profiles(wl.seed, wl.cfg, 0, wl.n_experts)
    kk = pm.pm_allocate_bits(ids, w, err, wl.budget)
    k = np.repeat(kk[:, :, None], 3, axis=2).astype(np.uint8)
    y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y, flags=pm.PM_BATCH_MFMA)
    got = host(y)
    rows = oc.sample_rows(wl.hidden, 16, 6)
    want, S = oc.token_layer(1, 0, ids[0], w[0], k[0], x[0], rows)
    assert_close(got[0][rows], want, S, "token 0")
    # tokens spread over the batch through both paths (another summation
    # order of the same products) against the oracle's per-output bound
    y1 = torch.empty_like(y)
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y1, flags=0)
    ref = host(y1)
    check_tokens({"mfma": got, "default": ref}, ids, w, k, x, range(0, B, 12),
                 oc.sample_rows(wl.hidden, 6, 16))


def test_mfma_with_topups_and_shape_check():
    report("PM_BATCH_MFMA: short slots topped up from pinned host; tiny shape rejected")
    wl = synth.WORKLOADS[1]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    st = pm.pm_store_create(e, 1, 4)
    filler = PoolFiller(wl)
    srcs = []
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    for i in range(4):
        filler.fill(st, 0, i)
        torch.cuda.synchronize()
        pp, lp = pm.pm_store_slot(st, 0, i)
        sp = torch.empty(8 * pw, dtype=torch.int32, pin_memory=True)
        sl = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
        assert hip.hipMemcpy(ctypes.c_void_p(sp.data_ptr()), ctypes.c_void_p(pp),
                             ctypes.c_size_t(8 * pw * 4), 2) == 0
        assert hip.hipMemcpy(ctypes.c_void_p(sl.data_ptr()), ctypes.c_void_p(lp),
                             ctypes.c_size_t(sl.numel() * 4), 2) == 0
        pm.pm_store_attach_host(st, 0, i, sp.data_ptr(), sl.data_ptr())
        srcs.append((sp, sl))
    B = 20
    ids = np.array([[t % 4, (t + 1) % 4] for t in range(B)], np.int32)
    w = np.full((B, 2), 0.5, np.float32)
    k = np.array([[[2, 3, 2], [4, 1, 5]] for _ in range(B)], np.uint8)
    x = np.stack([synth.activation(wl.seed, 1, 0, t, wl.hidden, step=3) for t in range(B)])
    for i in range(4):
        pm.pm_store_truncate(st, 0, i, 1)
    y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y, flags=pm.PM_BATCH_MFMA)
    assert ei.value.status == pm.PM_ERR_NOT_RESIDENT
    pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y,
                            flags=pm.PM_BATCH_MFMA | pm.PM_AUTO_TOPUP)
    got = host(y)
    assert all(pm.pm_store_resident(st, 0, i) == 5 for i in range(4))
    rows = oc.sample_rows(wl.hidden, 12, 8)
    for t in (0, 19):
        want, S = oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows)
        assert_close(got[t][rows], want, S, f"token {t}")
    st.close()
    tiny = synth.WORKLOADS[0]
    e0 = pm.eshape(tiny.hidden, tiny.inter, tiny.group)
    st0 = pm.pm_store_create(e0, 1, 1)
    PoolFiller(tiny).fill(st0, 0, 0)
    y0 = torch.empty((1, tiny.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st0, 0, np.array([[0]], np.int32), np.array([[1.0]], np.float32),
                                np.array([[[2, 2, 2]]], np.uint8),
                                dev(synth.activation(tiny.seed, 0, 0, 0, tiny.hidden)[None]), y0,
                                flags=pm.PM_BATCH_MFMA)
    assert ei.value.status == pm.PM_ERR_SHAPE
    # a call with more uses than jobs can name is refused before any work
    n_big = 32767 // 4 + 1
    xb = torch.zeros((n_big, tiny.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st0, 0, np.zeros((n_big, 4), np.int32),
                                np.full((n_big, 4), 0.25, np.float32),
                                np.full((n_big, 4, 3), 2, np.uint8), xb, torch.empty_like(xb))
    assert ei.value.status == pm.PM_ERR_ARG
    st0.close()


def test_default_path_large_batch(store512):
    """512 tokens, top-10 of 512 experts, allocator prefixes: the default path
    runs trains of full LUT launches (64 jobs each), cut per token, plus
    matrix-core tiles for the crowded (expert, matrix, k) groups.  Sampled
    tokens against the oracle; every token against PM_BATCH_MFMA."""
    report("default path: 512 tokens x top-10 of 512 experts, mean k 2.5")
    wl, st, ensure = store512
    B = 512
    ids, w, x = layer_batch(wl, B, wl.top_k, wl.n_experts, step=13)
    ensure(ids)
    err = synth.error_profiles(wl.seed, wl.cfg, 0, wl.n_experts)
    kk = pm.pm_allocate_bits(ids, w, err, wl.budget)
    k = np.repeat(kk[:, :, None], 3, axis=2).astype(np.uint8)
    xd = dev(x)
    y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
    pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y)
    got = host(y)
    rows = oc.sample_rows(wl.hidden, 8, 14)
    for t in (0, 255, 511):
        want, S = oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows)
        assert_close(got[t][rows], want, S, f"token {t}")
    y1 = torch.empty_like(y)
    pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y1, flags=pm.PM_BATCH_MFMA)
    ref = host(y1)
    check_tokens({"default": got, "mfma": ref}, ids, w, k, x, range(0, B, 100),
                 oc.sample_rows(wl.hidden, 6, 17))


@pytest.mark.parametrize("case", range(5))
def test_path_mixes_random(store512, case):
    """Seeded random calls that mix every path choice: batch sizes 3 to 33,
    top-2 to top-8 over 5 to 40 experts (so that experts are shared by up to
    about 30 uses), and an independent prefix 1..8 per (use, matrix).  The
    default path, PM_READ_ONCE and PM_BATCH_MFMA against the oracle on
    sampled tokens and rows, and against each other on every token."""
    wl, st, ensure = store512
    rng = np.random.default_rng(1000 + case)
    B = int(rng.integers(3, 34))
    top_k = int(rng.integers(2, 9))
    n_exp = int(rng.integers(max(top_k, 5), 41))
    report(f"random path mix {case}: B={B} top-{top_k} over {n_exp} experts")
    ids, w, x = layer_batch(wl, B, top_k, n_exp, step=40 + case)
    ensure(ids)
    k = rng.integers(1, 9, size=(B, top_k, 3)).astype(np.uint8)
    # a crowded prefix on one matrix of the most used expert, so that the
    # default path also forms a tile
    e0 = np.bincount(ids.reshape(-1)).argmax()
    k[..., 0][ids == e0] = 3
    xd = dev(x)
    outs = {}
    for name, flags in (("default", 0), ("read_once", pm.PM_READ_ONCE),
                        ("mfma", pm.PM_BATCH_MFMA)):
        y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, xd, y, flags=flags)
        outs[name] = host(y)
    # every token of every mode against the oracle's per-output bound
    check_tokens(outs, ids, w, k, x, range(B), oc.sample_rows(wl.hidden, 6, 50 + case))


def test_forward_degenerate_cases(store512):
    """Edge cases of one layer call, each against the oracle through every
    forward mode: no tokens; top-1; the same expert twice in one token; a
    zero routing weight; uses of one (expert, matrix, k) group exactly at the
    matrix-core threshold (6) and just below it (5)."""
    report("degenerate layer calls: empty, top-1, repeated expert, zero weight, tile threshold")
    wl, st, ensure = store512
    modes = (0, pm.PM_READ_ONCE, pm.PM_BATCH_MFMA)
    # no tokens: nothing to do, no error
    x0 = torch.empty((0, wl.hidden), dtype=torch.float32, device="cuda")
    for flags in modes:
        pm.pm_moe_token_forward(st, 0, np.zeros((0, 2), np.int32), np.zeros((0, 2), np.float32),
                                np.zeros((0, 2, 3), np.uint8), x0, torch.empty_like(x0),
                                flags=flags)
    rows = oc.sample_rows(wl.hidden, 6, 60)

    def check(ids, w, k, what):
        ids = np.asarray(ids, np.int32)
        w = np.asarray(w, np.float32)
        k = np.asarray(k, np.uint8)
        ensure(ids)
        B = ids.shape[0]
        x = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=61) for t in range(B)])
        wants = [oc.token_layer(1, 0, ids[t], w[t], k[t], x[t], rows) for t in range(B)]
        for flags in modes:
            y = torch.empty((B, wl.hidden), dtype=torch.float32, device="cuda")
            pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x), y, flags=flags)
            got = host(y)
            for t in range(B):
                assert_close(got[t][rows], wants[t][0], wants[t][1], f"{what}, flags {flags}, token {t}")

    check([[3], [4], [3]], [[1.0], [1.0], [1.0]], [[[2, 3, 4]], [[5, 1, 8]], [[8, 8, 8]]], "top-1")
    check([[5, 5]], [[0.6, 0.4]], [[[2, 2, 2], [4, 6, 1]]], "repeated expert")
    check([[6, 7]], [[1.0, 0.0]], [[[3, 3, 3], [2, 2, 2]]], "zero weight")
    # expert 8: gate at k = 3 for 6 uses (a tile in the default path), up at
    # k = 2 for 5 uses (LUT jobs) plus one at k = 7, down at k = 4 for all
    ids = [[8, 9 + t] for t in range(6)]
    w = [[0.7, 0.3]] * 6
    k = [[[3, 2 if t < 5 else 7, 4], [1 + t, 2, 3]] for t in range(6)]
    check(ids, w, k, "tile threshold")
