"""GPU tests of the plane store as a cache [T c13, c35]: a Zipf-routed token
trace replayed through a store far smaller than the expert pool, with the
prefix cache's decisions applied through top-ups and truncations, every
forward against the CPU oracle; and top-ups that race forwards still queued
on the device.  Through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import bitplane_quantized_expert_amd as pm
import oracle
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


def pinned_sources(wl, n_exp, gen=None):
    """Pinned host copies (planes, levels) of the device-encoded experts
    gen[i] (default i), in the store's slot layout."""
    gen = list(range(n_exp)) if gen is None else gen
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    donor = pm.pm_store_create(e, 1, 1)
    filler = PoolFiller(wl)
    hip = ctypes.CDLL("libamdhip64.so")
    out = []
    for i in range(n_exp):
        filler.fill(donor, 0, 0, gen_expert=gen[i])
        torch.cuda.synchronize()
        pp, lp = pm.pm_store_slot(donor, 0, 0)
        sp = torch.empty(8 * pw, dtype=torch.int32, pin_memory=True)
        sl = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
        assert hip.hipMemcpy(ctypes.c_void_p(sp.data_ptr()), ctypes.c_void_p(pp),
                             ctypes.c_size_t(8 * pw * 4), 2) == 0
        assert hip.hipMemcpy(ctypes.c_void_p(sl.data_ptr()), ctypes.c_void_p(lp),
                             ctypes.c_size_t(sl.numel() * 4), 2) == 0
        out.append((sp, sl))
    donor.close()
    return out


def token_ffn(experts, ids, w, k, x):
    """Oracle output of one token and its error scale: sum over its experts
    of w_j * expert_ffn at prefixes k[j] = (gate, up, down)."""
    y = np.zeros(x.shape[0])
    S = np.zeros(x.shape[0])
    for j, i in enumerate(ids):
        r = oracle.expert_ffn(experts[int(i)], int(k[j][0]), int(k[j][1]), int(k[j][2]), x)
        y += float(w[j]) * r["y"]
        S += abs(float(w[j])) * r["Sy"]
    return y, S


def test_zipf_trace_through_a_small_store():
    """48 tokens routed top-2 over 12 experts with Zipf popularity (s = 1),
    each use at its own (gate, up, down) prefixes.  The store may hold 24
    plane chunks, a quarter of the pool's 96.  Before each token the library's
    prefix cache takes the token's accesses one by one (checked against the
    oracle's PrefixPlaneCache, decision by decision); after each, the store
    drops the planes the cache evicted, and it reads the ones the cache lacks:
    by explicit top-ups on odd tokens, whose copies must be exactly the planes
    the cache reads, access by access, and by the forward's own top-ups on
    even tokens, whose copies must add up to the same.  The store's memory must equal the cache's resident
    planes after every token, and every output the oracle's."""
    report("Zipf trace (12 experts, top-2, 48 tokens) through a 24-plane store")
    wl = synth.WORKLOADS[0]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    pb = 4 * pw
    lb = 4 * pm.pm_expert_levels_floats(e)
    E, K, T, C = 12, 2, 48, 24
    srcs = pinned_sources(wl, E)
    experts = [oracle.encode_expert(synth.expert_inputs(wl, 0, i), wl.group) for i in range(E)]
    st = pm.pm_store_create(e, 1, E, C * pb + E * lb)
    for i in range(E):
        pm.pm_store_attach_host(st, 0, i, srcs[i][0].data_ptr(), srcs[i][1].data_ptr())
    cache = pm.pm_cache_create(E, C)
    ref = oracle.PrefixPlaneCache(C)
    ks = synth.words(wl.seed, synth.KIND_TRUNC, wl.cfg, 1, 0, 0, T * K * 3) % np.uint32(8) + 1
    ks = ks.astype(np.uint8).reshape(T, K, 3)
    copied = 0
    for t in range(T):
        lg = synth.zipf_router_logits(wl.seed, wl.cfg, 0, t, E, s=1.0)
        ids, w = oracle.route(lg, K)
        ids = np.asarray(ids, np.int32)[None]
        w = np.asarray(w, np.float32)[None]
        k = ks[t:t + 1]
        explicit = t % 2 == 1
        _, _, before, _ = pm.pm_store_copy_stats(st)
        reads = []
        for j in range(K):
            ex = int(ids[0, j])
            need = int(k[0, j].max())
            first, count = pm.pm_cache_access(cache, ex, need)
            want = ref.access(ex, need)
            assert list(range(first, first + count)) == want, (t, ex, need)
            reads.append(want)
            # this access's evictions shrink their slots at once (the planes
            # this token reads are the newest and are never the victims)
            for v in range(E):
                r_cache = pm.pm_cache_resident(cache, v)
                assert r_cache == ref.resident(v)
                if pm.pm_store_resident(st, 0, v) > r_cache:
                    pm.pm_store_truncate(st, 0, v, r_cache)
            if explicit:
                pm.pm_store_topup(st, 0, ex, need)
                first0, count, _, _ = pm.pm_store_copy_stats(st)
                if want:
                    assert (first0 + 1, count) == (want[0], len(want)), (t, ex)
                else:
                    assert count == 0, (t, ex)
        x = synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=31)
        y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")
        pm.pm_moe_token_forward(st, 0, ids, w, k, dev(x[None]), y,
                                flags=0 if explicit else pm.PM_AUTO_TOPUP)
        _, _, after, _ = pm.pm_store_copy_stats(st)
        n_read = sum(len(want) for want in reads)
        assert after - before == n_read, (t, after - before, n_read)
        copied += n_read
        res = [pm.pm_store_resident(st, 0, ex) for ex in range(E)]
        assert res == [ref.resident(ex) for ex in range(E)], t
        used, chunks, sets = pm.pm_store_usage(st)
        assert chunks == sum(res) <= C, t
        assert sets == sum(1 for r in res if r > 0), t
        assert used == chunks * pb + sets * lb, t
        want_y, S = token_ffn(experts, ids[0], w[0], k[0], x)
        assert_close(host(y)[0], want_y, S, f"token {t}")
    stats = pm.pm_cache_stats(cache)
    assert stats["planes_read"] == ref.planes_read == copied
    assert stats["accesses"] == T * K and stats["hits"] == ref.hits
    # the trace both hit and missed, and evicted: the store cycled memory
    assert 0 < ref.hits < T * K and copied > C
    cache.close()
    st.close()


@pytest.mark.parametrize("busy", [0, 2, 6])
def test_topups_of_slots_a_queued_forward_reads(busy):
    """Six late slots in one forward: three were read (and topped up) by a
    forward still queued behind `busy` matrix products, three were not.  The
    host sources hold other experts' planes than the device did (the levels
    are the device's own), so a top-up that did not happen, or that ran
    before the queued forward read the slot, changes a result.  Each slot's
    planes are tracked by origin; the copies must be exactly the missing
    planes, and both forwards must match the oracle."""
    report(f"top-ups of slots read by a queued forward ({busy} products queued ahead)")
    wl = synth.WORKLOADS[0]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    n = 6
    A = [oracle.encode_expert(synth.expert_inputs(wl, 0, i), wl.group) for i in range(n)]
    B = [oracle.encode_expert(synth.expert_inputs(wl, 0, n + i), wl.group) for i in range(n)]
    own = pinned_sources(wl, n)
    other = pinned_sources(wl, n, gen=[n + i for i in range(n)])
    st = pm.pm_store_create(e, 1, n)
    filler = PoolFiller(wl)
    for i in range(n):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    for i in range(n):
        # planes of expert n + i, levels of expert i
        pm.pm_store_attach_host(st, 0, i, other[i][0].data_ptr(), own[i][1].data_ptr())
    origin = [[0] * 8 for _ in range(n)]          # 0: expert i's plane, 1: expert n + i's

    def mixed(i):
        return {"group": wl.group, "levels": A[i]["levels"],
                "planes": [np.stack([(B if origin[i][p] else A)[i]["planes"][m][p]
                                     for p in range(8)]) for m in range(3)]}

    bz = torch.randn(2048, 2048, device="cuda")
    for rep in range(3):
        r = [1 + (i + rep) % 3 for i in range(n)]
        k1 = [r[i] + 2 for i in range(3)]
        for i in range(n):
            pm.pm_store_truncate(st, 0, i, r[i])
        torch.cuda.synchronize()
        x1 = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=40 + rep)
                       for t in range(3)])
        x2 = np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=50 + rep)
                       for t in range(n)])
        xd1, xd2 = dev(x1), dev(x2)
        y1 = torch.empty((3, wl.hidden), dtype=torch.float32, device="cuda")
        y2 = torch.empty((n, wl.hidden), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(busy):
            bz = bz @ bz
            bz = bz / bz.abs().max()
        ids1 = np.arange(3, dtype=np.int32)[:, None]
        ids2 = np.arange(n, dtype=np.int32)[:, None]
        w1 = np.ones((3, 1), np.float32)
        w2 = np.ones((n, 1), np.float32)
        kk1 = np.array([[[k1[i]] * 3] for i in range(3)], np.uint8)
        kk2 = np.full((n, 1, 3), 8, np.uint8)
        _, _, c0, _ = pm.pm_store_copy_stats(st)
        pm.pm_moe_token_forward(st, 0, ids1, w1, kk1, xd1, y1, flags=pm.PM_AUTO_TOPUP)
        pm.pm_moe_token_forward(st, 0, ids2, w2, kk2, xd2, y2, flags=pm.PM_AUTO_TOPUP)
        _, _, c1, _ = pm.pm_store_copy_stats(st)
        assert c1 - c0 == sum(8 - ri for ri in r), (rep, c1 - c0)
        assert [pm.pm_store_resident(st, 0, i) for i in range(n)] == [8] * n
        # the oracle's view: plane p of slot i came from the host source iff p >= r_i
        snap1 = []
        for i in range(3):
            for p in range(r[i], k1[i]):
                origin[i][p] = 1
            snap1.append(mixed(i))
        for i in range(n):
            for p in range(r[i], 8):
                origin[i][p] = 1
        got1, got2 = host(y1), host(y2)
        for t in range(3):
            want = oracle.expert_ffn(snap1[t], k1[t], k1[t], k1[t], x1[t])
            assert_close(got1[t], want["y"], want["Sy"], f"rep {rep}: first forward, token {t}")
        for t in range(n):
            want = oracle.expert_ffn(mixed(t), 8, 8, 8, x2[t])
            assert_close(got2[t], want["y"], want["Sy"], f"rep {rep}: second forward, token {t}")
    st.close()
