"""The library's expert caches (pm_cache_*) against the oracle's plane-aging
prefix cache, independent-object cache and downward-reuse cache: the
hand-worked golden traces,
seeded random traces at many capacities and a Zipf routing trace with
allocator-chosen prefixes.  Reads, residency and counters must agree exactly
after every access.  Host only."""
import json
import os

import numpy as np
import pytest

import bitplane_quantized_expert_amd as pm
import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def reads_of(first, count):
    return list(range(first, first + count))


POLICIES = [pm.PM_CACHE_PREFIX, pm.PM_CACHE_OBJECTS, pm.PM_CACHE_DOWNWARD]


def oracle_cache(policy, cap):
    return {pm.PM_CACHE_PREFIX: oracle.PrefixPlaneCache, pm.PM_CACHE_OBJECTS: oracle.ObjectCache,
            pm.PM_CACHE_DOWNWARD: oracle.DownwardCache}[policy](cap)


def oracle_resident(policy, oc, e):
    if policy != pm.PM_CACHE_OBJECTS:
        return oc.resident(e)
    return max([k for (x, k) in oc.order if x == e], default=0)


def stats_match(c, oc):
    st = pm.pm_cache_stats(c)
    held = len(oc.order) if isinstance(oc, oracle.PrefixPlaneCache) else oc.used
    assert (st["accesses"], st["hits"], st["partial"], st["planes_read"], st["planes_held"]) == \
        (oc.accesses, oc.hits, oc.partial, oc.planes_read, held)


def replay_both(policy, cap, n_experts, trace):
    c = pm.pm_cache_create(n_experts, cap, policy)
    oc = oracle_cache(policy, cap)
    for e, k in trace:
        got = reads_of(*pm.pm_cache_access(c, int(e), int(k)))
        assert got == oc.access(int(e), int(k)), (e, k)
        for x in range(n_experts):
            assert pm.pm_cache_resident(c, x) == oracle_resident(policy, oc, x)
    stats_match(c, oc)
    return c, oc


def test_golden_trace():
    g = json.load(open(os.path.join(GOLDEN, "plane_cache_trace.json")))
    for policy, key in ((pm.PM_CACHE_PREFIX, "prefix"), (pm.PM_CACHE_OBJECTS, "objects")):
        c = pm.pm_cache_create(4, g["capacity"], policy)
        for i, (e, k) in enumerate(g["trace"]):
            assert reads_of(*pm.pm_cache_access(c, e, k)) == g[key]["reads"][i]
            if policy == pm.PM_CACHE_PREFIX:
                want = {int(x): r for x, r in g[key]["resident_after"][i].items()}
                assert {x: pm.pm_cache_resident(c, x) for x in range(4)} == \
                    {x: want.get(x, 0) for x in range(4)}
        st = pm.pm_cache_stats(c)
        assert st["planes_read"] == g[key]["planes_read"] and st["hits"] == g[key]["hits"]
        if policy == pm.PM_CACHE_PREFIX:
            assert st["partial"] == g[key]["partial"]
    d = pm.pm_cache_create(4, g["capacity"], pm.PM_CACHE_DOWNWARD)
    g2 = json.load(open(os.path.join(GOLDEN, "plane_cache_downward_trace.json")))
    for (e, k), want in zip(g["trace"], g2["first_trace_downward"]["reads"]):
        assert reads_of(*pm.pm_cache_access(d, e, k)) == want


def test_golden_downward_trace():
    g = json.load(open(os.path.join(GOLDEN, "plane_cache_downward_trace.json")))
    for policy, key in ((pm.PM_CACHE_PREFIX, "prefix"), (pm.PM_CACHE_OBJECTS, "objects"),
                        (pm.PM_CACHE_DOWNWARD, "downward")):
        c = pm.pm_cache_create(3, g["capacity"], policy)
        for i, (e, k) in enumerate(g["trace"]):
            assert reads_of(*pm.pm_cache_access(c, e, k)) == g[key]["reads"][i]
            after = g[key].get("resident_after", g[key].get("width_after"))
            if after is not None:
                want = {int(x): r for x, r in after[i].items()}
                assert {x: pm.pm_cache_resident(c, x) for x in range(3)} == \
                    {x: want.get(x, 0) for x in range(3)}
        st = pm.pm_cache_stats(c)
        assert (st["planes_read"], st["hits"]) == (g[key]["planes_read"], g[key]["hits"])


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("cap", [0, 1, 3, 8, 9, 17, 40, 200])
def test_random_traces_match_oracle(policy, cap):
    n_experts = 11
    for seed in range(3):
        n = 400
        ex = synth.words(seed, synth.KIND_TRUNC, 0, 1, 0, 0, n) % np.uint32(n_experts)
        ks = synth.uniform_k(seed, 0, 2, 0, n)
        replay_both(policy, cap, n_experts, list(zip(ex.tolist(), ks.tolist())))


def zipf_allocated_trace(n_layers, n_experts, top_k, n_tokens, budget, s=1.0, cfg=1):
    """(cache expert id, k) of every use, tokens outermost, then layers, then
    the router's slot order; k from the library's pre-I/O allocator."""
    seed = synth.BASE_SEED + cfg
    out = []
    err = [synth.error_profiles(seed, cfg, layer, n_experts) for layer in range(n_layers)]
    for t in range(n_tokens):
        for layer in range(n_layers):
            lg = synth.zipf_router_logits(seed, cfg, layer, t, n_experts, s)
            ids, w = pm.pm_route_topk(lg[None], top_k)
            k = pm.pm_allocate_bits(ids, w, err[layer], budget)[0]
            out += [(layer * n_experts + int(e), int(b)) for e, b in zip(ids[0], k)]
    return out


@pytest.mark.parametrize("policy", POLICIES)
def test_zipf_allocated_trace_matches_oracle(policy):
    trace = zipf_allocated_trace(2, 64, 4, 60, 10)
    c = pm.pm_cache_create(128, 90, policy)
    oc = oracle_cache(policy, 90)
    for e, k in trace:
        assert reads_of(*pm.pm_cache_access(c, e, k)) == oc.access(e, k)
    stats_match(c, oc)
    # the batch entry point makes the same decisions
    c2 = pm.pm_cache_create(128, 90, policy)
    pm.pm_cache_replay(c2, np.array([e for e, _ in trace]), np.array([k for _, k in trace]))
    assert pm.pm_cache_stats(c2) == pm.pm_cache_stats(c)
    for x in range(128):
        assert pm.pm_cache_resident(c2, x) == pm.pm_cache_resident(c, x)


def test_unbounded_capacity_closed_forms():
    # nothing is ever evicted: the prefix cache reads max_k per expert, the
    # object cache k once per distinct (expert, k)
    ex = synth.words(5, synth.KIND_TRUNC, 0, 3, 0, 0, 500) % np.uint32(17)
    ks = synth.uniform_k(5, 0, 4, 0, 500)
    pairs = list(zip(ex.tolist(), ks.tolist()))
    c = pm.pm_cache_create(17, 17 * 8, pm.PM_CACHE_PREFIX)
    pm.pm_cache_replay(c, ex.astype(np.int32), ks)
    deepest = {}
    for e, k in pairs:
        deepest[e] = max(deepest.get(e, 0), k)
    assert pm.pm_cache_stats(c)["planes_read"] == sum(deepest.values())
    o = pm.pm_cache_create(17, 17 * 36, pm.PM_CACHE_OBJECTS)
    pm.pm_cache_replay(o, ex.astype(np.int32), ks)
    assert pm.pm_cache_stats(o)["planes_read"] == sum(k for _, k in set(pairs))


def test_pages_examples():
    # resident 3, request 5: planes 4 and 5; resident 5 (or 6), request 3: nothing
    c = pm.pm_cache_create(1, 8, pm.PM_CACHE_PREFIX)
    assert pm.pm_cache_access(c, 0, 3) == (1, 3)
    assert pm.pm_cache_access(c, 0, 5) == (4, 2)
    assert pm.pm_cache_access(c, 0, 3) == (4, 0)
    assert pm.pm_cache_access(c, 0, 6) == (6, 1)
    assert pm.pm_cache_access(c, 0, 3) == (4, 0)
    # the object cache cannot serve 4 bits from a resident 2-bit copy
    o = pm.pm_cache_create(1, 36, pm.PM_CACHE_OBJECTS)
    assert pm.pm_cache_access(o, 0, 2) == (1, 2)
    assert pm.pm_cache_access(o, 0, 4) == (1, 4)
    assert pm.pm_cache_access(o, 0, 2) == (3, 0)
    # all eight widths of one expert held side by side: 36 planes
    for k in range(1, 9):
        pm.pm_cache_access(o, 0, k)
    assert pm.pm_cache_stats(o)["planes_held"] == 36


def test_errors_leave_state_unchanged():
    with pytest.raises(pm.PMError) as ei:
        pm.pm_cache_create(4, 8, 3)
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError):
        pm.pm_cache_create(0, 8)
    with pytest.raises(pm.PMError):
        pm.pm_cache_create(4, -1)
    c = pm.pm_cache_create(4, 8)
    pm.pm_cache_access(c, 1, 2)
    before = pm.pm_cache_stats(c)
    for e, k, st in ((4, 2, pm.PM_ERR_ARG), (-1, 2, pm.PM_ERR_ARG), (0, 0, pm.PM_ERR_PREFIX),
                     (0, 9, pm.PM_ERR_PREFIX)):
        with pytest.raises(pm.PMError) as ei:
            pm.pm_cache_access(c, e, k)
        assert ei.value.status == st
    with pytest.raises(pm.PMError):
        pm.pm_cache_replay(c, np.array([0, 1, 5], np.int32), np.array([1, 2, 3], np.int32))
    assert pm.pm_cache_stats(c) == before
    assert pm.pm_cache_resident(c, 1) == 2
