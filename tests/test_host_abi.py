"""Host side of libpm without a GPU: the library loads and exports every
symbol include/pm.h declares, the host encoder, routing and allocator match
the oracle exactly, the plane store's bookkeeping follows the pages'
residency examples, and invalid arguments fail before any HIP call."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import bitplane_quantized_expert_amd as pm
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "pm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 25
    L = pm.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in pm.SIGNATURES, n
    assert pm.lib().pm_version().startswith(b"libpm")


def test_layout_sizes_real_shape():
    g = pm.mshape(1024, 4096, 128)
    assert pm.pm_plane_words(g) == 131072
    assert pm.pm_levels_floats(g) == 1024 * 32 * 510
    assert pm.pm_level_offset(g, 1) == 0
    assert pm.pm_level_offset(g, 2) == 1024 * 32 * 2
    assert pm.pm_level_offset(g, 8) == 1024 * 32 * 254
    assert pm.pm_level_offset(g, 0) == 2 ** 64 - 1
    assert pm.pm_plane_words(pm.mshape(4, 100, 32)) == 0          # cols % group != 0
    e = pm.eshape(4096, 1024, 128)
    assert pm.pm_expert_plane_words(e) == 3 * 131072
    assert pm.pm_expert_levels_floats(e) == 3 * 1024 * 32 * 510
    pw, lf, sh = pm.pm_expert_matrix_offsets(e, 2)
    assert (pw, lf, sh.rows, sh.cols) == (2 * 131072, 2 * 1024 * 32 * 510, 4096, 1024)
    # 1..8-bit variants stored apart would take 1+2+...+8 = 36 bits per weight,
    # nine times one 4-bit copy; the 8 shared planes are 8 bits (PagedMoE
    # transcript, cues 11 and 27)
    assert sum(range(1, 9)) == 36 and 36 / 4 == 9
    assert pm.pm_expert_plane_words(e) * 32 * 8 // 8 == 3 * 1024 * 4096


def oracle_levels_flat(levels):
    """The oracle's {d: [rows][nb][2^d]} laid out as include/pm.h documents."""
    return np.concatenate([levels[d].reshape(-1) for d in range(1, 9)])


@pytest.mark.parametrize("weighted", [False, True])
def test_host_encoder_matches_oracle(weighted):
    wl = synth.WORKLOADS[0]
    li = synth.expert_inputs(wl, 0, 0)
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    pw = pm.pm_expert_plane_words(e)
    planes = np.zeros((8, pw), dtype=np.uint32)
    levels = np.zeros(pm.pm_expert_levels_floats(e), dtype=np.float32)
    counts = [oracle.leaf_counts(cd, wl.group).astype(np.uint32) for _, cd in li] if weighted else None
    pm.pm_encode_expert(e, [cd for _, cd in li], [lv for lv, _ in li], counts, planes, levels)
    enc = oracle.encode_expert(li, wl.group, weighted=weighted)
    for m in range(3):
        po, lo, sh = pm.pm_expert_matrix_offsets(e, m)
        n = pm.pm_plane_words(sh)
        assert np.array_equal(planes[:, po:po + n].reshape(8, sh.rows, sh.cols // 32), enc["planes"][m])
        nl = pm.pm_levels_floats(sh)
        got = levels[lo:lo + nl]
        want = oracle_levels_flat(enc["levels"][m])
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_encoder_rejects_bad_input():
    s = pm.mshape(2, 64, 32)
    codes = np.zeros((2, 64), dtype=np.uint8)
    leaves = np.tile(np.arange(256, dtype=np.float32), (2, 2, 1))
    planes = np.zeros((8, 4), dtype=np.uint32)
    levels = np.zeros(pm.pm_levels_floats(s), dtype=np.float32)
    pm.pm_encode_matrix(s, codes, leaves, None, planes, 4, levels)
    bad = leaves.copy()
    bad[1, 1, 7] = 1e9
    with pytest.raises(pm.PMError) as ei:
        pm.pm_encode_matrix(s, codes, bad, None, planes, 4, levels)
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:
        pm.pm_encode_matrix(pm.mshape(2, 64, 48), codes, leaves, None, planes, 4, levels)
    assert ei.value.status == pm.PM_ERR_SHAPE
    with pytest.raises(pm.PMError) as ei:
        pm.pm_encode_matrix(s, codes, leaves, None, planes, 3, levels)
    assert ei.value.status == pm.PM_ERR_ARG


def test_route_matches_oracle():
    wl = synth.WORKLOADS[1]
    lg = np.stack([synth.router_logits(wl.seed, 1, 0, 0, 512, step=t) for t in range(32)])
    ids, w = pm.pm_route_topk(lg, 10)
    for t in range(32):
        oi, ow = oracle.route(lg[t], 10)
        assert ids[t].tolist() == oi.tolist()
        assert np.all(np.abs(w[t].view(np.int32) - ow.view(np.int32)) <= 1)
    ids, w = pm.pm_route_topk(np.array([[0.5, 2.0, 2.0, -1.0, 1.0]], np.float32), 3)
    assert ids[0].tolist() == [1, 2, 4]


def test_allocator_matches_oracle():
    wl = synth.WORKLOADS[1]
    err = synth.error_profiles(wl.seed, 1, 0, 512)
    for t in range(24):
        oi, ow = oracle.route(synth.router_logits(wl.seed, 1, 0, 0, 512, step=t), 10)
        for budget in (10, 17, 25, 40, 80):
            k = pm.pm_allocate_bits(oi[None], ow[None], err, budget)[0]
            assert k.tolist() == oracle.allocate_bits(ow, err[oi], budget).tolist()
    g = json.load(open(os.path.join(GOLDEN, "allocator_and_residency.json")))
    for case in g["ties"]:
        err2 = np.array([[s * 4.0 ** -b for b in range(1, 9)] for s in case["scale"]])
        k = pm.pm_allocate_bits(np.array([[0, 1]]), np.array([case["w"]], np.float32), err2,
                                case["budget"])
        assert k[0].tolist() == case["want"]
    bumpy = np.array([[1.0, 0.9, 0.5, 0.45, 0.2, 0.19, 0.18, 0.1],
                      [1.0, 0.5, 0.25, 0.2, 0.1, 0.05, 0.04, 0.01]])
    w = np.array([[0.6, 0.4]], np.float32)
    for budget in range(2, 17):
        assert pm.pm_allocate_bits(np.array([[0, 1]]), w, bumpy, budget)[0].tolist() == \
            oracle.allocate_bits(w[0], bumpy, budget).tolist()
    with pytest.raises(pm.PMError):
        pm.pm_allocate_bits(np.array([[0, 1]]), w, bumpy, 1)


def fake_store(n_experts=2):
    e = pm.eshape(64, 32, 32)
    return e, pm.pm_store_create(e, 1, n_experts, 0, pm.PM_STORE_HOST_FAKE)


def test_store_residency_pages_examples():
    g = json.load(open(os.path.join(GOLDEN, "allocator_and_residency.json")))
    e, st = fake_store()
    pw = pm.pm_expert_plane_words(e)
    hp = (np.arange(8 * pw, dtype=np.uint32) * 2654435761).astype(np.uint32).reshape(8, pw)
    hl = np.arange(pm.pm_expert_levels_floats(e), dtype=np.float32)
    pm.pm_store_attach_host(st, 0, 1, hp, hl)
    for case in g["residency"]:
        pm.pm_store_truncate(st, 0, 1, 0)
        if case["resident"]:
            pm.pm_store_topup(st, 0, 1, case["resident"])
        assert pm.pm_store_resident(st, 0, 1) == case["resident"]
        pm.pm_store_topup(st, 0, 1, case["k"])
        first, count, _, _ = pm.pm_store_copy_stats(st)
        assert list(range(first, first + count)) == case["fetch"]
        assert pm.pm_store_resident(st, 0, 1) == max(case["resident"], case["k"])
    # a top-up copies the missing planes and leaves the resident ones alone
    pm.pm_store_truncate(st, 0, 1, 0)
    pm.pm_store_topup(st, 0, 1, 3)
    def view():
        # the slot's memory as written: plane chunks and levels (this grows
        # the slot to 8 chunks, keeping the resident prefix)
        pp, lp = pm.pm_store_slot(st, 0, 1)
        slot = np.ctypeslib.as_array(ctypes.cast(pp, ctypes.POINTER(ctypes.c_uint32)), (8, pw))
        lev = np.ctypeslib.as_array(ctypes.cast(lp, ctypes.POINTER(ctypes.c_float)), hl.shape)
        return slot, lev

    slot, lev = view()
    assert np.array_equal(slot[:3], hp[:3]) and np.array_equal(lev, hl)
    slot[3:] = 0
    slot[1] = 7                        # scribble over a resident plane
    pm.pm_store_truncate(st, 0, 1, 2)
    pm.pm_store_topup(st, 0, 1, 5)
    slot, _ = view()
    assert np.array_equal(slot[2:5], hp[2:5]) and np.all(slot[5:] == 0) and np.all(slot[1] == 7)
    st.close()


def test_store_memory_follows_residency():
    """Plane chunks are held for the resident prefix only: a top-up grows the
    slot to k chunks, a truncation releases the chunks past the kept prefix
    and, at 0, the levels [T c35: the deepest planes age out first]."""
    e, st = fake_store()
    pw = pm.pm_expert_plane_words(e)
    lf = pm.pm_expert_levels_floats(e)
    pb, lb = 4 * pw, 4 * lf
    hp = np.arange(8 * pw, dtype=np.uint32).reshape(8, pw)
    hl = np.arange(lf, dtype=np.float32)
    for x in (0, 1):
        pm.pm_store_attach_host(st, 0, x, hp, hl)
    assert pm.pm_store_usage(st) == (0, 0, 0)
    pm.pm_store_topup(st, 0, 0, 3)
    assert pm.pm_store_usage(st) == (3 * pb + lb, 3, 1)
    pm.pm_store_topup(st, 0, 1, 5)
    assert pm.pm_store_usage(st) == (8 * pb + 2 * lb, 8, 2)
    pm.pm_store_truncate(st, 0, 1, 2)
    assert pm.pm_store_usage(st) == (5 * pb + 2 * lb, 5, 2)
    assert pm.pm_store_resident(st, 0, 1) == 2
    pm.pm_store_truncate(st, 0, 1, 4)          # keeping more than is held changes nothing
    assert pm.pm_store_usage(st) == (5 * pb + 2 * lb, 5, 2)
    pm.pm_store_topup(st, 0, 1, 4)             # copies planes 2 and 3 only
    first, count, _, _ = pm.pm_store_copy_stats(st)
    assert (first, count) == (2, 2)
    assert pm.pm_store_usage(st) == (7 * pb + 2 * lb, 7, 2)
    pm.pm_store_truncate(st, 0, 0, 0)
    assert pm.pm_store_usage(st) == (4 * pb + lb, 4, 1)
    pm.pm_store_truncate(st, 0, 1, 0)
    assert pm.pm_store_usage(st) == (0, 0, 0)
    # a slot emptied and topped up again reads its levels again
    _, _, _, bytes0 = pm.pm_store_copy_stats(st)
    pm.pm_store_topup(st, 0, 1, 1)
    _, _, _, bytes1 = pm.pm_store_copy_stats(st)
    assert bytes1 - bytes0 == pb + lb
    # capacity counts chunks and levels: room for 3 more chunks, not 4
    st2 = pm.pm_store_create(e, 1, 2, 3 * pb + lb, pm.PM_STORE_HOST_FAKE)
    pm.pm_store_attach_host(st2, 0, 0, hp, hl)
    with pytest.raises(pm.PMError) as ei:
        pm.pm_store_topup(st2, 0, 0, 4)
    assert ei.value.status == pm.PM_ERR_OOM
    assert pm.pm_store_usage(st2) == (0, 0, 0)
    pm.pm_store_topup(st2, 0, 0, 3)
    assert pm.pm_store_usage(st2) == (3 * pb + lb, 3, 1)
    st2.close()
    st.close()


def test_store_slots_grow_and_shrink_in_place():
    """A truncation gives the tail of a slot's range back in place, and a
    top-up extends the range in place when the range after it is free, else
    moves the resident prefix (copied along) to a new range.  Every resident
    plane keeps the host source's words through all of it."""
    e, st = fake_store(3)
    pw = pm.pm_expert_plane_words(e)
    lf = pm.pm_expert_levels_floats(e)
    hp = [np.arange(8 * pw, dtype=np.uint32).reshape(8, pw) + np.uint32(1000003 * x) for x in range(3)]
    hl = np.arange(lf, dtype=np.float32)
    for x in range(3):
        pm.pm_store_attach_host(st, 0, x, hp[x], hl)

    def planes_of(x):
        p, _, n = pm.pm_store_slot_info(st, 0, x)
        r = pm.pm_store_resident(st, 0, x)
        assert n >= r
        return p, np.ctypeslib.as_array((ctypes.c_uint32 * (r * pw)).from_address(p)).reshape(r, pw)

    def check(x):
        r = pm.pm_store_resident(st, 0, x)
        _, got = planes_of(x)
        assert np.array_equal(got, hp[x][:r]), x

    pm.pm_store_topup(st, 0, 0, 2)
    pm.pm_store_topup(st, 0, 1, 2)             # right after slot 0's range
    a0 = planes_of(0)[0]
    pm.pm_store_truncate(st, 0, 0, 1)
    pm.pm_store_topup(st, 0, 0, 2)             # its own tail again: in place
    assert planes_of(0)[0] == a0
    check(0)
    pm.pm_store_topup(st, 0, 0, 5)             # slot 1 follows: moves
    a0b = planes_of(0)[0]
    assert a0b != a0
    check(0)
    check(1)
    pm.pm_store_truncate(st, 0, 0, 3)
    pm.pm_store_topup(st, 0, 0, 5)             # in place at the new range
    assert planes_of(0)[0] == a0b
    check(0)
    pm.pm_store_topup(st, 0, 2, 1)             # first fit: slot 0's old range
    assert planes_of(2)[0] == a0
    check(2)
    assert pm.pm_store_usage(st)[1] == 5 + 2 + 1
    st.close()


def test_forward_validates_every_item_before_any_allocation():
    """A layer call whose later item cannot be served changes nothing in the
    store: no slot memory is taken for the earlier items."""
    e, st = fake_store()
    pw = pm.pm_expert_plane_words(e)
    lf = pm.pm_expert_levels_floats(e)
    hp = np.zeros((8, pw), np.uint32)
    hl = np.zeros(lf, np.float32)
    pm.pm_store_attach_host(st, 0, 0, hp, hl)          # expert 1: no host source
    ids = np.array([[0, 1]], np.int32)
    w = np.array([[0.5, 0.5]], np.float32)
    k = np.full((1, 2, 3), 3, np.uint8)
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st, 0, ids, w, k, 16, 16, flags=pm.PM_AUTO_TOPUP)
    assert ei.value.status == pm.PM_ERR_STATE
    assert pm.pm_store_usage(st) == (0, 0, 0)
    assert pm.pm_store_resident(st, 0, 0) == 0
    st.close()
    # capacity for one expert's top-up but not for both
    pb, lb = 4 * pw, 4 * lf
    st = pm.pm_store_create(e, 1, 3, 3 * pb + lb + 8, pm.PM_STORE_HOST_FAKE)
    for x in (0, 1):
        pm.pm_store_attach_host(st, 0, x, hp, hl)
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st, 0, ids, w, k, 16, 16, flags=pm.PM_AUTO_TOPUP)
    assert ei.value.status == pm.PM_ERR_OOM
    assert pm.pm_store_usage(st) == (0, 0, 0)
    st.close()


def test_store_errors():
    e, st = fake_store()
    with pytest.raises(pm.PMError) as ei:
        pm.pm_store_topup(st, 0, 0, 4)
    assert ei.value.status == pm.PM_ERR_STATE
    with pytest.raises(pm.PMError) as ei:
        pm.pm_store_topup(st, 0, 0, 9)
    assert ei.value.status == pm.PM_ERR_PREFIX
    with pytest.raises(pm.PMError) as ei:
        pm.pm_store_resident(st, 0, 2)
    assert ei.value.status == pm.PM_ERR_ARG
    # the timing hook takes 2 or 4 events, or none
    L = pm.lib()
    two = (ctypes.c_void_p * 4)(1, 2, 3, 4)
    for n, ok in ((2, True), (4, True), (0, True), (3, False), (1, False)):
        rc = L.pm_store_set_profile_events(st.handle, two if n else None, n)
        assert (rc == 0) == ok, n
    assert L.pm_store_set_profile_events(st.handle, None, 0) == 0
    # a host-backed store cannot run a forward (its inputs pass validation)
    pm.pm_store_slot(st, 0, 0)
    pm.pm_store_set_resident(st, 0, 0, 8)
    with pytest.raises(pm.PMError) as ei:
        pm.pm_moe_token_forward(st, 0, np.zeros((1, 1)), np.ones((1, 1)), np.ones((1, 1, 3)),
                                16, 16)
    assert ei.value.status == pm.PM_ERR_STATE
    st.close()
    # capacity cap
    cap_e = pm.eshape(64, 32, 32)
    one_slot = 8 * pm.pm_expert_plane_words(cap_e) * 4 + pm.pm_expert_levels_floats(cap_e) * 4
    st = pm.pm_store_create(cap_e, 1, 3, one_slot + 10, pm.PM_STORE_HOST_FAKE)
    pm.pm_store_slot(st, 0, 0)
    with pytest.raises(pm.PMError) as ei:
        pm.pm_store_slot(st, 0, 1)
    assert ei.value.status == pm.PM_ERR_OOM
    st.close()


def test_validation_before_any_hip_call():
    s = pm.mshape(4, 64, 32)
    for k, code in ((0, pm.PM_ERR_PREFIX), (9, pm.PM_ERR_PREFIX)):
        with pytest.raises(pm.PMError) as ei:
            pm.pm_expert_gemv(s, k, 1, 8, 1, 1, 1)
        assert ei.value.status == code
    with pytest.raises(pm.PMError) as ei:
        pm.pm_expert_gemv(pm.mshape(4, 64, 40), 2, 1, 8, 1, 1, 1)
    assert ei.value.status == pm.PM_ERR_SHAPE
    with pytest.raises(pm.PMError) as ei:
        pm.pm_expert_gemv(s, 2, None, 8, 1, 1, 1)
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:
        pm.pm_expert_gemv(s, 2, 1, 7, 1, 1, 1)          # stride below the plane size
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:
        pm.pm_debug_dequant(s, 0, 1, 8, 1, 1)
    assert ei.value.status == pm.PM_ERR_PREFIX
    with pytest.raises(pm.PMError):
        pm.pm_route_topk(np.zeros((1, 4), np.float32), 5)
    # empty inputs are no-ops that touch nothing
    pm.pm_expert_gemv(pm.mshape(0, 64, 32), 3, None, 0, None, None, None)


def test_kmeans_validation_before_any_hip_call():
    with pytest.raises(pm.PMError) as ei:
        pm.pm_kmeans_codebook_device(pm.mshape(2, 8192, 8192), 1, 25, 1, 1, 1)
    assert ei.value.status == pm.PM_ERR_SHAPE
    with pytest.raises(pm.PMError) as ei:
        pm.pm_kmeans_codebook_device(pm.mshape(2, 128, 128), 1, -1, 1, 1, 1)
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:
        pm.pm_kmeans_codebook_device(pm.mshape(2, 128, 128), 1, 5, None, 1, 1)
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:
        pm.pm_kmeans_codebook_device(pm.mshape(2, 100, 50), 1, 5, 1, 1, 1)
    assert ei.value.status == pm.PM_ERR_SHAPE
    pm.pm_kmeans_codebook_device(pm.mshape(0, 128, 128), None, 5, None, None, None)


def test_noalloc_gemv_validation_before_any_hip_call():
    # the same checks as pm_expert_gemv, then the fixed scratch's limit on
    # rows x column slices, whichever kernel the shape would take
    lim = pm.PM_GEMV_NOALLOC_MAX_PARTIALS
    with pytest.raises(pm.PMError) as ei:
        pm.pm_expert_gemv_noalloc(pm.mshape(4, 64, 32), 9, 16, 8, 16, 16, 16)
    assert ei.value.status == pm.PM_ERR_PREFIX
    with pytest.raises(pm.PMError) as ei:
        pm.pm_expert_gemv_noalloc(pm.mshape(4, 64, 32), 2, 16, 8, 16, 8, 16)
    assert ei.value.status == pm.PM_ERR_ARG                 # x not 16-byte aligned
    for rows, cols, k in ((lim // 2 + 8, 2048, 3), (lim + 8, 1024, 7), (lim // 3 + 1, 2080, 2)):
        sh = pm.mshape(rows, cols, 32 if cols % 128 else 128)
        with pytest.raises(pm.PMError) as ei:
            pm.pm_expert_gemv_noalloc(sh, k, 16, rows * cols // 32, 16, 16, 16)
        assert ei.value.status == pm.PM_ERR_SHAPE, (rows, cols)
        assert b"scratch" in pm.lib().pm_last_error()
    pm.pm_expert_gemv_noalloc(pm.mshape(0, 64, 32), 3, None, 0, None, None, None)


def test_comparator_batches_validate_before_any_hip_call():
    s = pm.mshape(64, 256, 128)
    with pytest.raises(pm.PMError) as ei:                     # more than 64 matrices
        pm.pm_materialize_fp16_batch([s] * 65, [2] * 65, [16] * 65, [512] * 65, [16] * 65,
                                     [16] * 65)
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:                     # k out of range in the 2nd
        pm.pm_materialize_fp16_batch([s, s], [2, 9], [16, 16], [512, 512], [16, 16], [16, 16])
    assert ei.value.status == pm.PM_ERR_PREFIX
    with pytest.raises(pm.PMError) as ei:                     # output not 16-byte aligned
        pm.pm_materialize_fp16_batch([s], [2], [16], [512], [16], [24])
    assert ei.value.status == pm.PM_ERR_ARG
    with pytest.raises(pm.PMError) as ei:                     # rows of 100 columns: 200 bytes
        pm.pm_gemv_fp16_batch([pm.mshape(4, 100, 4)], [16], [16], [16])
    assert ei.value.status in (pm.PM_ERR_ARG, pm.PM_ERR_SHAPE)
    with pytest.raises(pm.PMError) as ei:
        pm.pm_gemv_fp16_batch([s], [None], [16], [16])
    assert ei.value.status == pm.PM_ERR_ARG
    pm.pm_materialize_fp16_batch([], [], [], [], [], [])      # an empty batch is a no-op
    pm.pm_gemv_fp16_batch([pm.mshape(0, 256, 128)], [None], [None], [None])
