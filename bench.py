#!/usr/bin/env python3
"""Benchmark of direct bitplane-prefix expert execution on one MI355X.

A step is one pm_moe_token_forward: one decode token through one MoE layer
of 512 SwiGLU experts (hidden 4096, intermediate 1024, group 128), top-10
routing, per-expert prefixes from the greedy allocator at a mean of 2.5 bits.
Every step draws a fresh token (router logits, activation), so consecutive
steps read different experts of the 512-expert pool (109 GB in HBM) and the
256 MB Infinity Cache cannot serve repeated reads.

The JSON line reports achieved GB/s on the algorithmic bytes (planes 0..k-1
plus depth-k codebook nodes of every selected matrix, plus x and y), the rate
of expert GEMVs, the roofline of the dominant kernel (HIP events on the
library's stream) and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + expert-GEMVs/s at avg 2.5-bit prefixes"
PEAK_HBM_GBS = 8000.0
# Device code whose HBM traffic the counters below describe.
KERNEL_SOURCES = ("bitplane_quantized_expert_amd/csrc/pm_lut.hip",
                  "bitplane_quantized_expert_amd/csrc/pm_device.h",
                  "bitplane_quantized_expert_amd/csrc/pm_internal.h")
# HBM bytes per gate/up launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# passes of this benchmark, each scaled by the same counter on the 1 GiB
# negation kernel (see --summarize-counters); reported only while the kernel
# sources still have this digest.
TRAFFIC = {"sources_sha256": "a9ac987c52bbecf3103744cb021b755c2935f7cc515fff29b4b40c8247085af2",
           "bytes_per_launch": 44683503}
# Mean kernel durations of the same step in a rocprofv3 kernel trace of
# graph-replayed steps (back to back, as in the timed loop): the gate/up
# launch, the down launch with the combine folded in, and the step from one
# gate/up start to the next; reported only while the kernel sources still
# have this digest.
TRACE = {"sources_sha256": TRAFFIC["sources_sha256"], "gateup_us": 12.08, "down_us": 8.60,
         "step_us": 21.14, "profile": "profiles/lut_kernel_moe_layer_e512_h4096_i1024_g128_k2.5.md"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def matrix_bytes(rows, cols, group, k):
    """Bytes one matrix read at prefix k moves: planes 0..k-1 and the depth-k
    nodes of every block."""
    return rows * cols * k // 8 + rows * (cols // group) * (1 << k) * 4


def step_bytes(wl, kk):
    """Algorithmic bytes of one token-layer step: payload of the 30 matrices
    at their prefixes, x read, y written (h is internal and not counted)."""
    b = 0
    for k3 in kk:
        for m in range(3):
            r, c = (wl.inter, wl.hidden) if m < 2 else (wl.hidden, wl.inter)
            b += matrix_bytes(r, c, wl.group, int(k3[m]))
    return b + 2 * wl.hidden * 4


def grouped_bytes(wl, ids, k3):
    """Algorithmic bytes of one B-token layer call: every distinct expert once,
    each matrix at its largest prefix over the tokens that share it, plus the
    depth-k table of every distinct k it is read at; x read and y written per
    token."""
    b = 0
    for e in np.unique(ids):
        sel = k3[ids == e]                          # [uses][3]
        for m in range(3):
            r, c = (wl.inter, wl.hidden) if m < 2 else (wl.hidden, wl.inter)
            ks = sorted(set(int(v) for v in sel[:, m]))
            b += r * c * max(ks) // 8 + sum(r * (c // wl.group) * (1 << k) * 4 for k in ks)
    return b + 2 * len(ids) * wl.hidden * 4


PEAK_FP32_MFMA_TFLOPS = 157.3


def mfma_flops(wl, ids, k3):
    """Flops of one PM_BATCH_MFMA call: useful (2 per weight per use) and
    issued (every tile of up to 16 uses of one (expert, matrix, k) computes
    16 columns)."""
    useful = issued = 0
    for e in np.unique(ids):
        sel = k3[ids == e]
        for m in range(3):
            r, c = (wl.inter, wl.hidden) if m < 2 else (wl.hidden, wl.inter)
            n_by_k = np.bincount(sel[:, m].astype(np.int64), minlength=9)
            useful += 2 * r * c * int(n_by_k.sum())
            issued += 2 * r * c * 16 * int(sum((n + 15) // 16 for n in n_by_k))
    return useful, issued


def gateup_bytes(wl, kk):
    b = 0
    for k3 in kk:
        for m in range(2):
            b += matrix_bytes(wl.inter, wl.hidden, wl.group, int(k3[m]))
    return b + wl.hidden * 4


def routing_digest(ids, w, k):
    """SHA-256 over the exact ids (int32), w (fp32) and k (uint8) of every step,
    so that runs can be matched to their inputs (--log-inputs writes them)."""
    import hashlib
    h = hashlib.sha256()
    for a, t in ((ids, np.int32), (w, np.float32), (k, np.uint8)):
        h.update(np.ascontiguousarray(a, dtype=t).tobytes())
    return h.hexdigest()


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def summarize_counters(fetch_csv, write_csv, stats_csv):
    """Markdown summary of rocprofv3 runs of this benchmark: per-kernel mean
    duration (kernel trace) and HBM bytes per dispatch (FETCH_SIZE and
    WRITE_SIZE in KiB, each scaled by its reading on the 1 GiB negation
    kernel, which reads and writes exactly 1 GiB)."""
    import csv

    def per_kernel(path, col="Counter_Value"):
        out = {}
        for r in csv.DictReader(open(path)):
            out.setdefault(r["Kernel_Name"], []).append(float(r[col]))
        return out

    def short(name):
        for key, lab in (("lut_kernel<false, false>", "lut_kernel<false, false> (gate/up)"),
                         ("lut_kernel<true, true>", "lut_kernel<true, true> (down + combine)"),
                         ("lut_kernel<true, false>", "lut_kernel<true, false> (down)"),
                         ("combine_k_kernel", "combine_k_kernel"), ("neg_kernel", "torch.neg 1 GiB")):
            if key in name:
                return lab
        return None

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    ref = 1 << 20                                    # KiB in 1 GiB
    cal_f = ref / np.mean(next(v for k, v in fetch.items() if "neg_kernel" in k))
    cal_w = ref / np.mean(next(v for k, v in write.items() if "neg_kernel" in k))
    lines = ["| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM MB/dispatch (scaled) |",
             "|---|---|---|---|---|"]
    gate_up = None
    for k in fetch:
        lab = short(k)
        if lab is None or k not in write:
            continue
        f, w = float(np.mean(fetch[k])), float(np.mean(write[k]))
        mb = (f * cal_f + w * cal_w) * 1024 / 1e6
        if "gate/up" in lab:
            gate_up = (f * cal_f + w * cal_w) * 1024
        lines.append(f"| {lab} | {len(fetch[k])} | {f:.1f} | {w:.1f} | {mb:.2f} |")
    lines += ["", f"Scale factors: FETCH_SIZE x{cal_f:.3f}, WRITE_SIZE x{cal_w:.3f}.", "",
              "| kernel | calls | mean us | min us | max us |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        lab = short(r["Name"])
        if lab:
            lines.append(f"| {lab} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", f"gate/up HBM bytes per launch: {gate_up:.0f}",
              f"kernel sources sha256: {sources_digest()}"]
    return "\n".join(lines)


def copy_ceiling(torch, stream, nbytes=1 << 30, reps=5):
    """A plain elementwise kernel of known traffic (read nbytes, write
    nbytes, fp32 negation) on the same stream: the HBM rate this chip reaches
    on a pure stream, and the reference for the per-dispatch HBM counters."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").normal_()
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        torch.neg(a, out=b)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del a, b
    return {"kernel": "torch.neg fp32, 1 GiB read + 1 GiB written", "us": round(ms * 1e3, 1),
            "GBs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def gemv_share(wl, rows):
    """Expert GEMVs that one pass over an expert's three matrices cut to
    their first `rows` rows amounts to: each matrix counts rows / its rows
    (gate and up have `inter` rows, down has `hidden`), over three matrices."""
    import synth
    return sum(min(rows, synth.matrix_shape(wl, m)[0]) / synth.matrix_shape(wl, m)[0]
               for m in range(3)) / 3.0


def cpu_info():
    """CPU model (from /proc/cpuinfo) and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, usable


def cpu_baseline(wl, plans, budget_s, max_threads=16):
    """The oracle, untouched, on a bounded sample: the first token's 10
    experts, every matrix restricted to its first 256 rows, repeated until
    about budget_s / 2 seconds of oracle time, once on one thread and once
    with the matrices of a pass spread over the usable cores (at most
    max_threads worker threads, BLAS held to one thread in each)."""
    import concurrent.futures as cf
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    ids, w, kk = plans[0]
    rows = 256
    mats = []
    nbytes = 0
    gemv_equiv = 0.0            # expert GEMVs per pass: each matrix's share of its rows
    for j in range(len(ids)):
        for m in range(3):
            R, C = synth.matrix_shape(wl, m)
            lv = synth.leaves(wl.seed, wl.cfg, 0, int(ids[j]), m, R, C // wl.group, 0, rows)
            cd = synth.codes(wl.seed, wl.cfg, 0, int(ids[j]), m, R, C, 0, rows)
            x = synth.activation(wl.seed, wl.cfg, 0, 0, C)
            mats.append((oracle.pack_planes(cd), oracle.tree_levels(lv), int(kk[j][m]), x))
            nbytes += matrix_bytes(rows, C, wl.group, int(kk[j][m]))
        gemv_equiv += 3 * gemv_share(wl, rows)

    def one(mat):
        pl, lvl, k, x = mat
        oracle.gemv(pl, lvl, k, wl.group, x)

    def run(threads, seconds):
        limiter = threadpool_limits(limits=1) if threadpool_limits else None
        reps = 0
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            while True:
                if threads == 1:
                    for mat in mats:
                        one(mat)
                else:
                    list(ex.map(one, mats))
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
        if limiter is not None and hasattr(limiter, "unregister"):
            limiter.unregister()
        return reps, el

    model, usable = cpu_info()
    threads = max(1, min(usable, max_threads))
    reps1, el1 = run(1, budget_s / 2)
    repsn, eln = run(threads, budget_s / 2)
    one_thread = {"value": round(nbytes * reps1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                  "expert_gemvs_per_s": round(gemv_equiv * reps1 / el1, 3),
                  "passes": reps1, "seconds": round(el1, 1)}
    return {"value": round(nbytes * repsn / eln / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{len(mats)} matrices (10 experts x gate/up/down of step 0) x first "
                       f"{rows} rows; numpy fp64, BLAS one thread per worker; {repsn} passes in "
                       f"{eln:.1f} s on {threads} threads, then {reps1} passes in {el1:.1f} s on "
                       f"one thread"),
            "expert_gemvs_per_s": round(gemv_equiv * repsn / eln, 3),
            "single_thread": one_thread,
            "cpu_model": model, "usable_cores": usable}


def route_steps(pm, synth, wl, layer, steps, token=0, kfix=None, n_exp=None):
    """Product routing and allocation of `steps` fresh tokens of one layer:
    ids int32 [steps][top_k], w fp32, k uint8-ish [steps][top_k][3]."""
    err = synth.error_profiles(wl.seed, wl.cfg, layer, wl.n_experts)
    logits = np.stack([synth.router_logits(wl.seed, wl.cfg, layer, token, wl.n_experts, step=s)
                       for s in steps])
    if n_exp is not None and n_exp < wl.n_experts:
        logits[:, n_exp:] = -np.inf
    ids, w = pm.pm_route_topk(logits, wl.top_k)
    if kfix is None:
        kk = pm.pm_allocate_bits(ids, w, err, wl.budget)
    else:
        kk = np.full(ids.shape, kfix, np.int32)
    return ids, w, np.repeat(kk[:, :, None], 3, axis=2)


def timed(torch, fn, n):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def wg_timeline(pm, torch, run, steps, btb, groups=20, dump=None):
    """Workgroup timeline of the LUT launches (the stamped build): groups of
    `btb` steps run back to back; after each, the stamps of the group's last
    gate/up and down launches (s_memrealtime, 10 ns) give per launch:
    the span from the first workgroup's start to the last one's end, the
    spread of the starts, and per workgroup the prologue (start until the
    last wave computes) split into the builders' source load and their
    table, the duration and the end.  Medians over the groups of the
    per-launch figures (workgroup figures: their median, p90, max)."""
    import ctypes
    lib = pm.lib()
    lib.pm_lut_stamps_fetch.restype = ctypes.c_int
    lib.pm_lut_stamps_fetch.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    buf = np.zeros((2, 256 * 16, 12), np.uint64)
    per = {0: [], 1: []}
    raw = []
    for gi in range(groups):
        for i in range(btb):
            run(steps[(gi * btb + i) % len(steps)])
        torch.cuda.synchronize()
        assert lib.pm_lut_stamps_fetch(buf.ctypes.data, buf.nbytes) == 0
        if dump:
            raw.append(buf.copy())
        for down in (0, 1):
            b = buf[down].astype(np.int64)
            used = b[:, 4] > 0
            t = b[used]
            base = t[:, 0].min()
            per[down].append({
                "span": (t[:, 4].max() - base) / 100, "start_spread": (t[:, 0].max() - base) / 100,
                "prologue": np.median(t[:, 3] - t[:, 0]) / 100,
                "source": np.median(t[:, 1] - t[:, 0]) / 100,
                "table": np.median(t[:, 2] - t[:, 1]) / 100,
                "wg_median": np.median(t[:, 4] - t[:, 0]) / 100,
                "wg_p90": np.percentile(t[:, 4] - t[:, 0], 90) / 100,
                "wg_max": (t[:, 4] - t[:, 0]).max() / 100,
                "first_end": (t[:, 4].min() - base) / 100, "workgroups": int(used.sum()),
                "entry_spread": (t[:, 8].max() - t[:, 8].min()) / 100,
                "entry_to_start": np.median(t[:, 0] - t[:, 8]) / 100,
                **{f"k{k}_wg_median": float(np.median(t[t[:, 5] == k, 4] - t[t[:, 5] == k, 0]) / 100)
                   for k in range(1, 6) if (t[:, 5] == k).sum() >= 4}})
            b[:] = 0
        buf[:] = 0
    if dump:
        np.savez_compressed(dump, stamps=np.stack(raw))
    return {("down" if d else "gateup"): {k: round(float(np.median([r[k] for r in v if k in r])), 2)
                                          for k in sorted({k for r in v for k in r})}
            for d, v in per.items()}


def graph_replay(torch, cap, body, reps):
    """Capture body() (library calls on stream `cap`) into one HIP graph,
    replay it once, then `reps` more times: the same kernels with the same
    arguments, without the host's work per call.  Returns (graph, seconds per
    replay)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        body()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    return g, (time.perf_counter() - t0) / reps


def bench_sixty_layers(args, torch, pm, synth, PoolFiller):
    """One decode token through 60 independent layers (600 routed experts,
    all resident): a step is the 60 layer calls, fresh x and logits per layer."""
    wl = synth.WORKLOADS[2]
    st = pm.pm_store_create(pm.eshape(wl.hidden, wl.inter, wl.group), wl.n_layers, wl.n_experts)
    filler = PoolFiller(wl)
    plan, nbytes = [], 0
    for layer in range(wl.n_layers):
        ids, w, k3 = route_steps(pm, synth, wl, layer, [0])
        for i in ids[0]:
            filler.fill(st, layer, int(i))
        x = torch.from_numpy(synth.activation(wl.seed, wl.cfg, layer, 0, wl.hidden)[None]).cuda()
        plan.append((layer, ids, w, k3, x))
        nbytes += step_bytes(wl, k3[0])
    torch.cuda.synchronize()
    log(f"60-layer pool ready ({wl.n_layers * wl.top_k} experts)")
    y = torch.empty((1, wl.hidden), dtype=torch.float32, device="cuda")

    def token(_):
        for layer, ids, w, k3, x in plan:
            pm.pm_moe_token_forward(st, layer, ids, w, k3, x, y)

    timed(torch, token, max(2, args.warmup // 10))
    n = max(5, args.steps // 10)
    el = timed(torch, token, n)
    # the token's 60 layer calls captured into one HIP graph and replayed
    # (refused by the library if a layer needs the direct kernels)
    graph = {}
    try:
        cap = torch.cuda.Stream()

        def token_on(strm):
            for layer, ids, w, k3, x in plan:
                pm.pm_moe_token_forward(st, layer, ids, w, k3, x, y, strm)

        with torch.cuda.stream(cap):
            token_on(cap)          # the store's last stream becomes the capture stream
        torch.cuda.synchronize()
        eager_y = y.clone()
        _, g_el = graph_replay(torch, cap, lambda: token_on(cap), n)
        diff = float((y - eager_y).abs().max())
        graph = {"ms_per_token": round(g_el * 1e3, 4), "GBs": round(nbytes / g_el / 1e9, 1),
                 "replays": n, "max_abs_diff_vs_eager": diff,
                 "how": "the 60 layer calls of the token captured once on a side stream "
                        "(HIP graph), replayed; y of the last layer checked against the eager call"}
    except Exception as ex:
        graph = {"error": str(ex)[:300]}
    st.close()
    ms = el / n * 1e3
    return {"workload": wl.name, "ms_per_token": round(ms, 4),
            "GBs": round(nbytes * n / el / 1e9, 1),
            "expert_gemvs_per_s": round(3 * wl.top_k * wl.n_layers * n / el, 1),
            "bytes_per_token": nbytes, "hip_graph": graph}


def bench_precisions(args, torch, pm, synth, PoolFiller):
    """The one-layer step at k = 4, k = 8 and the mixed draw, each beside the
    materialize-then-GEMV comparator: the step's 30 matrices dequantized to
    fp16 in HBM by one launch (16-byte stores), then one fp16-weight GEMV
    launch for the 20 gate/up matrices and one for the 10 down matrices (the
    down input is a fixed vector: the comparator is timed, not checked, here).
    Its bytes: the prefix planes and tables read, the fp16 weights written and
    read again."""
    wl = synth.WORKLOADS[3]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    pw = pm.pm_expert_plane_words(e)
    offs = [pm.pm_expert_matrix_offsets(e, m) for m in range(3)]
    n_mat = 3 * wl.top_k
    w16 = torch.empty((n_mat, wl.hidden * wl.inter), dtype=torch.int16, device="cuda")
    yv = torch.empty((n_mat, wl.hidden), dtype=torch.float32, device="cuda")
    out = {}
    total = args.warmup + args.steps
    for label, kfix in (("k4", 4), ("k8", 8), ("mixed", None)):
        ids, w, k3 = route_steps(pm, synth, wl, 0, range(total), kfix=kfix)
        x = torch.from_numpy(np.stack([synth.activation(wl.seed, wl.cfg, 0, 0, wl.hidden, step=s)
                                       for s in range(total)])).cuda()
        hx = torch.randn(wl.inter, device="cuda")
        y = torch.empty_like(x)

        def direct(i, s0=args.warmup):
            s = s0 + i
            pm.pm_moe_token_forward(st, 0, ids[s:s + 1], w[s:s + 1], k3[s:s + 1], x[s:s + 1],
                                    y[s:s + 1], stream)

        # the comparator's launch arguments of every step, formed before timing
        margs = []
        for s in range(total):
            shapes, ks, pls, lvs = [], [], [], []
            for j in range(wl.top_k):
                pp, lp, _ = pm.pm_store_slot_info(st, 0, int(ids[s][j]))
                for m in range(3):
                    po, lo, sh = offs[m]
                    shapes.append(sh)
                    ks.append(int(k3[s][j][m]))
                    pls.append(pp + 4 * po)
                    lvs.append(lp + 4 * lo)
            gu = [q for q in range(n_mat) if q % 3 < 2]
            dn = [q for q in range(n_mat) if q % 3 == 2]
            margs.append((shapes, ks, pls, lvs,
                          ([shapes[q] for q in gu], [w16[q] for q in gu], [x[s]] * len(gu),
                           [yv[q] for q in gu]),
                          ([shapes[q] for q in dn], [w16[q] for q in dn], [hx] * len(dn),
                           [yv[q] for q in dn])))

        def materialize(i, s0=args.warmup):
            shapes, ks, pls, lvs, gu, dn = margs[s0 + i]
            pm.pm_materialize_fp16_batch(shapes, ks, pls, [pw] * n_mat, lvs, list(w16), stream)
            pm.pm_gemv_fp16_batch(*gu, stream)
            pm.pm_gemv_fp16_batch(*dn, stream)

        n = args.steps
        timed(torch, lambda i: direct(i, 0), min(args.warmup, 20))
        el_d = timed(torch, direct, n)
        nm = max(5, n // 10)
        timed(torch, lambda i: materialize(i, 0), 2)
        el_m = timed(torch, materialize, nm)
        b = np.mean([step_bytes(wl, k3[args.warmup + i]) for i in range(n)])
        bm = np.mean([step_bytes(wl, k3[args.warmup + i]) for i in range(nm)]) + \
            3 * wl.top_k * wl.hidden * wl.inter * 4
        out[label] = {"direct_us": round(el_d / n * 1e6, 2), "direct_GBs": round(b * n / el_d / 1e9, 1),
                      "materialize_us": round(el_m / nm * 1e6, 2),
                      "materialize_GBs": round(bm * nm / el_m / 1e9, 1),
                      "materialize_pct_of_peak": round(100 * bm * nm / el_m / 1e9 / PEAK_HBM_GBS, 1),
                      "speedup": round((el_m / nm) / (el_d / n), 2), "bytes_per_step": int(b),
                      "materialize_bytes_per_step": int(bm)}
        log(f"{label}: {out[label]}")
    st.close()
    return {"workload": wl.name, "results": out}


def bench_batch_topup(args, torch, pm, synth, PoolFiller):
    """B = 8 tokens per step, experts grouped; before each step 20% of the
    distinct experts (kmax >= 2) are cut back to a shorter resident prefix and
    the step tops them up from pinned host memory on the store's side stream.
    Timed on the default path and with PM_READ_ONCE (an expert shared by
    several tokens read once, by the direct kernels)."""
    wl = synth.WORKLOADS[4]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    pw = pm.pm_expert_plane_words(e)
    # pinned host sources: every expert's planes; levels stay resident (the
    # store never reads a host levels source once its levels are on the device)
    hplanes = torch.empty((wl.n_experts, 8 * pw), dtype=torch.int32, pin_memory=True)
    hlevels = torch.empty(pm.pm_expert_levels_floats(e), dtype=torch.float32, pin_memory=True)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
        hplanes[i].copy_(pm_slot_tensor(torch, pm, st, i, pw))
        pm.pm_store_attach_host(st, 0, i, hplanes[i].data_ptr(), hlevels.data_ptr())
    torch.cuda.synchronize()
    total = args.warmup + args.steps
    routes = [route_steps(pm, synth, wl, 0, range(total), token=t) for t in range(wl.n_tokens)]
    ids = np.stack([r[0] for r in routes], 1)          # [steps][B][top_k]
    w = np.stack([r[1] for r in routes], 1)
    k3 = np.stack([r[2] for r in routes], 1)
    x = torch.from_numpy(np.stack([np.stack([synth.activation(wl.seed, wl.cfg, 0, t, wl.hidden, step=s)
                                             for t in range(wl.n_tokens)]) for s in range(total)])).cuda()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    plans = []
    for s in range(total):
        distinct = sorted(set(int(i) for i in ids[s].reshape(-1)))
        kmax = {i: int(k3[s][ids[s] == i].max()) for i in distinct}
        cand = [i for i in distinct if kmax[i] >= 2]
        pick = synth.words(wl.seed, synth.KIND_TRUNC, wl.cfg, 0, s, 0, len(cand)).argsort()
        short = [cand[int(j)] for j in pick[:int(np.ceil(0.2 * len(distinct)))]]
        r = synth.words(wl.seed, synth.KIND_TRUNC, wl.cfg, 0, s, 1, len(short))
        plans.append([(i, 1 + int(r[j] % (kmax[i] - 1))) for j, i in enumerate(short)])
    gemv_bytes = float(np.mean([grouped_bytes(wl, ids[s], k3[s]) for s in range(total)]))
    copies = []

    def step(i, topup=True, s0=args.warmup, extra=0):
        s = s0 + i
        if topup:
            for e_, keep in plans[s]:
                pm.pm_store_truncate(st, 0, e_, keep)
        pm.pm_moe_token_forward(st, 0, ids[s], w[s], k3[s], x[s], y[s], stream,
                                flags=pm.PM_AUTO_TOPUP | extra)

    n = args.steps
    # warm-up: the warm-up steps, repeated for at least half a second (the
    # first copies and launches of a process run slower)
    t_end, i = time.perf_counter() + 0.5, 0
    while i < min(args.warmup, 10) or time.perf_counter() < t_end:
        step(i % max(1, min(args.warmup, 10)), True, 0)
        i += 1
    torch.cuda.synchronize()
    _, _, p0, b0 = pm.pm_store_copy_stats(st)
    el = timed(torch, step, n)
    _, _, p1, b1 = pm.pm_store_copy_stats(st)
    el_res = timed(torch, lambda i: step(i, False), n)
    el_once = timed(torch, lambda i: step(i, True, extra=pm.PM_READ_ONCE), n)
    el_once_res = timed(torch, lambda i: step(i, False, extra=pm.PM_READ_ONCE), n)
    st.close()
    return {"workload": wl.name, "ms_per_step": round(el / n * 1e3, 4),
            "ms_per_step_all_resident": round(el_res / n * 1e3, 4),
            "ms_per_step_read_once": round(el_once / n * 1e3, 4),
            "ms_per_step_all_resident_read_once": round(el_once_res / n * 1e3, 4),
            "gemv_GBs_all_resident": round(gemv_bytes * n / el_res / 1e9, 1),
            "h2d_MB_per_step": round((b1 - b0) / n / 1e6, 2),
            "h2d_GBs": round((b1 - b0) / el / 1e9, 2),
            "planes_per_step": round((p1 - p0) / n, 2),
            "expert_gemvs_per_s": round(3 * wl.top_k * wl.n_tokens * n / el, 1)}


def bench_gemv_by_k(args, torch, pm, synth):
    """pm_expert_gemv alone at k = 1..8 on two tall group-128 matrices
    (16384 x 4096 and 32768 x 1024: 16 gate/up and 8 down matrices stacked),
    planes and levels filled with random bits/values (the timing does not
    depend on them).  Reports us per call and GB/s on planes 0..k-1 plus the
    depth-k tables plus x."""
    stream = torch.cuda.current_stream()
    out = []
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.BASE_SEED)
    for rows, cols in ((16384, 4096), (32768, 1024)):
        s = pm.mshape(rows, cols, 128)
        pw, lf = pm.pm_plane_words(s), pm.pm_levels_floats(s)
        planes = torch.randint(-2**31, 2**31 - 1, (8 * pw,), dtype=torch.int32, device="cuda",
                               generator=g)
        levels = torch.randn(lf, device="cuda", generator=g)
        x = torch.randn(cols, device="cuda", generator=g)
        y = torch.empty(rows, device="cuda")
        for k in range(1, 9):
            for _ in range(3):
                pm.pm_expert_gemv(s, k, planes, pw, levels, x, y, stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 20
            a.record(stream)
            for _ in range(n):
                pm.pm_expert_gemv(s, k, planes, pw, levels, x, y, stream)
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / n * 1e3
            by = rows * cols * k // 8 + rows * (cols // 128) * (1 << k) * 4 + cols * 4
            out.append({"rows": rows, "cols": cols, "k": k, "us": round(us, 2),
                        "GBs": round(by / us / 1e3, 1)})
    return {"workload": "gemv-by-k-g128", "results": out}


BATCHES = (16, 64, 256, 1024)


def bench_batches(args, torch, pm, synth, PoolFiller):
    """Larger batches of one layer (512 experts, 4096/1024, group 128, top-10,
    allocator prefixes at mean 2.5, all experts resident): the layer step for
    B tokens through the default path (a LUT job per use, matrix-core tiles
    for the (expert, matrix, k) groups of at least 6 uses) and through the
    matrix-core path alone (PM_BATCH_MFMA: every group tiled 16 uses at a
    time).  Fresh tokens every step."""
    wl = synth.WORKLOADS[1]
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    for i in range(wl.n_experts):
        filler.fill(st, 0, i)
    torch.cuda.synchronize()
    err = synth.error_profiles(wl.seed, wl.cfg, 0, wl.n_experts)
    stream = torch.cuda.current_stream()
    out = []
    n_steps = 6
    for B in BATCHES:
        steps = []
        for s_ in range(n_steps + 1):
            lg = np.stack([synth.router_logits(wl.seed, wl.cfg, 0, t % 4096, wl.n_experts,
                                               step=100 + s_) for t in range(B)])
            ids, w = pm.pm_route_topk(lg, wl.top_k)
            kk = pm.pm_allocate_bits(ids, w, err, wl.budget)
            k3 = np.repeat(kk[:, :, None], 3, axis=2).astype(np.uint8)
            x = torch.randn(B, wl.hidden, device="cuda")
            steps.append((ids, w, k3, x, torch.empty_like(x)))
        res = {"tokens": B}
        for name, flags in (("default", 0), ("mfma", pm.PM_BATCH_MFMA)):
            # untimed pass over every step: the workspace reaches its size
            for ids, w, k3, x, y in steps:
                pm.pm_moe_token_forward(st, 0, ids, w, k3, x, y, stream, flags=flags)
            el = timed(torch, lambda i: pm.pm_moe_token_forward(
                st, 0, steps[1 + i][0], steps[1 + i][1], steps[1 + i][2], steps[1 + i][3],
                steps[1 + i][4], stream, flags=flags), n_steps)
            res[name + "_ms"] = round(el / n_steps * 1e3, 3)
        gb = float(np.mean([grouped_bytes(wl, st_[0], st_[2]) for st_ in steps[1:]]))
        res["algorithmic_MB"] = round(gb / 1e6, 1)
        res["default_GBs"] = round(gb / (res["default_ms"] / 1e3) / 1e9, 1)
        res["mfma_GBs"] = round(gb / (res["mfma_ms"] / 1e3) / 1e9, 1)
        fl = np.mean([mfma_flops(wl, st_[0], st_[2]) for st_ in steps[1:]], axis=0)
        res["mfma_useful_TFLOPs"] = round(float(fl[0]) / (res["mfma_ms"] / 1e3) / 1e12, 1)
        res["mfma_issued_TFLOPs"] = round(float(fl[1]) / (res["mfma_ms"] / 1e3) / 1e12, 1)
        res["mfma_tile_fill"] = round(float(fl[0] / fl[1]), 3)
        res["tokens_per_s_mfma"] = round(B / (res["mfma_ms"] / 1e3), 1)
        res["tokens_per_s"] = round(B / (res["default_ms"] / 1e3), 1)
        res["mfma_speedup"] = round(res["default_ms"] / res["mfma_ms"], 2)
        log(f"B={B}: {res}")
        out.append(res)
    st.close()
    return {"workload": "moe-layer-e512-h4096-i1024-g128-top10-k2.5-batches", "results": out}


ENCODE_ITERS = 25


def bench_encode(args, torch, pm, synth):
    """The encoder from fp32 weights on one expert (gate, up, down of hidden
    4096 / intermediate 1024, dense N(0, 0.02) weights): K-means per block
    (pm_kmeans_codebook_device) then planes and the count-weighted tree
    (pm_encode_matrix_device), at group 128 (the stored format; a block of
    128 weights gets one leaf per weight, so 7 and 8 bits are exact) and at
    group 1024.  Reports the time per expert and the relative weight error
    ||W - W_k|| / ||W|| for k = 1..8 (W_k decoded by pm_debug_dequant)."""
    wl = synth.WORKLOADS[1]
    shapes = [(wl.inter, wl.hidden), (wl.inter, wl.hidden), (wl.hidden, wl.inter)]
    W = [torch.from_numpy(synth.weights(wl.seed, wl.cfg, 0, 0, m, r, c)).cuda()
         for m, (r, c) in enumerate(shapes)]
    stream = torch.cuda.current_stream()
    out = []
    for group in (128, 1024):
        bufs = []
        for (r, c), w in zip(shapes, W):
            s = pm.mshape(r, c, group)
            nb = r * (c // group)
            bufs.append(dict(
                s=s, w=w, nb=nb,
                codes=torch.empty(r * c, dtype=torch.uint8, device="cuda"),
                leaves=torch.empty(nb * 256, dtype=torch.float32, device="cuda"),
                counts=torch.empty(nb * 256, dtype=torch.int32, device="cuda"),
                its=torch.empty(nb, dtype=torch.int32, device="cuda"),
                planes=torch.empty(8 * pm.pm_plane_words(s), dtype=torch.int32, device="cuda"),
                levels=torch.empty(pm.pm_levels_floats(s), dtype=torch.float32, device="cuda")))

        def encode():
            for b in bufs:
                pm.pm_kmeans_codebook_device(b["s"], b["w"], ENCODE_ITERS, b["codes"],
                                             b["leaves"], b["counts"], b["its"], stream)
                pm.pm_encode_matrix_device(b["s"], b["codes"], b["leaves"], b["counts"],
                                           b["planes"], pm.pm_plane_words(b["s"]), b["levels"],
                                           stream)

        encode()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        t0.record(stream)
        for _ in range(reps):
            encode()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        err = []
        wk = [torch.empty_like(b["w"]) for b in bufs]
        for k in range(1, 9):
            num = den = 0.0
            for b, d in zip(bufs, wk):
                pm.pm_debug_dequant(b["s"], k, b["planes"], pm.pm_plane_words(b["s"]),
                                    b["levels"], d, stream)
                num += float(((b["w"].double() - d.double()) ** 2).sum())
                den += float((b["w"].double() ** 2).sum())
            err.append(round(100 * (num / den) ** 0.5, 3))
        its = torch.cat([b["its"] for b in bufs]).double()
        n_w = sum(r * c for r, c in shapes)
        out.append({"group": group, "ms_per_expert": round(ms, 3),
                    "M_weights_per_s": round(n_w / ms / 1e3, 1),
                    "mean_iters": round(float(its.mean()), 2), "max_iters": int(its.max()),
                    "rel_weight_error_pct_k1_to_k8": err})
    return {"workload": "encode-expert-h4096-i1024-normal0.02-kmeans256", "results": out}


CACHE_TOKENS = 500
CACHE_ZIPF_S = 1.0
CACHE_GIB = (12, 24, 48)


def bench_cache_replay(args, pm, synth):
    """Replay of a synthetic decode trace through the expert caches (host
    only).  Shapes of the 60-layer workload: 512 experts per layer, top-10,
    500 tokens from a cold cache; expert popularity per layer is Zipf (s = 1)
    over a seeded rank order, tokens are independent; the allocator picks the
    prefixes at a mean of 2.5 bits.  A plane of one expert (gate, up and down)
    is hidden * inter * 3 / 8 bytes = 1.5 MiB.  Policies: fixed 4 and fixed 3
    bits (one width per expert, so all caches behave alike), then at the
    allocator's widths the independent-object cache, the downward-reuse cache
    and the plane-aging prefix cache, at 12, 24 and 48 GiB."""
    wl = synth.WORKLOADS[2]
    L, E, K, T = wl.n_layers, wl.n_experts, wl.top_k, CACHE_TOKENS
    t0 = time.perf_counter()
    ex = np.zeros((T, L, K), np.int32)
    kk = np.zeros((T, L, K), np.int32)
    for layer in range(L):
        lg = np.stack([synth.zipf_router_logits(wl.seed, wl.cfg, layer, t, E, CACHE_ZIPF_S)
                       for t in range(T)])
        ids, w = pm.pm_route_topk(lg, K)
        ex[:, layer] = ids + layer * E
        kk[:, layer] = pm.pm_allocate_bits(ids, w, synth.error_profiles(wl.seed, wl.cfg, layer, E),
                                           wl.budget)
    log(f"cache trace: {T * L * K} accesses, mean k {kk.mean():.3f} "
        f"({time.perf_counter() - t0:.1f} s)")
    e, k = ex.reshape(-1), kk.reshape(-1)
    plane_bytes = wl.hidden * wl.inter * 3 // 8
    runs = (("fixed4", pm.PM_CACHE_PREFIX, np.full_like(k, 4)),
            ("fixed3", pm.PM_CACHE_PREFIX, np.full_like(k, 3)),
            ("dynamic2.5_objects", pm.PM_CACHE_OBJECTS, k),
            ("dynamic2.5_downward", pm.PM_CACHE_DOWNWARD, k),
            ("dynamic2.5_prefix", pm.PM_CACHE_PREFIX, k))
    out = []
    for gib in CACHE_GIB:
        cap = (gib << 30) // plane_bytes
        for name, policy, ks in runs:
            c = pm.pm_cache_create(L * E, cap, policy)
            t1 = time.perf_counter()
            pm.pm_cache_replay(c, e, ks)
            dt = time.perf_counter() - t1
            st = pm.pm_cache_stats(c)
            out.append({"cache_GiB": gib, "policy": name,
                        "hit_pct": round(100 * st["hits"] / st["accesses"], 2),
                        "partial_pct": round(100 * st["partial"] / st["accesses"], 2),
                        "planes_read_per_token": round(st["planes_read"] / T, 1),
                        "GiB_read_per_token": round(st["planes_read"] * plane_bytes / T / 2**30, 3),
                        "replay_M_accesses_per_s": round(st["accesses"] / dt / 1e6, 1)})
            c.close()
    return {"workload": f"cache-replay-{L}layers-e{E}-top{K}-{T}tokens-zipf{CACHE_ZIPF_S}-k2.5",
            "plane_MiB": plane_bytes / 2**20, "results": out}


def pm_slot_tensor(torch, pm, st, expert, pw):
    """The device planes of a store slot as a torch view (for copying out)."""
    pp, _ = pm.pm_store_slot(st, 0, expert)
    import ctypes
    buf = torch.empty(8 * pw, dtype=torch.int32, device="cuda")
    hip = ctypes.CDLL("libamdhip64.so")
    stream = torch.cuda.current_stream().cuda_stream
    rc = hip.hipMemcpyAsync(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(pp),
                            ctypes.c_size_t(8 * pw * 4), 3, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed: {rc}")
    return buf


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--experts", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--wg-timeline", type=int, default=0, metavar="N",
                    help="with the stamped build (libpm_stamps.so): after the timed loop, run "
                         "groups of N steps back to back and report the workgroup timeline of "
                         "each group's last gate/up and down launches")
    ap.add_argument("--wg-dump", metavar="FILE",
                    help="with --wg-timeline: also save the raw stamps of every group (.npz)")
    ap.add_argument("--kfix", type=int, default=0, metavar="K",
                    help="every use of the layer step at prefix K (per-prefix profiles)")
    ap.add_argument("--graph-only", type=int, default=0, metavar="R",
                    help="after the timed loop, capture its steps into a HIP graph, replay it "
                         "R times and print only that (for kernel traces of back-to-back steps)")
    ap.add_argument("--log-inputs", metavar="FILE",
                    help="write the ids, w and k of every step of the layer benchmark (JSON lines)")
    ap.add_argument("--workload", default="1",
                    choices=["1", "2", "3", "4", "cache", "encode", "gemv", "batch", "all"],
                    help="1: the one-layer step (the reported line); 2: 60 layers; "
                         "3: k = 4 / 8 / mixed against materialize; 4: B = 8 with top-ups; "
                         "cache: Zipf trace replay through the expert caches (host only); "
                         "encode: K-means encoder from fp32 weights; "
                         "gemv: pm_expert_gemv alone at k = 1..8; "
                         "batch: B = 16/64/256/1024 through the default path and the matrix cores")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "STATS_CSV"),
                    help="print a summary of rocprofv3 outputs of this benchmark and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path is built and timed on a single MI355X)", file=sys.stderr)
        return 2
    if args.workload in ("cache", "all"):
        import bitplane_quantized_expert_amd as pm
        import synth
        print(json.dumps({"workload_result": bench_cache_replay(args, pm, synth)}), flush=True)
        if args.workload == "cache":
            return 0

    if args.wg_timeline:
        stamps = os.path.join(ROOT, "bitplane_quantized_expert_amd", "libpm_stamps.so")
        if not os.path.exists(stamps):
            print(f"{stamps} is missing: build it (bitplane_quantized_expert_amd/build.py)",
                  file=sys.stderr)
            return 1
        os.environ["PM_LIB"] = stamps
    import torch
    import bitplane_quantized_expert_amd as pm
    import synth
    from synth.pool import PoolFiller

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.workload != "1":
        extra = {"2": bench_sixty_layers, "3": bench_precisions, "4": bench_batch_topup,
                 "encode": lambda a, t, p, s, _: bench_encode(a, t, p, s),
                 "gemv": lambda a, t, p, s, _: bench_gemv_by_k(a, t, p, s),
                 "batch": bench_batches}
        for key in (["2", "3", "4", "encode", "gemv", "batch"] if args.workload == "all"
                    else [args.workload]):
            res = extra[key](args, torch, pm, synth, PoolFiller)
            print(json.dumps({"workload_result": res}), flush=True)
        return 0
    wl = synth.WORKLOADS[1]
    n_exp = args.experts
    e = pm.eshape(wl.hidden, wl.inter, wl.group)
    st = pm.pm_store_create(e, 1, wl.n_experts)
    filler = PoolFiller(wl)
    t0 = time.time()
    for i in range(n_exp):
        filler.fill(st, 0, i)
        if i % 64 == 63:
            torch.cuda.synchronize()
            log(f"filled {i + 1}/{n_exp} experts ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    log(f"pool ready: {n_exp} experts, {time.time() - t0:.1f} s")

    # per-step inputs: fresh token, product routing and allocation
    total = args.warmup + args.steps
    err = synth.error_profiles(wl.seed, wl.cfg, 0, wl.n_experts)
    logits = np.stack([synth.router_logits(wl.seed, wl.cfg, 0, 0, wl.n_experts, step=s)
                       for s in range(total)])
    if n_exp < wl.n_experts:
        logits[:, n_exp:] = -np.inf
    ids, w = pm.pm_route_topk(logits, wl.top_k)
    kk = pm.pm_allocate_bits(ids, w, err, wl.budget)
    if args.kfix:
        kk = np.full_like(kk, args.kfix)
    k3 = np.repeat(kk[:, :, None], 3, axis=2)
    x = torch.from_numpy(np.stack([synth.activation(wl.seed, wl.cfg, 0, 0, wl.hidden, step=s)
                                   for s in range(total)])).cuda()
    y = torch.empty_like(x)
    plans = [(ids[s], w[s], k3[s]) for s in range(total)]
    stream = torch.cuda.current_stream()
    log(f"inputs ready: {total} tokens, mean k {kk.mean():.3f}")
    inputs_digest = routing_digest(ids, w, kk)
    if args.log_inputs:
        with open(args.log_inputs, "w") as fh:
            for s in range(total):
                fh.write(json.dumps({"step": s, "timed": s >= args.warmup,
                                     "ids": ids[s].tolist(), "w": w[s].tolist(),
                                     "k": kk[s].tolist()}) + "\n")

    def run(s):
        pm.pm_moe_token_forward(st, 0, ids[s:s + 1], w[s:s + 1], k3[s:s + 1], x[s:s + 1],
                                y[s:s + 1], stream)

    for s in range(args.warmup):
        run(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, total):
        run(s)
    issued = time.perf_counter() - t0
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    steps = range(args.warmup, total)
    nbytes = sum(step_bytes(wl, k3[s]) for s in steps)
    gbs = nbytes / el / 1e9
    ms = el / args.steps * 1e3
    log(f"timed {args.steps} steps: {ms:.4f} ms/step, {gbs:.1f} GB/s "
        f"(host issue {issued / args.steps * 1e6:.1f} us/step)")

    # the timed steps as library calls on a side stream, for capture into a
    # HIP graph (the store's last stream becomes that stream first).  A call
    # that needs the direct kernels (a prefix above 5) cannot be captured:
    # those steps are left out of the graph and counted.
    cap = torch.cuda.Stream()
    g_steps = [s for s in steps if int(k3[s].max()) <= 5]
    g_bytes = sum(step_bytes(wl, k3[s]) for s in g_steps)

    def run_cap(s):
        pm.pm_moe_token_forward(st, 0, ids[s:s + 1], w[s:s + 1], k3[s:s + 1], x[s:s + 1],
                                y[s:s + 1], cap)

    def all_steps():
        for s in g_steps:
            run_cap(s)

    if args.wg_timeline:
        res = wg_timeline(pm, torch, run, list(steps), args.wg_timeline, dump=args.wg_dump)
        st.close()
        print(json.dumps({"wg_timeline": res}), flush=True)
        return 0

    if args.graph_only:
        with torch.cuda.stream(cap):
            run_cap(steps[0])
        torch.cuda.synchronize()
        _, g_el = graph_replay(torch, cap, all_steps, args.graph_only)
        st.close()
        print(json.dumps({"graph_only": {"replays": args.graph_only, "steps": len(g_steps),
                                         "left_out": args.steps - len(g_steps),
                                         "ms_per_step": round(g_el / len(g_steps) * 1e3, 5),
                                         "GBs": round(g_bytes / g_el / 1e9, 2)}}), flush=True)
        return 0

    ceiling = copy_ceiling(torch, stream)
    log(f"stream ceiling: {ceiling['GBs']} GB/s ({ceiling['kernel']})")

    # roofline pass: the gate/up launch's own start and stop events (HIP
    # events on the library's stream), nothing else queued; then a pass with
    # events after every stage for the stage split
    def event_pass(n_ev):
        evs = []
        for s in steps:
            group = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
            for ev in group:
                ev.record(stream)
            evs.append(group)
        torch.cuda.synchronize()
        for s, group in zip(steps, evs):
            pm.pm_store_set_profile_events(st, group)
            run(s)
        pm.pm_store_set_profile_events(st, [])
        torch.cuda.synchronize()
        return evs

    # the distribution of single steps: an event at every step boundary
    def boundary_pass(order):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i, s in enumerate(order):
            run(s)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(len(order))]) * 1e3

    def pct(us):
        return {"mean": round(float(us.mean()), 2),
                **{f"p{q}": round(float(np.percentile(us, q)), 2) for q in (10, 50, 90)}}

    step_dist = pct(boundary_pass(list(steps)))
    # host time of one call, with the device queue kept short (a sync every 8
    # calls, so that no call waits for queue space): the C entry point with
    # the argument addresses worked out beforehand (as a caller that owns its
    # buffers makes it), and the numpy binding
    ids_c, w_c, k_c = (np.ascontiguousarray(a) for a in (ids, w, k3))
    tk = wl.top_k
    a_ids, a_w, a_k = ids_c.ctypes.data, w_c.ctypes.data, k_c.ctypes.data
    a_x, a_y, row = x.data_ptr(), y.data_ptr(), 4 * wl.hidden
    sh = stream.cuda_stream

    def raw(s):
        pm.pm_moe_token_forward_ptr(st, 0, 1, tk, a_ids + 4 * tk * s, a_w + 4 * tk * s,
                                    a_k + 3 * tk * s, a_x + row * s, a_y + row * s, sh)

    def host_pass(fn):
        d = []
        for i, s in enumerate(steps):
            if i % 8 == 0:
                torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn(s)
            d.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        return pct(np.array(d) * 1e6)

    host_raw = host_pass(raw)
    host_binding = host_pass(run)

    # the timed steps captured into one HIP graph and replayed (no host work
    # between launches)
    graph = {}
    try:
        with torch.cuda.stream(cap):
            run_cap(steps[0])
        torch.cuda.synchronize()
        _, g_el = graph_replay(torch, cap, all_steps, 3)
        graph = {"ms_per_step": round(g_el / len(g_steps) * 1e3, 5),
                 "GBs": round(g_bytes / g_el / 1e9, 2), "replays": 3, "steps": len(g_steps),
                 "left_out": args.steps - len(g_steps),
                 "how": "the timed steps captured once on a side stream and replayed; steps "
                        "with a prefix above 5 (direct kernels, not capturable) left out"}
        log(f"graph replay: {graph['ms_per_step'] * 1e3:.2f} us/step, {graph['GBs']} GB/s")
    except Exception as ex:
        graph = {"error": str(ex)[:300]}
        log(f"graph capture failed: {graph['error']}")
    log(f"host time per call: C entry {host_raw['mean']} us (p50 {host_raw['p50']}), "
        f"numpy binding {host_binding['mean']} us")
    # one step alone (GPU idle before it, its own events), cold and warm:
    # cold after 512 MiB of writes that evict the 256 MB Infinity Cache,
    # warm right after the same step ran (its experts' planes cached)
    n_cw = min(50, args.steps)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def alone(s, cold):
        if cold:
            flush.zero_()
        else:
            run(s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run(s)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    cold, warm = [], []
    for s in list(steps)[:n_cw]:
        cold.append(alone(s, True))
        warm.append(alone(s, False))
    del flush
    cache_state = {"cold_us": pct(np.array(cold)), "warm_us": pct(np.array(warm)),
                   "steps": n_cw,
                   "how": "each of the first timed steps alone: cold after 512 MiB of writes, "
                          "warm right after the same step"}
    log(f"steps p10/p50/p90 {step_dist['p10']}/{step_dist['p50']}/{step_dist['p90']} us; "
        f"warm p50 {cache_state['warm_us']['p50']} us, cold p50 {cache_state['cold_us']['p50']} us")

    gu_ms = np.array([a.elapsed_time(b) for a, b in event_pass(2)])
    evs = event_pass(4)
    dn_ms = np.array([b.elapsed_time(c) for _, b, c, _ in evs])
    cb_ms = np.array([c.elapsed_time(d) for _, _, c, d in evs])
    # a step whose down launches fold the combine in runs no combine kernel:
    # its third stage holds only the events themselves.  One token forms no
    # matrix-core tiles, so every step folds.
    folded = np.ones(len(steps), bool)
    gu_b = np.array([gateup_bytes(wl, k3[s]) for s in steps])
    achieved = float(gu_b.mean() / (gu_ms.mean() * 1e-3) / 1e9)
    log(f"gate/up {gu_ms.mean() * 1e3:.1f} us, down {dn_ms.mean() * 1e3:.1f} us, "
        f"combine {cb_ms.mean() * 1e3:.1f} us; gate/up {achieved:.1f} GB/s")

    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "experts": wl.n_experts, "hidden": wl.hidden,
                   "inter": wl.inter, "group": wl.group, "top_k": wl.top_k, "batch": 1,
                   "mean_k": round(float(kk[args.warmup:].mean()), 4), "pool_experts": n_exp},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "hip_graph": graph,
        "host_issue_us_per_step": host_raw["mean"],
        "host_issue": {"c_entry_us": host_raw, "numpy_binding_us": host_binding,
                       "timed_loop_issue_us_per_step": round(issued / args.steps * 1e6, 2),
                       "how": "wall time of one call on the host, the device queue kept short "
                              "(a sync every 8 calls); the timed loop's figure includes waits "
                              "for queue space once the device falls behind"},
        "expert_gemvs_per_s": round(3 * wl.top_k * args.steps / el, 1),
        "step_us": step_dist,
        "cache_state": cache_state,
        "stage_us": {"gateup": round(gu_ms.mean() * 1e3, 2), "down": round(dn_ms.mean() * 1e3, 2),
                     "combine": (round(cb_ms[~folded].mean() * 1e3, 2) if (~folded).any()
                                 else None),
                     "steps_with_combine_kernel": int((~folded).sum()),
                     "how": "HIP events on the library's stream: gate/up between its own start "
                            "and stop events (one pass), down between events after each stage "
                            "(another pass); each launch that carries events runs longer than "
                            "in the timed loop. The down launches add the routing-weighted terms "
                            "into y themselves, so no step runs a combine kernel"},
        "kernel_sum_us": (round(TRACE["gateup_us"] + TRACE["down_us"], 2)
                          if TRACE["sources_sha256"] == sources_digest() else None),
        "kernel_trace": ({k: TRACE[k] for k in ("gateup_us", "down_us", "step_us", "profile")}
                         if TRACE["sources_sha256"] == sources_digest() else None),
        "roofline": {"bound": "hbm", "kernel": "gateup", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": (TRAFFIC["bytes_per_launch"]
                                 if TRAFFIC["sources_sha256"] == sources_digest() else None),
                     "trace_launch_us": (TRACE["gateup_us"]
                                         if TRACE["sources_sha256"] == sources_digest() else None),
                     "trace_frac": (round(float(gu_b.mean()) / (TRACE["gateup_us"] * 1e-6) / 1e9
                                          / PEAK_HBM_GBS, 4)
                                    if TRACE["sources_sha256"] == sources_digest() else None),
                     "bytes_per_launch": int(gu_b.mean()),
                     "launch_us": round(gu_ms.mean() * 1e3, 2)},
        "stream_ceiling": ceiling,
        "inputs_sha256": inputs_digest,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(wl, plans, args.cpu_seconds)
    st.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
