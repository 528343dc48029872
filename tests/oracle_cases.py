"""Test-side helpers that run the CPU oracle on the seeded workloads: whole
experts for small shapes, and sampled output rows for the full-size layers
(gate and up are computed whole, because every row of h feeds every output;
down only at the sampled rows)."""
from functools import lru_cache

import numpy as np

import oracle
import synth


def _wl(w):
    return synth.WORKLOADS[w] if isinstance(w, int) else w


@lru_cache(maxsize=64)
def gate_up(cfg, layer, expert):
    """Oracle-encoded gate and up matrices of one seeded expert (cfg is a
    workload index or a Workload)."""
    wl = _wl(cfg)
    cfg = wl.cfg
    out = []
    for m in (0, 1):
        rows, cols = synth.matrix_shape(wl, m)
        lv = synth.leaves(wl.seed, cfg, layer, expert, m, rows, cols // wl.group)
        cd = synth.codes(wl.seed, cfg, layer, expert, m, rows, cols)
        out.append((oracle.pack_planes(cd), oracle.tree_levels(lv)))
    return out


def down_rows(cfg, layer, expert, rows):
    """Oracle-encoded sampled rows of the down matrix."""
    wl = _wl(cfg)
    cfg = wl.cfg
    R, cols = synth.matrix_shape(wl, 2)
    lv = np.concatenate([synth.leaves(wl.seed, cfg, layer, expert, 2, R, cols // wl.group, r, r + 1)
                         for r in rows])
    cd = np.concatenate([synth.codes(wl.seed, cfg, layer, expert, 2, R, cols, r, r + 1)
                         for r in rows])
    return oracle.pack_planes(cd), oracle.tree_levels(lv)


@lru_cache(maxsize=48)
def gate_up_dense(cfg, layer, expert, m, k):
    """oracle.dequant of gate (m = 0) or up (m = 1) at prefix k: float32
    [rows][cols], exact node values (kept for the many tokens of a batch)."""
    p, lv = gate_up(cfg, layer, expert)[m]
    return oracle.dequant(p, lv, k, _wl(cfg).group)


def _gemv_gate_up(cfg, layer, expert, m, k, x):
    # oracle.gemv written out on the cached dequantized matrix: the same fp64
    # products and sums
    w = gate_up_dense(cfg, layer, expert, m, k).astype(np.float64)
    x = np.asarray(x, dtype=np.float64)
    return w @ x, np.abs(w) @ np.abs(x)


def token_layer(cfg, layer, ids, w, k, x, rows, materialized=False):
    """Oracle y[rows] and its error scale for one token of one layer.
    k: int [top_k][3] prefixes of gate, up, down."""
    wl = _wl(cfg)
    G = wl.group
    gemv = oracle.gemv_materialized_fp16 if materialized else oracle.gemv
    y = np.zeros(len(rows))
    S = np.zeros(len(rows))
    for j in range(len(ids)):
        if materialized:
            (pg, lg), (pu, lu) = gate_up(cfg, layer, int(ids[j]))
            g, _ = gemv(pg, lg, int(k[j][0]), G, x)
            u, _ = gemv(pu, lu, int(k[j][1]), G, x)
        else:
            g, _ = _gemv_gate_up(cfg, layer, int(ids[j]), 0, int(k[j][0]), x)
            u, _ = _gemv_gate_up(cfg, layer, int(ids[j]), 1, int(k[j][1]), x)
        h = oracle.silu(g) * u
        pd, ld = down_rows(cfg, layer, int(ids[j]), rows)
        yd, sd = gemv(pd, ld, int(k[j][2]), G, h)
        y += float(w[j]) * yd
        S += abs(float(w[j])) * sd
    return y, S


def route_and_bits(cfg, layer, step, token=0, kfix=None):
    """Oracle routing and allocation of one token: ids, w, k[top_k][3]."""
    wl = _wl(cfg)
    cfg = wl.cfg
    lg = synth.router_logits(wl.seed, cfg, layer, token, wl.n_experts, step=step)
    ids, w = oracle.route(lg, wl.top_k)
    if kfix is None:
        err = synth.error_profiles(wl.seed, cfg, layer, wl.n_experts)
        kk = oracle.allocate_bits(w, err[ids], wl.budget)
    else:
        kk = np.full(wl.top_k, kfix, dtype=np.int32)
    return ids, w, np.repeat(kk[:, None], 3, axis=1)


def sample_rows(n, count, seed):
    """Sorted distinct sample of output rows, always with the first and last."""
    w = synth.words(seed, synth.KIND_TRUNC, 0, 0, 0, 0, 4 * count) % np.uint32(n)
    return sorted(set([0, n - 1] + [int(v) for v in w[:count]]))
