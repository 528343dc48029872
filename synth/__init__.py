"""Seeded synthetic inputs for the bitplane-prefix expert path.

This module only draws inputs: leaf codebooks, 8-bit codes, activations,
router logits and synthetic per-expert error profiles.  It holds none of the
method's arithmetic (no tree construction, no bitplane packing, no decoding,
no routing, no allocation): the product library and the CPU oracle each do
that in their own code and consume what is drawn here.

Every random number comes from one counter-based generator, Philox4x32-10
(Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
SC'11), so that any slice of any array can be regenerated alone and so that
the device-side filler (``synth_device.hip``) produces bit-identical leaves and
codes for the large expert pools that are too big to draw on the host.

Value recipes (the pages fix none of them; these are the workload's stated
forms, read plainly):
  * leaves: per (matrix, row, group) 256 ascending fp32 values, the N(0, 0.02)
    quantile midpoints q_j = 0.02 * Phi^-1((j + 0.5) / 256) plus a jitter
    0.25 * u_j * gap_j, u_j uniform in (-1, 1), gap_j the distance from q_j to
    its nearest neighbour quantile (one-sided at the ends).  The jitter keeps
    the leaves strictly ascending without a sort.
  * codes: independent uniform bytes (every bitplane is fair coin flips).
  * x and router logits: N(0, 1) by Box-Muller, fp64 then rounded to fp32.
  * dense weights for the encoder: N(0, 0.02) by Box-Muller, rounded to fp32.
  * routing traces for cache replay: per-layer Zipf popularity over a seeded
    rank permutation, logits -s ln(rank) plus Gumbel noise (see
    zipf_router_logits); independent across tokens.
  * error profiles: err_e(b) = s_e * 4**(-b), s_e = exp(sigma * z_e),
    z_e ~ N(0, 1), sigma = 1 -- a convex stand-in for the offline profiles
    measured on trained weights.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# Philox4x32-10 (published definition: two 32x32->64 multiplies per round,
# Weyl-sequence key schedule, 10 rounds)
# ---------------------------------------------------------------------------
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counters are uint32 arrays (broadcastable),
    the key two Python ints.  Returns four uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for _ in range(10):
        p0 = c0 * m0
        p1 = c2 * m1
        hi0 = p0 >> np.uint64(32)
        lo0 = p0 & _MASK32
        hi1 = p1 >> np.uint64(32)
        lo1 = p1 & _MASK32
        n0 = hi1 ^ c1 ^ np.uint64(k0)
        n2 = hi0 ^ c3 ^ np.uint64(k1)
        c0, c1, c2, c3 = n0, lo1, n2, lo0
        k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


# Stream kinds (top nibble of key word 1).
KIND_LEAVES = 1
KIND_CODES = 2
KIND_X = 3
KIND_LOGITS = 4
KIND_PROFILE = 5
KIND_KDRAW = 6
KIND_POISON = 7
KIND_TRUNC = 8
KIND_ZIPF = 9
KIND_RANK = 10
KIND_WEIGHTS = 11


def stream_key(seed: int, kind: int, cfg: int, layer: int, unit: int, matrix: int):
    """Key of one stream.  key0 = seed; key1 packs kind(4) | cfg(4) |
    layer(8) | unit(12, expert or token) | matrix(4)."""
    if not (0 <= kind < 16 and 0 <= cfg < 16 and 0 <= layer < 256
            and 0 <= unit < 4096 and 0 <= matrix < 16):
        raise ValueError("stream key field out of range")
    k1 = (kind << 28) | (cfg << 24) | (layer << 16) | (unit << 4) | matrix
    return int(seed) & 0xFFFFFFFF, k1


def philox_words(key, n_first: int, n_calls: int, extra: int = 0):
    """Words of calls n_first .. n_first+n_calls-1 of a stream, flattened so
    that word i of call n lands at position 4*(n - n_first) + i."""
    n = np.arange(n_first, n_first + n_calls, dtype=np.uint64)
    lo = (n & _MASK32).astype(np.uint32)
    hi = (n >> np.uint64(32)).astype(np.uint32)
    w = philox4x32_10(lo, hi, np.uint32(extra), np.uint32(0), key[0], key[1])
    return np.stack(w, axis=-1).reshape(-1)


# ---------------------------------------------------------------------------
# Leaf quantiles
# ---------------------------------------------------------------------------
LEAF_SIGMA = 0.02
N_LEAVES = 256


def leaf_quantiles():
    """(q, gap): the 256 N(0, 0.02) quantile midpoints and each one's distance
    to its nearest neighbour, both float64."""
    from scipy.special import ndtri
    j = np.arange(N_LEAVES, dtype=np.float64)
    q = LEAF_SIGMA * ndtri((j + 0.5) / N_LEAVES)
    d = np.diff(q)
    gap = np.empty_like(q)
    gap[0] = d[0]
    gap[-1] = d[-1]
    gap[1:-1] = np.minimum(d[:-1], d[1:])
    return q, gap


_QG = None


def _qgap():
    global _QG
    if _QG is None:
        _QG = leaf_quantiles()
    return _QG


def uniform_pm1(words):
    """uint32 -> float64 in (-1, 1): (r + 0.5) * 2^-31 - 1, exact in fp64."""
    return (words.astype(np.float64) + 0.5) * (2.0 ** -31) - 1.0


def uniform_01(words):
    """uint32 -> float64 in (0, 1): (r + 0.5) * 2^-32, exact in fp64."""
    return (words.astype(np.float64) + 0.5) * (2.0 ** -32)


def leaves(seed, cfg, layer, expert, matrix, rows, ngroups, row0=0, row1=None):
    """fp32 [row1-row0][ngroups][256] leaves of rows row0..row1-1."""
    if row1 is None:
        row1 = rows
    q, gap = _qgap()
    key = stream_key(seed, KIND_LEAVES, cfg, layer, expert, matrix)
    per_row = ngroups * N_LEAVES            # leaves per row; multiple of 4
    first = row0 * per_row // 4
    calls = (row1 - row0) * per_row // 4
    u = uniform_pm1(philox_words(key, first, calls))
    u = u.reshape(row1 - row0, ngroups, N_LEAVES)
    # one rounding per operation: (0.25*u) is exact, then *gap, then +q
    val = q + (0.25 * u) * gap
    return val.astype(np.float32)


def codes(seed, cfg, layer, expert, matrix, rows, cols, row0=0, row1=None):
    """uint8 [row1-row0][cols]; code of (o, i) is byte ((o*cols+i) % 4) of
    word ((o*cols+i) // 4) of the stream (16 codes per Philox call)."""
    if row1 is None:
        row1 = rows
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    key = stream_key(seed, KIND_CODES, cfg, layer, expert, matrix)
    first = row0 * cols // 16
    calls = (row1 - row0) * cols // 16
    w = philox_words(key, first, calls)
    return w.view(np.uint8).reshape(row1 - row0, cols).copy()


def normals(key, n, extra=0):
    """n float64 N(0,1) values by Box-Muller: call c gives words (r0..r3);
    (r0, r1) -> values 4c, 4c+1 and (r2, r3) -> values 4c+2, 4c+3."""
    calls = (n + 3) // 4
    w = philox_words(key, 0, calls, extra).reshape(calls, 2, 2)
    u1 = uniform_01(w[:, :, 0])
    u2 = uniform_01(w[:, :, 1])
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.stack([rad * np.cos(2.0 * math.pi * u2),
                  rad * np.sin(2.0 * math.pi * u2)], axis=-1)
    return z.reshape(-1)[:n]


def activation(seed, cfg, layer, token, n, step=0):
    """fp32 [n] N(0,1) activation of one token (per step)."""
    key = stream_key(seed, KIND_X, cfg, layer, token, 0)
    return normals(key, n, extra=step).astype(np.float32)


WEIGHT_SIGMA = 0.02


def weights(seed, cfg, layer, expert, matrix, rows, cols):
    """fp32 [rows][cols] dense N(0, 0.02) weights of one matrix (the input of
    the encoder from fp32 weights)."""
    key = stream_key(seed, KIND_WEIGHTS, cfg, layer, expert, matrix)
    return (WEIGHT_SIGMA * normals(key, rows * cols)).astype(np.float32).reshape(rows, cols)


def router_logits(seed, cfg, layer, token, n_experts, step=0):
    """fp32 [n_experts] N(0,1) router logits of one token (per step)."""
    key = stream_key(seed, KIND_LOGITS, cfg, layer, token, 0)
    return normals(key, n_experts, extra=step).astype(np.float32)


def expert_popularity_rank(seed, cfg, layer, n_experts):
    """int64 [n_experts]: the 1-based popularity rank of every expert of one
    layer, a seeded permutation (stable argsort of Philox words)."""
    key = stream_key(seed, KIND_RANK, cfg, layer, 0, 0)
    w = philox_words(key, 0, (n_experts + 3) // 4)[:n_experts]
    rank = np.empty(n_experts, np.int64)
    rank[np.argsort(w, kind="stable")] = np.arange(1, n_experts + 1)
    return rank


def zipf_router_logits(seed, cfg, layer, token, n_experts, s=1.0, step=0):
    """fp32 [n_experts] router logits of one token for a synthetic routing
    trace with Zipf popularity: -s * ln(rank_e) + G_e, G_e standard Gumbel
    (-ln(-ln u)).  Their top-k is a draw of k distinct experts without
    replacement with probabilities proportional to rank^-s (the Gumbel-top-k
    trick: Kool, van Hoof and Welling, ICML 2019)."""
    rank = expert_popularity_rank(seed, cfg, layer, n_experts)
    key = stream_key(seed, KIND_ZIPF, cfg, layer, token, 0)
    u = uniform_01(philox_words(key, 0, (n_experts + 3) // 4, extra=step)[:n_experts])
    return (-s * np.log(rank.astype(np.float64)) - np.log(-np.log(u))).astype(np.float32)


PROFILE_SIGMA = 1.0


def error_profiles(seed, cfg, layer, n_experts, nbits=8):
    """float64 [n_experts][nbits]: err_e(b) for b = 1..nbits, the synthetic
    convex stand-in s_e * 4**(-b), s_e = exp(PROFILE_SIGMA * z_e)."""
    key = stream_key(seed, KIND_PROFILE, cfg, layer, 0, 0)
    z = normals(key, n_experts)
    s = np.exp(PROFILE_SIGMA * z)
    b = np.arange(1, nbits + 1, dtype=np.float64)
    return s[:, None] * (4.0 ** (-b))[None, :]


def uniform_k(seed, cfg, layer, unit, n, kmax=8):
    """n integers uniform in 1..kmax (kmax a power of two): word % kmax + 1."""
    if kmax & (kmax - 1):
        raise ValueError("kmax must be a power of two")
    key = stream_key(seed, KIND_KDRAW, cfg, layer, unit, 0)
    w = philox_words(key, 0, (n + 3) // 4)[:n]
    return (w % np.uint32(kmax)).astype(np.int32) + 1


def words(seed, kind, cfg, layer, unit, matrix, n, extra=0):
    """n raw uint32 words of a stream (poison patterns, truncation draws)."""
    key = stream_key(seed, kind, cfg, layer, unit, matrix)
    return philox_words(key, 0, (n + 3) // 4, extra)[:n]


# ---------------------------------------------------------------------------
# Workload shapes (one per configuration of the workload description)
# ---------------------------------------------------------------------------
BASE_SEED = 20261105


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    hidden: int
    inter: int
    group: int
    n_experts: int
    top_k: int
    n_layers: int
    n_tokens: int
    mean_bits: float      # average prefix length the allocator is budgeted for

    @property
    def seed(self):
        return BASE_SEED + self.cfg

    @property
    def budget(self):
        return int(round(self.mean_bits * self.top_k))


WORKLOADS = {
    0: Workload(0, "tiny-expert-h256-i128-g64", 256, 128, 64, 1, 1, 1, 1, 0.0),
    1: Workload(1, "moe-layer-e512-h4096-i1024-g128-top10-b1-k2.5", 4096, 1024, 128,
                512, 10, 1, 1, 2.5),
    2: Workload(2, "moe-60layers-e512-h4096-i1024-g128-top10-b1-k2.5", 4096, 1024,
                128, 512, 10, 60, 1, 2.5),
    3: Workload(3, "moe-layer-e512-h4096-i1024-g128-top10-b1-k4|k8|k2.5-vs-materialize",
                4096, 1024, 128, 512, 10, 1, 1, 2.5),
    4: Workload(4, "moe-layer-e512-h4096-i1024-g128-top10-b8-k2.5-topup20pct", 4096,
                1024, 128, 512, 10, 1, 8, 2.5),
}


def matrix_shape(wl: Workload, matrix: int):
    """(rows, cols) of matrix 0 = gate, 1 = up, 2 = down; rows are outputs."""
    if matrix in (0, 1):
        return wl.inter, wl.hidden
    if matrix == 2:
        return wl.hidden, wl.inter
    raise ValueError(matrix)


def expert_inputs(wl: Workload, layer: int, expert: int, row_ranges=None):
    """Leaves and codes of one expert: lists [gate, up, down] of
    (leaves fp32 [rows][ngroups][256], codes uint8 [rows][cols]).
    row_ranges optionally restricts matrix m to rows row_ranges[m]."""
    out = []
    for m in range(3):
        rows, cols = matrix_shape(wl, m)
        r0, r1 = (0, rows) if row_ranges is None or row_ranges[m] is None else row_ranges[m]
        lv = leaves(wl.seed, wl.cfg, layer, expert, m, rows, cols // wl.group, r0, r1)
        cd = codes(wl.seed, wl.cfg, layer, expert, m, rows, cols, r0, r1)
        out.append((lv, cd))
    return out
