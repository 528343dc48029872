"""CPU oracle for direct bitplane-prefix expert execution.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product library never calls
it, shares no code with it, and must fail loudly when its HIP build is absent.

It is a plain, slow, obviously correct NumPy implementation: fp32 where the
stored format is fp32 (the tree codebook), fp64 for every sum.

Sources (titles of the pages the method is described on):
  [T]   "PagedMoE: Cross-Precision Expert Caching for SSD-Resident MoE
        Inference", podcast episode transcript; "T cN" = subtitle cue N.
  [Abs] "PagedMoE: Cross-Precision Expert Caching for Token-Level Dynamic
        Precision in SSD-Resident MoE Inference", arxivlens page, Abstract.
  [Met] the same arxivlens page, Analysis, "Methodology".
The numeric format (group size, fp32 nodes, MSB-first uint32 planes along the
input dimension, SwiGLU experts, unweighted parent mean) is the workload's
stated form; the pages leave it open.

Pins: every function here is pinned in tests/test_oracle_pins.py against
closed forms, library routines, hand-worked fixtures (tests/golden/) or brute
force; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

NBITS = 8                  # stored code width: 8 planes, 256 leaves per block
NLEAF = 1 << NBITS


# ---------------------------------------------------------------------------
# Tree codebook  ([T] c19, c21; [Abs]: a tree codebook whose prefixes nest)
# ---------------------------------------------------------------------------
def tree_levels(leaves, counts=None, depth=NBITS):
    """Levels of the binary-tree codebook over sorted leaves.

    leaves: float32 [..., 2**depth], ascending along the last axis.  They are
    the deepest level (depth `depth`).  Each parent is the mean of its two
    children ([T] c19: parent = average of its two children), so node p at
    depth d is the reconstruction of every code whose top d bits equal p
    ([T] c21: truncating an index lands on a valid reconstruction).

    counts=None: the unweighted mean, (left + right) * 0.5 in fp32.
    counts: integer [..., 2**depth], how many weights landed on each leaf;
    a parent is then the frequency-weighted mean of its children ([T] c19,
    c21), evaluated in fp64 from the fp32 children and rounded to fp32; its
    count is the sum of the children's.  A parent whose children hold no
    weights falls back to the unweighted mean.

    Returns {d: float32 [..., 2**d]} for d = 1..depth (depth 0, the root, is
    not a usable prefix: k >= 1).
    """
    leaves = np.asarray(leaves, dtype=np.float32)
    if leaves.shape[-1] != (1 << depth):
        raise ValueError("last axis must hold 2**depth leaves")
    if np.any(np.diff(leaves, axis=-1) < 0):
        raise ValueError("leaves must be ascending")
    levels = {depth: leaves.copy()}
    node = leaves
    cnt = None if counts is None else np.asarray(counts, dtype=np.float64)
    for d in range(depth - 1, 0, -1):
        left = node[..., 0::2]
        right = node[..., 1::2]
        if cnt is None:
            parent = (left + right) * np.float32(0.5)
        else:
            nl = cnt[..., 0::2]
            nr = cnt[..., 1::2]
            tot = nl + nr
            mean = (left + right) * np.float32(0.5)
            with np.errstate(invalid="ignore", divide="ignore"):
                wmean = (nl * left.astype(np.float64) + nr * right.astype(np.float64)) / tot
            parent = np.where(tot > 0, wmean.astype(np.float32), mean)
            cnt = tot
        levels[d] = parent.astype(np.float32)
        node = levels[d]
    return levels


def leaf_counts(codes, group):
    """How many weights of each block landed on each leaf: int64
    [rows][cols/group][256], the frequencies of the weighted tree ([T] c19)."""
    codes = np.asarray(codes)
    rows, cols = codes.shape
    blocks = codes.reshape(rows, cols // group, group).astype(np.int64)
    out = np.zeros((rows, cols // group, NLEAF), dtype=np.int64)
    for g in range(cols // group):
        for o in range(rows):
            out[o, g] = np.bincount(blocks[o, g], minlength=NLEAF)
    return out


# ---------------------------------------------------------------------------
# Bitplanes  ([T] c25: plane one holds the first index bit of every weight)
# ---------------------------------------------------------------------------
def pack_planes(codes):
    """codes uint8 [rows][cols] -> uint32 [8][rows][cols/32].

    Plane p holds bit (7 - p) of every code (MSB first: plane 0 is the first
    index bit).  Along the input dimension the bits are packed 32 to a word:
    bit j of word w is column 32*w + j.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    c = codes.reshape(rows, cols // 32, 32).astype(np.uint32)
    planes = np.zeros((NBITS, rows, cols // 32), dtype=np.uint32)
    for p in range(NBITS):
        bit = (c >> np.uint32(NBITS - 1 - p)) & np.uint32(1)
        for j in range(32):
            planes[p] |= bit[:, :, j] << np.uint32(j)
    return planes


def plane_bits(planes, p):
    """Bit of plane p for every weight: uint8 [rows][cols]."""
    w = np.asarray(planes[p], dtype=np.uint32)
    rows, nw = w.shape
    j = np.arange(32, dtype=np.uint32)
    bits = (w[:, :, None] >> j[None, None, :]) & np.uint32(1)
    return bits.reshape(rows, nw * 32).astype(np.uint8)


def prefix_codes(planes, k):
    """k-bit prefix of every weight, read from planes 0..k-1 only:
    prefix = sum_{p<k} bit_p << (k-1-p).  Planes k..7 are never touched
    ([T] c25: going from k-1 to k bits reads exactly one more plane)."""
    if not 1 <= k <= NBITS:
        raise ValueError("k must be in 1..8")
    pre = None
    for p in range(k):
        b = plane_bits(planes, p).astype(np.int64)
        pre = b if pre is None else (pre << 1) | b
    return pre


# ---------------------------------------------------------------------------
# Decode and GEMV  ([Abs]: execution straight from a cached 1-8-bit prefix;
# [T] c37: indices assembled from the requested planes, codebook lookup,
# dot product; no full-precision matrix is needed)
# ---------------------------------------------------------------------------
def dequant(planes, levels, k, group):
    """W_k[o][i] = node at depth k of block (o, i // group) selected by the
    k-bit prefix of (o, i).  float32 [rows][cols], exact table values."""
    pre = prefix_codes(planes, k)
    rows, cols = pre.shape
    lv = levels[k]                                   # [rows][cols/group][2**k]
    gidx = np.arange(cols) // group
    return lv[np.arange(rows)[:, None], gidx[None, :], pre]


def gemv(planes, levels, k, group, x):
    """y[o] = sum_i W_k[o][i] * x[i] in fp64, with the error scale
    S[o] = sum_i |W_k[o][i] * x[i]|.  Returns (y float64, S float64)."""
    w = dequant(planes, levels, k, group).astype(np.float64)
    x = np.asarray(x, dtype=np.float64)
    return w @ x, np.abs(w) @ np.abs(x)


def gemv_materialized_fp16(planes, levels, k, group, x):
    """The materialize-then-multiply comparator ([T] c37): the decoded matrix
    is first written at fp16 (round to nearest even), then multiplied."""
    w = dequant(planes, levels, k, group).astype(np.float16).astype(np.float64)
    x = np.asarray(x, dtype=np.float64)
    return w @ x, np.abs(w) @ np.abs(x)


def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)), fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(expert, kg, ku, kd, x):
    """One SwiGLU expert read at prefixes (kg, ku, kd) of gate, up, down.

    expert: dict with 'planes' [3] (uint32 [8][rows][cols/32]), 'levels' [3]
    ({d: fp32}), 'group'.  g = W_gate x, u = W_up x, h = silu(g) * u,
    y = W_down h (fp64 throughout).  Returns dict with g, u, h, y and the
    error scales Sg, Su, Sy (Sy computed with this h)."""
    G = expert["group"]
    g, sg = gemv(expert["planes"][0], expert["levels"][0], kg, G, x)
    u, su = gemv(expert["planes"][1], expert["levels"][1], ku, G, x)
    h = silu(g) * u
    y, sy = gemv(expert["planes"][2], expert["levels"][2], kd, G, h)
    return {"g": g, "u": u, "h": h, "y": y, "Sg": sg, "Su": su, "Sy": sy}


def encode_expert(leaves_codes, group, weighted=False):
    """Encode one expert from its [gate, up, down] (leaves, codes): the tree
    levels of every block and the 8 bitplanes of every matrix."""
    planes, levels = [], []
    for lv, cd in leaves_codes:
        counts = leaf_counts(cd, group) if weighted else None
        levels.append(tree_levels(lv, counts))
        planes.append(pack_planes(cd))
    return {"planes": planes, "levels": levels, "group": group}


# ---------------------------------------------------------------------------
# Encoder from fp32 weights  ([T] c19: per block, K-means learns 256 values,
# which are sorted and become the leaves of the frequency-weighted tree)
# ---------------------------------------------------------------------------
KMEANS_ITERS = 25


def kmeans_init(w, n):
    """Starting centroids: the (2j+1)/(2n) quantiles of the block's weights,
    j = 0..n-1, by the inverted empirical distribution (a sample value, no
    interpolation).  Blocks of fewer than n weights repeat values."""
    s = np.sort(np.asarray(w, dtype=np.float32))
    g = s.size
    idx = -(-(2 * np.arange(n) + 1) * g // (2 * n)) - 1          # ceil(q g) - 1
    return s[idx].copy()


def kmeans_assign(w, c):
    """Index of the nearest centroid of every weight; distances |w - c| in
    fp64 (exact for fp32 operands of similar scale); ties go to the lowest
    index (argmin returns the first minimum), which for the ascending
    centroids of kmeans_block is the lower value."""
    d = np.abs(np.asarray(w, np.float64)[:, None] - np.asarray(c, np.float64)[None, :])
    return d.argmin(axis=1)


def kmeans_update(w, a, c):
    """New centroids: the mean of each centroid's members, summed in
    ascending order in fp64, divided by their count in fp64 and rounded to
    fp32; a centroid without members keeps its value."""
    w = np.asarray(w, np.float32)
    out = np.array(c, dtype=np.float32, copy=True)
    for j in range(out.size):
        m = np.sort(w[a == j]).astype(np.float64)
        if m.size:
            out[j] = np.float32(np.add.accumulate(m)[-1] / m.size)
    return out


def kmeans_block(w, n=NLEAF, max_iters=KMEANS_ITERS):
    """Lloyd's algorithm on one block: start at kmeans_init, then update,
    sort the centroids ([T] c19 sorts the learned values; done after every
    update, a relabelling, so that a tie between two values always goes to
    the lower one) and re-assign, until an update leaves the assignment
    unchanged or max_iters updates have run.  Sorting matters when starting
    centroids repeat (blocks with many equal weights): the first of a run of
    equal centroids can take members above the run and move past its empty
    twins.  The final sort and renumbering below are then no-ops.
    Returns (leaves fp32 [n] ascending, codes int64 [G], counts int64 [n],
    updates run); codes are the nearest leaves of the weights."""
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    c = kmeans_init(w, n)
    a = kmeans_assign(w, c)
    it = 0
    while it < max_iters:
        c = np.sort(kmeans_update(w, a, c))
        it += 1
        a_new = kmeans_assign(w, c)
        done = np.array_equal(a_new, a)
        a = a_new
        if done:
            break
    order = np.argsort(c, kind="stable")
    rank = np.empty_like(order)
    rank[order] = np.arange(order.size)
    return c[order], rank[a], np.bincount(rank[a], minlength=n), it


def encode_weights(W, group, max_iters=KMEANS_ITERS):
    """Encoder from a dense fp32 matrix W [rows][cols] ([T] c19, c21, c25):
    K-means per block of `group` inputs of one row, sorted leaves, the
    count-weighted tree, bitplanes.  Returns dict(codes uint8, leaves fp32
    [rows][nb][256], counts int64 [rows][nb][256], levels, planes)."""
    W = np.asarray(W, dtype=np.float32)
    rows, cols = W.shape
    nb = cols // group
    codes = np.empty((rows, cols), np.uint8)
    leaves = np.empty((rows, nb, NLEAF), np.float32)
    counts = np.empty((rows, nb, NLEAF), np.int64)
    for o in range(rows):
        for g in range(nb):
            lv, cd, n, _ = kmeans_block(W[o, g * group:(g + 1) * group], NLEAF, max_iters)
            codes[o, g * group:(g + 1) * group] = cd
            leaves[o, g] = lv
            counts[o, g] = n
    return {"codes": codes, "leaves": leaves, "counts": counts,
            "levels": tree_levels(leaves, counts), "planes": pack_planes(codes)}


def relative_weight_error(W, planes, levels, k, group):
    """||W - W_k||_F / ||W||_F in fp64, W_k the depth-k reconstruction
    ([T] c23 reports this measure at 4 bits)."""
    W = np.asarray(W, np.float64)
    Wk = dequant(planes, levels, k, group).astype(np.float64)
    return float(np.sqrt(np.sum((W - Wk) ** 2) / np.sum(W ** 2)))


# ---------------------------------------------------------------------------
# Routing  ([T] c4: a router picks a few experts per token, weights sum to 1)
# ---------------------------------------------------------------------------
def route(logits, top_k):
    """Top-k experts by descending logit (ties: lower index first) and their
    softmax weights renormalised over the selected k, computed in fp64 and
    rounded to fp32.  Returns (ids int32 [k], w float32 [k])."""
    logits = np.asarray(logits, dtype=np.float32)
    n = logits.shape[0]
    order = sorted(range(n), key=lambda e: (-float(logits[e]), e))
    ids = np.array(order[:top_k], dtype=np.int32)
    sel = logits[ids].astype(np.float64)
    ex = np.exp(sel - sel.max())
    w = (ex / ex.sum()).astype(np.float32)
    return ids, w


# ---------------------------------------------------------------------------
# Pre-I/O bit allocation  ([T] c29, c31; [Abs]: the prefix length is chosen
# before any read, from the token's routing weights and per-expert error
# profiles measured offline)
# ---------------------------------------------------------------------------
def isotonic_nonincreasing(d):
    """Least-squares fit of a non-increasing sequence to d (pool adjacent
    violators, equal weights)."""
    blocks = []                        # [sum, count]
    for v in d:
        blocks.append([float(v), 1])
        while len(blocks) > 1 and blocks[-2][0] / blocks[-2][1] < blocks[-1][0] / blocks[-1][1]:
            s, c = blocks.pop()
            blocks[-1][0] += s
            blocks[-1][1] += c
    out = []
    for s, c in blocks:
        out.extend([s / c] * c)
    return np.array(out, dtype=np.float64)


def repair_profile(err):
    """Make a profile convex: the marginal gains err(b) - err(b+1) are
    replaced by their non-increasing isotonic fit ([T] c31: each extra bit
    must help less than the one before; profiles that do not are repaired by
    isotonic regression).  err: float64 [nbits] for b = 1..nbits."""
    err = np.asarray(err, dtype=np.float64)
    gains = err[:-1] - err[1:]
    fit = isotonic_nonincreasing(gains)
    out = np.empty_like(err)
    out[0] = err[0]
    for b in range(1, err.shape[0]):
        out[b] = out[b - 1] - fit[b - 1]
    return out


def allocate_bits(w, err, budget, kmin=1, kmax=NBITS):
    """Greedy prefix-length allocation for one token ([T] c29).

    Minimises sum_e w_e^2 * err_e(b_e) subject to sum_e b_e = budget: every
    expert starts at kmin bits, then the single bit with the largest gain
    w_e^2 * (err_e(b_e) - err_e(b_e + 1)) is granted, repeatedly, until the
    budget is spent.  Profiles are repaired to convexity first ([T] c31), so
    the granted bits of an expert always form a prefix.  Gains are compared in
    fp64 as (w*w) * (err(b) - err(b+1)) with w widened from fp32; ties go to
    the larger routing weight, then the lower slot.

    w: float32 [n]; err: float64 [n][kmax] (err[e][b-1] for b = 1..kmax).
    Returns int32 [n]."""
    w = np.asarray(w, dtype=np.float32)
    n = w.shape[0]
    if not n * kmin <= budget <= n * kmax:
        raise ValueError("budget outside [n*kmin, n*kmax]")
    prof = [repair_profile(err[e]) for e in range(n)]
    b = [kmin] * n
    for _ in range(budget - n * kmin):
        best = None
        for e in range(n):
            if b[e] >= kmax:
                continue
            wd = float(w[e])
            gain = (wd * wd) * (prof[e][b[e] - 1] - prof[e][b[e]])
            key = (gain, wd, -e)
            if best is None or key > best[0]:
                best = (key, e)
        b[best[1]] += 1
    return np.array(b, dtype=np.int32)


# ---------------------------------------------------------------------------
# Residency rule  ([T] c13, c35: a plane is usable only when every earlier
# plane is resident; a request reads only the missing planes)
# ---------------------------------------------------------------------------
def missing_planes(resident, k):
    """Planes (0-based) to fetch when `resident` leading planes are held and a
    k-bit prefix is requested."""
    return list(range(resident, k)) if resident < k else []


# ---------------------------------------------------------------------------
# Expert caches of limited capacity, counted in planes  ([T] c11, c13, c35)
# ---------------------------------------------------------------------------
class PrefixPlaneCache:
    """One shared state per expert: its resident planes form a prefix 1..r.

    An access of expert e at k bits reads the missing planes r+1..k ([T] c35:
    3 resident and 5 requested reads planes 4 and 5; 5 resident and 3
    requested reads nothing) and refreshes planes k, k-1, .., 1 in that
    order, so that an expert's deeper planes are always older than its
    shallower ones and age out first ([T] c35).  Eviction takes the least
    recently used plane over all experts, which is then always the deepest
    resident plane of its expert, so every resident set stays a prefix.
    Planes needed by the access itself are never evicted for it; a request
    deeper than the whole capacity is read and not kept.

    Plain reference implementation: a list of (expert, plane) from least to
    most recently used."""

    def __init__(self, capacity_planes):
        self.cap = int(capacity_planes)
        self.order = []                 # [(expert, plane)], oldest first
        self.res = {}                   # expert -> resident prefix r
        self.accesses = self.hits = self.partial = self.planes_read = 0

    def resident(self, e):
        return self.res.get(e, 0)

    def _touch(self, e, p):
        if (e, p) in self.order:
            self.order.remove((e, p))
        self.order.append((e, p))

    def access(self, e, k):
        """Planes (1-based) read for this access."""
        self.accesses += 1
        r = self.resident(e)
        if r >= k:
            self.hits += 1
            for p in range(k, 0, -1):
                self._touch(e, p)
            return []
        if r > 0:
            self.partial += 1
        read = list(range(r + 1, k + 1))
        self.planes_read += len(read)
        if k > self.cap:                # cannot be held: read, keep nothing new
            for p in range(r, 0, -1):
                self._touch(e, p)
            return read
        # room for the missing planes; the victim is the oldest plane of any
        # expert but e (e's planes 1..r are about to be refreshed)
        while len(self.order) + (k - r) > self.cap:
            victim = next(x for x in self.order if x[0] != e)
            self.order.remove(victim)
            ve, vp = victim
            assert vp == self.res[ve], "an evicted plane must be its expert's deepest"
            self.res[ve] = vp - 1
            if self.res[ve] == 0:
                del self.res[ve]
        for p in range(k, 0, -1):
            self._touch(e, p)
        self.res[e] = k
        return read


class ObjectCache:
    """The independent-object baseline ([T] c11): every (expert, bit-width)
    is its own cache entry of k planes, so a resident 2-bit copy cannot serve
    a 4-bit request.  LRU over entries; a request larger than the capacity is
    read and not kept."""

    def __init__(self, capacity_planes):
        self.cap = int(capacity_planes)
        self.order = []                 # [(expert, k)], oldest first
        self.used = 0
        self.accesses = self.hits = self.partial = self.planes_read = 0

    def access(self, e, k):
        self.accesses += 1
        if (e, k) in self.order:
            self.hits += 1
            self.order.remove((e, k))
            self.order.append((e, k))
            return []
        self.planes_read += k
        if k > self.cap:
            return list(range(1, k + 1))
        while self.used + k > self.cap:
            _, vk = self.order.pop(0)
            self.used -= vk
        self.order.append((e, k))
        self.used += k
        return list(range(1, k + 1))


# ---------------------------------------------------------------------------
# One MoE layer for a batch of tokens
# ---------------------------------------------------------------------------
def moe_forward(experts, ids, w, k, x):
    """y[t] = sum_j w[t][j] * FFN_{ids[t][j]}(x[t]) at prefixes k[t][j][0..2].

    experts: {expert id: encoded expert}; ids int [B][topk]; w float32
    [B][topk]; k int [B][topk][3]; x float32 [B][hidden].  Returns (y fp64
    [B][hidden], S fp64 [B][hidden]) with S[t][o] = sum_j |w_tj| * Sy_tj[o]."""
    B, topk = np.asarray(ids).shape
    out = None
    scale = None
    for t in range(B):
        yt = None
        st = None
        for j in range(topk):
            e = int(ids[t][j])
            r = expert_ffn(experts[e], int(k[t][j][0]), int(k[t][j][1]), int(k[t][j][2]), x[t])
            wt = float(w[t][j])
            yt = wt * r["y"] if yt is None else yt + wt * r["y"]
            st = abs(wt) * r["Sy"] if st is None else st + abs(wt) * r["Sy"]
        if out is None:
            out = np.zeros((B, yt.shape[0]))
            scale = np.zeros((B, yt.shape[0]))
        out[t] = yt
        scale[t] = st
    return out, scale


def within_tolerance(got, want, scale, rel=1e-4, abs_=1e-6):
    """The acceptance bound |got - want| <= rel * scale + abs_ per output."""
    got = np.asarray(got, dtype=np.float64)
    return np.abs(got - want) <= rel * np.asarray(scale) + abs_


class DownwardCache:
    """The middle option the pages name and never measure ([T] c51): copies
    of different widths are still separate encodings, but a resident copy of
    width r serves every request at k <= r with no I/O (downward reuse), and a
    request at k > r reads a fresh k-bit copy in full, which replaces the old
    one (promotion).  One copy per expert at most; LRU over the copies, which
    are evicted whole.  The superseded copy is dropped before room is made.
    A request larger than the capacity is read and not kept; the resident
    copy then stays and is refreshed."""

    def __init__(self, capacity_planes):
        self.cap = int(capacity_planes)
        self.order = []                 # [expert], oldest first
        self.width = {}                 # expert -> width of its copy
        self.used = 0
        self.accesses = self.hits = self.partial = self.planes_read = 0

    def resident(self, e):
        return self.width.get(e, 0)

    def access(self, e, k):
        self.accesses += 1
        r = self.resident(e)
        if r >= k:
            self.hits += 1
            self.order.remove(e)
            self.order.append(e)
            return []
        self.planes_read += k
        if k > self.cap:
            if r:
                self.order.remove(e)
                self.order.append(e)
            return list(range(1, k + 1))
        if r:
            self.order.remove(e)
            self.used -= self.width.pop(e)
        while self.used + k > self.cap:
            self.used -= self.width.pop(self.order.pop(0))
        self.order.append(e)
        self.width[e] = k
        self.used += k
        return list(range(1, k + 1))
