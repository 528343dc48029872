// Expert caches of limited capacity counted in planes: the plane-aging prefix
// cache, the independent-object baseline and the downward-reuse middle option
// ("PagedMoE: Cross-Precision Expert Caching for SSD-Resident MoE Inference",
// podcast transcript, cues 11, 13, 35 and 51).  Host code; the replacement
// decisions only (the copies are the plane store's).
#include <cstdint>
#include <vector>

#include "pm_error.h"

namespace {

constexpr int kPlanes = 8;
constexpr int32_t kNil = -1;

// Intrusive LRU list over node ids (oldest at head).
struct Lru {
    std::vector<int32_t> prev, next;
    std::vector<uint8_t> in;
    int32_t head = kNil, tail = kNil;
    int64_t size = 0;

    explicit Lru(size_t n) : prev(n, kNil), next(n, kNil), in(n, 0) {}
    void unlink(int32_t x) {
        if (!in[x]) return;
        const int32_t p = prev[x], q = next[x];
        if (p != kNil) next[p] = q; else head = q;
        if (q != kNil) prev[q] = p; else tail = p;
        prev[x] = next[x] = kNil;
        in[x] = 0;
        --size;
    }
    void push_back(int32_t x) {       // most recently used
        unlink(x);
        prev[x] = tail;
        next[x] = kNil;
        if (tail != kNil) next[tail] = x; else head = x;
        tail = x;
        in[x] = 1;
        ++size;
    }
};

}  // namespace

struct pm_cache {
    int n_experts;
    int64_t cap;                       // planes
    int policy;
    // node = expert * 8 + (plane or width) - 1; the downward policy uses
    // node expert * 8 for the expert's one copy
    Lru lru;
    std::vector<int8_t> res;           // prefix: resident prefix; downward: copy width
    int64_t used = 0;                  // object and downward policies: planes held
    uint64_t accesses = 0, hits = 0, partial = 0, planes_read = 0;

    pm_cache(int n, int64_t c, int p)
        : n_experts(n), cap(c), policy(p), lru(size_t(n) * kPlanes), res(size_t(n), 0) {}
};

namespace {

// Prefix policy: an access at k refreshes planes k, k-1, .., 1 (in that
// order), so each expert's deeper planes are older and the globally oldest
// plane is always the deepest resident plane of its expert.
void access_prefix(pm_cache* c, int e, int k, int* first, int* count) {
    const int r = c->res[e];
    const int32_t base = e * kPlanes;
    if (r >= k) {
        ++c->hits;
        for (int p = k; p >= 1; --p) c->lru.push_back(base + p - 1);
        *first = k + 1;
        *count = 0;
        return;
    }
    if (r > 0) ++c->partial;
    *first = r + 1;
    *count = k - r;
    c->planes_read += uint64_t(k - r);
    if (k > c->cap) {                  // cannot be held: read, keep nothing new
        for (int p = r; p >= 1; --p) c->lru.push_back(base + p - 1);
        return;
    }
    // room for the missing planes: evict the oldest plane of any expert but
    // e (whose planes 1..r are refreshed below)
    while (c->lru.size + (k - r) > c->cap) {
        int32_t v = c->lru.head;
        while (v != kNil && v / kPlanes == e) v = c->lru.next[v];
        const int ve = v / kPlanes;
        c->lru.unlink(v);
        c->res[ve] = int8_t(v % kPlanes);          // its deepest plane went
    }
    for (int p = k; p >= 1; --p) c->lru.push_back(base + p - 1);
    c->res[e] = int8_t(k);
}

// Object policy: (expert, k) is one entry of k planes.
void access_object(pm_cache* c, int e, int k, int* first, int* count) {
    const int32_t node = e * kPlanes + k - 1;
    if (c->lru.in[node]) {
        ++c->hits;
        c->lru.push_back(node);
        *first = k + 1;
        *count = 0;
        return;
    }
    *first = 1;
    *count = k;
    c->planes_read += uint64_t(k);
    if (k > c->cap) return;
    while (c->used + k > c->cap) {
        const int32_t v = c->lru.head;
        c->lru.unlink(v);
        c->used -= v % kPlanes + 1;
    }
    c->lru.push_back(node);
    c->used += k;
}

// Downward policy: one copy per expert; a copy of width r >= k serves the
// request, a wider request reads a fresh copy in full and replaces it.
void access_downward(pm_cache* c, int e, int k, int* first, int* count) {
    const int32_t node = e * kPlanes;
    const int r = c->res[e];
    if (r >= k) {
        ++c->hits;
        c->lru.push_back(node);
        *first = k + 1;
        *count = 0;
        return;
    }
    *first = 1;
    *count = k;
    c->planes_read += uint64_t(k);
    if (k > c->cap) {                  // read, not kept; the old copy stays
        if (r) c->lru.push_back(node);
        return;
    }
    if (r) {                           // superseded before room is made
        c->lru.unlink(node);
        c->used -= r;
    }
    while (c->used + k > c->cap) {
        const int32_t v = c->lru.head;
        c->lru.unlink(v);
        c->used -= c->res[v / kPlanes];
        c->res[v / kPlanes] = 0;
    }
    c->lru.push_back(node);
    c->used += k;
    c->res[e] = int8_t(k);
}

void access(pm_cache* c, int e, int k, int* first, int* count) {
    if (c->policy == PM_CACHE_PREFIX)
        access_prefix(c, e, k, first, count);
    else if (c->policy == PM_CACHE_OBJECTS)
        access_object(c, e, k, first, count);
    else
        access_downward(c, e, k, first, count);
}

}  // namespace

extern "C" pm_status pm_cache_create(int n_experts, int64_t capacity_planes, int policy,
                                     pm_cache** out) {
    if (!out) return pm::failf(PM_ERR_ARG, "null output");
    *out = nullptr;
    if (n_experts <= 0 || n_experts > (1 << 27) || capacity_planes < 0)
        return pm::failf(PM_ERR_ARG, "bad expert count or capacity");
    if (policy != PM_CACHE_PREFIX && policy != PM_CACHE_OBJECTS && policy != PM_CACHE_DOWNWARD)
        return pm::failf(PM_ERR_ARG, "unknown cache policy %d", policy);
    *out = new pm_cache(n_experts, capacity_planes, policy);
    return PM_OK;
}

extern "C" pm_status pm_cache_destroy(pm_cache* c) {
    delete c;
    return PM_OK;
}

extern "C" pm_status pm_cache_access(pm_cache* c, int expert, int k, int* first, int* count) {
    if (!c || !first || !count) return pm::failf(PM_ERR_ARG, "null argument");
    if (expert < 0 || expert >= c->n_experts) return pm::failf(PM_ERR_ARG, "expert out of range");
    if (k < 1 || k > kPlanes) return pm::failf(PM_ERR_PREFIX, "k = %d outside 1..8", k);
    ++c->accesses;
    access(c, expert, k, first, count);
    return PM_OK;
}

extern "C" pm_status pm_cache_replay(pm_cache* c, const int32_t* experts, const int32_t* ks,
                                     size_t n) {
    if (!c || (n && (!experts || !ks))) return pm::failf(PM_ERR_ARG, "null argument");
    for (size_t i = 0; i < n; ++i) {
        if (experts[i] < 0 || experts[i] >= c->n_experts || ks[i] < 1 || ks[i] > kPlanes)
            return pm::failf(PM_ERR_ARG, "trace entry %zu out of range", i);
    }
    int first, count;
    for (size_t i = 0; i < n; ++i) {
        ++c->accesses;
        access(c, experts[i], ks[i], &first, &count);
    }
    return PM_OK;
}

extern "C" pm_status pm_cache_resident(const pm_cache* c, int expert, int* out) {
    if (!c || !out) return pm::failf(PM_ERR_ARG, "null argument");
    if (expert < 0 || expert >= c->n_experts) return pm::failf(PM_ERR_ARG, "expert out of range");
    if (c->policy != PM_CACHE_OBJECTS) {
        *out = c->res[expert];
    } else {
        int best = 0;
        for (int k = 1; k <= kPlanes; ++k)
            if (c->lru.in[expert * kPlanes + k - 1]) best = k;
        *out = best;
    }
    return PM_OK;
}

extern "C" pm_status pm_cache_stats(const pm_cache* c, uint64_t* accesses, uint64_t* hits,
                                    uint64_t* partial, uint64_t* planes_read,
                                    int64_t* planes_held) {
    if (!c) return pm::failf(PM_ERR_ARG, "null cache");
    if (accesses) *accesses = c->accesses;
    if (hits) *hits = c->hits;
    if (partial) *partial = c->partial;
    if (planes_read) *planes_read = c->planes_read;
    if (planes_held) *planes_held = c->policy == PM_CACHE_PREFIX ? c->lru.size : c->used;
    return PM_OK;
}
