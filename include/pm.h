/*
 * pm.h -- C ABI of libpm: direct execution of mixture-of-experts experts from
 * a cached k-bit prefix (k = 1..8) of a prefix-compatible binary-tree
 * codebook stored as bitplanes, on one AMD MI355X (gfx950).
 *
 * Sources (page titles):
 *   [T]   "PagedMoE: Cross-Precision Expert Caching for SSD-Resident MoE
 *         Inference", podcast episode transcript; "T cN" = subtitle cue N.
 *   [Abs] "PagedMoE: Cross-Precision Expert Caching for Token-Level Dynamic
 *         Precision in SSD-Resident MoE Inference", arxivlens page, Abstract.
 *   [Met] the same page, Analysis, "Methodology".
 *
 * Stored format (the pages fix the idea, the workload fixes the numbers):
 *   - A matrix has `rows` outputs and `cols` inputs.  Each weight is an 8-bit
 *     index into the codebook of its block; a block is `group` consecutive
 *     inputs of one row (group % 32 == 0, cols % group == 0).
 *   - Planes [T c25]: uint32 [8][rows][cols/32].  Plane p holds bit (7 - p)
 *     of every index (MSB first), and bit j of word w of a row is input
 *     column 32*w + j.  Planes are `plane_stride_words` apart (>= rows*cols/32)
 *     so that the three matrices of an expert can share one contiguous chunk
 *     per plane.
 *   - Levels [T c19, c21]: the tree over a block's 256 sorted leaves; each
 *     parent is the mean of its two children.  Depths 1..8 are stored
 *     (510 fp32 per block), level-major: the node of depth d, row o, block g,
 *     value v (v < 2^d) sits at
 *         pm_level_offset(s, d) + ((o * (cols/group) + g) << d) + v,
 *     pm_level_offset(s, d) = rows * (cols/group) * (2^d - 2).
 *   - The k-bit prefix of a weight is sum_{p<k} bit_p << (k-1-p), i.e. the top
 *     k bits of its index [T c21]; its value at precision k is the depth-k
 *     node of its block selected by that prefix.  Reading precision k touches
 *     planes 0..k-1 and depth k only [T c25; Abs].
 *
 * Conventions:
 *   - Every call validates all arguments before any launch or copy; on error
 *     nothing is launched and pm_last_error() describes the failure.
 *   - d_ pointers are device memory, h_ pointers host memory; the caller owns
 *     both unless a call says otherwise.  Streams are hipStream_t handles
 *     passed as void* (NULL = the null stream).  Device calls are
 *     asynchronous on their stream and never synchronise the device.
 *   - Every HIP error is returned as PM_ERR_HIP with HIP's text in
 *     pm_last_error().  Reductions run in a fixed order: the same call on the
 *     same inputs gives bit-identical outputs.
 *   - A pm_store is not thread-safe.
 */
#ifndef PM_H
#define PM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pm_status;
enum {
    PM_OK = 0,
    PM_ERR_ARG = -1,          /* null pointer, bad count, bad flag            */
    PM_ERR_SHAPE = -2,        /* group/cols/rows not of the stored format      */
    PM_ERR_PREFIX = -3,       /* k outside 1..8                                */
    PM_ERR_NOT_RESIDENT = -4, /* a prefix longer than the resident planes      */
    PM_ERR_OOM = -5,          /* store capacity or device memory exhausted     */
    PM_ERR_HIP = -6,          /* a HIP runtime call failed                     */
    PM_ERR_STATE = -7         /* call out of order (e.g. no host source)       */
};

/* Thread-local text of the last failure on this thread ("" if none). */
const char* pm_last_error(void);
/* Library version string. */
const char* pm_version(void);

typedef struct { int32_t rows, cols, group; } pm_matrix_shape;
/* An expert: gate [inter x hidden], up [inter x hidden], down [hidden x inter]. */
typedef struct { int32_t hidden, inter, group; } pm_expert_shape;

/* Sizes of the stored format; 0 for a shape that is not valid.
 * pm_level_offset returns (size_t)-1 for d outside 1..8. */
size_t pm_plane_words(pm_matrix_shape s);            /* rows*cols/32           */
size_t pm_levels_floats(pm_matrix_shape s);          /* rows*(cols/group)*510  */
size_t pm_level_offset(pm_matrix_shape s, int d);
/* Expert layout: plane p of an expert is one chunk of
 * pm_expert_plane_words(e) words holding gate, up, down planes back to back
 * (the unit of a top-up [T c25, c35]); levels are gate, up, down back to back.
 * pm_expert_matrix_offsets gives, for matrix m (0 gate, 1 up, 2 down), its word
 * offset inside a plane chunk and its float offset inside the levels. */
size_t pm_expert_plane_words(pm_expert_shape e);
size_t pm_expert_levels_floats(pm_expert_shape e);
pm_status pm_expert_matrix_offsets(pm_expert_shape e, int m, size_t* plane_word_off,
                                   size_t* level_float_off, pm_matrix_shape* shape_out);

/* ---------------------------------------------------------------- encoding
 * Offline encoder [T c19, c21, c25; Abs: one stored copy per expert, in a
 * tree codebook whose prefixes nest, laid out as bitplanes].
 *   codes:  uint8 [rows][cols], the 8-bit leaf index of every weight.
 *   leaves: fp32 [rows][cols/group][256], ascending per block (else
 *           PM_ERR_ARG).
 *   counts: uint32 [rows][cols/group][256] or NULL.  NULL: parent =
 *           (left + right) * 0.5f in fp32.  Otherwise parent = the
 *           count-weighted mean of its children [T c19, c21], evaluated in
 *           fp64 from the fp32 children and rounded to fp32, the parent's
 *           count being the sum of its children's; a parent whose children
 *           hold no weight takes the unweighted mean.
 *   planes_out: uint32, planes p at planes_out + p*plane_stride_words.
 *   levels_out: fp32 [pm_levels_floats(s)].
 * The host versions compute on the calling thread; the device versions take
 * device pointers and run on `stream`. */
pm_status pm_encode_matrix(pm_matrix_shape s, const uint8_t* codes, const float* leaves,
                           const uint32_t* counts, uint32_t* planes_out,
                           size_t plane_stride_words, float* levels_out);
pm_status pm_encode_expert(pm_expert_shape e, const uint8_t* const codes[3],
                           const float* const leaves[3], const uint32_t* const counts[3],
                           uint32_t* planes_out, float* levels_out);
pm_status pm_encode_matrix_device(pm_matrix_shape s, const uint8_t* d_codes,
                                  const float* d_leaves, const uint32_t* d_counts,
                                  uint32_t* d_planes_out, size_t plane_stride_words,
                                  float* d_levels_out, void* stream);

/* Encoder from fp32 weights, first half [T c19: per block, K-means learns 256
 * values, which are sorted and become the leaves of the tree].  For every
 * block of `group` inputs of one row of d_w fp32 [rows][cols] (device), 1-D
 * Lloyd's K-means with 256 centroids:
 *   start   centroid j = the ceil((2j+1)*group/512)-th smallest weight;
 *   assign  each weight to its nearest centroid, ties to the lowest index
 *           (distances exact in fp64 for weights within 2^29 of each other);
 *   update  each centroid with members = fp32 of their mean (fp64 sum in
 *           ascending order, fp64 division); one without members stays;
 *   stop    once an update changes no assignment, or after max_iters updates.
 * Outputs (device): d_codes uint8 [rows][cols] (each weight's nearest leaf),
 * d_leaves fp32 [rows][cols/group][256] ascending, d_counts uint32
 * [rows][cols/group][256] (weights per leaf), d_iters int32 [blocks] (updates
 * run; may be NULL).  Pass codes, leaves and counts to
 * pm_encode_matrix_device for the planes and the count-weighted tree.
 * group <= 4096 (else PM_ERR_SHAPE); max_iters >= 0.  Weights must be finite
 * (other values give unspecified codes). */
pm_status pm_kmeans_codebook_device(pm_matrix_shape s, const float* d_w, int max_iters,
                                    uint8_t* d_codes, float* d_leaves, uint32_t* d_counts,
                                    int32_t* d_iters, void* stream);

/* ---------------------------------------------------------------- prefix GEMV
 * y[o] = sum_i node(k, o, i/group, prefix_k(o, i)) * x[i]: one matrix read
 * directly at a k-bit prefix, no decoded matrix is formed [Abs: execution
 * straight from a cached prefix of 1 to 8 bits, never a full-precision copy;
 * T c37].  Reads planes 0..k-1 and depth k only.
 *   d_x fp32 [cols], 16-byte aligned; d_y fp32 [rows] (overwritten; cols == 0
 *   gives zeros).
 *   Errors: PM_ERR_PREFIX (k), PM_ERR_SHAPE, PM_ERR_ARG (null pointer or
 *   plane_stride_words < rows*cols/32). */
pm_status pm_expert_gemv(pm_matrix_shape s, int k, const uint32_t* d_planes,
                         size_t plane_stride_words, const float* d_levels,
                         const float* d_x, float* d_y, void* stream);

/* pm_expert_gemv for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same result, bit for bit, with the slice partials
 * (rows x cols/1024 floats when the columns span several 1024-column slices)
 * in a fixed array of PM_GEMV_NOALLOC_MAX_PARTIALS floats (2 MiB) that each
 * device holds from the first call until the process ends.  No allocation
 * and no memset: every partial is written before it is read.  Calls that
 * overlap on one device (concurrent streams or threads) share that array and
 * race; serialise them.  The first call on a device looks the array's
 * address up (not allocating).  Errors: those of pm_expert_gemv, and
 * PM_ERR_SHAPE when rows x ceil(cols/1024) > PM_GEMV_NOALLOC_MAX_PARTIALS,
 * whichever kernel the shape takes. */
#define PM_GEMV_NOALLOC_MAX_PARTIALS 524288
pm_status pm_expert_gemv_noalloc(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                 size_t plane_stride_words, const float* d_levels,
                                 const float* d_x, float* d_y, void* stream);

/* ---------------------------------------------------------------- routing
 * [T c4]: a router picks a few experts per token with weights summing to 1.
 * logits fp32 [n_tokens][n_experts] -> ids int32 [n_tokens][top_k] (largest
 * logit first, ties to the lower expert id) and w fp32 [n_tokens][top_k], the
 * softmax over the selected logits computed in fp64 and rounded to fp32.
 * Host memory. */
pm_status pm_route_topk(int n_tokens, int n_experts, int top_k, const float* logits,
                        int32_t* ids_out, float* w_out);

/* Pre-I/O prefix-length allocation [T c29, c31; Abs: the prefix length is
 * chosen before any read, from the token's routing weights and per-expert
 * error profiles measured offline].  Per token: minimise
 * sum_j w_j^2 * err_{ids_j}(b_j) subject to sum_j b_j = budget: start every
 * selected expert at 1 bit and grant, one at a time, the bit with the largest
 * gain (w*w) * (err(b) - err(b+1)) (fp64, w widened from fp32; ties to the
 * larger w, then the lower slot).  Profiles are first made convex: their
 * marginal gains are replaced by the least-squares non-increasing fit (pool
 * adjacent violators) [T c31].
 *   err_profiles float64 [n_experts][8] (err(b) at b = 1..8), host.
 *   k_out uint8 [n_tokens][top_k]; budget in [top_k, 8*top_k]. */
pm_status pm_allocate_bits(int n_tokens, int top_k, const int32_t* ids, const float* w,
                           int n_experts, const double* err_profiles, int budget,
                           uint8_t* k_out);

/* ---------------------------------------------------------------- plane store
 * HBM store of encoded experts with plane-granular residency [T c13, c35;
 * Abs: a cached prefix is reused as is or extended by reading only the planes
 * it lacks].  A slot (layer, expert) holds the plane chunks and the levels of
 * one expert; its resident prefix r counts the leading planes that are valid.
 * A plane is usable only when every earlier plane is resident, so r is always
 * a prefix count.  The store owns all slot memory, and memory follows
 * residency: a slot's planes sit in one buffer of as many plane chunks as a
 * top-up needed (plane p at planes + p * pm_expert_plane_words(e)), a
 * truncation releases the chunks past the kept prefix, and a slot holds its
 * levels while it holds any plane.  Growing or shrinking a buffer moves it
 * (the resident prefix is copied along), so slot addresses are valid only
 * until the next store call on that slot.  Slot memory is carved out of
 * arenas of the store's own (large device allocations kept until the store is
 * destroyed): a truncation gives the tail back in place and a top-up extends
 * a slot in place when it can, so neither allocates or frees device memory
 * in the common case.  Memory given back returns to the arenas once every
 * queued forward that read it and every copy from or into it has ended
 * (checked by later store calls).
 * flags: PM_STORE_HOST_FAKE backs slots with host memory and copies with
 * memcpy (bookkeeping tests without a GPU; compute calls reject such a
 * store).  capacity_bytes > 0 caps the slot memory, plane chunks plus levels
 * (PM_ERR_OOM beyond). */
typedef struct pm_store pm_store;
enum { PM_STORE_HOST_FAKE = 1u };
pm_status pm_store_create(pm_expert_shape e, int n_layers, int n_experts,
                          size_t capacity_bytes, uint32_t flags, pm_store** out);
pm_status pm_store_destroy(pm_store* s);
/* Slot memory for direct writes: all 8 plane chunks and the levels are
 * allocated (the resident prefix kept) and usable when the call returns;
 * plane chunk p at *planes + p * pm_expert_plane_words(e); levels at
 * *levels. */
pm_status pm_store_slot(pm_store* s, int layer, int expert, uint32_t** planes,
                        float** levels);
/* Declare that the caller has written planes 0..r-1 and all levels of a slot
 * (e.g. with pm_encode_matrix_device); r in 0..8. */
pm_status pm_store_set_resident(pm_store* s, int layer, int expert, int r);
/* Register the host source of a slot: h_planes uint32 [8][plane words],
 * h_levels fp32 [levels floats].  Caller-owned, pinned (hipHostMalloc) for an
 * asynchronous copy, alive as long as the store uses it. */
pm_status pm_store_attach_host(pm_store* s, int layer, int expert,
                               const uint32_t* h_planes, const float* h_levels);
/* Make planes r..k-1 resident by copying exactly those plane chunks from the
 * host source (plus the levels on a slot's first fill) on `side` (null: a
 * store side stream), then record the slot's ready event there; r becomes k.
 * A slot holding fewer than k chunks grows first, in place or by moving the
 * resident prefix to a new range (copied on `side`).  A copy that overwrites
 * chunks the slot already held waits for an earlier forward still reading
 * the slot; every copy waits for an earlier copy into the slot still in
 * flight.  No copy if r >= k [T c13, c35: a resident deeper prefix serves a
 * shallower request].  PM_ERR_STATE without a host source. */
pm_status pm_store_topup(pm_store* s, int layer, int expert, int k, void* side);
/* r = min(r, keep): the deepest planes age out first [T c35].  The plane
 * chunks past keep are released in place (at keep 0 the levels too); their
 * memory returns to the store's arenas once the slot's last reader and last
 * copy have ended. */
pm_status pm_store_truncate(pm_store* s, int layer, int expert, int keep);
/* Slot memory held by the store's slots: bytes (plane chunks and levels,
 * what capacity_bytes caps), plane chunks, and slots holding levels.  Memory
 * released but still in use by queued work, and free arena space, are not
 * counted.  Any output may be null. */
pm_status pm_store_usage(const pm_store* s, size_t* used_bytes, size_t* plane_chunks,
                         size_t* level_sets);
pm_status pm_store_resident(const pm_store* s, int layer, int expert, int* r_out);
/* Where a slot's memory is now, without changing it: its planes (null when
 * it holds no chunk), its levels (null when it holds none) and the plane
 * chunks it holds.  Valid until the next store call on the slot.  Any output
 * may be null. */
pm_status pm_store_slot_info(const pm_store* s, int layer, int expert, const uint32_t** planes,
                             const float** levels, int* chunks);
/* Planes copied by the last top-up of any slot (first plane, count) and the
 * running totals of plane chunks and bytes copied by top-ups. */
pm_status pm_store_copy_stats(const pm_store* s, int* last_first, int* last_count,
                              uint64_t* total_planes, uint64_t* total_bytes);
/* Optional timing hook: when n >= 4, each pm_moe_token_forward on this store
 * records events[0] before its first kernel, events[1] after the gate/up
 * kernels, events[2] after the down kernels and events[3] after the combine
 * (right after events[2] when the combine is folded into the down launch)
 * (hipEvent_t handles on the compute stream); n = 2 records events[0] and
 * events[1] only.  When the gate/up stage is a single launch, events[0] and
 * events[1] are that launch's own start and stop.  n = 0 switches it off;
 * other n are PM_ERR_ARG. */
pm_status pm_store_set_profile_events(pm_store* s, void* const* events, int n);

/* ---------------------------------------------------------------- expert caches
 * Replacement decisions for an expert cache whose capacity is counted in
 * planes (one plane = one bit of every index of one expert), for trace
 * replay and for a caller that drives pm_store_topup / pm_store_truncate.
 * Host only; no device memory.
 *   PM_CACHE_PREFIX  one state per expert: its resident planes are a prefix
 *     1..r.  An access at k reads only planes r+1..k; a deeper resident prefix
 *     serves a shallower request [T c13, c35].  The access then refreshes
 *     planes k, k-1, .., 1 in that order, so an expert's deeper planes are
 *     always older and leave first [T c35]; eviction takes the least recently
 *     used plane of any other expert, always the deepest plane of its expert.
 *   PM_CACHE_OBJECTS the independent-object baseline [T c11]: every (expert,
 *     k) is its own LRU entry of k planes and serves only requests at k.
 *   PM_CACHE_DOWNWARD the middle option [T c51]: copies are still separate
 *     encodings, one per expert; a resident copy of width r serves requests
 *     at k <= r, a wider request reads a k-plane copy in full and replaces it
 *     (the old copy is dropped before room is made).  LRU over whole copies.
 * Under both, a request deeper than the whole capacity is read and not kept.
 * Experts are 0..n_experts-1 (a caller numbers layer * n_experts + expert);
 * k in 1..8 (else PM_ERR_PREFIX from pm_cache_access). */
typedef struct pm_cache pm_cache;
enum { PM_CACHE_PREFIX = 0, PM_CACHE_OBJECTS = 1, PM_CACHE_DOWNWARD = 2 };
pm_status pm_cache_create(int n_experts, int64_t capacity_planes, int policy,
                          pm_cache** out);
pm_status pm_cache_destroy(pm_cache* c);
/* One access: *first (1-based) and *count are the planes it reads (count 0
 * on a hit, with *first = k + 1). */
pm_status pm_cache_access(pm_cache* c, int expert, int k, int* first, int* count);
/* n accesses from host arrays; the whole trace is checked (PM_ERR_ARG) before
 * the first access. */
pm_status pm_cache_replay(pm_cache* c, const int32_t* experts, const int32_t* ks, size_t n);
/* Planes of the expert now held: the prefix r (PREFIX), the largest k of its
 * resident entries (OBJECTS) or its copy's width (DOWNWARD); 0 if none. */
pm_status pm_cache_resident(const pm_cache* c, int expert, int* out);
/* Running totals (any output may be null): accesses, full hits, partial hits
 * (PREFIX: some planes resident, more read), planes read, planes held. */
pm_status pm_cache_stats(const pm_cache* c, uint64_t* accesses, uint64_t* hits,
                         uint64_t* partial, uint64_t* planes_read, int64_t* planes_held);

/* ---------------------------------------------------------------- MoE layer
 * One MoE layer for n_tokens tokens:
 *   y[t] = sum_j w[t][j] * W_down(k2) (silu(W_gate(k0) x[t]) * W_up(k1) x[t])
 * with expert ids[t][j] read at prefixes h_k[t][j][0..2] (gate, up, down)
 * [T c4, c37; Abs].  Tokens that share an expert are grouped: the store
 * tops it up once, to the largest prefix any of them needs, and each token
 * stops at its own prefix [Abs; T c25].  Each (use, matrix) runs as an
 * activation-LUT job (k <= 5 on the 1024-column grid) or on the direct
 * kernels; the uses that read one matrix of one expert at one prefix go to
 * the matrix-core tiles below when there are at least 6 of them.
 *   h_ids int32 [n_tokens][top_k], h_w fp32 [n_tokens][top_k],
 *   h_k uint8 [n_tokens][top_k][3] -- host memory, read before return.
 *   d_x fp32 [n_tokens][hidden] (16-byte aligned), d_y fp32 [n_tokens][hidden]
 *   (overwritten; it may be d_x itself).  At most 32767 uses
 *   (n_tokens * top_k) per call, else PM_ERR_ARG.
 * The routing-weighted sum over j [T c37] is folded into the down launch when
 * every down product is a LUT job and d_y does not overlap d_x: the first
 * gate/up launch clears d_y and each down row sum is added into it, times its
 * weight, with a float atomic, so the top_k terms of an output add up in the
 * order they arrive (the last bits may differ from call to call).  Otherwise,
 * and always under PM_DETERMINISTIC, a combine kernel adds them in slot
 * order.
 * flags: PM_AUTO_TOPUP tops up every short slot from its host source on the
 * store's side streams (copies that need no wait alternate over two, copies
 * that wait for an earlier forward's reads use a third) and makes `compute`
 * wait for them (kernels of resident experts are issued first); without it a
 * short slot is PM_ERR_NOT_RESIDENT.
 * PM_BATCH_MFMA puts every use on the matrix cores (larger batches [T c65:
 * untested on the pages]): the uses that read one matrix of one expert at one
 * prefix form tiles of up to 16, each weight is decoded once per tile (its
 * depth-k node) and multiplied on fp32 MFMA, so the values are the same
 * products in another summation order.  It needs group 128 and hidden, inter
 * multiples of 128 (else PM_ERR_SHAPE).
 * PM_READ_ONCE keeps every expert of several uses off the LUT path: the
 * direct kernels read its kmax planes once for all of them, each use taking
 * prefix_kmax >> (kmax - k) [T c25, c35] (the matrix-core tiles still take
 * groups of at least 6 uses).  Same values as the default path; the default
 * (a LUT job per use) re-reads the planes but needs fewer instructions.
 * PM_DETERMINISTIC keeps the separate combine: every sum then runs in a fixed
 * order (no atomics), so the same call on the same inputs gives the same bits.
 * The store keeps per-call workspace; calls on one store are serialised on
 * `compute`. */
enum { PM_AUTO_TOPUP = 1u, PM_BATCH_MFMA = 2u, PM_READ_ONCE = 4u, PM_DETERMINISTIC = 8u };
pm_status pm_moe_token_forward(pm_store* s, int layer, int n_tokens, int top_k,
                               const int32_t* h_ids, const float* h_w, const uint8_t* h_k,
                               const float* d_x, float* d_y, void* compute, uint32_t flags);

/* ---------------------------------------------------------------- checks and baselines
 * Bit-exact views of what the kernels decode (not on the hot path):
 *   pm_debug_unpack_prefix: d_prefix_out uint8 [rows][cols], the k-bit prefix.
 *   pm_debug_dequant:       d_w_out fp32 [rows][cols], the depth-k node.
 * The materialize-then-multiply comparator [T c37; Met]:
 *   pm_materialize_fp16: d_w_fp16 uint16 [rows][cols], the depth-k node
 *                        rounded to fp16 (nearest even).
 *   pm_gemv_fp16:        y[o] = sum_i fp16 W[o][i] * x[i] (fp32 sums).
 *   The _batch forms do the same for n <= 64 matrices in one launch, with
 *   the same results bit for bit; their arrays (shapes, ks, strides and the
 *   device pointers) are host memory.  Outputs and fp16 weight rows must be
 *   16-byte aligned (PM_ERR_ARG otherwise). */
pm_status pm_debug_unpack_prefix(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                 size_t plane_stride_words, uint8_t* d_prefix_out,
                                 void* stream);
pm_status pm_debug_dequant(pm_matrix_shape s, int k, const uint32_t* d_planes,
                           size_t plane_stride_words, const float* d_levels, float* d_w_out,
                           void* stream);
pm_status pm_materialize_fp16(pm_matrix_shape s, int k, const uint32_t* d_planes,
                              size_t plane_stride_words, const float* d_levels,
                              uint16_t* d_w_fp16, void* stream);
pm_status pm_materialize_fp16_batch(int n, const pm_matrix_shape* shapes, const int* ks,
                                    const uint32_t* const* d_planes,
                                    const size_t* plane_stride_words,
                                    const float* const* d_levels, uint16_t* const* d_w_fp16,
                                    void* stream);
pm_status pm_gemv_fp16_batch(int n, const pm_matrix_shape* shapes, const uint16_t* const* d_w,
                             const float* const* d_x, float* const* d_y, void* stream);
pm_status pm_gemv_fp16(pm_matrix_shape s, const uint16_t* d_w, const float* d_x, float* d_y,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PM_H */
