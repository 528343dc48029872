// Host side of libpm: argument validation, the offline encoder, routing, the
// pre-I/O bit allocator, the plane store and the orchestration of one MoE
// layer.  Every device computation is a HIP kernel in pm_kernels.hip.
#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "pm_encoder.h"
#include "pm_mfma.h"
#include "pm_error.h"
#include "pm_internal.h"

using namespace pm;

// ---------------------------------------------------------------- errors
static thread_local std::string g_last_error;

pm_status pm::failf(pm_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

static pm_status hip_fail(hipError_t e, const char* what) {
    return failf(PM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr)                                           \
    do {                                                        \
        hipError_t _e = (expr);                                 \
        if (_e != hipSuccess) return hip_fail(_e, #expr);       \
    } while (0)

extern "C" const char* pm_last_error(void) { return g_last_error.c_str(); }
extern "C" const char* pm_version(void) { return "libpm 0.1 (gfx950)"; }

// ---------------------------------------------------------------- shapes
static bool shape_ok(pm_matrix_shape s) {
    return s.rows >= 0 && s.cols >= 0 && s.group >= 32 && s.group % 32 == 0 &&
           s.cols % s.group == 0;
}

static pm_status check_shape(pm_matrix_shape s) {
    if (!shape_ok(s))
        return failf(PM_ERR_SHAPE,
                    "shape rows=%d cols=%d group=%d: need rows>=0, group a positive "
                    "multiple of 32, cols a multiple of group",
                    s.rows, s.cols, s.group);
    return PM_OK;
}

static pm_status check_k(int k) {
    if (k < 1 || k > kBits) return failf(PM_ERR_PREFIX, "prefix k=%d outside 1..8", k);
    return PM_OK;
}

static size_t nblocks(pm_matrix_shape s) { return size_t(s.rows) * size_t(s.cols / s.group); }

extern "C" size_t pm_plane_words(pm_matrix_shape s) {
    return shape_ok(s) ? size_t(s.rows) * size_t(s.cols) / 32 : 0;
}
extern "C" size_t pm_levels_floats(pm_matrix_shape s) {
    return shape_ok(s) ? nblocks(s) * kLevelFloatsPerBlock : 0;
}
extern "C" size_t pm_level_offset(pm_matrix_shape s, int d) {
    if (!shape_ok(s) || d < 1 || d > kBits) return size_t(-1);
    return level_offset(nblocks(s), d);
}

static bool expert_ok(pm_expert_shape e) {
    return e.hidden > 0 && e.inter > 0 && e.group >= 32 && e.group % 32 == 0 &&
           e.hidden % e.group == 0 && e.inter % e.group == 0;
}

static pm_matrix_shape matrix_of(pm_expert_shape e, int m) {
    if (m == 2) return pm_matrix_shape{e.hidden, e.inter, e.group};
    return pm_matrix_shape{e.inter, e.hidden, e.group};
}

extern "C" size_t pm_expert_plane_words(pm_expert_shape e) {
    if (!expert_ok(e)) return 0;
    return 2 * pm_plane_words(matrix_of(e, 0)) + pm_plane_words(matrix_of(e, 2));
}
extern "C" size_t pm_expert_levels_floats(pm_expert_shape e) {
    if (!expert_ok(e)) return 0;
    return 2 * pm_levels_floats(matrix_of(e, 0)) + pm_levels_floats(matrix_of(e, 2));
}
extern "C" pm_status pm_expert_matrix_offsets(pm_expert_shape e, int m, size_t* pw, size_t* lf,
                                              pm_matrix_shape* shape_out) {
    if (!expert_ok(e)) return failf(PM_ERR_SHAPE, "invalid expert shape");
    if (m < 0 || m > 2) return failf(PM_ERR_ARG, "matrix index %d outside 0..2", m);
    size_t p = 0, l = 0;
    for (int i = 0; i < m; ++i) {
        p += pm_plane_words(matrix_of(e, i));
        l += pm_levels_floats(matrix_of(e, i));
    }
    if (pw) *pw = p;
    if (lf) *lf = l;
    if (shape_out) *shape_out = matrix_of(e, m);
    return PM_OK;
}

static Geom make_geom(pm_expert_shape e) {
    Geom g{};
    g.hidden = e.hidden;
    g.inter = e.inter;
    g.group = e.group;
    g.plane_words = pm_expert_plane_words(e);
    for (int m = 0; m < 3; ++m) {
        pm_matrix_shape s;
        pm_expert_matrix_offsets(e, m, &g.plane_off[m], &g.level_off[m], &s);
        g.rows[m] = s.rows;
        g.cols[m] = s.cols;
    }
    return g;
}

// ---------------------------------------------------------------- host encoder
// The tree rule of the stored format: parent = (left + right) * 0.5f, or the
// count-weighted mean in fp64 when counts are given.  Compiled without FP
// contraction so both rules round exactly as written.
static pm_status encode_host(pm_matrix_shape s, const uint8_t* codes, const float* leaves,
                             const uint32_t* counts, uint32_t* planes, size_t pstride,
                             float* levels) {
    const int W = s.cols / 32;
    const int nb_row = s.cols / s.group;
    const size_t nb = nblocks(s);
    for (size_t b = 0; b < nb; ++b) {
        const float* lf = leaves + b * kLeaves;
        for (int v = 1; v < kLeaves; ++v)
            if (!(lf[v - 1] <= lf[v]))
                return failf(PM_ERR_ARG, "leaves of block %zu are not ascending at %d", b, v);
    }
    for (int p = 0; p < kBits; ++p) {
        for (int o = 0; o < s.rows; ++o) {
            for (int w = 0; w < W; ++w) {
                const uint8_t* c = codes + size_t(o) * s.cols + size_t(32) * w;
                uint32_t word = 0;
                for (int j = 0; j < 32; ++j) word |= uint32_t((c[j] >> (7 - p)) & 1u) << j;
                planes[size_t(p) * pstride + size_t(o) * W + w] = word;
            }
        }
    }
    std::vector<float> node(kLeaves), parent(kLeaves);
    std::vector<uint64_t> cnt(kLeaves), pcnt(kLeaves);
    for (size_t b = 0; b < nb; ++b) {
        (void)nb_row;
        const float* lf = leaves + b * kLeaves;
        for (int v = 0; v < kLeaves; ++v) {
            node[v] = lf[v];
            cnt[v] = counts ? counts[b * kLeaves + v] : 0;
        }
        float* out8 = levels + level_offset(nb, kBits) + (b << kBits);
        for (int v = 0; v < kLeaves; ++v) out8[v] = node[v];
        for (int d = kBits - 1; d >= 1; --d) {
            const int n = 1 << d;
            for (int p = 0; p < n; ++p) {
                const float L = node[2 * p], R = node[2 * p + 1];
                const float mean = (L + R) * 0.5f;
                if (counts) {
                    const uint64_t nl = cnt[2 * p], nr = cnt[2 * p + 1];
                    const uint64_t tot = nl + nr;
                    if (tot > 0) {
                        const double num = double(nl) * double(L) + double(nr) * double(R);
                        parent[p] = float(num / double(tot));
                    } else {
                        parent[p] = mean;
                    }
                    pcnt[p] = tot;
                } else {
                    parent[p] = mean;
                }
            }
            float* out = levels + level_offset(nb, d) + (b << d);
            for (int p = 0; p < n; ++p) {
                out[p] = parent[p];
                node[p] = parent[p];
                cnt[p] = pcnt[p];
            }
        }
    }
    return PM_OK;
}

extern "C" pm_status pm_encode_matrix(pm_matrix_shape s, const uint8_t* codes,
                                      const float* leaves, const uint32_t* counts,
                                      uint32_t* planes_out, size_t pstride, float* levels_out) {
    pm_status st = check_shape(s);
    if (st) return st;
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    if (!codes || !leaves || !planes_out || !levels_out)
        return failf(PM_ERR_ARG, "pm_encode_matrix: null pointer");
    if (pstride < pm_plane_words(s))
        return failf(PM_ERR_ARG, "plane stride %zu below plane size %zu", pstride,
                    pm_plane_words(s));
    return encode_host(s, codes, leaves, counts, planes_out, pstride, levels_out);
}

extern "C" pm_status pm_encode_expert(pm_expert_shape e, const uint8_t* const codes[3],
                                      const float* const leaves[3],
                                      const uint32_t* const counts[3], uint32_t* planes_out,
                                      float* levels_out) {
    if (!expert_ok(e)) return failf(PM_ERR_SHAPE, "invalid expert shape");
    if (!codes || !leaves || !planes_out || !levels_out)
        return failf(PM_ERR_ARG, "pm_encode_expert: null pointer");
    const size_t pw = pm_expert_plane_words(e);
    for (int m = 0; m < 3; ++m) {
        size_t po, lo;
        pm_matrix_shape s;
        pm_expert_matrix_offsets(e, m, &po, &lo, &s);
        pm_status st = pm_encode_matrix(s, codes[m], leaves[m], counts ? counts[m] : nullptr,
                                        planes_out + po, pw, levels_out + lo);
        if (st) return st;
    }
    return PM_OK;
}

extern "C" pm_status pm_encode_matrix_device(pm_matrix_shape s, const uint8_t* d_codes,
                                             const float* d_leaves, const uint32_t* d_counts,
                                             uint32_t* d_planes, size_t pstride, float* d_levels,
                                             void* stream) {
    pm_status st = check_shape(s);
    if (st) return st;
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    if (!d_codes || !d_leaves || !d_planes || !d_levels)
        return failf(PM_ERR_ARG, "pm_encode_matrix_device: null pointer");
    if (pstride < pm_plane_words(s))
        return failf(PM_ERR_ARG, "plane stride %zu below plane size %zu", pstride,
                    pm_plane_words(s));
    HIP_TRY(launch_encode_device(s.rows, s.cols, s.group, d_codes, d_leaves, d_counts,
                                 d_planes, pstride, d_levels, (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_kmeans_codebook_device(pm_matrix_shape s, const float* d_w,
                                               int max_iters, uint8_t* d_codes, float* d_leaves,
                                               uint32_t* d_counts, int32_t* d_iters,
                                               void* stream) {
    pm_status st = check_shape(s);
    if (st) return st;
    if (s.group > kMaxKmeansGroup)
        return failf(PM_ERR_SHAPE, "K-means block of %d weights above %d", s.group,
                     kMaxKmeansGroup);
    if (max_iters < 0) return failf(PM_ERR_ARG, "max_iters %d below 0", max_iters);
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    if (!d_w || !d_codes || !d_leaves || !d_counts)
        return failf(PM_ERR_ARG, "pm_kmeans_codebook_device: null pointer");
    if (nblocks(s) > 0xFFFFFFFFu) return failf(PM_ERR_SHAPE, "more than 2^32-1 blocks");
    HIP_TRY(launch_kmeans_device(s.rows, s.cols, s.group, d_w, max_iters, d_codes, d_leaves,
                                 d_counts, d_iters, (hipStream_t)stream));
    return PM_OK;
}

// ---------------------------------------------------------------- device calls
static pm_status check_matrix_call(pm_matrix_shape s, int k, const void* planes,
                                   size_t pstride, const void* a, const void* b) {
    pm_status st = check_shape(s);
    if (st) return st;
    st = check_k(k);
    if (st) return st;
    if (s.rows == 0) return PM_OK;
    if (!planes || !a || !b) return failf(PM_ERR_ARG, "null device pointer");
    if (pstride < pm_plane_words(s))
        return failf(PM_ERR_ARG, "plane stride %zu below plane size %zu", pstride,
                    pm_plane_words(s));
    return PM_OK;
}

// The LUT kernels address planes and tables with 32-bit byte offsets from a
// slice's base: planes 0..k-1 and the depth-k tables of one matrix must fit.
static bool lut_offsets_fit(pm_matrix_shape s, int k, size_t pstride) {
    const uint64_t lim = uint64_t(1) << 31;
    const uint64_t planes = (uint64_t(k - 1) * pstride + uint64_t(s.rows) * (s.cols / 32)) * 4;
    const uint64_t tables = uint64_t(s.rows) * (s.cols / s.group) * (uint64_t(1) << k) * 4;
    return planes < lim && tables < lim;
}

// partials: S * rows floats for the slice partials when the columns span
// S > 1 slices; null takes the calling stream's own (growing) buffer.
pm_status gemv_lut(pm_matrix_shape s, int k, const uint32_t* d_planes, size_t pstride,
                   const float* d_levels, const float* d_x, float* d_y, hipStream_t st,
                   float* partials);

static pm_status check_gemv_call(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                 size_t pstride, const float* d_levels, const float* d_x,
                                 float* d_y) {
    pm_status st = check_matrix_call(s, k, d_planes, pstride, d_levels, d_y);
    if (st) return st;
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    if (!d_x) return failf(PM_ERR_ARG, "null x");
    if (reinterpret_cast<uintptr_t>(d_x) % 16) return failf(PM_ERR_ARG, "x not 16-byte aligned");
    return PM_OK;
}

static bool gemv_takes_lut(pm_matrix_shape s, int k, size_t pstride) {
    return k <= kGemvLutMaxK && s.cols > 0 && s.cols % kSliceCols == 0 && s.group == kLutGroup &&
           s.rows % kLutRows == 0 && lut_offsets_fit(s, k, pstride);
}

extern "C" pm_status pm_expert_gemv(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                    size_t pstride, const float* d_levels, const float* d_x,
                                    float* d_y, void* stream) {
    pm_status st = check_gemv_call(s, k, d_planes, pstride, d_levels, d_x, d_y);
    if (st) return st;
    if (s.rows == 0) return PM_OK;
    if (gemv_takes_lut(s, k, pstride))
        return gemv_lut(s, k, d_planes, pstride, d_levels, d_x, d_y, (hipStream_t)stream,
                        nullptr);
    HIP_TRY(launch_gemv(s.rows, s.cols, s.group, k, d_planes, pstride, d_levels, d_x, d_y,
                        (hipStream_t)stream));
    return PM_OK;
}

// ---- pm_expert_gemv without allocation: the slice partials live in a fixed
// array of device memory, one per device (each device loaded the library's
// code object holds its own copy, for the life of the process).
namespace {
constexpr size_t kScratchFloats = PM_GEMV_NOALLOC_MAX_PARTIALS;
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kScratchDevices] = {};
}  // namespace

static __device__ __align__(256) float scratch[kScratchFloats];

// The device address of the current device's array, looked up once per
// device with that device current.  The host-side name `scratch` is not a
// device address and is never passed to a kernel or a copy.
static pm_status scratch_address(float** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kScratchDevices)
        return failf(PM_ERR_STATE, "device %d beyond the %d with a scratch address", dev,
                     kScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return failf(PM_ERR_HIP, "scratch address on device %d: %s", dev,
                         hipGetErrorString(e));
        }
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return PM_OK;
}

extern "C" pm_status pm_expert_gemv_noalloc(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                            size_t pstride, const float* d_levels,
                                            const float* d_x, float* d_y, void* stream) {
    pm_status st = check_gemv_call(s, k, d_planes, pstride, d_levels, d_x, d_y);
    if (st) return st;
    const size_t slices = (size_t(s.cols) + kSliceCols - 1) / kSliceCols;
    if (size_t(s.rows) * slices > kScratchFloats)
        return failf(PM_ERR_SHAPE,
                     "rows x column slices = %d x %zu exceeds the %zu partials of the fixed "
                     "scratch (use pm_expert_gemv)",
                     s.rows, slices, kScratchFloats);
    if (s.rows == 0) return PM_OK;
    if (gemv_takes_lut(s, k, pstride)) {
        float* partials = nullptr;
        if (s.cols / kSliceCols > 1) {
            st = scratch_address(&partials);
            if (st) return st;
        }
        return gemv_lut(s, k, d_planes, pstride, d_levels, d_x, d_y, (hipStream_t)stream,
                        partials);
    }
    HIP_TRY(launch_gemv(s.rows, s.cols, s.group, k, d_planes, pstride, d_levels, d_x, d_y,
                        (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_debug_unpack_prefix(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                            size_t pstride, uint8_t* d_out, void* stream) {
    pm_status st = check_matrix_call(s, k, d_planes, pstride, d_out, d_out);
    if (st) return st;
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    HIP_TRY(launch_unpack_prefix(s.rows, s.cols, k, d_planes, pstride, d_out,
                                 (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_debug_dequant(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                      size_t pstride, const float* d_levels, float* d_w,
                                      void* stream) {
    pm_status st = check_matrix_call(s, k, d_planes, pstride, d_levels, d_w);
    if (st) return st;
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    HIP_TRY(launch_dequant(s.rows, s.cols, s.group, k, d_planes, pstride, d_levels, d_w,
                           nullptr, (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_materialize_fp16(pm_matrix_shape s, int k, const uint32_t* d_planes,
                                         size_t pstride, const float* d_levels, uint16_t* d_w,
                                         void* stream) {
    pm_status st = check_matrix_call(s, k, d_planes, pstride, d_levels, d_w);
    if (st) return st;
    if (s.rows == 0 || s.cols == 0) return PM_OK;
    HIP_TRY(launch_dequant(s.rows, s.cols, s.group, k, d_planes, pstride, d_levels, nullptr,
                           d_w, (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_materialize_fp16_batch(int n, const pm_matrix_shape* shapes,
                                               const int* ks, const uint32_t* const* d_planes,
                                               const size_t* pstrides,
                                               const float* const* d_levels,
                                               uint16_t* const* d_w_fp16, void* stream) {
    if (n < 0 || n > kMaxBatchMats) return failf(PM_ERR_ARG, "batch of %d matrices outside 0..%d",
                                                 n, kMaxBatchMats);
    if (n == 0) return PM_OK;
    if (!shapes || !ks || !d_planes || !pstrides || !d_levels || !d_w_fp16)
        return failf(PM_ERR_ARG, "null batch array");
    KDequantBatch B{};
    size_t max_elems = 0;
    for (int m = 0; m < n; ++m) {
        const pm_matrix_shape s = shapes[m];
        pm_status st = check_matrix_call(s, ks[m], d_planes[m], pstrides[m], d_levels[m], d_w_fp16[m]);
        if (st) return st;
        if (reinterpret_cast<uintptr_t>(d_w_fp16[m]) % 16)
            return failf(PM_ERR_ARG, "output %d not 16-byte aligned", m);
        const size_t nb = size_t(s.rows) * (s.cols / s.group);
        B.rows[B.n] = s.rows;
        B.cols[B.n] = s.cols;
        B.group[B.n] = s.group;
        B.k[B.n] = ks[m];
        B.pstride[B.n] = pstrides[m];
        B.planes[B.n] = d_planes[m];
        B.lvk[B.n] = d_levels[m] + level_offset(nb, ks[m]);
        B.w[B.n] = d_w_fp16[m];
        max_elems = std::max(max_elems, size_t(s.rows) * s.cols);
        if (size_t(s.rows) * s.cols > 0) ++B.n;
    }
    HIP_TRY(launch_dequant_batch(B, max_elems, (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_gemv_fp16_batch(int n, const pm_matrix_shape* shapes,
                                        const uint16_t* const* d_w, const float* const* d_x,
                                        float* const* d_y, void* stream) {
    if (n < 0 || n > kMaxBatchMats) return failf(PM_ERR_ARG, "batch of %d matrices outside 0..%d",
                                                 n, kMaxBatchMats);
    if (n == 0) return PM_OK;
    if (!shapes || !d_w || !d_x || !d_y) return failf(PM_ERR_ARG, "null batch array");
    KGemv16Batch B{};
    int max_rows = 0;
    for (int m = 0; m < n; ++m) {
        const pm_matrix_shape s = shapes[m];
        pm_status st = check_shape(s);
        if (st) return st;
        if (s.rows == 0) continue;
        if (s.cols == 0) return failf(PM_ERR_SHAPE, "matrix %d has no columns", m);
        if (!d_w[m] || !d_x[m] || !d_y[m]) return failf(PM_ERR_ARG, "null device pointer");
        if (reinterpret_cast<uintptr_t>(d_w[m]) % 16 || (size_t(s.cols) * 2) % 16)
            return failf(PM_ERR_ARG, "weights %d: rows not 16-byte aligned", m);
        if (reinterpret_cast<uintptr_t>(d_x[m]) % 16)
            return failf(PM_ERR_ARG, "x %d not 16-byte aligned", m);
        B.rows[B.n] = s.rows;
        B.cols[B.n] = s.cols;
        B.w[B.n] = d_w[m];
        B.x[B.n] = d_x[m];
        B.y[B.n] = d_y[m];
        ++B.n;
        max_rows = std::max(max_rows, s.rows);
    }
    HIP_TRY(launch_gemv_fp16_batch(B, max_rows, (hipStream_t)stream));
    return PM_OK;
}

extern "C" pm_status pm_gemv_fp16(pm_matrix_shape s, const uint16_t* d_w, const float* d_x,
                                  float* d_y, void* stream) {
    pm_status st = check_shape(s);
    if (st) return st;
    if (s.rows == 0) return PM_OK;
    if (!d_y || (s.cols > 0 && (!d_w || !d_x))) return failf(PM_ERR_ARG, "null device pointer");
    if (s.cols > 0 && (reinterpret_cast<uintptr_t>(d_w) % 16 || reinterpret_cast<uintptr_t>(d_x) % 16))
        return failf(PM_ERR_ARG, "weights and x must be 16-byte aligned");
    HIP_TRY(launch_gemv_fp16(s.rows, s.cols, d_w, d_x, d_y, (hipStream_t)stream));
    return PM_OK;
}

// ---------------------------------------------------------------- routing
extern "C" pm_status pm_route_topk(int n_tokens, int n_experts, int top_k, const float* logits,
                                   int32_t* ids_out, float* w_out) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts)
        return failf(PM_ERR_ARG, "route: n_tokens=%d n_experts=%d top_k=%d", n_tokens,
                    n_experts, top_k);
    if (n_tokens == 0) return PM_OK;
    if (!logits || !ids_out || !w_out) return failf(PM_ERR_ARG, "route: null pointer");
    std::vector<int32_t> order(n_experts);
    std::vector<double> ex(top_k);
    for (int t = 0; t < n_tokens; ++t) {
        const float* l = logits + size_t(t) * n_experts;
        for (int e = 0; e < n_experts; ++e) {
            if (std::isnan(l[e])) return failf(PM_ERR_ARG, "route: NaN logit");
            order[e] = e;
        }
        std::partial_sort(order.begin(), order.begin() + top_k, order.end(),
                          [l](int32_t a, int32_t b) {
                              return l[a] > l[b] || (l[a] == l[b] && a < b);
                          });
        const double lmax = double(l[order[0]]);
        double sum = 0.0;
        for (int j = 0; j < top_k; ++j) {
            ex[j] = std::exp(double(l[order[j]]) - lmax);
            sum += ex[j];
        }
        for (int j = 0; j < top_k; ++j) {
            ids_out[size_t(t) * top_k + j] = order[j];
            w_out[size_t(t) * top_k + j] = float(ex[j] / sum);
        }
    }
    return PM_OK;
}

// ---------------------------------------------------------------- allocator
// Least-squares non-increasing fit by pooling adjacent violators.
static void fit_nonincreasing(const double* d, int n, double* out) {
    std::vector<double> bsum;
    std::vector<int> bcnt;
    for (int i = 0; i < n; ++i) {
        bsum.push_back(d[i]);
        bcnt.push_back(1);
        while (bsum.size() > 1) {
            const size_t z = bsum.size();
            if (!(bsum[z - 2] / bcnt[z - 2] < bsum[z - 1] / bcnt[z - 1])) break;
            bsum[z - 2] += bsum[z - 1];
            bcnt[z - 2] += bcnt[z - 1];
            bsum.pop_back();
            bcnt.pop_back();
        }
    }
    int i = 0;
    for (size_t b = 0; b < bsum.size(); ++b)
        for (int c = 0; c < bcnt[b]; ++c) out[i++] = bsum[b] / bcnt[b];
}

static void convex_profile(const double* err, double* out) {
    double gains[kBits - 1], fit[kBits - 1];
    for (int b = 0; b < kBits - 1; ++b) gains[b] = err[b] - err[b + 1];
    fit_nonincreasing(gains, kBits - 1, fit);
    out[0] = err[0];
    for (int b = 1; b < kBits; ++b) out[b] = out[b - 1] - fit[b - 1];
}

extern "C" pm_status pm_allocate_bits(int n_tokens, int top_k, const int32_t* ids,
                                      const float* w, int n_experts, const double* err,
                                      int budget, uint8_t* k_out) {
    if (n_tokens < 0 || top_k < 1 || n_experts < 1)
        return failf(PM_ERR_ARG, "allocate: n_tokens=%d top_k=%d n_experts=%d", n_tokens, top_k,
                    n_experts);
    if (budget < top_k || budget > kBits * top_k)
        return failf(PM_ERR_ARG, "allocate: budget %d outside [%d, %d]", budget, top_k,
                    kBits * top_k);
    if (n_tokens == 0) return PM_OK;
    if (!ids || !w || !err || !k_out) return failf(PM_ERR_ARG, "allocate: null pointer");
    std::vector<double> prof(size_t(top_k) * kBits);
    std::vector<int> b(top_k);
    for (int t = 0; t < n_tokens; ++t) {
        for (int j = 0; j < top_k; ++j) {
            const int32_t e = ids[size_t(t) * top_k + j];
            if (e < 0 || e >= n_experts)
                return failf(PM_ERR_ARG, "allocate: expert id %d outside 0..%d", e,
                            n_experts - 1);
            convex_profile(err + size_t(e) * kBits, &prof[size_t(j) * kBits]);
            b[j] = 1;
        }
        for (int step = 0; step < budget - top_k; ++step) {
            int best = -1;
            double bg = 0.0, bw = 0.0;
            for (int j = 0; j < top_k; ++j) {
                if (b[j] >= kBits) continue;
                const double wd = double(w[size_t(t) * top_k + j]);
                const double* p = &prof[size_t(j) * kBits];
                const double gain = (wd * wd) * (p[b[j] - 1] - p[b[j]]);
                if (best < 0 || gain > bg || (gain == bg && wd > bw)) {
                    best = j;
                    bg = gain;
                    bw = wd;
                }
            }
            b[best] += 1;
        }
        for (int j = 0; j < top_k; ++j) k_out[size_t(t) * top_k + j] = uint8_t(b[j]);
    }
    return PM_OK;
}

// ---------------------------------------------------------------- store
namespace {

// A slot's planes live in one buffer of `cap` plane chunks (plane p at
// planes + p * plane_words), so the kernels address any resident prefix with
// one stride; the buffer grows and shrinks with the resident prefix, and the
// levels are held while the slot holds any plane.
struct Slot {
    uint32_t* planes = nullptr;    // cap chunks of plane_words
    int cap = 0;                   // plane chunks allocated
    float* levels = nullptr;
    int resident = 0;              // leading planes that are valid
    bool levels_ready = false;
    const uint32_t* h_planes = nullptr;
    const float* h_levels = nullptr;
    hipEvent_t ready = nullptr;    // recorded after the slot's last top-up copy
    // `ready` marks the slot's last copy (top-up or move): `copied` once it
    // has been recorded at all; `pending` until a forward's compute stream
    // has waited for it.  Another copy from or into the slot waits for it
    // whatever `pending` says: a forward's wait orders only its own stream.
    bool copied = false;
    bool pending = false;
    uint64_t read_seq = 0;         // last forward that read the slot (0: none)
};

// A range of slot memory given back while a queued forward or copy may still
// use it: it returns to its arena once the copy event has completed and the
// forward `reader` has ended.
struct Released {
    char* p;
    size_t len;
    hipEvent_t ev;                 // after the last copy from or into it (null: none)
    uint64_t reader;               // the last forward that read it (0: none)
};

// One block of slot memory (hipMalloc, or calloc for a host-backed store),
// carved into ranges first fit; its free ranges by offset, coalesced.
struct Arena {
    char* base;
    size_t size;
    std::map<size_t, size_t> free;
};

struct Workspace {
    float* d_buf = nullptr;        // G, U, Y partial results
    size_t d_floats = 0;
    char* h_ring = nullptr;        // pinned staging of work lists
    char* d_ring = nullptr;
    size_t slot_bytes = 0;
    static constexpr int kSlots = 16;
    hipEvent_t ring_ev[kSlots] = {};
    int next = 0;
};

}  // namespace

struct pm_store {
    pm_expert_shape shape;
    Geom geom;
    int n_layers, n_experts;
    size_t capacity, used = 0;         // bytes: allocated plane chunks and levels
    bool host_fake;
    size_t plane_bytes, level_bytes;   // per plane chunk, per slot levels
    std::vector<Slot> slots;
    std::vector<int> item_of;          // forward scratch: expert -> item, -1 between calls
    // The store's own streams.  side[0] is the memory stream: the waits that
    // a truncation's release of memory follows.
    // Top-up copies that need no wait take side[1] and side[2] in turn (more
    // than one copy in flight keeps the link busier); copies that wait for an
    // earlier forward still reading their slot take side[3], so that a wait
    // holds up no other copy.
    static constexpr int kSides = 4;
    static constexpr int kMem = 0, kWaits = 3;
    hipStream_t side[kSides] = {};
    uint32_t next_side = 0;
    // Slot memory: arenas of the store's own.  Ranges a queued forward or
    // copy may still use wait in `released` until a later store call finds
    // them idle.
    std::vector<Arena> arenas;
    size_t arena_bytes = 0;            // size of a new arena (a larger request gets its own)
    std::vector<Released> released;
    std::vector<hipEvent_t> spare_events;
    // Ends of recent forwards: done[n % kDone] marks the end of forward n
    // (n >= 1).  A forward records it only when the store has host sources
    // (a top-up may need it); otherwise it is recorded later on the last
    // forward's stream, when a forward on another stream or a top-up needs
    // it, and then marks everything queued there so far.  Every queued event
    // costs the launch-bound layer step about 3 us.  Forwards of one store
    // complete in order, so an entry that marks a later forward than the one
    // asked for is still safe to wait on.
    static constexpr int kDone = 32;
    hipEvent_t done[kDone] = {};
    uint64_t done_seq[kDone] = {};     // the forward each entry marks the end of
    uint64_t fwd_seq = 0;              // forwards issued
    uint64_t recorded_seq = 0;         // last forward whose end is recorded
    hipStream_t last_compute = nullptr;    // stream of the last forward
    bool has_sources = false;          // some slot has a host source
    Workspace ws;
    int last_first = -1, last_count = 0;
    uint64_t total_planes = 0, total_bytes = 0;
    hipEvent_t prof[4] = {};
    bool profiling = false;
    int n_prof = 0;                    // 2: gate/up only; 4: every stage
};

static pm_status slot_of(const pm_store* s, int layer, int expert, size_t* idx) {
    if (!s) return failf(PM_ERR_ARG, "null store");
    if (layer < 0 || layer >= s->n_layers || expert < 0 || expert >= s->n_experts)
        return failf(PM_ERR_ARG, "slot (%d, %d) outside %d layers x %d experts", layer, expert,
                    s->n_layers, s->n_experts);
    *idx = size_t(layer) * s->n_experts + expert;
    return PM_OK;
}

// ---- slot memory.  A store carves slot memory out of arenas of its own
// (large hipMalloc blocks, never returned before the store is destroyed), so
// growing, shrinking and releasing a slot are host bookkeeping: no device
// allocation or free in the path of a top-up or a truncation.  A slot's
// planes are one range of `cap` plane chunks; a truncation gives the tail
// back in place, and a top-up extends the range in place when the range after
// it is free, else moves the resident prefix to a new range.  A range given
// back while a queued forward may read it, or a copy may still write or read
// it, waits with an event until a later store call finds it idle.
static bool slot_reader_running(pm_store* s, const Slot& sl, hipEvent_t* ev);
static hipEvent_t forward_end(pm_store* s, uint64_t n);

constexpr size_t kRangeAlign = 256;
static size_t range_len(size_t bytes) { return (bytes + kRangeAlign - 1) & ~(kRangeAlign - 1); }

static Arena* arena_of(pm_store* s, const char* p) {
    for (Arena& a : s->arenas)
        if (p >= a.base && p < a.base + a.size) return &a;
    return nullptr;
}

// Give [p, p + len) back to its arena now, merged with free neighbours.
static void arena_put(pm_store* s, char* p, size_t len) {
    Arena* a = arena_of(s, p);
    if (!a || len == 0) return;
    size_t off = size_t(p - a->base);
    auto next = a->free.lower_bound(off);
    if (next != a->free.end() && off + len == next->first) {
        len += next->second;
        next = a->free.erase(next);
    }
    if (next != a->free.begin()) {
        auto prev = std::prev(next);
        if (prev->first + prev->second == off) {
            prev->second += len;
            return;
        }
    }
    a->free.emplace(off, len);
}

static pm_status take_event(pm_store* s, hipEvent_t* ev) {
    if (!s->spare_events.empty()) {
        *ev = s->spare_events.back();
        s->spare_events.pop_back();
        return PM_OK;
    }
    HIP_TRY(hipEventCreateWithFlags(ev, hipEventDisableTiming));
    return PM_OK;
}

// Return the released ranges whose last copy and last reader have ended.
static void reclaim(pm_store* s) {
    if (s->released.empty()) return;
    std::vector<Released> keep;
    for (const Released& r : s->released) {
        bool idle = !r.ev || hipEventQuery(r.ev) == hipSuccess;
        if (idle && r.reader) idle = hipEventQuery(forward_end(s, r.reader)) == hipSuccess;
        if (!idle) {
            keep.push_back(r);
            continue;
        }
        arena_put(s, r.p, r.len);
        if (r.ev) s->spare_events.push_back(r.ev);
    }
    s->released.swap(keep);
}

// Give back [p, p + len): at once in a host-backed store, else after the
// copies issued on `last` so far (an event recorded there now; null: none in
// flight) and the end of forward `reader`.
static pm_status release_range(pm_store* s, char* p, size_t len, hipStream_t last,
                               uint64_t reader) {
    if (!p || len == 0) return PM_OK;
    if (s->host_fake) {
        arena_put(s, p, len);
        return PM_OK;
    }
    hipEvent_t ev = nullptr;
    if (last) {
        pm_status st = take_event(s, &ev);
        if (st) return st;
        const hipError_t e = hipEventRecord(ev, last);
        if (e != hipSuccess) {
            s->spare_events.push_back(ev);
            return hip_fail(e, "hipEventRecord");
        }
    }
    s->released.push_back({p, len, ev, reader});
    if (s->released.size() > 256) reclaim(s);
    return PM_OK;
}

static bool arena_fit(pm_store* s, size_t len, char** out) {
    for (Arena& a : s->arenas)
        for (auto it = a.free.begin(); it != a.free.end(); ++it)
            if (it->second >= len) {
                const size_t off = it->first, rest = it->second - len;
                a.free.erase(it);
                if (rest) a.free.emplace(off + len, rest);
                *out = a.base + off;
                return true;
            }
    return false;
}

// A free range of `bytes` (rounded up to kRangeAlign): first fit, then after
// reclaiming, then from a new arena.
static pm_status arena_alloc(pm_store* s, size_t bytes, char** out) {
    *out = nullptr;
    const size_t len = range_len(bytes);
    if (len == 0) return PM_OK;
    if (arena_fit(s, len, out)) return PM_OK;
    reclaim(s);
    if (arena_fit(s, len, out)) return PM_OK;
    const size_t size = std::max(s->arena_bytes, len);
    char* base = nullptr;
    if (s->host_fake) {
        base = static_cast<char*>(std::calloc(size, 1));
        if (!base) return failf(PM_ERR_OOM, "host allocation of %zu bytes failed", size);
    } else {
        hipError_t e = hipMalloc(&base, size);
        if (e != hipSuccess) {
            // what queued work still holds may be enough once it ends
            (void)hipGetLastError();
            HIP_TRY(hipDeviceSynchronize());
            reclaim(s);
            if (arena_fit(s, len, out)) return PM_OK;
            return failf(PM_ERR_OOM, "device allocation of %zu bytes failed: %s", size,
                         hipGetErrorString(e));
        }
    }
    Arena a{base, size, {}};
    if (size > len) a.free.emplace(len, size - len);
    s->arenas.push_back(std::move(a));
    *out = base;
    return PM_OK;
}

// Take the range right after [p, p + old_len) so that the range spans
// new_len bytes, if it is free.
static bool arena_extend(pm_store* s, char* p, size_t have, size_t want) {
    Arena* a = arena_of(s, p);
    if (!a) return false;
    if (want <= have) return true;
    const size_t end = size_t(p - a->base) + have, need = want - have;
    auto it = a->free.find(end);
    if (it == a->free.end() || it->second < need) return false;
    const size_t rest = it->second - need;
    a->free.erase(it);
    if (rest) a->free.emplace(end + need, rest);
    return true;
}

// Take back ranges given back right after [p, p + *have) while they still
// wait in `released` (most often the slot's own tail, cut by a truncation
// whose readers have not ended), up to `want` bytes: `st` waits for their
// last copy and reader instead of the slot moving.  *have grows by what was
// taken.
static pm_status take_back_tail(pm_store* s, char* p, size_t* have, size_t want, hipStream_t st) {
    if (s->host_fake) return PM_OK;
    for (bool found = true; found && *have < want;) {
        found = false;
        for (size_t i = 0; i < s->released.size(); ++i) {
            Released& r = s->released[i];
            if (r.p != p + *have) continue;
            const size_t take = std::min(r.len, want - *have);
            if (r.ev) HIP_TRY(hipStreamWaitEvent(st, r.ev, 0));
            if (r.reader) {
                const hipEvent_t end = forward_end(s, r.reader);
                if (hipEventQuery(end) != hipSuccess) HIP_TRY(hipStreamWaitEvent(st, end, 0));
            }
            if (take == r.len) {
                if (r.ev) s->spare_events.push_back(r.ev);
                s->released.erase(s->released.begin() + long(i));
            } else {
                r.p += take;
                r.len -= take;
            }
            *have += take;
            found = true;
            break;
        }
    }
    return PM_OK;
}

// Make `st` wait for the last forward that read the slot (unless it has
// finished) and for a copy into the slot still in flight.
static pm_status order_after_readers(pm_store* s, Slot& sl, hipStream_t st) {
    if (s->host_fake) return PM_OK;
    hipEvent_t reader = nullptr;
    if (slot_reader_running(s, sl, &reader)) HIP_TRY(hipStreamWaitEvent(st, reader, 0));
    if (sl.copied) HIP_TRY(hipStreamWaitEvent(st, sl.ready, 0));
    return PM_OK;
}

// The slot's planes become `cap` chunks, keeping its first `keep` valid
// chunks (keep <= both capacities).  Shrinking gives the tail back in place;
// growing extends the range in place if it can, else copies the kept prefix
// to a new range on `st`.  The caller has ordered `st` after the slot's last
// copy; a range given back waits for that stream and for the slot's last
// reader.
static pm_status resize_planes(pm_store* s, Slot& sl, int cap, int keep, hipStream_t st) {
    if (cap == sl.cap) return PM_OK;
    const size_t pb = s->plane_bytes;
    const size_t old_len = size_t(sl.cap) * pb, new_len = size_t(cap) * pb;
    char* p = reinterpret_cast<char*>(sl.planes);
    pm_status r = PM_OK;
    if (cap < sl.cap) {
        const size_t keep_len = cap ? range_len(new_len) : 0;
        r = release_range(s, p + keep_len, range_len(old_len) - keep_len, st, sl.read_seq);
        if (r) return r;
        if (cap == 0) sl.planes = nullptr;
    } else {
        // grow in place (ranges given back right after the slot, then free
        // arena space), else move the kept prefix to a new range
        size_t have = range_len(old_len);
        const size_t want = range_len(new_len);
        if (p) {
            r = take_back_tail(s, p, &have, want, st);
            if (r) return r;
        }
        if (!(p && arena_extend(s, p, have, want))) {
            char* nb = nullptr;
            r = arena_alloc(s, new_len, &nb);
            if (r) return r;
            if (keep > 0) {
                if (s->host_fake)
                    std::memcpy(nb, p, size_t(keep) * pb);
                else
                    HIP_TRY(hipMemcpyAsync(nb, p, size_t(keep) * pb, hipMemcpyDeviceToDevice, st));
            }
            r = release_range(s, p, have, st, sl.read_seq);
            if (r) return r;
            sl.planes = reinterpret_cast<uint32_t*>(nb);
        }
    }
    s->used = s->used - old_len + new_len;
    sl.cap = cap;
    return PM_OK;
}

static pm_status ensure_levels(pm_store* s, Slot& sl) {
    if (sl.levels) return PM_OK;
    char* lv = nullptr;
    pm_status r = arena_alloc(s, s->level_bytes, &lv);
    if (r) return r;
    sl.levels = reinterpret_cast<float*>(lv);
    sl.levels_ready = false;
    s->used += s->level_bytes;
    return PM_OK;
}

// Bytes a slot still needs to hold k planes and its levels.
static size_t bytes_to_hold(const pm_store* s, const Slot& sl, int k) {
    size_t b = k > sl.cap ? size_t(k - sl.cap) * s->plane_bytes : 0;
    if (!sl.levels) b += s->level_bytes;
    return b;
}

static pm_status check_capacity(const pm_store* s, size_t more) {
    if (s->capacity && s->used + more > s->capacity)
        return failf(PM_ERR_OOM, "store capacity %zu bytes exceeded (%zu used, %zu more)",
                     s->capacity, s->used, more);
    return PM_OK;
}

// A slot ready for direct writes by the caller: all 8 chunks and the levels,
// with the memory usable on return (the caller writes it from another stream
// or the host).
static pm_status slot_for_writes(pm_store* s, Slot& sl) {
    if (sl.cap == kBits && sl.levels) return PM_OK;
    pm_status r = check_capacity(s, bytes_to_hold(s, sl, kBits));
    if (r) return r;
    hipStream_t st = s->side[pm_store::kMem];
    if (!s->host_fake && sl.copied) HIP_TRY(hipStreamWaitEvent(st, sl.ready, 0));
    r = ensure_levels(s, sl);
    if (r) return r;
    r = resize_planes(s, sl, kBits, sl.resident, st);
    if (r) return r;
    if (!s->host_fake) {
        HIP_TRY(hipStreamSynchronize(st));
        sl.pending = false;
    }
    return PM_OK;
}

extern "C" pm_status pm_store_create(pm_expert_shape e, int n_layers, int n_experts,
                                     size_t capacity, uint32_t flags, pm_store** out) {
    if (!out) return failf(PM_ERR_ARG, "null output pointer");
    *out = nullptr;
    if (!expert_ok(e)) return failf(PM_ERR_SHAPE, "invalid expert shape");
    if (n_layers < 1 || n_experts < 1) return failf(PM_ERR_ARG, "empty store");
    if (flags & ~uint32_t(PM_STORE_HOST_FAKE)) return failf(PM_ERR_ARG, "unknown store flags");
    pm_store* s = new pm_store();
    s->shape = e;
    s->geom = make_geom(e);
    s->n_layers = n_layers;
    s->n_experts = n_experts;
    s->capacity = capacity;
    s->host_fake = flags & PM_STORE_HOST_FAKE;
    s->plane_bytes = pm_expert_plane_words(e) * sizeof(uint32_t);
    s->level_bytes = pm_expert_levels_floats(e) * sizeof(float);
    s->slots.resize(size_t(n_layers) * n_experts);
    s->item_of.assign(size_t(n_experts), -1);
    // arenas of about eight whole experts (within 64 MiB .. 2 GiB), no larger
    // than a capacity the store is given
    {
        const size_t expert_bytes = kBits * s->plane_bytes + s->level_bytes;
        size_t ab = std::min(std::max(8 * expert_bytes, size_t(64) << 20), size_t(2) << 30);
        if (capacity) ab = std::min(ab, std::max(capacity, expert_bytes));
        s->arena_bytes = ab;
    }
    if (!s->host_fake) {
        hipError_t er = hipSuccess;
        for (int i = 0; i < pm_store::kSides && er == hipSuccess; ++i)
            er = hipStreamCreateWithFlags(&s->side[i], hipStreamNonBlocking);
        for (int i = 0; i < pm_store::kDone && er == hipSuccess; ++i)
            er = hipEventCreateWithFlags(&s->done[i], hipEventDisableTiming);
        if (er != hipSuccess) {
            pm_store_destroy(s);
            return hip_fail(er, "store stream/event creation");
        }
    }
    *out = s;
    return PM_OK;
}

extern "C" pm_status pm_store_destroy(pm_store* s) {
    if (!s) return PM_OK;
    if (!s->host_fake) (void)hipDeviceSynchronize();
    for (Slot& sl : s->slots)
        if (sl.ready) (void)hipEventDestroy(sl.ready);
    for (const Released& r : s->released)
        if (r.ev) (void)hipEventDestroy(r.ev);
    for (hipEvent_t ev : s->spare_events) (void)hipEventDestroy(ev);
    for (Arena& a : s->arenas) {
        if (s->host_fake)
            std::free(a.base);
        else
            (void)hipFree(a.base);
    }
    if (!s->host_fake) {
        Workspace& w = s->ws;
        if (w.d_buf) (void)hipFree(w.d_buf);
        if (w.d_ring) (void)hipFree(w.d_ring);
        if (w.h_ring) (void)hipHostFree(w.h_ring);
        for (hipEvent_t ev : w.ring_ev)
            if (ev) (void)hipEventDestroy(ev);
        for (hipEvent_t ev : s->done)
            if (ev) (void)hipEventDestroy(ev);
        for (hipStream_t st : s->side)
            if (st) (void)hipStreamDestroy(st);
    }
    delete s;
    return PM_OK;
}

extern "C" pm_status pm_store_slot(pm_store* s, int layer, int expert, uint32_t** planes,
                                   float** levels) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    st = slot_for_writes(s, s->slots[i]);
    if (st) return st;
    if (planes) *planes = s->slots[i].planes;
    if (levels) *levels = s->slots[i].levels;
    return PM_OK;
}

extern "C" pm_status pm_store_set_resident(pm_store* s, int layer, int expert, int r) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    if (r < 0 || r > kBits) return failf(PM_ERR_PREFIX, "resident prefix %d outside 0..8", r);
    if (s->slots[i].cap < r || !s->slots[i].levels)
        return failf(PM_ERR_STATE, "slot (%d, %d) holds %d plane chunks, %d declared", layer,
                     expert, s->slots[i].cap, r);
    s->slots[i].resident = r;
    s->slots[i].levels_ready = true;
    s->slots[i].pending = false;
    return PM_OK;
}

extern "C" pm_status pm_store_attach_host(pm_store* s, int layer, int expert,
                                          const uint32_t* h_planes, const float* h_levels) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    if (!h_planes || !h_levels) return failf(PM_ERR_ARG, "null host source");
    s->slots[i].h_planes = h_planes;
    s->slots[i].h_levels = h_levels;
    s->has_sources = true;
    return PM_OK;
}

// The event that marks the end of forward n (1 <= n <= fwd_seq) or of a later
// forward: its own entry, else the earliest recorded end after it, else an
// end recorded now on the last forward's stream.
static hipEvent_t forward_end(pm_store* s, uint64_t n) {
    const int e = int(n % pm_store::kDone);
    if (s->done_seq[e] == n) return s->done[e];
    if (s->recorded_seq >= n) {
        // the earliest recorded end after n: waiting on a later one would
        // also wait for every forward queued since
        int best = -1;
        for (int i = 0; i < pm_store::kDone; ++i)
            if (s->done_seq[i] >= n && (best < 0 || s->done_seq[i] < s->done_seq[best])) best = i;
        return s->done[best];
    }
    const int f = int(s->fwd_seq % pm_store::kDone);
    if (hipEventRecord(s->done[f], s->last_compute) == hipSuccess) {
        s->done_seq[f] = s->fwd_seq;
        s->recorded_seq = s->fwd_seq;
    }
    return s->done[f];
}

// Whether the last forward that read the slot may still run; *ev is the event
// that marks its end (or a later forward's).
static bool slot_reader_running(pm_store* s, const Slot& sl, hipEvent_t* ev) {
    if (sl.read_seq == 0) return false;
    *ev = forward_end(s, sl.read_seq);
    return hipEventQuery(*ev) != hipSuccess;
}

static pm_status slot_event(pm_store* s, Slot& sl) {
    if (!s->host_fake && !sl.ready) HIP_TRY(hipEventCreateWithFlags(&sl.ready, hipEventDisableTiming));
    return PM_OK;
}

static pm_status topup_slot(pm_store* s, Slot& sl, int k, hipStream_t side) {
    if (k <= sl.resident) {            // a resident deeper prefix serves it: no copy
        s->last_first = sl.resident;
        s->last_count = 0;
        return PM_OK;
    }
    if (!sl.h_planes || !sl.h_levels) return failf(PM_ERR_STATE, "slot has no host source");
    pm_status st = check_capacity(s, bytes_to_hold(s, sl, k));
    if (st) return st;
    st = slot_event(s, sl);
    if (st) return st;
    st = ensure_levels(s, sl);
    if (st) return st;
    // The copy must not overwrite planes a forward may still read (those
    // past a resident prefix that was lowered below the chunks held), and it
    // follows any earlier copy into the slot on another stream.
    if (k <= sl.cap || sl.resident < sl.cap) {
        st = order_after_readers(s, sl, side);
        if (st) return st;
    } else if (!s->host_fake && sl.copied) {
        HIP_TRY(hipStreamWaitEvent(side, sl.ready, 0));
    }
    if (k > sl.cap) {
        st = resize_planes(s, sl, k, sl.resident, side);
        if (st) return st;
    }
    const int first = sl.resident;
    const size_t pw = s->plane_bytes / sizeof(uint32_t);
    if (s->host_fake) {
        if (!sl.levels_ready) std::memcpy(sl.levels, sl.h_levels, s->level_bytes);
        std::memcpy(sl.planes + size_t(first) * pw, sl.h_planes + size_t(first) * pw,
                    size_t(k - first) * s->plane_bytes);
    } else {
        if (!sl.levels_ready)
            HIP_TRY(hipMemcpyAsync(sl.levels, sl.h_levels, s->level_bytes,
                                   hipMemcpyHostToDevice, side));
        HIP_TRY(hipMemcpyAsync(sl.planes + size_t(first) * pw, sl.h_planes + size_t(first) * pw,
                               size_t(k - first) * s->plane_bytes, hipMemcpyHostToDevice, side));
        HIP_TRY(hipEventRecord(sl.ready, side));
        sl.copied = true;
        sl.pending = true;
    }
    if (!sl.levels_ready) s->total_bytes += s->level_bytes;
    sl.levels_ready = true;
    sl.resident = k;
    s->last_first = first;
    s->last_count = k - first;
    s->total_planes += uint64_t(k - first);
    s->total_bytes += uint64_t(k - first) * s->plane_bytes;
    return PM_OK;
}

// Top-ups of the short slots of one forward (slot i to prefix k[i]): copies
// that need no wait first, spread over the store's first side streams, then
// those that wait for an earlier forward's reads, on the last side stream.
static pm_status issue_topups(pm_store* s, const std::vector<Slot*>& slots,
                              const std::vector<int>& k) {
    constexpr int n_free = pm_store::kWaits - 1;
    // whether each in-place copy must wait for the slot's last reader, asked
    // once: the answer can change between the two passes, and a slot must be
    // in exactly one (a copy into a new buffer never waits for a reader)
    std::vector<char> waits(slots.size());
    for (size_t i = 0; i < slots.size(); ++i) {
        hipEvent_t ev = nullptr;
        waits[i] = k[i] <= slots[i]->cap && slot_reader_running(s, *slots[i], &ev);
    }
    for (int pass = 0; pass < 2; ++pass) {
        for (size_t i = 0; i < slots.size(); ++i) {
            if (bool(waits[i]) != (pass == 1)) continue;
            hipStream_t st = waits[i] ? s->side[pm_store::kWaits]
                                      : s->side[1 + s->next_side++ % n_free];
            const pm_status r = topup_slot(s, *slots[i], k[i], st);
            if (r) return r;
        }
    }
    for (size_t i = 0; i < slots.size(); ++i)
        if (slots[i]->resident < k[i])
            return failf(PM_ERR_STATE, "top-up left a slot at %d planes, %d needed",
                         slots[i]->resident, k[i]);
    return PM_OK;
}

extern "C" pm_status pm_store_topup(pm_store* s, int layer, int expert, int k, void* side) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    st = check_k(k);
    if (st) return st;
    return topup_slot(s, s->slots[i], k, side ? (hipStream_t)side : s->side[1]);
}

extern "C" pm_status pm_store_truncate(pm_store* s, int layer, int expert, int keep) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    if (keep < 0 || keep > kBits) return failf(PM_ERR_PREFIX, "keep %d outside 0..8", keep);
    Slot& sl = s->slots[i];
    sl.resident = std::min(sl.resident, keep);
    // the plane chunks past `keep` (and at keep 0 the levels) go back to the
    // store's arenas in place, once the slot's last copy and last reader
    // have ended
    if (keep >= sl.cap && (keep > 0 || !sl.levels)) return PM_OK;
    hipStream_t mem = s->host_fake ? nullptr : s->side[pm_store::kMem];
    if (mem && sl.copied) HIP_TRY(hipStreamWaitEvent(mem, sl.ready, 0));
    st = resize_planes(s, sl, std::min(sl.cap, keep), sl.resident, mem);
    if (st) return st;
    if (keep == 0 && sl.levels) {
        st = release_range(s, reinterpret_cast<char*>(sl.levels), range_len(s->level_bytes), mem,
                           sl.read_seq);
        if (st) return st;
        sl.levels = nullptr;
        sl.levels_ready = false;
        s->used -= s->level_bytes;
    }
    return PM_OK;
}

extern "C" pm_status pm_store_slot_info(const pm_store* s, int layer, int expert,
                                       const uint32_t** planes, const float** levels,
                                       int* chunks) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    const Slot& sl = s->slots[i];
    if (planes) *planes = sl.planes;
    if (levels) *levels = sl.levels;
    if (chunks) *chunks = sl.cap;
    return PM_OK;
}

extern "C" pm_status pm_store_usage(const pm_store* s, size_t* used_bytes, size_t* plane_chunks,
                                    size_t* level_sets) {
    if (!s) return failf(PM_ERR_ARG, "null store");
    size_t chunks = 0, sets = 0;
    for (const Slot& sl : s->slots) {
        chunks += size_t(sl.cap);
        sets += sl.levels ? 1 : 0;
    }
    if (used_bytes) *used_bytes = s->used;
    if (plane_chunks) *plane_chunks = chunks;
    if (level_sets) *level_sets = sets;
    return PM_OK;
}

extern "C" pm_status pm_store_resident(const pm_store* s, int layer, int expert, int* r_out) {
    size_t i;
    pm_status st = slot_of(s, layer, expert, &i);
    if (st) return st;
    if (!r_out) return failf(PM_ERR_ARG, "null output pointer");
    *r_out = s->slots[i].resident;
    return PM_OK;
}

extern "C" pm_status pm_store_copy_stats(const pm_store* s, int* last_first, int* last_count,
                                         uint64_t* total_planes, uint64_t* total_bytes) {
    if (!s) return failf(PM_ERR_ARG, "null store");
    if (last_first) *last_first = s->last_first;
    if (last_count) *last_count = s->last_count;
    if (total_planes) *total_planes = s->total_planes;
    if (total_bytes) *total_bytes = s->total_bytes;
    return PM_OK;
}

extern "C" pm_status pm_store_set_profile_events(pm_store* s, void* const* events, int n) {
    if (!s) return failf(PM_ERR_ARG, "null store");
    if (n == 0) {
        s->profiling = false;
        return PM_OK;
    }
    if ((n != 2 && n < 4) || !events) return failf(PM_ERR_ARG, "need 2 or 4 events");
    s->n_prof = n >= 4 ? 4 : 2;
    for (int i = 0; i < s->n_prof; ++i) s->prof[i] = (hipEvent_t)events[i];
    s->profiling = true;
    return PM_OK;
}

// ---- LUT path: launch descriptions travel as kernel arguments.
// Target number of LUT workgroups per launch: one per compute unit (each
// holds its 128 KiB activation table in LDS).
static int lut_wg_target() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus > 0)
            n = cus;
        else
            n = 256;
    }
    return n;
}

namespace {
struct JobSpec {                       // a LUT job before it is packed into a launch
    KJob job;
};
}  // namespace

// Workgroups of a launch whose jobs come in runs of one source (one
// activation table) and one prefix: every run gets whole workgroups (largest
// remainder, at least one each), and no workgroup spans two runs, so a
// workgroup builds its table once and runs one prefix's code throughout.
// Each workgroup takes an even share of its run's 8-row steps (the kernel
// works it out from the run's description).
// The shares balance the modelled workgroup time, fixed part plus steps:
// run r with C_r ns of steps at fixed part A_r gets C_r / (T - A_r)
// workgroups, T chosen so that the shares add up to the workgroups there are.
static void split_runs(KLaunch& L, int n_total) {
    const int n = L.n_jobs;
    int r0[kMaxLaunchJobs + 1];                // first job of every run
    int R = 0;
    for (int j = 0; j < n; ++j)
        if (j == 0 || L.job[j].src != L.job[j - 1].src || L.job[j].k != L.job[j - 1].k)
            r0[R++] = j;
    r0[R] = n;
    n_total = std::min(kMaxLaunchWgq, std::max(n_total, R));
    double cost[kMaxLaunchJobs], fixed[kMaxLaunchJobs], share[kMaxLaunchJobs];
    double C = 0, Amax = 0;
    const bool down = L.gu != nullptr;
    for (int r = 0; r < R; ++r) {
        const int k = L.job[r0[r]].k;         // one prefix per run
        cost[r] = double(r0[r + 1] - r0[r]) * double(L.rows / kLutRows) *
                  double(lut_step_ns(k, down));
        fixed[r] = double(lut_fixed_ns(k, down));
        C += cost[r];
        Amax = std::max(Amax, fixed[r]);
    }
    if (C > 0) {
        // f(T) = sum_r cost_r / (T - fixed_r) - n_total is convex and falls
        // from +inf just above Amax.  Newton steps from a point left of the
        // root (where a run at Amax alone wants 2 n_total workgroups) stay
        // left of it and converge from there.
        double cmax = 0;
        for (int r = 0; r < R; ++r)
            if (fixed[r] == Amax) cmax = std::max(cmax, cost[r]);
        double T = Amax + cmax / (2.0 * n_total);
        for (int it = 0; it < 100; ++it) {
            double f = -double(n_total), df = 0;
            for (int r = 0; r < R; ++r) {
                const double d = 1.0 / (T - fixed[r]);
                f += cost[r] * d;
                df -= cost[r] * d * d;
            }
            const double step = -f / df;
            T += step;
            if (!(step > 1e-9 * T)) break;
        }
        for (int r = 0; r < R; ++r) share[r] = cost[r] / (T - fixed[r]);
    } else {
        for (int r = 0; r < R; ++r) share[r] = double(n_total) / R;
    }
    int a[kMaxLaunchJobs];
    int sum = 0;
    for (int r = 0; r < R; ++r) {
        a[r] = std::max(1, int(share[r]));
        sum += a[r];
    }
    while (sum > n_total) {
        int b = 0;
        for (int r = 1; r < R; ++r)
            if (a[r] > a[b]) b = r;
        if (a[b] <= 1) break;
        --a[b];
        --sum;
    }
    while (sum < n_total) {
        int b = 0;
        for (int r = 1; r < R; ++r)
            if (share[r] - a[r] > share[b] - a[b]) b = r;
        ++a[b];
        ++sum;
    }
    int w = 0;
    for (int r = 0; r < R; ++r) {
        const KJob& jb = L.job[r0[r]];
        KRun& run = L.run[r];
        run.g0 = r0[r] * L.rows;
        run.nsteps = (r0[r + 1] - r0[r]) * (L.rows / kLutRows);
        run.wg0 = int16_t(w);
        run.nwg = int16_t(a[r]);
        run.meta = uint32_t(uint16_t(jb.src)) | (uint32_t(jb.k) << 16) | (uint32_t(jb.gsl) << 24);
        const uint32_t info = uint32_t(r) | (uint32_t(uint16_t(jb.src)) << 8) |
                              (uint32_t(jb.gsl) << 24);
        for (int q = w; q < w + a[r]; ++q) L.wg_info[q] = info;
        w += a[r];
    }
    L.n_wgq = w;
}

// Jobs of one token share an activation table, and a workgroup runs one
// prefix: order a stage's jobs by (source, prefix), stably.  Insertion sort
// for the short lists of a call (no allocation), std::stable_sort beyond.
static void sort_jobs(std::vector<JobSpec>& js) {
    auto less = [](const JobSpec& a, const JobSpec& b) {
        return a.job.src != b.job.src ? a.job.src < b.job.src : a.job.k < b.job.k;
    };
    if (js.size() > 64) {
        std::stable_sort(js.begin(), js.end(), less);
        return;
    }
    for (size_t i = 1; i < js.size(); ++i) {
        const JobSpec v = js[i];
        size_t j = i;
        for (; j > 0 && less(v, js[j - 1]); --j) js[j] = js[j - 1];
        js[j] = v;
    }
}

// Pack jobs into launches of at most kMaxLaunchJobs, cut by source
// (split_runs); jobs of one source should be adjacent.
static void pack_launches(const std::vector<JobSpec>& js, const KLaunch& proto,
                          std::vector<KLaunch>& out) {
    // the launches of one stage run one after another: each takes the whole
    // target (one workgroup per compute unit)
    const int n = std::max(1, std::min(kMaxLaunchWgq, lut_wg_target() / proto.S));
    for (size_t j0 = 0; j0 < js.size(); j0 += kMaxLaunchJobs) {
        const size_t j1 = std::min(js.size(), j0 + kMaxLaunchJobs);
        out.push_back(proto);
        KLaunch& L = out.back();
        L.n_jobs = int(j1 - j0);
        for (size_t j = j0; j < j1; ++j) L.job[j - j0] = js[j].job;
        split_runs(L, n);
    }
}

// Per-stream partial-sum buffers of pm_expert_gemv's LUT path.
namespace {
struct StreamBuf {
    float* p = nullptr;
    size_t n = 0;
};
// Never destroyed: no destructor of this library runs at process exit.
std::mutex g_gemv_mu;
std::map<hipStream_t, StreamBuf>& g_gemv_bufs = *new std::map<hipStream_t, StreamBuf>();
}  // namespace

static pm_status gemv_partials(hipStream_t st, size_t n, float** out) {
    std::lock_guard<std::mutex> lk(g_gemv_mu);
    StreamBuf& b = g_gemv_bufs[st];
    if (b.n < n) {
        if (b.p) {
            HIP_TRY(hipStreamSynchronize(st));
            HIP_TRY(hipFree(b.p));
            b.p = nullptr;
            b.n = 0;
        }
        hipError_t e = hipMalloc(&b.p, n * sizeof(float));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return failf(PM_ERR_OOM, "GEMV workspace allocation failed: %s", hipGetErrorString(e));
        }
        b.n = n;
    }
    *out = b.p;
    return PM_OK;
}

pm_status gemv_lut(pm_matrix_shape s, int k, const uint32_t* d_planes, size_t pstride,
                   const float* d_levels, const float* d_x, float* d_y, hipStream_t st,
                   float* partials) {
    const int S = s.cols / kSliceCols;
    const size_t nb = size_t(s.rows) * (s.cols / s.group);
    KLaunch L{};
    L.x = d_x;
    L.pstride = pstride;
    L.S = S;
    L.rows = s.rows;
    L.W = s.cols / 32;
    L.wpg = s.group / 32;
    L.out_stride = s.rows;
    L.x_stride = 0;
    L.n_jobs = 1;
    KJob& jb = L.job[0];
    jb.planes = d_planes;
    jb.lvk = d_levels + level_offset(nb, k);
    jb.k = int8_t(k);
    jb.src = 0;
    if (S == 1) {
        jb.out = d_y;
    } else if (partials) {
        jb.out = partials;
    } else {
        pm_status r = gemv_partials(st, size_t(S) * s.rows, &jb.out);
        if (r) return r;
    }
    // workgroups per slice: enough to fill the device, at least 32 rows each
    const int target = std::max(1, std::min(kMaxLaunchWgq, lut_wg_target() / S));
    split_runs(L, std::max(1, std::min(target, (s.rows + 31) / 32)));
    HIP_TRY(launch_lut(L, false, st));
    if (S > 1) HIP_TRY(launch_sum_slices(jb.out, S, s.rows, d_y, st));
    return PM_OK;
}

// ---------------------------------------------------------------- MoE forward
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static pm_status ensure_workspace(pm_store* s, size_t floats, size_t list_bytes) {
    Workspace& w = s->ws;
    if (floats > w.d_floats) {
        if (w.d_buf) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(hipFree(w.d_buf));
            w.d_buf = nullptr;
        }
        size_t n = std::max(floats, size_t(1) << 20);
        hipError_t e = hipMalloc(&w.d_buf, n * sizeof(float));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return failf(PM_ERR_OOM, "workspace allocation failed: %s", hipGetErrorString(e));
        }
        w.d_floats = n;
    }
    if (list_bytes > w.slot_bytes) {
        if (w.h_ring) {
            HIP_TRY(hipDeviceSynchronize());
            HIP_TRY(hipHostFree(w.h_ring));
            HIP_TRY(hipFree(w.d_ring));
            w.h_ring = nullptr;
            w.d_ring = nullptr;
        }
        size_t sb = std::max(align256(list_bytes), size_t(64) << 10);
        HIP_TRY(hipHostMalloc(&w.h_ring, sb * Workspace::kSlots, 0));
        HIP_TRY(hipMalloc(&w.d_ring, sb * Workspace::kSlots));
        for (hipEvent_t& ev : w.ring_ev)
            if (!ev) HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
        w.slot_bytes = sb;
    }
    return PM_OK;
}

// The end of a forward: its sequence number, its stream, the event a later
// top-up may wait on (only when top-ups are possible) and the slots it read.
static pm_status finish_forward(pm_store* s, hipStream_t compute, const std::vector<Slot*>& read) {
    const uint64_t seq = ++s->fwd_seq;
    s->last_compute = compute;
    if (s->has_sources) {
        HIP_TRY(hipEventRecord(s->done[seq % pm_store::kDone], compute));
        s->done_seq[seq % pm_store::kDone] = seq;
        s->recorded_seq = seq;
    }
    for (Slot* sl : read) sl->read_seq = seq;
    return PM_OK;
}

// ---------------------------------------------------------------- batched forward, matrix cores
#ifndef PM_TILE_MIN_USES
#define PM_TILE_MIN_USES 6
#endif
// In the default forward the uses that read one matrix of one expert at one
// prefix go to the matrix cores from this many on (fewer: a LUT job each, or
// the direct kernels)
constexpr int kTileMinUses = PM_TILE_MIN_USES;

// The uses of one item (expert) of a forward call: a range of a flat list.
struct UseList {
    const int* b;
    int n;
    const int* begin() const { return b; }
    const int* end() const { return b + n; }
    size_t size() const { return size_t(n); }
};

// The matrix-core tiles of one expert (slot) for matrices m0..m1-1: per
// prefix k, the uses that read matrix m at k, 16 at a time, when at least
// min_uses of them do.  Their (use, matrix) is marked 2 (tile, one slice).
static void add_tiles(std::vector<Use>& uses, const UseList& item_uses,
                      const Slot& sl, const Geom& g, int m0, int m1, int min_uses,
                      std::vector<MTile> (&out)[kBits + 1]) {
    const size_t nb_gu = size_t(g.inter) * (g.hidden / g.group);
    const size_t nb_dn = size_t(g.hidden) * (g.inter / g.group);
    for (int m = m0; m < m1; ++m) {
        for (int k = 1; k <= kBits; ++k) {
            int count = 0;
            for (int u : item_uses) count += uses[u].k[m] == k;
            if (count == 0 || count < min_uses) continue;
            MTile t{};
            t.planes = sl.planes + g.plane_off[m];
            t.lvk = sl.levels + g.level_off[m] + level_offset(m < 2 ? nb_gu : nb_dn, k);
            t.m = m;
            for (int u : item_uses) {
                if (uses[u].k[m] != k) continue;
                uses[u].direct[m] = 2;
                uses[u].slices[m] = 1;
                t.use[t.n++] = u;
                if (t.n == kMfmaTileUses) {
                    out[k].push_back(t);
                    t.n = 0;
                }
            }
            if (t.n) out[k].push_back(t);
        }
    }
}

static pm_status launch_tiles(MLaunch L, const MTile* d_tiles, const size_t* off,
                              const std::vector<MTile> (&tiles)[kBits + 1], hipStream_t st) {
    for (int k = 1; k <= kBits; ++k) {
        L.tiles = d_tiles + off[k];
        L.n_tiles = int(tiles[k].size());
        L.k = k;
        HIP_TRY(launch_mfma(L, st));
    }
    return PM_OK;
}
// Uses that read one matrix of one expert at one prefix k form tiles of up to
// 16 (mfma_kernel); one launch per stage and k, then SwiGLU and the combine
// over all tokens.  Every use keeps its own prefix.
static pm_status forward_mfma(pm_store* s, int layer, int n_tokens, int top_k,
                              std::vector<Use>& uses, const std::vector<int>& item_expert,
                              const std::vector<UseList>& item_uses,
                              const std::vector<int>& kneed, const std::vector<char>& late,
                              const float* d_x, float* d_y, hipStream_t compute) {
    const Geom& g = s->geom;
    const int n_uses = n_tokens * top_k, n_items = int(item_expert.size());
    std::vector<Slot*> slot(n_items);
    for (int d = 0; d < n_items; ++d)
        slot[d] = &s->slots[size_t(layer) * s->n_experts + item_expert[d]];
    for (Use& us : uses)
        for (int m = 0; m < 3; ++m) {
            us.direct[m] = 1;
            us.slices[m] = 1;
        }
    // tiles of every stage (0 gate/up, 1 down) and prefix
    std::vector<MTile> tiles[2][kBits + 1];
    for (int d = 0; d < n_items; ++d) {
        add_tiles(uses, item_uses[d], *slot[d], g, 0, 2, 1, tiles[0]);
        add_tiles(uses, item_uses[d], *slot[d], g, 2, 3, 1, tiles[1]);
    }
    size_t n_tiles = 0;
    for (auto& st2 : tiles)
        for (auto& v : st2) n_tiles += v.size();
    const size_t fGU = align256(size_t(n_uses) * 2 * g.inter);
    const size_t fH = align256(size_t(n_uses) * g.inter);
    const size_t fY = align256(size_t(n_uses) * g.hidden);
    const size_t o_tiles = align256(sizeof(Use) * n_uses);
    const size_t list_bytes = o_tiles + align256(sizeof(MTile) * n_tiles);
    pm_status st = ensure_workspace(s, fGU + fH + fY, list_bytes);
    if (st) return st;
    Partials P{};
    P.gu = s->ws.d_buf;
    P.h = s->ws.d_buf + fGU;
    P.y = s->ws.d_buf + fGU + fH;
    P.gu_smax = 1;
    P.dn_smax = 1;

    // uses and tiles through the pinned ring
    Workspace& w = s->ws;
    const int rs = w.next;
    w.next = (w.next + 1) % Workspace::kSlots;
    HIP_TRY(hipEventSynchronize(w.ring_ev[rs]));
    char* hb = w.h_ring + size_t(rs) * w.slot_bytes;
    char* db = w.d_ring + size_t(rs) * w.slot_bytes;
    std::memcpy(hb, uses.data(), sizeof(Use) * n_uses);
    size_t off[2][kBits + 1], pos = 0;
    for (int stage = 0; stage < 2; ++stage)
        for (int k = 1; k <= kBits; ++k) {
            off[stage][k] = pos;
            if (!tiles[stage][k].empty())
                std::memcpy(hb + o_tiles + pos * sizeof(MTile), tiles[stage][k].data(),
                            sizeof(MTile) * tiles[stage][k].size());
            pos += tiles[stage][k].size();
        }
    HIP_TRY(hipMemcpyAsync(db, hb, list_bytes, hipMemcpyHostToDevice, compute));
    HIP_TRY(hipEventRecord(w.ring_ev[rs], compute));
    const Use* duses = reinterpret_cast<const Use*>(db);
    const MTile* dtiles = reinterpret_cast<const MTile*>(db + o_tiles);
    for (int d = 0; d < n_items; ++d) {
        if (slot[d]->pending) {
            HIP_TRY(hipStreamWaitEvent(compute, slot[d]->ready, 0));
            slot[d]->pending = false;
        }
    }

    MLaunch L{};
    L.uses = duses;
    L.x = d_x;
    L.P = P;
    L.pstride = g.plane_words;
    for (int stage = 0; stage < 2; ++stage) {
        L.rows = stage == 0 ? g.inter : g.hidden;
        L.cols = stage == 0 ? g.hidden : g.inter;
        L.down = stage;
        st = launch_tiles(L, dtiles, off[stage], tiles[stage], compute);
        if (st) return st;
        if (stage == 0) HIP_TRY(launch_swiglu(duses, n_uses, P, g.inter, compute));
    }
    HIP_TRY(launch_combine(n_tokens, top_k, g.hidden, duses, P, d_y, compute));
    return finish_forward(s, compute, slot);
}

extern "C" pm_status pm_moe_token_forward(pm_store* s, int layer, int n_tokens, int top_k,
                                          const int32_t* h_ids, const float* h_w,
                                          const uint8_t* h_k, const float* d_x, float* d_y,
                                          void* compute_v, uint32_t flags) {
    if (!s) return failf(PM_ERR_ARG, "null store");
    if (flags & ~uint32_t(PM_AUTO_TOPUP | PM_BATCH_MFMA | PM_READ_ONCE | PM_DETERMINISTIC))
        return failf(PM_ERR_ARG, "unknown forward flags");
    const bool mfma = flags & PM_BATCH_MFMA;
    const bool read_once = flags & PM_READ_ONCE;
    if (layer < 0 || layer >= s->n_layers) return failf(PM_ERR_ARG, "layer %d outside store", layer);
    if (n_tokens < 0 || top_k < 1) return failf(PM_ERR_ARG, "n_tokens=%d top_k=%d", n_tokens, top_k);
    if (n_tokens == 0) return PM_OK;
    if (!h_ids || !h_w || !h_k || !d_x || !d_y) return failf(PM_ERR_ARG, "null pointer");
    if (reinterpret_cast<uintptr_t>(d_x) % 16) return failf(PM_ERR_ARG, "x not 16-byte aligned");
    if (top_k > kMaxLaunchUses)
        return failf(PM_ERR_ARG, "top_k=%d above %d", top_k, kMaxLaunchUses);
    hipStream_t compute = (hipStream_t)compute_v;
    const Geom& g = s->geom;
    if (mfma && (g.group != kMfmaGroup || g.hidden % kMfmaGroup || g.inter % kMfmaGroup))
        return failf(PM_ERR_SHAPE, "the matrix-core path needs group %d and hidden, inter "
                     "multiples of %d", kMfmaGroup, kMfmaGroup);

    // ---- validate and group uses by expert (order of first appearance)
    if (int64_t(n_tokens) * top_k > kMaxCallUses)
        return failf(PM_ERR_ARG, "%d tokens x top-%d: more than %d uses in one call", n_tokens,
                     top_k, kMaxCallUses);
    const int n_uses = n_tokens * top_k;
    std::vector<Use> uses(n_uses);
    for (int t = 0; t < n_tokens; ++t) {
        for (int j = 0; j < top_k; ++j) {
            const int u = t * top_k + j;
            const int e = h_ids[u];
            if (e < 0 || e >= s->n_experts)
                return failf(PM_ERR_ARG, "ids[%d][%d]=%d outside 0..%d", t, j, e, s->n_experts - 1);
            if (!std::isfinite(h_w[u])) return failf(PM_ERR_ARG, "w[%d][%d] not finite", t, j);
            Use& us = uses[u];
            for (int m = 0; m < 3; ++m) {
                const int k = h_k[size_t(u) * 3 + m];
                if (k < 1 || k > kBits)
                    return failf(PM_ERR_PREFIX, "k[%d][%d][%d]=%d outside 1..8", t, j, m, k);
                us.k[m] = k;
            }
            us.w = h_w[u];
            us.tok = t;
            us.slot = j;
        }
    }
    // items in order of first appearance, each with its uses in call order
    // (a counting sort through the store's expert -> item map, which is all
    // -1 between calls)
    std::vector<int> item_expert;
    item_expert.reserve(std::min(n_uses, s->n_experts));
    std::vector<int> use_item(n_uses), list_off(1, 0);
    for (int u = 0; u < n_uses; ++u) {
        int& d = s->item_of[h_ids[u]];
        if (d < 0) {
            d = int(item_expert.size());
            item_expert.push_back(h_ids[u]);
            list_off.push_back(0);
        }
        use_item[u] = d;
        ++list_off[d + 1];
    }
    for (int e : item_expert) s->item_of[e] = -1;
    for (size_t d = 1; d < list_off.size(); ++d) list_off[d] += list_off[d - 1];
    std::vector<int> use_list(n_uses);
    {
        std::vector<int> fill(list_off.begin(), list_off.end() - 1);
        for (int u = 0; u < n_uses; ++u) use_list[fill[use_item[u]]++] = u;
    }
    std::vector<UseList> item_uses(item_expert.size());
    for (size_t d = 0; d < item_expert.size(); ++d)
        item_uses[d] = UseList{use_list.data() + list_off[d], list_off[d + 1] - list_off[d]};
    const int n_items = int(item_expert.size());
    std::vector<int> kneed(n_items, 0);
    std::vector<std::array<int, 3>> kmax(n_items, {0, 0, 0});
    for (int d = 0; d < n_items; ++d) {
        for (int u : item_uses[d])
            for (int m = 0; m < 3; ++m) kmax[d][m] = std::max(kmax[d][m], uses[u].k[m]);
        kneed[d] = std::max(kmax[d][0], std::max(kmax[d][1], kmax[d][2]));
    }
    // ---- residency: every short slot must be topped up (or the call fails).
    // Every item is checked, and the memory of all new slots counted against
    // the capacity, before any slot is allocated: a failing call leaves the
    // store as it was.
    std::vector<char> late(n_items, 0);
    size_t new_bytes = 0;
    for (int d = 0; d < n_items; ++d) {
        Slot& sl = s->slots[size_t(layer) * s->n_experts + item_expert[d]];
        const bool ok = sl.levels_ready && sl.resident >= kneed[d];
        if (!ok) {
            if (!(flags & PM_AUTO_TOPUP))
                return failf(PM_ERR_NOT_RESIDENT,
                            "expert (%d, %d) holds %d planes, %d requested", layer,
                            item_expert[d], sl.resident, kneed[d]);
            if (!sl.h_planes || !sl.h_levels)
                return failf(PM_ERR_STATE, "expert (%d, %d) is short and has no host source",
                            layer, item_expert[d]);
            new_bytes += bytes_to_hold(s, sl, kneed[d]);
            late[d] = 1;
        }
    }
    {
        pm_status st = check_capacity(s, new_bytes);
        if (st) return st;
    }
    if (s->host_fake) return failf(PM_ERR_STATE, "a host-backed store cannot compute");
    // resident items first so their kernels can run while top-ups copy
    std::vector<int> order(n_items);
    for (int d = 0; d < n_items; ++d) order[d] = d;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return late[a] < late[b]; });

    // Under stream capture (a HIP graph) a call may only hold LUT jobs on
    // resident slots: a top-up, or a work list uploaded for the direct
    // kernels or the tiles, would be recorded as a copy of host memory that
    // later calls rewrite.  The test is conservative (an item of 6 or more
    // uses might form tiles) and runs before any stream operation.
    if (compute) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        HIP_TRY(hipStreamIsCapturing(compute, &cs));
        if (cs != hipStreamCaptureStatusNone) {
            const bool tile_shape = g.group == kMfmaGroup && g.hidden % kMfmaGroup == 0 &&
                                    g.inter % kMfmaGroup == 0;
            const pm_matrix_shape ms[2] = {{g.inter, g.hidden, g.group},
                                           {g.hidden, g.inter, g.group}};
            bool ok = !mfma && g.group == kLutGroup && g.hidden % kSliceCols == 0 &&
                      g.hidden / kSliceCols <= 15 && g.inter % kLutRows == 0 &&
                      g.inter % kSliceCols == 0 && g.hidden % kLutRows == 0;
            for (int d = 0; ok && d < n_items; ++d) {
                const size_t nu = item_uses[d].size();
                ok = !late[d] && !(read_once && nu > 1) &&
                     !(tile_shape && nu >= size_t(kTileMinUses));
                for (int u : item_uses[d])
                    for (int m = 0; ok && m < 3; ++m)
                        ok = uses[u].k[m] <= kLutMaxK &&
                             lut_offsets_fit(ms[m / 2], uses[u].k[m], g.plane_words);
            }
            if (!ok)
                return failf(PM_ERR_STATE, "under stream capture a layer call may only run LUT "
                             "jobs (k <= %d) on resident experts, with fewer than %d uses per "
                             "expert and no PM_BATCH_MFMA", kLutMaxK, kTileMinUses);
        }
    }
    // forwards on one store run in order; on the same stream they already do
    if (s->fwd_seq > 0 && compute != s->last_compute)
        HIP_TRY(hipStreamWaitEvent(compute, forward_end(s, s->fwd_seq), 0));
    // top-ups (side streams) of the late items, before any work list takes a
    // slot address: a top-up may move the slot's plane buffer
    {
        std::vector<Slot*> ls;
        std::vector<int> lk;
        for (int d = 0; d < n_items; ++d) {
            if (!late[d]) continue;
            ls.push_back(&s->slots[size_t(layer) * s->n_experts + item_expert[d]]);
            lk.push_back(kneed[d]);
        }
        pm_status st = issue_topups(s, ls, lk);
        if (st) return st;
    }
    if (mfma)
        return forward_mfma(s, layer, n_tokens, top_k, uses, item_expert, item_uses, kneed, late,
                            d_x, d_y, compute);
    int n_res = 0;
    while (n_res < n_items && !late[order[n_res]]) ++n_res;
    auto slot_of_item = [&](int d) -> Slot& {
        return s->slots[size_t(layer) * s->n_experts + item_expert[d]];
    };

    // ---- the uses that read one matrix of one expert at one prefix go to
    // the matrix-core tiles when there are at least kTileMinUses of them and
    // the shape allows (marked 2: one slice, h by the SwiGLU kernel)
    const bool tile_shape = g.group == kMfmaGroup && g.hidden % kMfmaGroup == 0 &&
                            g.inter % kMfmaGroup == 0;
    std::vector<MTile> t_gu[2][kBits + 1], t_dn[kBits + 1];
    size_t n_tiles = 0;
    if (tile_shape) {
        for (int i = 0; i < n_items; ++i) {
            const int d = order[i];
            if (int(item_uses[d].size()) < kTileMinUses) continue;
            add_tiles(uses, item_uses[d], slot_of_item(d), g, 0, 2, kTileMinUses,
                      t_gu[i < n_res ? 0 : 1]);
            add_tiles(uses, item_uses[d], slot_of_item(d), g, 2, 3, kTileMinUses, t_dn);
        }
        for (int k = 1; k <= kBits; ++k)
            n_tiles += t_gu[0][k].size() + t_gu[1][k].size() + t_dn[k].size();
    }

    auto any_tiles = [](const std::vector<MTile> (&v)[kBits + 1]) {
        for (const auto& t : v)
            if (!t.empty()) return true;
        return false;
    };
    // ---- path of every (use, matrix) outside the tiles: LUT at k <= 5 when
    // the columns split into 1024-column slices (at most 15), else direct
    // the LUT path takes rows in steps of kLutRows and blocks of kLutGroup
    // inputs
    const bool gu_lut_shape = g.hidden % kSliceCols == 0 && g.group == kLutGroup &&
                              g.hidden / kSliceCols <= 15 && g.inter % kLutRows == 0;
    const bool dn_lut_shape = g.inter % kSliceCols == 0 && g.group == kLutGroup &&
                              g.hidden % kLutRows == 0;
    const int S_gu = gu_lut_shape ? g.hidden / kSliceCols : 1;
    const int S_dn = dn_lut_shape ? g.inter / kSliceCols : 1;
    for (int d = 0; d < n_items; ++d) {
        // PM_READ_ONCE: an expert of several uses is read once by the direct
        // kernels (each use shifts the kmax prefix down to its own k)
        const bool lut_item = !read_once || item_uses[d].size() == 1;
        for (int u : item_uses[d]) {
            for (int m = 0; m < 3; ++m) {
                if (uses[u].direct[m] == 2) continue;
                const bool shape_ok = m < 2 ? gu_lut_shape : dn_lut_shape;
                const pm_matrix_shape ms = m < 2 ? pm_matrix_shape{g.inter, g.hidden, g.group}
                                                 : pm_matrix_shape{g.hidden, g.inter, g.group};
                const bool lut = lut_item && shape_ok && uses[u].k[m] <= kLutMaxK &&
                                 lut_offsets_fit(ms, uses[u].k[m], g.plane_words);
                uses[u].direct[m] = lut ? 0 : 1;
                uses[u].slices[m] = lut ? (m < 2 ? S_gu : S_dn) : 1;
            }
        }
    }

    // ---- workspace: partial sums (device)
    const size_t fGU = align256(size_t(n_uses) * 2 * S_gu * g.inter);
    const size_t fH = align256(size_t(n_uses) * g.inter);
    const size_t fY = align256(size_t(n_uses) * S_dn * g.hidden);
    // the work list is uploaded only when direct-path items or tiles exist
    std::vector<int> dir_gu[2], dir_dn;      // positions in `order`
    for (int grp = 0; grp < 2; ++grp) {
        const int i0 = grp == 0 ? 0 : n_res, i1 = grp == 0 ? n_res : n_items;
        for (int i = i0; i < i1; ++i) {
            bool any = false;
            for (int u : item_uses[order[i]]) any |= uses[u].direct[0] == 1 || uses[u].direct[1] == 1;
            if (any) dir_gu[grp].push_back(i);
        }
    }
    for (int i = 0; i < n_items; ++i) {
        bool any = false;
        for (int u : item_uses[order[i]]) any |= uses[u].direct[2] == 1;
        if (any) dir_dn.push_back(i);
    }
    const size_t n_dir = dir_gu[0].size() + dir_gu[1].size() + dir_dn.size();
    const bool upload = n_dir > 0 || n_tiles > 0;
    const size_t list_bytes = !upload ? 0
                              : align256(sizeof(Item) * n_items) + align256(sizeof(Use) * n_uses) +
                                    align256(sizeof(int32_t) * n_uses) +
                                    align256(sizeof(Item) * n_dir) + align256(sizeof(MTile) * n_tiles);
    pm_status st = ensure_workspace(s, fGU + fH + fY, list_bytes);
    if (st) return st;
    Partials P;
    P.gu = s->ws.d_buf;
    P.h = s->ws.d_buf + fGU;
    P.y = s->ws.d_buf + fGU + fH;
    P.gu_smax = S_gu;
    P.dn_smax = S_dn;

    // ---- LUT launches
    KLaunch gu_proto{};
    gu_proto.x = d_x;
    gu_proto.pstride = g.plane_words;
    gu_proto.S = S_gu;
    gu_proto.rows = g.inter;
    gu_proto.W = g.hidden / 32;
    gu_proto.wpg = g.group / 32;
    gu_proto.out_stride = g.inter;
    gu_proto.x_stride = n_tokens == 1 ? 0 : g.hidden;     // 0: one activation for all jobs
    KLaunch dn_proto{};
    dn_proto.gu = P.gu;
    dn_proto.gu_smax = S_gu;
    dn_proto.inter = g.inter;
    dn_proto.pstride = g.plane_words;
    dn_proto.S = S_dn;
    dn_proto.rows = g.hidden;
    dn_proto.W = g.inter / 32;
    dn_proto.wpg = g.group / 32;
    dn_proto.out_stride = g.hidden;
    std::vector<KLaunch> L_gu[2], L_dn;
    for (int grp = 0; grp < 2; ++grp) {
        const int i0 = grp == 0 ? 0 : n_res, i1 = grp == 0 ? n_res : n_items;
        std::vector<JobSpec> js;
        js.reserve(size_t(2) * n_uses);
        for (int i = i0; i < i1; ++i) {
            const int d = order[i];
            const Slot& sl = slot_of_item(d);
            for (int u : item_uses[d]) {
                for (int m = 0; m < 2; ++m) {
                    if (uses[u].direct[m]) continue;
                    const int k = uses[u].k[m];
                    JobSpec j{};
                    j.job.planes = sl.planes + g.plane_off[m];
                    j.job.lvk = sl.levels + g.level_off[m] +
                                level_offset(size_t(g.inter) * (g.hidden / g.group), k);
                    j.job.out = P.gu + (size_t(u) * 2 + m) * S_gu * g.inter;
                    j.job.src = int16_t(uses[u].tok);
                    j.job.k = int8_t(k);
                    js.push_back(j);
                }
            }
        }
        sort_jobs(js);
        pack_launches(js, gu_proto, L_gu[grp]);
    }
    // The routing-weighted combine folds into the down launches (LUT and
    // direct) when no down product runs in a matrix-core tile: each row sum
    // is added, times its use's weight, into y with a float atomic (y cleared
    // by the first gate/up launch).  The top-k terms of an output then add up in the order they
    // arrive; PM_DETERMINISTIC keeps the separate combine, which adds them in
    // use order.  y may not overlap x (the clearing would race the reads).
    const size_t xy_bytes = sizeof(float) * size_t(n_tokens) * g.hidden;
    const bool xy_apart = reinterpret_cast<uintptr_t>(d_y) + xy_bytes <=
                              reinterpret_cast<uintptr_t>(d_x) ||
                          reinterpret_cast<uintptr_t>(d_x) + xy_bytes <=
                              reinterpret_cast<uintptr_t>(d_y);
    const bool lut_gu = !L_gu[0].empty() || !L_gu[1].empty();
    const bool dir_gu_any = !dir_gu[0].empty() || !dir_gu[1].empty();
    const bool fold = !(flags & PM_DETERMINISTIC) && !any_tiles(t_dn) && (lut_gu || dir_gu_any) &&
                      xy_apart && size_t(n_tokens) * g.hidden < (size_t(1) << 31);
    // the first gate/up launch clears y: a LUT launch if there is one, else
    // the first direct gate/up launch
    float* dir_zero = nullptr;
    int dir_n_zero = 0;
    if (fold) {
        if (lut_gu) {
            KLaunch& first = !L_gu[0].empty() ? L_gu[0].front() : L_gu[1].front();
            first.zero = d_y;
            first.n_zero = n_tokens * g.hidden;
        } else {
            dir_zero = d_y;
            dir_n_zero = n_tokens * g.hidden;
        }
        dn_proto.fold = 1;
        dn_proto.out_stride = 0;
    }
    {
        std::vector<JobSpec> js;
        js.reserve(size_t(n_uses));
        for (int i = 0; i < n_items; ++i) {
            const int d = order[i];
            const Slot& sl = slot_of_item(d);
            for (int u : item_uses[d]) {
                if (uses[u].direct[2]) continue;
                const int k = uses[u].k[2];
                JobSpec j{};
                j.job.planes = sl.planes + g.plane_off[2];
                j.job.lvk = sl.levels + g.level_off[2] +
                            level_offset(size_t(g.hidden) * (g.inter / g.group), k);
                j.job.out = fold ? d_y + size_t(uses[u].tok) * g.hidden
                                 : P.y + size_t(u) * S_dn * g.hidden;
                j.job.wt = uses[u].w;
                j.job.src = int16_t(u);
                j.job.k = int8_t(k);
                j.job.gsl = uint8_t(uses[u].slices[0] | (uses[u].slices[1] << 4));
                js.push_back(j);
            }
        }
        pack_launches(js, dn_proto, L_dn);
    }



    // ---- direct-path work list and tiles into the pinned ring, then to the device
    const Use* duses = nullptr;
    const int32_t* dlist = nullptr;
    const Item* ddir = nullptr;
    const MTile* dtiles = nullptr;
    size_t off_gu[2][kBits + 1] = {}, off_dn[kBits + 1] = {};
    if (upload) {
        Workspace& w = s->ws;
        const int rs = w.next;
        w.next = (w.next + 1) % Workspace::kSlots;
        HIP_TRY(hipEventSynchronize(w.ring_ev[rs]));
        char* hb = w.h_ring + size_t(rs) * w.slot_bytes;
        char* db = w.d_ring + size_t(rs) * w.slot_bytes;
        size_t off = 0;
        auto carve = [&](size_t bytes) {
            const size_t o = off;
            off += align256(bytes);
            return o;
        };
        const size_t o_items = carve(sizeof(Item) * n_items);
        const size_t o_uses = carve(sizeof(Use) * n_uses);
        const size_t o_list = carve(sizeof(int32_t) * n_uses);
        const size_t o_dir = carve(sizeof(Item) * n_dir);
        const size_t o_tiles = carve(sizeof(MTile) * n_tiles);
        size_t tpos = 0;
        auto put = [&](const std::vector<MTile>& v) {
            const size_t at = tpos;
            if (!v.empty())
                std::memcpy(hb + o_tiles + tpos * sizeof(MTile), v.data(), sizeof(MTile) * v.size());
            tpos += v.size();
            return at;
        };
        for (int k = 1; k <= kBits; ++k) {
            off_gu[0][k] = put(t_gu[0][k]);
            off_gu[1][k] = put(t_gu[1][k]);
            off_dn[k] = put(t_dn[k]);
        }
        Item* hitems = reinterpret_cast<Item*>(hb + o_items);
        int32_t* hlist = reinterpret_cast<int32_t*>(hb + o_list);
        int lpos = 0;
        for (int i = 0; i < n_items; ++i) {
            const int d = order[i];
            const Slot& sl = slot_of_item(d);
            Item& it = hitems[i];
            it.planes = sl.planes;
            it.levels = sl.levels;
            it.use0 = lpos;
            it.nuse = int(item_uses[d].size());
            for (int m = 0; m < 3; ++m) it.kmax[m] = kmax[d][m];
            it.pad = 0;
            for (int u : item_uses[d]) hlist[lpos++] = u;
        }
        std::memcpy(hb + o_uses, uses.data(), sizeof(Use) * n_uses);
        Item* hdir = reinterpret_cast<Item*>(hb + o_dir);
        size_t ndi = 0;
        for (auto* v : {&dir_gu[0], &dir_gu[1], &dir_dn})
            for (int i : *v) hdir[ndi++] = hitems[i];
        HIP_TRY(hipMemcpyAsync(db, hb, off, hipMemcpyHostToDevice, compute));
        HIP_TRY(hipEventRecord(w.ring_ev[rs], compute));
        duses = reinterpret_cast<const Use*>(db + o_uses);
        dlist = reinterpret_cast<const int32_t*>(db + o_list);
        ddir = reinterpret_cast<const Item*>(db + o_dir);
        dtiles = reinterpret_cast<const MTile*>(db + o_tiles);
    }
    MLaunch TL{};
    TL.uses = duses;
    TL.x = d_x;
    TL.P = P;
    TL.pstride = g.plane_words;
    auto tiles_of = [&](const std::vector<MTile> (&v)[kBits + 1], const size_t* off, int down) {
        TL.rows = down ? g.hidden : g.inter;
        TL.cols = down ? g.inter : g.hidden;
        TL.down = down;
        return launch_tiles(TL, dtiles, off, v, compute);
    };
    const size_t d_gu0 = dir_gu[0].size(), d_gu1 = dir_gu[1].size();

    // ---- kernels
    // resident slots topped up by an earlier explicit call may still be copying
    for (int i = 0; i < n_res; ++i) {
        Slot& sl = slot_of_item(order[i]);
        if (sl.pending) {
            HIP_TRY(hipStreamWaitEvent(compute, sl.ready, 0));
            sl.pending = false;
        }
    }
    // a gate/up stage of one LUT launch is timed by the launch itself, except
    // under stream capture, where the events become graph nodes of their own
    bool gu_single = L_gu[0].size() == 1 && d_gu0 == 0 && n_res == n_items && n_tiles == 0;
    if (s->profiling && gu_single) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        HIP_TRY(hipStreamIsCapturing(compute, &cs));
        if (cs != hipStreamCaptureStatusNone) gu_single = false;
    }
    if (s->profiling && !gu_single) HIP_TRY(hipEventRecord(s->prof[0], compute));
    for (const KLaunch& L : L_gu[0]) {
        if (s->profiling && gu_single)
            HIP_TRY(launch_lut(L, false, compute, s->prof[0], s->prof[1]));
        else
            HIP_TRY(launch_lut(L, false, compute));
    }
    if (d_gu0)
        HIP_TRY(launch_direct_gateup(g, ddir, int(d_gu0), duses, dlist, d_x, P, compute, dir_zero,
                                     dir_n_zero));
    if (any_tiles(t_gu[0])) {
        st = tiles_of(t_gu[0], off_gu[0], 0);
        if (st) return st;
    }
    if (n_res < n_items) {
        for (int i = n_res; i < n_items; ++i) {
            Slot& sl = slot_of_item(order[i]);
            HIP_TRY(hipStreamWaitEvent(compute, sl.ready, 0));
            sl.pending = false;
        }
        for (const KLaunch& L : L_gu[1]) HIP_TRY(launch_lut(L, false, compute));
        if (d_gu1)
            HIP_TRY(launch_direct_gateup(g, ddir + d_gu0, int(d_gu1), duses, dlist, d_x, P,
                                         compute, d_gu0 ? nullptr : dir_zero,
                                         d_gu0 ? 0 : dir_n_zero));
        if (any_tiles(t_gu[1])) {
            st = tiles_of(t_gu[1], off_gu[1], 0);
            if (st) return st;
        }
    }
    if (s->profiling && !gu_single) HIP_TRY(hipEventRecord(s->prof[1], compute));
    if (!dir_dn.empty() || any_tiles(t_dn)) {
        // h of the direct and tiled down products, where the direct gate/up
        // kernel has not formed it
        bool swiglu = false;
        for (int u = 0; u < n_uses && !swiglu; ++u)
            swiglu = uses[u].direct[2] != 0 && !h_by_gateup(uses[u]);
        if (swiglu) HIP_TRY(launch_swiglu(duses, n_uses, P, g.inter, compute));
        if (!dir_dn.empty())
            HIP_TRY(launch_direct_down(g, ddir + d_gu0 + d_gu1, int(dir_dn.size()), duses, dlist,
                                       P, compute, fold ? d_y : nullptr));
        if (any_tiles(t_dn)) {
            st = tiles_of(t_dn, off_dn, 1);
            if (st) return st;
        }
    }
    for (const KLaunch& L : L_dn) HIP_TRY(launch_lut(L, true, compute));
    if (s->profiling && s->n_prof >= 4) HIP_TRY(hipEventRecord(s->prof[2], compute));
    const int tok_per = std::max(1, kMaxLaunchUses / top_k);
    for (int t0 = 0; !fold && t0 < n_tokens; t0 += tok_per) {
        KCombine C{};
        C.Y = P.y;
        C.y = d_y;
        C.t0 = t0;
        C.n_tokens = std::min(tok_per, n_tokens - t0);
        C.top_k = top_k;
        C.hidden = g.hidden;
        C.dn_smax = S_dn;
        for (int a = 0; a < C.n_tokens * top_k; ++a) {
            const Use& us = uses[size_t(t0) * top_k + a];
            C.w[a] = us.w;
            C.sl[a] = uint8_t(us.slices[2]);
        }
        HIP_TRY(launch_combine_k(C, compute));
    }
    if (s->profiling && s->n_prof >= 4) HIP_TRY(hipEventRecord(s->prof[3], compute));
    std::vector<Slot*> read(n_items);
    for (int i = 0; i < n_items; ++i) read[i] = &slot_of_item(order[i]);
    return finish_forward(s, compute, read);
}
