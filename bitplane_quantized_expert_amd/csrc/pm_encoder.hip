// Encoder from fp32 weights, first half: per block of weights, K-means learns
// 256 values that become the sorted leaves of the tree codebook ("PagedMoE:
// Cross-Precision Expert Caching for SSD-Resident MoE Inference", podcast
// transcript, cue 19).  The planes and the count-weighted tree follow from
// the codes, leaves and counts written here (encode kernels in
// pm_kernels.hip).
//
// One workgroup of 256 threads per block, one centroid per thread.  The block
// is sorted once in LDS (bitonic network); in one dimension every nearest-
// centroid cell is an interval of the sorted weights, so an assignment is 256
// cut positions and a centroid update is a sequential fp64 sum over one
// interval, in ascending order.  Lloyd's iteration:
//   start   c_j = the ceil((2j+1) G / 512)-th smallest weight (1-based);
//   assign  nearest centroid, ties to the lowest index: a weight x between
//           the values lo <= x < hi goes to hi iff 2x > lo + hi (fp64, exact
//           for fp32 operands within 2^29 of each other), else to the first
//           index holding lo;
//   update  c_j = fp32(sum of members / count), members summed in fp64;
//           an empty cell keeps its centroid; then the centroids are sorted
//           again (a relabelling; needed when starting centroids repeat,
//           since the first of a run of equal centroids can take members
//           above the run and pass its empty twins);
//   stop    when an update leaves every cut in place, or after max_iters
//           updates.
#include <hip/hip_runtime.h>

#include "pm_encoder.h"

namespace pm {

namespace {

constexpr int kKm = 256;                       // centroids = threads

// Number of centroids <= x (c ascending).
__device__ inline int count_le(const float* c, float x) {
    int pos = 0;
#pragma unroll
    for (int step = kKm; step >= 1; step >>= 1)
        if (pos + step <= kKm && c[pos + step - 1] <= x) pos += step;
    return pos;
}

// Number of centroids < x (c ascending).
__device__ inline int count_lt(const float* c, float x) {
    int pos = 0;
#pragma unroll
    for (int step = kKm; step >= 1; step >>= 1)
        if (pos + step <= kKm && c[pos + step - 1] < x) pos += step;
    return pos;
}

__device__ inline int assign(const float* c, const int* first, float x) {
    const int hi = count_le(c, x);
    if (hi == 0) return 0;
    if (hi == kKm) return first[kKm - 1];
    const double two_x = 2.0 * double(x);
    const double mid2 = double(c[hi - 1]) + double(c[hi]);
    return two_x > mid2 ? hi : first[hi - 1];
}

// Cut positions of the current assignment: cut[j] = number of sorted weights
// whose code is below j (codes are non-decreasing along the sorted block).
__device__ inline int cut_of(const uint8_t* code, int g, int j) {
    int lo = 0, hi = g;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (int(code[mid]) < j) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kKm) void kmeans_block_kernel(int cols, int group,
                                                           const float* __restrict__ w,
                                                           int max_iters,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ leaves,
                                                           uint32_t* __restrict__ counts,
                                                           int32_t* __restrict__ iters) {
#pragma clang fp contract(off)
    __shared__ float key[kMaxKmeansGroup];
    __shared__ uint16_t idx[kMaxKmeansGroup];
    __shared__ uint8_t code[kMaxKmeansGroup];
    __shared__ uint8_t out[kMaxKmeansGroup];
    __shared__ float c[kKm];
    __shared__ float c2[kKm];
    __shared__ int first[kKm];
    __shared__ int cut[kKm + 1];

    const int t = threadIdx.x;
    const int nbr = cols / group;
    const size_t b = blockIdx.x;
    const size_t row = b / nbr;
    const size_t base = row * size_t(cols) + (b - row * nbr) * size_t(group);
    const int g = group;
    int p2 = 1;
    while (p2 < g) p2 <<= 1;

    // load and pad to a power of two with +inf
    for (int i = t; i < p2; i += kKm) {
        key[i] = i < g ? w[base + i] : __builtin_inff();
        idx[i] = uint16_t(i);
    }
    __syncthreads();

    // bitonic sort, ascending
    for (int k = 2; k <= p2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < (p2 >> 1); i += kKm) {
                const int a = 2 * i - (i & (j - 1));
                const int bb = a + j;
                const bool up = (a & k) == 0;
                const float ka = key[a], kb = key[bb];
                if ((ka > kb) == up) {
                    key[a] = kb;
                    key[bb] = ka;
                    const uint16_t ia = idx[a];
                    idx[a] = idx[bb];
                    idx[bb] = ia;
                }
            }
            __syncthreads();
        }
    }

    // starting centroids: sample quantiles
    c[t] = key[((2 * t + 1) * g + 2 * kKm - 1) / (2 * kKm) - 1];
    __syncthreads();
    first[t] = count_lt(c, c[t]);
    __syncthreads();
    for (int i = t; i < g; i += kKm) code[i] = uint8_t(assign(c, first, key[i]));
    __syncthreads();
    cut[t] = cut_of(code, g, t);
    if (t == 0) cut[kKm] = g;
    __syncthreads();

    int it = 0;
    while (it < max_iters) {
        const int lo = cut[t], hi = cut[t + 1];
        if (hi > lo) {
            double s = 0.0;
            for (int i = lo; i < hi; ++i) s += double(key[i]);
            c[t] = float(s / double(hi - lo));
        }
        ++it;
        __syncthreads();
        if (__syncthreads_or(t + 1 < kKm && c[t] > c[t + 1])) {
            // stable rank: smaller values, then equal values at lower index
            const float v = c[t];
            int r = 0;
            for (int i = 0; i < kKm; ++i) {
                const float u = c[i];
                r += (u < v) || (u == v && i < t);
            }
            c2[r] = v;
            __syncthreads();
            c[t] = c2[t];
            __syncthreads();
        }
        first[t] = count_lt(c, c[t]);
        __syncthreads();
        for (int i = t; i < g; i += kKm) code[i] = uint8_t(assign(c, first, key[i]));
        __syncthreads();
        const int nc = cut_of(code, g, t);
        const bool moved = nc != lo;
        __syncthreads();                 // every cut read above before it changes
        cut[t] = nc;
        const int any = __syncthreads_or(moved);
        if (!any) break;
    }

    for (int i = t; i < g; i += kKm) out[idx[i]] = code[i];
    leaves[b * kKm + t] = c[t];
    counts[b * kKm + t] = uint32_t(cut[t + 1] - cut[t]);
    if (iters && t == 0) iters[b] = it;
    __syncthreads();
    for (int i = t; i < g; i += kKm) codes[base + i] = out[i];
}

}  // namespace

hipError_t launch_kmeans_device(int rows, int cols, int group, const float* w, int max_iters,
                                uint8_t* codes, float* leaves, uint32_t* counts,
                                int32_t* iters, hipStream_t st) {
    const size_t nb = size_t(rows) * (cols / group);
    hipLaunchKernelGGL(kmeans_block_kernel, dim3(unsigned(nb)), dim3(kKm), 0, st, cols, group, w,
                       max_iters, codes, leaves, counts, iters);
    return hipGetLastError();
}

}  // namespace pm
