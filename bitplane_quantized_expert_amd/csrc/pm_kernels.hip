// HIP kernels of libpm for gfx950 (CDNA4, 64-wide wavefronts).
//
// Prefix GEMV [Abs "directly executes cached 1-8-bit prefixes without
// materializing full-precision experts"; T c25, c37]: a wave owns one output
// row; each lane walks the row's plane words (32 weights each), reads the k
// leading plane words of that word, forms each weight's k-bit prefix, looks
// its value up in the depth-k node table of its block and accumulates
// value * x in fp32.  Rows are reduced across the wave in a fixed butterfly
// order, so results are deterministic.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "pm_internal.h"

namespace pm {

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kRowsPerBlock = kBlock / kWave;

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// This lane's share of row o of one matrix at prefix k.
//   planes: plane 0 of the matrix, planes pstride words apart
//   lv_k:   depth-k nodes of the matrix (levels + level_offset(k))
//   W:      words per row; wpg: words per block
__device__ inline float row_dot_lane(const uint32_t* __restrict__ planes, size_t pstride,
                                     const float* __restrict__ lv_k, int k, int o, int W,
                                     int wpg, const float* __restrict__ x, int lane) {
    float acc = 0.f;
    const int nb_row = W / wpg;
    for (int w = lane; w < W; w += kWave) {
        uint32_t pw[kBits];
#pragma unroll
        for (int p = 0; p < kBits; ++p)
            pw[p] = p < k ? planes[size_t(p) * pstride + size_t(o) * W + w] : 0u;
        const float* tab = lv_k + ((size_t(o) * nb_row + w / wpg) << k);
        const float* xw = x + 32 * w;
#pragma unroll 4
        for (int j = 0; j < 32; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int p = 0; p < kBits; ++p)
                if (p < k) v = (v << 1) | ((pw[p] >> j) & 1u);
            acc = fmaf(tab[v], xw[j], acc);
        }
    }
    return acc;
}

__global__ __launch_bounds__(kBlock) void gemv_kernel(int rows, int cols, int group, int k,
                                                      const uint32_t* __restrict__ planes,
                                                      size_t pstride,
                                                      const float* __restrict__ levels,
                                                      const float* __restrict__ x,
                                                      float* __restrict__ y) {
    const int lane = threadIdx.x % kWave;
    const int o = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= rows) return;
    const int W = cols / 32;
    const size_t nb = size_t(rows) * (cols / group);
    float acc = row_dot_lane(planes, pstride, levels + level_offset(nb, k), k, o, W, group / 32,
                             x, lane);
    acc = wave_sum(acc);
    if (lane == 0) y[o] = acc;
}

// ---- MoE stages ---------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void gateup_kernel(Geom g, const Item* __restrict__ items,
                                                        int item0, int bpi,
                                                        const Use* __restrict__ uses,
                                                        const int32_t* __restrict__ list,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ G,
                                                        float* __restrict__ U) {
    const Item it = items[item0 + blockIdx.x / bpi];
    const int lane = threadIdx.x % kWave;
    const int o = (blockIdx.x % bpi) * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= g.inter) return;
    const int W = g.hidden / 32;
    const size_t nb = size_t(g.inter) * (g.hidden / g.group);
    for (int q = 0; q < it.nuse; ++q) {
        const int u = list[it.use0 + q];
        const Use us = uses[u];
        const float* xt = x + size_t(us.tok) * g.hidden;
        for (int m = 0; m < 2; ++m) {
            const int k = us.k[m];
            float acc = row_dot_lane(it.planes + g.plane_off[m], g.plane_words,
                                     it.levels + g.level_off[m] + level_offset(nb, k), k, o, W,
                                     g.group / 32, xt, lane);
            acc = wave_sum(acc);
            if (lane == 0) (m == 0 ? G : U)[size_t(u) * g.inter + o] = acc;
        }
    }
}

// h = silu(g) * u, in place over G.
__global__ __launch_bounds__(kBlock) void swiglu_kernel(size_t n, float* __restrict__ G,
                                                        const float* __restrict__ U) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= n) return;
    const float gv = G[i];
    G[i] = gv / (1.0f + expf(-gv)) * U[i];
}

__global__ __launch_bounds__(kBlock) void down_kernel(Geom g, const Item* __restrict__ items,
                                                      int bpi, const Use* __restrict__ uses,
                                                      const int32_t* __restrict__ list,
                                                      const float* __restrict__ H,
                                                      float* __restrict__ Y) {
    const Item it = items[blockIdx.x / bpi];
    const int lane = threadIdx.x % kWave;
    const int o = (blockIdx.x % bpi) * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= g.hidden) return;
    const int W = g.inter / 32;
    const size_t nb = size_t(g.hidden) * (g.inter / g.group);
    for (int q = 0; q < it.nuse; ++q) {
        const int u = list[it.use0 + q];
        const int k = uses[u].k[2];
        float acc = row_dot_lane(it.planes + g.plane_off[2], g.plane_words,
                                 it.levels + g.level_off[2] + level_offset(nb, k), k, o, W,
                                 g.group / 32, H + size_t(u) * g.inter, lane);
        acc = wave_sum(acc);
        if (lane == 0) Y[size_t(u) * g.hidden + o] = acc;
    }
}

// y[t][o] = sum_j w[t][j] * Y[t*top_k + j][o], slots in order.
__global__ __launch_bounds__(kBlock) void combine_kernel(int n_tokens, int top_k, int hidden,
                                                         const Use* __restrict__ uses,
                                                         const float* __restrict__ Y,
                                                         float* __restrict__ y) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(n_tokens) * hidden) return;
    const int t = int(i / hidden), o = int(i % hidden);
    float acc = 0.f;
    for (int j = 0; j < top_k; ++j) {
        const int u = t * top_k + j;
        acc = fmaf(uses[u].w, Y[size_t(u) * hidden + o], acc);
    }
    y[i] = acc;
}

// ---- encoder -------------------------------------------------------------------
// Planes: one thread per (row, word); bit j of plane p = bit (7-p) of code 32w+j.
__global__ __launch_bounds__(kBlock) void encode_planes_kernel(int rows, int W,
                                                               const uint8_t* __restrict__ codes,
                                                               uint32_t* __restrict__ planes,
                                                               size_t pstride) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(rows) * W) return;
    const uint32_t* c4 = reinterpret_cast<const uint32_t*>(codes + i * 32);
    uint32_t word[kBits] = {};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t c = c4[q];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t code = (c >> (8 * b)) & 0xFFu;
            const int j = 4 * q + b;
#pragma unroll
            for (int p = 0; p < kBits; ++p) word[p] |= ((code >> (7 - p)) & 1u) << j;
        }
    }
#pragma unroll
    for (int p = 0; p < kBits; ++p) planes[size_t(p) * pstride + i] = word[p];
}

// Levels: one block of 256 threads per codebook block.  Depth 8 is the leaves;
// each shallower node is (left + right) * 0.5f, or the count-weighted mean in
// fp64 when counts are given (fallback to the plain mean for empty subtrees).
__global__ __launch_bounds__(kLeaves) void encode_levels_kernel(size_t nb,
                                                                const float* __restrict__ leaves,
                                                                const uint32_t* __restrict__ counts,
                                                                float* __restrict__ levels) {
#pragma clang fp contract(off)
    __shared__ float val[2][kLeaves];
    __shared__ unsigned long long cnt[2][kLeaves];
    const size_t b = blockIdx.x;
    const int t = threadIdx.x;
    const float leaf = leaves[b * kLeaves + t];
    val[0][t] = leaf;
    cnt[0][t] = counts ? counts[b * kLeaves + t] : 0ull;
    levels[level_offset(nb, kBits) + (b << kBits) + t] = leaf;
    __syncthreads();
    int cur = 0;
    for (int d = kBits - 1; d >= 1; --d) {
        const int n = 1 << d;
        if (t < n) {
            const float L = val[cur][2 * t], R = val[cur][2 * t + 1];
            const float mean = (L + R) * 0.5f;
            float pv = mean;
            unsigned long long tot = 0;
            if (counts) {
                const unsigned long long nl = cnt[cur][2 * t], nr = cnt[cur][2 * t + 1];
                tot = nl + nr;
                if (tot > 0) {
                    const double num = __dadd_rn(__dmul_rn(double(nl), double(L)),
                                                 __dmul_rn(double(nr), double(R)));
                    pv = float(__ddiv_rn(num, double(tot)));
                }
            }
            val[cur ^ 1][t] = pv;
            cnt[cur ^ 1][t] = tot;
            levels[level_offset(nb, d) + (b << d) + t] = pv;
        }
        __syncthreads();
        cur ^= 1;
    }
}

// ---- checks and baselines -------------------------------------------------------
__device__ inline uint32_t prefix_at(const uint32_t* __restrict__ planes, size_t pstride,
                                     size_t word, int bit, int k) {
    uint32_t v = 0;
    for (int p = 0; p < k; ++p) v = (v << 1) | ((planes[size_t(p) * pstride + word] >> bit) & 1u);
    return v;
}

__global__ __launch_bounds__(kBlock) void unpack_prefix_kernel(int rows, int cols, int k,
                                                               const uint32_t* __restrict__ planes,
                                                               size_t pstride,
                                                               uint8_t* __restrict__ out) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(rows) * cols) return;
    out[i] = uint8_t(prefix_at(planes, pstride, i / 32, int(i % 32), k));
}

__global__ __launch_bounds__(kBlock) void dequant_kernel(int rows, int cols, int group, int k,
                                                         const uint32_t* __restrict__ planes,
                                                         size_t pstride,
                                                         const float* __restrict__ levels,
                                                         float* __restrict__ out32,
                                                         uint16_t* __restrict__ out16) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(rows) * cols) return;
    const size_t nb = size_t(rows) * (cols / group);
    const size_t o = i / cols, c = i % cols;
    const uint32_t v = prefix_at(planes, pstride, i / 32, int(i % 32), k);
    const float val = levels[level_offset(nb, k) + ((o * (cols / group) + c / group) << k) + v];
    if (out32) out32[i] = val;
    if (out16) out16[i] = __half_as_ushort(__float2half_rn(val));
}

__global__ __launch_bounds__(kBlock) void gemv_fp16_kernel(int rows, int cols,
                                                           const uint16_t* __restrict__ w,
                                                           const float* __restrict__ x,
                                                           float* __restrict__ y) {
    const int lane = threadIdx.x % kWave;
    const int o = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= rows) return;
    const uint16_t* row = w + size_t(o) * cols;
    float acc = 0.f;
    for (int c = lane * 8; c < cols; c += kWave * 8) {
        const uint4 pk = *reinterpret_cast<const uint4*>(row + c);
        const uint32_t q[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __half2float(__ushort_as_half(uint16_t(q[i] & 0xFFFFu)));
            const float hi = __half2float(__ushort_as_half(uint16_t(q[i] >> 16)));
            acc = fmaf(lo, x[c + 2 * i], acc);
            acc = fmaf(hi, x[c + 2 * i + 1], acc);
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) y[o] = acc;
}

inline unsigned grid_for(size_t n, int per) { return unsigned((n + per - 1) / per); }

}  // namespace

int gateup_rows_per_block() { return kRowsPerBlock; }
int down_rows_per_block() { return kRowsPerBlock; }
int max_uses_per_item() { return 64; }

hipError_t launch_gemv(int rows, int cols, int group, int k, const uint32_t* planes,
                       size_t pstride, const float* levels, const float* x, float* y,
                       hipStream_t st) {
    hipLaunchKernelGGL(gemv_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(kBlock), 0, st,
                       rows, cols, group, k, planes, pstride, levels, x, y);
    return hipGetLastError();
}

hipError_t launch_encode_device(int rows, int cols, int group, const uint8_t* codes,
                                const float* leaves, const uint32_t* counts, uint32_t* planes,
                                size_t pstride, float* levels, hipStream_t st) {
    const int W = cols / 32;
    hipLaunchKernelGGL(encode_planes_kernel, dim3(grid_for(size_t(rows) * W, kBlock)),
                       dim3(kBlock), 0, st, rows, W, codes, planes, pstride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t nb = size_t(rows) * (cols / group);
    hipLaunchKernelGGL(encode_levels_kernel, dim3(unsigned(nb)), dim3(kLeaves), 0, st, nb,
                       leaves, counts, levels);
    return hipGetLastError();
}

hipError_t launch_unpack_prefix(int rows, int cols, int k, const uint32_t* planes,
                                size_t pstride, uint8_t* out, hipStream_t st) {
    hipLaunchKernelGGL(unpack_prefix_kernel, dim3(grid_for(size_t(rows) * cols, kBlock)),
                       dim3(kBlock), 0, st, rows, cols, k, planes, pstride, out);
    return hipGetLastError();
}

hipError_t launch_dequant(int rows, int cols, int group, int k, const uint32_t* planes,
                          size_t pstride, const float* levels, float* out32, uint16_t* out16,
                          hipStream_t st) {
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(size_t(rows) * cols, kBlock)),
                       dim3(kBlock), 0, st, rows, cols, group, k, planes, pstride, levels,
                       out32, out16);
    return hipGetLastError();
}

hipError_t launch_gemv_fp16(int rows, int cols, const uint16_t* w, const float* x, float* y,
                            hipStream_t st) {
    hipLaunchKernelGGL(gemv_fp16_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(kBlock), 0,
                       st, rows, cols, w, x, y);
    return hipGetLastError();
}

hipError_t launch_gateup(const Geom& g, const Item* items, int item0, int n_items,
                         int n_blocks, const Use* uses, const int32_t* list, int top_k,
                         const float* x, float* G, float* U, hipStream_t st) {
    (void)top_k;
    if (n_items == 0) return hipSuccess;
    const int bpi = n_blocks / n_items;
    hipLaunchKernelGGL(gateup_kernel, dim3(n_blocks), dim3(kBlock), 0, st, g, items, item0, bpi,
                       uses, list, x, G, U);
    return hipGetLastError();
}

hipError_t launch_down(const Geom& g, const Item* items, int n_items, int n_blocks,
                       const Use* uses, const int32_t* list, int n_uses, float* G,
                       const float* U, float* Y, hipStream_t st) {
    if (n_items == 0) return hipSuccess;
    const size_t n = size_t(n_uses) * g.inter;
    hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(n, kBlock)), dim3(kBlock), 0, st, n, G, U);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bpi = n_blocks / n_items;
    hipLaunchKernelGGL(down_kernel, dim3(n_blocks), dim3(kBlock), 0, st, g, items, bpi, uses,
                       list, G, Y);
    return hipGetLastError();
}

hipError_t launch_combine(int n_tokens, int top_k, int hidden, const Use* uses, const float* Y,
                          float* y, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(size_t(n_tokens) * hidden, kBlock)),
                       dim3(kBlock), 0, st, n_tokens, top_k, hidden, uses, Y, y);
    return hipGetLastError();
}

}  // namespace pm
