// HIP kernels of libpm for gfx950 (CDNA4, 64-wide wavefronts), except the
// LUT path (pm_lut.hip).
//
// Direct path (any k, any shape; an expert of several uses is read once for
// all of them): per weight, the prefix is assembled from the k plane words
// and its node read from the depth-k table, which for group 128 and rows of
// whole 1024-column runs is first staged in LDS (row_dot_lds) [Abs; T c25,
// c37: execution straight from a cached prefix, no full-precision copy].
// Also the offline encoder, the combine, and the checks and baselines.
//
// All sums run in a fixed order (DPP row reductions, slices and slots in
// index order), so every output is deterministic.
#include <algorithm>

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "pm_device.h"
#include "pm_internal.h"

namespace pm {

namespace {
// ---------------------------------------------------------------- direct path
// This lane's share of row o of one matrix at prefix k.
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
        // the word's 32 activations as eight 16-byte loads (a lane's columns
        // are contiguous; one value per load would touch 64 lines per load)
        float xv[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 a = *(g_f32x4*)(x + 32 * w + 4 * q);
            xv[4 * q] = a.x;
            xv[4 * q + 1] = a.y;
            xv[4 * q + 2] = a.z;
            xv[4 * q + 3] = a.w;
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int p = 0; p < kBits; ++p)
                if (p < k) v = (v << 1) | ((pw[p] >> j) & 1u);
            acc = fmaf(tab[v], xv[j], acc);
        }
    }
    return acc;
}

// Group 128, rows of whole 1024-column runs, any k (staging was first needed
// at k >= 5, where the depth-k tables dominate the bytes: 8 << k per 32-word
// run against k words of planes, and a per-weight gather straight from
// global memory touches up to 64 cache lines per instruction; it also won at
// smaller k, for experts shared by several uses).  Here a
// wave takes a row in runs of 32 words (8 blocks, 1024 inputs); each lane
// takes half a word.  The run's 8 tables are one contiguous range of the
// level-major layout: they arrive as coalesced 16-byte loads (the next run's
// issued while this one computes) and are written to the wave's own LDS
// region, where every weight's node is read.  The wave alone writes and
// reads its region, and LDS operations of one wave complete in order.
constexpr int kRunWords = 32;
constexpr int kRunTabFloatsMax = 8 << kBits;
#ifndef PM_LDS_MIN_K
#define PM_LDS_MIN_K 1
#endif
constexpr int kLdsMinK = PM_LDS_MIN_K;   // smallest k read through the staged tables
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

template <int K>
__device__ __attribute__((always_inline)) inline float row_dot_lds(
    const uint32_t* __restrict__ planes, size_t pstride, const float* __restrict__ rowtab, int o,
    int W, const float* __restrict__ x, lds_f32* __restrict__ tabs, int lane) {
    constexpr int kRunFloats = 8 << K;
    // 16-byte pieces per lane; below k = 5 only the first lanes hold one
    constexpr bool kPartial = kRunFloats < 4 * kWave;
    constexpr int kLoads = kPartial ? 1 : kRunFloats / (4 * kWave);
    const bool holds = !kPartial || lane < kRunFloats / 4;
    const int h = lane & 1;
    const int runs = W / kRunWords;
    f32x4 T[kLoads];
    if (holds) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) T[i] = *(g_f32x4*)(rowtab + 4 * (lane + kWave * i));
    }
    const lds_f32* bt = tabs + ((lane >> 3) << K);        // this lane's block of the run
    float acc = 0.f;
    for (int r = 0; r < runs; ++r) {
        const int w = r * kRunWords + (lane >> 1);
        uint32_t pw[K];
#pragma unroll
        for (int p = 0; p < K; ++p)
            pw[p] = planes[size_t(p) * pstride + size_t(o) * W + w] >> (16 * h);
        f32x4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = *(g_f32x4*)(x + 32 * w + 16 * h + 4 * q);
        if (holds) {
#pragma unroll
            for (int i = 0; i < kLoads; ++i) *(lds_f32x4*)(tabs + 4 * (lane + kWave * i)) = T[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (holds && r + 1 < runs) {
#pragma unroll
            for (int i = 0; i < kLoads; ++i)
                T[i] = *(g_f32x4*)(rowtab + size_t(r + 1) * kRunFloats + 4 * (lane + kWave * i));
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int p = 0; p < K; ++p) v = (v << 1) | ((pw[p] >> j) & 1u);
            acc = fmaf(bt[v], xv[j >> 2][j & 3], acc);
        }
        __builtin_amdgcn_wave_barrier();
    }
    return acc;
}

// This lane's share of row o at prefix k: the LDS-staged form where it
// applies (group 128, k >= kLdsMinK, whole runs), else row_dot_lane.  The
// choice is uniform over the wave.
__device__ __attribute__((always_inline)) inline float row_dot(
    const uint32_t* __restrict__ planes, size_t pstride, const float* __restrict__ lv_k, int k,
    int o, int W, int wpg, const float* __restrict__ x, lds_f32* __restrict__ tabs, int lane) {
    if (wpg == 4 && k >= kLdsMinK && W % kRunWords == 0) {
        const float* rowtab = lv_k + ((size_t(o) * (W / 4)) << k);
        if ((reinterpret_cast<uintptr_t>(rowtab) & 15) == 0 &&
            (reinterpret_cast<uintptr_t>(x) & 15) == 0) {
            switch (k) {
            case 1:
                if constexpr (kLdsMinK <= 1)
                    return row_dot_lds<1>(planes, pstride, rowtab, o, W, x, tabs, lane);
                break;
            case 2:
                if constexpr (kLdsMinK <= 2)
                    return row_dot_lds<2>(planes, pstride, rowtab, o, W, x, tabs, lane);
                break;
            case 3:
                if constexpr (kLdsMinK <= 3)
                    return row_dot_lds<3>(planes, pstride, rowtab, o, W, x, tabs, lane);
                break;
            case 4:
                if constexpr (kLdsMinK <= 4)
                    return row_dot_lds<4>(planes, pstride, rowtab, o, W, x, tabs, lane);
                break;
            case 5: return row_dot_lds<5>(planes, pstride, rowtab, o, W, x, tabs, lane);
            case 6: return row_dot_lds<6>(planes, pstride, rowtab, o, W, x, tabs, lane);
            case 7: return row_dot_lds<7>(planes, pstride, rowtab, o, W, x, tabs, lane);
            default: return row_dot_lds<8>(planes, pstride, rowtab, o, W, x, tabs, lane);
            }
        }
    }
    return row_dot_lane(planes, pstride, lv_k, k, o, W, wpg, x, lane);
}

__global__ __launch_bounds__(kBlock) void gemv_direct_kernel(int rows, int cols, int group, int k,
                                                             const uint32_t* __restrict__ planes,
                                                             size_t pstride,
                                                             const float* __restrict__ levels,
                                                             const float* __restrict__ x,
                                                             float* __restrict__ y) {
    __shared__ float tabs[kRowsPerBlock][kRunTabFloatsMax];
    const int lane = threadIdx.x % kWave;
    const int o = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= rows) return;
    const int W = cols / 32;
    const size_t nb = size_t(rows) * (cols / group);
    float acc = row_dot(planes, pstride, levels + level_offset(nb, k), k, o, W, group / 32, x,
                        (lds_f32*)tabs[threadIdx.x / kWave], lane);
    acc = wave_sum(acc);
    if (lane == kWave - 1) y[o] = acc;
}

__global__ __launch_bounds__(kBlock) void direct_gateup_kernel(Geom g,
                                                               const Item* __restrict__ items,
                                                               int bpi,
                                                               const Use* __restrict__ uses,
                                                               const int32_t* __restrict__ list,
                                                               const float* __restrict__ x,
                                                               Partials P,
                                                               float* __restrict__ zero,
                                                               int n_zero) {
    __shared__ float tabs[kRowsPerBlock][kRunTabFloatsMax];
    // clear the layer output a folded down stage adds into (it runs after
    // this launch on the same stream)
    for (int i = int(blockIdx.x) * kBlock + int(threadIdx.x); i < n_zero;
         i += int(gridDim.x) * kBlock)
        zero[i] = 0.f;
    const Item it = items[blockIdx.x / bpi];
    const int lane = threadIdx.x % kWave;
    const int o = (blockIdx.x % bpi) * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= g.inter) return;
    const int W = g.hidden / 32;
    const size_t nb = size_t(g.inter) * (g.hidden / g.group);
    // one (use, matrix) per step; fields read from memory by index, so no
    // copy of the use record is indexed in registers.  A use whose gate and
    // up rows both run here (gate first) also gets h = SiLU(g) * u of row o
    // (a direct matrix has one slice, so this is the SwiGLU kernel's value).
    float acc_gate = 0.f;
    for (int qm = 0; qm < 2 * it.nuse; ++qm) {
        const int m = qm & 1;
        const int u = list[it.use0 + (qm >> 1)];
        const Use* up = uses + u;
        if (up->direct[m] != 1) continue;      // 0: LUT job, 2: tile
        const int k = up->k[m];
        const float* xt = x + size_t(up->tok) * g.hidden;
        float acc = row_dot(it.planes + g.plane_off[m], g.plane_words,
                            it.levels + g.level_off[m] + level_offset(nb, k), k, o, W,
                            g.group / 32, xt, (lds_f32*)tabs[threadIdx.x / kWave], lane);
        acc = wave_sum(acc);
        if (lane == kWave - 1) {
            P.gu[(size_t(u) * 2 + m) * P.gu_smax * g.inter + o] = acc;
            if (m == 0)
                acc_gate = acc;
            else if (h_by_gateup(*up))
                P.h[size_t(u) * g.inter + o] = silu_mul(acc_gate, acc);
        }
    }
}

// Gate/up partial sums of use u summed over their slices, in slice order.
__device__ inline float gu_sum(const Partials& P, const Use& us, int u, int m, int inter, int c) {
    const float* base = P.gu + (size_t(u) * 2 + m) * P.gu_smax * inter + c;
    float s = base[0];
    for (int q = 1; q < us.slices[m]; ++q) s += base[size_t(q) * inter];
    return s;
}

__global__ __launch_bounds__(kBlock) void swiglu_kernel(const Use* __restrict__ uses, int n_uses,
                                                        Partials P, int inter) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(n_uses) * inter) return;
    const int u = int(i / inter), c = int(i % inter);
    const Use us = uses[u];
    // h of the direct and tile paths, unless the direct gate/up kernel formed it
    if (!us.direct[2] || h_by_gateup(us)) return;
    P.h[i] = silu_mul(gu_sum(P, us, u, 0, inter, c), gu_sum(P, us, u, 1, inter, c));
}

__global__ __launch_bounds__(kBlock) void direct_down_kernel(Geom g, const Item* __restrict__ items,
                                                             int bpi,
                                                             const Use* __restrict__ uses,
                                                             const int32_t* __restrict__ list,
                                                             Partials P, float* __restrict__ yf) {
    __shared__ float tabs[kRowsPerBlock][kRunTabFloatsMax];
    const Item it = items[blockIdx.x / bpi];
    const int lane = threadIdx.x % kWave;
    const int o = (blockIdx.x % bpi) * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= g.hidden) return;
    const int W = g.inter / 32;
    const size_t nb = size_t(g.hidden) * (g.inter / g.group);
    for (int q = 0; q < it.nuse; ++q) {
        const int u = list[it.use0 + q];
        const Use us = uses[u];
        if (us.direct[2] != 1) continue;
        const int k = us.k[2];
        float acc = row_dot(it.planes + g.plane_off[2], g.plane_words,
                            it.levels + g.level_off[2] + level_offset(nb, k), k, o, W,
                            g.group / 32, P.h + size_t(u) * g.inter, (lds_f32*)tabs[threadIdx.x / kWave],
                            lane);
        acc = wave_sum(acc);
        if (lane == kWave - 1) {
            if (yf)    // the routing-weighted combine folded in: y[tok][o] += w * row sum
                __hip_atomic_fetch_add(yf + size_t(us.tok) * g.hidden + o, us.w * acc,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                P.y[size_t(u) * P.dn_smax * g.hidden + o] = acc;
        }
    }
}

// y[t][o] = sum_j w[t][j] * sum_s Y[u][s][o], u = t*top_k + j; tokens
// t0 .. t0 + n_tokens - 1, their weights and slice counts in the arguments.
__global__ __launch_bounds__(kBlock) void combine_k_kernel(const KCombine C) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(C.n_tokens) * C.hidden) return;
    const int t = int(i / C.hidden), o = int(i % C.hidden);
    const int tg = C.t0 + t;
    const float* yt = C.Y + size_t(tg) * C.top_k * C.dn_smax * C.hidden + o;
    const size_t js = size_t(C.dn_smax) * C.hidden;   // between slots
    float acc = 0.f;
    for (int j0 = 0; j0 < C.top_k; j0 += 16) {
        // every slot's first partial in flight at once, then summed in order
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = j0 + q < C.top_k ? yt[(j0 + q) * js] : 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int j = j0 + q;
            if (j >= C.top_k) break;
            const int a = t * C.top_k + j;
            float s = v[q];
            for (int r = 1; r < C.sl[a]; ++r) s += yt[j * js + size_t(r) * C.hidden];
            acc = fmaf(C.w[a], s, acc);
        }
    }
    C.y[size_t(tg) * C.hidden + o] = acc;
}

// y[t][o] = sum_j w[t][j] * sum_s Y[u][s][o], u = t*top_k + j.
__global__ __launch_bounds__(kBlock) void combine_kernel(int n_tokens, int top_k, int hidden,
                                                         const Use* __restrict__ uses, Partials P,
                                                         float* __restrict__ y) {
    const size_t i = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= size_t(n_tokens) * hidden) return;
    const int t = int(i / hidden), o = int(i % hidden);
    float acc = 0.f;
    for (int j = 0; j < top_k; ++j) {
        const int u = t * top_k + j;
        const Use us = uses[u];
        const float* yb = P.y + size_t(u) * P.dn_smax * hidden + o;
        float s = yb[0];
        for (int q = 1; q < us.slices[2]; ++q) s += yb[size_t(q) * hidden];
        acc = fmaf(us.w, s, acc);
    }
    y[i] = acc;
}

// ---------------------------------------------------------------- encoder
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
// fp64 when counts are given (the plain mean for subtrees holding no weight).
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
            float pv = (L + R) * 0.5f;
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

// ---------------------------------------------------------------- checks and baselines
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

// One row of an fp16 weight matrix times x, by one wave (16-byte loads; lane
// sums in column order, then the wave sum).
__device__ inline float row_dot_fp16(const uint16_t* __restrict__ row, int cols,
                                     const float* __restrict__ x, int lane) {
    float acc = 0.f;
    for (int c = lane * 8; c < cols; c += kWave * 8) {
        const uint4 pk = *reinterpret_cast<const uint4*>(row + c);
        const f32x4 xa = *reinterpret_cast<const f32x4*>(x + c);
        const f32x4 xb = *reinterpret_cast<const f32x4*>(x + c + 4);
        const uint32_t q[4] = {pk.x, pk.y, pk.z, pk.w};
        const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __half2float(__ushort_as_half(uint16_t(q[i] & 0xFFFFu)));
            const float hi = __half2float(__ushort_as_half(uint16_t(q[i] >> 16)));
            acc = fmaf(lo, xv[2 * i], acc);
            acc = fmaf(hi, xv[2 * i + 1], acc);
        }
    }
    return wave_sum(acc);
}

__global__ __launch_bounds__(kBlock) void gemv_fp16_kernel(int rows, int cols,
                                                           const uint16_t* __restrict__ w,
                                                           const float* __restrict__ x,
                                                           float* __restrict__ y) {
    const int lane = threadIdx.x % kWave;
    const int o = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= rows) return;
    const float acc = row_dot_fp16(w + size_t(o) * cols, cols, x, lane);
    if (lane == kWave - 1) y[o] = acc;
}

// Matrix blockIdx.y of the batch: row o of its fp16 weights times its x.
__global__ __launch_bounds__(kBlock) void gemv_fp16_batch_kernel(const KGemv16Batch B) {
    const int m = blockIdx.y;
    const int lane = threadIdx.x % kWave;
    const int o = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= B.rows[m]) return;
    const int cols = B.cols[m];
    const float acc = row_dot_fp16(B.w[m] + size_t(o) * cols, cols, B.x[m], lane);
    if (lane == kWave - 1) B.y[m][o] = acc;
}

// Matrix blockIdx.y of the batch in tiles of consecutive weights (a
// workgroup's share of a step, 8 or 16 per thread).  The depth-k tables of
// the blocks a tile touches are one contiguous range of the levels: the
// workgroup stages them in LDS with coalesced loads, then every thread takes
// its weights' k-bit prefixes from one byte (8 weights) or half (16) of each
// plane word, looks their nodes up in LDS (they share a block), rounds them
// to fp16 (nearest even) and stores 16 bytes per 8 weights.
constexpr int kDqStagedK = 5;
// Weights per thread: 16 (half of each plane word) where the tables are
// staged in LDS, 8 (a byte) where they are read from global memory (k > 5):
// the gathers of 16 weights per thread left too few threads in flight.
template <int PER>
constexpr int dq_tile() {
    return kBlock * PER;
}
template <int PER>
__device__ inline void dequant_tiles(const KDequantBatch& B, int m, float* tabs) {
    constexpr int kTile = dq_tile<PER>();
    const int cols = B.cols[m], group = B.group[m], k = B.k[m];
    const uint32_t* __restrict__ pl = B.planes[m];
    const float* __restrict__ lvk = B.lvk[m];
    uint16_t* __restrict__ out = B.w[m];
    const size_t pstride = B.pstride[m];
    const size_t n = size_t(B.rows[m]) * cols;
    const size_t n_tiles = (n + kTile - 1) / kTile;
    const bool staged = k <= kDqStagedK;
    for (size_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const size_t i_begin = t * kTile, i_end = std::min(n, i_begin + kTile);
        // weight i is in block i / group (blocks row-major over (row, group):
        // a row holds a whole number of blocks)
        const size_t b0 = i_begin / group, b1 = (i_end - 1) / group + 1;
        const float* src = lvk + (b0 << k);
        // the plane words first: they do not depend on the staged tables, so
        // their loads and the tables' are in flight together
        const size_t i0 = i_begin + size_t(threadIdx.x) * PER;
        const bool mine = i0 < i_end;
        const size_t word = i0 / 32;
        const int sh = int(i0 % 32);
        uint32_t pw[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) pw[p] = (mine && p < k) ? pl[size_t(p) * pstride + word] : 0u;
        // deep tables are read where they lie: a tile touches a small part
        // of each, and staging them whole would cost more than it saves
        if (staged) {
            const size_t n_tab = (b1 - b0) << k;
#pragma unroll 4
            for (size_t q = threadIdx.x; q < n_tab; q += kBlock) tabs[q] = src[q];
        }
        __syncthreads();
        if (mine) {
            uint32_t v[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) v[j] = 0u;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                if (p >= k) break;
                const uint32_t bits = (pw[p] >> sh) & ((1u << PER) - 1u);
#pragma unroll
                for (int j = 0; j < PER; ++j) v[j] = (v[j] << 1) | ((bits >> j) & 1u);
            }
            // the thread's weights lie in one block (groups are multiples of 32)
            const size_t at = (i0 / group - b0) << k;
            float node[PER];
            if (staged) {
#pragma unroll
                for (int j = 0; j < PER; ++j) node[j] = tabs[at + v[j]];
            } else {
#pragma unroll
                for (int j = 0; j < PER; ++j) node[j] = src[at + v[j]];
            }
#pragma unroll
            for (int h = 0; h < PER / 8; ++h) {
                uint32_t q[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = __half_as_ushort(__float2half_rn(node[8 * h + 2 * j]));
                    const uint32_t hi = __half_as_ushort(__float2half_rn(node[8 * h + 2 * j + 1]));
                    q[j] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4*>(out + i0 + 8 * h) = uint4{q[0], q[1], q[2], q[3]};
            }
        }
        __syncthreads();
    }
}
__global__ __launch_bounds__(kBlock) void dequant_batch_kernel(const KDequantBatch B) {
    extern __shared__ float tabs[];
    const int m = blockIdx.y;
    if (B.k[m] <= kDqStagedK)
        dequant_tiles<16>(B, m, tabs);
    else
        dequant_tiles<8>(B, m, tabs);
}

}  // namespace

hipError_t launch_gemv(int rows, int cols, int group, int k, const uint32_t* planes,
                       size_t pstride, const float* levels, const float* x, float* y,
                       hipStream_t st) {
    hipLaunchKernelGGL(gemv_direct_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(kBlock), 0,
                       st, rows, cols, group, k, planes, pstride, levels, x, y);
    return hipGetLastError();
}

hipError_t launch_direct_gateup(const Geom& g, const Item* items, int n_items, const Use* uses,
                                const int32_t* list, const float* x, Partials P,
                                hipStream_t st, float* zero, int n_zero) {
    if (n_items == 0) return hipSuccess;
    const int bpi = (g.inter + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(direct_gateup_kernel, dim3(n_items * bpi), dim3(kBlock), 0, st, g, items,
                       bpi, uses, list, x, P, zero, n_zero);
    return hipGetLastError();
}

hipError_t launch_direct_down(const Geom& g, const Item* items, int n_items, const Use* uses,
                              const int32_t* list, Partials P, hipStream_t st, float* y_fold) {
    if (n_items == 0) return hipSuccess;
    const int bpi = (g.hidden + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(direct_down_kernel, dim3(n_items * bpi), dim3(kBlock), 0, st, g, items,
                       bpi, uses, list, P, y_fold);
    return hipGetLastError();
}

hipError_t launch_swiglu(const Use* uses, int n_uses, Partials P, int inter, hipStream_t st) {
    hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(size_t(n_uses) * inter, kBlock)),
                       dim3(kBlock), 0, st, uses, n_uses, P, inter);
    return hipGetLastError();
}

hipError_t launch_combine(int n_tokens, int top_k, int hidden, const Use* uses, Partials P,
                          float* y, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(size_t(n_tokens) * hidden, kBlock)),
                       dim3(kBlock), 0, st, n_tokens, top_k, hidden, uses, P, y);
    return hipGetLastError();
}

hipError_t launch_combine_k(const KCombine& C, hipStream_t st) {
    if (C.n_tokens == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_k_kernel, dim3(grid_for(size_t(C.n_tokens) * C.hidden, kBlock)),
                       dim3(kBlock), 0, st, C);
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

hipError_t launch_dequant_batch(const KDequantBatch& B, size_t max_elems, hipStream_t st) {
    if (B.n == 0 || max_elems == 0) return hipSuccess;
    // LDS for the tables of the most blocks a tile can touch, at the deepest
    // staged k (up to 16.5 KiB: group 32 at k = 5, 16 weights per thread)
    size_t lds = 0;
    for (int m = 0; m < B.n; ++m)
        if (B.k[m] <= kDqStagedK)
            lds = std::max(lds, (size_t(dq_tile<16>() / B.group[m] + 1) << B.k[m]) * sizeof(float));
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(dequant_batch_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (attr != hipSuccess) return attr;
    // a workgroup per tile: the hardware starts the next as one ends, which
    // hides the latency of a tile's loads better than a loop over tiles
    const unsigned bx =
        unsigned(std::min<size_t>((max_elems + dq_tile<8>() - 1) / dq_tile<8>(), 1u << 20));
    hipLaunchKernelGGL(dequant_batch_kernel, dim3(bx, unsigned(B.n)), dim3(kBlock), lds, st, B);
    return hipGetLastError();
}

hipError_t launch_gemv_fp16_batch(const KGemv16Batch& B, int max_rows, hipStream_t st) {
    if (B.n == 0 || max_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_fp16_batch_kernel, dim3(grid_for(max_rows, kRowsPerBlock), unsigned(B.n)),
                       dim3(kBlock), 0, st, B);
    return hipGetLastError();
}

hipError_t launch_gemv_fp16(int rows, int cols, const uint16_t* w, const float* x, float* y,
                            hipStream_t st) {
    hipLaunchKernelGGL(gemv_fp16_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(kBlock), 0,
                       st, rows, cols, w, x, y);
    return hipGetLastError();
}

}  // namespace pm
