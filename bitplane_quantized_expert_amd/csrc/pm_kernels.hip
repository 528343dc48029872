// HIP kernels of libpm for gfx950 (CDNA4, 64-wide wavefronts).
//
// Two ways to execute a matrix directly from its k-bit prefix, without ever
// forming a full-precision copy [Abs; T c25, c37]:
//
// LUT path (k <= 5 in a layer, k <= 4 in a single GEMV; columns in slices of
// 1024, rows in steps of 8).  The result of one block of a row is
// sum_v node[v] * S_v, where S_v is the sum of x over the block's weights
// whose prefix is v.  A weight word (32 inputs) has prefix v exactly where the
// AND of the k plane words (each taken plain or inverted by the bits of v) is
// set, and the sum of x under a 32-bit mask is four lookups in a table of all
// 256 subset sums of each 8-input chunk of x (an activation lookup table, as
// in T-MAC).  The table of one 1024-column slice is 128 KiB of LDS; every
// lookup is one v_perm (the mask byte becomes the address) and one ds_read.
// One lane owns one 128-input block of one row: its four plane words arrive
// as one 16-byte load per plane and its 2^k nodes as 16-byte loads, so the
// codebook enters as one multiply per lookup with no cross-lane traffic, and
// no weight value is ever formed.  One-hot x gives exact columns.
//
// Direct path (any k, any shape; an expert of several uses is read once for
// all of them): per weight, the prefix is assembled from the k plane words
// and its node read from the depth-k table, which for group 128 and rows of
// whole 1024-column runs is first staged in LDS (row_dot_lds).
//
// All sums run in a fixed order (DPP row reductions, slices and slots in
// index order), so every output is deterministic.
#include <algorithm>

#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pm_internal.h"

namespace pm {

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kRowsPerBlock = kBlock / kWave;

template <int CTRL, int ROW_MASK>
__device__ inline float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                           false));
}

// Sum over each 16-lane row; every lane of the row gets the row's sum.
__device__ inline float row16_sum(float v) {
    v += dpp<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141, 0xF>(v);   // row_half_mirror
    v += dpp<0x140, 0xF>(v);   // row_mirror
    return v;
}

// Sum over each 32-lane half of the wave; the total lands in lanes 16..31
// (first half) and 48..63 (second half).
__device__ inline float half_sum(float v) {
    v = row16_sum(v);
    v += dpp<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
    return v;
}

// Sum over the wave; the total lands in lane 63.
__device__ inline float wave_sum(float v) {
    v = half_sum(v);
    v += dpp<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
    return v;
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Values the whole wave shares, made explicit so that they live in scalar
// registers: arguments of out-of-line functions and values read from LDS
// arrive in vector registers.
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline uint64_t uni64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return (uint64_t(hi) << 32) | lo;
}
template <class T>
__device__ inline T* uni_ptr(T* p) {
    return reinterpret_cast<T*>(uni64(reinterpret_cast<uint64_t>(p)));
}

// ---------------------------------------------------------------- LUT path
typedef __attribute__((address_space(3))) float lds_float;
// Global-memory views: in out-of-line functions a plain pointer would be
// generic and its loads flat_load, which also count against the LDS wait
// counter and would serialise the prefetch with the table lookups.
typedef __attribute__((address_space(1))) const float g_f32;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
typedef __attribute__((address_space(1))) float g_f32_out;

// LDS table of one 1024-column slice of the activation.  Chunk c = 16g + 4w + b
// covers columns 8c .. 8c + 7 (block g of the slice, word w of the block, byte
// b of the word); its entry for the subset v (bit j of v: column 8c + j) is at
//   (w >> 1) << 16 | v << 8 | (w & 1) << 7 | g << 4 | b << 2.
// The bank of an entry is g << 2 | b.  Lane (r, g) of a wave (row r of the
// step's 8, block g) reads byte (b + r) & 3 of its word at lookup b, so the 32
// lanes of a half-wave (4 rows x 8 blocks) hit 32 different banks whatever the
// mask bytes are.
__device__ inline uint32_t lut_addr(int c, int v) {
    const int g = c >> 4, w = (c >> 2) & 3, b = c & 3;
    return uint32_t(((w >> 1) << 16) | (v << 8) | ((w & 1) << 7) | (g << 4) | (b << 2));
}
__device__ inline float lds_at(uint32_t a) {
    return *reinterpret_cast<const lds_float*>(size_t(a));
}

// Sum over each 8-lane group (the 8 blocks of one row); every lane of the
// group gets it.
__device__ inline float row8_sum(float v) {
    v += dpp<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141, 0xF>(v);   // row_half_mirror
    return v;
}

// Per-lane constants of the lookups: the lane's table slot (block g, byte
// position (b + r) & 3) merged with a mask byte by one v_perm, which drops
// byte (b + r) & 3 of the mask into address bits 8..15 and keeps the slot in
// bits 0..7 and the half (bit 16) from base.  xg: the activation summed over
// the lane's block.
struct LaneLut {
    uint32_t base[2][4];
    uint32_t sel[4];
    float xg;
};

__device__ inline LaneLut lane_lut(int lane, const lds_float* tab) {
    const int g = lane & 7, r = lane >> 3;
    // the table's own address (0: it is the kernel's one LDS object) enters
    // the lookup addresses, so the compiler keeps the stores that build it
    const uint32_t t0 = uint32_t(reinterpret_cast<uintptr_t>(tab));
    LaneLut L;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t bb = uint32_t((b + r) & 3);
        L.sel[b] = 0x0C060004u | (bb << 8);
        L.base[0][b] = t0 + (uint32_t(g << 4) | (bb << 2));
        L.base[1][b] = L.base[0][b] | 0x10000u;
    }
    float xg = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) xg += tab[lut_addr(16 * g + c, 255) >> 2];
    L.xg = xg;
    return L;
}

// One step of a wave: 8 rows of one matrix over one column slice.  Lane
// (r, g) holds the four plane words of block g of row r for planes 0..K-1 and
// the block's 2^K depth-K node values.
template <int K>
struct StepIn {
    u32x4 p[K];
    f32x4 n[K == 1 ? 1 : (1 << K) / 4];
};

// Buffer resource over `bytes` bytes from p: loads take a wave-uniform byte
// offset (scalar) plus the lane's byte offset, and return 0 past the end.
__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), 0x00020000);
}

// Where a step reads and writes.  planes: plane 0, row 0 of the step, first
// word of the slice; nodes: depth-K nodes of the slice's first block, row 0
// of the step; out: the slice partial of row 0 of the step.
struct StepAt {
    const uint32_t* planes;
    const float* nodes;
    float* out;
};

// Lane byte offsets that stay fixed through a launch: the plane words and
// the node values of (row r, block g) from the step's row 0.
struct LaneOff {
    uint32_t pw, nd;
};

// Plane words are read once per launch: non-temporal loads (the "nt" cache
// policy; on gfx950 a stream of them reaches about 7.3 TB/s, plain loads
// about 4 TB/s).  Node loads keep the default policy: from k = 3 a lane's
// nodes span 32-64 bytes, so one load instruction touches lines that the
// lane's next node loads read again.
constexpr int kNT = 2;
constexpr int kNodePolicy = 0;

// A step past the end (ok false) still issues its loads, against an empty
// buffer (they return 0 and read nothing), so that every wave issues the
// same loads in the same order and the waits on them stay exact.
template <int K>
__device__ inline void step_load(StepIn<K>& in, const StepAt& at, const LaneOff& lo,
                                 uint32_t pstride_b, uint32_t row_b, uint32_t nrow_b, bool ok) {
    const __amdgpu_buffer_rsrc_t rp =
        buffer_of(at.planes, ok ? uint32_t(K - 1) * pstride_b + 8u * row_b : 0u);
    const __amdgpu_buffer_rsrc_t rn = buffer_of(at.nodes, ok ? 8u * nrow_b : 0u);
#pragma unroll
    for (int p = 0; p < K; ++p)
        in.p[p] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, int(lo.pw), int(p * pstride_b), kNT));
    if constexpr (K == 1) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rn, int(lo.nd), 0, kNodePolicy);
        const f32x2 f = __builtin_bit_cast(f32x2, v);
        in.n[0] = f32x4{f.x, f.y, 0.f, 0.f};
    } else {
#pragma unroll
        for (int i = 0; i < (1 << K) / 4; ++i)
            in.n[i] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, int(lo.nd + 16 * i), 0, kNodePolicy));
    }
}

// The row's contribution of this lane's block at prefix K:
//   sum_v node[v] * S_v,  S_v = sum of x over the block's inputs with prefix v.
// S_v for v != M is the four lookups per word of the mask of prefix v (the
// AND of the K plane words, each plain or inverted by the bits of v); S_M is
// what remains of the block's activation sum X.  M is a middle bucket (0 at
// K = 1): the nodes are ascending, so node[M] is the value nearest the
// block's median and the rounding of X - sum S_v, scaled by node[M], stays
// within a small multiple of sum |w * x| also for codebooks with large outer
// leaves.  One-hot x gives exact columns: every S_v is 0 or 1.
template <int K>
__device__ inline float step_compute(const StepIn<K>& in, const LaneLut& L) {
    constexpr int NV = 1 << K;
    constexpr int M = K == 1 ? 0 : NV / 2;
    // accumulators per bucket: four (one per lookup byte) at K = 1, where a
    // single bucket would be one long dependent chain
    constexpr int J = K == 1 ? 4 : 1;
    // a scheduling region is RW words x CB buckets: its lookups are issued
    // together and summed before the next region starts (larger regions would
    // not fit the registers)
    constexpr int RW = K <= 2 ? 4 : (K == 3 ? 2 : 1);
    constexpr int CB = K <= 4 ? NV : 8;
    float S[NV][J];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < J; ++j) S[v][j] = 0.f;
#pragma unroll
    for (int w0 = 0; w0 < 4; w0 += RW) {
#pragma unroll
        for (int v0 = 0; v0 < NV; v0 += CB) {
#pragma unroll
            for (int w = w0; w < w0 + RW; ++w) {
                uint32_t pw[K];
#pragma unroll
                for (int p = 0; p < K; ++p) pw[p] = in.p[p][w];
                // masks of the 3-bit prefixes (deeper prefixes refine them)
                uint32_t l3[8];
                if constexpr (K > 3) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        l3[u] = ((u & 4) ? pw[0] : ~pw[0]) & ((u & 2) ? pw[1] : ~pw[1]) &
                                ((u & 1) ? pw[2] : ~pw[2]);
                }
#pragma unroll
                for (int v = v0; v < v0 + CB; ++v) {
                    if (v == M) continue;
                    uint32_t m;
                    if constexpr (K <= 3) {
                        m = 0xFFFFFFFFu;
#pragma unroll
                        for (int p = 0; p < K; ++p)
                            m &= ((v >> (K - 1 - p)) & 1) ? pw[p] : ~pw[p];
                    } else {
                        m = l3[v >> (K - 3)];
#pragma unroll
                        for (int p = 3; p < K; ++p)
                            m &= ((v >> (K - 1 - p)) & 1) ? pw[p] : ~pw[p];
                    }
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t a = __builtin_amdgcn_perm(L.base[w >> 1][b], m, L.sel[b]);
                        S[v][b % J] += lds_at(a + 128u * (w & 1));
                    }
                }
            }
            // the region's sums complete inside it (otherwise they sink to the
            // end of the step and every lookup result stays live)
#pragma unroll
            for (int v = v0; v < v0 + CB; ++v)
#pragma unroll
                for (int j = 0; j < J; ++j)
                    if (v != M) __asm__ volatile("" : "+v"(S[v][j]));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float Sv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        if constexpr (J == 4)
            Sv[v] = (S[v][0] + S[v][1]) + (S[v][2] + S[v][3]);
        else
            Sv[v] = S[v][0];
    }
    float rest = L.xg;
#pragma unroll
    for (int v = 0; v < NV; ++v)
        if (v != M) rest -= Sv[v];
    Sv[M] = rest;
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) acc = fmaf(in.n[v >> 2][v & 3], Sv[v], acc);
    return acc;
}

// Table build by the builder waves: thread t (t < 128) owns chunk
// c = 16g + 4w + b with g << 2 | b = t % 32, w = t / 32, and writes all 256
// subset sums of it; a half-wave writes 32 different banks.  Each entry is a
// plain fp32 sum of its columns (a zero term adds nothing, so one-hot x gives
// exact columns).
#ifndef PM_LUT_THREADS
#define PM_LUT_THREADS 512
#endif
constexpr int kLutThreads = PM_LUT_THREADS;
constexpr int kLutWaves = kLutThreads / kWave;
constexpr int kLutBytes = 128 * 1024;
#ifndef PM_BUILD_WAVES
#define PM_BUILD_WAVES 2
#endif
// 128 chunks: one per builder thread (2 waves) or half of one (4 waves)
constexpr int kBuildWaves = PM_BUILD_WAVES;
constexpr int kBuildParts = kBuildWaves / 2;
static_assert(kBuildWaves == 2 || kBuildWaves == 4, "two or four builder waves");
static_assert(kLutThreads % 256 == 0 && kLutThreads <= 1024, "whole waves on every SIMD");

__device__ inline int build_chunk(int t) {
    return 16 * ((t & 31) >> 2) + 4 * ((t >> 5) & 3) + (t & 3);
}

__device__ inline void build_table(lds_float* tab, int c, const float (&v)[8], int part) {
    float sub[32];
    sub[0] = 0.f;
#pragma unroll
    for (int i = 1; i < 32; ++i) sub[i] = sub[i & (i - 1)] + v[__builtin_ctz(i)];
#pragma unroll
    for (int q0 = 0; q0 < 8 / kBuildParts; ++q0) {
        const int q = kBuildParts == 1 ? q0 : part * (8 / kBuildParts) + q0;
        float base = 0.f;
        if (q & 1) base += v[5];
        if (q & 2) base += v[6];
        if (q & 4) base += v[7];
#pragma unroll
        for (int i = 0; i < 32; ++i) tab[lut_addr(c, 32 * q + i) >> 2] = base + sub[i];
    }
}

// The 8 activation values of chunk c: x of token `src`, or h of use `src`
// formed from its gate/up partials (slices summed in order; slices past a
// matrix's count read slice 0 again and add 0).
#ifndef PM_X_FIRST
#define PM_X_FIRST 1
#endif
// Count a builder wave's source loads as issued (on `issued`, in LDS): the
// other waves hold their first plane loads back until every builder wave's
// are in the queue, so that the table does not wait behind them.
__device__ inline void loads_issued(uint32_t* issued) {
    if constexpr (PM_X_FIRST) {
        __builtin_amdgcn_sched_barrier(0);
        __hip_atomic_fetch_add(issued, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool DOWN>
__device__ inline void chunk_source(const KLaunch& L, int src, int gsl, int slice, int c,
                                    float (&v)[8], uint32_t* issued) {
    const int col = kSliceCols * slice + 8 * c;
    if constexpr (!DOWN) {
        const float* x = L.x + size_t(src) * L.x_stride + col;
        const f32x4 a = *(g_f32x4*)x, b = *(g_f32x4*)(x + 4);
        loads_issued(issued);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const int ngs = gsl & 15, nus = gsl >> 4;
        const int inter = L.inter, smax = L.gu_smax;
        const float* pg = L.gu + (size_t(src) * 2) * smax * inter + col;
        const float* pu = pg + size_t(smax) * inter;
        f32x4 gs[2], us[2];
        if (smax <= 4) {
            f32x4 gv[4][2], uv[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    gv[q][h] = *(g_f32x4*)(pg + size_t(q < ngs ? q : 0) * inter + 4 * h);
                    uv[q][h] = *(g_f32x4*)(pu + size_t(q < nus ? q : 0) * inter + 4 * h);
                }
            loads_issued(issued);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                gs[h] = gv[0][h];
                us[h] = uv[0][h];
#pragma unroll
                for (int q = 1; q < 4; ++q) {
                    gs[h] += q < ngs ? gv[q][h] : f32x4{0.f, 0.f, 0.f, 0.f};
                    us[h] += q < nus ? uv[q][h] : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        } else {
            loads_issued(issued);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                gs[h] = *(g_f32x4*)(pg + 4 * h);
                for (int q = 1; q < ngs; ++q) gs[h] += *(g_f32x4*)(pg + size_t(q) * inter + 4 * h);
                us[h] = *(g_f32x4*)(pu + 4 * h);
                for (int q = 1; q < nus; ++q) us[h] += *(g_f32x4*)(pu + size_t(q) * inter + 4 * h);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = silu_mul(gs[0][i], us[0][i]);
            v[4 + i] = silu_mul(gs[1][i], us[1][i]);
        }
    }
}

// Steps in flight per wave (the ring): deeper where a step is short.
#ifndef PM_RING
#define PM_RING 4, 3, 2, 2, 2
#endif
constexpr int kRing[5] = {PM_RING};
template <int K>
constexpr int lut_ring() {
    return kRing[K - 1];
}

// The rows [g0, g1) of a launch (row r of job j is j * rows + r; both ends
// multiples of 8) over column slice `slice`, every job at prefix K and of
// activation source `src`, in 8-row steps.  Each wave keeps D steps in
// flight, also across job boundaries.  The builder waves form the table while
// the others already stream their first steps (a wave stalls at issue once
// its compute unit's vector-memory queue is full, so waves that issue loads
// early must not be the ones that build).
struct LutCtx {
    int slice, g0, g1, src, gsl;
    int wave, lane;
};

template <bool DOWN, int K>
__device__ __attribute__((always_inline)) inline void lut_body(const KLaunch& L, LutCtx c,
                                                               lds_float* tab, uint32_t* ready,
                                                               uint32_t* next) {
    const int lane = c.lane, r = lane >> 3, g = lane & 7;
    const int rows = uni(L.rows), W = uni(L.W);
    const int ng = W / 4;                                  // blocks per row
    const uint32_t pstride_b = uni(uint32_t(L.pstride * 4u));
    const uint32_t row_b = uint32_t(W) * 4u;               // bytes per plane row
    const uint32_t nrow_b = uint32_t(ng << K) * 4u;        // node bytes per row
    const LaneOff lo{uint32_t(r * W + 4 * g) * 4u, uint32_t((r * ng + g) << K) * 4u};
    const int nsteps = (c.g1 - c.g0) / 8;
    const int w0 = (kSliceCols / 32) * c.slice;            // first word of the slice
    // a wave's steps only move forward: a cursor on the current job reads a
    // job description only when a step crosses into the next job
    int cj = c.g0 / rows;                                  // current job
    int cend = (cj + 1) * rows;                            // its end in the row sequence
    const uint32_t* cpl = uni_ptr(L.job[cj].planes);
    const float* clv = uni_ptr(L.job[cj].lvk);
    float* cout = uni_ptr(L.job[cj].out);
    const size_t out_off = size_t(c.slice) * L.out_stride;
    auto at = [&](int s) {
        const int gr = c.g0 + 8 * s;
        while (gr >= cend) {
            ++cj;
            cend += rows;
            cpl = uni_ptr(L.job[cj].planes);
            clv = uni_ptr(L.job[cj].lvk);
            cout = uni_ptr(L.job[cj].out);
        }
        const int row0 = gr - (cend - rows);
        StepAt a;
        a.planes = cpl + size_t(row0) * W + w0;
        a.nodes = clv + ((size_t(row0) * ng + (w0 >> 2)) << K);
        a.out = cout + out_off + row0;
        return a;
    };
    constexpr int D = lut_ring<K>();
    StepIn<K> buf[D];
    StepAt sat[D];
    int sv[D];                 // the step in ring slot d (nsteps or more: none)
    // steps are handed out in order from an LDS counter, one per slot refill,
    // so waves that start late (the builders) or run slower take fewer
    auto grab = [&]() {
        uint32_t t = 0;
        if (lane == 0) t = __hip_atomic_fetch_add(next, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
        return int(__builtin_amdgcn_readfirstlane(t));
    };
    auto fill = [&](int d) {
        sv[d] = grab();
        const bool ok = sv[d] < nsteps;
        sat[d] = at(ok ? sv[d] : nsteps - 1);
        step_load<K>(buf[d], sat[d], lo, pstride_b, row_b, nrow_b, ok);
    };
    // builders form the table and announce it on `ready`; the other waves
    // take their first step at once and wait for the table only when they
    // are about to compute (no workgroup barrier: a wave stalled at issue
    // must not hold up the others)
    const bool builder = c.wave < kBuildWaves;
    if (builder) {
        const int ch = build_chunk(int(threadIdx.x) & 127);
        float v[8];
        chunk_source<DOWN>(L, c.src, c.gsl, c.slice, ch, v, ready + 2);
        build_table(tab, ch, v, int(threadIdx.x) >> 7);
        // LDS operations of one wave execute in order: once another wave
        // sees this count, the table writes before it are done.  (A release
        // here would also wait for global memory, which this does not need.)
        __asm__ volatile("" ::: "memory");
        __hip_atomic_fetch_add(ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (PM_X_FIRST && !builder) {
        while (__hip_atomic_load(ready + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <
               uint32_t(kBuildWaves * kWave))
            __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) fill(d);
    __builtin_amdgcn_sched_barrier(0);
    while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <
           uint32_t(kBuildWaves * kWave))
        __builtin_amdgcn_s_sleep(1);
    __asm__ volatile("" ::: "memory");
    const LaneLut LL = lane_lut(lane, tab);

    // Slots are filled in step order, so once the first slot of a round
    // holds no step, none does.  Every wave issues the same vector-memory
    // operations in the same order, with no branch around any of them (a
    // step past the end loads from and stores to an empty buffer; lanes
    // other than the first of a row store out of range), so the compiler's
    // waits on them stay exact.  The scheduling barriers keep the loads ahead
    // of the next step's arithmetic.
    const uint32_t so = g == 0 ? uint32_t(r) * 4u : 64u;
    for (;;) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const bool ok = sv[d] < nsteps;
            float acc = 0.f;
            if (ok) acc = row8_sum(step_compute<K>(buf[d], LL));
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc),
                                                  buffer_of(sat[d].out, ok ? 32u : 0u),
                                                  int(so), 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            fill(d);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (sv[0] >= nsteps) break;
    }
}

// Workgroup (q, slice) runs the rows [start[q], start[q + 1]) of the
// launch's row sequence; the host cuts them so that every range holds jobs of
// one prefix and one activation source, named in meta[q] with the range's k,
// so that a workgroup's first reads do not depend on one another.  Job
// descriptions are read straight from the argument block.
// One workgroup per compute unit (its table fills the LDS).
template <bool DOWN>
__global__ __launch_bounds__(kLutThreads) __attribute__((amdgpu_waves_per_eu(kLutWaves / 4,
                                                                              kLutWaves / 4))) void
lut_kernel(const KLaunch L) {
    // the kernel's one LDS object, at address 0: the lookups use the v_perm
    // result as the address; then the count of builder threads done
    __shared__ __attribute__((aligned(16))) float lds_buf[kLutBytes / 4 + 4];
    uint32_t* ready = reinterpret_cast<uint32_t*>(lds_buf + kLutBytes / 4);
    uint32_t* next = ready + 1;
    if (threadIdx.x == 0) {
        *ready = 0u;
        *next = 0u;
        ready[2] = 0u;
    }
    __syncthreads();
    const int q = blockIdx.x, slice = blockIdx.y;
    const uint32_t meta = L.meta[q];
    const int g0 = L.start[q], g1 = L.start[q + 1];
    if (g0 >= g1) return;
    LutCtx c{slice, g0, g1, int(meta & 0xFFFFu), int(meta >> 24),
             uni(int(threadIdx.x) / kWave), int(threadIdx.x) % kWave};
    switch ((meta >> 16) & 15) {
        case 1: lut_body<DOWN, 1>(L, c, (lds_float*)lds_buf, ready, next); break;
        case 2: lut_body<DOWN, 2>(L, c, (lds_float*)lds_buf, ready, next); break;
        case 3: lut_body<DOWN, 3>(L, c, (lds_float*)lds_buf, ready, next); break;
        case 4: lut_body<DOWN, 4>(L, c, (lds_float*)lds_buf, ready, next); break;
#if PM_LUT_THREADS == 512
        default: lut_body<DOWN, 5>(L, c, (lds_float*)lds_buf, ready, next); break;
#endif
    }
}

__global__ __launch_bounds__(kBlock) void sum_slices_kernel(const float* __restrict__ part,
                                                            int slices, int rows,
                                                            float* __restrict__ y) {
    const int r = blockIdx.x * kBlock + threadIdx.x;
    if (r >= rows) return;
    float s = part[r];
    for (int q = 1; q < slices; ++q) s += part[size_t(q) * rows + r];
    y[r] = s;
}

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
                                                               Partials P) {
    __shared__ float tabs[kRowsPerBlock][kRunTabFloatsMax];
    const Item it = items[blockIdx.x / bpi];
    const int lane = threadIdx.x % kWave;
    const int o = (blockIdx.x % bpi) * kRowsPerBlock + threadIdx.x / kWave;
    if (o >= g.inter) return;
    const int W = g.hidden / 32;
    const size_t nb = size_t(g.inter) * (g.hidden / g.group);
    // one (use, matrix) per step; fields read from memory by index, so no
    // copy of the use record is indexed in registers
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
        if (lane == kWave - 1) P.gu[(size_t(u) * 2 + m) * P.gu_smax * g.inter + o] = acc;
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
    if (!us.direct[2]) return;                   // h of the direct and tile paths
    P.h[i] = silu_mul(gu_sum(P, us, u, 0, inter, c), gu_sum(P, us, u, 1, inter, c));
}

__global__ __launch_bounds__(kBlock) void direct_down_kernel(Geom g, const Item* __restrict__ items,
                                                             int bpi,
                                                             const Use* __restrict__ uses,
                                                             const int32_t* __restrict__ list,
                                                             Partials P) {
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
        if (lane == kWave - 1) P.y[size_t(u) * P.dn_smax * g.hidden + o] = acc;
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

// Matrix blockIdx.y of the batch in tiles of kDqTile consecutive weights (a
// workgroup's share of a step, 8 per thread).  The depth-k tables of the
// blocks a tile touches are one contiguous range of the levels: the
// workgroup stages them in LDS with coalesced loads, then every thread takes
// its 8 weights' k-bit prefixes from one byte of each plane word, looks their
// nodes up in LDS (the 8 share a block), rounds them to fp16 (nearest even)
// and stores 16 bytes.
constexpr int kDqTile = kBlock * 8;
constexpr int kDqStagedK = 5;
__global__ __launch_bounds__(kBlock) void dequant_batch_kernel(const KDequantBatch B) {
    extern __shared__ float tabs[];
    const int m = blockIdx.y;
    const int cols = B.cols[m], group = B.group[m], k = B.k[m];
    const uint32_t* __restrict__ pl = B.planes[m];
    const float* __restrict__ lvk = B.lvk[m];
    uint16_t* __restrict__ out = B.w[m];
    const size_t pstride = B.pstride[m];
    const size_t n = size_t(B.rows[m]) * cols;
    const size_t n_tiles = (n + kDqTile - 1) / kDqTile;
    for (size_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const size_t i_begin = t * kDqTile, i_end = std::min(n, i_begin + kDqTile);
        // weight i is in block i / group (blocks row-major over (row, group):
        // a row holds a whole number of blocks)
        const size_t b0 = i_begin / group, b1 = (i_end - 1) / group + 1;
        const float* src = lvk + (b0 << k);
        // deep tables are read where they lie: a tile touches a small part
        // of each, and staging them whole would cost more than it saves
        const bool staged = k <= kDqStagedK;
        if (staged) {
            const size_t n_tab = (b1 - b0) << k;
            for (size_t q = threadIdx.x; q < n_tab; q += kBlock) tabs[q] = src[q];
        }
        __syncthreads();
        const size_t i0 = i_begin + size_t(threadIdx.x) * 8;
        if (i0 < i_end) {
            const size_t word = i0 / 32;
            const int sh = int(i0 % 32);
            uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int p = 0; p < k; ++p) {
                const uint32_t bits = (pl[size_t(p) * pstride + word] >> sh) & 0xFFu;
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (v[j] << 1) | ((bits >> j) & 1u);
            }
            const size_t at = (i0 / group - b0) << k;
            float node[8];
            if (staged) {
#pragma unroll
                for (int j = 0; j < 8; ++j) node[j] = tabs[at + v[j]];
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) node[j] = src[at + v[j]];
            }
            uint32_t q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = __half_as_ushort(__float2half_rn(node[2 * j]));
                const uint32_t hi = __half_as_ushort(__float2half_rn(node[2 * j + 1]));
                q[j] = lo | (hi << 16);
            }
            *reinterpret_cast<uint4*>(out + i0) = uint4{q[0], q[1], q[2], q[3]};
        }
        __syncthreads();
    }
}

inline unsigned grid_for(size_t n, int per) { return unsigned((n + per - 1) / per); }

}  // namespace

hipError_t launch_gemv(int rows, int cols, int group, int k, const uint32_t* planes,
                       size_t pstride, const float* levels, const float* x, float* y,
                       hipStream_t st) {
    hipLaunchKernelGGL(gemv_direct_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(kBlock), 0,
                       st, rows, cols, group, k, planes, pstride, levels, x, y);
    return hipGetLastError();
}

hipError_t launch_lut(const KLaunch& L, bool down, hipStream_t st, hipEvent_t t0,
                      hipEvent_t t1) {
    if (L.n_jobs == 0 || L.n_wgq == 0) return hipSuccess;
    const dim3 grid(unsigned(L.n_wgq), unsigned(L.S));
    if (t0 || t1) {
        if (down)
            hipExtLaunchKernelGGL(lut_kernel<true>, grid, dim3(kLutThreads), 0, st, t0, t1, 0, L);
        else
            hipExtLaunchKernelGGL(lut_kernel<false>, grid, dim3(kLutThreads), 0, st, t0, t1, 0, L);
    } else if (down) {
        hipLaunchKernelGGL(lut_kernel<true>, grid, dim3(kLutThreads), 0, st, L);
    } else {
        hipLaunchKernelGGL(lut_kernel<false>, grid, dim3(kLutThreads), 0, st, L);
    }
    return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, int slices, int rows, float* y, hipStream_t st) {
    hipLaunchKernelGGL(sum_slices_kernel, dim3(grid_for(rows, kBlock)), dim3(kBlock), 0, st, part,
                       slices, rows, y);
    return hipGetLastError();
}

hipError_t launch_direct_gateup(const Geom& g, const Item* items, int n_items, const Use* uses,
                                const int32_t* list, const float* x, Partials P,
                                hipStream_t st) {
    if (n_items == 0) return hipSuccess;
    const int bpi = (g.inter + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(direct_gateup_kernel, dim3(n_items * bpi), dim3(kBlock), 0, st, g, items,
                       bpi, uses, list, x, P);
    return hipGetLastError();
}

hipError_t launch_direct_down(const Geom& g, const Item* items, int n_items, const Use* uses,
                              const int32_t* list, Partials P, hipStream_t st) {
    if (n_items == 0) return hipSuccess;
    const int bpi = (g.hidden + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(direct_down_kernel, dim3(n_items * bpi), dim3(kBlock), 0, st, g, items,
                       bpi, uses, list, P);
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
    // staged k (up to 8.1 KiB: group 32 at k = 5)
    size_t lds = 0;
    for (int m = 0; m < B.n; ++m)
        if (B.k[m] <= kDqStagedK)
            lds = std::max(lds, (size_t(kDqTile / B.group[m] + 1) << B.k[m]) * sizeof(float));
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(dequant_batch_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (attr != hipSuccess) return attr;
    // a workgroup per tile: the hardware starts the next as one ends, which
    // hides the latency of a tile's loads better than a loop over tiles
    const unsigned bx = unsigned(std::min<size_t>((max_elems + kDqTile - 1) / kDqTile, 1u << 20));
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
