// The LUT path of libpm for gfx950 (CDNA4, 64-wide wavefronts): a matrix
// executed directly from its k-bit prefix, without ever forming a
// full-precision copy [Abs; T c25, c37] (k <= 5 in a layer, k <= 4 in a single
// GEMV; columns in slices of 1024, rows in steps of 8).
//
// The result of one block of a row is sum_v node[v] * S_v, where S_v is the
// sum of x over the block's weights whose prefix is v.  A weight word (32
// inputs) has prefix v exactly where the AND of the k plane words (each taken
// plain or inverted by the bits of v) is set, and the sum of x under a 32-bit
// mask is four lookups in a table of all 256 subset sums of each 8-input
// chunk of x (an activation lookup table, as in T-MAC).  The table of one
// 1024-column slice is 128 KiB of LDS; every lookup is one v_perm (the mask
// byte becomes the address) and one ds_read.  One lane owns one 128-input
// block of one row: its four plane words arrive as one 16-byte load per plane
// and its 2^k nodes as 16-byte loads, so the codebook enters as one multiply
// per lookup with no cross-lane traffic, and no weight value is ever formed.
// One-hot x gives exact columns.
//
// The sums of a row run in a fixed order (DPP row reductions, slices in
// index order), so every row sum is deterministic; a down launch with the
// combine folded in adds the weighted row sums of the uses into the layer
// output with float atomics, in the order they arrive.  This source is compiled with the
// machine scheduler's ILP strategy (the lookups of a step are kept in
// flight); the other kernels are not.
#include <atomic>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pm_device.h"
#include "pm_internal.h"

namespace pm {

namespace {

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
    float wt;                  // the job's routing weight (a folded down launch)
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
// A workgroup is 16 waves (4 per SIMD): at 126 VGPRs each, enough waves to
// hide the lookups' LDS latency and the loads' HBM latency between them.
#ifndef PM_LUT_THREADS
#define PM_LUT_THREADS 1024
#endif
constexpr int kLutThreads = PM_LUT_THREADS;
constexpr int kLutWaves = kLutThreads / kWave;
constexpr int kLutBytes = 128 * 1024;
// Builder waves: 2 for gate/up (one chunk per thread), 4 for down (half a
// chunk per thread), whose builders also sum the gate/up slices and apply
// SwiGLU before they write.
#ifndef PM_BUILD_WAVES_GU
#define PM_BUILD_WAVES_GU 2
#endif
#ifndef PM_BUILD_WAVES_DN
#define PM_BUILD_WAVES_DN 4
#endif
template <bool DOWN>
constexpr int build_waves() {
    return DOWN ? PM_BUILD_WAVES_DN : PM_BUILD_WAVES_GU;
}
static_assert(build_waves<false>() == 2 || build_waves<false>() == 4, "two or four builder waves");
static_assert(build_waves<true>() == 2 || build_waves<true>() == 4, "two or four builder waves");
static_assert(kLutThreads % 256 == 0 && kLutThreads <= 1024, "whole waves on every SIMD");

__device__ inline int build_chunk(int t) {
    return 16 * ((t & 31) >> 2) + 4 * ((t >> 5) & 3) + (t & 3);
}

// 128 chunks: with 2 builder waves a thread writes all 256 entries of one,
// with 4 waves half of them (PARTS = 2).
template <int PARTS>
__device__ inline void build_table(lds_float* tab, int c, const float (&v)[8], int part) {
    float sub[32];
    sub[0] = 0.f;
#pragma unroll
    for (int i = 1; i < 32; ++i) sub[i] = sub[i & (i - 1)] + v[__builtin_ctz(i)];
#pragma unroll
    for (int q0 = 0; q0 < 8 / PARTS; ++q0) {
        const int q = PARTS == 1 ? q0 : part * (8 / PARTS) + q0;
        float base = 0.f;
        if (q & 1) base += v[5];
        if (q & 2) base += v[6];
        if (q & 4) base += v[7];
#pragma unroll
        for (int i = 0; i < 32; ++i) tab[lut_addr(c, 32 * q + i) >> 2] = base + sub[i];
    }
}

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

// The 8 values of x of token `src` in chunk c of the slice.
__device__ inline void chunk_x(const KLaunch& L, int src, int slice, int c, float (&v)[8],
                               uint32_t* issued) {
    const float* x = L.x + size_t(src) * L.x_stride + kSliceCols * slice + 8 * c;
    const f32x4 a = *(g_f32x4*)x, b = *(g_f32x4*)(x + 4);
    loads_issued(issued);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Down's h = SiLU(g) * u for the slice's columns 4t .. 4t + 3 of use `src`
// (t < 256, one builder thread each): the gate/up partials of those columns
// summed over the slices of each matrix in slice order (slices past a
// matrix's count read slice 0 again and add 0).  The loads are counted on
// `issued` once they are in the memory queue.
__device__ inline f32x4 h_cols(const KLaunch& L, int src, int gsl, int slice, int t,
                               uint32_t* issued) {
    const int ngs = gsl & 15, nus = gsl >> 4;
    const int inter = L.inter, smax = L.gu_smax;
    const int col = kSliceCols * slice + 4 * t;
    const float* pg = L.gu + (size_t(src) * 2) * smax * inter + col;
    const float* pu = pg + size_t(smax) * inter;
    f32x4 gs, us;
    if (smax <= 4) {
        f32x4 gv[4], uv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            gv[q] = *(g_f32x4*)(pg + size_t(q < ngs ? q : 0) * inter);
            uv[q] = *(g_f32x4*)(pu + size_t(q < nus ? q : 0) * inter);
        }
        loads_issued(issued);
        gs = gv[0];
        us = uv[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            gs += q < ngs ? gv[q] : f32x4{0.f, 0.f, 0.f, 0.f};
            us += q < nus ? uv[q] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    } else {
        loads_issued(issued);
        gs = *(g_f32x4*)pg;
        for (int q = 1; q < ngs; ++q) gs += *(g_f32x4*)(pg + size_t(q) * inter);
        us = *(g_f32x4*)pu;
        for (int q = 1; q < nus; ++q) us += *(g_f32x4*)(pu + size_t(q) * inter);
    }
    return f32x4{silu_mul(gs.x, us.x), silu_mul(gs.y, us.y), silu_mul(gs.z, us.z),
                 silu_mul(gs.w, us.w)};
}

// Steps in flight per wave (the ring): two at k = 1, one from k = 2.  With
// 16 waves the first rings alone take about 3 us of HBM; a second step at
// k = 2 made the k = 2 launch 9% slower, at k = 4 a third slower.
#ifndef PM_RING
#define PM_RING 2, 1, 1, 1, 1
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
    int slice, g0, g1;
    int wave, lane;
};

// Workgroup timeline, in a build with PM_LUT_STAMPS only (a profiling build;
// the product build has none of it): s_memrealtime (100 MHz) at the
// workgroup's start (0, once it holds its info word), when the builders hold
// their source values (1), when their table writes are issued (2), when the
// last wave starts to compute (3) and at the end (4); then k (5), steps (6)
// and the XCD (7); then the workgroup's first instruction (8).
// The last launch of each kind (gate/up, down) leaves its stamps.
#ifdef PM_LUT_STAMPS
constexpr int kStampWgs = kMaxLaunchWgq * 16;
constexpr int kStampFields = 12;
__device__ unsigned long long pm_lut_stamps[2][kStampWgs][kStampFields];
#define PM_STAMP(i, v)                                                                      \
    pm_lut_stamps[DOWN][(blockIdx.y * gridDim.x + blockIdx.x) % kStampWgs][i] = (v)
#define PM_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define PM_STAMP(i, v) ((void)0)
#endif

// The builder waves form the table: the slice's activation (x of token
// `src`, or h of use `src`, formed once per column by the builders together
// in LDS behind the table and its counters), then its subset sums, and
// announce it on `ready`.  This needs no more than the workgroup's info word,
// so it starts before the workgroup reads its run.
template <bool DOWN>
__device__ inline void build_lut(const KLaunch& L, int src, int gsl, int slice, lds_float* tab,
                                 uint32_t* ready) {
    constexpr int kBuildWaves = build_waves<DOWN>();
    const int ch = build_chunk(int(threadIdx.x) & 127);
    float v[8];
    if constexpr (!DOWN) {
        chunk_x(L, src, slice, ch, v, ready + 2);
    } else {
        static_assert(build_waves<true>() * kWave * 4 == kSliceCols, "4 columns per builder");
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        lds_float* hb = tab + kLutBytes / 4 + 4;
        const int t = int(threadIdx.x);
        *reinterpret_cast<lds_f32x4*>(hb + 4 * t) = h_cols(L, src, gsl, slice, t, ready + 2);
        __asm__ volatile("" ::: "memory");
        __hip_atomic_fetch_add(ready + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (__hip_atomic_load(ready + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <
               uint32_t(kBuildWaves * kWave))
            __builtin_amdgcn_s_sleep(1);
        __asm__ volatile("" ::: "memory");
        const f32x4 a = *reinterpret_cast<const lds_f32x4*>(hb + 8 * ch);
        const f32x4 b = *reinterpret_cast<const lds_f32x4*>(hb + 8 * ch + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#ifdef PM_LUT_STAMPS
    if (threadIdx.x == 0) {
        // the stamp follows the arrival of the builder's source values
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sum += v[i];
        __asm__ volatile("" ::"v"(sum));
        PM_STAMP(1, PM_NOW());
    }
#endif
    build_table<kBuildWaves / 2>(tab, ch, v, int(threadIdx.x) >> 7);
#ifdef PM_LUT_STAMPS
    if (threadIdx.x == 0) PM_STAMP(2, PM_NOW());
#endif
    // LDS operations of one wave execute in order: once another wave sees
    // this count, the table writes before it are done.  (A release here
    // would also wait for global memory, which this does not need.)
    __asm__ volatile("" ::: "memory");
    __hip_atomic_fetch_add(ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <bool DOWN, bool FOLD, int K>
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
    float cwt = FOLD ? uni_f(L.job[cj].wt) : 0.f;
    const size_t out_off = size_t(c.slice) * L.out_stride;
    auto at = [&](int s) {
        const int gr = c.g0 + 8 * s;
        while (gr >= cend) {
            ++cj;
            cend += rows;
            cpl = uni_ptr(L.job[cj].planes);
            clv = uni_ptr(L.job[cj].lvk);
            cout = uni_ptr(L.job[cj].out);
            if (FOLD) cwt = uni_f(L.job[cj].wt);
        }
        const int row0 = gr - (cend - rows);
        StepAt a;
        a.planes = cpl + size_t(row0) * W + w0;
        a.nodes = clv + ((size_t(row0) * ng + (w0 >> 2)) << K);
        a.out = cout + out_off + row0;
        a.wt = cwt;
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
    constexpr int kBuildWaves = build_waves<DOWN>();
    const bool builder = c.wave < kBuildWaves;
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
#ifdef PM_LUT_STAMPS
    if (threadIdx.x == kWave * (kLutWaves - 1)) PM_STAMP(3, PM_NOW());
#endif
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
            if (FOLD)      // the routing-weighted combine: y[row] += w * row sum
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                    acc * sat[d].wt, buffer_of(sat[d].out, ok ? 32u : 0u), int(so), 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc),
                                                      buffer_of(sat[d].out, ok ? 32u : 0u),
                                                      int(so), 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            fill(d);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (sv[0] >= nsteps) break;
    }
#ifdef PM_LUT_STAMPS
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t xcc;
        __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        PM_STAMP(4, PM_NOW());
        PM_STAMP(5, K);
        PM_STAMP(6, nsteps);
        PM_STAMP(7, xcc);
    }
#endif
}

// Workgroup (q, slice) runs its share of the rows of its run (named in its
// info word, with the run's source): jobs of one prefix and one activation
// source, named in the run's meta with k.  Its builder waves start on the
// table as soon as the info word is read; job descriptions are read straight
// from the argument block.  One workgroup per compute unit (its table fills
// the LDS).
template <bool DOWN, bool FOLD>
__global__ __launch_bounds__(kLutThreads) __attribute__((amdgpu_waves_per_eu(kLutWaves / 4,
                                                                              kLutWaves / 4))) void
lut_kernel(const KLaunch L) {
    // the kernel's one LDS object, at address 0: the lookups use the v_perm
    // result as the address; then the count of builder threads done
#ifdef PM_LUT_STAMPS
    const unsigned long long t_entry = PM_NOW();
#endif
    __shared__ __attribute__((aligned(16))) float lds_buf[kLutBytes / 4 + 4 + (DOWN ? kSliceCols : 0)];
    uint32_t* ready = reinterpret_cast<uint32_t*>(lds_buf + kLutBytes / 4);
    uint32_t* next = ready + 1;
    if (threadIdx.x == 0) {
        *ready = 0u;
        *next = 0u;
        ready[2] = 0u;
        ready[3] = 0u;
    }
    __syncthreads();
    const int q = blockIdx.x, slice = blockIdx.y;
    const uint32_t info = L.wg_info[q];
#ifdef PM_LUT_STAMPS
    if (threadIdx.x == 0) {
        PM_STAMP(0, PM_NOW());
        PM_STAMP(8, t_entry);
    }
#endif
    const int wave = uni(int(threadIdx.x) / kWave);
    if (wave < build_waves<DOWN>())
        build_lut<DOWN>(L, int((info >> 8) & 0xFFFFu), int(info >> 24), slice,
                        (lds_float*)lds_buf, ready);
    // the workgroup's share of its run's steps (an even split)
    const KRun& run = L.run[info & 255u];
    const uint32_t meta = run.meta;
    const int i = q - run.wg0, nwg = run.nwg;
    const int g0 = run.g0 + kLutRows * (run.nsteps * i / nwg);
    const int g1 = run.g0 + kLutRows * (run.nsteps * (i + 1) / nwg);
    if (g0 < g1) {
        LutCtx c{slice, g0, g1, wave, int(threadIdx.x) % kWave};
        switch ((meta >> 16) & 15) {
            case 1: lut_body<DOWN, FOLD, 1>(L, c, (lds_float*)lds_buf, ready, next); break;
            case 2: lut_body<DOWN, FOLD, 2>(L, c, (lds_float*)lds_buf, ready, next); break;
            case 3: lut_body<DOWN, FOLD, 3>(L, c, (lds_float*)lds_buf, ready, next); break;
            case 4: lut_body<DOWN, FOLD, 4>(L, c, (lds_float*)lds_buf, ready, next); break;
            default: lut_body<DOWN, FOLD, 5>(L, c, (lds_float*)lds_buf, ready, next); break;
        }
    }
    if (!DOWN) {
        // clear the output a folded down launch will add into (it runs after
        // this launch on the same stream), last, so that no wait of this
        // launch covers these stores
        const int nz = L.n_zero;
        const int nt = int(gridDim.x * gridDim.y) * kLutThreads;
        for (int j = int(blockIdx.y * gridDim.x + blockIdx.x) * kLutThreads + int(threadIdx.x);
             j < nz; j += nt)
            L.zero[j] = 0.f;
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

}  // namespace

// The LUT launches go through hipModuleLaunchKernel with the argument block
// as one buffer: about 1 us less host time per launch than the triple-chevron
// path, which copies the 4 KiB block through a parameter array.  The kernel
// handles are looked up once per device.
namespace {
constexpr int kMaxDevices = 64;
std::atomic<hipFunction_t> g_lut_fn[kMaxDevices][3];

hipError_t lut_function(int which, hipFunction_t* f) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    hipFunction_t h = g_lut_fn[dev][which].load(std::memory_order_acquire);
    if (!h) {
        const void* sym = which == 0   ? reinterpret_cast<const void*>(lut_kernel<false, false>)
                          : which == 1 ? reinterpret_cast<const void*>(lut_kernel<true, false>)
                                       : reinterpret_cast<const void*>(lut_kernel<true, true>);
        e = hipGetFuncBySymbol(&h, sym);
        if (e != hipSuccess) return e;
        g_lut_fn[dev][which].store(h, std::memory_order_release);
    }
    *f = h;
    return hipSuccess;
}
}  // namespace

hipError_t launch_lut(const KLaunch& L, bool down, hipStream_t st, hipEvent_t t0,
                      hipEvent_t t1) {
    if (L.n_jobs == 0 || L.n_wgq == 0) return hipSuccess;
    hipFunction_t f = nullptr;
    hipError_t e = lut_function(!down ? 0 : L.fold ? 2 : 1, &f);
    if (e != hipSuccess) return e;
    size_t bytes = sizeof(KLaunch);
    void* extra[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, const_cast<KLaunch*>(&L),
                     HIP_LAUNCH_PARAM_BUFFER_SIZE, &bytes, HIP_LAUNCH_PARAM_END};
    if (t0 || t1)
        return hipExtModuleLaunchKernel(f, unsigned(L.n_wgq) * kLutThreads, unsigned(L.S), 1,
                                        kLutThreads, 1, 1, 0, st, nullptr, extra, t0, t1, 0);
    return hipModuleLaunchKernel(f, unsigned(L.n_wgq), unsigned(L.S), 1, kLutThreads, 1, 1, 0,
                                 st, nullptr, extra);
}

hipError_t launch_sum_slices(const float* part, int slices, int rows, float* y, hipStream_t st) {
    hipLaunchKernelGGL(sum_slices_kernel, dim3(grid_for(rows, kBlock)), dim3(kBlock), 0, st, part,
                       slices, rows, y);
    return hipGetLastError();
}

}  // namespace pm

#ifdef PM_LUT_STAMPS
// Copies the stamps of the last gate/up and down launches to host memory
// (2 x 4096 workgroups x 12 uint64) and clears them; a profiling build only.
// Synchronous: call it with no launch in flight.
extern "C" int pm_lut_stamps_fetch(void* host, size_t bytes) {
    if (bytes < sizeof(pm::pm_lut_stamps)) return -1;
    void* dev = nullptr;
    hipError_t e = hipGetSymbolAddress(&dev, HIP_SYMBOL(pm::pm_lut_stamps));
    if (e == hipSuccess) e = hipMemcpy(host, dev, sizeof(pm::pm_lut_stamps), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemset(dev, 0, sizeof(pm::pm_lut_stamps));
    return int(e);
}
#endif
