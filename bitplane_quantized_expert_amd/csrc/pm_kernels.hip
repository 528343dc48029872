// HIP kernels of libpm for gfx950 (CDNA4, 64-wide wavefronts).
//
// Two ways to execute a matrix directly from its k-bit prefix, without ever
// forming a full-precision copy [Abs; T c25, c37]:
//
// LUT path (k <= 5 in a layer, k <= 4 in a single GEMV; columns in slices of
// 1024).  The result of one block of a row is sum_v node[v] * S_v, where S_v
// is the sum of x over the block's weights whose prefix is v.  A weight word (32 inputs) has prefix v exactly
// where the AND of the k plane words (each taken plain or inverted by the
// bits of v) is set, and the sum of x under a 32-bit mask is four lookups in
// a table of all 256 subset sums of each 8-input chunk of x (an activation
// lookup table, as in T-MAC).  The table of one 1024-column slice is 128 KiB
// of LDS; every lookup is one v_perm (the mask byte becomes the address) and
// one ds_read.  2^k - 1 masks per word, the last bucket by subtraction from
// the word's total.  The codebook enters as 2^k FMAs per block and row, so no
// weight value is ever formed.  One-hot x gives exact columns.
//
// Direct path (any k, any shape; an expert of several uses is read once for
// all of them): per weight, the prefix is assembled from the k plane words
// and its node read from the depth-k table, which for group 128 and rows of
// whole 1024-column runs is first staged in LDS (row_dot_lds).
//
// All sums run in a fixed order (DPP row reductions, slices and slots in
// index order), so every output is deterministic.
#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pm_internal.h"

namespace pm {

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kRowsPerBlock = kBlock / kWave;
#ifndef PM_LUT_THREADS
#define PM_LUT_THREADS 1024
#endif
constexpr int kLutThreads = PM_LUT_THREADS;
constexpr int kLutWaves = kLutThreads / kWave;
constexpr int kLutBytes = 128 * 1024;
constexpr int kHbufBytes = (kSliceCols + kSliceCols / 32) * 4;

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
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;
// Global-memory views: in out-of-line functions a plain pointer would be
// generic and its loads flat_load, which also count against the LDS wait
// counter and would serialise the prefetch with the table lookups.
typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef __attribute__((address_space(1))) const float g_f32;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const f32x2 g_f32x2;
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
typedef __attribute__((address_space(1))) float g_f32_out;

// LDS layout of the activation table of one 1024-column slice: chunk c (8
// columns 8c..8c+7), byte value b (a subset of the chunk), t = c & 3,
// l = c >> 2 (the word of the slice the chunk belongs to):
//   address = (t >> 1) << 16 | b << 8 | (l + 32 * (t & 1)) << 2.
// Lane l of a half-wave reads chunks 4l..4l+3; at every lookup the 32 lanes of
// a half-wave touch 32 different banks.
__device__ inline uint32_t lut_addr(int c, int b) {
    const int t = c & 3, l = c >> 2;
    return uint32_t(((t >> 1) << 16) | (b << 8) | ((l + 32 * (t & 1)) << 2));
}

// Sum of x over the set bits of mask m for lane word l: four lookups, each a
// v_perm (mask byte -> address bits 8..15 over the lane's base b0 / b1) and a
// ds_read.  The table sits at LDS address 0, so the perm result is the
// address and the +128 of odd chunks is the instruction's offset.
__device__ inline float lds_at(uint32_t a) {
    return *reinterpret_cast<const lds_float*>(size_t(a));
}
__device__ inline void lds_put(uint32_t a, float v) {
    *reinterpret_cast<lds_float*>(size_t(a)) = v;
}
__device__ inline float lut_sum(uint32_t m, uint32_t b0, uint32_t b1) {
    const uint32_t a0 = __builtin_amdgcn_perm(b0, m, 0x0C060004u);
    const uint32_t a1 = __builtin_amdgcn_perm(b0, m, 0x0C060104u);
    const uint32_t a2 = __builtin_amdgcn_perm(b1, m, 0x0C060204u);
    const uint32_t a3 = __builtin_amdgcn_perm(b1, m, 0x0C060304u);
    float s = lds_at(a0);
    s += lds_at(a1 + 128);
    s += lds_at(a2);
    s += lds_at(a3 + 128);
    return s;
}

// Masks of the prefix tree of one word, depth first: leaf V (D == K) gets the
// mask of the weights whose prefix is V.  Leaf 2^K - 1 is not needed (its sum
// comes by subtraction from the word's total).
template <int K, int D, int V>
struct PrefixMasks {
    static __device__ inline void go(const uint32_t (&w)[K], uint32_t m,
                                     uint32_t (&out)[(1 << K) - 1]) {
        PrefixMasks<K, D + 1, 2 * V>::go(w, m & ~w[D], out);
        PrefixMasks<K, D + 1, 2 * V + 1>::go(w, m & w[D], out);
    }
};
template <int K, int V>
struct PrefixMasks<K, K, V> {
    static __device__ inline void go(const uint32_t (&)[K], uint32_t m,
                                     uint32_t (&out)[(1 << K) - 1]) {
        if constexpr (V != (1 << K) - 1) out[V] = m;
    }
};

// Floats of a block's depth-K table held by each lane of the block's four
// lanes (a block is 128 inputs, four 32-bit words): lane q of the quad holds
// values q*NQ .. q*NQ + NQ - 1 (K = 1: lane q holds value q & 1).
template <int K>
constexpr int quad_share() {
    return (1 << K) >= 4 ? (1 << K) / 4 : 1;
}

// Node value V of this lane's block, from the quad lane that holds it.
template <int K, int V>
__device__ inline float quad_node(const float (&tq)[quad_share<K>()]) {
    constexpr int NQ = quad_share<K>();
    constexpr int owner = K == 1 ? V : V / NQ;
    constexpr int j = K == 1 ? 0 : V % NQ;
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, tq[j]), owner * 0x55, 0xF, 0xF,
                                        true));
}

// One row's contribution of this lane's word at prefix K:
// sum_v node(v) * S_v, S_v = sum of x where the prefix is v.  The buckets go
// in chunks of PM_LUT_CHUNK: a chunk's masks, then all its lookups (one LDS
// round trip), then its bucket sums in v order, each taken off the word's
// total xw; the last bucket is what remains.  Chunks keep the k = 4 and 5 rows
// within the register budget of four waves per SIMD (all 2^k - 1 lookups at
// once spilled); the order of the sums is the same for any chunk size.
#ifndef PM_LUT_CHUNK
#define PM_LUT_CHUNK 8
#endif
// Bucket V (V0 <= V < V1) of one row: its sum S from the four chunk lookups
// (in chunk order), taken off the running remainder, times node V.
template <int K, int V, int V0, int V1>
__device__ inline void lut_terms(const float* r, const float (&tq)[quad_share<K>()], float& acc,
                                 float& last) {
    if constexpr (V < V1) {
        float S = r[4 * (V - V0)];
        S += r[4 * (V - V0) + 1];
        S += r[4 * (V - V0) + 2];
        S += r[4 * (V - V0) + 3];
        last -= S;
        acc = fmaf(quad_node<K, V>(tq), S, acc);
        lut_terms<K, V + 1, V0, V1>(r, tq, acc, last);
    }
}
// The masks of leaves V0 .. V1 - 1 only (subtrees outside are not visited).
template <int K, int D, int V, int V0, int V1>
struct PrefixMasksIn {
    static __device__ inline void go(const uint32_t (&w)[K], uint32_t m, uint32_t (&out)[V1 - V0]) {
        if constexpr (D == K) {
            if constexpr (V >= V0 && V < V1) out[V - V0] = m;
        } else if constexpr (((V + 1) << (K - D)) > V0 && (V << (K - D)) < V1) {
            PrefixMasksIn<K, D + 1, 2 * V, V0, V1>::go(w, m & ~w[D], out);
            PrefixMasksIn<K, D + 1, 2 * V + 1, V0, V1>::go(w, m & w[D], out);
        }
    }
};

template <int K, int V0, int N>
__device__ inline void lut_chunks(const uint32_t (&w)[K], const float (&tq)[quad_share<K>()],
                                  uint32_t b0, uint32_t b1, float& acc, float& last) {
    constexpr int C = PM_LUT_CHUNK > 0 ? PM_LUT_CHUNK : N;
    constexpr int V1 = V0 + C < N ? V0 + C : N;
    uint32_t m[V1 - V0];
    PrefixMasksIn<K, 0, 0, V0, V1>::go(w, 0xFFFFFFFFu, m);
    float r[4 * (V1 - V0)];
#pragma unroll
    for (int v = 0; v < V1 - V0; ++v) {
        r[4 * v + 0] = lds_at(__builtin_amdgcn_perm(b0, m[v], 0x0C060004u));
        r[4 * v + 1] = lds_at(__builtin_amdgcn_perm(b0, m[v], 0x0C060104u) + 128);
        r[4 * v + 2] = lds_at(__builtin_amdgcn_perm(b1, m[v], 0x0C060204u));
        r[4 * v + 3] = lds_at(__builtin_amdgcn_perm(b1, m[v], 0x0C060304u) + 128);
    }
    lut_terms<K, V0, V0, V1>(r, tq, acc, last);
    if constexpr (V1 < N) lut_chunks<K, V1, N>(w, tq, b0, b1, acc, last);
}

template <int K>
__device__ inline float lut_row(const uint32_t (&w)[K], const float (&tq)[quad_share<K>()],
                                float xw, uint32_t b0, uint32_t b1) {
    constexpr int N = (1 << K) - 1;
    float acc = 0.f, last = xw;
    lut_chunks<K, 0, N>(w, tq, b0, b1, acc, last);
    return fmaf(quad_node<K, N>(tq), last, acc);
}

// The activation slice of this workgroup into the LUT.  Thread tid owns
// chunk c = 4l + t, l = tid % 32, t = (tid / 32) % 4, and writes its subset
// sums b = 32q .. 32q + 31 for q = tid / 128 + j * (kLutThreads / 128),
// j < 1024 / kLutThreads; a half-wave writes 32 different banks.  Gate/up: x
// points at the slice.  Down: h of one use for columns tid, tid + kLutThreads,
// .. of the slice, from the gate/up partials pg (gate, ng slices) and pu (up,
// nu slices), `stride` floats apart.  Sums with a zero term are exact.  h is
// staged with one pad word per 32 so that the chunk-wise reads hit 32
// different banks.
// A thread's eight activation values of its chunk, loaded ahead of time (a
// vector type, so that it travels in registers into out-of-line calls).
typedef float X8 __attribute__((ext_vector_type(8)));

__device__ inline X8 load_x8(const float* x) {
    const int tid = threadIdx.x;
    const int c8 = 8 * (4 * (tid & 31) + ((tid >> 5) & 3));
    const f32x4 a = *(g_f32x4*)(x + c8);
    const f32x4 b = *(g_f32x4*)(x + c8 + 4);
    return X8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

__device__ inline void build_lut(lds_float* hbuf, const float* x, const float* pg,
                                 const float* pu, int ng, int nu, int stride, const X8& xv) {
    constexpr int kQ = kLutThreads / 128;          // q values spread over threads
    constexpr int kPer = 8 / kQ;                   // q values per thread
    const int tid = threadIdx.x;
    const int l = tid & 31, t = (tid >> 5) & 3;
    const int c8 = 8 * (4 * l + t);
    float v[8];
    if (pg) {
#pragma unroll
        for (int half = 0; half < kSliceCols / kLutThreads; ++half) {
            g_f32* g = (g_f32*)(pg + half * kLutThreads);
            g_f32* u = (g_f32*)(pu + half * kLutThreads);
            float gs, us;
            if (ng <= 4 && nu <= 4) {      // all loads in flight at once
                float gv[4], uv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    gv[q] = q < ng ? g[size_t(q) * stride] : 0.f;
                    uv[q] = q < nu ? u[size_t(q) * stride] : 0.f;
                }
                gs = gv[0];
                us = uv[0];
#pragma unroll
                for (int q = 1; q < 4; ++q) {
                    if (q < ng) gs += gv[q];
                    if (q < nu) us += uv[q];
                }
            } else {
                gs = g[0];
                for (int q = 1; q < ng; ++q) gs += g[size_t(q) * stride];
                us = u[0];
                for (int q = 1; q < nu; ++q) us += u[size_t(q) * stride];
            }
            const int c = tid + half * kLutThreads;
            hbuf[c + (c >> 5)] = silu_mul(gs, us);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = hbuf[c8 + i + ((c8 + i) >> 5)];
    } else if (x) {
        const f32x4 a = *(g_f32x4*)(x + c8);
        const f32x4 b = *(g_f32x4*)(x + c8 + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xv[i];
    }
    const int c = 4 * l + t;
    float sub[32];
    sub[0] = 0.f;
#pragma unroll
    for (int i = 1; i < 32; ++i) sub[i] = sub[i & (i - 1)] + v[__builtin_ctz(i)];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int q = (tid >> 7) + j * kQ;
        float base = 0.f;
        if (q & 1) base += v[5];
        if (q & 2) base += v[6];
        if (q & 4) base += v[7];
#pragma unroll
        for (int i = 0; i < 32; ++i) lds_put(lut_addr(c, 32 * q + i), base + sub[i]);
    }
}

template <int K>
struct LutRowIn {
    uint32_t w[K];
    float tq[quad_share<K>()];
};

// Buffer resource over `bytes` bytes from p: loads through it take a
// wave-uniform byte offset (scalar) plus the lane's byte offset, and return 0
// past the end.
__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), 0x00020000);
}

// One row pair's inputs for this lane: its word of planes 0..K-1 and its
// share of its block's depth-K table.  prow / trow: the pair's wave-uniform
// byte offsets into the plane and table buffers; wo / to: the lane's.
template <int K>
__device__ inline void lut_load(LutRowIn<K>& in, __amdgpu_buffer_rsrc_t rp, __amdgpu_buffer_rsrc_t rt,
                                uint32_t wo, uint32_t to, uint32_t prow, uint32_t trow,
                                uint32_t pbytes) {
#pragma unroll
    for (int p = 0; p < K; ++p)
        in.w[p] = uint32_t(__builtin_amdgcn_raw_buffer_load_b32(rp, int(wo), int(prow + p * pbytes), 0));
#pragma unroll
    for (int j = 0; j < quad_share<K>(); ++j)
        in.tq[j] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rt, int(to + 4 * j), int(trow), 0));
}

template <int K>
constexpr int lut_unroll() {
#if PM_LUT_THREADS == 1024
    return K == 1 ? 4 : K == 2 ? 2 : 1;
#else
    return K == 1 ? 8 : K == 2 ? 4 : K == 3 ? 3 : K == 4 ? 2 : 1;
#endif
}

// One job segment: the slice's first word and first block table in row 0
// (shared by the wave), and the lane's byte offsets from them.  The LUT path
// takes an even number of rows per matrix and cuts segments at even rows, so
// every row pair of a segment lies inside it.
struct Seg {
    const uint32_t* pw;    // plane 0, row 0, first word of the slice
    const float* tab;      // depth-k table of the slice's first block, row 0
    float* out;            // outputs of this slice
    uint64_t pstride;      // words between planes
    int W;                 // words per row
    int tab_row;           // floats between tables of consecutive rows
    int r0, r1;            // rows [r0, r1), both even
    uint32_t wo, to, oo;   // lane byte offsets: word, table, output
};

// A batch: U row pairs of this wave, pairs p, p + kLutWaves, ... (rows 2p + hw).
template <int K, int U>
struct Batch {
    LutRowIn<K> in[U];
    int pp[U];             // pair index (wave-uniform)
    bool ok[U];            // the pair lies in the segment (wave-uniform)
};

template <class T>
__device__ inline const T* at_bytes(const T* base, uint32_t off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

// Loads are unconditional (a pair past the segment reloads its last pair
// and is not stored), so that the batch is straight-line code; every
// address is a wave-uniform base plus the lane's fixed byte offset.
template <int K, int U>
__device__ inline void batch_load(Batch<K, U>& B, const Seg& sg, __amdgpu_buffer_rsrc_t rp,
                                  __amdgpu_buffer_rsrc_t rt, int p, int p1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = p + u * kLutWaves;
        const int pp = min(q, p1 - 1);
        B.pp[u] = pp;
        B.ok[u] = q < p1;
        lut_load<K>(B.in[u], rp, rt, sg.wo, sg.to, uint32_t(2 * pp * sg.W) * 4u,
                    uint32_t(2 * pp * sg.tab_row) * 4u, uint32_t(sg.pstride) * 4u);
    }
}

// The rows of a batch are computed and reduced as one straight-line block
// (their lookups and reductions interleave), and stored after it.
template <int K, int U>
__device__ inline void batch_compute(const Batch<K, U>& B, const Seg& sg, float xw, uint32_t b0,
                                     uint32_t b1, int l) {
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = lut_row<K>(B.in[u].w, B.in[u].tq, xw, b0, b1);
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = half_sum(acc[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (B.ok[u] && l == 31)
            *(g_f32_out*)at_bytes(sg.out + 2 * B.pp[u], sg.oo) = acc[u];
}

// Where the LUT of a workgroup comes from (see build_lut).
struct LutSrc {
    const float* x;        // null with pg null: the values are in xv
    const float* pg;
    const float* pu;
    int ng, nu, stride;
    X8 xv;
};

// Rows [r0, r1) of one job for this wave, double-buffered: the next batch is
// in flight while this one computes.  FIRST: the workgroup's first segment --
// its first batch is issued before the LUT is built, and the lane's total of
// x over its word is returned.  Out of line so that every prefix gets its own
// register allocation.
template <int K, bool FIRST>
__device__ __noinline__ float lut_segment(lds_float* hbuf, const uint32_t* pw, const float* tab,
                                          float* out, uint64_t pstride, int W, int tab_row,
                                          int wpg, int r0, int r1, const float* x,
                                          const float* pg, const float* pu, int ngnu,
                                          int hstride, X8 xv, float xw) {
    constexpr int U = lut_unroll<K>();
    const int tid = threadIdx.x, wave = uni(tid / kWave), lane = tid % kWave;
    const int hw = lane >> 5, l = lane & 31;
    Seg sg{uni_ptr(pw), uni_ptr(tab), uni_ptr(out), uni64(pstride), uni(W), uni(tab_row),
           uni(r0), uni(r1), 0, 0, 0};
    // planes 0..K-1 and the tables of the rows below r1
    const __amdgpu_buffer_rsrc_t rp =
        buffer_of(sg.pw, uint32_t(((K - 1) * sg.pstride + uint64_t(sg.r1) * sg.W) * 4));
    const __amdgpu_buffer_rsrc_t rt = buffer_of(sg.tab, uint32_t(uint64_t(sg.r1) * sg.tab_row * 4));
    sg.wo = uint32_t(l + hw * sg.W) * 4u;
    // the lane's quad share of its block's table (four lanes per block)
    sg.to = uint32_t(hw * sg.tab_row + ((l >> 2) << K) +
                     (K == 1 ? (l & 1) : (l & 3) * quad_share<K>())) * 4u;
    sg.oo = uint32_t(hw) * 4u;
    const uint32_t b0 = uint32_t(l) << 2, b1 = b0 | 0x10000u;
    const int p1 = (sg.r1 + 1) >> 1;
    constexpr int step = kLutWaves * U;
    int p = (sg.r0 >> 1) + wave;
    Batch<K, U> A, B;
    batch_load<K, U>(A, sg, rp, rt, p, p1);
    if constexpr (FIRST) {
        build_lut(hbuf, x, pg, pu, ngnu & 15, ngnu >> 4, hstride, xv);
        __syncthreads();
        xw = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) xw += lds_at(lut_addr(4 * l + t, 255));
    }
    // the scheduling barriers keep each batch's loads ahead of the other
    // batch's arithmetic (hoisting that arithmetic would make the loads wait)
    while (p < p1) {
        batch_load<K, U>(B, sg, rp, rt, p + step, p1);
        __builtin_amdgcn_sched_barrier(0);
        batch_compute<K, U>(A, sg, xw, b0, b1, l);
        __builtin_amdgcn_sched_barrier(0);
        p += step;
        if (p >= p1) break;
        batch_load<K, U>(A, sg, rp, rt, p + step, p1);
        __builtin_amdgcn_sched_barrier(0);
        batch_compute<K, U>(B, sg, xw, b0, b1, l);
        __builtin_amdgcn_sched_barrier(0);
        p += step;
    }
    return xw;
}

template <bool FIRST>
__device__ inline float lut_segment_k(int k, lds_float* hbuf, const Seg& sg, int wpg,
                                      const LutSrc& src, float xw) {
    const int ngnu = src.ng | (src.nu << 4);
#define PM_SEG(KK)                                                                            \
    lut_segment<KK, FIRST>(hbuf, sg.pw, sg.tab, sg.out, sg.pstride, sg.W, sg.tab_row, wpg,   \
                           sg.r0, sg.r1, src.x, src.pg, src.pu, ngnu, src.stride, src.xv, xw)
    switch (k) {
        case 1: return PM_SEG(1);
        case 2: return PM_SEG(2);
        case 3: return PM_SEG(3);
        case 4: return PM_SEG(4);
        default: return PM_SEG(5);
    }
#undef PM_SEG
}

// Shape of the matrices of one launch.
struct MatArgs {
    uint64_t pstride;      // words between planes
    int rows, W, wpg;      // rows, words per row, words per block
    int out_stride;        // floats between the slice outputs of a job
};

__device__ inline MatArgs mat_of(const KLaunch& L) {
    return MatArgs{L.pstride, L.rows, L.W, L.wpg, L.out_stride};
}

// The segment description of job jb, rows [r0, r1), for this lane.
__device__ inline Seg make_seg(const MatArgs& M, const KJob& jb, int slice, int r0, int r1) {
    const int w0 = (kSliceCols / 32) * slice;
    Seg sg;
    sg.pw = jb.planes + w0;
    sg.tab = jb.lvk + (size_t(w0 / M.wpg) << jb.k);
    sg.out = jb.out + size_t(slice) * M.out_stride;
    sg.pstride = M.pstride;
    sg.W = M.W;
    sg.tab_row = (M.W / M.wpg) << jb.k;
    sg.r0 = r0;
    sg.r1 = r1;
    sg.wo = sg.to = sg.oo = 0;
    return sg;
}

// LUT sources: the activation slice of x, or h of a use from its gate/up
// partials (gu: [use][2][gu_smax][inter]).
__device__ inline LutSrc src_x(const float* x, int slice) {
    LutSrc r{};
    r.x = x + kSliceCols * slice;
    return r;
}
__device__ inline LutSrc src_h(const float* gu, int gu_smax, int inter, const KJob& jb, int use,
                               int slice) {
    LutSrc r{};
    const int c = kSliceCols * slice + int(threadIdx.x);     // and c + kLutThreads ..
    r.pg = gu + (size_t(use) * 2) * gu_smax * inter + c;
    r.pu = r.pg + size_t(gu_smax) * inter;
    r.ng = jb.gsl & 15;
    r.nu = jb.gsl >> 4;
    r.stride = inter;
    return r;
}

// Rows g0 .. g1-1 of the launch's row sequence (row r of job j is
// j * rows + r), the first segment building the LUT from its job's source.
// Every value here is the same across the workgroup; the job descriptions
// are read straight from the argument block.
template <bool DOWN>
__global__ __launch_bounds__(kLutThreads) void lut_kernel(const KLaunch L) {
    // one LDS object: the table at address 0 (lut_sum relies on it), then
    // the padded h of the down stage
    __shared__ __attribute__((aligned(16))) char lds_buf[kLutBytes + (DOWN ? kHbufBytes : 0)];
    lds_float* hb = (lds_float*)(lds_buf + kLutBytes);
    const int slice = blockIdx.x % L.S, q = blockIdx.x / L.S;
    // one activation for the whole launch (x_stride 0): its slice is loaded
    // before the row range is known
    X8 xpre{};
    const bool pre = !DOWN && L.x_stride == 0;
    if (pre) xpre = load_x8(L.x + kSliceCols * slice);
    const int g0 = L.start[q], g1 = L.start[q + 1];
    if (g0 >= g1) return;
    const int rows = L.rows;
    const int ja = g0 / rows, ra = g0 - ja * rows;
    const int jl = (g1 - 1) / rows, rl = g1 - jl * rows;
    const MatArgs M = mat_of(L);
    float xw = 0.f;
    for (int j = ja; j <= jl; ++j) {
        const KJob job = L.job[j];
        const int r0 = j == ja ? ra : 0, r1 = j == jl ? rl : rows;
        const Seg sg = make_seg(M, job, slice, r0, r1);
        if (j == ja) {
            LutSrc src = DOWN ? src_h(L.gu, L.gu_smax, L.inter, job, job.src, slice)
                              : src_x(L.x + size_t(job.src) * L.x_stride, slice);
            if (pre) {
                src.x = nullptr;
                src.xv = xpre;
            }
            xw = lut_segment_k<true>(job.k, hb, sg, M.wpg, src, 0.f);
        } else {
            xw = lut_segment_k<false>(job.k, hb, sg, M.wpg, LutSrc{}, xw);
        }
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
    if (lane == kWave - 1) y[o] = acc;
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
    const dim3 grid(unsigned(L.n_wgq * L.S));
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

hipError_t launch_gemv_fp16(int rows, int cols, const uint16_t* w, const float* x, float* y,
                            hipStream_t st) {
    hipLaunchKernelGGL(gemv_fp16_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(kBlock), 0,
                       st, rows, cols, w, x, y);
    return hipGetLastError();
}

}  // namespace pm
