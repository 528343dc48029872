// Internal declarations shared by the host side (pm_host.cpp) and the HIP
// kernels (pm_kernels.hip) of libpm.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pm.h"

namespace pm {

constexpr int kBits = 8;          // stored index width (8 planes, 256 leaves)
constexpr int kLeaves = 1 << kBits;
constexpr int kLevelFloatsPerBlock = 2 * kLeaves - 2;   // depths 1..8: 510

// Float offset of depth d inside a matrix's levels, in blocks of one node row.
__host__ __device__ inline size_t level_offset(size_t nblocks, int d) {
    return nblocks * ((size_t(1) << d) - 2);
}

// Geometry of an expert as the kernels see it.  Matrix m: 0 gate, 1 up, 2 down.
struct Geom {
    int hidden, inter, group;
    size_t plane_words;            // words of one expert plane chunk (all 3 matrices)
    size_t plane_off[3];           // word offset of matrix m inside a plane chunk
    size_t level_off[3];           // float offset of matrix m inside the levels
    int rows[3], cols[3];
};

// One distinct expert of a forward call and the token uses that read it.
struct Item {
    const uint32_t* planes;        // plane chunk 0 of the expert
    const float* levels;           // gate, up, down levels back to back
    int32_t use0, nuse;            // uses are list[use0 .. use0 + nuse)
    int32_t kmax[3];               // largest prefix of any use, per matrix
    int32_t pad;
};

// A use: token `tok` reads the expert in routing slot `slot` with weight w.
// Its index is tok * top_k + slot.  slices[m] is the number of partial sums
// the stage of matrix m leaves for it (one per 1024-column slice on the LUT
// path, else 1); direct[m] is its path: 0 LUT job, 1 direct kernels, 2 a
// matrix-core tile.
struct Use {
    int32_t k[3];
    float w;
    int32_t tok, slot;
    int32_t slices[3];
    int32_t direct[3];
};

// Whether the direct gate/up kernel forms h = SiLU(g) * u of a use: its gate
// and up rows both run there, and a direct or tiled down product reads h.
__host__ __device__ inline bool h_by_gateup(const Use& u) {
    return u.direct[0] == 1 && u.direct[1] == 1 && u.direct[2] != 0;
}

// LUT path: one matrix of one use.  Row r's partial sum over column slice s
// goes to out[s * out_stride + r].
struct LutJob {
    const uint32_t* planes;        // plane 0, row 0 of the matrix
    const float* lvk;              // depth-k nodes of the matrix
    float* out;
    uint64_t pstride;              // words between planes
    int32_t k, rows, W, wpg;       // prefix, rows, words per row, words per block
    int32_t out_stride, pad;
};

// LUT path: the rows one workgroup processes, [(job0, row0), (job1, row1)),
// against the activation slice `slice` of source `src` (a token for gate/up,
// a use for down).  Row boundaries are even.
struct LutWG {
    int32_t job0, row0, job1, row1;
    int32_t src, slice;
};

// Partial-sum workspace of a forward call (device pointers).
struct Partials {
    float* gu;                     // [n_uses][2][gu_smax][inter]
    float* h;                      // [n_uses][inter], direct down only
    float* y;                      // [n_uses][dn_smax][hidden]
    int gu_smax, dn_smax;
};

constexpr int kSliceCols = 1024;   // columns of x covered by one LUT
// Block size of the LUT path: one lane holds a block's four plane words and
// its depth-k nodes.
constexpr int kLutGroup = 128;
// Rows of one wave step on the LUT path (8 rows x the 8 blocks of a slice);
// matrices on the LUT path have a multiple of 8 rows.
constexpr int kLutRows = 8;
// Largest prefix read through the LUT path: in a layer forward (one launch
// for all experts; larger prefixes add the direct launches) and in a single
// GEMV (from k = 5 the staged-table direct path is faster).
constexpr int kLutMaxK = 5;
constexpr int kGemvLutMaxK = 4;

// LUT-path launch description, passed as kernel arguments (no upload).
constexpr int kMaxLaunchJobs = 56;
// Uses in one forward call: a job names its token or use in 16 bits.
constexpr int kMaxCallUses = 32767;
struct KJob {                      // one matrix of one use
    const uint32_t* planes;        // plane 0, row 0
    const float* lvk;              // depth-k nodes
    float* out;                    // row r, slice s -> out[s * out_stride + r]
    float wt;                      // down with the combine folded in: routing weight
    int16_t src;                   // gate/up: token; down: use
    int8_t k;
    uint8_t gsl;                   // down: gate slices (bits 0-3), up slices (bits 4-7)
};
// One LUT launch: n_wgq x S workgroups.  The rows of the jobs are numbered
// as one sequence (row r of job j is g = j * rows + r).  The jobs come in
// runs of one activation source and one prefix; run i covers the rows
// [g0, g0 + 8 * nsteps) and has the workgroups wg0 .. wg0 + nwg - 1 of every
// slice, which split its 8-row steps evenly (a run's steps all cost the
// same).  Scalars come first so that the fields every workgroup reads at its
// start share one cache line.
constexpr int kMaxLaunchWgq = 256;
struct KRun {
    int32_t g0, nsteps;
    int16_t wg0, nwg;
    // activation source (bits 0-15: token or use), prefix k (bits 16-19),
    // gate/up slice counts of a down job (bits 24-31)
    uint32_t meta;
};
struct KLaunch {
    const float* x;                // gate/up: activation of token t at x + t * x_stride
                                   // (x_stride 0: every job reads x itself)
    const float* gu;               // down: gate/up partials [use][2][gu_smax][inter]
    float* zero;                   // gate/up: n_zero floats to clear (the layer output
                                   // that a folded down launch adds into)
    uint64_t pstride;              // words between planes
    int32_t n_jobs, n_wgq, S, rows;
    int32_t W, wpg, out_stride, x_stride;
    int32_t gu_smax, inter, n_zero;
    int32_t fold;                  // down: add wt * row sum into out (float atomics)
                                   // instead of storing the partial
    // workgroup q: its run (bits 0-7) and that run's activation source
    // (bits 8-23) and gate/up slice counts (bits 24-31), so that its first
    // reads of the source need no second lookup
    uint32_t wg_info[kMaxLaunchWgq];
    KRun run[kMaxLaunchJobs];
    KJob job[kMaxLaunchJobs];
};
static_assert(sizeof(KLaunch) <= 4096, "kernel arguments are limited to 4 KiB");
// Cost model of a LUT workgroup (16 waves, one 1024-column slice), fitted on
// gfx950 to the workgroup timelines of the 512-expert layer step (rows
// streamed from HBM; greedy prefixes at a mean of 2.5 bits): a part per
// 8-row step, the workgroup's steady rate from its first computing step to
// its end, plus a fixed part per workgroup at prefix k, the median remainder
// of its end after the launch's first workgroup started (prologue, latency of
// the first and last steps), both in ns, for gate/up launches and for down
// launches (whose prologue also forms h from the gate/up partials).  At
// k = 4, 5 a workgroup holds fewer steps than waves, so there the "step" part
// is mostly the latency of one step.
#ifndef PM_LUT_FIXED_GU
#define PM_LUT_FIXED_GU 2720, 2530, 2760, 4180, 5280
#endif
#ifndef PM_LUT_STEP_GU
#define PM_LUT_STEP_GU 55, 96, 167, 293, 1390
#endif
#ifndef PM_LUT_FIXED_DN
#define PM_LUT_FIXED_DN 2880, 2880, 2910, 3250, 3550
#endif
#ifndef PM_LUT_STEP_DN
#define PM_LUT_STEP_DN 48, 95, 179, 434, 2910
#endif
inline int64_t lut_step_ns(int k, bool down) {
    constexpr int64_t gu[5] = {PM_LUT_STEP_GU}, dn[5] = {PM_LUT_STEP_DN};
    const int i = k < 1 ? 0 : (k > 5 ? 4 : k - 1);
    return down ? dn[i] : gu[i];
}
inline int64_t lut_fixed_ns(int k, bool down) {
    constexpr int64_t gu[5] = {PM_LUT_FIXED_GU}, dn[5] = {PM_LUT_FIXED_DN};
    const int i = k < 1 ? 0 : (k > 5 ? 4 : k - 1);
    return down ? dn[i] : gu[i];
}

// Kernel launchers (pm_kernels.hip).  All return hipError_t of the launch.
hipError_t launch_gemv(int rows, int cols, int group, int k, const uint32_t* planes,
                       size_t pstride, const float* levels, const float* x, float* y,
                       hipStream_t st);
hipError_t launch_encode_device(int rows, int cols, int group, const uint8_t* codes,
                                const float* leaves, const uint32_t* counts,
                                uint32_t* planes, size_t pstride, float* levels,
                                hipStream_t st);
hipError_t launch_unpack_prefix(int rows, int cols, int k, const uint32_t* planes,
                                size_t pstride, uint8_t* out, hipStream_t st);
hipError_t launch_dequant(int rows, int cols, int group, int k, const uint32_t* planes,
                          size_t pstride, const float* levels, float* out_f32,
                          uint16_t* out_f16, hipStream_t st);
// The materialize-then-multiply comparator, batched: up to kMaxBatchMats
// matrices per launch, described in the kernel arguments.
constexpr int kMaxBatchMats = 64;
struct KDequantBatch {
    int32_t n, pad;
    int32_t rows[kMaxBatchMats], cols[kMaxBatchMats], group[kMaxBatchMats], k[kMaxBatchMats];
    uint64_t pstride[kMaxBatchMats];
    const uint32_t* planes[kMaxBatchMats];
    const float* lvk[kMaxBatchMats];    // depth-k nodes
    uint16_t* w[kMaxBatchMats];
};
static_assert(sizeof(KDequantBatch) <= 4096, "kernel arguments are limited to 4 KiB");
struct KGemv16Batch {
    int32_t n, pad;
    int32_t rows[kMaxBatchMats], cols[kMaxBatchMats];
    const uint16_t* w[kMaxBatchMats];
    const float* x[kMaxBatchMats];
    float* y[kMaxBatchMats];
};
static_assert(sizeof(KGemv16Batch) <= 4096, "kernel arguments are limited to 4 KiB");
hipError_t launch_dequant_batch(const KDequantBatch& B, size_t max_elems, hipStream_t st);
hipError_t launch_gemv_fp16_batch(const KGemv16Batch& B, int max_rows, hipStream_t st);
hipError_t launch_gemv_fp16(int rows, int cols, const uint16_t* w, const float* x, float* y,
                            hipStream_t st);

// LUT path: n_wgq x S workgroups of 1024 threads, 128 KiB of LDS each; every
// workgroup's rows hold jobs of one source and one k.
// Gate/up (down == false): the activation slice comes from L.x; down: h of
// use src, formed from the gate/up partials L.gu.
// t0 / t1: if given, the launch's own start and stop events.
hipError_t launch_lut(const KLaunch& L, bool down, hipStream_t st, hipEvent_t t0 = nullptr,
                      hipEvent_t t1 = nullptr);
// Combine with the weights in the kernel arguments: tokens t0 .. t0+n-1.
constexpr int kMaxLaunchUses = 128;
struct KCombine {
    const float* Y;                // [n_uses][dn_smax][hidden]
    float* y;                      // [n_tokens][hidden]
    int32_t t0, n_tokens, top_k, hidden, dn_smax, pad;
    float w[kMaxLaunchUses];
    uint8_t sl[kMaxLaunchUses];
};
hipError_t launch_combine_k(const KCombine& C, hipStream_t st);
// Sum of the slice partials of one GEMV: y[r] = sum_s part[s * rows + r].
hipError_t launch_sum_slices(const float* part, int slices, int rows, float* y, hipStream_t st);

// Direct path (any prefix, any shape, shared experts read once per call):
// over `n_items` items, rows_per_block rows per block.  Writes slice 0 of the
// partials of every (use, matrix) marked direct.  The gate/up launch also
// clears n_zero floats at `zero` (the output a folded down stage adds into);
// with y_fold the down launch adds w * row sum into y_fold[tok] (device-scope
// float atomics) instead of writing its partials.
hipError_t launch_direct_gateup(const Geom& g, const Item* items, int n_items,
                                const Use* uses, const int32_t* list, const float* x,
                                Partials P, hipStream_t st, float* zero = nullptr,
                                int n_zero = 0);
hipError_t launch_direct_down(const Geom& g, const Item* items, int n_items, const Use* uses,
                              const int32_t* list, Partials P, hipStream_t st,
                              float* y_fold = nullptr);
// h of every use marked direct for down, from the gate/up partials.
hipError_t launch_swiglu(const Use* uses, int n_uses, Partials P, int inter, hipStream_t st);
// y[t][o] = sum_j w[t][j] * sum_s Y[t*top_k + j][s][o], slots then slices in order.
hipError_t launch_combine(int n_tokens, int top_k, int hidden, const Use* uses, Partials P,
                          float* y, hipStream_t st);

}  // namespace pm
