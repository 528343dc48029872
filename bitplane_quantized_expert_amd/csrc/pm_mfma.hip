// Batched expert execution on the matrix cores, for calls where several uses
// read one matrix of one expert at one prefix k (larger batches; the pages
// name them untested: "PagedMoE: Cross-Precision Expert Caching for
// SSD-Resident MoE Inference", podcast transcript, cue 65).  The values are
// those of the direct path: every weight is the depth-k node its k-bit prefix
// selects (cues 21 and 25), never a stored dense matrix.
//
// A tile is up to 16 uses of one (expert, matrix, k); a workgroup of 4 waves
// takes 64 rows of it, a wave 16 rows, and computes the 16 x n block of
// products with v_mfma_f32_16x16x4_f32 (fp32 operands, fp32 sums): A is
// 16 rows x 4 inputs of decoded weights, B 4 inputs x 16 uses of their
// activations.  Per 128-input codebook block the workgroup stages in LDS
//   - the activations of its uses (16 x 128 fp32, rows padded to 132 floats
//     so that the 16 uses of one step fall in distinct banks),
//   - each wave's 16 depth-k tables (16 x 2^k fp32),
// then runs 32 steps of 4 inputs.  In step s lane (i, q) = (lane % 16,
// lane / 16) decodes input 4s + q of row i from its k plane words: the k
// bits give the table index, the node is A[i][q]; B[q][j] is activation
// 4s + q of use j.  Accumulator lane layout: D[4q + r][lane % 16].
#include <hip/hip_runtime.h>

#include "pm_mfma.h"

namespace pm {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const f32x4 g_f32x4;
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;

constexpr int kXPad = kMfmaGroup + 4;

template <int K>
__global__ __launch_bounds__(256) void mfma_kernel(const MLaunch L) {
#pragma clang fp contract(off)
    constexpr int T = 1 << K;
    __shared__ __attribute__((aligned(16))) float xs[kMfmaTileUses][kXPad];
    __shared__ __attribute__((aligned(16))) float tabs[4][16 * T];
    const int rbs = L.rows / kMfmaRowBlock;
    const MTile& tile = L.tiles[blockIdx.x / rbs];
    const int n = tile.n, m = tile.m;
    const int r0 = (blockIdx.x % rbs) * kMfmaRowBlock;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int i = lane & 15, q = lane >> 4;
    const int W = L.cols / 32, nb = L.cols / kMfmaGroup;
    const int wrow = r0 + wv * 16;                       // the wave's first row
    const uint32_t* prow = tile.planes + size_t(wrow + i) * W;

    // activation staging: thread t loads 8 inputs of use t / 16
    const int xu = threadIdx.x >> 4, xc = (threadIdx.x & 15) * 8;
    const float* xsrc = nullptr;
    if (xu < n) {
        const int u = tile.use[xu];
        xsrc = L.down ? L.P.h + size_t(u) * L.cols : L.x + size_t(L.uses[u].tok) * L.cols;
    }
    // table staging: the wave's 16 tables of a block are 16 runs of T floats
    constexpr int kPieces = 16 * T / 4;                  // 16-byte pieces per wave
    constexpr int kPerLane = kPieces >= 64 ? kPieces / 64 : 1;
    float* wt = tabs[wv];

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int blk = 0; blk < nb; ++blk) {
        u32x4 pw[K];
#pragma unroll
        for (int p = 0; p < K; ++p)
            pw[p] = *(g_u32x4*)(prow + size_t(p) * L.pstride + blk * 4);
        f32x4 xa = {0.f, 0.f, 0.f, 0.f}, xb = {0.f, 0.f, 0.f, 0.f};
        if (xsrc) {
            xa = *(g_f32x4*)(xsrc + blk * kMfmaGroup + xc);
            xb = *(g_f32x4*)(xsrc + blk * kMfmaGroup + xc + 4);
        }
        f32x4 tp[kPerLane];
#pragma unroll
        for (int c = 0; c < kPerLane; ++c) {
            const int pi = lane + 64 * c;
            if (kPieces >= 64 || pi < kPieces) {
                const int rr = pi / (T >= 4 ? T / 4 : 1), within = pi % (T >= 4 ? T / 4 : 1);
                if constexpr (T >= 4) {
                    tp[c] = *(g_f32x4*)(tile.lvk + ((size_t(wrow + rr) * nb + blk) << K) +
                                        4 * within);
                } else {
                    (void)within;
                    tp[c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        __syncthreads();                                 // last block's reads are done
        *(f32x4*)&xs[xu][xc] = xa;
        *(f32x4*)&xs[xu][xc + 4] = xb;
        if constexpr (T >= 4) {
#pragma unroll
            for (int c = 0; c < kPerLane; ++c) {
                const int pi = lane + 64 * c;
                if (kPieces >= 64 || pi < kPieces) *(f32x4*)&wt[4 * pi] = tp[c];
            }
        } else {
            // k = 1: two nodes per table, 32 floats per wave
            if (lane < 32)
                wt[lane] = tile.lvk[((size_t(wrow + lane / 2) * nb + blk) << K) + (lane & 1)];
        }
        __syncthreads();
        const float* ta = wt + i * T;
        const float* xb_row = &xs[i][q];
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int w = s >> 3, bit = 4 * (s & 7) + q;
            uint32_t v = 0;
#pragma unroll
            for (int p = 0; p < K; ++p) v = (v << 1) | ((pw[p][w] >> bit) & 1u);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[v], xb_row[4 * s], acc, 0, 0, 0);
        }
    }
    if (i < n) {
        const int u = tile.use[i];
        float* out = L.down ? L.P.y + size_t(u) * L.P.dn_smax * L.rows
                            : L.P.gu + (size_t(u) * 2 + m) * L.P.gu_smax * L.rows;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[wrow + 4 * q + r] = acc[r];
    }
}

}  // namespace

hipError_t launch_mfma(const MLaunch& L, hipStream_t st) {
    if (L.n_tiles == 0) return hipSuccess;
    const dim3 grid(unsigned(size_t(L.n_tiles) * (L.rows / kMfmaRowBlock)));
    switch (L.k) {
    case 1: hipLaunchKernelGGL(mfma_kernel<1>, grid, dim3(256), 0, st, L); break;
    case 2: hipLaunchKernelGGL(mfma_kernel<2>, grid, dim3(256), 0, st, L); break;
    case 3: hipLaunchKernelGGL(mfma_kernel<3>, grid, dim3(256), 0, st, L); break;
    case 4: hipLaunchKernelGGL(mfma_kernel<4>, grid, dim3(256), 0, st, L); break;
    case 5: hipLaunchKernelGGL(mfma_kernel<5>, grid, dim3(256), 0, st, L); break;
    case 6: hipLaunchKernelGGL(mfma_kernel<6>, grid, dim3(256), 0, st, L); break;
    case 7: hipLaunchKernelGGL(mfma_kernel<7>, grid, dim3(256), 0, st, L); break;
    default: hipLaunchKernelGGL(mfma_kernel<8>, grid, dim3(256), 0, st, L); break;
    }
    return hipGetLastError();
}

}  // namespace pm
