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
    int32_t blk_gu;                // first block of this item in the gate/up grid
    int32_t blk_dn;                // first block of this item in the down grid
};

// A use: token `tok` reads the expert in routing slot `slot` with weight w.
// Its index is tok * top_k + slot.
struct Use {
    int32_t k[3];
    float w;
    int32_t tok, slot;
};

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
hipError_t launch_gemv_fp16(int rows, int cols, const uint16_t* w, const float* x, float* y,
                            hipStream_t st);

// MoE forward stages.  `items`, `uses`, `list` are device copies of the work
// list; G, U: fp32 [n_uses][inter]; Y: fp32 [n_uses][hidden].
hipError_t launch_gateup(const Geom& g, const Item* items, int item0, int n_items,
                         int n_blocks, const Use* uses, const int32_t* list, int top_k,
                         const float* x, float* G, float* U, hipStream_t st);
// launch_down first turns G into h = silu(G) * U in place (n_uses rows).
hipError_t launch_down(const Geom& g, const Item* items, int n_items, int n_blocks,
                       const Use* uses, const int32_t* list, int n_uses, float* G,
                       const float* U, float* Y, hipStream_t st);
hipError_t launch_combine(int n_tokens, int top_k, int hidden, const Use* uses,
                          const float* Y, float* y, hipStream_t st);

// Rows of a matrix handled by one block of the gate/up and down stages.
int gateup_rows_per_block();
int down_rows_per_block();
// Largest number of uses of one expert the down stage can hold in LDS.
int max_uses_per_item();

}  // namespace pm
