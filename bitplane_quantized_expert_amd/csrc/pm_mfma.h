// Batched expert path on the matrix cores (pm_mfma.hip).  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pm_internal.h"

namespace pm {

constexpr int kMfmaTileUses = 16;      // uses (columns of the product) per tile
constexpr int kMfmaRowBlock = 64;      // rows per workgroup (4 waves x 16)
constexpr int kMfmaGroup = 128;        // codebook block = one K step of a workgroup

// Up to 16 uses of one matrix of one expert read at one prefix k.
struct MTile {
    const uint32_t* planes;            // plane 0, row 0 of the matrix
    const float* lvk;                  // its depth-k nodes
    int32_t m;                         // 0 gate, 1 up, 2 down
    int32_t n;                         // uses in the tile, 1..16
    int32_t use[kMfmaTileUses];
};

// One launch: tiles of one prefix k and one stage.  Gate/up: the source of
// use u is x + uses[u].tok * cols, its output slice 0 of P.gu, at
// (2u + m) * gu_smax * rows.  Down: the source is P.h + u * cols, the output
// slice 0 of P.y, at u * dn_smax * rows.
struct MLaunch {
    const MTile* tiles;
    int32_t n_tiles, k, rows, cols;
    size_t pstride;
    const Use* uses;
    const float* x;
    Partials P;
    int32_t down;
};

hipError_t launch_mfma(const MLaunch& L, hipStream_t st);

}  // namespace pm
