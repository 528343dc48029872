// Device side of the encoder from fp32 weights (pm_encoder.hip).  Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pm {

// Largest block the K-means kernel sorts in LDS.
constexpr int kMaxKmeansGroup = 4096;

// Lloyd's K-means with 256 centroids on every block of `group` inputs of one
// row of w [rows][cols]; one workgroup per block.
hipError_t launch_kmeans_device(int rows, int cols, int group, const float* w, int max_iters,
                                uint8_t* codes, float* leaves, uint32_t* counts,
                                int32_t* iters, hipStream_t st);

}  // namespace pm
