// Device-side filler for the seeded synthetic inputs: the same
// Philox4x32-10 streams and the same leaf/code recipes as synth/__init__.py,
// so a GPU-filled expert pool is bit-identical to what the host generator
// draws for any slice of it.  Holds none of the method's arithmetic.
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round
//   (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2,
//   c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), then k += (W0, W1).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct u32x4 { uint32_t v[4]; };

__device__ inline u32x4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = uint64_t(0xD2511F53u) * c0;
        const uint64_t p1 = uint64_t(0xCD9E8D57u) * c2;
        const uint32_t n0 = uint32_t(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = uint32_t(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = uint32_t(p1);
        c2 = n2;
        c3 = uint32_t(p0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return u32x4{{c0, c1, c2, c3}};
}

// One thread per Philox call: leaves 4n .. 4n+3 of the stream, written at
// out[4 (n - first) + i]; leaf index inside its block is (4n + i) % 256.
__global__ void leaves_kernel(uint32_t k0, uint32_t k1, uint64_t first, uint64_t calls,
                              const double* __restrict__ q, const double* __restrict__ gap,
                              float* __restrict__ out) {
    const uint64_t t = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= calls) return;
    const uint64_t n = first + t;
    const u32x4 r = philox(uint32_t(n), uint32_t(n >> 32), 0u, 0u, k0, k1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = int((4 * n + i) & 255u);
        // u in (-1, 1) exactly: (r + 0.5) * 2^-31 - 1
        const double u = __dadd_rn(__dmul_rn(__dadd_rn(double(r.v[i]), 0.5), 0x1p-31), -1.0);
        const double val = __dadd_rn(q[j], __dmul_rn(__dmul_rn(0.25, u), gap[j]));
        out[4 * t + i] = float(val);
    }
}

// One thread per Philox call: 16 codes, byte b of word i is code 4i + b.
__global__ void codes_kernel(uint32_t k0, uint32_t k1, uint64_t first, uint64_t calls,
                             uint8_t* __restrict__ out) {
    const uint64_t t = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= calls) return;
    const uint64_t n = first + t;
    const u32x4 r = philox(uint32_t(n), uint32_t(n >> 32), 0u, 0u, k0, k1);
    reinterpret_cast<uint4*>(out)[t] = make_uint4(r.v[0], r.v[1], r.v[2], r.v[3]);
}

// One thread per Philox call: raw words (poison fills).
__global__ void words_kernel(uint32_t k0, uint32_t k1, uint64_t calls, uint32_t* __restrict__ out) {
    const uint64_t t = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= calls) return;
    const u32x4 r = philox(uint32_t(t), uint32_t(t >> 32), 0u, 0u, k0, k1);
    reinterpret_cast<uint4*>(out)[t] = make_uint4(r.v[0], r.v[1], r.v[2], r.v[3]);
}

inline unsigned blocks(uint64_t n) { return unsigned((n + 255) / 256); }

}  // namespace

extern "C" {

// Leaves of rows row0..row0+nrows-1 of a matrix with ngroups blocks per row:
// fp32 [nrows][ngroups][256] into d_out.  q, gap: device fp64 [256].
int pmsynth_leaves(uint32_t k0, uint32_t k1, int ngroups, int row0, int nrows,
                   const double* q, const double* gap, float* d_out, void* stream) {
    const uint64_t per_row = uint64_t(ngroups) * 256 / 4;
    const uint64_t first = uint64_t(row0) * per_row, calls = uint64_t(nrows) * per_row;
    if (calls == 0) return 0;
    hipLaunchKernelGGL(leaves_kernel, dim3(blocks(calls)), dim3(256), 0, (hipStream_t)stream,
                       k0, k1, first, calls, q, gap, d_out);
    return int(hipGetLastError());
}

// Codes of rows row0..row0+nrows-1 of a matrix with cols columns (cols % 16
// == 0): uint8 [nrows][cols].
int pmsynth_codes(uint32_t k0, uint32_t k1, int cols, int row0, int nrows, uint8_t* d_out,
                  void* stream) {
    const uint64_t per_row = uint64_t(cols) / 16;
    const uint64_t first = uint64_t(row0) * per_row, calls = uint64_t(nrows) * per_row;
    if (calls == 0 || cols % 16) return cols % 16 ? 1 : 0;
    hipLaunchKernelGGL(codes_kernel, dim3(blocks(calls)), dim3(256), 0, (hipStream_t)stream, k0,
                       k1, first, calls, d_out);
    return int(hipGetLastError());
}

// n (a multiple of 4) raw words of a stream.
int pmsynth_words(uint32_t k0, uint32_t k1, uint64_t n, uint32_t* d_out, void* stream) {
    if (n % 4) return 1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(words_kernel, dim3(blocks(n / 4)), dim3(256), 0, (hipStream_t)stream, k0,
                       k1, n / 4, d_out);
    return int(hipGetLastError());
}

}  // extern "C"
