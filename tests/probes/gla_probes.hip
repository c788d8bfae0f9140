// gla_probes.hip -- device probes behind design choices of the library's
// kernels, built beside the tests (tests/probes/build.py) and never linked
// into libgla.so.
//
//  * gla_probe_tr16: the lane layout of the gfx950 LDS transpose read as the
//    kernels use it (ld_tr / tr_addr / tr_frag_s of gla_device.h): every lane
//    of one wavefront reads a known binary16 tile and reports what it got.
//  * gla_probe_read / gla_probe_copy / gla_probe_gather: streaming kernels
//    whose timing gives the practical HBM ceilings quoted with the roofline
//    (16-byte-per-lane reads, read + write copy, and the kernels' row-gather
//    pattern: 16 rows x 64 bytes per wavefront instruction in a permuted row
//    order, 512-thread workgroups).
//
// Every launch is bounds-checked on the host: the byte counts must be
// multiples of the per-thread access and the grids cover them exactly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"

namespace {

using gla::half4;
using gla::half8;
using gla::u32x4;

typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 72;  // row stride (elements) of the probed tile, as SH in the kernels
constexpr int kRows = 32;

// Tile element (r, c) holds r * 64 + c (exact in binary16 for r < 32, c < 64).
__global__ __launch_bounds__(64) void probe_tr16_kernel(uint16_t* out)
{
    __shared__ __attribute__((aligned(16))) _Float16 tile[kRows * kTile];
    const int lane = threadIdx.x;
    for (int i = lane; i < kRows * kTile; i += 64) {
        const int r = i / kTile, c = i % kTile;
        tile[i] = (_Float16)(c < 64 ? r * 64 + c : 0);
    }
    __syncthreads();
    const int g = lane >> 4, l16 = lane & 15;
    // (a) four rows through one read: lane group g asks for rows 4g .. 4g+3 of
    //     columns 16 g' .. : row0 = 4g, col0 = 16 (g % 4)
    const half4 a = gla::ld_tr(gla::tr_addr<kTile>(tile, 4 * g, 16 * (g & 3), l16));
    // (b) the eight-row fragment: rows 8g .. 8g+7 of columns 32 + l16
    const half8 b = gla::tr_frag_s<kTile>(tile, 8 * g, 32, l16);
    // whole vectors are bit-cast (this compiler's __builtin_bit_cast of one
    // element of an ext_vector_type value reads element 0 whatever the index)
    const u16x4 au = __builtin_bit_cast(u16x4, a);
    const u16x8 bu = __builtin_bit_cast(u16x8, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[lane * 12 + e] = au[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[lane * 12 + 4 + e] = bu[e];
}

// Sum of 16-byte loads, grid-stride; one word per thread keeps the loads live.
__global__ __launch_bounds__(512) void probe_read_kernel(const u32x4* src, size_t n16, unsigned* sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    unsigned acc = 0u;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] + v[1] + v[2] + v[3];
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(512) void probe_copy_kernel(const u32x4* src, u32x4* dst, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Rows of 128 bytes (64 binary16 channels) visited in the order of a
// top-to-bottom scan of a side x side grid stored left-to-right (row index
// (t mod side) * side + t / side for scan position t).  Lane (g, l16) of a
// wavefront reads 16 bytes at channel 8 g of half h = wave & 1 of the row at
// scan position 16 (4 pass + wave / 2) + l16 of each pass over 64 scan
// positions: the access shape of the kernels' chunk loads.
__global__ __launch_bounds__(512) void probe_gather_kernel(const u32x4* src, int side, int npass,
                                                           unsigned* sink)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15, h = wave & 1;
    unsigned acc = 0u;
    const int rows = side * side;
    for (int pass = blockIdx.x; pass < npass; pass += gridDim.x) {
        // 4 groups of 16 scan positions per workgroup pass (waves 2j, 2j+1 share one)
        const int t = (pass * 4 + (wave >> 1)) * 16 + l16;
        if (t < rows) {
            const int row = (t % side) * side + t / side;
            const u32x4 v = src[(size_t)row * 8 + 4 * h + g];
            acc ^= v[0] + v[1] + v[2] + v[3];
        }
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// out: 64 lanes x 12 binary16 values (the 4 of the single read, then the 8 of
// the fragment), device memory.  Returns 0, or 1 on a launch error.
__attribute__((visibility("default"))) int gla_probe_tr16(uint16_t* out, void* stream)
{
    hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Reads `bytes` (a multiple of 16) from src; sink holds blocks x 512 words.
__attribute__((visibility("default"))) int gla_probe_read(const void* src, size_t bytes, unsigned* sink,
                                                          int blocks, void* stream)
{
    if (bytes % 16 || blocks <= 0) return 2;
    hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const u32x4*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

__attribute__((visibility("default"))) int gla_probe_copy(const void* src, void* dst, size_t bytes, int blocks,
                                                          void* stream)
{
    if (bytes % 16 || blocks <= 0) return 2;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// src holds side * side rows of 128 bytes; sink holds blocks x 512 words.
__attribute__((visibility("default"))) int gla_probe_gather(const void* src, int side, unsigned* sink,
                                                            int blocks, void* stream)
{
    if (side <= 0 || blocks <= 0) return 2;
    const int npass = (side * side + 63) / 64;
    hipLaunchKernelGGL(probe_gather_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const u32x4*)src, side, npass, sink);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
