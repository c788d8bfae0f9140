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
//  * gla_probe_handoff: latency of the exchange's flag handoff between two
//    workgroups on one XCD or on two, for each store / load cache policy
//    (the kernels: sc1 loads; sc1 stores across XCDs, default-policy flag
//    stores within one), and whether a policy pair sees the handoff at all.
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

// Flag handoff between two single-wave workgroups (the exchange's protocol
// reduced to one word): the producer stores i to word 0 and waits until the
// consumer has copied it to word 32; the consumer waits for i in word 0 and
// stores it to word 32.  Stores and polls are relaxed atomics, so every poll
// is issued again; agent scope compiles to the sc1 policy the kernels use on
// their buffer instructions, workgroup scope to the default policy (SC1: 1
// for sc1 stores / loads).  Every wait is bounded (kSpin polls); a wait that
// runs out ends both sides (the other one runs out too) and is reported.
// Workgroup 0 produces; the consumer is workgroup `consumer` (1: the next XCD
// under turn-by-turn dispatch, 8: the same XCD on an 8-XCD device); every
// other workgroup returns at once.  out[0]: realtime ticks (100 MHz) of the
// producer's loop, out[1]: handoffs completed, out[2], out[3]: XCC_ID of
// producer and consumer, out[4], out[5]: a wait ran out (producer, consumer).
constexpr unsigned kSpin = 1u << 20;
constexpr int kXccId = 20 | (0 << 6) | ((4 - 1) << 11);

template <bool SC1>
__device__ __forceinline__ unsigned hload(const unsigned* p)
{
    return SC1 ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
template <bool SC1>
__device__ __forceinline__ void hstore(unsigned* p, unsigned v)
{
    if (SC1)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <bool SS, bool LS>
__global__ __launch_bounds__(64) void probe_handoff_kernel(unsigned* words, int iters, int consumer,
                                                           unsigned long long* out)
{
    const int b = blockIdx.x;
    if (b != 0 && b != consumer) return;
    if (threadIdx.x != 0) return;
    const unsigned xcc = __builtin_amdgcn_s_getreg(kXccId) & 15u;
    bool timeout = false;
    if (b == 0) {
        out[2] = xcc;
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        int done = 0;
        for (int i = 1; i <= iters; ++i) {
            hstore<SS>(words, (unsigned)i);
            unsigned spins = 0;
            while (hload<LS>(words + 32) != (unsigned)i && spins <= kSpin) ++spins;
            if (spins > kSpin) {
                timeout = true;
                break;
            }
            done = i;
        }
        const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
        out[0] = t1 - t0;
        out[1] = (unsigned long long)done;
        out[4] = timeout ? 1ull : 0ull;
    } else {
        out[3] = xcc;
        for (int i = 1; i <= iters; ++i) {
            unsigned spins = 0;
            while (hload<LS>(words) != (unsigned)i && spins <= kSpin) ++spins;
            if (spins > kSpin) {
                timeout = true;
                break;
            }
            hstore<SS>(words + 32, (unsigned)i);
        }
        out[5] = timeout ? 1ull : 0ull;
    }
}

}  // namespace

extern "C" {

// words: 64 zeroed device words; out: 6 zeroed device 64-bit words.
// store_sc1 / load_sc1: 1 for the sc1 policy, 0 for the default one.
__attribute__((visibility("default"))) int gla_probe_handoff(unsigned* words, int iters, int consumer,
                                                             int store_sc1, int load_sc1,
                                                             unsigned long long* out, void* stream)
{
    if (iters <= 0 || consumer < 1 || consumer > 64) return 2;
    const dim3 grid(consumer + 1), block(64);
    hipStream_t st = (hipStream_t)stream;
    if (store_sc1 && load_sc1)
        hipLaunchKernelGGL((probe_handoff_kernel<true, true>), grid, block, 0, st, words, iters, consumer, out);
    else if (!store_sc1 && load_sc1)
        hipLaunchKernelGGL((probe_handoff_kernel<false, true>), grid, block, 0, st, words, iters, consumer, out);
    else if (store_sc1 && !load_sc1)
        hipLaunchKernelGGL((probe_handoff_kernel<true, false>), grid, block, 0, st, words, iters, consumer, out);
    else
        hipLaunchKernelGGL((probe_handoff_kernel<false, false>), grid, block, 0, st, words, iters, consumer, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}


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
