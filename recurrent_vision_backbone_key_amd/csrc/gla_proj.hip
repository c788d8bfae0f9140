// gla_proj.hip -- low-rank retention-gate logits for gfx950.
//
// Paper "GTR: Gated Token Recurrence for Efficient Dense Prediction",
// Section 2.1 (retention gate): the gate logits of a token are x_t W1 W2 + b
// with W1: d_model x rank and W2: rank x (NH*dk).  Both products run on the
// matrix cores, one wavefront per 16 tokens:
//   1. hp^T = W1^T x^T per 16-row rank tile, accumulated in binary32 over
//      d_model (binary16 storage: v_mfma_f32_16x16x32_f16; binary32 storage:
//      v_mfma_f32_16x16x4_f32);
//   2. z^T = W2^T hp^T + b per 16-column output tile with
//      v_mfma_f32_16x16x4_f32, the hp fragments of step 1 feeding the B
//      operand directly: lane (l16, g) holds hp[token l16][16 rt + 4 g + e],
//      which at step (rt, e) is the k = g element of a 4-deep contraction
//      over ranks 16 rt + 4 g + e.
// A lane ends with z[token l16][o0 + 4g .. o0 + 4g + 3] and stores 16 bytes.
// Weights (W1: rank x d_model transposed storage, W2: NH*dk x rank) are
// read straight from memory; they stay in the L2 across workgroups.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"
#include "gla_launch.h"

namespace gla {
namespace proj {

constexpr int kMaxRankTiles = 4;  // rank <= 64

// One fragment of x (token row) or W1 (rank row) for k-step s.
template <typename T> struct Frag;
template <> struct Frag<_Float16> {
    typedef half8 type;
    static constexpr int KSTEP = 32;
    // elements 32 s + 8 g .. +7 of a row of n elements (n a multiple of 8)
    static __device__ __forceinline__ half8 load(const _Float16* row, int n, int s, int g, bool ok)
    {
        const int m = KSTEP * s + 8 * g;
        if (!ok || m >= n) return half8{0, 0, 0, 0, 0, 0, 0, 0};
        return *(const half8*)(row + m);
    }
};
template <> struct Frag<float> {
    typedef float type;
    static constexpr int KSTEP = 4;
    static __device__ __forceinline__ float load(const float* row, int n, int s, int g, bool ok)
    {
        const int m = KSTEP * s + g;
        if (!ok || m >= n) return 0.f;
        return row[m];
    }
};

template <typename T>
__global__ __launch_bounds__(256) void gla_gate_logits_kernel(const T* __restrict__ x,
                                                              const T* __restrict__ w1,
                                                              const float* __restrict__ w2,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ z, int tokens,
                                                              int d_model, int rank, int nout)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int tok0 = (blockIdx.x * 4 + wave) * 16;
    if (tok0 >= tokens) return;
    const int tok = tok0 + l16;
    const bool tv = tok < tokens;
    const T* xrow = x + (size_t)(tv ? tok : tok0) * d_model;
    const int nrt = (rank + 15) / 16;
    const int ksteps = (d_model + Frag<T>::KSTEP - 1) / Frag<T>::KSTEP;

    // ---- 1. hp^T tiles: rows = ranks 16 rt + (0..15), columns = the 16 tokens
    float4v hp[kMaxRankTiles];
#pragma unroll
    for (int rt = 0; rt < kMaxRankTiles; ++rt) hp[rt] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ksteps; ++s) {
        const typename Frag<T>::type b = Frag<T>::load(xrow, d_model, s, g, tv);
#pragma unroll
        for (int rt = 0; rt < kMaxRankTiles; ++rt) {
            if (rt >= nrt) break;
            const int j = 16 * rt + l16;
            const typename Frag<T>::type a =
                Frag<T>::load(w1 + (size_t)(j < rank ? j : 0) * d_model, d_model, s, g, j < rank);
            hp[rt] = mma(a, b, hp[rt]);
        }
    }

    // ---- 2. z^T tiles: rows = outputs o0 + (0..15), columns = the 16 tokens
    for (int o0 = 0; o0 < nout; o0 += 16) {
        const int orow = o0 + l16;  // A row of this lane
        float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
        if (bias) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = bias[o0 + 4 * g + e];
        }
#pragma unroll
        for (int rt = 0; rt < kMaxRankTiles; ++rt) {
            if (rt >= nrt) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * rt + 4 * g + e;
                const float a = (j < rank) ? w2[(size_t)orow * rank + j] : 0.f;
                acc = mma(a, hp[rt][e], acc);
            }
        }
        if (tv) *(float4v*)(z + (size_t)tok * nout + o0 + 4 * g) = acc;
    }
}

}  // namespace proj

int launch_gate_logits(const GateProj& G, int dtype, int tokens, int nout, float* z, void* stream)
{
    if (tokens <= 0) return GLA_OK;
    const unsigned blocks = (unsigned)((tokens + 63) / 64);
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GLA_F16) {
        hipLaunchKernelGGL(proj::gla_gate_logits_kernel<_Float16>, dim3(blocks), dim3(256), 0, st,
                           (const _Float16*)G.x, (const _Float16*)G.w1, G.w2, G.bias, z, tokens,
                           G.d_model, G.rank, nout);
    } else {
        hipLaunchKernelGGL(proj::gla_gate_logits_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           (const float*)G.x, (const float*)G.w1, G.w2, G.bias, z, tokens,
                           G.d_model, G.rank, nout);
    }
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

}  // namespace gla
