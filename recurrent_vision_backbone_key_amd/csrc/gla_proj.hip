// gla_proj.hip -- low-rank retention-gate projection for gfx950.
//
// Paper "GTR: Gated Token Recurrence for Efficient Dense Prediction",
// Section 2.1 (retention gate): the gate logits of a token are x_t W1 W2 + b
// with W1: d_model x rank and W2: rank x (NH*dk).  Two kernels, both on the
// matrix cores:
//
//  gla_gate_rank_kernel    hp = x W1 only: rank values per token (binary32,
//                          64 bytes per token at rank 16).  The single pass
//                          reads these and expands them with W2 and b itself,
//                          so the NH*dk logits of a token never reach memory.
//  gla_gate_logits_kernel  z = (x W1) W2 + b written out: NH*dk binary32
//                          values per token (gla_gate_logits, and the staged
//                          path of every configuration the single pass does
//                          not cover).
//
// Products:
//   1. hp^T = W1^T x^T per 16-row rank tile, accumulated in binary32 over
//      d_model (binary16 storage: v_mfma_f32_16x16x32_f16; binary32 storage:
//      v_mfma_f32_16x16x4_f32), one wavefront per 16 tokens, with KB
//      k-steps fetched per batch so that their loads are in flight together
//      (d_model <= 512 at rank 16 is one batch).  Lane (l16, g) ends with
//      hp[token l16][16 rt + 4 g + e], e = 0..3.
//   2. z^T = W2^T hp^T + b per 16-row output tile with v_mfma_f32_16x16x4_f32:
//      at step (rt, e) the k = g element of the 4-deep contraction is rank
//      16 rt + 4 g + e, which is element e of the lane's own hp fragment, so
//      step 1's accumulators feed the B operand directly.  Lane (l16, g) ends
//      with z[token l16][o0 + 4g .. o0 + 4g + 3] and stores 16 bytes.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"
#include "gla_launch.h"

namespace gla {
namespace proj {

constexpr int kMaxRankTiles = 4;  // rank <= 64
constexpr int kOutTiles = 4;      // 16-row output tiles per wavefront (logits kernel)

// One fragment of x (token row) or W1 (rank row) for k-step s.  KB k-steps
// are fetched per batch: as many as keep the batch's fragments within about
// 128 registers for NRT rank tiles.
template <typename T, int NRT> struct Frag;
template <int NRT> struct Frag<_Float16, NRT> {
    typedef half8 type;
    static constexpr int KSTEP = 32, KB = NRT == 1 ? 16 : NRT == 2 ? 8 : 4;
    // elements 32 s + 8 g .. +7 of a row of n elements (n a multiple of 8)
    static __device__ __forceinline__ half8 load(const _Float16* row, int n, int s, int g, bool ok)
    {
        const int m = KSTEP * s + 8 * g;
        if (!ok || m >= n) return half8{0, 0, 0, 0, 0, 0, 0, 0};
        return *(const half8*)(row + m);
    }
};
template <int NRT> struct Frag<float, NRT> {
    typedef float type;
    static constexpr int KSTEP = 4, KB = NRT == 1 ? 48 : NRT == 2 ? 32 : 16;
    static __device__ __forceinline__ float load(const float* row, int n, int s, int g, bool ok)
    {
        const int m = KSTEP * s + g;
        if (!ok || m >= n) return 0.f;
        return row[m];
    }
};

// Step 1 for the 16 tokens tok0 .. tok0 + 15 (rows past `tokens` read as 0)
// and NRT = ceil(rank / 16) rank tiles.
template <typename T, int NRT>
__device__ __forceinline__ void rank_tiles(const T* __restrict__ x, const T* __restrict__ w1,
                                           int tok0, int tokens, int d_model, int rank, int l16,
                                           int g, float4v (&hp)[NRT])
{
    typedef typename Frag<T, NRT>::type frag;
    constexpr int KB = Frag<T, NRT>::KB;
    const int tok = tok0 + l16;
    const bool tv = tok < tokens;
    const T* xrow = x + (size_t)(tv ? tok : tok0) * d_model;
    const int ksteps = (d_model + Frag<T, NRT>::KSTEP - 1) / Frag<T, NRT>::KSTEP;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) hp[rt] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ksteps; s0 += KB) {
        frag b[KB], a[KB][NRT];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            b[u] = Frag<T, NRT>::load(xrow, d_model, s0 + u, g, tv);
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int j = 16 * rt + l16;
                a[u][rt] = Frag<T, NRT>::load(w1 + (size_t)(j < rank ? j : 0) * d_model, d_model,
                                              s0 + u, g, j < rank);
            }
        }
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) hp[rt] = mma(a[u][rt], b[u], hp[rt]);
    }
}

// hp = x W1: [tokens][ld] binary32, ld = 16 NRT (columns past rank hold 0).
template <typename T, int NRT>
__global__ __launch_bounds__(256) void gla_gate_rank_kernel(const T* __restrict__ x,
                                                            const T* __restrict__ w1,
                                                            float* __restrict__ hpo, int tokens,
                                                            int d_model, int rank)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int tok0 = (blockIdx.x * 4 + wave) * 16;
    if (tok0 >= tokens) return;
    float4v hp[NRT];
    rank_tiles<T, NRT>(x, w1, tok0, tokens, d_model, rank, l16, g, hp);
    const int tok = tok0 + l16;
    if (tok >= tokens) return;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
        *(float4v*)(hpo + (size_t)tok * (16 * NRT) + 16 * rt + 4 * g) = hp[rt];
}

// z = (x W1) W2 + b: [tokens][nout] binary32.  A wavefront takes 16 tokens
// and kOutTiles * 16 output rows (one head at dk = 64), so a call spreads
// over (tokens / 16) x (nout / 64) wavefronts; each recomputes the small
// first product of its tokens.  Every W2 and bias value a wavefront needs is
// loaded before its first expansion product.
template <typename T, int NRT>
__global__ __launch_bounds__(256) void gla_gate_logits_kernel(const T* __restrict__ x,
                                                              const T* __restrict__ w1,
                                                              const float* __restrict__ w2,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ z, int tokens,
                                                              int d_model, int rank, int nout)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int ngroups = (nout + 16 * kOutTiles - 1) / (16 * kOutTiles);
    const int id = blockIdx.x * 4 + wave;
    const int tb = id / ngroups, og = id - tb * ngroups;
    const int tok0 = tb * 16;
    if (tok0 >= tokens) return;
    const int tok = tok0 + l16;
    // W2 A fragments (row o0 + l16, ranks 16 rt + 4 g + e) and bias
    float wv[kOutTiles][NRT][4];
    float4v acc[kOutTiles];
#pragma unroll
    for (int t = 0; t < kOutTiles; ++t) {
        const int o0 = (og * kOutTiles + t) * 16;
        const bool ok = o0 < nout;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] = (ok && bias) ? bias[o0 + 4 * g + e] : 0.f;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * rt + 4 * g + e;
                wv[t][rt][e] = (ok && j < rank) ? w2[(size_t)(o0 + l16) * rank + j] : 0.f;
            }
    }
    float4v hp[NRT];
    rank_tiles<T, NRT>(x, w1, tok0, tokens, d_model, rank, l16, g, hp);
#pragma unroll
    for (int t = 0; t < kOutTiles; ++t)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t] = mma(wv[t][rt][e], hp[rt][e], acc[t]);
    if (tok < tokens) {
#pragma unroll
        for (int t = 0; t < kOutTiles; ++t) {
            const int o0 = (og * kOutTiles + t) * 16;
            if (o0 < nout) *(float4v*)(z + (size_t)tok * nout + o0 + 4 * g) = acc[t];
        }
    }
}

}  // namespace proj

namespace {

template <typename T, int NRT>
void launch_logits_t(const GateProj& G, int tokens, int nout, float* z, hipStream_t st)
{
    const long long groups = (nout + 16 * proj::kOutTiles - 1) / (16 * proj::kOutTiles);
    const long long waves = (long long)((tokens + 15) / 16) * groups;
    hipLaunchKernelGGL((proj::gla_gate_logits_kernel<T, NRT>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, st, (const T*)G.x, (const T*)G.w1, G.w2, G.bias, z, tokens,
                       G.d_model, G.rank, nout);
}

template <typename T, int NRT>
void launch_rank_t(const GateProj& G, int tokens, float* hp, hipStream_t st)
{
    hipLaunchKernelGGL((proj::gla_gate_rank_kernel<T, NRT>), dim3((unsigned)((tokens + 63) / 64)),
                       dim3(256), 0, st, (const T*)G.x, (const T*)G.w1, hp, tokens, G.d_model,
                       G.rank);
}

template <typename T>
void launch_logits_d(const GateProj& G, int tokens, int nout, float* z, hipStream_t st)
{
    switch ((G.rank + 15) / 16) {
    case 1: launch_logits_t<T, 1>(G, tokens, nout, z, st); break;
    case 2: launch_logits_t<T, 2>(G, tokens, nout, z, st); break;
    case 3: launch_logits_t<T, 3>(G, tokens, nout, z, st); break;
    default: launch_logits_t<T, 4>(G, tokens, nout, z, st); break;
    }
}

template <typename T>
void launch_rank_d(const GateProj& G, int tokens, float* hp, hipStream_t st)
{
    switch ((G.rank + 15) / 16) {
    case 1: launch_rank_t<T, 1>(G, tokens, hp, st); break;
    case 2: launch_rank_t<T, 2>(G, tokens, hp, st); break;
    case 3: launch_rank_t<T, 3>(G, tokens, hp, st); break;
    default: launch_rank_t<T, 4>(G, tokens, hp, st); break;
    }
}

}  // namespace

int launch_gate_logits(const GateProj& G, int dtype, int tokens, int nout, float* z, void* stream)
{
    if (tokens <= 0) return GLA_OK;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GLA_F16) launch_logits_d<_Float16>(G, tokens, nout, z, st);
    else launch_logits_d<float>(G, tokens, nout, z, st);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

int launch_gate_rank(const GateProj& G, int dtype, int tokens, float* hp, void* stream)
{
    if (tokens <= 0) return GLA_OK;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GLA_F16) launch_rank_d<_Float16>(G, tokens, hp, st);
    else launch_rank_d<float>(G, tokens, hp, st);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

}  // namespace gla
