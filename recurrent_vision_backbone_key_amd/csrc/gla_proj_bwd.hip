// gla_proj_bwd.hip -- gradients of the low-rank retention-gate projection
// for gfx950.
//
// Paper "GTR: Gated Token Recurrence for Efficient Dense Prediction",
// Section 2.1 (retention gate): the gate logits are z = x W1 W2 + b, stored as
// in gla_gate_logits (W1 transposed [rank][d_model], W2 transposed
// [nout][rank], nout = heads * dk).  With hp = x W1 (the rank values of each
// token) and dz = dL/dz [tokens][nout] binary32, the chain rule gives
//     dhp = dz W2^T        [tokens][rank]
//     dx  = dhp W1^T       [tokens][d_model]   (storage type of x)
//     dW1 = dhp^T x        [rank][d_model]     (the transposed storage of W1)
//     dW2 = dz^T hp        [nout][rank]        (the transposed storage of W2)
//     db  = sum_t dz[t]    [nout]
// in binary32.  Each is a plain matrix product with a short side (the rank,
// at most 64), run by one kernel: a wavefront computes a 16 x 16 output tile
// with v_mfma_f32_16x16x4_f32, contracting 16 indices per step (lane (g, l16)
// supplies four consecutive k of its A row and B column per step); products
// over the tokens (dW1, dW2, db) are split into blocks of kSplitK tokens whose
// partial tiles are added afterwards in block order, so every result is the
// same for equal inputs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gla.h"
#include "gla_device.h"
#include "gla_launch.h"

namespace gla {
namespace pbwd {

constexpr int kSplitK = kProjBwdSplit;  // tokens per partial product

template <typename T> __device__ __forceinline__ float ldf(const T* p) { return (float)*p; }

// C[m][n] = sum_{k in this wavefront's block} A(m, k) B(k, n) with
// A(m, k) = a[m sam + k sak] and B(k, n) = b[k sbk + n sbn] (ONES: B(k, 0) = 1,
// the other columns 0).  Wavefront w takes tile w mod (tm tn) (row-major over
// the tiles) and k block w / (tm tn); it writes C[m][n] to
// c[block * M * N + m scm + n scn] as TC.  Elements outside M x N or past K
// read as 0 and are not written.  CV: rows are consecutive in memory (scm = 1)
// and M is a multiple of 4, so a lane's four rows go out in one store.
template <typename TA, typename TB, typename TC, bool ONES, int KU, bool CV>
__global__ __launch_bounds__(256) void gla_pbwd_gemm_kernel(const TA* __restrict__ a, long long sam,
                                                            long long sak, const TB* __restrict__ b,
                                                            long long sbk, long long sbn,
                                                            TC* __restrict__ c, long long scm,
                                                            long long scn, int M, int N, int K,
                                                            int kblock, int tm, int tn, long long waves)
{
    const int lane = threadIdx.x & 63;
    const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= waves) return;
    const int l16 = lane & 15, g = lane >> 4;
    const long long tiles = (long long)tm * tn;
    const int tile = (int)(w % tiles);
    const int blk = (int)(w / tiles);
    const int m0 = 16 * (tile / tn), n0 = 16 * (tile % tn);
    const int kb = blk * kblock, ke = min(K, kb + kblock);
    const int m = m0 + l16, n = n0 + l16;
    const bool mv = m < M, nv = n < N;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    // KU 16-index steps per round: every load of a round is issued before
    // its first product, so their latencies overlap
    for (int k0 = kb; k0 < ke; k0 += 16 * KU) {
        float av[KU][4], bv[KU][4];
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = k0 + 16 * u + 4 * g + e;
                const bool kv = k < ke;
                av[u][e] = (mv && kv) ? ldf(a + (long long)m * sam + (long long)k * sak) : 0.f;
                if (ONES) bv[u][e] = (kv && n == 0) ? 1.f : 0.f;
                else bv[u][e] = (kv && nv) ? ldf(b + (long long)k * sbk + (long long)n * sbn) : 0.f;
            }
        // step (u, e) contracts k = k0 + 16 u + 4 g' + e over the four lane groups g'
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mma(av[u][e], bv[u][e], acc);
    }
    TC* out = c + (long long)blk * M * N;
    if (CV) {
        typedef TC tc4 __attribute__((ext_vector_type(4)));
        const int row = m0 + 4 * g;
        if (row < M && nv)
            *(tc4*)(out + row + (long long)n * scn) = tc4{(TC)acc[0], (TC)acc[1], (TC)acc[2], (TC)acc[3]};
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = m0 + 4 * g + e;
            if (row < M && nv) out[(long long)row * scm + (long long)n * scn] = (TC)acc[e];
        }
    }
}

// out[i] = sum over the nsplit partial sums part[s * count + i] in a fixed
// order: thread (i, q) of a workgroup (64 outputs x 4 quarters) adds the
// partials of quarter q in order (eight loads in flight before their
// additions), then the four quarter sums are added in order.
__global__ __launch_bounds__(256) void gla_pbwd_reduce_kernel(const float* __restrict__ part,
                                                              float* __restrict__ out,
                                                              long long count, int nsplit)
{
    __shared__ float qs[4][64];
    const int o = threadIdx.x & 63, q = threadIdx.x >> 6;
    const long long i = (long long)blockIdx.x * 64 + o;
    const int per = (nsplit + 3) / 4;
    const int z1 = min(nsplit, (q + 1) * per);
    float s = 0.f;
    if (i < count) {
        for (int z0 = q * per; z0 < z1; z0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = z0 + u < z1 ? part[(long long)(z0 + u) * count + i] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
    }
    qs[q][o] = s;
    __syncthreads();
    if (q == 0 && i < count) out[i] = ((qs[0][o] + qs[1][o]) + qs[2][o]) + qs[3][o];
}

template <typename TA, typename TB, typename TC, bool ONES, int KU, bool CV = false>
void gemm(const TA* a, long long sam, long long sak, const TB* b, long long sbk, long long sbn, TC* c,
          long long scm, long long scn, int M, int N, int K, int kblock, hipStream_t st)
{
    const int tm = (M + 15) / 16, tn = (N + 15) / 16;
    const int nblk = (K + kblock - 1) / kblock;
    const long long waves = (long long)tm * tn * nblk;
    hipLaunchKernelGGL((gla_pbwd_gemm_kernel<TA, TB, TC, ONES, KU, CV>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, st, a, sam, sak, b, sbk, sbn, c, scm, scn, M, N, K, kblock, tm, tn,
                       waves);
}

void reduce(const float* part, float* out, long long count, int nsplit, hipStream_t st)
{
    hipLaunchKernelGGL(gla_pbwd_reduce_kernel, dim3((unsigned)((count + 63) / 64)), dim3(256), 0, st,
                       part, out, count, nsplit);
}

template <typename T>
int run(const GateProj& G, int tokens, int nout, const float* dz, void* dx, float* dw1, float* dw2,
        float* db, const ProjBwdWs& W, hipStream_t st)
{
    const int R = G.rank, RP = 16 * ((R + 15) / 16), DM = G.d_model;
    const int ns = (tokens + kSplitK - 1) / kSplitK;
    // hp = x W1 ([tokens][RP], columns past the rank 0)
    const int rs = launch_gate_rank(G, std::is_same<T, float>::value ? GLA_F32 : GLA_F16, tokens, W.hp, st);
    if (rs != GLA_OK) return rs;
    // dhp = dz W2^T: A = dz [tokens][nout], B(k = o, n = j) = w2[o][j]
    gemm<float, float, float, false, 4>(dz, nout, 1, G.w2, R, 1, W.dhp, R, 1, tokens, R, nout, nout, st);
    // dx^T = W1 dhp^T: A(m = d, k = j) = w1[j][d], B(k = j, n = t) = dhp[t][j],
    // C[d][t] = dx[t][d] (a lane's four d are consecutive: one store)
    gemm<T, float, T, false, 1, true>((const T*)G.w1, 1, DM, W.dhp, 1, R, (T*)dx, 1, DM, DM, tokens, R, R,
                                      st);
    // dW1 = dhp^T x: A(m = j, k = t) = dhp[t][j], B(k = t, n = m) = x[t][m]
    gemm<float, T, float, false, 4>(W.dhp, 1, R, (const T*)G.x, DM, 1, W.p1, DM, 1, R, DM, tokens, kSplitK,
                                    st);
    // dW2 = dz^T hp: A(m = o, k = t) = dz[t][o], B(k = t, n = j) = hp[t][j]
    gemm<float, float, float, false, 4>(dz, 1, nout, W.hp, RP, 1, W.p2, R, 1, nout, R, tokens, kSplitK, st);
    // db = dz^T 1: one output column
    gemm<float, float, float, true, 4>(dz, 1, nout, nullptr, 0, 0, W.pb, 1, 1, nout, 1, tokens, kSplitK,
                                       st);
    reduce(W.p1, dw1, (long long)R * DM, ns, st);
    reduce(W.p2, dw2, (long long)nout * R, ns, st);
    reduce(W.pb, db, nout, ns, st);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

}  // namespace pbwd

int launch_gate_proj_bwd(const GateProj& G, int dtype, int tokens, int nout, const float* dz, void* dx,
                         float* dw1, float* dw2, float* db, const ProjBwdWs& W, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GLA_F16) return pbwd::run<_Float16>(G, tokens, nout, dz, dx, dw1, dw2, db, W, st);
    if (dtype == GLA_F32) return pbwd::run<float>(G, tokens, nout, dz, dx, dw1, dw2, db, W, st);
    return GLA_EUNSUPPORTED;
}

}  // namespace gla
