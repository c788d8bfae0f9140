// gla_bwd.hip -- chunkwise backward of key-only gated linear attention
// (no output gate) for gfx950.
//
// Paper "GTR: Gated Token Recurrence for Efficient Dense Prediction",
// Section 2.1: S_t = Diag(gamma_t) S_{t-1} + k_t^T v_t, o_t = s q_t S_t,
// gamma_t = sigmoid(z_t)^(1/tau).  Given dO, with b_t the cumulative log2
// decay along the scan and dS_t = sum_{u >= t} 2^{b_u - b_t} (.) s q_u^T dO_u:
//     dq_t = s dO_t S_t^T                 (decay on the output channel)
//     dk_t = dS_t v_t^T,  dv_t = k_t dS_t
//     dz_t = (1 - sigmoid(z_t)) / tau (.) sum_{u >= t} (q_u (.) dq_u - k_u (.) dk_u)
// (the last because L depends on b only through q (.) 2^b and k (.) 2^-b).
//
// Passes, chunks of C = 64 scan positions, one workgroup (4 wavefronts) each:
//   1. forward chunk-entry states S_in (the forward's aggregate and fold
//      passes with one-chunk segments, gla_kernel.hip);
//   2. reverse aggregates RA_c = s (q (.) 2^{b - b_start})^T dO per chunk and
//      the chunk's log2 decay (gla_bwd_agg_kernel), folded from the end of the
//      scan: R_c = RA_{c+1} + 2^{G_{c+1}} (.) R_{c+1} (gla_bwd_fold_kernel), the
//      gradient entering chunk c from the later tokens;
//   3. the chunk kernel (gla_bwd_chunk_kernel): dq, dk, dv of the chunk and the
//      chunk-local reverse sums of q (.) dq - k (.) dk;
//   4. gla_bwd_dz_kernel: adds the later chunks' sums and the gate derivative.
// Inside a chunk, with sub-chunks i of 16 positions and c_i the cumulative
// decay at the end of sub-chunk i (c_{-1} = 0), every factor applied to an
// operand is a power of two with exponent <= 0 except inside the diagonal
// sub-chunk block:
//   dq_i = 2^{b - c_{i-1}} (.) [ sum_{j<i} 2^{c_{i-1} - c_j} (.) P_ij (K (.) 2^{c_j - b})_j
//                                + P_ii (K (.) 2^{c_{i-1} - b})_i + s 2^{c_{i-1}} (.) dO_i S_in^T ]
//   dk_i = 2^{c_i - b} (.) [ sum_{j>i} 2^{c_{j-1} - c_i} (.) P_ji^T (Q (.) 2^{b - c_{j-1}})_j
//                            + P_ii^T (Q (.) 2^{b - c_i})_i + 2^{B - c_i} (.) V_i R^T ]
//   dv_i = sum_{j>=i} A_ji^T dO_j + (K (.) 2^{B - b})_i R
// with P = s dO V^T (lower block triangle), A_ji the decayed scores s q_u k_t
// 2^{b_u - b_t} (u in j, t in i, u >= t) and B the chunk's total decay.  All
// products run on v_mfma_f32_16x16x4_f32 (binary32 operands and sums).  The
// diagonal blocks carry factors up to 2^{c_{i-1} - c_i}; a sub-chunk whose
// decay exceeds 2^60 on some channel evaluates its diagonal blocks pair by
// pair instead, each pair's factor 2^{b_u - b_t} <= 1 taken directly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"
#include "gla_geometry.h"
#include "gla_launch.h"

namespace gla {
namespace bwd {

constexpr int C = 64;   // chunk
constexpr int NS = 4;   // 16-position sub-chunks
constexpr int NT = 256; // 4 wavefronts

template <int D> struct Lay {
    static constexpr int SD = D + 4;        // row stride (floats), [C][D] and [D][D] tiles
    static constexpr int SC = C + 4;        // row stride of the [C][C] tile
    static constexpr int TILE = C * SD;
    static constexpr int P = 0;             // s dO V^T            [C][SC]
    static constexpr int DO = P + C * SC;   // dO                  [C][SD]
    static constexpr int V = DO + TILE;     // v
    static constexpr int KT = V + TILE;     // k (.) 2^{c_i - b}
    static constexpr int KB = KT + TILE;    // k (.) 2^{c_{i-1} - b}; then q (.) 2^{b - c_i}
    static constexpr int SS = KB + TILE;    // S_in [D][SD]; then R [D][SD]
    static constexpr int QH = SS + D * SD;  // q (.) 2^{b - c_{i-1}}
    static constexpr int BB = QH + TILE;    // a, then b (log2 decay from the chunk start, inclusive)
    static constexpr int CB = BB + TILE;    // c_{i-1}: [NS + 1][D], row 0 = 0
    static constexpr int TOTAL = CB + (NS + 1) * D;  // floats
    static constexpr int ROWS = TOTAL;      // int rows [C]
    static constexpr int FLAGS = ROWS + C;  // int per sub-chunk: pairwise diagonal
    static constexpr int WORDS = FLAGS + NS;
    static constexpr int BYTES = WORDS * 4;
    // aggregate kernel: q, dO, a/b tiles and the rows
    static constexpr int A_Q = 0, A_DO = TILE, A_B = 2 * TILE, A_ROWS = 3 * TILE;
    static constexpr int A_WORDS = A_ROWS + C;
};
static_assert(Lay<64>::BYTES <= kLdsLimit, "LDS budget of one CU exceeded");
// Largest per-channel decay span (log2) of a sub-chunk whose diagonal blocks
// take the factorised product: operands grow by at most 2^60.
constexpr float kDiagSpan = 60.0f;

// One element of a [rows][D] tensor as binary32 (0 for row < 0).
template <typename T>
__device__ __forceinline__ float ld1(const void* base, int row, int D, int col)
{
    return row < 0 ? 0.f : (float)((const T*)base)[(size_t)row * D + col];
}

// Load 8 consecutive elements of a row as binary32 (zeros for row < 0).
template <typename T>
__device__ __forceinline__ void load8(const T* base, int row, int D, int col, float (&x)[8])
{
    if (row < 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
        return;
    }
    const T* p = base + (size_t)row * D + col;
    if constexpr (sizeof(T) == 2) {
        const half8 h = *(const half8*)p;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)h[e];
    } else {
        const float4v a = *(const float4v*)p, b = *(const float4v*)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    }
}

template <typename T>
__device__ __forceinline__ void store1(T* base, size_t idx, float x)
{
    base[idx] = (T)x;
}

// Chunk geometry shared by the aggregate and chunk kernels: row table, the
// gate stage and raw tiles.  Loads q into `tq`, k into `tk`, v into `tv`, dO
// into `tdo` (each [C][SD] binary32, any may be null) and the clamped per-token
// log2 decay a into `ta` (0 past the end).
template <typename T, int D>
__device__ __forceinline__ void load_chunk(const Params& P, const BwdParams& Q, int unit, int c, int tid,
                                           int* sRows, float* tq, float* tk, float* tv, float* tdo,
                                           float* ta)
{
    constexpr int SD = Lay<D>::SD;
    for (int i = tid; i < C; i += NT) sRows[i] = scan_row(P, unit, c * C + i);
    __syncthreads();
    constexpr int G8 = D / 8;
    for (int i = tid; i < C * G8; i += NT) {
        const int t = i / G8, c8 = 8 * (i - t * G8);
        const int row = sRows[t];
        float x[8];
        if (tq) {
            load8<T>((const T*)P.q, row, D, c8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) tq[t * SD + c8 + e] = x[e];
        }
        if (tk) {
            load8<T>((const T*)P.k, row, D, c8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) tk[t * SD + c8 + e] = x[e];
        }
        if (tv) {
            load8<T>((const T*)P.v, row, D, c8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) tv[t * SD + c8 + e] = x[e];
        }
        if (tdo) {
            load8<T>((const T*)Q.dout, row, D, c8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) tdo[t * SD + c8 + e] = x[e];
        }
        load8<float>(P.z, row, D, c8, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ta[t * SD + c8 + e] = row >= 0 ? log2_decay(x[e], P.inv_tau) : 0.f;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Reverse aggregates: slot c - 1 <- (RA_c, G_c) for chunks c >= 1.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NT) void gla_bwd_agg_kernel(Params P, BwdParams Q)
{
    using Y = Lay<D>;
    constexpr int SD = Y::SD;
    __shared__ __attribute__((aligned(16))) float lds[Y::A_WORDS];
    float* sQ = lds + Y::A_Q;
    float* sDO = lds + Y::A_DO;
    float* sA = lds + Y::A_B;
    int* sRows = (int*)(lds + Y::A_ROWS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int units = P.B * P.NH;
    const int unit = blockIdx.x % units;
    const int c = 1 + blockIdx.x / units;
    load_chunk<T, D>(P, Q, unit, c, tid, sRows, sQ, nullptr, nullptr, sDO, sA);
    // cumulative decay from the chunk start (inclusive), q (.) 2^{b}
    float* slot = Q.ws_r + ((size_t)unit * (P.nchunks - 1) + (c - 1)) * ((size_t)D * D + D);
    for (int ch = tid; ch < D; ch += NT) {
        float b = 0.f;
        for (int t = 0; t < C; ++t) {
            b += sA[t * SD + ch];
            sQ[t * SD + ch] *= exp2_fast(b);
        }
        slot[D * D + ch] = b;  // log2 decay of the whole chunk
    }
    __syncthreads();
    // RA = s Qt^T dO: tile (a, bb), a over key channels, bb over value channels
    constexpr int NTL = D / 16;
    for (int tile = wave; tile < NTL * NTL; tile += NT / 64) {
        const int a = tile / NTL, bb = tile - a * NTL;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int ks = 0; ks < C / 4; ++ks) {
            const int u = 4 * ks + g;
            acc = mma(sQ[u * SD + 16 * a + l16], sDO[u * SD + 16 * bb + l16], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) slot[(size_t)(16 * a + 4 * g + e) * D + 16 * bb + l16] = P.scale * acc[e];
    }
}

// Reverse fold: slot s <- R_s = RA_{s+1} + 2^{G_{s+1}} (.) R_{s+1}, R_{last} = 0.
template <int D>
__global__ __launch_bounds__(NT) void gla_bwd_fold_kernel(Params P, BwdParams Q)
{
    constexpr int ENTRIES = D * D;
    constexpr int BLKS = (ENTRIES + NT - 1) / NT;
    const int unit = blockIdx.x / BLKS;
    const int idx = (blockIdx.x - unit * BLKS) * NT + threadIdx.x;
    if (idx >= ENTRIES) return;
    const int ch = idx / D;
    const size_t slot_floats = (size_t)D * D + D;
    const int nslot = P.nchunks - 1;
    float* base = Q.ws_r + (size_t)unit * nslot * slot_floats;
    float x = 0.f;
    for (int s = nslot - 1; s >= 0; --s) {
        x = exp2_fast(base[(size_t)s * slot_floats + ENTRIES + ch]) * x + base[(size_t)s * slot_floats + idx];
        base[(size_t)s * slot_floats + idx] = x;
    }
}

// ---------------------------------------------------------------------------
// Diagonal blocks pair by pair (sub-chunks whose decay span exceeds 2^60).
// Raw q and k come from global memory; b from LDS.  Every factor is
// 2^{min(b_u - b_t, 0)}: pairs outside the causal triangle meet a zero score.
// ---------------------------------------------------------------------------

// dq_t += sum_{tau <= t, same sub-chunk} P[t][tau] k_tau 2^{b_t - b_tau}
// for t = 16 si + 4 g + e, channel ch.
template <typename T, int D>
__device__ __forceinline__ void diag_dq(const Params& P, const int* sRows, const float* sP,
                                        const float* sB, int si, int g, int ch, float (&out)[4])
{
    constexpr int SD = Lay<D>::SD, SC = Lay<D>::SC;
    float kr[16], bk[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        kr[x] = ld1<T>(P.k, sRows[16 * si + x], D, ch);
        bk[x] = sB[(16 * si + x) * SD + ch];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 16 * si + 4 * g + e;
        const float bt = sB[t * SD + ch];
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x)
            acc += sP[t * SC + 16 * si + x] * kr[x] * exp2_fast(fminf(bt - bk[x], 0.f));
        out[e] = acc;
    }
}

// dk_t += sum_{u >= t, same sub-chunk} P[u][t] q_u 2^{b_u - b_t}.
template <typename T, int D>
__device__ __forceinline__ void diag_dk(const Params& P, const int* sRows, const float* sP,
                                        const float* sB, int si, int g, int ch, float (&out)[4])
{
    constexpr int SD = Lay<D>::SD, SC = Lay<D>::SC;
    float qr[16], bq[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        qr[x] = ld1<T>(P.q, sRows[16 * si + x], D, ch);
        bq[x] = sB[(16 * si + x) * SD + ch];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 16 * si + 4 * g + e;
        const float bt = sB[t * SD + ch];
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x)
            acc += sP[(16 * si + x) * SC + t] * qr[x] * exp2_fast(fminf(bq[x] - bt, 0.f));
        out[e] = acc;
    }
}

// A[u][t] = s sum_ch q_u k_t 2^{b_u - b_t} for u = 16 si + 4 g + e >= t = 16 si + l16.
template <typename T, int D>
__device__ __forceinline__ float4v diag_scores(const Params& P, const int* sRows, const float* sB,
                                               int si, int g, int l16)
{
    constexpr int SD = Lay<D>::SD;
    const int t = 16 * si + l16;
    const int rt = sRows[t];
    float4v a = {0.f, 0.f, 0.f, 0.f};
    for (int c8 = 0; c8 < D; c8 += 8) {
        float kk[8];
        load8<T>((const T*)P.k, rt, D, c8, kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 16 * si + 4 * g + e;
            float qq[8];
            load8<T>((const T*)P.q, sRows[u], D, c8, qq);
#pragma unroll
            for (int x = 0; x < 8; ++x)
                a[e] += qq[x] * kk[x] * exp2_fast(fminf(sB[u * SD + c8 + x] - sB[t * SD + c8 + x], 0.f));
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (4 * g + e >= l16) ? P.scale * a[e] : 0.f;
    return a;
}

// ---------------------------------------------------------------------------
// Chunk kernel: dq, dk, dv and the chunk-local reverse sums for dz.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(NT) void gla_bwd_chunk_kernel(Params P, BwdParams Q)
{
    using Y = Lay<D>;
    constexpr int SD = Y::SD, SC = Y::SC, NTL = D / 16, KS = D / 4;
    __shared__ __attribute__((aligned(16))) float lds[Y::WORDS];
    float* sP = lds + Y::P;
    float* sDO = lds + Y::DO;
    float* sV = lds + Y::V;
    float* sKT = lds + Y::KT;
    float* sKB = lds + Y::KB;
    float* sSS = lds + Y::SS;
    float* sQH = lds + Y::QH;
    float* sB = lds + Y::BB;
    float* sCB = lds + Y::CB;
    int* sRows = (int*)(lds + Y::ROWS);
    int* sFlag = (int*)(lds + Y::FLAGS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int units = P.B * P.NH;
    const int unit = blockIdx.x % units;
    const int c = blockIdx.x / units;
    const int si = wave;  // this wave's sub-chunk
    const float s = P.scale;
    const size_t slot_floats = (size_t)D * D + D;
    const bool has_in = c > 0;                 // a state enters from earlier chunks
    const bool has_r = c < P.nchunks - 1;      // a gradient enters from later chunks
    if (tid < NS) sFlag[tid] = 0;

    // raw q -> QH, k -> KT, v, dO, a -> BB (the loader's barriers order the flags)
    load_chunk<T, D>(P, Q, unit, c, tid, sRows, sQH, sKT, sV, sDO, sB);

    // ---- gate: thread (ch, i) runs over the 16 positions of sub-chunk i
    const bool gate_thread = tid < D * NS;
    const int gch = tid % D, gi = tid / D;
    float qr[16], br[16];
    if (gate_thread) {
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            run += sB[(16 * gi + u) * SD + gch];
            br[u] = run;  // within the sub-chunk
        }
        sCB[(gi + 1) * D + gch] = run;  // sub-chunk total, turned into c_i below
        if (run < -kDiagSpan) sFlag[gi] = 1;
    }
    if (tid < D) sCB[tid] = 0.f;
    __syncthreads();
    float off = 0.f, ci = 0.f;
    if (gate_thread) {
        for (int m = 0; m < gi; ++m) off += sCB[(m + 1) * D + gch];
        ci = off + sCB[(gi + 1) * D + gch];
    }
    __syncthreads();
    if (gate_thread) {
        sCB[(gi + 1) * D + gch] = ci;  // c_i; row 0 = c_{-1} = 0
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * gi + u;
            const float b = br[u] + off;  // cumulative from the chunk start
            br[u] = b;
            qr[u] = sQH[t * SD + gch];
            const float k = sKT[t * SD + gch];
            sQH[t * SD + gch] = qr[u] * exp2_fast(b - off);  // <= 1
            sKT[t * SD + gch] = k * exp2_fast(ci - b);       // <= 1
            sKB[t * SD + gch] = k * exp2_fast(off - b);      // >= 1 (diagonal block)
            sB[t * SD + gch] = b;
        }
    }
    // S_in (state entering this chunk) -> SS, zero for the first chunk
    if (has_in) {
        const float* src = Q.ws_f + ((size_t)unit * (P.nchunks - 1) + (c - 1)) * slot_floats;
        for (int i = tid; i < D * D; i += NT) {
            const int r = i / D, cc = i - r * D;
            sSS[r * SD + cc] = src[i];
        }
    }
    __syncthreads();
    const bool pairwise = sFlag[si] != 0;  // wave-uniform

    // ---- P = s dO V^T on the blocks j <= i, diagonal blocks masked to u >= t
    for (int j = 0; j <= si; ++j) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int ks = 0; ks < KS; ++ks) {
            const int col = 4 * ks + g;
            acc = mma(sDO[(16 * si + l16) * SD + col], sV[(16 * j + l16) * SD + col], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 4 * g + e;
            sP[(16 * si + u) * SC + 16 * j + l16] = (j == si && l16 > u) ? 0.f : s * acc[e];
        }
    }
    __syncthreads();

    // ---- dq of sub-chunk si (rows 16 si + 4g + e, columns 16 ct + l16)
    float dqv[NTL][4];
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
        const int ch = 16 * ct + l16;
        const float cim1 = sCB[si * D + ch];
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j <= si; ++j) {
            if (j == si && pairwise) break;
            const float* kt = (j == si) ? sKB : sKT;
            float4v m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int sp = 16 * j + 4 * ks + g;
                m = mma(sP[(16 * si + l16) * SC + sp], kt[sp * SD + ch], m);
            }
            const float f = (j == si) ? 1.f : exp2_fast(cim1 - sCB[(j + 1) * D + ch]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += m[e] * f;
        }
        if (has_in) {
            float4v m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int ks = 0; ks < KS; ++ks) {
                const int jj = 4 * ks + g;
                m = mma(sDO[(16 * si + l16) * SD + jj], sSS[ch * SD + jj], m);
            }
            const float f = s * exp2_fast(cim1);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += m[e] * f;
        }
        float dg[4] = {0.f, 0.f, 0.f, 0.f};
        if (pairwise) diag_dq<T, D>(P, sRows, sP, sB, si, g, ch, dg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * si + 4 * g + e;
            dqv[ct][e] = acc[e] * exp2_fast(sB[t * SD + ch] - cim1) + dg[e];
            const int row = sRows[t];
            if (row >= 0) store1<T>((T*)Q.dq, (size_t)row * D + ch, dqv[ct][e]);
        }
    }
    __syncthreads();

    // ---- phase B tiles: R -> SS, q (.) 2^{b - c_i} -> KB
    if (has_r) {
        const float* src = Q.ws_r + ((size_t)unit * (P.nchunks - 1) + c) * slot_floats;
        for (int i = tid; i < D * D; i += NT) {
            const int r = i / D, cc = i - r * D;
            sSS[r * SD + cc] = src[i];
        }
    }
    if (gate_thread) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * gi + u;
            sKB[t * SD + gch] = qr[u] * exp2_fast(br[u] - ci);  // >= 1 (diagonal block)
        }
    }
    __syncthreads();

    // ---- dk of sub-chunk si
    float dkv[NTL][4];
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
        const int ch = 16 * ct + l16;
        const float cic = sCB[(si + 1) * D + ch];
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = pairwise ? si + 1 : si; j < NS; ++j) {
            const float* qh = (j == si) ? sKB : sQH;
            float4v m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int up = 16 * j + 4 * ks + g;
                m = mma(sP[up * SC + 16 * si + l16], qh[up * SD + ch], m);
            }
            const float f = (j == si) ? 1.f : exp2_fast(sCB[j * D + ch] - cic);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += m[e] * f;
        }
        if (has_r) {
            float4v m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int ks = 0; ks < KS; ++ks) {
                const int jj = 4 * ks + g;
                m = mma(sV[(16 * si + l16) * SD + jj], sSS[ch * SD + jj], m);
            }
            const float f = exp2_fast(sCB[NS * D + ch] - cic);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += m[e] * f;
        }
        float dg[4] = {0.f, 0.f, 0.f, 0.f};
        if (pairwise) diag_dk<T, D>(P, sRows, sP, sB, si, g, ch, dg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * si + 4 * g + e;
            dkv[ct][e] = acc[e] * exp2_fast(cic - sB[t * SD + ch]) + dg[e];
            const int row = sRows[t];
            if (row >= 0) store1<T>((T*)Q.dk, (size_t)row * D + ch, dkv[ct][e]);
        }
    }

    // ---- dv of sub-chunk si: sum_{j >= si} A_ji^T dO_j + (K (.) 2^{B - b})_si R
    float4v dvacc[NTL];
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) dvacc[ct] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int j = si; j < NS; ++j) {
        // A_ji[u = 16 j + 4g + e][t = 16 si + l16]
        float4v a = {0.f, 0.f, 0.f, 0.f};
        if (j == si && pairwise) {
            a = diag_scores<T, D>(P, sRows, sB, si, g, l16);
        } else {
            const float* qh = (j == si) ? sKB : sQH;
#pragma unroll 4
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = 4 * ks + g;
                const float f = (j == si) ? 1.f : exp2_fast(sCB[j * D + ch] - sCB[(si + 1) * D + ch]);
                a = mma(qh[(16 * j + l16) * SD + ch], sKT[(16 * si + l16) * SD + ch] * f, a);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool keep = (j > si) || (4 * g + e >= l16);
                a[e] = keep ? s * a[e] : 0.f;
            }
        }
        // dv[t][col] += sum_u A[u][t] dO[u][col], k-slot g of step e is u = 16 j + 4g + e
#pragma unroll
        for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dvacc[ct] = mma(a[e], sDO[(16 * j + 4 * g + e) * SD + 16 * ct + l16], dvacc[ct]);
    }
    if (has_r) {
#pragma unroll
        for (int ct = 0; ct < NTL; ++ct) {
#pragma unroll 4
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = 4 * ks + g;
                const float kf = sKT[(16 * si + l16) * SD + ch] *
                                 exp2_fast(sCB[NS * D + ch] - sCB[(si + 1) * D + ch]);
                dvacc[ct] = mma(kf, sSS[ch * SD + 16 * ct + l16], dvacc[ct]);
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = sRows[16 * si + 4 * g + e];
            if (row >= 0) store1<T>((T*)Q.dv, (size_t)row * D + 16 * ct + l16, dvacc[ct][e]);
        }
    __syncthreads();  // every reader of P and CB is done: reuse them

    // ---- q (.) dq - k (.) dk into P ([C][SD] view), raw q and k reloaded
    float* sZ = sP;
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * si + 4 * g + e, ch = 16 * ct + l16;
            const int row = sRows[t];
            sZ[t * SD + ch] = ld1<T>(P.q, row, D, ch) * dqv[ct][e] - ld1<T>(P.k, row, D, ch) * dkv[ct][e];
        }
    __syncthreads();
    // reverse sums inside the chunk: thread (ch, i) over sub-chunk i
    if (gate_thread) {
        float run = 0.f;
#pragma unroll
        for (int u = 15; u >= 0; --u) {
            run += sZ[(16 * gi + u) * SD + gch];
            br[u] = run;
        }
        sCB[gi * D + gch] = run;  // sub-chunk total
    }
    __syncthreads();
    if (gate_thread) {
        float later = 0.f;
        for (int m = gi + 1; m < NS; ++m) later += sCB[m * D + gch];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int row = sRows[16 * gi + u];
            if (row >= 0) Q.dz[(size_t)row * D + gch] = br[u] + later;
        }
        if (gi == 0) Q.ws_s[((size_t)unit * P.nchunks + c) * D + gch] = br[0] + later;  // chunk total
    }
}

// dz = (1 - sigmoid(z)) / tau (.) (in-chunk reverse sum + later chunks' totals);
// 1 - sigmoid(z) evaluated as sigmoid(-z).
template <int D>
__global__ __launch_bounds__(NT) void gla_bwd_dz_kernel(Params P, BwdParams Q)
{
    __shared__ float carry[D];
    const int units = P.B * P.NH;
    const int unit = blockIdx.x % units;
    const int c = blockIdx.x / units;
    for (int ch = threadIdx.x; ch < D; ch += NT) {
        float x = 0.f;
        for (int cc = P.nchunks - 1; cc > c; --cc) x += Q.ws_s[((size_t)unit * P.nchunks + cc) * D + ch];
        carry[ch] = x;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < C * D; i += NT) {
        const int ch = i % D, t = i / D;
        const int row = scan_row(P, unit, c * C + t);
        if (row < 0) continue;
        const size_t idx = (size_t)row * D + ch;
        const float nsig = rcp_fast(1.0f + exp2_fast(P.z[idx] * kLog2e));
        Q.dz[idx] = (Q.dz[idx] + carry[ch]) * nsig * P.inv_tau;
    }
}

template <typename T, int D>
static int run_bwd(const Params& P, const BwdParams& Q, hipStream_t st)
{
    const unsigned units = (unsigned)(P.B * P.NH);
    if (P.nchunks > 1) {
        const int rs = launch_fwd_states(P, sizeof(T) == 2 ? GLA_F16 : GLA_F32, D, st);
        if (rs != GLA_OK) return rs;
        hipLaunchKernelGGL((gla_bwd_agg_kernel<T, D>), dim3(units * (P.nchunks - 1)), dim3(NT), 0, st, P, Q);
        constexpr unsigned blks = (D * D + NT - 1) / NT;
        hipLaunchKernelGGL((gla_bwd_fold_kernel<D>), dim3(units * blks), dim3(NT), 0, st, P, Q);
    }
    hipLaunchKernelGGL((gla_bwd_chunk_kernel<T, D>), dim3(units * P.nchunks), dim3(NT), 0, st, P, Q);
    hipLaunchKernelGGL((gla_bwd_dz_kernel<D>), dim3(units * P.nchunks), dim3(NT), 0, st, P, Q);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

template <typename T>
static int run_bwd_d(const Params& P, const BwdParams& Q, int d, hipStream_t st)
{
    switch (d) {
    case 16: return run_bwd<T, 16>(P, Q, st);
    case 32: return run_bwd<T, 32>(P, Q, st);
    case 64: return run_bwd<T, 64>(P, Q, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace bwd

int launch_bwd(const Params& P, const BwdParams& Q, int dtype, int d, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GLA_F16) return bwd::run_bwd_d<_Float16>(P, Q, d, st);
    if (dtype == GLA_F32) return bwd::run_bwd_d<float>(P, Q, d, st);
    return GLA_EUNSUPPORTED;
}

}  // namespace gla
