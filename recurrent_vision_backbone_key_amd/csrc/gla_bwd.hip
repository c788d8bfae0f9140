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
// dz needs no pass of its own: the suffix sum from the first position f of
// chunk c+1 on equals sum_j R_c[ch][j] S_in(c+1)[ch][j] (both sides are the
// derivative of L by the log-decay at f), so the later chunks' part of dz is a
// row-wise dot product of two states known before the chunk kernel runs.
//
// Passes, chunks of C = 64 scan positions:
//   1. gla_bwd_states_kernel (4 wavefronts per chunk): the chunk's forward
//      local state L_c = sum_t 2^{B - b_t} k_t^T v_t and reverse aggregate
//      RA_c = s sum_u 2^{b_u} q_u^T dO_u with its log2 decay B (b: cumulative
//      from the chunk start, inclusive);
//   2. gla_bwd_fold_kernel: S_in(c+1) = 2^{B_c} S_in(c) + L_c along the scan,
//      R_c = RA_{c+1} + 2^{B_{c+1}} R_{c+1} back from its end, and the carry
//      sum_j R_c S_in(c+1) per channel;
//   3. gla_bwd_chunk_kernel (8 wavefronts per chunk): dq, dk, dv of the chunk
//      and dz = (1 - sigmoid(z)) / tau (.) (in-chunk reverse sum + carry).
// Inside a chunk, with sub-chunks i of 16 positions, c_i the cumulative decay
// at the end of sub-chunk i (c_{-1} = 0), for a position of sub-chunk i
// Qh = q (.) 2^{b - c_{i-1}}, Kh = k (.) 2^{c_i - b} (both <= 1 in size), and
// E_xy = 2^{c_{x-1} - c_y} per channel (x >= y; x = 4 gives the chunk decay B):
//   dq_i = 2^{b - c_{i-1}} (.) [ sum_{j<=i} E_ij (.) P_ij Kh_j + s 2^{c_{i-1}} (.) dO_i S_in^T ]
//   dk_i = 2^{c_i - b} (.) [ sum_{j>=i} E_ji (.) P_ji^T Qh_j + E_4i (.) V_i R^T ]
//   dv_i = sum_{j>=i} A_ji^T dO_j + (Kh_i (.) E_4i) R,   A_ji = s Qh_j (Kh_i (.) E_ji)^T
// with P = s dO V^T (lower block triangle, diagonal blocks masked to u >= t)
// and A_ji masked likewise.  E_xy <= 1 off the diagonal; E_ii = 2^{c_{i-1} -
// c_i} >= 1 is the diagonal blocks' factor.  All products run on
// v_mfma_f32_16x16x4_f32 (binary32 operands and sums).  A sub-chunk whose decay
// exceeds 2^60 on some channel evaluates its diagonal blocks pair by pair
// instead, each pair's factor 2^{b_u - b_t} <= 1 taken directly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"
#include "gla_epi.h"
#include "gla_geometry.h"
#include "gla_launch.h"

namespace gla {
namespace bwd {

constexpr int C = 64;     // chunk
constexpr int NS = 4;     // 16-position sub-chunks
constexpr int NT = 512;   // chunk kernel: 8 wavefronts, two per sub-chunk
constexpr int NTS = 256;  // states and fold kernels: 4 wavefronts

template <int D> struct Lay {
    static constexpr int SD = D + 4;        // row stride (floats), [C][D] and [D][D] tiles
    static constexpr int SC = C + 4;        // row stride of the [C][C] tile
    static constexpr int TILE = C * SD;
    static constexpr int P = 0;             // s dO V^T            [C][SC]
    static constexpr int DO = P + C * SC;   // dO                  [C][SD]
    static constexpr int V = DO + TILE;     // v
    static constexpr int KT = V + TILE;     // Kh = k (.) 2^{c_i - b}
    static constexpr int QH = KT + TILE;    // Qh = q (.) 2^{b - c_{i-1}}
    static constexpr int SS = QH + TILE;    // S_in [D][SD]
    static constexpr int RR = SS + D * SD;  // R [D][SD]
    static constexpr int BB = RR + D * SD;  // a, then b (log2 decay from the chunk start, inclusive)
    static constexpr int CC = BB + TILE;    // c_{i-1}: [NS + 1][D], row 0 = 0
    static constexpr int EE = CC + (NS + 1) * D;  // E_xy: [NS + 1][NS][D]
    static constexpr int TOT = EE + (NS + 1) * NS * D;  // sub-chunk sums [NS][D]
    static constexpr int TOTAL = TOT + NS * D;  // floats
    static constexpr int ROWS = TOTAL;      // int rows [C]
    static constexpr int FLAGS = ROWS + C;  // int per sub-chunk: pairwise diagonal
    static constexpr int WORDS = FLAGS + NS;
    static constexpr int BYTES = WORDS * 4;
    // states kernel: q (.) 2^b, dO, k (.) 2^{B - b}, v ([C][D] each, unpadded,
    // columns swizzled by row), sub-chunk decays, rows
    static constexpr int S_TILE = C * D;
    static constexpr int S_Q = 0, S_DO = S_TILE, S_K = 2 * S_TILE, S_V = 3 * S_TILE;
    static constexpr int S_CB = 4 * S_TILE, S_ROWS = S_CB + NS * D;
    static constexpr int S_WORDS = S_ROWS + C;
    // Element (t, col) of a states tile.  Reads take rows 4ks + g (g = 0..3)
    // and columns 16x + l16: flipping column bit 4 (D = 32) or bits 4-5
    // (D = 64) with the row's low bits puts the four rows of a read on
    // disjoint banks.
    static __device__ __forceinline__ int sidx(int t, int col)
    {
        const int sw = D >= 64 ? 16 * (t & 3) : D == 32 ? 16 * (t & 1) : 0;
        return t * D + (col ^ sw);
    }
};
static_assert(Lay<64>::BYTES <= kLdsLimit, "LDS budget of one CU exceeded");
static_assert(2 * Lay<64>::S_WORDS * 4 <= kLdsLimit, "two states workgroups per CU");
// Largest per-channel decay span (log2) of a sub-chunk whose diagonal blocks
// take the factorised product: operands grow by at most 2^60.
constexpr float kDiagSpan = 60.0f;

// One element of a [rows][D] tensor as binary32 (0 for row < 0).  Loads are
// unconditional (row 0 stands in past the end) so that a batch of them can be
// in flight together; the value is dropped afterwards.
template <typename T>
__device__ __forceinline__ float ld1(const void* base, int row, int D, int col)
{
    const float x = (float)((const T*)base)[(size_t)(row < 0 ? 0 : row) * D + col];
    return row < 0 ? 0.f : x;
}

// Load 8 consecutive elements of a row as binary32 (zeros for row < 0).
// (unconditional load, as ld1)
template <typename T>
__device__ __forceinline__ void load8(const T* base, int row, int D, int col, float (&x)[8])
{
    const T* p = base + (size_t)(row < 0 ? 0 : row) * D + col;
    const bool ok = row >= 0;
    if constexpr (sizeof(T) == 2) {
        const half8 h = *(const half8*)p;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ok ? (float)h[e] : 0.f;
    } else {
        const float4v a = *(const float4v*)p, b = *(const float4v*)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = ok ? a[e] : 0.f;
            x[4 + e] = ok ? b[e] : 0.f;
        }
    }
}

// 8 consecutive elements of a row in storage form: all loads of a thread are
// issued before any is converted, so that their latencies overlap.
template <typename T> struct Raw8;
template <> struct Raw8<_Float16> {
    u32x4 x;
    __device__ __forceinline__ void load(const _Float16* base, int row, int D, int col)
    {
        x = *(const u32x4*)(base + (size_t)(row < 0 ? 0 : row) * D + col);
    }
    // binary32 values (0 for row < 0) into dst[0..7]
    __device__ __forceinline__ void put(float* dst, bool ok) const
    {
        const half8 h = __builtin_bit_cast(half8, x);
        *(float4v*)dst = ok ? float4v{(float)h[0], (float)h[1], (float)h[2], (float)h[3]}
                            : float4v{0.f, 0.f, 0.f, 0.f};
        *(float4v*)(dst + 4) = ok ? float4v{(float)h[4], (float)h[5], (float)h[6], (float)h[7]}
                                  : float4v{0.f, 0.f, 0.f, 0.f};
    }
};
template <> struct Raw8<float> {
    float4v a, b;
    __device__ __forceinline__ void load(const float* base, int row, int D, int col)
    {
        const float* p = base + (size_t)(row < 0 ? 0 : row) * D + col;
        a = *(const float4v*)p;
        b = *(const float4v*)(p + 4);
    }
    __device__ __forceinline__ void put(float* dst, bool ok) const
    {
        *(float4v*)dst = ok ? a : float4v{0.f, 0.f, 0.f, 0.f};
        *(float4v*)(dst + 4) = ok ? b : float4v{0.f, 0.f, 0.f, 0.f};
    }
};

// Gradient outputs are written once and not read back: non-temporal stores.
template <typename T>
__device__ __forceinline__ void store1(T* base, size_t idx, float x)
{
    __builtin_nontemporal_store((T)x, base + idx);
}

// One gradient element: stored (mode 0); or, in a quarter of a d = 128 call,
// kept as a binary32 partial sum (mode 1) or added to the partial sum the
// other quarter left and stored (mode 2).
template <typename T>
__device__ __forceinline__ void put_grad(T* fin, size_t fi, float* part, size_t pi, int mode, float x)
{
    if (mode == 1) {
        part[pi] = x;
        return;
    }
    if (mode == 2) x += part[pi];
    store1<T>(fin, fi, x);
}

// ---------------------------------------------------------------------------
// Chunk states: slot c of ws_f <- (L_c, B_c) for c < nchunks - 1 and slot
// c - 1 of ws_r <- (RA_c, B_c) for c >= 1.
// ---------------------------------------------------------------------------
// T: storage type of q, k, v; TD: of dO (binary32 when it comes from the
// output gate's backward).  FWD / REV select the local states / the reverse
// aggregates (the gated backward needs the states before dO exists).
template <typename T, typename TD, int D, bool FWD, bool REV>
__global__ __launch_bounds__(NTS) void gla_bwd_states_kernel(Params P, BwdParams Q)
{
    using Y = Lay<D>;
    constexpr int NTL = D / 16;
    __shared__ __attribute__((aligned(16))) float lds[Y::S_WORDS];
    float* sQ = lds + Y::S_Q;
    float* sDO = lds + Y::S_DO;
    float* sK = lds + Y::S_K;
    float* sV = lds + Y::S_V;
    float* sCB = lds + Y::S_CB;
    int* sRows = (int*)(lds + Y::S_ROWS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int units = P.B * P.NH;
    const int unit = blockIdx.x % units;
    const int c = blockIdx.x / units;
    const bool do_r = REV && c >= 1, do_f = FWD && c < P.nchunks - 1;
    for (int i = tid; i < C; i += NTS) sRows[i] = scan_row(P, unit, c * C + i);
    __syncthreads();
    // raw tiles (q, dO for the reverse aggregate, k, v for the local state;
    // all four are fetched, every load issued before the first conversion)
    constexpr int G8 = D / 8;
    constexpr int IT = (C * G8 + NTS - 1) / NTS;
    Raw8<T> rq[IT], rk[IT], rv[IT];
    Raw8<TD> rd[IT];
    int rows[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int i = tid + it * NTS;
        const int t = (i < C * G8 ? i : 0) / G8, c8 = 8 * (i % G8);
        rows[it] = sRows[t];
        if (REV) {
            rq[it].load((const T*)P.q, rows[it], Q.ld, c8);
            rd[it].load((const TD*)Q.dout, rows[it], Q.ld, c8);
        }
        if (FWD) {
            rk[it].load((const T*)P.k, rows[it], Q.ld, c8);
            rv[it].load((const T*)P.v, rows[it], Q.ld, c8);
        }
    }
    // the gate logits of thread (ch, i)'s 16 positions, in flight as well
    const bool gate_thread = tid < D * NS;
    const int gch = tid % D, gi = tid / D;
    float br[16];
    if (gate_thread) {
#pragma unroll
        for (int u = 0; u < 16; ++u) br[u] = ld1<float>(P.z, sRows[16 * gi + u], Q.ld, gch);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int i = tid + it * NTS;
        if (i < C * G8) {
            const int t = i / G8, c8 = 8 * (i % G8);
            const bool ok = rows[it] >= 0;
            // 8 consecutive columns stay consecutive under the swizzle
            const int o = Y::sidx(t, c8);
            if (REV) {
                rq[it].put(sQ + o, ok);
                rd[it].put(sDO + o, ok);
            }
            if (FWD) {
                rk[it].put(sK + o, ok);
                rv[it].put(sV + o, ok);
            }
        }
    }

    // gate: thread (ch, i) over the 16 positions of sub-chunk i, decays in registers
    if (gate_thread) {
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            run += sRows[16 * gi + u] >= 0 ? log2_decay(br[u], P.inv_tau) : 0.f;
            br[u] = run;
        }
        sCB[gi * D + gch] = run;
    }
    __syncthreads();
    const size_t slot_floats = (size_t)D * D + D;
    float* dst_f = do_f ? Q.ws_f + ((size_t)unit * (P.nchunks - 1) + c) * slot_floats : nullptr;
    float* dst_r = do_r ? Q.ws_r + ((size_t)unit * (P.nchunks - 1) + (c - 1)) * slot_floats : nullptr;
    if (gate_thread) {
        float off = 0.f, tot = 0.f;
        for (int m = 0; m < NS; ++m) {
            const float x = sCB[m * D + gch];
            off += m < gi ? x : 0.f;
            tot += x;
        }
        float xq[16], xk[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int o = Y::sidx(16 * gi + u, gch);
            xq[u] = sQ[o];
            xk[u] = sK[o];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int o = Y::sidx(16 * gi + u, gch);
            const float b = br[u] + off;
            sQ[o] = xq[u] * exp2_fast(b);        // <= 1
            sK[o] = xk[u] * exp2_fast(tot - b);  // <= 1
        }
        if (gi == 0) {
            if (do_f) dst_f[D * D + gch] = tot;
            if (do_r) dst_r[D * D + gch] = tot;
        }
    }
    __syncthreads();
    // strip (product, a): rows 16a .. 16a + 15 of RA (product 0) or L (1) over
    // all value-channel tiles, the key-channel operand read once per k-step
    constexpr int STRIPS = 2 * NTL;
    constexpr int BT = NTL;  // value-channel tiles of a strip
    for (int strip = wave; strip < STRIPS; strip += NTS / 64) {
        const bool rev = strip < NTL;
        if (rev ? !do_r : !do_f) continue;
        const int a = rev ? strip : strip - NTL;
        const float* X = rev ? sQ : sK;
        const float* Yt = rev ? sDO : sV;
        float4v acc[BT];
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) acc[bb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int ks = 0; ks < C / 4; ++ks) {
            const int u = 4 * ks + g;
            const float x = X[Y::sidx(u, 16 * a + l16)];
#pragma unroll
            for (int bb = 0; bb < BT; ++bb) acc[bb] = mma(x, Yt[Y::sidx(u, 16 * bb + l16)], acc[bb]);
        }
        float* dst = rev ? dst_r : dst_f;
        const float f = rev ? P.scale : 1.f;
#pragma unroll
        for (int bb = 0; bb < BT; ++bb)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(size_t)(16 * a + 4 * g + e) * D + 16 * bb + l16] = f * acc[bb][e];
    }
}

// Folds, one thread per state entry (ch, j) of one scan:
//   forward: slot s <- S_in(s + 1) = 2^{B_s} S_in(s) + L_s, S_in(0) = 0;
//   reverse: slot s <- R_s = RA_{s+1} + 2^{B_{s+1}} R_{s+1}, R_{last} = 0;
//   carry:   ws_s[s][ch] = sum_j R_s[ch][j] S_in(s + 1)[ch][j]  (a row of D
//            entries is D consecutive lanes of one wavefront).
// Loads of a batch of slots are issued before the dependent multiply-adds.
template <int D, bool FWD, bool REV>
__global__ __launch_bounds__(NTS) void gla_bwd_fold_kernel(Params P, BwdParams Q)
{
    constexpr int ENTRIES = D * D;
    static_assert(ENTRIES % NTS == 0 && 64 % D == 0, "rows must tile the wavefronts");
    constexpr int BLKS = ENTRIES / NTS;
    constexpr int BATCH = 8;
    const int unit = blockIdx.x / BLKS;
    const int idx = (blockIdx.x - unit * BLKS) * NTS + threadIdx.x;
    const int ch = idx / D, j = idx - ch * D;
    const size_t slot_floats = (size_t)D * D + D;
    const int nslot = P.nchunks - 1;
    float* bf = Q.ws_f + (size_t)unit * nslot * slot_floats;
    float* br = Q.ws_r + (size_t)unit * nslot * slot_floats;
    float x = 0.f;
    for (int s0 = 0; FWD && s0 < nslot; s0 += BATCH) {
        float lv[BATCH], gv[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int s = s0 + u;
            lv[u] = (s < nslot) ? bf[(size_t)s * slot_floats + idx] : 0.f;
            gv[u] = (s < nslot) ? bf[(size_t)s * slot_floats + ENTRIES + ch] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int s = s0 + u;
            if (s < nslot) {
                x = exp2_fast(gv[u]) * x + lv[u];
                bf[(size_t)s * slot_floats + idx] = x;
            }
        }
    }
    float y = 0.f;
    for (int s0 = nslot - 1; REV && s0 >= 0; s0 -= BATCH) {
        float lv[BATCH], gv[BATCH], sv[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int s = s0 - u;
            lv[u] = (s >= 0) ? br[(size_t)s * slot_floats + idx] : 0.f;
            gv[u] = (s >= 0) ? br[(size_t)s * slot_floats + ENTRIES + ch] : 0.f;
            sv[u] = (s >= 0) ? bf[(size_t)s * slot_floats + idx] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int s = s0 - u;
            // slot s holds RA_{s+1} and B_{s+1}; y enters as R_{s+1}
            if (s >= 0) {
                y = exp2_fast(gv[u]) * y + lv[u];
                br[(size_t)s * slot_floats + idx] = y;
                float p = y * sv[u];
#pragma unroll
                for (int o = D / 2; o >= 1; o >>= 1) p += __shfl_xor(p, o);
                if (j == 0) Q.ws_s[((size_t)unit * P.nchunks + s) * D + ch] = p;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Diagonal blocks pair by pair (sub-chunks whose decay span exceeds 2^60).
// Raw q and k come from global memory; b from LDS.  Every factor is
// 2^{min(b_u - b_t, 0)}: pairs outside the causal triangle meet a zero score.
// ---------------------------------------------------------------------------

// E_{x, y} = 2^{c_{x-1} - c_y} for x = y .. NS (c_m the decay from the chunk
// start to the end of sub-chunk m): 2^{-tot_y} for x = y, then the running
// sums of the totals of the sub-chunks strictly between y and x, so each
// exponent is a short sum and never a difference of two large cumulative
// decays.
template <int D>
__device__ __forceinline__ void write_e_factors(float* sE, const float* sTot, int y, int ch)
{
    sE[(y * NS + y) * D + ch] = exp2_fast(-sTot[y * D + ch]);
    float acc = 0.f;
#pragma unroll
    for (int x = 1; x <= NS; ++x) {
        if (x > y) {
            sE[(x * NS + y) * D + ch] = exp2_fast(acc);
            if (x < NS) acc += sTot[x * D + ch];
        }
    }
}

// dq_t += sum_{tau <= t, same sub-chunk} P[t][tau] k_tau 2^{b_t - b_tau}
// for t = 16 si + 4 g + e, channel ch.
template <typename T, int D>
__device__ __forceinline__ void diag_dq(const Params& P, int ld, const int* sRows, const float* sP,
                                        const float* sB, int si, int g, int ch, float (&out)[4])
{
    constexpr int SD = Lay<D>::SD, SC = Lay<D>::SC;
    float kr[16], bk[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        kr[x] = ld1<T>(P.k, sRows[16 * si + x], ld, ch);
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
__device__ __forceinline__ void diag_dk(const Params& P, int ld, const int* sRows, const float* sP,
                                        const float* sB, int si, int g, int ch, float (&out)[4])
{
    constexpr int SD = Lay<D>::SD, SC = Lay<D>::SC;
    float qr[16], bq[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
        qr[x] = ld1<T>(P.q, sRows[16 * si + x], ld, ch);
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
__device__ __forceinline__ float4v diag_scores(const Params& P, int ld, const int* sRows, const float* sB,
                                               int si, int g, int l16)
{
    constexpr int SD = Lay<D>::SD;
    const int t = 16 * si + l16;
    const int rt = sRows[t];
    float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int c8 = 0; c8 < D; c8 += 8) {
        float kk[8];
        load8<T>((const T*)P.k, rt, ld, c8, kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 16 * si + 4 * g + e;
            float qq[8];
            load8<T>((const T*)P.q, sRows[u], ld, c8, qq);
#pragma unroll
            for (int x = 0; x < 8; ++x)
                a[e] += qq[x] * kk[x] * exp2_fast(fminf(sB[u * SD + c8 + x] - sB[t * SD + c8 + x], 0.f));
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (4 * g + e >= l16) ? P.scale * a[e] : 0.f;
    return a;
}

// scores[t][tau] = s sum_ch q_t k_tau 2^{b_t - b_tau} for t = 16 si + l16 >=
// tau = 16 si + 4 g + e (the layout of the output product's A operand).
template <typename T, int D>
__device__ __forceinline__ float4v diag_scores_out(const Params& P, int ld, const int* sRows, const float* sB,
                                                   int si, int g, int l16)
{
    constexpr int SD = Lay<D>::SD;
    const int t = 16 * si + l16;
    const int rt = sRows[t];
    float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int c8 = 0; c8 < D; c8 += 8) {
        float qq[8];
        load8<T>((const T*)P.q, rt, ld, c8, qq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 16 * si + 4 * g + e;
            float kk[8];
            load8<T>((const T*)P.k, sRows[u], ld, c8, kk);
#pragma unroll
            for (int x = 0; x < 8; ++x)
                a[e] += qq[x] * kk[x] * exp2_fast(fminf(sB[t * SD + c8 + x] - sB[u * SD + c8 + x], 0.f));
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (4 * g + e <= l16) ? P.scale * a[e] : 0.f;
    return a;
}

// ---------------------------------------------------------------------------
// Chunk kernel: dq, dk, dv and dz.  Wavefront w takes sub-chunk si = w / 2
// and half h = w % 2 of the 16-channel column tiles (the two halves of a
// sub-chunk sit on different SIMDs next to the halves of another sub-chunk).
// ---------------------------------------------------------------------------
template <typename T, typename TD, int D>
__global__ __launch_bounds__(NT) void gla_bwd_chunk_kernel(Params P, BwdParams Q)
{
    using Y = Lay<D>;
    constexpr int SD = Y::SD, SC = Y::SC, NTL = D / 16, KS = D / 4;
    constexpr int CT = NTL >= 2 ? NTL / 2 : 1;  // column tiles per wavefront
    __shared__ __attribute__((aligned(16))) float lds[Y::WORDS];
    float* sP = lds + Y::P;
    float* sDO = lds + Y::DO;
    float* sV = lds + Y::V;
    float* sKT = lds + Y::KT;
    float* sQH = lds + Y::QH;
    float* sSS = lds + Y::SS;
    float* sRR = lds + Y::RR;
    float* sB = lds + Y::BB;
    float* sCC = lds + Y::CC;
    float* sE = lds + Y::EE;
    float* sTot = lds + Y::TOT;
    int* sRows = (int*)(lds + Y::ROWS);
    int* sFlag = (int*)(lds + Y::FLAGS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int units = P.B * P.NH;
    const int unit = blockIdx.x % units;
    const int c = blockIdx.x / units;
    const int si = wave >> 1, h = wave & 1;
    const int ct0 = h * CT;
    const bool cols = ct0 < NTL;                // D = 16: the second half has no columns
    const float s = P.scale;
    const size_t slot_floats = (size_t)D * D + D;
    const bool has_in = c > 0;                  // a state enters from earlier chunks
    const bool has_r = c < P.nchunks - 1;       // a gradient enters from later chunks
    if (tid < NS) sFlag[tid] = 0;
    // E_xy of channel ch: sE[(x * NS + y) * D + ch]
    auto E = [&](int x, int y, int ch) { return sE[(x * NS + y) * D + ch]; };

    // ---- one load phase: the states entering from both sides, raw q -> QH,
    //      k -> KT, v, dO, the gate logits of the gate threads (their 16
    //      positions of one channel) and the later chunks' part of dz; rows
    //      come from the scan order directly, and every load is issued before
    //      the first one is used
    const bool gate_thread = tid < D * NS;
    const int gch = tid % D, gi = tid / D;
    float zz[16];
    unsigned zok = 0;
    float later_c = 0.f;
    {
        constexpr int SQ4 = D * D / 4;
        constexpr int SIT = (SQ4 + NT - 1) / NT;
        float4v st_in[SIT], st_r[SIT];
        const float4v* src_in = (const float4v*)(Q.ws_f + ((size_t)unit * (P.nchunks - 1) + (has_in ? c - 1 : 0)) * slot_floats);
        const float4v* src_r = (const float4v*)(Q.ws_r + ((size_t)unit * (P.nchunks - 1) + (has_r ? c : 0)) * slot_floats);
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            const int i = tid + it * NT;
            const int ii = i < SQ4 ? i : 0;
            if (has_in) st_in[it] = src_in[ii];
            if (has_r) st_r[it] = src_r[ii];
        }
        constexpr int G8 = D / 8;
        constexpr int IT = (C * G8 + NT - 1) / NT;
        Raw8<T> rq[IT], rk[IT], rv[IT];
        Raw8<TD> rd[IT];
        int rows[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + it * NT;
            const int t = (i < C * G8 ? i : 0) / G8, c8 = 8 * (i % G8);
            rows[it] = scan_row(P, unit, c * C + t);
            rq[it].load((const T*)P.q, rows[it], Q.ld, c8);
            rk[it].load((const T*)P.k, rows[it], Q.ld, c8);
            rv[it].load((const T*)P.v, rows[it], Q.ld, c8);
            rd[it].load((const TD*)Q.dout, rows[it], Q.ld, c8);
        }
        if (gate_thread) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int row = scan_row(P, unit, c * C + 16 * gi + u);
                zok |= (row >= 0 ? 1u : 0u) << u;
                zz[u] = ld1<float>(P.z, row, Q.ld, gch);
            }
            later_c = has_r ? Q.ws_s[((size_t)unit * P.nchunks + c) * D + gch] : 0.f;
        }
        for (int i = tid; i < C; i += NT) sRows[i] = scan_row(P, unit, c * C + i);
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            const int i = tid + it * NT;
            if (i < SQ4) {
                const int r = (4 * i) / D, cc = 4 * i - r * D;
                if (has_in) *(float4v*)(sSS + r * SD + cc) = st_in[it];
                if (has_r) *(float4v*)(sRR + r * SD + cc) = st_r[it];
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + it * NT;
            if (i < C * G8) {
                const int o = (i / G8) * SD + 8 * (i % G8);
                const bool ok = rows[it] >= 0;
                rq[it].put(sQH + o, ok);
                rk[it].put(sKT + o, ok);
                rv[it].put(sV + o, ok);
                rd[it].put(sDO + o, ok);
            }
        }
    }
    __syncthreads();

    // ---- gate: thread (ch, i) runs over the 16 positions of sub-chunk i
    float br[16];
    if (gate_thread) {
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            run += ((zok >> u) & 1u) ? log2_decay(zz[u], P.inv_tau) : 0.f;
            br[u] = run;  // within the sub-chunk
        }
        sTot[gi * D + gch] = run;
        if (run < -kDiagSpan) sFlag[gi] = 1;
    }
    __syncthreads();
    if (gate_thread) {
        // c_{-1} .. c_3 of this channel
        float cv[NS + 1];
        cv[0] = 0.f;
#pragma unroll
        for (int m = 0; m < NS; ++m) cv[m + 1] = cv[m] + sTot[m * D + gch];
        const float ci = cv[gi + 1], tot = br[15];
        sCC[(gi + 1) * D + gch] = ci;
        if (gi == 0) sCC[gch] = 0.f;
        // E_{x, gi} = 2^{c_{x-1} - c_gi} for x = gi .. NS, from the short sums
        // of the sub-chunk totals between them (no differences of the large
        // cumulative decays, whose rounding would dominate when decays are
        // strong)
        write_e_factors<D>(sE, sTot, gi, gch);
        float xq[16], xk[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            xq[u] = sQH[(16 * gi + u) * SD + gch];
            xk[u] = sKT[(16 * gi + u) * SD + gch];
        }
        // b is kept relative to the sub-chunk start: pairwise factors and the
        // per-position scalings take differences of these short sums only
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * gi + u;
            sQH[t * SD + gch] = xq[u] * exp2_fast(br[u]);        // <= 1
            sKT[t * SD + gch] = xk[u] * exp2_fast(tot - br[u]);  // <= 1
            sB[t * SD + gch] = br[u];
        }
    }
    __syncthreads();
    const bool pairwise = sFlag[si] != 0;  // wave-uniform

    // ---- P = s dO V^T on the blocks j <= si (this half: j = h mod 2),
    //      diagonal blocks masked to u >= t
    for (int j = h; j <= si; j += 2) {
        // operands of PB steps read before their products, two chains
        constexpr int PB = KS < 8 ? KS : 8;
        float4v acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += PB) {
            float av[PB], bv[PB];
#pragma unroll
            for (int u = 0; u < PB; ++u) {
                const int col = 4 * (k0 + u) + g;
                av[u] = sDO[(16 * si + l16) * SD + col];
                bv[u] = sV[(16 * j + l16) * SD + col];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < PB; ++u) {
                if (u & 1) acc1 = mma(av[u], bv[u], acc1);
                else acc = mma(av[u], bv[u], acc);
            }
        }
        acc = acc + acc1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 4 * g + e;
            sP[(16 * si + u) * SC + 16 * j + l16] = (j == si && l16 > u) ? 0.f : s * acc[e];
        }
    }
    __syncthreads();

    float dqv[CT][4], dkv[CT][4];
    if (cols) {
        // ---- dq of sub-chunk si (rows 16 si + 4g + e, columns 16 ct + l16);
        //      the column tiles innermost: one A read serves CT products
        {
            float4v acc[CT];
#pragma unroll
            for (int cl = 0; cl < CT; ++cl) acc[cl] = float4v{0.f, 0.f, 0.f, 0.f};
            const int jend = pairwise ? si - 1 : si;
            for (int j = 0; j <= jend; ++j) {
                float4v m[CT];
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) m[cl] = float4v{0.f, 0.f, 0.f, 0.f};
                float av[4], bv[4][CT];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int sp = 16 * j + 4 * ks + g;
                    av[ks] = sP[(16 * si + l16) * SC + sp];
#pragma unroll
                    for (int cl = 0; cl < CT; ++cl) bv[ks][cl] = sKT[sp * SD + 16 * (ct0 + cl) + l16];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int cl = 0; cl < CT; ++cl) m[cl] = mma(av[ks], bv[ks][cl], m[cl]);
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) {
                    const float f = E(si, j, 16 * (ct0 + cl) + l16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[cl][e] += m[cl][e] * f;
                }
            }
            if (has_in) {
                float4v m[CT];
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) m[cl] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int ks = 0; ks < KS; ++ks) {
                    const int jj = 4 * ks + g;
                    const float a = sDO[(16 * si + l16) * SD + jj];
#pragma unroll
                    for (int cl = 0; cl < CT; ++cl)
                        m[cl] = mma(a, sSS[(16 * (ct0 + cl) + l16) * SD + jj], m[cl]);
                }
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) {
                    const float f = s * exp2_fast(sCC[si * D + 16 * (ct0 + cl) + l16]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[cl][e] += m[cl][e] * f;
                }
            }
#pragma unroll
            for (int cl = 0; cl < CT; ++cl) {
                const int ch = 16 * (ct0 + cl) + l16;
                float dg[4] = {0.f, 0.f, 0.f, 0.f};
                if (pairwise) diag_dq<T, D>(P, Q.ld, sRows, sP, sB, si, g, ch, dg);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * si + 4 * g + e;
                    dqv[cl][e] = acc[cl][e] * exp2_fast(sB[t * SD + ch]) + dg[e];
                    const int row = sRows[t];
                    if (row >= 0) put_grad<T>((T*)Q.dq, (size_t)row * Q.ld + ch, Q.pq, (size_t)row * Q.ldp + ch, Q.mode_qk, dqv[cl][e]);
                }
            }
        }

        // ---- dk of sub-chunk si
        {
            float4v acc[CT];
#pragma unroll
            for (int cl = 0; cl < CT; ++cl) acc[cl] = float4v{0.f, 0.f, 0.f, 0.f};
            for (int j = pairwise ? si + 1 : si; j < NS; ++j) {
                float4v m[CT];
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) m[cl] = float4v{0.f, 0.f, 0.f, 0.f};
                float av[4], bv[4][CT];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int up = 16 * j + 4 * ks + g;
                    av[ks] = sP[up * SC + 16 * si + l16];
#pragma unroll
                    for (int cl = 0; cl < CT; ++cl) bv[ks][cl] = sQH[up * SD + 16 * (ct0 + cl) + l16];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int cl = 0; cl < CT; ++cl) m[cl] = mma(av[ks], bv[ks][cl], m[cl]);
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) {
                    const float f = E(j, si, 16 * (ct0 + cl) + l16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[cl][e] += m[cl][e] * f;
                }
            }
            if (has_r) {
                float4v m[CT];
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) m[cl] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int ks = 0; ks < KS; ++ks) {
                    const int jj = 4 * ks + g;
                    const float a = sV[(16 * si + l16) * SD + jj];
#pragma unroll
                    for (int cl = 0; cl < CT; ++cl)
                        m[cl] = mma(a, sRR[(16 * (ct0 + cl) + l16) * SD + jj], m[cl]);
                }
#pragma unroll
                for (int cl = 0; cl < CT; ++cl) {
                    const float f = E(NS, si, 16 * (ct0 + cl) + l16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[cl][e] += m[cl][e] * f;
                }
            }
#pragma unroll
            for (int cl = 0; cl < CT; ++cl) {
                const int ch = 16 * (ct0 + cl) + l16;
                float dg[4] = {0.f, 0.f, 0.f, 0.f};
                if (pairwise) diag_dk<T, D>(P, Q.ld, sRows, sP, sB, si, g, ch, dg);
                const float tot = sTot[si * D + ch];  // this sub-chunk's decay
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * si + 4 * g + e;
                    dkv[cl][e] = acc[cl][e] * exp2_fast(tot - sB[t * SD + ch]) + dg[e];
                    const int row = sRows[t];
                    if (row >= 0) put_grad<T>((T*)Q.dk, (size_t)row * Q.ld + ch, Q.pk, (size_t)row * Q.ldp + ch, Q.mode_qk, dkv[cl][e]);
                }
            }
        }

        // ---- dv of sub-chunk si: sum_{j >= si} A_ji^T dO_j + (Kh (.) E_4i)_si R
        float4v dvacc[CT];
#pragma unroll
        for (int cl = 0; cl < CT; ++cl) dvacc[cl] = float4v{0.f, 0.f, 0.f, 0.f};
        // this lane's Kh values: row 16 si + l16, channels 4 ks + g
        float kh[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kh[ks] = sKT[(16 * si + l16) * SD + 4 * ks + g];
        for (int j = si; j < NS; ++j) {
            // A_ji[u = 16 j + 4g + e][t = 16 si + l16] (both halves form it),
            // even and odd k-steps on two independent chains
            float4v a = {0.f, 0.f, 0.f, 0.f};
            if (j == si && pairwise) {
                a = diag_scores<T, D>(P, Q.ld, sRows, sB, si, g, l16);
            } else {
                // the block's B operands first (all factor loads in flight
                // together), then the two MFMA chains
                float kb[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kb[ks] = kh[ks] * E(j, si, 4 * ks + g);
                float qv[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) qv[ks] = sQH[(16 * j + l16) * SD + 4 * ks + g];
                __builtin_amdgcn_sched_barrier(0);
                float4v a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ks += 2) {
                    a = mma(qv[ks], kb[ks], a);
                    a1 = mma(qv[ks + 1], kb[ks + 1], a1);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = (j > si) || (4 * g + e >= l16);
                    a[e] = keep ? s * (a[e] + a1[e]) : 0.f;
                }
            }
            // dv[t][col] += sum_u A[u][t] dO[u][col], k-slot g of step e is u = 16 j + 4g + e
            float dov[CT][4];
#pragma unroll
            for (int cl = 0; cl < CT; ++cl)
#pragma unroll
                for (int e = 0; e < 4; ++e) dov[cl][e] = sDO[(16 * j + 4 * g + e) * SD + 16 * (ct0 + cl) + l16];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cl = 0; cl < CT; ++cl)
#pragma unroll
                for (int e = 0; e < 4; ++e) dvacc[cl] = mma(a[e], dov[cl][e], dvacc[cl]);
        }
        if (has_r) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = 4 * ks + g;
                const float kf = kh[ks] * E(NS, si, ch);
#pragma unroll
                for (int cl = 0; cl < CT; ++cl)
                    dvacc[cl] = mma(kf, sRR[ch * SD + 16 * (ct0 + cl) + l16], dvacc[cl]);
            }
        }
#pragma unroll
        for (int cl = 0; cl < CT; ++cl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = sRows[16 * si + 4 * g + e];
                const size_t idx = (size_t)row * Q.ld + 16 * (ct0 + cl) + l16;
                if (row >= 0) put_grad<T>((T*)Q.dv, idx, Q.pv, idx, Q.mode_v, dvacc[cl][e]);
            }
    }
    __syncthreads();  // every reader of P is done: reuse it

    // ---- q (.) dq - k (.) dk into P ([C][SD] view), raw q and k reloaded
    float* sZ = sP;
    if (cols) {
        float qv[CT][4], kv[CT][4];
#pragma unroll
        for (int cl = 0; cl < CT; ++cl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = sRows[16 * si + 4 * g + e], ch = 16 * (ct0 + cl) + l16;
                qv[cl][e] = ld1<T>(P.q, row, Q.ld, ch);
                kv[cl][e] = ld1<T>(P.k, row, Q.ld, ch);
            }
#pragma unroll
        for (int cl = 0; cl < CT; ++cl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * si + 4 * g + e, ch = 16 * (ct0 + cl) + l16;
                sZ[t * SD + ch] = qv[cl][e] * dqv[cl][e] - kv[cl][e] * dkv[cl][e];
            }
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
        sTot[gi * D + gch] = run;  // sub-chunk total
    }
    __syncthreads();
    if (gate_thread) {
        // later chunks: sum_j R_c S_in(c + 1) from the fold
        float later = later_c;
        for (int m = gi + 1; m < NS; ++m) later += sTot[m * D + gch];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int row = sRows[16 * gi + u];
            // 1 - sigmoid(z) as sigmoid(-z)
            const float nsig = rcp_fast(1.0f + exp2_fast(zz[u] * kLog2e));
            const size_t idx = (size_t)row * Q.ld + gch;
            if (row >= 0) put_grad<float>(Q.dz, idx, Q.dz, idx, Q.mode_qk, (br[u] + later) * nsig * P.inv_tau);
        }
    }
}

// ---------------------------------------------------------------------------
// Gated backward, first half: the ungated output o of a chunk recomputed in
// binary32 from the entering state (paper Sec. 2.1 recurrence, the forward's
// chunkwise form with the same sub-chunk factors), then the output gate's
// backward on it (u = SiLU(r) (.) w (.) o rho, rho = (mean(o^2) + eps)^-1/2):
//     do = rho g - (rho^3 / d) o sum(g (.) o),  g = du (.) SiLU(r) (.) w
//     dr = du (.) w (.) o rho (.) SiLU'(r),     dw partial = sum_rows du SiLU(r) o rho
// do (binary32) feeds the reverse aggregates and the chunk kernel.  Same
// geometry as the chunk kernel: wavefront (si, h) owns sub-chunk si and half
// h of the column tiles; o of a block is sum_{j <= si} scores_ij V_j +
// s Qh_si (2^{c_{si-1}} (.) S_in) with scores_ij = s Qh_i (Kh_j (.) E_ij)^T.
// ---------------------------------------------------------------------------
// OONLY: o alone (a quarter of a d = 128 call), added to G.o_out.
template <typename T, int D, bool OONLY>
__global__ __launch_bounds__(NT) void gla_bwd_oepi_kernel(Params P, BwdParams Q, GatedBwd G)
{
    using Y = Lay<D>;
    constexpr int SD = Y::SD, NTL = D / 16, KS = D / 4;
    constexpr int CT = NTL >= 2 ? NTL / 2 : 1;
    __shared__ __attribute__((aligned(16))) float lds[Y::WORDS];
    float* sQB = lds + Y::P;     // q (.) 2^b (b from the chunk start): the reverse aggregate's operand
    float* sDO = lds + Y::DO;    // dO of the chunk (binary32)
    float* sV = lds + Y::V;
    float* sKT = lds + Y::KT;
    float* sQH = lds + Y::QH;
    float* sSS = lds + Y::SS;
    float* sRed = lds + Y::RR;   // dw partial sums [NS][D]
    float* sX = sRed + NS * D;   // row sums of the two halves [2 sums][2 halves][C]
    float* sB = lds + Y::BB;
    float* sCC = lds + Y::CC;
    float* sE = lds + Y::EE;
    float* sTot = lds + Y::TOT;
    int* sRows = (int*)(lds + Y::ROWS);
    int* sFlag = (int*)(lds + Y::FLAGS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int units = P.B * P.NH;
    const int unit = blockIdx.x % units;
    const int c = blockIdx.x / units;
    const int si = wave >> 1, h = wave & 1;
    const int ct0 = h * CT;
    const bool cols = ct0 < NTL;
    const float s = P.scale;
    const size_t slot_floats = (size_t)D * D + D;
    const bool has_in = c > 0;
    if (tid < NS) sFlag[tid] = 0;
    auto E = [&](int x, int y, int ch) { return sE[(x * NS + y) * D + ch]; };

    // ---- loads: S_in, raw q -> QH, k -> KT, v, the gate threads' logits
    const bool gate_thread = tid < D * NS;
    const int gch = tid % D, gi = tid / D;
    float zz[16];
    unsigned zok = 0;
    {
        constexpr int SQ4 = D * D / 4;
        constexpr int SIT = (SQ4 + NT - 1) / NT;
        float4v st_in[SIT];
        const float4v* src_in = (const float4v*)(Q.ws_f + ((size_t)unit * (P.nchunks - 1) + (has_in ? c - 1 : 0)) * slot_floats);
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            const int i = tid + it * NT;
            if (has_in) st_in[it] = src_in[i < SQ4 ? i : 0];
        }
        constexpr int G8 = D / 8;
        constexpr int IT = (C * G8 + NT - 1) / NT;
        Raw8<T> rq[IT], rk[IT], rv[IT];
        int rows[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + it * NT;
            const int t = (i < C * G8 ? i : 0) / G8, c8 = 8 * (i % G8);
            rows[it] = scan_row(P, unit, c * C + t);
            rq[it].load((const T*)P.q, rows[it], Q.ld, c8);
            rk[it].load((const T*)P.k, rows[it], Q.ld, c8);
            rv[it].load((const T*)P.v, rows[it], Q.ld, c8);
        }
        if (gate_thread) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int row = scan_row(P, unit, c * C + 16 * gi + u);
                zok |= (row >= 0 ? 1u : 0u) << u;
                zz[u] = ld1<float>(P.z, row, Q.ld, gch);
            }
        }
        for (int i = tid; i < C; i += NT) sRows[i] = scan_row(P, unit, c * C + i);
#pragma unroll
        for (int it = 0; it < SIT; ++it) {
            const int i = tid + it * NT;
            if (i < SQ4 && has_in) {
                const int r = (4 * i) / D, cc = 4 * i - r * D;
                *(float4v*)(sSS + r * SD + cc) = st_in[it];
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int i = tid + it * NT;
            if (i < C * G8) {
                const int o = (i / G8) * SD + 8 * (i % G8);
                const bool ok = rows[it] >= 0;
                rq[it].put(sQH + o, ok);
                rk[it].put(sKT + o, ok);
                rv[it].put(sV + o, ok);
            }
        }
    }
    __syncthreads();

    // ---- gate stage (as in the chunk kernel)
    float br[16];
    if (gate_thread) {
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            run += ((zok >> u) & 1u) ? log2_decay(zz[u], P.inv_tau) : 0.f;
            br[u] = run;
        }
        sTot[gi * D + gch] = run;
        if (run < -kDiagSpan) sFlag[gi] = 1;
    }
    __syncthreads();
    if (gate_thread) {
        float cv[NS + 1];
        cv[0] = 0.f;
#pragma unroll
        for (int m = 0; m < NS; ++m) cv[m + 1] = cv[m] + sTot[m * D + gch];
        const float off = cv[gi], ci = cv[gi + 1], tot = br[15];
        sCC[(gi + 1) * D + gch] = ci;
        if (gi == 0) sCC[gch] = 0.f;
        write_e_factors<D>(sE, sTot, gi, gch);
        float xq[16], xk[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            xq[u] = sQH[(16 * gi + u) * SD + gch];
            xk[u] = sKT[(16 * gi + u) * SD + gch];
        }
        // b relative to the sub-chunk start, as in the chunk kernel
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * gi + u;
            sQH[t * SD + gch] = xq[u] * exp2_fast(br[u]);
            sKT[t * SD + gch] = xk[u] * exp2_fast(tot - br[u]);
            sQB[t * SD + gch] = xq[u] * exp2_fast(br[u] + off);  // <= 1, from the chunk start
            sB[t * SD + gch] = br[u];
        }
    }
    __syncthreads();
    const bool pairwise = sFlag[si] != 0;

    // ---- o of sub-chunk si: rows 16 si + 4g + e, columns 16 (ct0 + cl) + l16
    float4v oacc[CT];
#pragma unroll
    for (int cl = 0; cl < CT; ++cl) oacc[cl] = float4v{0.f, 0.f, 0.f, 0.f};
    if (cols) {
        for (int j = 0; j <= si; ++j) {
            // scores[t = 16 si + l16][tau = 16 j + 4g + e], two chains
            float4v a = {0.f, 0.f, 0.f, 0.f};
            if (j == si && pairwise) {
                a = diag_scores_out<T, D>(P, Q.ld, sRows, sB, si, g, l16);
            } else {
                // the block's A operands first (all loads in flight together),
                // then the two MFMA chains
                float ka[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    ka[ks] = sKT[(16 * j + l16) * SD + 4 * ks + g] * E(si, j, 4 * ks + g);
                float qv[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) qv[ks] = sQH[(16 * si + l16) * SD + 4 * ks + g];
                __builtin_amdgcn_sched_barrier(0);
                float4v a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ks += 2) {
                    a = mma(ka[ks], qv[ks], a);
                    a1 = mma(ka[ks + 1], qv[ks + 1], a1);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = (j < si) || (4 * g + e <= l16);
                    a[e] = keep ? s * (a[e] + a1[e]) : 0.f;
                }
            }
            // o[t][col] += sum_tau scores[t][tau] v[tau][col]; k-slot g of step e is tau = 16 j + 4g + e
            float vv[CT][4];
#pragma unroll
            for (int cl = 0; cl < CT; ++cl)
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[cl][e] = sV[(16 * j + 4 * g + e) * SD + 16 * (ct0 + cl) + l16];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cl = 0; cl < CT; ++cl)
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[cl] = mma(a[e], vv[cl][e], oacc[cl]);
        }
        if (has_in) {
#pragma unroll 4
            for (int ks = 0; ks < KS; ++ks) {
                const int jj = 4 * ks + g;
                const float a = sQH[(16 * si + l16) * SD + jj];
                const float f = s * exp2_fast(sCC[si * D + jj]);
#pragma unroll
                for (int cl = 0; cl < CT; ++cl)
                    oacc[cl] = mma(a, sSS[jj * SD + 16 * (ct0 + cl) + l16] * f, oacc[cl]);
            }
        }
    }

    int rowe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rowe[e] = sRows[16 * si + 4 * g + e];
    if constexpr (OONLY) {
        if (cols) {
#pragma unroll
            for (int cl = 0; cl < CT; ++cl)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (rowe[e] < 0) continue;
                    const size_t idx = (size_t)rowe[e] * Q.ld + 16 * (ct0 + cl) + l16;
                    G.o_out[idx] = G.o_acc ? G.o_out[idx] + oacc[cl][e] : oacc[cl][e];
                }
        }
        return;
    }

    // ---- output gate backward at (t = 16 si + 4g + e, col = 16 (ct0 + cl) + l16)
    float rv[CT][4], uv[CT][4], wv[CT];
#pragma unroll
    for (int cl = 0; cl < CT; ++cl) {
        const int col = 16 * (ct0 + cl) + l16;
        const int colc = cols ? col : 0;
        wv[cl] = G.w ? G.w[colc] : 1.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rv[cl][e] = ld1<T>(G.r, cols ? rowe[e] : -1, Q.ld, colc);
            uv[cl][e] = ld1<T>(G.du, cols ? rowe[e] : -1, Q.ld, colc);
        }
    }
    float ss[4], dot[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ss[e] = 0.f;
        dot[e] = 0.f;
#pragma unroll
        for (int cl = 0; cl < CT; ++cl) {
            const float o = oacc[cl][e];
            ss[e] += o * o;
            dot[e] += uv[cl][e] * silu(rv[cl][e]) * wv[cl] * o;
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
            ss[e] += __shfl_xor(ss[e], m);
            dot[e] += __shfl_xor(dot[e], m);
        }
    }
    if (l16 == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * si + 4 * g + e;
            sX[(0 * 2 + h) * C + t] = ss[e];
            sX[(1 * 2 + h) * C + t] = dot[e];
        }
    }
    __syncthreads();
    float dwl[CT];
#pragma unroll
    for (int cl = 0; cl < CT; ++cl) dwl[cl] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 16 * si + 4 * g + e;
        const float sst = sX[(0 * 2 + 0) * C + t] + sX[(0 * 2 + 1) * C + t];
        const float dt = sX[(1 * 2 + 0) * C + t] + sX[(1 * 2 + 1) * C + t];
        const float rho = rsq_fast(sst * (1.0f / D) + G.eps);
        const float k3 = rho * rho * rho * (1.0f / D) * dt;
#pragma unroll
        for (int cl = 0; cl < CT; ++cl) {
            const float o = oacc[cl][e], r = rv[cl][e], du = uv[cl][e];
            const float sig = rcp_fast(1.0f + exp2_fast(-r * kLog2e));
            const float sr = r * sig;
            const float dov = rho * du * sr * wv[cl] - k3 * o;
            const float drv = du * wv[cl] * o * rho * sig * (1.0f + r * (1.0f - sig));
            dwl[cl] += du * sr * o * rho;
            const int row = rowe[e];
            if (cols) sDO[t * SD + 16 * (ct0 + cl) + l16] = dov;  // rows past the end: 0
            if (cols && row >= 0) {
                const size_t idx = (size_t)row * Q.ld + 16 * (ct0 + cl) + l16;
                ((float*)Q.dout)[idx] = dov;
                store1<T>((T*)G.dr, idx, drv);
            }
        }
    }
    // dw partial sums of this chunk: over the wavefront's rows (lanes g), then
    // over the sub-chunks in order
#pragma unroll
    for (int cl = 0; cl < CT; ++cl) {
        dwl[cl] += __shfl_xor(dwl[cl], 16);
        dwl[cl] += __shfl_xor(dwl[cl], 32);
        if (cols && g == 0) sRed[si * D + 16 * (ct0 + cl) + l16] = dwl[cl];
    }
    __syncthreads();
    for (int col = tid; col < D; col += NT) {
        float x = 0.f;
#pragma unroll
        for (int m = 0; m < NS; ++m) x += sRed[m * D + col];
        G.dwp[(size_t)blockIdx.x * D + col] = x;
    }
    // reverse aggregate of this chunk from the dO just formed (the states
    // kernel's other half): slot c - 1 of ws_r <- (s (q (.) 2^b)^T dO, B)
    if (c >= 1) {
        float* dst = Q.ws_r + ((size_t)unit * (P.nchunks - 1) + (c - 1)) * slot_floats;
        if (tid < D) dst[D * D + tid] = sCC[NS * D + tid];  // c_3 = the chunk's decay
        // wavefront w: key-channel tile a = w / 2, value tiles of half w % 2
        constexpr int VT = NTL >= 2 ? NTL / 2 : 1;
        const int a = wave >> 1, v0 = (wave & 1) * VT;
        if (a < NTL && v0 < NTL) {
            float4v acc[VT];
#pragma unroll
            for (int vb = 0; vb < VT; ++vb) acc[vb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int ks = 0; ks < C / 4; ++ks) {
                const int u = 4 * ks + g;
                const float x = sQB[u * SD + 16 * a + l16];
#pragma unroll
                for (int vb = 0; vb < VT; ++vb) acc[vb] = mma(x, sDO[u * SD + 16 * (v0 + vb) + l16], acc[vb]);
            }
#pragma unroll
            for (int vb = 0; vb < VT; ++vb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(size_t)(16 * a + 4 * g + e) * D + 16 * (v0 + vb) + l16] = s * acc[vb][e];
        }
    }
}

// Output gate backward row by row, for a d = 128 call whose o (binary32,
// complete) sits in `od` (row stride d): dO replaces o there, dr is stored,
// and block b leaves its rows' dw partial sums in dwp[b] (the formulas of the
// o kernel's epilogue; fixed summation order).  Block b takes rows
// [64 b, 64 b + 64), 16 per wavefront; lane l the columns l + 64 p.
constexpr int NER = 256;
template <typename T, int D>
__global__ __launch_bounds__(NER) void gla_bwd_epi_rows_kernel(float* __restrict__ od, GatedBwd G,
                                                              int rows)
{
    constexpr int PER = D / 64;
    __shared__ float sRed[NER / 64][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float wv[PER], dwl[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        wv[p] = G.w ? G.w[lane + 64 * p] : 1.0f;
        dwl[p] = 0.f;
    }
    const int row0 = blockIdx.x * 64 + wave * 16;
    for (int i = 0; i < 16 && row0 + i < rows; ++i) {
        const size_t base = (size_t)(row0 + i) * D;
        float o[PER], rr[PER], uu[PER];
        float ss = 0.f, dot = 0.f;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const size_t idx = base + lane + 64 * p;
            o[p] = od[idx];
            rr[p] = (float)((const T*)G.r)[idx];
            uu[p] = (float)((const T*)G.du)[idx];
        }
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            ss += o[p] * o[p];
            dot += uu[p] * silu(rr[p]) * wv[p] * o[p];
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            ss += __shfl_xor(ss, m);
            dot += __shfl_xor(dot, m);
        }
        const float rho = rsq_fast(ss * (1.0f / D) + G.eps);
        const float k3 = rho * rho * rho * (1.0f / D) * dot;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const size_t idx = base + lane + 64 * p;
            const float r = rr[p], du = uu[p];
            const float sig = rcp_fast(1.0f + exp2_fast(-r * kLog2e));
            const float sr = r * sig;
            od[idx] = rho * du * sr * wv[p] - k3 * o[p];
            store1<T>((T*)G.dr, idx, du * wv[p] * o[p] * rho * sig * (1.0f + r * (1.0f - sig)));
            dwl[p] += du * sr * o[p] * rho;
        }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) sRed[wave][lane + 64 * p] = dwl[p];
    __syncthreads();
    for (int col = threadIdx.x; col < D; col += NER) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NER / 64; ++w) x += sRed[w][col];
        G.dwp[(size_t)blockIdx.x * D + col] = x;
    }
}

// dw[c] = sum_b dwp[b][c] in a fixed order: part p of NDW / D parts adds the
// blocks b = p (mod parts) in increasing order, eight loads in flight, then
// the parts are added in order.
constexpr int NDW = 1024;
template <int D>
__global__ __launch_bounds__(NDW) void gla_bwd_dw_kernel(const float* __restrict__ dwp,
                                                         float* __restrict__ dw, int nblk)
{
    constexpr int PARTS = NDW / D;
    __shared__ float part[PARTS][D];
    const int c = threadIdx.x % D, p = threadIdx.x / D;
    float x = 0.f;
    for (int b0 = p; b0 < nblk; b0 += 8 * PARTS) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int b = b0 + u * PARTS;
            v[u] = b < nblk ? dwp[(size_t)b * D + c] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) x += v[u];
    }
    part[p][c] = x;
    __syncthreads();
    if (threadIdx.x < D) {
        float y = 0.f;
        for (int q = 0; q < PARTS; ++q) y += part[q][threadIdx.x];
        dw[threadIdx.x] = y;
    }
}

template <typename T, int D>
static int run_bwd_gated(const Params& P, const BwdParams& Q, const GatedBwd& G, hipStream_t st)
{
    const unsigned units = (unsigned)(P.B * P.NH);
    constexpr unsigned blks = D * D / NTS;
    if (P.nchunks > 1) {
        // entering states first (o needs them); the o kernel leaves the reverse
        // aggregates (dO exists there)
        hipLaunchKernelGGL((gla_bwd_states_kernel<T, float, D, true, false>), dim3(units * P.nchunks),
                           dim3(NTS), 0, st, P, Q);
        hipLaunchKernelGGL((gla_bwd_fold_kernel<D, true, false>), dim3(units * blks), dim3(NTS), 0, st, P, Q);
    }
    hipLaunchKernelGGL((gla_bwd_oepi_kernel<T, D, false>), dim3(units * P.nchunks), dim3(NT), 0, st, P, Q, G);
    if (G.dw)
        hipLaunchKernelGGL((gla_bwd_dw_kernel<D>), dim3(1), dim3(NDW), 0, st, G.dwp, G.dw,
                           (int)(units * P.nchunks));
    if (P.nchunks > 1)
        hipLaunchKernelGGL((gla_bwd_fold_kernel<D, false, true>), dim3(units * blks), dim3(NTS), 0, st, P, Q);
    hipLaunchKernelGGL((gla_bwd_chunk_kernel<T, float, D>), dim3(units * P.nchunks), dim3(NT), 0, st, P, Q);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

template <typename T, typename TD, int D>
static int run_bwd(const Params& P, const BwdParams& Q, hipStream_t st)
{
    const unsigned units = (unsigned)(P.B * P.NH);
    if (P.nchunks > 1) {
        hipLaunchKernelGGL((gla_bwd_states_kernel<T, TD, D, true, true>), dim3(units * P.nchunks),
                           dim3(NTS), 0, st, P, Q);
        constexpr unsigned blks = D * D / NTS;
        hipLaunchKernelGGL((gla_bwd_fold_kernel<D, true, true>), dim3(units * blks), dim3(NTS), 0, st, P, Q);
    }
    hipLaunchKernelGGL((gla_bwd_chunk_kernel<T, TD, D>), dim3(units * P.nchunks), dim3(NT), 0, st, P, Q);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

// d = 128 as four d = 64 quarters.  The decay acts on each key channel alone
// and o is linear in v, so with key half a and value half cv the quarter's
// state is the block S[a][cv] of the full state, and the quarter (a, cv) is
// the d = 64 problem on the columns [64 a, 64 a + 64) of q, k, z and
// [64 cv, 64 cv + 64) of v and dO, at the full problem's scale.  dq, dk and
// dz of key half a are the sums over cv of the quarters' gradients, dv of
// value half cv the sum over a.  In the order (0,0), (0,1), (1,0), (1,1)
// the first quarter of each output half keeps a binary32 partial sum (dz its
// own buffer) and the second adds it and stores.
template <typename T, typename TD>
static Params quarter(const Params& P0, BwdParams& Q, const BwdParams& Q0, int a, int cv)
{
    Params P = P0;
    P.q = (const T*)P0.q + 64 * a;
    P.k = (const T*)P0.k + 64 * a;
    P.z = P0.z + 64 * a;
    P.v = (const T*)P0.v + 64 * cv;
    Q = Q0;
    Q.dout = (const TD*)Q0.dout + 64 * cv;
    Q.dq = (T*)Q0.dq + 64 * a;
    Q.dk = (T*)Q0.dk + 64 * a;
    Q.dz = Q0.dz + 64 * a;
    Q.dv = (T*)Q0.dv + 64 * cv;
    Q.pv = Q0.pv + 64 * cv;
    Q.mode_qk = cv == 0 ? 1 : 2;
    Q.mode_v = a == 0 ? 1 : 2;
    return P;
}

template <typename T, typename TD>
static int run_bwd_quarters(const Params& P0, const BwdParams& Q0, hipStream_t st)
{
    for (int a = 0; a < 2; ++a)
        for (int cv = 0; cv < 2; ++cv) {
            BwdParams Q;
            const Params P = quarter<T, TD>(P0, Q, Q0, a, cv);
            const int rc = run_bwd<T, TD, 64>(P, Q, st);
            if (rc != GLA_OK) return rc;
        }
    return GLA_OK;
}

// Gated d = 128: o (binary32) of the quarters added up in the dO area, the
// output gate's backward row by row (dO in place of o), then the quarters'
// gradients from dO.  Each quarter keeps the entering states of its o phase
// (its own workspace array), so its gradient phase runs only the reverse
// halves of the states and fold kernels.
template <typename T>
static int run_bwd_gated_quarters(const Params& P0, const BwdParams& Q0, const GatedBwd& G0,
                                  hipStream_t st)
{
    const unsigned units = (unsigned)(P0.B * P0.NH);
    constexpr unsigned blks = 64 * 64 / NTS;
    float* od = (float*)Q0.dout;
    auto states_of = [&](int a, int cv) {
        const int q = 2 * a + cv;
        return q == 0 ? Q0.ws_f : G0.fq + (size_t)(q - 1) * G0.fq_floats;
    };
    for (int a = 0; a < 2; ++a)
        for (int cv = 0; cv < 2; ++cv) {
            BwdParams Q;
            const Params P = quarter<T, float>(P0, Q, Q0, a, cv);
            Q.ws_f = states_of(a, cv);
            if (P.nchunks > 1) {
                hipLaunchKernelGGL((gla_bwd_states_kernel<T, float, 64, true, false>),
                                   dim3(units * P.nchunks), dim3(NTS), 0, st, P, Q);
                hipLaunchKernelGGL((gla_bwd_fold_kernel<64, true, false>), dim3(units * blks), dim3(NTS),
                                   0, st, P, Q);
            }
            GatedBwd G = G0;
            G.o_out = od + 64 * cv;
            G.o_acc = a;
            hipLaunchKernelGGL((gla_bwd_oepi_kernel<T, 64, true>), dim3(units * P.nchunks), dim3(NT), 0,
                               st, P, Q, G);
        }
    const int rows = P0.B * P0.L * P0.NH;
    const int nblk = (rows + 63) / 64;
    hipLaunchKernelGGL((gla_bwd_epi_rows_kernel<T, 128>), dim3(nblk), dim3(NER), 0, st, od, G0, rows);
    if (G0.dw)
        hipLaunchKernelGGL((gla_bwd_dw_kernel<128>), dim3(1), dim3(NDW), 0, st, G0.dwp, G0.dw, nblk);
    for (int a = 0; a < 2; ++a)
        for (int cv = 0; cv < 2; ++cv) {
            BwdParams Q;
            const Params P = quarter<T, float>(P0, Q, Q0, a, cv);
            Q.ws_f = states_of(a, cv);
            if (P.nchunks > 1) {
                hipLaunchKernelGGL((gla_bwd_states_kernel<T, float, 64, false, true>),
                                   dim3(units * P.nchunks), dim3(NTS), 0, st, P, Q);
                hipLaunchKernelGGL((gla_bwd_fold_kernel<64, false, true>), dim3(units * blks), dim3(NTS),
                                   0, st, P, Q);
            }
            hipLaunchKernelGGL((gla_bwd_chunk_kernel<T, float, 64>), dim3(units * P.nchunks), dim3(NT), 0, st,
                               P, Q);
        }
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

template <typename T, typename TD>
static int run_bwd_d(const Params& P, const BwdParams& Q, int d, hipStream_t st)
{
    switch (d) {
    case 16: return run_bwd<T, TD, 16>(P, Q, st);
    case 32: return run_bwd<T, TD, 32>(P, Q, st);
    case 64: return run_bwd<T, TD, 64>(P, Q, st);
    case 128: return run_bwd_quarters<T, TD>(P, Q, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace bwd

int launch_bwd(const Params& P, const BwdParams& Q, int dtype, int d, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (dtype == GLA_F16) return bwd::run_bwd_d<_Float16, _Float16>(P, Q, d, st);
    if (dtype == GLA_F32) return bwd::run_bwd_d<float, float>(P, Q, d, st);
    return GLA_EUNSUPPORTED;
}

int launch_bwd_gated(const Params& P, const BwdParams& Q, const GatedBwd& G, int dtype, int d,
                     void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (dtype != GLA_F16 && dtype != GLA_F32) return GLA_EUNSUPPORTED;
    const bool h = dtype == GLA_F16;
    switch (d) {
    case 16: return h ? bwd::run_bwd_gated<_Float16, 16>(P, Q, G, st) : bwd::run_bwd_gated<float, 16>(P, Q, G, st);
    case 32: return h ? bwd::run_bwd_gated<_Float16, 32>(P, Q, G, st) : bwd::run_bwd_gated<float, 32>(P, Q, G, st);
    case 64: return h ? bwd::run_bwd_gated<_Float16, 64>(P, Q, G, st) : bwd::run_bwd_gated<float, 64>(P, Q, G, st);
    case 128: return h ? bwd::run_bwd_gated_quarters<_Float16>(P, Q, G, st) : bwd::run_bwd_gated_quarters<float>(P, Q, G, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace gla
