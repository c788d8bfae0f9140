// gla_wide.hip -- chunkwise forward of key-only gated linear attention for
// d_k = d_v = 128 with binary16 storage and 64-token chunks on gfx950: the
// aggregate and output passes of the three-pass scheme (the fold pass between
// them is shared with gla_kernel.hip).
//
// Same mathematics as gla_kernel.hip (paper "GTR: Gated Token Recurrence for
// Efficient Dense Prediction", Section 2.1; chunkwise regrouping of the GLA
// recurrence).  With bl the cumulative log2-decay inside a 16-token
// sub-chunk, tot_m the total of sub-chunk m and R_i = sum_{m < i} tot_m:
//     Qbase_t = q_t (.) 2^{bl_t}                   (<= |q|)
//     E_s     = k_s (.) 2^{tot_j - bl_s}           (<= |k|)
//     A(t, s) = (Qbase_t (.) 2^{R_i - R_j - tot_j}) . E_s   for s in sub-chunk j <= i
//     o_t     = scale [ (Qbase_t (.) 2^{R_i}) S_prev + sum_{s <= t} A(t, s) v_s ]
//     S_new   = Diag(2^{R_4}) S_prev + sum_s (E_s (.) 2^{R_4 - R_j - tot_j})^T v_s
// The diagonal blocks use split binary16 operands and fall back to an exact
// pairwise fp32 evaluation when a sub-chunk's decay span exceeds 2^8.
//
// A workgroup of 8 wavefronts walks the chunks of one segment of one scan.
// Each wavefront plays two roles per chunk:
//  row role    wave w = (i, h): the 16 tokens of sub-chunk i = w & 3 and key
//              channels 64h .. 64h+63 (h = w >> 2).  A lane holds 16 channels
//              of one token: the gate stage (log-decay prefix along the
//              sub-chunk with DPP row scans), the operand forms and the
//              intra-chunk scores over the wave's channels.
//  state role  wave w owns value columns 16w .. 16w+15 of the 128x128 fp32
//              state for every key channel (8 MFMA tiles in registers) and
//              computes those output columns for all 64 tokens: the
//              inter-chunk term, scores times values, the epilogue and the
//              state update.
// Operands that contract over tokens (k-hat^T, v^T) are kept row-major in LDS
// and read with the gfx950 transpose load (ds_read_b64_tr_b16); the state
// enters the inter-chunk product straight from its accumulator registers
// (the k-slots of both operands are permuted to match the accumulator
// layout), so it never passes through LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"
#include "gla_geometry.h"
#include "gla_launch.h"

namespace gla {
namespace wide {

constexpr int NT = 512;   // threads per workgroup
constexpr int NW = 8;     // wavefronts
constexpr int D = 128;    // head dim (d_k = d_v)
constexpr int C = 64;     // chunk
constexpr int NSUB = 4;   // sub-chunks per chunk
constexpr int SH = D + 8;     // binary16 [token][channel] rows (272 bytes)
constexpr int SA = C + 8;     // binary16 score rows [t][s] (144 bytes)
constexpr int SAL = 16 + 8;   // binary16 diagonal low parts [t][s mod 16] (48 bytes)
// per-wave factor tables over the wave's 64 channels
constexpr int FD = 0;   // 2^{-tot_i}                 diagonal query factor (>= 1)
constexpr int FQ = 1;   // 2^{R_i}                    query factor of the inter-chunk term
constexpr int FK = 2;   // 2^{R_4 - R_i - tot_i}      k-hat from E
constexpr int F1 = 3;   // 2^{tot_{i-1}}              query factor for key sub-chunk i-2
constexpr int F2 = 4;   // 2^{tot_{i-1} + tot_{i-2}}  query factor for key sub-chunk i-3
constexpr int NFAC = 5;
constexpr int NPA = 10; // partial score tiles exchanged per chunk

// LDS layout (bytes)
constexpr int L_E = 0;                          // E hi            [C][SH] f16
constexpr int L_QH = L_E + C * SH * 2;          // q (.) 2^{b}     [C][SH] f16
constexpr int L_KH = L_QH + C * SH * 2;         // k-hat           [C][SH] f16
constexpr int L_V = L_KH + C * SH * 2;          // v               [C][SH] f16
constexpr int L_R = L_V + C * SH * 2;           // r, then output staging [C][SH] f16
constexpr int L_PA = L_R + C * SH * 2;          // partial scores  [NPA][64 lanes][4] f32
constexpr int L_A = L_PA + NPA * 64 * 16;       // scores hi       [C][SA] f16
constexpr int L_AL = L_A + C * SA * 2;          // diagonal lo     [C][SAL] f16
constexpr int L_FAC = L_AL + C * SAL * 2;       // factors         [NW][NFAC][64] f32
constexpr int L_TOT = L_FAC + NW * NFAC * 64 * 4;  // sub-chunk totals [NSUB][D] f32
constexpr int L_DEC = L_TOT + NSUB * D * 4;     // 2^{chunk total} [D] f32
constexpr int L_SS = L_DEC + D * 4;             // RMS partials    [C][NW] f32
constexpr int L_ROWS = L_SS + C * NW * 4;       // row tables      [2][C] i32
constexpr int L_MISC = L_ROWS + 2 * C * 4;      // wide flags      [NW] i32
constexpr int LDS_TOTAL = L_MISC + 64;
static_assert(LDS_TOTAL <= kLdsLimit, "LDS budget of one CU exceeded");

// The aggregate pass uses only k-hat, v and the gate tables: its own compact
// layout lets two of its workgroups share a CU.
template <bool AGG> struct Lay {
    static constexpr int KH = AGG ? 0 : L_KH;
    static constexpr int V = AGG ? C * SH * 2 : L_V;
    static constexpr int FAC = AGG ? V + C * SH * 2 : L_FAC;
    static constexpr int TOT = AGG ? FAC + NW * NFAC * 64 * 4 : L_TOT;
    static constexpr int DEC = AGG ? TOT + NSUB * D * 4 : L_DEC;
    static constexpr int ROWS = AGG ? DEC + D * 4 : L_ROWS;
    static constexpr int MISC = AGG ? ROWS + 2 * C * 4 : L_MISC;
    static constexpr int TOTAL = AGG ? MISC + 64 : LDS_TOTAL;
};
static_assert(2 * Lay<true>::TOTAL <= kLdsLimit, "two aggregate workgroups must share a CU");

// MFMA fragment of a row-major [token][col] tile contracted over tokens.
__device__ __forceinline__ half8 tr_frag(const _Float16* base, int row0, int col0, int l16)
{
    return tr_frag_s<SH>(base, row0, col0, l16);
}

// Inputs of one token for the lane's 16 channels cb + {0..7} and cb + 32 + {0..7}.
struct Raw {
    u32x4 q[2], k[2], v[2], r[2], z[4];
};

enum Part { PZ, PK, PQ, PV, PR };

// One input of one token (the lane's 16 channels), zero past the end: read
// through a buffer resource bounded by the tensor's size, where a row past
// the end takes an offset beyond every record (no select per dword).
template <int PART>
__device__ __forceinline__ void load_part(Raw& x, const Params& P, int row, int cb)
{
    const unsigned rows = (unsigned)(P.B * P.L * P.NH);
    const unsigned es = PART == PZ ? 4u : 2u;
    const void* base = PART == PZ ? (const void*)P.z : PART == PK ? P.k : PART == PQ ? P.q
                     : PART == PV ? P.v : P.r;
    // without an output gate r has no records: its loads read zero
    const __amdgpu_buffer_rsrc_t rs = xrsrc(base, (PART == PR && !P.r) ? 0u : rows * D * es);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const unsigned off = row >= 0 ? (unsigned)(row * D + cb + 32 * kb) * es : kPastEnd;
        if (PART == PZ) {
            x.z[2 * kb] = ld_b128(rs, off);
            x.z[2 * kb + 1] = ld_b128(rs, off + 16u);
        }
        if (PART == PK) x.k[kb] = ld_b128(rs, off);
        if (PART == PQ) x.q[kb] = ld_b128(rs, off);
        if (PART == PV) x.v[kb] = ld_b128(rs, off);
        if (PART == PR) x.r[kb] = ld_b128(rs, off);
    }
}

template <bool AGG>
__device__ __forceinline__ void load_raw(Raw& x, const Params& P, int row, int cb, bool gated)
{
    load_part<PZ>(x, P, row, cb);
    load_part<PK>(x, P, row, cb);
    load_part<PV>(x, P, row, cb);
    if (!AGG) {
        load_part<PQ>(x, P, row, cb);
        load_part<PR>(x, P, row, cb);
    }
}

// Clamped per-token log2-decay a = log2(sigmoid(z)) / tau of 16 channels,
// prefix-summed along the sub-chunk.  Tokens past the end of the scan (zero
// inputs, only in the scan's last chunk, which the aggregate pass never
// takes) keep the finite decay of z = 0: it enters only the state after the
// last chunk, which is never used, and sub-chunk totals that cancel in the
// scores.
__device__ __forceinline__ void gate_prefix(const Raw& x, float inv_tau, float (&bl)[16])
{
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float4v zz = __builtin_bit_cast(float4v, x.z[j >> 2]);
        bl[j] = log2_decay(zz[j & 3], inv_tau);
    }
    row_scan_n(bl);
}

// Exact diagonal block over the wave's 64 channels, pairwise in fp32:
// lane (g, l16) returns A(t = l16, s = 4g + e) = sum_c q_t k_s 2^{bl_t - bl_s}
// for s <= t (0 above the diagonal).  Taken only when the factorised form
// would leave the binary16 range; the token's inputs are reloaded.
__device__ __forceinline__ float4v diag_pairwise(const Params& P, int row, int cb, int g,
                                              int l16)
{
    Raw x;
    load_raw<false>(x, P, row, cb, false);
    float bl[16], qv[16], kv[16];
    gate_prefix(x, P.inv_tau, bl);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        qv[j] = (float)__builtin_bit_cast(half8, x.q[j >> 3])[j & 7];
        kv[j] = (float)__builtin_bit_cast(half8, x.k[j >> 3])[j & 7];
    }
    float4v res = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int s = 0; s < 16; ++s) {
        const int src = (g << 4) | s;
        float val = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float ks = __shfl(kv[j], src);
            const float bs = __shfl(bl[j], src);
            val += qv[j] * ks * exp2_fast(bl[j] - bs);
        }
        if (s > l16) val = 0.f;
        val += __shfl_xor(val, 16);
        val += __shfl_xor(val, 32);
        if ((s >> 2) == g) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((s & 3) == e) res[e] = val;
        }
    }
    return res;
}

// Aggregate pass: at most 128 VGPRs (four waves per SIMD) and the compact LDS
// layout, so two workgroups share a CU.  Output pass: one workgroup per CU
// (LDS), up to 256 VGPRs.
template <bool AGG>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(AGG ? 4 : 2, AGG ? 4 : 2)))
void gla_wide_kernel(Params P)
{
    typedef Lay<AGG> LY;
    __shared__ __attribute__((aligned(16))) char lds[LY::TOTAL];
    // buffers of the output pass only (not touched by the aggregate pass)
    _Float16* sE = (_Float16*)(lds + (AGG ? 0 : L_E));
    _Float16* sQH = (_Float16*)(lds + (AGG ? 0 : L_QH));
    _Float16* sR = (_Float16*)(lds + (AGG ? 0 : L_R));
    float* sPA = (float*)(lds + (AGG ? 0 : L_PA));
    _Float16* sA = (_Float16*)(lds + (AGG ? 0 : L_A));
    _Float16* sAL = (_Float16*)(lds + (AGG ? 0 : L_AL));
    float* sSS = (float*)(lds + (AGG ? 0 : L_SS));
    // buffers of both passes
    _Float16* sKH = (_Float16*)(lds + LY::KH);
    _Float16* sV = (_Float16*)(lds + LY::V);
    float* sFac = (float*)(lds + LY::FAC);
    float* sTot = (float*)(lds + LY::TOT);
    float* sDec = (float*)(lds + LY::DEC);
    int* sRows = (int*)(lds + LY::ROWS);
    int* sMisc = (int*)(lds + LY::MISC);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int si = wave & 3;        // row role: sub-chunk
    const int h = wave >> 2;        // row role: channel half
    const int tl = 16 * si + l16;   // row role: token in the chunk
    const int cb = 64 * h + 8 * g;  // row role: channels cb + {0..7}, cb + 32 + {0..7}

    const int nunits = P.B * P.NH;
    // The output pass takes the segments in reverse order: its first round
    // re-reads the inputs the aggregate pass read last, which the last-level
    // cache still holds (about 1 % per call).
    const int seg = AGG ? blockIdx.x / nunits : P.nseg - 1 - blockIdx.x / nunits;
    const int unit = blockIdx.x % nunits;
    const int c_begin = seg * P.seg_chunks;
    const int c_end = min(P.nchunks, c_begin + P.seg_chunks);
    const bool gated = !AGG && P.r != nullptr;
    const size_t slot_floats = (size_t)D * D + D;

    // state role: S[a][e] = S[16a + 4g + e][16 wave + l16]
    float4v S[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) S[a] = float4v{0.f, 0.f, 0.f, 0.f};
    if (!AGG && seg > 0) {
        const float* src = P.ws + ((size_t)unit * (P.nseg - 1) + (seg - 1)) * slot_floats;
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[a][e] = src[(size_t)(16 * a + 4 * g + e) * D + 16 * wave + l16];
    }
    bool have_state = AGG || seg > 0;
    float gacc = 0.f;  // aggregate pass: segment log2-decay of channel 64h + lane (si == 0)
    float wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = (gated && P.w) ? P.w[16 * wave + 4 * g + e] : 1.f;

    if (!AGG) {
        // score tiles above the diagonal that the value product reads: zero for good
        for (int i = tid; i < 2 * 16 * 16; i += NT) {
            const int blk = i >> 8, rr = (i >> 4) & 15, cc = i & 15;
            sA[(32 * blk + rr) * SA + 32 * blk + 16 + cc] = (_Float16)0.f;
        }
    }
    if (tid < C) sRows[tid] = scan_row(P, unit, c_begin * C + tid);
    __syncthreads();

    Raw raw;
    load_raw<AGG>(raw, P, sRows[tl], cb, gated);

    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1;

        // ================= row role: gate stage =================
        float bl[16];
        gate_prefix(raw, P.inv_tau, bl);
        // The aggregate pass has too little work per chunk to hide a load
        // issued late in it: each input of its next chunk is fetched as soon
        // as this chunk's copy is consumed, from a row index of its own.
        const bool pf = (c + 1 < c_end);
        const int arow = (AGG && pf) ? scan_row(P, unit, (c + 1) * C + tl) : -1;
        if (AGG) load_part<PZ>(raw, P, arow, cb);
        if (l16 == 15) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                *(float4v*)(sTot + si * D + cb + 32 * kb) =
                    float4v{bl[8 * kb], bl[8 * kb + 1], bl[8 * kb + 2], bl[8 * kb + 3]};
                *(float4v*)(sTot + si * D + cb + 32 * kb + 4) =
                    float4v{bl[8 * kb + 4], bl[8 * kb + 5], bl[8 * kb + 6], bl[8 * kb + 7]};
            }
        }
        __syncthreads();  // (1) sub-chunk totals; every reader of the last chunk is done

        if (tid < C && c + 1 < c_end) sRows[(buf ^ 1) * C + tid] = scan_row(P, unit, (c + 1) * C + tid);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            *(u32x4*)(sV + tl * SH + cb + 32 * kb) = raw.v[kb];
            if (gated) *(u32x4*)(sR + tl * SH + cb + 32 * kb) = raw.r[kb];
        }
        if (AGG) load_part<PV>(raw, P, arow, cb);

        // ---- per-channel factors of this wave's sub-chunk, one channel per lane
        float* fac = sFac + wave * NFAC * 64;
        bool wide = false;
        {
            const int ch = 64 * h + lane;
            float tm[NSUB];
#pragma unroll
            for (int m = 0; m < NSUB; ++m) tm[m] = sTot[m * D + ch];
            float rr = 0.f, ti = 0.f, all = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
            for (int m = 0; m < NSUB; ++m) {
                all += tm[m];
                if (m < si) rr += tm[m];
                if (m == si) ti = tm[m];
                if (m == si - 1) t1 = tm[m];
                if (m == si - 2) t2 = tm[m];
            }
            fac[FK * 64 + lane] = exp2_fast(all - rr - ti);
            if (!AGG) {
                fac[FD * 64 + lane] = exp2_fast(-ti);
                fac[FQ * 64 + lane] = exp2_fast(rr);
                fac[F1 * 64 + lane] = exp2_fast(t1);
                fac[F2 * 64 + lane] = exp2_fast(t1 + t2);
                wide = !(-ti <= Fmt<_Float16>::kSpan);
            }
            if (si == 0) {
                sDec[ch] = exp2_fast(all);
                gacc += all;
            }
        }
        // the tables are read back by other lanes of the same wavefront
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- operand forms of this token's 16 channels
        half8 eh[2], el[2], qdh[2], qdl[2], qa[2], qo1[2], qo2[2];
        {
            float maxqd = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int co = 8 * g + 32 * kb;  // channel offset inside the wave's half
                float ti8[8], fk[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ti8[e] = sTot[si * D + cb + 32 * kb + e];
                    fk[e] = fac[FK * 64 + co + e];
                }
                const half8 kh = __builtin_bit_cast(half8, raw.k[kb]);
                half8 khat;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 8 * kb + e;
                    const float ef = (float)kh[e] * exp2_fast(ti8[e] - bl[j]);
                    khat[e] = (_Float16)(ef * fk[e]);
                    if (!AGG) {
                        eh[kb][e] = (_Float16)ef;
                        el[kb][e] = (_Float16)(ef - (float)eh[kb][e]);
                    }
                }
                *(half8*)(sKH + tl * SH + cb + 32 * kb) = khat;
                if (!AGG) {
                    *(half8*)(sE + tl * SH + cb + 32 * kb) = eh[kb];
                    float fd[8], fq[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        fd[e] = fac[FD * 64 + co + e];
                        fq[e] = fac[FQ * 64 + co + e];
                    }
                    const half8 qh = __builtin_bit_cast(half8, raw.q[kb]);
                    half8 qhat;
                    float qb[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        qb[e] = (float)qh[e] * exp2_fast(bl[8 * kb + e]);
                        const float qd = qb[e] * fd[e];
                        maxqd = fmaxf(maxqd, fabsf(qd));
                        qdh[kb][e] = (_Float16)qd;
                        qdl[kb][e] = (_Float16)(qd - (float)qdh[kb][e]);
                        qhat[e] = (_Float16)(qb[e] * fq[e]);
                        qa[kb][e] = (_Float16)qb[e];
                    }
                    *(half8*)(sQH + tl * SH + cb + 32 * kb) = qhat;
                    qo1[kb] = qa[kb];
                    qo2[kb] = qa[kb];
                    if (si >= 2) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) qo1[kb][e] = (_Float16)(qb[e] * fac[F1 * 64 + co + e]);
                    }
                    if (si == 3) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) qo2[kb][e] = (_Float16)(qb[e] * fac[F2 * 64 + co + e]);
                    }
                }
            }
            if (!AGG) {
                // the amplified diagonal query operand must stay in binary16
                // range (a NaN also takes the pairwise path, which propagates it)
                wide |= !(maxqd <= Fmt<_Float16>::kMaxOperand);
                const bool ww = __any(wide);
                if (lane == 0) sMisc[wave] = ww ? 1 : 0;
            }
        }
        if (AGG) load_part<PK>(raw, P, arow, cb);
        const int myrow = sRows[buf * C + tl];
        __syncthreads();  // (2) operands of every wave

        // output pass: the next chunk's inputs (row table written after (1))
        // are fetched in parts spread over this chunk, so the loads stream
        // while it computes
        const int nrow = pf ? sRows[(buf ^ 1) * C + tl] : -1;
        if (!AGG) load_part<PZ>(raw, P, nrow, cb);

        // value fragments, shared by the value product and the state update:
        // lane (g, l16) holds v[32p + 8g + e][16 wave + l16]
        half8 vf[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) vf[p] = tr_frag(sV, 32 * p + 8 * g, 16 * wave, l16);

        float4v o[4];
        if (!AGG) {
            // ================= row role: scores over this wave's 64 channels =================
            const bool wide_i = (sMisc[si] | sMisc[si + 4]) != 0;
            float4v part[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                part[j] = float4v{0.f, 0.f, 0.f, 0.f};
                if (j >= si) continue;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const half8 ek = *(const half8*)(sE + (16 * j + l16) * SH + cb + 32 * kb);
                    const half8 qf = (j == si - 1) ? qa[kb] : (j == si - 2) ? qo1[kb] : qo2[kb];
                    part[j] = mma(ek, qf, part[j]);
                }
            }
            float4v pd = float4v{0.f, 0.f, 0.f, 0.f};
            if (!wide_i) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    pd = mma(eh[kb], qdh[kb], pd);
                    pd = mma(el[kb], qdh[kb], pd);
                    pd = mma(eh[kb], qdl[kb], pd);
                }
            } else {
                pd = diag_pairwise(P, myrow, cb, g, l16);
            }
            // exchange: half 0 finishes the off-diagonal tiles, half 1 the diagonal
            // slots: [0, 4) diagonal partials of half 0, [4, 10) off-diagonal of half 1
            const int tri = si * (si - 1) / 2;  // off-diagonal tiles of earlier sub-chunks
            if (h == 0) {
                *(float4v*)(sPA + (si * 64 + lane) * 4) = pd;
            } else {
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    if (j < si) *(float4v*)(sPA + ((4 + tri + j) * 64 + lane) * 4) = part[j];
            }

            load_part<PK>(raw, P, nrow, cb);
            // ================= state role: inter-chunk term =================
            // o^T[16 wave + 4g + e][16 i + l16] = sum_c S[c][dv] (q (.) 2^b)[t][c]
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = float4v{0.f, 0.f, 0.f, 0.f};
            if (have_state) {
                // the query operands of step p + 1 are read before step p's
                // products, so the LDS latency overlaps them
                auto qop = [&](int p, int i) {
                    const _Float16* qrow = sQH + (16 * i + l16) * SH + 32 * p + 4 * g;
                    const half4 b0 = *(const half4*)qrow;
                    const half4 b1 = *(const half4*)(qrow + 16);
                    return half8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                };
                half8 bq[2][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) bq[0][i] = qop(0, i);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (p + 1 < 4) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) bq[(p + 1) & 1][i] = qop(p + 1, i);
                    }
                    // keep those reads ahead of this step's products
                    __builtin_amdgcn_sched_barrier(0);
                    // k-slots 8g + e: channel 32p + 4g + e (e < 4), 32p + 16 + 4g + e - 4
                    // (the state enters as its binary16 high part)
                    half8 ah;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ah[e] = (_Float16)S[2 * p][e];
                        ah[4 + e] = (_Float16)S[2 * p + 1][e];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = mma(ah, bq[p & 1][i], o[i]);
                }
            }
            __syncthreads();  // (3) partial scores
            load_part<PQ>(raw, P, nrow, cb);

            // ---- row role: full scores of sub-chunk si into the score matrix
            if (h == 0) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    if (j >= si) continue;
                    const float4v at = part[j] + *(const float4v*)(sPA + ((4 + tri + j) * 64 + lane) * 4);
                    *(half4*)(sA + tl * SA + 16 * j + 4 * g) =
                        half4{(_Float16)at[0], (_Float16)at[1], (_Float16)at[2], (_Float16)at[3]};
                }
            } else {
                float4v at = pd + *(const float4v*)(sPA + (si * 64 + lane) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * g + e > l16) at[e] = 0.f;
                half4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = (_Float16)at[e];
                    lo[e] = lo_part(at[e]);
                }
                *(half4*)(sA + tl * SA + 16 * si + 4 * g) = hi;
                *(half4*)(sAL + tl * SAL + 4 * g) = lo;
            }
            __syncthreads();  // (4) scores
            load_part<PV>(raw, P, nrow, cb);

            // ================= state role: scores times values =================
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16* arow = sA + (16 * i + l16) * SA + 8 * g;
#pragma unroll
                for (int p = 0; p <= i / 2; ++p) o[i] = mma(vf[p], *(const half8*)(arow + 32 * p), o[i]);
                // low parts of the diagonal tile: k-slots of lane groups 2(i&1), 2(i&1)+1
                half8 blo = {0, 0, 0, 0, 0, 0, 0, 0};
                if ((g >> 1) == (i & 1)) blo = *(const half8*)(sAL + (16 * i + l16) * SAL + 8 * (g & 1));
                o[i] = mma(vf[i / 2], blo, o[i]);
            }
            // epilogue, part 1: scale and per-token sums of squares
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = o[i] * P.scale;
            if (gated) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float ss = o[i][0] * o[i][0] + o[i][1] * o[i][1] + o[i][2] * o[i][2] + o[i][3] * o[i][3];
                    ss += __shfl_xor(ss, 16);
                    ss += __shfl_xor(ss, 32);
                    if (g == 0) sSS[(16 * i + l16) * NW + wave] = ss;
                }
            }
        }

        // ================= state role: S = Diag(2^{chunk total}) S + k-hat^T v =================
        // k-hat fragments of tile a + 1 read before tile a's products
        half8 kf[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) kf[0][p] = tr_frag(sKH, 32 * p + 8 * g, 0, l16);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            if (a + 1 < 8) {
#pragma unroll
                for (int p = 0; p < 2; ++p) kf[(a + 1) & 1][p] = tr_frag(sKH, 32 * p + 8 * g, 16 * (a + 1), l16);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this tile's products
            const float4v dec = *(const float4v*)(sDec + 16 * a + 4 * g);
            S[a] = S[a] * dec;
#pragma unroll
            for (int p = 0; p < 2; ++p) S[a] = mma(kf[a & 1][p], vf[p], S[a]);
        }
        have_state = true;

        if (!AGG) {
            if (gated) __syncthreads();  // (5) sums of squares
            load_part<PR>(raw, P, nrow, cb);
            // epilogue, part 2: u = SiLU(r) (.) w (.) o / rms(o), staged over r
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * i + l16;
                _Float16* srow = sR + t * SH + 16 * wave + 4 * g;
                half4 u;
                if (gated) {
                    const float4v s0 = *(const float4v*)(sSS + t * NW);
                    const float4v s1 = *(const float4v*)(sSS + t * NW + 4);
                    const float ss = (s0[0] + s0[1]) + (s0[2] + s0[3]) + ((s1[0] + s1[1]) + (s1[2] + s1[3]));
                    const float inv = rsq_fast(ss * (1.0f / D) + P.eps);
                    const half4 rv = *(const half4*)srow;
#pragma unroll
                    for (int e = 0; e < 4; ++e) u[e] = (_Float16)(silu((float)rv[e]) * wv[e] * o[i][e] * inv);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) u[e] = (_Float16)o[i][e];
                }
                *(half4*)srow = u;
            }
            __syncthreads();  // (6) staged rows
            // coalesced row stores: 16 pieces of 16 bytes per row, non-temporal
            // (written once; measured 324 -> 315 us per call on the 16K-token
            // 12-block stack)
            const int* rows = sRows + buf * C;
            const __amdgpu_buffer_rsrc_t ro = xrsrc(P.out, (unsigned)(P.B * P.L * P.NH) * D * 2u);
#pragma unroll
            for (int p = 0; p < C * 16 / NT; ++p) {
                const int idx = tid + p * NT;
                const int row = idx >> 4, piece = idx & 15;
                const int t = rows[row];
                // rows past the end of the scan take an offset past every record
                // (the store is dropped), so no store sits behind a branch
                const unsigned off = t >= 0 ? (unsigned)t * D * 2u + 16u * piece : kPastEnd;
                __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)((const char*)(sR + row * SH) + piece * 16),
                                                       ro, (int)off, 0, kNonTemporal);
            }
        }
    }

    if (AGG) {
        // segment aggregate: local state from zero and total log2-decay,
        // written through to memory (agent-scope stores), where the fold
        // kernel reads them
        float* dst = P.ws + ((size_t)unit * (P.nseg - 1) + seg) * slot_floats;
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __hip_atomic_store(dst + (size_t)(16 * a + 4 * g + e) * D + 16 * wave + l16, S[a][e],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (si == 0)
            __hip_atomic_store(dst + (size_t)D * D + 64 * h + lane, gacc, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace wide

int launch_wide(const Params& P, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    const unsigned units = (unsigned)(P.B * P.NH);
    if (P.nseg > 1) {
        hipLaunchKernelGGL(wide::gla_wide_kernel<true>, dim3((P.nseg - 1) * units), dim3(wide::NT),
                           0, st, P);
        const int st1 = launch_fold(P, wide::D, stream);
        if (st1 != GLA_OK) return st1;
    }
    hipLaunchKernelGGL(wide::gla_wide_kernel<false>, dim3(P.nseg * units), dim3(wide::NT), 0, st, P);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

}  // namespace gla
