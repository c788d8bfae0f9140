// gla_onepass.hip -- single-pass chunkwise forward of key-only gated linear
// attention for gfx950 (binary16 storage, d_k = d_v = 64, 64-token chunks).
//
// Same mathematics as gla_kernel.hip (paper "GTR: Gated Token Recurrence for
// Efficient Dense Prediction", Section 2.1; chunkwise regrouping of the GLA
// recurrence), organised so every input byte is read from HBM once:
//
//  phase 1  each workgroup (8 wavefronts) takes a ticket, which fixes its
//           (scan, segment), and walks the segment's chunks with a local state
//           that starts at zero, keeping the partial outputs and the query
//           operand relative to the segment start in registers.
//  phase 2  it publishes its segment aggregate (local state, total decay),
//           waits until the earlier segments of the same scan have published
//           and folds their transfers from zero, in segment order:
//               S_in = fold_{i < seg} (S -> Diag(2^{G_i}) S + L_i),
//           with the multipliers 2^{G_i} published as computed by segment i;
//           scans of many segments fold per-group combined transfers first
//           (two levels, see the exchange).  The order is fixed, so the bits
//           do not depend on timing (deterministic).  Workgroups only wait on
//           smaller tickets.
//  phase 3  adds (q (.) 2^{b from segment start}) S_in to the kept partial
//           outputs, applies the epilogue and stores every row; the scan's
//           last segment then waits until every earlier one has finished
//           its exchange and clears the scan's flags for the next call.
//
// Work split inside a chunk: wavefront w handles the 16-token sub-chunk
// i = w & 3 and the half h = w >> 2 of the channels.  A lane holds 8 channels
// of one token, which is both the row layout of the MFMA operands and the
// layout the gate stage needs: the log-decay is accumulated along the 16
// tokens of the sub-chunk with a DPP prefix scan across the lane row.  With
// bl the cumulative log2-decay inside the sub-chunk, tot_m the total of
// sub-chunk m and R_i = sum_{m < i} tot_m:
//     Qbase_t = q_t (.) 2^{bl_t}                   (<= |q|)
//     E_s     = k_s (.) 2^{tot_j - bl_s}           (<= |k|, key relative to its sub-chunk end)
//     A(t, s) = (Qbase_t (.) 2^{R_i - R_j - tot_j}) . E_s   for s in sub-chunk j <= i
// The factor is 1 for adjacent sub-chunks and <= 1 for earlier ones; on the
// diagonal it is 2^{-tot_i} >= 1, so that block uses split binary16
// operands and falls back to an exact pairwise fp32 evaluation when the
// sub-chunk's decay span exceeds 2^8.  The two wavefronts of a sub-chunk each
// contract their own 32 channels and exchange the partial score tiles.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_device.h"
#include "gla_geometry.h"
#include "gla_launch.h"

namespace gla {
namespace onepass {

constexpr int NT = 512;   // threads per workgroup
constexpr int NW = 8;     // wavefronts
constexpr int D = 64;     // head dim (d_k = d_v)
constexpr int C = 64;     // chunk
constexpr int NSUB = 4;   // 16-token sub-chunks per chunk
constexpr int NCH = kOnePassMaxChunks;  // chunks per segment (upper bound)
constexpr int SH = D + 8; // binary16 row stride (elements): 144-byte rows
constexpr int SF = D + 4; // fp32 row stride (elements): 272-byte rows
// The incoming state of a segment enters its outputs as binary16 hi + lo.
#ifndef GLA_ONEPASS_IN_LO
#define GLA_ONEPASS_IN_LO 0
#endif
constexpr bool kInLo = GLA_ONEPASS_IN_LO;
// Per-wave factor table rows (sub-chunk i of the wave, 32 channels of its half):
constexpr int FD = 0;     // 2^{-tot_i}                 diagonal query factor (>= 1)
constexpr int FQ = 1;     // 2^{R_i}                    q (.) 2^b for the local inter-chunk term
constexpr int FS = 2;     // 2^{R_i + D_seg}            q (.) 2^b from the segment start
constexpr int FK = 3;     // 2^{total - R_i - tot_i}    k-hat from E
constexpr int F1 = 4;     // 2^{tot_{i-1}}              query factor for key sub-chunk i-2
constexpr int F2 = 5;     // 2^{tot_{i-1} + tot_{i-2}}  query factor for key sub-chunk i-3

// LDS layout (bytes)
constexpr int L_E = 0;                        // E hi          [C][SH] f16 ([token][ch])
constexpr int L_EL = L_E + C * SH * 2;        // E lo          [C][SH] f16
constexpr int L_KT = L_EL + C * SH * 2;       // k-hat         [C][SH] f16 ([token][ch]), read transposed
constexpr int L_VT = L_KT + C * SH * 2;       // v             [C][SH] f16 ([token][dv]), read transposed
constexpr int L_ST = L_VT + C * SH * 2;       // S^T           [D][SH] f16 ([dv][ch])
constexpr int L_QH = L_ST + D * SH * 2;       // q (.) 2^b     [C][SH] f16 ([token][ch])
constexpr int L_PA = L_QH + C * SH * 2;       // partial scores [NW][NSUB][64 lanes][4] f32
constexpr int L_FQ = L_PA + NW * NSUB * 64 * 16;  // raw q      [C][SH] f16 (pairwise fallback)
constexpr int L_FK = L_FQ + C * SH * 2;       // raw k         [C][SH] f16 (pairwise fallback)
constexpr int L_FB = L_FK + C * SH * 2;       // bl            [C][SF] f32 (pairwise fallback)
constexpr int L_TOT = L_FB + C * SF * 4;      // sub-chunk totals [NSUB][D] f32
constexpr int L_DEC = L_TOT + NSUB * D * 4;   // 2^{chunk total} [D] f32
constexpr int L_FAC = L_DEC + D * 4;         // per-wave factors [NW][NFAC][32] f32
constexpr int L_ROWS = L_FAC + NW * 8 * 32 * 4;  // row tables  [NCH][C] i32
constexpr int L_SS = L_ROWS + NCH * C * 4;    // RMS partials   [NCH][2][C] f32
constexpr int L_MISC = L_SS + NCH * 2 * C * 4;  // ticket, wide flags, look-back result
constexpr int LDS_TOTAL = L_MISC + 64;
static_assert(LDS_TOTAL <= kLdsLimit, "LDS budget of one CU exceeded");
// fused gate expansion (z = hp W2 + b with hp = x W1 of rank 16 read per
// token): this head's W2 rows and bias
constexpr int L_W2 = LDS_TOTAL;               // W2^T of the head [D][16] f32
constexpr int L_GB = L_W2 + D * 16 * 4;       // gate bias of the head [D] f32
constexpr int LDS_PROJ = L_GB + D * 4;
static_assert(kFusedProjRank == 16, "the fused gate expansion is built for rank 16");
static_assert(LDS_PROJ <= kLdsLimit, "LDS budget of one CU exceeded (fused gate expansion)");
// phase-2/3 aliases
constexpr int L_LSEG = L_PA;                  // segment local state [D][D] f32 (16 KiB)
constexpr int L_GSEG = L_PA + D * D * 4;      // segment total decay [D] f32
constexpr int L_STL = L_E;                    // S_in^T lo [D][SH] f16
constexpr int L_OUT = L_PA;                   // output staging [NCH][C][SH] f16
static_assert(L_GSEG + D * 4 <= L_TOT, "segment aggregate overlaps live buffers");
static_assert(L_OUT + NCH * C * SH * 2 <= L_TOT, "output staging overlaps live buffers");

// Exchange through device memory.  Every exchanged word (states, decays,
// flags, counters) is accessed with agent-scope atomics, which on gfx950
// bypass the per-XCD L2's non-coherent state (sc1 loads and stores), so no L2
// write-back or invalidate is needed.  A publisher waits until all its state
// stores are acknowledged (s_waitcnt) before any wave sets the flag; a reader
// issues its state loads only after it has seen the flag.
__device__ __forceinline__ unsigned ld_u(const unsigned* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u(unsigned* p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bulk exchange data moves 16 bytes per lane through buffer instructions whose
// record count bounds every access.  Loads always use sc1, which misses the
// CU's L1 and reads the XCD's L2 (or memory).  Aggregates and inclusive states
// are always stored with sc1 (write-through to memory: the policy the compiler
// gives the relaxed agent-scope atomics above, coherent across the per-XCD
// L2s).  Flags: sc1 as well when the workgroups of a scan may run on different
// XCDs; when every workgroup of a scan runs on one XCD (LOCAL), the default
// policy, which leaves the line in that XCD's L2 where the sc1 loads of the
// same XCD find it (about half the round-trip latency).  Measured on MI355X,
// write-back exchange data kept the kernel running 2-3 us after its last
// workgroup had ended (one 1600-token frame with 6 heads: 18.7 us per call
// with write-back aggregates and inclusive states, 15.6 us written through,
// though the exchange inside the workgroups takes about 0.4 us longer), while
// write-through flags slowed every look-back.
template <bool LOCAL> struct Pol {
    static constexpr int kLoad = 16;
    static constexpr int kStore = LOCAL ? 0 : 16;
};
constexpr int kStoreThrough = 16;  // sc1
template <bool LOCAL>
__device__ __forceinline__ float4v ld_x4(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, Pol<LOCAL>::kLoad));
}
template <bool LOCAL>
__device__ __forceinline__ float ld_x1(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, Pol<LOCAL>::kLoad));
}
__device__ __forceinline__ void st_x4(__amdgpu_buffer_rsrc_t r, unsigned off, float4v v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kStoreThrough);
}
__device__ __forceinline__ void st_x1(__amdgpu_buffer_rsrc_t r, unsigned off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off, 0, kStoreThrough);
}
// Segment flags of one scan (0 none, 1 aggregate, 2 inclusive state).
template <bool LOCAL>
__device__ __forceinline__ unsigned ld_flag(const unsigned* flags, int nseg, int i)
{
    if (!LOCAL) return ld_u(flags + i);
    return (unsigned)__builtin_amdgcn_raw_buffer_load_b32(xrsrc(flags, 4u * nseg), 4 * i, 0, Pol<LOCAL>::kLoad);
}
template <bool LOCAL>
__device__ __forceinline__ void st_flag(unsigned* flags, int nseg, int i, unsigned v)
{
    if (!LOCAL) {
        st_u(flags + i, v);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(v, xrsrc(flags, 4u * nseg), 4 * i, 0, Pol<LOCAL>::kStore);
    }
}
// Hardware register XCC_ID: bits 3:0 hold the XCD that runs this workgroup.
constexpr int kXccIdReg = 20 | (0 << 6) | ((4 - 1) << 11);

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// One forward step of the segment fold, S -> Diag(2^G) S + L, with the
// multiplier 2^G as published (identical wherever it is evaluated).
__device__ __forceinline__ float fold_step(float g_mul, float s, float l)
{
    return __builtin_fmaf(g_mul, s, l);
}

template <int N>
__device__ __forceinline__ void ld8f(const float* p, float (&x)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
}

struct Raw {
    u32x4 q, k, v, z0, z1;  // 8 channels of one token (q, k, v binary16; z binary32)
};

// Inputs are read through buffer resources whose record count is the
// tensor's size: a row past the end of the scan (row < 0) takes an offset
// beyond every record and reads zeros, with no branch and no zero-fill.
// (The plan keeps the largest tensor below 2^31 bytes.)
struct Src {
    __amdgpu_buffer_rsrc_t q, k, v, z;
};
__device__ __forceinline__ Src make_src(const Params& P, bool proj)
{
    const unsigned rows = (unsigned)(P.B * P.L * P.NH);
    Src s;
    s.q = xrsrc(P.q, rows * D * 2);
    s.k = xrsrc(P.k, rows * D * 2);
    s.v = xrsrc(P.v, rows * D * 2);
    s.z = proj ? xrsrc(P.ghp, (unsigned)(P.B * P.L) * kFusedProjRank * 4) : xrsrc(P.z, rows * D * 4);
    return s;
}
// PROJ: instead of the 8 gate logits, the lane loads the 4 rank values
// hp[token][4g .. 4g + 3] of its token (the B fragment of the expansion below).
template <bool PROJ>
__device__ __forceinline__ void load_raw(Raw& r, const Src& S, const Params& P, int row, int c0, int g)
{
    const unsigned oh = row >= 0 ? (unsigned)(row * D + c0) * 2u : kPastEnd;
    r.q = ld_b128(S.q, oh);
    r.k = ld_b128(S.k, oh);
    r.v = ld_b128(S.v, oh);
    if (PROJ) {
        r.z0 = ld_b128(S.z, row >= 0 ? (unsigned)((row / P.NH) * kFusedProjRank + 4 * g) * 4u : kPastEnd);
        r.z1 = u32x4{0u, 0u, 0u, 0u};
    } else {
        const unsigned oz = row >= 0 ? (unsigned)(row * D + c0) * 4u : kPastEnd;
        r.z0 = ld_b128(S.z, oz);
        r.z1 = ld_b128(S.z, oz + 16u);
    }
}

// Fused gate expansion.  Gate logits of this lane's token and 8 channels
// 32h + 8g + (0..7): z^T = W2^T hp^T + b with v_mfma_f32_16x16x4_f32 in
// binary32, where the lane (token l16, group g) holds hp[token][4g + e].
// Output tile T
// takes as its row r the channel 32h + 8 (r / 4) + 4T + r % 4, so that the
// accumulator element e of lane (l16, g) is channel 32h + 8g + 4T + e of
// token l16 -- the gate stage's layout.  At step s the lane's k element is
// rank 4g + s, which is exactly element s of its hp fragment.
__device__ __forceinline__ void proj_logits(const float4v& hp, const float* sW2, const float* sGB,
                                            int h, int g, int l16, float (&zv)[8])
{
    float4v acc[2], w[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        acc[T] = *(const float4v*)(sGB + 32 * h + 8 * g + 4 * T);
        const int ch = 32 * h + 8 * (l16 >> 2) + 4 * T + (l16 & 3);
        w[T] = *(const float4v*)(sW2 + ch * 16 + 4 * g);
    }
    // the two tiles' chains interleaved
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int T = 0; T < 2; ++T) acc[T] = mma(w[T][s], hp[s], acc[T]);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[4 * T + e] = acc[T][e];
}

// Intra-chunk scores (M1, with the exchange of the two channel halves) and
// scores times values (M2) for query sub-chunk SI: a compile-time sub-chunk
// keeps every tile selection out of the control flow, so no register array is
// merged across branches.
template <int SI>
__device__ __forceinline__ void scores_values(const Params& P, const _Float16* sE, const _Float16* sEL,
                                              const _Float16* sVT, float* sPA, const int* sMisc,
                                              const _Float16* sFQ, const _Float16* sFK, const float* sFB,
                                              int wave, int lane, int g, int l16, int h, int c0, int tl,
                                              const half8& qa, const half8& qo1, const half8& qo2,
                                              const half8& qd_h, const half8& qd_l, float4v (&o)[2])
{
    // ---- M1 partial scores over this wave's 32 channels, tiles j <= SI
    //      (j < SI off the diagonal; the diagonal tile separately)
    const bool wide_i = (sMisc[4 + SI] | sMisc[4 + SI + 4]) != 0;
    float4v part[NSUB];
#pragma unroll
    for (int j = 0; j < NSUB - 1; ++j) {
        part[j] = float4v{0.f, 0.f, 0.f, 0.f};
        if (j >= SI) continue;
        const half8 ek = *(const half8*)(sE + (16 * j + l16) * SH + c0);
        const half8 qf = (j == SI - 1) ? qa : (j == SI - 2) ? qo1 : qo2;
        part[j] = mma(ek, qf, part[j]);
        *(float4v*)(sPA + ((wave * NSUB + j) * 64 + lane) * 4) = part[j];
    }
    float4v pd = float4v{0.f, 0.f, 0.f, 0.f};
    if (!wide_i) {
        const half8 ek = *(const half8*)(sE + tl * SH + c0);
        const half8 ekl = *(const half8*)(sEL + tl * SH + c0);
        pd = mma(ek, qd_h, pd);
        pd = mma(ekl, qd_h, pd);
        pd = mma(ek, qd_l, pd);
    } else {
        // exact pairwise over this wave's channels: q_t k_s 2^{bl_t - bl_s}
        // (rare: a sub-chunk whose decay span is too wide for binary16)
#pragma unroll 1
        for (int e = 0; e < 4; ++e) {
            const int sl = 4 * g + e;
            float acc = 0.f;
            if (sl <= l16) {
                const int ts = 16 * SI + sl;
#pragma unroll 1
                for (int cc = 32 * h; cc < 32 * h + 32; ++cc)
                    acc += (float)sFQ[tl * SH + cc] * (float)sFK[ts * SH + cc] *
                           exp2_fast(sFB[tl * SF + cc] - sFB[ts * SF + cc]);
            }
            pd[e] = acc;
        }
    }
    *(float4v*)(sPA + ((wave * NSUB + SI) * 64 + lane) * 4) = pd;
    __syncthreads();  // (3) partial scores of both halves
    float4v at[NSUB];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
        at[j] = float4v{0.f, 0.f, 0.f, 0.f};
        if (j > SI) continue;
        const float4v other = *(const float4v*)(sPA + (((wave ^ 4) * NSUB + j) * 64 + lane) * 4);
        if (j < SI) {
            at[j] = part[j] + other;
        } else {
            at[j] = pd + other;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * g + e > l16) at[j][e] = 0.f;
        }
    }

    // ---- M2: O^T[dv][t] += V^T A^T, this wave's 32 value channels
    o[0] = o[1] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NSUB / 2; ++p) {
        if (2 * p > SI) continue;
        const bool hi = (2 * p + 1 <= SI);
        half8 bfr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bfr[e] = (_Float16)at[2 * p][e];
            bfr[4 + e] = hi ? (_Float16)at[2 * p + 1][e] : (_Float16)0.f;
        }
        half8 blo = {0, 0, 0, 0, 0, 0, 0, 0};
        if (2 * p == SI) {
#pragma unroll
            for (int e = 0; e < 4; ++e) blo[e] = lo_part(at[2 * p][e]);
        }
        if (2 * p + 1 == SI) {
#pragma unroll
            for (int e = 0; e < 4; ++e) blo[4 + e] = lo_part(at[2 * p + 1][e]);
        }
        const bool has_diag = (2 * p == SI) || (2 * p + 1 == SI);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            // value rows 32p + 4g + e and 32p + 16 + 4g + e of column 32h + 16m + l16
            const half4 v0 = ld_tr(tr_addr<SH>(sVT, 32 * p + 4 * g, 32 * h + 16 * m, l16));
            half4 v1 = {0, 0, 0, 0};
            if (hi) v1 = ld_tr(tr_addr<SH>(sVT, 32 * p + 16 + 4 * g, 32 * h + 16 * m, l16));
            half8 afr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                afr[e] = v0[e];
                afr[4 + e] = v1[e];
            }
            o[m] = mma(afr, bfr, o[m]);
            if (has_diag) o[m] = mma(afr, blo, o[m]);
        }
    }
}

template <bool LOCAL, bool PROJ, int NCHK>
__global__ __launch_bounds__(NT) void gla_onepass_kernel(Params P)
{
    __shared__ __attribute__((aligned(16))) char lds[PROJ ? LDS_PROJ : LDS_TOTAL];
    _Float16* sE = (_Float16*)(lds + L_E);
    _Float16* sEL = (_Float16*)(lds + L_EL);
    _Float16* sKT = (_Float16*)(lds + L_KT);
    _Float16* sVT = (_Float16*)(lds + L_VT);
    _Float16* sST = (_Float16*)(lds + L_ST);
    _Float16* sQH = (_Float16*)(lds + L_QH);
    float* sPA = (float*)(lds + L_PA);
    _Float16* sFQ = (_Float16*)(lds + L_FQ);
    _Float16* sFK = (_Float16*)(lds + L_FK);
    float* sFB = (float*)(lds + L_FB);
    float* sTot = (float*)(lds + L_TOT);
    float* sDec = (float*)(lds + L_DEC);
    float* sFac = (float*)(lds + L_FAC);
    int* sRows = (int*)(lds + L_ROWS);
    float* sSS = (float*)(lds + L_SS);
    int* sMisc = (int*)(lds + L_MISC);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int si = wave & 3;        // sub-chunk of this wave
    const int h = wave >> 2;        // channel half (phase 1) / value half (outputs)
    const int cht = lane & 31;      // table layout: channel 32*h + cht
    const int ht = lane >> 5;       //               first or second group of tables
    const int c0 = 32 * h + 8 * g;  // this lane's 8 channels (row layout)
    const int tl = 16 * si + l16;   // this lane's token in the chunk
    const int nunits = P.B * P.NH;
    const int grid = nunits * P.nseg;

    // ---- ticket: logical (segment, scan) in start order.  LOCAL: scan u runs
    //      on XCD u mod 8; the workgroups of an XCD number their tasks with the
    //      XCD's own counter (the grid gives every XCD the same count).
    if (tid == 0) {
        if (LOCAL) {
            const unsigned x = __builtin_amdgcn_s_getreg(kXccIdReg) & 7u;
            unsigned* ctr = P.ticket + 16 * (1 + x);
            const unsigned t = atomicAdd(ctr, 1u);
            if (t == (unsigned)P.xcd_tasks - 1u) st_u(ctr, 0u);  // every ticket is taken
            sMisc[0] = (int)t;
            sMisc[2] = (int)x;
        } else {
            const unsigned t = atomicAdd(P.ticket, 1u);
            if (t == (unsigned)grid - 1u) st_u(P.ticket, 0u);  // every ticket is taken
            sMisc[0] = (int)t;
        }
    }
    __syncthreads();
    const int ticket = sMisc[0];
    int seg, unit;
    if (LOCAL) {
        const int x = sMisc[2];
        if (ticket >= P.xcd_tasks) {  // workspace not initialised: report, do nothing
            if (tid == 0) atomicOr(P.err, 2u);
            return;
        }
        const int units_x = (nunits - x + 7) / 8;  // scans x, x + 8, ... run here
        if (ticket >= units_x * P.nseg) return;     // spare workgroup of this XCD
        seg = ticket / units_x;
        unit = x + 8 * (ticket - seg * units_x);
    } else {
        if (ticket >= grid) {  // workspace not initialised: report, do nothing
            if (tid == 0) atomicOr(P.err, 2u);
            return;
        }
        seg = ticket / nunits;
        unit = ticket - seg * nunits;
    }
    const int c_begin = seg * P.seg_chunks;
    const int nch = min(P.nchunks, c_begin + P.seg_chunks) - c_begin;
    const bool gated = (P.r != nullptr);

    // ---- first chunk's operands of this lane: issued before anything waits
    const Src src = make_src(P, PROJ);
    Raw raw;
    load_raw<PROJ>(raw, src, P, scan_row(P, unit, c_begin * C + tl), c0, g);

    // ---- row tables of every chunk of the segment
    for (int i = tid; i < nch * C; i += NT) sRows[i] = scan_row(P, unit, c_begin * C + i);
    float* sW2 = (float*)(lds + L_W2);
    float* sGB = (float*)(lds + L_GB);
    if (PROJ) {
        // this head's W2^T rows (D x 16) and bias: one 16-byte load per thread
        const int hd = unit % P.NH;
        if (tid < D * 16 / 4) {
            *(float4v*)(sW2 + 4 * tid) = *(const float4v*)(P.gw2 + (size_t)hd * D * 16 + 4 * tid);
        } else if (tid < D * 16 / 4 + D / 4) {
            const int i = tid - D * 16 / 4;
            *(float4v*)(sGB + 4 * i) =
                P.gb ? *(const float4v*)(P.gb + hd * D + 4 * i) : float4v{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();

    float4v okeep[NCHK][2];
    half8 qkeep[NCHK];    // this lane's 8 channels of the segment-relative query
    float4v S[2];        // this wave's two 16x16 tiles of the local state
    S[0] = S[1] = float4v{0.f, 0.f, 0.f, 0.f};
    const int sa = wave >> 1;         // state tile row block (key channels)
    const int sb0 = 2 * (wave & 1);   // first state tile column block (value channels)
    float dseg = 0.f;                 // decay since segment start, channel 32*h + cht

#pragma unroll
    for (int c = 0; c < NCHK; ++c) {
        if (c >= nch) break;
        float qv[8], kv[8], zv[8];
        const u32x4 raw_v = raw.v;
        {
            const half8 qh = __builtin_bit_cast(half8, raw.q);
            const half8 kh8 = __builtin_bit_cast(half8, raw.k);
            const float4v z0 = __builtin_bit_cast(float4v, raw.z0);
            const float4v z1 = __builtin_bit_cast(float4v, raw.z1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[e] = (float)qh[e];
                kv[e] = (float)kh8[e];
                zv[e] = e < 4 ? z0[e] : z1[e - 4];
            }
            // raw copies for the pairwise fallback of a wide diagonal block
            *(u32x4*)(sFQ + tl * SH + c0) = raw.q;
            *(u32x4*)(sFK + tl * SH + c0) = raw.k;
        }
        if (PROJ) proj_logits(__builtin_bit_cast(float4v, raw.z0), sW2, sGB, h, g, l16, zv);
        if (c + 1 < nch) load_raw<PROJ>(raw, src, P, sRows[(c + 1) * C + tl], c0, g);

        // ---- gate stage: log2-decay, prefix along the 16 tokens of the sub-chunk.
        //      Tokens past the end of the scan (zero q, k, v, only in its last
        //      chunk) keep their finite decay: it enters only quantities after
        //      every valid token (sub-chunk totals that cancel in the scores,
        //      the state after the last chunk, which is never published).
        float bl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bl[e] = log2_decay(zv[e], P.inv_tau);
        row_scan_n(bl);
        if (l16 == 15) {
            *(float4v*)(sTot + si * D + c0) = float4v{bl[0], bl[1], bl[2], bl[3]};
            *(float4v*)(sTot + si * D + c0 + 4) = float4v{bl[4], bl[5], bl[6], bl[7]};
        }
        *(float4v*)(sFB + tl * SF + c0) = float4v{bl[0], bl[1], bl[2], bl[3]};
        *(float4v*)(sFB + tl * SF + c0 + 4) = float4v{bl[4], bl[5], bl[6], bl[7]};
        __syncthreads();  // (1) sub-chunk totals

        // ---- per-channel factors of this wave's sub-chunk and channel half,
        //      computed once per channel (table layout) and read back per lane
        float* fac = sFac + wave * 8 * 32;
        bool wide = false;
        {
            const int ch = 32 * h + cht;
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
            if (ht == 0) {
                fac[FD * 32 + cht] = exp2_fast(-ti);
                fac[FQ * 32 + cht] = exp2_fast(rr);
                fac[FS * 32 + cht] = exp2_fast(rr + dseg);
                wide = !(-ti <= Fmt<_Float16>::kSpan);
                if (si == 0) sDec[ch] = exp2_fast(all);
            } else {
                fac[FK * 32 + cht] = exp2_fast(all - rr - ti);
                fac[F1 * 32 + cht] = exp2_fast(t1);
                fac[F2 * 32 + cht] = exp2_fast(t1 + t2);
            }
            dseg += all;
        }
        // the tables are read back by other lanes of the same wavefront
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- operands of this token and channel group
        float ti8[8], fd[8], fq[8], fs[8], fk[8];
        ld8f(sTot + si * D + c0, ti8);
        ld8f(fac + FD * 32 + 8 * g, fd);
        ld8f(fac + FQ * 32 + 8 * g, fq);
        ld8f(fac + FS * 32 + 8 * g, fs);
        ld8f(fac + FK * 32 + 8 * g, fk);
        float qb[8];
        half8 eh, el, kt8, qd_h, qd_l, qhat, qs, qa;
        float maxqd = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qb[e] = qv[e] * exp2_fast(bl[e]);
            const float ef = kv[e] * exp2_fast(ti8[e] - bl[e]);
            eh[e] = (_Float16)ef;
            el[e] = (_Float16)(ef - (float)eh[e]);
            kt8[e] = (_Float16)(ef * fk[e]);
            const float qd = qb[e] * fd[e];
            maxqd = fmaxf(maxqd, fabsf(qd));
            qd_h[e] = (_Float16)qd;
            qd_l[e] = (_Float16)(qd - (float)qd_h[e]);
            qhat[e] = (_Float16)(qb[e] * fq[e]);
            qs[e] = (_Float16)(qb[e] * fs[e]);
            qa[e] = (_Float16)qb[e];
        }
        // the amplified diagonal query operand must stay in binary16 range
        // (a NaN also takes the pairwise path, which propagates it)
        wide |= !(maxqd <= Fmt<_Float16>::kMaxOperand);
        *(half8*)(sE + tl * SH + c0) = eh;
        *(half8*)(sEL + tl * SH + c0) = el;
        *(half8*)(sQH + tl * SH + c0) = qhat;
        *(half8*)(sKT + tl * SH + c0) = kt8;
        *(u32x4*)(sVT + tl * SH + c0) = raw_v;
        {
            const bool ww = __any(wide);
            if (lane == 0) sMisc[4 + wave] = ww ? 1 : 0;
        }
        qkeep[c] = qs;
        // off-diagonal query operands for key sub-chunks i-2 and i-3
        half8 qo1 = qa, qo2 = qa;
        if (si >= 2) {
            float f[8];
            ld8f(fac + F1 * 32 + 8 * g, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) qo1[e] = (_Float16)(qb[e] * f[e]);
        }
        if (si == 3) {
            float f[8];
            ld8f(fac + F2 * 32 + 8 * g, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) qo2[e] = (_Float16)(qb[e] * f[e]);
        }
        __syncthreads();  // (2) operands of every wave

        float4v o[2];
        switch (si) {
        case 0: scores_values<0>(P, sE, sEL, sVT, sPA, sMisc, sFQ, sFK, sFB, wave, lane, g, l16, h, c0, tl, qa, qo1, qo2, qd_h, qd_l, o); break;
        case 1: scores_values<1>(P, sE, sEL, sVT, sPA, sMisc, sFQ, sFK, sFB, wave, lane, g, l16, h, c0, tl, qa, qo1, qo2, qd_h, qd_l, o); break;
        case 2: scores_values<2>(P, sE, sEL, sVT, sPA, sMisc, sFQ, sFK, sFB, wave, lane, g, l16, h, c0, tl, qa, qo1, qo2, qd_h, qd_l, o); break;
        default: scores_values<3>(P, sE, sEL, sVT, sPA, sMisc, sFQ, sFK, sFB, wave, lane, g, l16, h, c0, tl, qa, qo1, qo2, qd_h, qd_l, o); break;
        }
        // ---- M3: O^T += S_loc^T (q (.) 2^b)^T, local state from the segment start
        if (c > 0) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const half8 qf = *(const half8*)(sQH + tl * SH + 32 * kb + 8 * g);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const half8 sfr = *(const half8*)(sST + (32 * h + 16 * m + l16) * SH + 32 * kb + 8 * g);
                    o[m] = mma(sfr, qf, o[m]);
                }
            }
        }
        okeep[c][0] = o[0];
        okeep[c][1] = o[1];

        // ---- M4: local state update S = Diag(2^{chunk total}) S + k-hat^T v
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int bb = sb0 + jj;
#pragma unroll
            for (int e = 0; e < 4; ++e) S[jj][e] *= sDec[16 * sa + 4 * g + e];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const half8 kf = tr_frag_s<SH>(sKT, 32 * kb + 8 * g, 16 * sa, l16);
                const half8 vf = tr_frag_s<SH>(sVT, 32 * kb + 8 * g, 16 * bb, l16);
                S[jj] = mma(kf, vf, S[jj]);
            }
        }
        __syncthreads();  // (4) all readers of this chunk's buffers are done
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int bb = sb0 + jj;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sST[(16 * bb + l16) * SH + 16 * sa + 4 * g + e] = (_Float16)S[jj][e];
        }
    }

    // r of every chunk at this lane's output positions (token tl, value
    // channels 32h + 16m + 4g .. +3): loads issued now, in flight during the
    // exchange
    half4 rreg[NCHK][2];
#pragma unroll
    for (int cc = 0; cc < NCHK; ++cc) {
#pragma unroll
        for (int m = 0; m < 2; ++m) rreg[cc][m] = half4{0, 0, 0, 0};
        if (gated && cc < nch) {
            const int t = sRows[cc * C + tl];
            if (t >= 0) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    rreg[cc][m] = *(const half4*)((const _Float16*)P.r + (size_t)t * D + 32 * h + 16 * m + 4 * g);
            }
        }
    }

    // ================= phase 2: segment exchange =================
    const size_t aggf = (size_t)D * D + D;
    const size_t slot = (size_t)unit * P.nseg + seg;
    float* sL = (float*)(lds + L_LSEG);
    float* sG = (float*)(lds + L_GSEG);
    _Float16* sSTL = (_Float16*)(lds + L_STL);
    const bool need_in = (seg > 0);
    if (P.nseg > 1) {
        // local state and total decay into LDS, row-major [ch][dv]
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int bb = sb0 + jj;
#pragma unroll
            for (int e = 0; e < 4; ++e) sL[(16 * sa + 4 * g + e) * D + 16 * bb + l16] = S[jj][e];
        }
        // total decay of the segment as the factor 2^G (the fold's multiplier)
        if (si == 0 && ht == 0) sG[32 * h + cht] = exp2_fast(dseg);
        __syncthreads();
        const bool last = (seg == P.nseg - 1);
        unsigned* flags = P.flags + (size_t)unit * P.nseg;
        // this thread's 8 state entries: rows ch0 = tid / 16 and ch0 + 32,
        // columns 4 (tid % 16) .. +3 (16 contiguous bytes in each row)
        const int ch0 = tid >> 4, cl0 = 4 * (tid & 15);
        const unsigned off0 = 16u * tid, off1 = off0 + 16u * NT;  // bytes
        const float4v l0 = *(const float4v*)(sL + ch0 * D + cl0);
        const float4v l1 = *(const float4v*)(sL + (ch0 + 32) * D + cl0);
        const unsigned agg_bytes = (unsigned)(aggf * 4), st_bytes = (unsigned)(D * D * 4);
        // Plans whose workgroups all run in one round (every segment starts
        // at the same time) fold published aggregates directly; plans of
        // several rounds use inclusive states, which the segments of earlier
        // rounds have published by the time later ones look back.
        const bool one_round = LOCAL ? (P.xcd_tasks <= 32) : (nunits * P.nseg <= 256);
        if (one_round) {
            // Exchange.  Every segment but the last publishes its aggregate and
            // segment j folds the aggregates of segments 0 .. j-1 from zero, in
            // order.  Scans of many segments use two levels: the segments form
            // groups of G = ceil(sqrt(nseg)); the last segment of a group that has
            // segments after it (the group's leader) publishes the group's
            // combined transfer (its aggregates folded from zero, multipliers
            // multiplied) instead of its own aggregate, and segment j of group g
            // folds the combined transfers of groups 0 .. g-1 and then the
            // aggregates of its own group before it (about 2 sqrt(nseg) transfers
            // instead of j).  The extra publish round trip of the leaders pays off
            // from about two dozen segments on (measured: 28 one-chunk segments
            // 16.7 -> 14.9 us per call, 5 segments 34.1 -> 35.7 us).  The fixed
            // order makes the result independent of timing.  Flag bits: 1
            // aggregate, 2 combined transfer, 4 done reading.
            int G = P.nseg;
            if (P.nseg >= 24) {
                G = 1;
                while (G * G < P.nseg) ++G;
            }
            const int grp = seg / G, gfirst = grp * G;
            const bool leader = !last && seg == gfirst + G - 1;
            auto leader_slot = [&](int gg) { return (size_t)unit * P.nseg + (size_t)(gg * G + G - 1); };
            // wave 0 waits until groups 0 .. ng-1 have their combined transfers and
            // segments first .. first+cnt-1 their aggregates (ng + cnt <= 64)
            auto wait_for = [&](int ng, int first, int cnt) {
                if (wave == 0) {
                    unsigned spins = 0;
                    for (;;) {
                        bool ok = true;
                        if (lane < ng) ok = (ld_flag<LOCAL>(flags, P.nseg, lane * G + G - 1) & 2u) != 0u;
                        else if (lane < ng + cnt) ok = (ld_flag<LOCAL>(flags, P.nseg, first + lane - ng) & 1u) != 0u;
                        if (__all(ok)) break;
                        if (++spins > (1u << 22)) {
                            if (lane == 0) atomicOr(P.err, 1u);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                __syncthreads();
            };
            // fold, from (s0, s1), the combined transfers of groups 0 .. ng-1 and
            // then the aggregates of segments first .. first+cnt-1, in that order;
            // m0, m1 collect the product of the multipliers
            auto fold = [&](float4v& s0, float4v& s1, float& m0, float& m1, int ng, int first, int cnt) {
                constexpr int FW = 8;  // transfers per round of loads
                const int n = ng + cnt;
                for (int t0 = 0; t0 < n; t0 += FW) {
                    float4v a0[FW], a1[FW];
                    float g0[FW], g1[FW];
    #pragma unroll
                    for (int b = 0; b < FW; ++b) {
                        const int t = min(t0 + b, n - 1);
                        const float* base = t < ng ? P.incl + leader_slot(t) * aggf
                                                   : P.agg + ((size_t)unit * P.nseg + first + t - ng) * aggf;
                        const __amdgpu_buffer_rsrc_t r = xrsrc(base, agg_bytes);
                        a0[b] = ld_x4<LOCAL>(r, off0);
                        a1[b] = ld_x4<LOCAL>(r, off1);
                        g0[b] = ld_x1<LOCAL>(r, st_bytes + 4u * ch0);
                        g1[b] = ld_x1<LOCAL>(r, st_bytes + 4u * (ch0 + 32));
                    }
    #pragma unroll
                    for (int b = 0; b < FW; ++b)
                        if (t0 + b < n) {
    #pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                s0[e] = fold_step(g0[b], s0[e], a0[b][e]);
                                s1[e] = fold_step(g1[b], s1[e], a1[b][e]);
                            }
                            m0 *= g0[b];
                            m1 *= g1[b];
                        }
                }
            };
            auto set_flag = [&](unsigned v) {
                wait_mem();
                __syncthreads();
                if (tid == 0) st_flag<LOCAL>(flags, P.nseg, seg, v);
            };
            if (!last && !leader) {
                // aggregate: local state and multiplier 2^G
                const __amdgpu_buffer_rsrc_t r = xrsrc(P.agg + slot * aggf, agg_bytes);
                st_x4(r, off0, l0);
                st_x4(r, off1, l1);
                if (tid < D / 4) st_x4(r, st_bytes + 16u * tid, *(const float4v*)(sG + 4 * tid));
                set_flag(need_in ? 1u : 5u);  // the first segment reads nothing
            }
            if (leader) {
                // combined transfer of this group: its earlier aggregates, then this
                // segment's own local state, folded from zero
                wait_for(0, gfirst, seg - gfirst);
                float4v c0v = {0.f, 0.f, 0.f, 0.f}, c1v = c0v;
                float m0 = 1.f, m1 = 1.f;
                fold(c0v, c1v, m0, m1, 0, gfirst, seg - gfirst);
                const float gm0 = sG[ch0], gm1 = sG[ch0 + 32];
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    c0v[e] = fold_step(gm0, c0v[e], l0[e]);
                    c1v[e] = fold_step(gm1, c1v[e], l1[e]);
                }
                m0 *= gm0;
                m1 *= gm1;
                const __amdgpu_buffer_rsrc_t r = xrsrc(P.incl + slot * aggf, agg_bytes);
                st_x4(r, off0, c0v);
                st_x4(r, off1, c1v);
                if ((tid & 15) == 0) {
                    st_x1(r, st_bytes + 4u * ch0, m0);
                    st_x1(r, st_bytes + 4u * (ch0 + 32), m1);
                }
                set_flag(2u);
            }
            if (need_in) {
                wait_for(grp, gfirst, seg - gfirst);
                float4v s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
                float m0 = 1.f, m1 = 1.f;
                fold(s0, s1, m0, m1, grp, gfirst, seg - gfirst);
                // S_in^T (hi, lo) for phase 3
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const _Float16 h0 = (_Float16)s0[e], h1 = (_Float16)s1[e];
                    sST[(cl0 + e) * SH + ch0] = h0;
                    if (kInLo) sSTL[(cl0 + e) * SH + ch0] = (_Float16)(s0[e] - (float)h0);
                    sST[(cl0 + e) * SH + ch0 + 32] = h1;
                    if (kInLo) sSTL[(cl0 + e) * SH + ch0 + 32] = (_Float16)(s1[e] - (float)h1);
                }
                if (!last) set_flag(leader ? 6u : 5u);
            }
        } else {
            // Look back: each segment publishes its aggregate, waits until
            // every earlier segment has published, starts from the latest
            // inclusive state and folds the aggregates after it in segment
            // order (each inclusive state is itself that left fold, so the
            // result does not depend on which one was found), then publishes
            // its own inclusive state.  Flag bits as above, 2 meaning an
            // inclusive state.
            if (seg > 0 && !last) {
                const __amdgpu_buffer_rsrc_t r = xrsrc(P.agg + slot * aggf, agg_bytes);
                st_x4(r, off0, l0);
                st_x4(r, off1, l1);
                if (tid < D / 4) st_x4(r, st_bytes + 16u * tid, *(const float4v*)(sG + 4 * tid));
                wait_mem();
                __syncthreads();
                if (tid == 0) st_flag<LOCAL>(flags, P.nseg, seg, 1u);  // aggregate
            }
            if (need_in) {
                // look back: wait until every earlier segment has published, then
                // start from the latest inclusive state
                if (wave == 0) {
                    unsigned spins = 0;
                    int k = -1;
                    for (;;) {
                        const int idx = seg - 1 - lane;
                        const unsigned f = (idx >= 0) ? ld_flag<LOCAL>(flags, P.nseg, idx) : 2u;
                        if (__all((f & 3u) != 0u)) {
                            const unsigned long long inc = __ballot(idx >= 0 && (f & 2u) != 0u);
                            // lowest lane with an inclusive state = latest segment
                            // (segment 0 always publishes one, so inc != 0)
                            k = inc ? seg - 1 - (int)__builtin_ctzll(inc) : -1;
                            break;
                        }
                        if (++spins > (1u << 22)) {
                            if (lane == 0) atomicOr(P.err, 1u);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                    if (lane == 0) sMisc[1] = k;
                }
                __syncthreads();
                const int k = sMisc[1];
                // forward fold from the inclusive state of segment k
                float4v s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
                if (k >= 0) {
                    const __amdgpu_buffer_rsrc_t r = xrsrc(P.incl + ((size_t)unit * P.nseg + k) * aggf, st_bytes);
                    s0 = ld_x4<LOCAL>(r, off0);
                    s1 = ld_x4<LOCAL>(r, off1);
                }
                constexpr int FW = 8;  // aggregates per round of loads
                for (int sg0 = k + 1; sg0 < seg; sg0 += FW) {
                    // issue the loads of up to FW aggregates, then fold them in order
                    float4v a0[FW], a1[FW];
                    float g0[FW], g1[FW];
    #pragma unroll
                    for (int b = 0; b < FW; ++b) {
                        const int sg = min(sg0 + b, seg - 1);
                        const __amdgpu_buffer_rsrc_t r = xrsrc(P.agg + ((size_t)unit * P.nseg + sg) * aggf, agg_bytes);
                        a0[b] = ld_x4<LOCAL>(r, off0);
                        a1[b] = ld_x4<LOCAL>(r, off1);
                        g0[b] = ld_x1<LOCAL>(r, st_bytes + 4u * ch0);
                        g1[b] = ld_x1<LOCAL>(r, st_bytes + 4u * (ch0 + 32));
                    }
    #pragma unroll
                    for (int b = 0; b < FW; ++b)
                        if (sg0 + b < seg) {
    #pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                s0[e] = fold_step(g0[b], s0[e], a0[b][e]);
                                s1[e] = fold_step(g1[b], s1[e], a1[b][e]);
                            }
                        }
                }
                // S_in^T (hi, lo) for phase 3; inclusive state for successors
    #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const _Float16 h0 = (_Float16)s0[e], h1 = (_Float16)s1[e];
                    sST[(cl0 + e) * SH + ch0] = h0;
                    if (kInLo) sSTL[(cl0 + e) * SH + ch0] = (_Float16)(s0[e] - (float)h0);
                    sST[(cl0 + e) * SH + ch0 + 32] = h1;
                    if (kInLo) sSTL[(cl0 + e) * SH + ch0 + 32] = (_Float16)(s1[e] - (float)h1);
                }
                if (!last) {
                    const float gm0 = sG[ch0], gm1 = sG[ch0 + 32];
                    float4v i0, i1;
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        i0[e] = fold_step(gm0, s0[e], l0[e]);
                        i1[e] = fold_step(gm1, s1[e], l1[e]);
                    }
                    const __amdgpu_buffer_rsrc_t r = xrsrc(P.incl + slot * aggf, st_bytes);
                    st_x4(r, off0, i0);
                    st_x4(r, off1, i1);
                }
            } else {
                // first segment: its local state is the inclusive state
                const __amdgpu_buffer_rsrc_t r = xrsrc(P.incl + slot * aggf, st_bytes);
                st_x4(r, off0, l0);
                st_x4(r, off1, l1);
            }
            if (!last) {
                wait_mem();
                __syncthreads();
                if (tid == 0) st_flag<LOCAL>(flags, P.nseg, seg, seg > 0 ? 7u : 6u);  // inclusive, done
            }
        }
    }
    __syncthreads();

    // ================= phase 3: incoming state, epilogue, stores =================
    _Float16* sOut = (_Float16*)(lds + L_OUT);
    if (need_in) {
        // exchange the query-operand halves through the staging area
#pragma unroll
        for (int cc = 0; cc < NCHK; ++cc)
            if (cc < nch) *(half8*)(sOut + (cc * C + tl) * SH + c0) = qkeep[cc];
        __syncthreads();
    }
#pragma unroll
    for (int cc = 0; cc < NCHK; ++cc) {
        if (cc >= nch) break;
        float4v o0 = okeep[cc][0], o1 = okeep[cc][1];
        if (need_in) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int k0 = 32 * kb + 8 * g;
                const half8 qf = *(const half8*)(sOut + (cc * C + tl) * SH + k0);
                const half8 h0 = *(const half8*)(sST + (32 * h + l16) * SH + k0);
                const half8 h1 = *(const half8*)(sST + (32 * h + 16 + l16) * SH + k0);
                o0 = mma(h0, qf, o0);
                o1 = mma(h1, qf, o1);
                if (kInLo) {
                    const half8 l0 = *(const half8*)(sSTL + (32 * h + l16) * SH + k0);
                    const half8 l1 = *(const half8*)(sSTL + (32 * h + 16 + l16) * SH + k0);
                    o0 = mma(l0, qf, o0);
                    o1 = mma(l1, qf, o1);
                }
            }
        }
        okeep[cc][0] = o0 * P.scale;
        okeep[cc][1] = o1 * P.scale;
        if (gated) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ss += okeep[cc][0][e] * okeep[cc][0][e] + okeep[cc][1][e] * okeep[cc][1][e];
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            if (g == 0) sSS[(cc * 2 + h) * C + tl] = ss;
        }
    }
    if (gated) __syncthreads();  // sums of squares of both value halves
    float wv[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wv[m][e] = (gated && P.w) ? P.w[32 * h + 16 * m + 4 * g + e] : 1.f;
    // epilogue and stores straight from the output fragments: 8 bytes per lane
    // and value block (the two halves' stores of a row meet in the L2)
#pragma unroll
    for (int cc = 0; cc < NCHK; ++cc) {
        if (cc >= nch) break;
        float inv = 1.f;
        if (gated) {
            const float ss = sSS[(cc * 2) * C + tl] + sSS[(cc * 2 + 1) * C + tl];
            inv = rsq_fast(ss * (1.0f / D) + P.eps);
        }
        const int t = sRows[cc * C + tl];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            half4 hv;
            if (gated) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hv[e] = (_Float16)(silu((float)rreg[cc][m][e]) * wv[m][e] * okeep[cc][m][e] * inv);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = (_Float16)okeep[cc][m][e];
            }
            if (t >= 0) *(half4*)((_Float16*)P.out + (size_t)t * D + 32 * h + 16 * m + 4 * g) = hv;
        }
    }

    // The scan's last segment leaves its flags zero for the next call.  Every
    // earlier segment sets flag bit 4 only after its look-back and folds have
    // read all they need, so once every flag has it the exchange is over; each
    // lane then clears the one flag it read (the clear is ordered after the
    // store it saw).  This runs after the outputs, where the other segments
    // have long finished.
    if (P.nseg > 1 && seg == P.nseg - 1 && wave == 0) {
        unsigned* flags = P.flags + (size_t)unit * P.nseg;
        const bool mine = lane < seg;  // segments 0 .. nseg-2 (at most 64)
        unsigned spins = 0;
        for (;;) {
            const unsigned f = mine ? ld_flag<LOCAL>(flags, P.nseg, lane) : 4u;
            if (__all((f & 4u) != 0u)) break;
            if (++spins > (1u << 22)) {
                if (lane == 0) atomicOr(P.err, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (mine) st_flag<LOCAL>(flags, P.nseg, lane, 0u);
    }
}

// Zero-fills the single-pass workspace header and flags.
__global__ __launch_bounds__(256) void gla_onepass_init(unsigned* words, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        words[i] = 0u;
}

}  // namespace onepass

int launch_onepass(const Params& P, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    const dim3 grid(P.xcd_local ? 8 * P.xcd_tasks : P.B * P.NH * P.nseg);
    const bool proj = (P.ghp != nullptr);
    // one-chunk segments take an instance with a single chunk's registers and
    // a straight-line body (a small code footprint for the cold instruction
    // cache of workgroups that run it once)
    void (*kern)(Params);
    if (P.seg_chunks == 1)
        kern = P.xcd_local ? (proj ? onepass::gla_onepass_kernel<true, true, 1>
                                   : onepass::gla_onepass_kernel<true, false, 1>)
                           : (proj ? onepass::gla_onepass_kernel<false, true, 1>
                                   : onepass::gla_onepass_kernel<false, false, 1>);
    else
        kern = P.xcd_local ? (proj ? onepass::gla_onepass_kernel<true, true, onepass::NCH>
                                   : onepass::gla_onepass_kernel<true, false, onepass::NCH>)
                           : (proj ? onepass::gla_onepass_kernel<false, true, onepass::NCH>
                                   : onepass::gla_onepass_kernel<false, false, onepass::NCH>);
    hipLaunchKernelGGL(kern, grid, dim3(onepass::NT), 0, st, P);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

int launch_workspace_init(void* ws, size_t bytes, void* stream)
{
    const size_t n = bytes / 4;
    if (n == 0) return GLA_OK;
    unsigned blocks = (unsigned)((n + 255) / 256);
    if (blocks > 1024u) blocks = 1024u;
    hipLaunchKernelGGL(onepass::gla_onepass_init, dim3(blocks), dim3(256), 0,
                       (hipStream_t)stream, (unsigned*)ws, n);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

}  // namespace gla
