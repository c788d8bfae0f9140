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
// in binary32.  hp comes from the forward's rank kernel.  One workgroup of
// eight wavefronts then takes a block of 64 tokens through all five products:
// it reads the block's dz once, in 64-column chunks staged in LDS with the
// matching rows of W2, for dhp (four waves) and the block's partial dW2 and
// db (the other four); keeps dhp in LDS; and reads the block's x once, in
// 64-column chunks with the matching columns of W1, for dx and the block's
// partial dW1.  The loads of the next chunk are issued before the current
// chunk's products and written to the other of two LDS buffers after them.
// Every product runs on v_mfma_f32_16x16x4_f32 (lane (g, l16) supplies one k
// of its A row and B column per step; sums over a chunk in two or four
// interleaved chains).  The partial sums of the token blocks are then added
// in block order by one reduction launch, so every result is the same for
// equal inputs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gla.h"
#include "gla_device.h"
#include "gla_launch.h"

namespace gla {
namespace pbwd {

constexpr int TB = kProjBwdSplit;  // tokens per workgroup (and per partial sum)
constexpr int NT = 512;            // threads: eight wavefronts
constexpr int CC = 64;             // columns per staged chunk (of dz and of x)
constexpr int RMAX = 64;           // largest rank
constexpr int SZ = CC + 4;         // binary32 row stride of the dz chunk
constexpr int SR = RMAX + 4;       // binary32 row stride of hp, dhp and the W2 chunk
constexpr int KB = 8;              // MFMA steps whose operands are read from LDS in one batch
static_assert(TB == 64, "one 16-token tile per wavefront");

template <typename T> struct XS { static constexpr int S = CC + (sizeof(T) == 2 ? 8 : 4); };

// LDS: hp and dhp of the block [TB][SR] (binary32), then one region that the
// dz chunks use first (two buffers of the dz chunk [TB][SZ] and the W2 chunk
// [CC][SR], binary32) and the x chunks after them (two buffers of the x chunk
// [TB][XS] and the W1 chunk [RMAX][XS], storage type).
template <typename T> struct Lay {
    static constexpr int HP = 0;
    static constexpr int DHP = HP + TB * SR * 4;
    static constexpr int U = DHP + TB * SR * 4;
    static constexpr int ZBUF = TB * SZ * 4 + CC * SR * 4;                    // one dz + W2 buffer
    static constexpr int XBUF = (TB + RMAX) * XS<T>::S * (int)sizeof(T);      // one x + W1 buffer
    static constexpr int TOTAL = U + 2 * (ZBUF > XBUF ? ZBUF : XBUF);
};

// Chunk staging in registers (the next chunk's loads are issued before the
// current chunk's products and stored to the other LDS buffer after them):
// thread i holds dz pieces i and i + 512 (four values each), W2 entries
// i + 512 u, and x and W1 pieces of eight values.  Every load goes through a buffer resource bounded by its
// array, and a masked element takes an offset past every record (it reads
// zero), so the loads carry no branches and the compiler waits for exactly
// the ones a chunk needs.
struct ZStage {
    u32x4 z[2];
    float w[8];
};
template <typename T> struct XStage {
    u32x4 x[sizeof(T) / 2], w[sizeof(T) / 2];
};

__device__ __forceinline__ unsigned boff(bool ok, long long elem, unsigned es)
{
    return ok ? (unsigned)(elem * es) : kPastEnd;
}

template <bool VEC, int RP>
__device__ __forceinline__ void load_z(ZStage& S, __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rw, int tid,
                                       int t0, int tokens, int nout, int oc, int R)
{
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NT * u;  // 1024 pieces of four columns
        const int r = i >> 4, c4 = 4 * (i & 15);
        const long long e0 = (long long)(t0 + r) * nout + oc + c4;
        const bool rok = t0 + r < tokens;
        if (VEC) {
            S.z[u] = ld_b128(rz, boff(rok && oc + c4 < nout, e0, 4u));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S.z[u][e] = (unsigned)__builtin_amdgcn_raw_buffer_load_b32(
                    rz, (int)boff(rok && oc + c4 + e < nout, e0 + e, 4u), 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < (CC * RP + NT - 1) / NT; ++u) {
        const int i = tid + NT * u;  // CC rows x RP ranks
        const int k = i / RP, j = i - k * RP;
        S.w[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            rw, (int)boff(oc + k < nout && j < R, (long long)(oc + k) * R + j, 4u), 0, 0));
    }
}

template <int RP>
__device__ __forceinline__ void store_z(const ZStage& S, float* sDZ, float* sW2, int tid)
{
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NT * u;
        *(u32x4*)(sDZ + (i >> 4) * SZ + 4 * (i & 15)) = S.z[u];
    }
#pragma unroll
    for (int u = 0; u < (CC * RP + NT - 1) / NT; ++u) {
        const int i = tid + NT * u;
        const int k = i / RP, j = i - k * RP;
        sW2[k * SR + j] = S.w[u];
    }
}

template <typename T>
__device__ __forceinline__ void load_x(XStage<T>& S, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw, int tid,
                                       int t0, int tokens, int DM, int dc, int R)
{
    constexpr unsigned es = sizeof(T);
    const int r = tid >> 3, c8 = 8 * (tid & 7);  // 512 pieces of eight columns (x), RMAX ranks (W1)
    const bool cok = dc + c8 < DM;
    const unsigned ox = boff(t0 + r < tokens && cok, (long long)(t0 + r) * DM + dc + c8, es);
    const unsigned ow = boff(r < R && cok, (long long)r * DM + dc + c8, es);
#pragma unroll
    for (int h = 0; h < (int)(es / 2); ++h) {
        S.x[h] = ld_b128(rx, ox == kPastEnd ? kPastEnd : ox + 16u * h);
        S.w[h] = ld_b128(rw, ow == kPastEnd ? kPastEnd : ow + 16u * h);
    }
}

template <typename T>
__device__ __forceinline__ void store_x(const XStage<T>& S, T* sX, T* sW1, int tid)
{
    constexpr int SX = XS<T>::S;
    const int r = tid >> 3, c8 = 8 * (tid & 7);
#pragma unroll
    for (int h = 0; h < (int)(sizeof(T) / 2); ++h) {
        *(u32x4*)(sX + r * SX + c8 + h * 16 / (int)sizeof(T)) = S.x[h];
        *(u32x4*)(sW1 + r * SX + c8 + h * 16 / (int)sizeof(T)) = S.w[h];
    }
}

// Sum of an output element over its accumulation chains, in chain order.
template <int NCH, int RT>
__device__ __forceinline__ float chain_sum(const float4v (&acc)[NCH][RT], int n, int e)
{
    float v = acc[0][n][e];
#pragma unroll
    for (int h = 1; h < NCH; ++h) v += acc[h][n][e];
    return v;
}
template <int NCH>
__device__ __forceinline__ float chain_sum1(const float4v (&acc)[NCH], int e)
{
    float v = acc[0][e];
#pragma unroll
    for (int h = 1; h < NCH; ++h) v += acc[h][e];
    return v;
}

// RT = ceil(rank / 16) rank tiles (a compile-time count, so every product
// loop is straight-line code whose LDS reads are issued in batches of KB
// steps ahead of their MFMAs); VEC: nout is a multiple of 4 (dz rows load as
// 16-byte pieces)
template <typename T, int RT, bool VEC>
__global__ __launch_bounds__(NT) void gla_pbwd_fused_kernel(const T* __restrict__ x, const T* __restrict__ w1,
                                                          const float* __restrict__ w2,
                                                          const float* __restrict__ hp,
                                                          const float* __restrict__ dz, T* __restrict__ dx,
                                                          float* __restrict__ p1, float* __restrict__ p2,
                                                          float* __restrict__ pb, int tokens, int DM,
                                                          int nout, int R)
{
    typedef Lay<T> LY;
    constexpr int SX = XS<T>::S;
    constexpr int BUF = LY::ZBUF > LY::XBUF ? LY::ZBUF : LY::XBUF;
    __shared__ __attribute__((aligned(16))) char lds[LY::TOTAL];
    float* sHP = (float*)(lds + LY::HP);
    float* sDHP = (float*)(lds + LY::DHP);
    auto zbuf = [&](int b) { return (float*)(lds + LY::U + b * BUF); };            // dz chunk, then W2 chunk
    auto w2buf = [&](int b) { return (float*)(lds + LY::U + b * BUF) + TB * SZ; };
    auto xbuf = [&](int b) { return (T*)(lds + LY::U + b * BUF); };                // x chunk, then W1 chunk
    auto w1buf = [&](int b) { return (T*)(lds + LY::U + b * BUF) + TB * SX; };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int w = wave & 3;           // tile of this wave
    const bool second = wave >= 4;    // waves 4-7: the sums over tokens
    const int blk = blockIdx.x;
    const int t0 = blk * TB;
    constexpr int RP = 16 * RT;
    // independent accumulation chains per output tile: with one rank tile,
    // four (a dependent 16x16x4 step waits for the one before it)
    constexpr int NCH = RT == 1 ? 4 : 2;
    const long long T0 = t0;
    const __amdgpu_buffer_rsrc_t rz = xrsrc(dz, (unsigned)((long long)tokens * nout * 4));
    const __amdgpu_buffer_rsrc_t rw2 = xrsrc(w2, (unsigned)((long long)nout * R * 4));
    const __amdgpu_buffer_rsrc_t rx = xrsrc(x, (unsigned)((long long)tokens * DM * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rw1 = xrsrc(w1, (unsigned)((long long)R * DM * sizeof(T)));
    const int ncz = (nout + CC - 1) / CC, ncx = (DM + CC - 1) / CC;

    // first chunks of both passes (the x chunk's registers are consumed after
    // the dz chunks) and hp of the block (rows past the last token read zero)
    ZStage zs;
    XStage<T> xs;
    load_z<VEC, RP>(zs, rz, rw2, tid, t0, tokens, nout, 0, R);
    load_x<T>(xs, rx, rw1, tid, t0, tokens, DM, 0, R);
    for (int i = tid; i < TB * RP; i += NT) {
        const int r = i / RP, j = i - r * RP;
        sHP[r * SR + j] = (t0 + r < tokens) ? hp[(T0 + r) * RP + j] : 0.f;
    }
    store_z<RP>(zs, zbuf(0), w2buf(0), tid);
    __syncthreads();

    // ---- dz chunks.  Waves 0-3: dhp of tokens 16w..16w+15 (every rank
    //      tile).  Waves 4-7: the block's dW2 rows and db entries of chunk
    //      columns 16w..16w+15.
    float4v acc_h[NCH][RT];
#pragma unroll
    for (int h = 0; h < NCH; ++h)
#pragma unroll
        for (int n = 0; n < RT; ++n) acc_h[h][n] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < ncz; ++c) {
        const int oc = CC * c;
        const bool nxt = c + 1 < ncz;
        if (nxt) load_z<VEC, RP>(zs, rz, rw2, tid, t0, tokens, nout, oc + CC, R);
        const float* sDZ = zbuf(c & 1);
        const float* sW2 = w2buf(c & 1);
        float4v acc_w[NCH][RT], acc_b[NCH];
        if (!second) {
            // dhp[16w + i][16n + j] += sum_k dz[16w + i][oc + k] w2[oc + k][16n + j]
#pragma unroll
            for (int s0 = 0; s0 < CC / 4; s0 += KB) {
                float av[KB], bv[KB][RT];
#pragma unroll
                for (int s = 0; s < KB; ++s) {
                    const int k = 4 * (s0 + s) + g;
                    av[s] = sDZ[(16 * w + l16) * SZ + k];
#pragma unroll
                    for (int n = 0; n < RT; ++n) bv[s][n] = sW2[k * SR + 16 * n + l16];
                }
#pragma unroll
                for (int s = 0; s < KB; ++s)
#pragma unroll
                    for (int n = 0; n < RT; ++n) acc_h[s % NCH][n] = mma(av[s], bv[s][n], acc_h[s % NCH][n]);
            }
        } else {
            // dW2 rows oc + 16w + i over the block's tokens: dz[t][col] hp[t][j];
            // db: the same against a column of ones
#pragma unroll
            for (int h = 0; h < NCH; ++h) {
                acc_b[h] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n = 0; n < RT; ++n) acc_w[h][n] = float4v{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int s0 = 0; s0 < TB / 4; s0 += KB) {
                float av[KB], bv[KB][RT];
#pragma unroll
                for (int s = 0; s < KB; ++s) {
                    const int t = 4 * (s0 + s) + g;
                    av[s] = sDZ[t * SZ + 16 * w + l16];
#pragma unroll
                    for (int n = 0; n < RT; ++n) bv[s][n] = sHP[t * SR + 16 * n + l16];
                }
#pragma unroll
                for (int s = 0; s < KB; ++s) {
#pragma unroll
                    for (int n = 0; n < RT; ++n) acc_w[s % NCH][n] = mma(av[s], bv[s][n], acc_w[s % NCH][n]);
                    acc_b[s % NCH] = mma(av[s], l16 == 0 ? 1.f : 0.f, acc_b[s % NCH]);
                }
            }
        }
        // the next chunk into the other buffer (its readers finished before
        // the last barrier), then this chunk's partial sums
        if (nxt) store_z<RP>(zs, zbuf((c + 1) & 1), w2buf((c + 1) & 1), tid);
        if (second) {
            float* dst2 = p2 + (long long)blk * nout * R;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = oc + 16 * w + 4 * g + e;
                if (col < nout) {
#pragma unroll
                    for (int n = 0; n < RT; ++n) {
                        const int j = 16 * n + l16;
                        if (j < R) dst2[(long long)col * R + j] = chain_sum<NCH>(acc_w, n, e);
                    }
                    if (l16 == 0) pb[(long long)blk * nout + col] = chain_sum1<NCH>(acc_b, e);
                }
            }
        }
        __syncthreads();
    }
    // dhp into LDS (lane holds dhp[16w + 4g + e][16n + l16]) and the first x
    // chunk into buffer 0 (every dz chunk's readers are done)
    if (!second) {
#pragma unroll
        for (int n = 0; n < RT; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sDHP[(16 * w + 4 * g + e) * SR + 16 * n + l16] = chain_sum<NCH>(acc_h, n, e);
    }
    store_x<T>(xs, xbuf(0), w1buf(0), tid);
    __syncthreads();

    // ---- x chunks.  Waves 0-3: dx, formed transposed (columns 16w..16w+15
    //      of the chunk for all 64 tokens: four consecutive columns per lane
    //      and store).  Waves 4-7: the block's dW1 entries of those columns.
    for (int c = 0; c < ncx; ++c) {
        const int dc = CC * c;
        const bool nxt = c + 1 < ncx;
        if (nxt) load_x<T>(xs, rx, rw1, tid, t0, tokens, DM, dc + CC, R);
        const T* sX = xbuf(c & 1);
        const T* sW1 = w1buf(c & 1);
        float4v acc_x[4], acc_1[NCH][RT];
        if (!second) {
            // dx^T[col][t] = sum_j w1[j][col] dhp[t][j]
#pragma unroll
            for (int b = 0; b < 4; ++b) acc_x[b] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < RP / 4; s0 += 4) {
                float av[4], bv[4][4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int j = 4 * (s0 + s) + g;
                    av[s] = (float)sW1[j * SX + 16 * w + l16];
#pragma unroll
                    for (int b = 0; b < 4; ++b) bv[s][b] = sDHP[(16 * b + l16) * SR + j];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc_x[b] = mma(av[s], bv[s][b], acc_x[b]);
            }
        } else {
            // dW1[j][col] over the block: sum_t dhp[t][j] x[t][col]
#pragma unroll
            for (int h = 0; h < NCH; ++h)
#pragma unroll
                for (int n = 0; n < RT; ++n) acc_1[h][n] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < TB / 4; s0 += KB) {
                float bx[KB], av[KB][RT];
#pragma unroll
                for (int s = 0; s < KB; ++s) {
                    const int t = 4 * (s0 + s) + g;
                    bx[s] = (float)sX[t * SX + 16 * w + l16];
#pragma unroll
                    for (int n = 0; n < RT; ++n) av[s][n] = sDHP[t * SR + 16 * n + l16];
                }
#pragma unroll
                for (int s = 0; s < KB; ++s)
#pragma unroll
                    for (int n = 0; n < RT; ++n) acc_1[s % NCH][n] = mma(av[s][n], bx[s], acc_1[s % NCH][n]);
            }
        }
        if (nxt) store_x<T>(xs, xbuf((c + 1) & 1), w1buf((c + 1) & 1), tid);
        if (!second) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            const int c4 = dc + 16 * w + 4 * g;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int t = t0 + 16 * b + l16;
                if (t < tokens && c4 < DM)
                    *(t4*)(dx + (long long)t * DM + c4) =
                        t4{(T)acc_x[b][0], (T)acc_x[b][1], (T)acc_x[b][2], (T)acc_x[b][3]};
            }
        } else {
            const int col = dc + 16 * w + l16;
            float* dst1 = p1 + (long long)blk * R * DM;
            if (col < DM) {
#pragma unroll
                for (int n = 0; n < RT; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 16 * n + 4 * g + e;
                        if (j < R) dst1[(long long)j * DM + col] = chain_sum<NCH>(acc_1, n, e);
                    }
            }
        }
        __syncthreads();
    }
}

// out_q[i] = sum over the nsplit partial sums part_q[s * count_q + i], in
// block order, for the three partial arrays q (dW1, dW2, db) in one launch:
// a workgroup takes 32 outputs of one array; thread (i, q8) adds the partials
// of the q8-th eighth of the blocks in order (sixteen loads in flight before
// their additions), then the eight partial sums are added in order.
struct ReduceArgs {
    const float* part[3];
    float* out[3];
    long long count[3];
    long long first_block[4];  // workgroups of array q: [first_block[q], first_block[q + 1])
};

constexpr int ROUT = 32;  // outputs per reduction workgroup

__global__ __launch_bounds__(256) void gla_pbwd_reduce_kernel(ReduceArgs A, int nsplit)
{
    __shared__ float qs[8][ROUT];
    const int o = threadIdx.x & (ROUT - 1), q8 = threadIdx.x / ROUT;
    const long long b = blockIdx.x;
    const int q = b < A.first_block[1] ? 0 : b < A.first_block[2] ? 1 : 2;
    const float* part = A.part[q];
    const long long count = A.count[q];
    const long long i = (b - A.first_block[q]) * ROUT + o;
    const int per = (nsplit + 7) / 8;
    const int z1 = min(nsplit, (q8 + 1) * per);
    float s = 0.f;
    if (i < count) {
        for (int z0 = q8 * per; z0 < z1; z0 += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = z0 + u < z1 ? part[(long long)(z0 + u) * count + i] : 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) s += v[u];
        }
    }
    qs[q8][o] = s;
    __syncthreads();
    if (q8 == 0 && i < count) {
        float t = qs[0][o];
#pragma unroll
        for (int k = 1; k < 8; ++k) t += qs[k][o];
        A.out[q][i] = t;
    }
}

template <typename T>
int run(const GateProj& G, int tokens, int nout, const float* dz, void* dx, float* dw1, float* dw2,
        float* db, const ProjBwdWs& W, hipStream_t st)
{
    const int R = G.rank, DM = G.d_model;
    const int ns = (tokens + TB - 1) / TB;
    // hp = x W1 ([tokens][16 ceil(rank / 16)], columns past the rank 0)
    const int rs = launch_gate_rank(G, std::is_same<T, float>::value ? GLA_F32 : GLA_F16, tokens, W.hp, st);
    if (rs != GLA_OK) return rs;
    void (*kern)(const T*, const T*, const float*, const float*, const float*, T*, float*, float*, float*, int,
                 int, int, int);
    const bool vec = (nout & 3) == 0;
    switch ((R + 15) / 16) {
    case 1: kern = vec ? gla_pbwd_fused_kernel<T, 1, true> : gla_pbwd_fused_kernel<T, 1, false>; break;
    case 2: kern = vec ? gla_pbwd_fused_kernel<T, 2, true> : gla_pbwd_fused_kernel<T, 2, false>; break;
    case 3: kern = vec ? gla_pbwd_fused_kernel<T, 3, true> : gla_pbwd_fused_kernel<T, 3, false>; break;
    default: kern = vec ? gla_pbwd_fused_kernel<T, 4, true> : gla_pbwd_fused_kernel<T, 4, false>; break;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)ns), dim3(NT), 0, st, (const T*)G.x, (const T*)G.w1, G.w2,
                       (const float*)W.hp, dz, (T*)dx, W.p1, W.p2, W.pb, tokens, DM, nout, R);
    ReduceArgs A;
    A.part[0] = W.p1;
    A.part[1] = W.p2;
    A.part[2] = W.pb;
    A.out[0] = dw1;
    A.out[1] = dw2;
    A.out[2] = db;
    A.count[0] = (long long)R * DM;
    A.count[1] = (long long)nout * R;
    A.count[2] = nout;
    A.first_block[0] = 0;
    for (int q = 0; q < 3; ++q) A.first_block[q + 1] = A.first_block[q] + (A.count[q] + ROUT - 1) / ROUT;
    hipLaunchKernelGGL(gla_pbwd_reduce_kernel, dim3((unsigned)A.first_block[3]), dim3(256), 0, st, A, ns);
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
