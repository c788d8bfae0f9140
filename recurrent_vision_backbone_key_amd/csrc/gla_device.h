// gla_device.h -- device helpers shared by the chunkwise GLA kernels (gfx950).
#ifndef GLA_DEVICE_H
#define GLA_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gla_launch.h"

namespace gla {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 16;            // tokens per sub-chunk (MFMA tile edge)
constexpr float kLog2e = 1.4426950408889634f;
// Per-token log-decay floor, natural-log units (gamma >= e^-40 per token).
constexpr float kMinLog2Decay = -40.0f * kLog2e;

// Operand-format traits: the widest safe decay span (log2 units) of the
// factorised diagonal block and the largest operand magnitude allowed there.
template <typename T> struct Fmt;
template <> struct Fmt<_Float16> {
    static constexpr float kSpan = 8.0f;          // key factor <= 2^8
    static constexpr float kMaxOperand = 30000.0f;
};
template <> struct Fmt<float> {
    static constexpr float kSpan = 60.0f;
    static constexpr float kMaxOperand = 1e30f;
};

// MFMA shape for a contraction of length K: K-step, elements per lane per
// K-step (lane group g = lane/16 holds k = KPL*g .. KPL*g+KPL-1), fragment type.
//   binary16, K >= 32: v_mfma_f32_16x16x32_f16  (KSTEP 32, KPL 8)
//   binary16, K == 16: v_mfma_f32_16x16x16_f16  (KSTEP 16, KPL 4)
//   binary32:          v_mfma_f32_16x16x4_f32   (KSTEP 4,  KPL 1)
template <typename T, int K> struct KS;
template <int K> struct KS<_Float16, K> {
    static constexpr int KSTEP = K >= 32 ? 32 : 16, KPL = KSTEP / 4;
    typedef typename std::conditional<KPL == 8, half8, half4>::type frag;
};
template <int K> struct KS<float, K> {
    static constexpr int KSTEP = 4, KPL = 1;
    typedef float frag;
};

__device__ __forceinline__ float4v mma(half8 a, half8 b, float4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mma(half4 a, half4 b, float4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mma(float a, float b, float4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Buffer resource over `bytes` bytes at `base` (raw addressing): a load at an
// offset past the record count returns zeros, which reads the rows past the
// end of a scan without a branch or a select.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(const void* base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// Offset past every record (the tensors it is used on stay below 2^31 bytes).
constexpr unsigned kPastEnd = 0x80000000u;
// Cache-policy operand of buffer instructions: non-temporal (streaming).
constexpr int kNonTemporal = 2;
__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Four binary16 values through the gfx950 LDS transpose read: within each
// group of 16 lanes, lane j supplies the address of 4 consecutive elements
// and receives element (j mod 4) of the reads of lanes 4e + j/4, e = 0..3.
// With lane j pointing at row row0 + j/4, columns col0 + 4 (j mod 4) .. +3 of
// a row-major tile, lane j receives rows row0 .. row0 + 3 of column col0 + j.
// Every lane of the wavefront must execute it.
__device__ __forceinline__ half4 ld_tr(const _Float16* p)
{
    const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p);
    return __builtin_bit_cast(half4, x);
}
// Address lane (l16) supplies so that it receives rows row0 .. row0 + 3 of
// column col0 + l16 of a row-major tile with row stride STRIDE elements.
template <int STRIDE>
__device__ __forceinline__ const _Float16* tr_addr(const _Float16* base, int row0, int col0, int l16)
{
    return base + (row0 + (l16 >> 2)) * STRIDE + col0 + 4 * (l16 & 3);
}
// MFMA fragment of a row-major [token][col] tile contracted over tokens: lane
// (g, l16) receives rows row0 + 0..7 of column col0 + l16, where row0 is the
// first of 8 consecutive tokens of its lane group.
template <int STRIDE>
__device__ __forceinline__ half8 tr_frag_s(const _Float16* base, int row0, int col0, int l16)
{
    const _Float16* p = tr_addr<STRIDE>(base, row0, col0, l16);
    const half4 a = ld_tr(p), b = ld_tr(p + 4 * STRIDE);
    return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-token log2-decay a = log2(sigmoid(z)) / tau, floored at kMinLog2Decay,
// from log2 sigmoid(z) = -log2(1 + 2^{-z log2 e}) with the hardware 2^x and
// log2 (five VALU operations).  For z < -88.7 the power overflows to +inf,
// giving -inf and then the floor; z = +inf gives 0; NaN propagates (the
// floor's comparison is false for NaN).  The result's error is about one ulp
// of log2(1 + 2^{-z log2 e}), as for the two-sided softplus form.
__device__ __forceinline__ float log2_decay(float z, float inv_tau)
{
    const float a = __builtin_amdgcn_logf(1.0f + exp2_fast(z * -kLog2e)) * -inv_tau;
    return (a < kMinLog2Decay) ? kMinLog2Decay : a;
}

// x from the lane N places lower in the same 16-lane row (0 for the first N).
template <int N>
__device__ __forceinline__ float row_shr(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), 0x110 | N, 0xF, 0xF, true));
}

// Inclusive prefix sums along the 16 lanes of each row for M independent
// values, stage by stage (Hillis-Steele): the M shifted adds of a stage are
// independent, so the DPP hazards of one value overlap the others.
template <int M>
__device__ __forceinline__ void row_scan_n(float (&x)[M])
{
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] += row_shr<1>(x[i]);
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] += row_shr<2>(x[i]);
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] += row_shr<4>(x[i]);
#pragma unroll
    for (int i = 0; i < M; ++i) x[i] += row_shr<8>(x[i]);
}

// Hardware reciprocal and reciprocal square root (about 1 ulp).
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsq_fast(float x) { return __builtin_amdgcn_rsqf(x); }

// SiLU(x) = x sigmoid(x) = x / (1 + e^{-x}).
__device__ __forceinline__ float silu(float x) { return x * rcp_fast(1.0f + exp2_fast(-x * kLog2e)); }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// x rounded to binary16 and back: the high part of a hi + lo split.
__device__ __forceinline__ float lo_part_base(float x) { return (float)(_Float16)x; }
// The binary16 low part x - fl16(x) of a hi + lo split.
__device__ __forceinline__ _Float16 lo_part(float x) { return (_Float16)(x - (float)(_Float16)x); }

// Coalesced 16-byte-per-thread row loader for a [ROWS][ROWBYTES] tile whose
// rows sit at scattered global row indices (the scan-order remap).
template <int ROWS, int ROWBYTES, int NT = 256>
struct RowTile {
    static constexpr int PIECES = ROWBYTES / 16;
    static constexpr int PASSES = (ROWS * PIECES + NT - 1) / NT;
    u32x4 reg[PASSES];

    __device__ __forceinline__ void load(const char* base, const int* tok, int tid)
    {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int idx = tid + p * NT;
            const int row = idx / PIECES, piece = idx % PIECES;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (row < ROWS) {
                const int t = tok[row];
                if (t >= 0)
                    val = *(const u32x4*)(base + (size_t)t * ROWBYTES + piece * 16);
            }
            reg[p] = val;
        }
    }
    // Row-major store into LDS with a padded row stride (bytes).
    __device__ __forceinline__ void store_rows(char* lds, int stride, int tid) const
    {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int idx = tid + p * NT;
            const int row = idx / PIECES, piece = idx % PIECES;
            if (row < ROWS)
                *(u32x4*)(lds + row * stride + piece * 16) = reg[p];
        }
    }
    // Transposed store: element e of row `row` goes to ldsT[col][row].
    template <typename T>
    __device__ __forceinline__ void store_transposed(T* ldsT, int strideT, int tid) const
    {
        constexpr int EPP = 16 / sizeof(T);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int idx = tid + p * NT;
            const int row = idx / PIECES, piece = idx % PIECES;
            if (row < ROWS) {
                const T* vals = (const T*)&reg[p];
#pragma unroll
                for (int e = 0; e < EPP; ++e)
                    ldsT[(piece * EPP + e) * strideT + row] = vals[e];
            }
        }
    }
};

// Scan position -> global row index ((b*L + t)*NH + h), or -1 past the end.
// The four orders of paper Sec. 2.1: raster (L2R), reversed raster (R2L),
// column-major (T2B), reversed column-major (B2T); t = h_grid*W + w_grid.
__device__ __forceinline__ int scan_row(const Params& P, int unit, int pos)
{
    if (pos >= P.L) return -1;
    const int pp = (P.dir & 1) ? (P.L - 1 - pos) : pos;
    int t = pp;
    if (P.dir >= 2) {
        const int wcol = pp / P.H;
        const int hrow = pp - wcol * P.H;
        t = hrow * P.W + wcol;
    }
    const int b = unit / P.NH, h = unit - (unit / P.NH) * P.NH;
    return (b * P.L + t) * P.NH + h;
}

template <typename T, int N>
__device__ __forceinline__ void ld_f(const T* p, float (&x)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = to_f(p[i]);
}

template <int N>
__device__ __forceinline__ void ld_f32(const float* p, float (&x)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
}

__device__ __forceinline__ half8 pack(const float (&x)[8])
{
    half8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)x[i];
    return r;
}
__device__ __forceinline__ half4 pack(const float (&x)[4])
{
    half4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (_Float16)x[i];
    return r;
}
__device__ __forceinline__ float pack(const float (&x)[1]) { return x[0]; }

// KPL consecutive elements from LDS as an MFMA fragment.
template <typename T, int KPL> struct Frag;
template <> struct Frag<_Float16, 8> {
    static __device__ __forceinline__ half8 ld(const _Float16* p) { return *(const half8*)p; }
};
template <> struct Frag<_Float16, 4> {
    static __device__ __forceinline__ half4 ld(const _Float16* p) { return *(const half4*)p; }
};
template <> struct Frag<float, 1> {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
};

}  // namespace gla

#endif
