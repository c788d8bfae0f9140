// gla_kernel.hip -- launch entry points of the generic chunkwise forward
// (kernels in gla_chunk.h, instantiated per storage type and head-size shape
// in the gla_chunk_*.hip units) and the segment fold used by the d = 128
// three passes.
#include "gla_chunk.h"

namespace gla {

// Instantiation units (gla_chunk_f16.hip, gla_chunk_f32.hip,
// gla_chunk_f16_mixed.hip, gla_chunk_f32_mixed.hip).
int launch_chunk_f16(const Params& P, int d, int chunk, hipStream_t st);
int launch_chunk_f32(const Params& P, int d, int chunk, hipStream_t st);
int launch_chunk_f16_mixed(const Params& P, int dk, int dv, hipStream_t st);
int launch_chunk_f32_mixed(const Params& P, int dk, int dv, hipStream_t st);

int launch_fold(const Params& P, int d, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    const unsigned units = (unsigned)(P.B * P.NH);
    switch (d) {
    case 64:
        hipLaunchKernelGGL((gla_fold_kernel<64, 64>), dim3(units * ((64 * 64 + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, st, P);
        break;
    case 128:
        hipLaunchKernelGGL((gla_fold_kernel<128, 128>),
                           dim3(units * ((128 * 128 + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, P);
        break;
    default: return GLA_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_EHIP;
}

int launch_fwd(const Params& P, int dtype, int dk, int dv, int chunk, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    // the d = 128 kernels address inputs with 32-bit buffer offsets: fp32
    // gate logits (512 bytes per row) below 2^31 bytes
    const long long rows = (long long)P.B * P.L * P.NH;
    if (dtype == GLA_F16 && dk == 128 && dv == 128 && chunk == 64 && rows < (1ll << 22))
        return launch_wide(P, stream);
    if (dk != dv) {
        // d_v != d_k: 64-token chunks only
        if (chunk != 64) return GLA_EUNSUPPORTED;
        if (dtype == GLA_F16) return launch_chunk_f16_mixed(P, dk, dv, st);
        if (dtype == GLA_F32) return launch_chunk_f32_mixed(P, dk, dv, st);
        return GLA_EUNSUPPORTED;
    }
    if (dtype == GLA_F16) return launch_chunk_f16(P, dk, chunk, st);
    if (dtype == GLA_F32) return launch_chunk_f32(P, dk, chunk, st);
    return GLA_EUNSUPPORTED;
}

}  // namespace gla
