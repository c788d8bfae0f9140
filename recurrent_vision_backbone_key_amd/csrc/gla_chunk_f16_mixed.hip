// gla_chunk_f16_mixed.hip -- instantiations of the generic chunkwise
// forward (gla_chunk.h) for binary16 storage, d_k != d_v (64-token chunks).  Split from the
// other instantiations so the units compile in parallel.
#include "gla_chunk.h"

namespace gla {

namespace {

template <int DK, int DV>
int run_pair(const Params& P, hipStream_t st)
{
    if constexpr (DK == DV) {
        return GLA_EUNSUPPORTED;  // the square shapes live in gla_chunk_f16.hip
    } else {
        return run<_Float16, DK, DV, 64>(P, st);
    }
}

template <int DK>
int run_mixed(const Params& P, int dv, hipStream_t st)
{
    switch (dv) {
    case 16: return run_pair<DK, 16>(P, st);
    case 32: return run_pair<DK, 32>(P, st);
    case 64: return run_pair<DK, 64>(P, st);
    case 128: return run_pair<DK, 128>(P, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace

int launch_chunk_f16_mixed(const Params& P, int dk, int dv, hipStream_t st)
{
    if (dk == dv) return GLA_EUNSUPPORTED;
    switch (dk) {
    case 16: return run_mixed<16>(P, dv, st);
    case 32: return run_mixed<32>(P, dv, st);
    case 64: return run_mixed<64>(P, dv, st);
    case 128: return run_mixed<128>(P, dv, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace gla
