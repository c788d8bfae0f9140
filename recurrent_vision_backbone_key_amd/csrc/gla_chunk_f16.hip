// gla_chunk_f16.hip -- instantiations of the generic chunkwise
// forward (gla_chunk.h) for binary16 storage, d_k = d_v (every built chunk).  Split from the
// other instantiations so the units compile in parallel.
#include "gla_chunk.h"

namespace gla {

namespace {

template <int D>
int run_square(const Params& P, int chunk, hipStream_t st)
{
    switch (chunk) {
    case 16: return run<_Float16, D, D, 16>(P, st);
    case 32: return run<_Float16, D, D, 32>(P, st);
    case 64: return run<_Float16, D, D, 64>(P, st);
    case 128: return run<_Float16, D, D, 128>(P, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace

int launch_chunk_f16(const Params& P, int d, int chunk, hipStream_t st)
{
    switch (d) {
    case 16: return run_square<16>(P, chunk, st);
    case 32: return run_square<32>(P, chunk, st);
    case 64: return run_square<64>(P, chunk, st);
    case 128: return run_square<128>(P, chunk, st);
    default: return GLA_EUNSUPPORTED;
    }
}

}  // namespace gla
