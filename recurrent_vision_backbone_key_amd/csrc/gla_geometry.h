// gla_geometry.h -- shared-memory footprint of one workgroup (host and device).
#ifndef GLA_GEOMETRY_H
#define GLA_GEOMETRY_H

namespace gla {

constexpr int kLdsLimit = 160 * 1024;  // LDS of one gfx950 compute unit

// Bytes of LDS used by the chunk kernel for storage size ts (2 or 4 bytes),
// head dims dk, dv and chunk c.  Row strides carry a 16-byte pad.
constexpr int lds_bytes(int ts, int dk, int dv, int c)
{
    const int pad = 16 / ts;
    const int nsub = c / 16;
    const int lpc = dk >= 64 ? 1 : 64 / dk;
    return c * (dk + pad) * ts * 2        // q, k rows
           + dv * (c + pad) * ts          // v^T
           + dk * (c + pad) * ts          // k-hat^T
           + dv * (dk + pad) * ts         // S^T
           + c * (dv + pad) * ts          // r / output rows
           + c * (dk + 4) * 4             // fp32 gate logits / log-decay
           + nsub * lpc * dk * 4          // gate partial totals
           + dk * 4                       // chunk total log-decay
           + 2 * c * 4;                   // row tables (double buffered)
}

constexpr bool config_fits(int ts, int dk, int dv, int c) { return lds_bytes(ts, dk, dv, c) <= kLdsLimit; }

}  // namespace gla

#endif
