// gla_epi.h -- the backward through the fused output gate (gla_bwd.hip).
#ifndef GLA_EPI_H
#define GLA_EPI_H

namespace gla {

struct Params;
struct BwdParams;

// Output-gate operands of the gated backward.  Per (batch, token, head) row
// of d channels, with rho = (mean(o^2) + eps)^-1/2 and g = du (.) SiLU(r) (.) w:
//   dO  = rho g - (rho^3 / d) o sum(g (.) o)     (binary32, into BwdParams::dout)
//   dr  = du (.) w (.) o rho (.) SiLU'(r)        (storage type)
//   dwp[chunk workgroup][c] = the workgroup's rows' du SiLU(r) o rho, and
//   dw[c] = their sum in workgroup order (if dw is not null).
struct GatedBwd {
    const void* r;    // [B, L, NH, d] storage type
    const void* du;   // dL/du, [B, L, NH, d] storage type
    const float* w;   // [d] or null (ones)
    void* dr;         // [B, L, NH, d] storage type
    float* dwp;       // [units * nchunks][d]
    float* dw;        // [d] or null
    float eps;
    // d = 128 (quarters): o of one quarter alone, added in binary32 to o_out
    // (row stride BwdParams::ld) unless it is the first of its value half
    float* o_out;
    int o_acc;
    // d = 128: entering states of quarters 1 .. 3 (quarter 0: BwdParams::ws_f),
    // fq_floats apart
    float* fq;
    size_t fq_floats;
};

// Gated backward: entering states, o and the output gate's backward (dO into
// Q.dout, binary32), reverse aggregates from dO, then the chunk kernel.
int launch_bwd_gated(const Params& P, const BwdParams& Q, const GatedBwd& G, int dtype, int d,
                     void* stream);

}  // namespace gla

#endif
