// gla_launch.h -- internal interface between the C-ABI layer and the kernels.
#ifndef GLA_LAUNCH_H
#define GLA_LAUNCH_H

#include <stddef.h>

#include "gla.h"

namespace gla {

// Largest segment (in chunks) the single-pass kernel keeps on chip, and the
// largest one its mid-size instance takes (fewer registers: segments of up to
// kOnePassMidChunks chunks run there, longer ones in the eight-chunk instance).
constexpr int kOnePassMaxChunks = 8;
constexpr int kOnePassMidChunks = 5;

// Arguments of one forward call, already validated.
struct Params {
    const void* q;      // [B, L, NH, DK]
    const void* k;      // [B, L, NH, DK]
    const void* v;      // [B, L, NH, DV]
    const float* z;     // [B, L, NH, DK] gate logits
    const void* r;      // [B, L, NH, DV] output-gate pre-activation, or null
    const float* w;     // [DV] RMSNorm weight, or null (ones)
    void* out;          // [B, L, NH, DV]
    float* ws;          // three-pass: segment slots [units][nseg-1][DK*DV + DK] fp32
    // single-pass exchange (workspace): header words, one flag per (scan,
    // segment), segment aggregates and group transfers
    unsigned* ticket;   // workspace header (words GLA_HDR_* of gla_plan.h)
    unsigned* err;      // header word GLA_HDR_ERR: sticky error bits (GLA_WS_ERR_*),
                        // followed by the initialisation mark
    unsigned* flags;    // [units][nseg]: bits 1 aggregate, 2 group transfer, 4 done
    float* agg;         // [units][nseg][DK*DV + DK]
    float* incl;        // [units][nseg][DK*DV + DK]: group transfers (leaders' slots)
    int B, NH, H, W, L, dir;
    int nchunks;        // ceil(L / chunk)
    int seg_chunks;     // chunks per segment
    int nseg;           // segments per scan
    int xcd_local;      // single pass: scan u runs on XCD u mod xcds (exchange in that L2)
    int xcd_tasks;      // single pass, xcd_local: workgroups per XCD (grid / xcds)
    int xcds;           // single pass: XCDs of the device
    int one_round;      // single pass: every workgroup of the call is resident at once
    int group;          // single pass, one round: segments per group of the two-level
                        // exchange (nseg: one level)
    float scale;        // output scale
    float inv_tau;      // 1 / tau
    float eps;          // RMSNorm epsilon
    // single pass with the gate expansion fused (z == null): rank 16
    const float* ghp;   // [B*L, 16] x W1 of every token
    const float* gw2;   // [NH*DK, 16] W2 transposed
    const float* gb;    // [NH*DK] gate bias, or null (zeros)
};

// Low-rank gate projection operands (include/gla.h, gla_gate_proj).
struct GateProj {
    const void* x;
    const void* w1;
    const float* w2;
    const float* bias;
    int d_model;
    int rank;
};

// Rank of the gate projection whose W2 expansion is fused into the single pass.
constexpr int kFusedProjRank = 16;

// Launches the aggregate, fold and output passes (or only the output pass
// when nseg == 1) on `stream`.  Returns a gla_status value.
int launch_fwd(const Params& P, int dtype, int dk, int dv, int chunk, void* stream);

// Fold pass alone: turns the segment aggregates in P.ws into incoming states.
int launch_fold(const Params& P, int d, void* stream);

// Aggregate, fold and output passes of the d = 128 binary16 chunk-64 path
// (8-wavefront kernels; the fold pass when nseg > 1).
int launch_wide(const Params& P, void* stream);

// Single-pass kernel (binary16, d = 64, chunk 64): one launch.
int launch_onepass(const Params& P, void* stream);

// Gate logits z [tokens, nout] binary32 from the low-rank projection.
int launch_gate_logits(const GateProj& G, int dtype, int tokens, int nout, float* z, void* stream);

// First factor alone: hp = x W1, [tokens, 16 ceil(rank / 16)] binary32.
int launch_gate_rank(const GateProj& G, int dtype, int tokens, float* hp, void* stream);

// Tokens per partial product of the gate projection's backward (its products
// over the tokens are added up block by block in this order).
constexpr int kProjBwdSplit = 64;

// Workspace parts of the gate projection's backward (binary32): hp [tokens][16
// ceil(rank/16)] and the per-block partial sums of dW1 [nsplit][rank][d_model],
// dW2 [nsplit][nout][rank] and db [nsplit][nout].
struct ProjBwdWs {
    float* hp;
    float* p1;
    float* p2;
    float* pb;
};

// Gradients of the gate projection (include/gla.h, gla_gate_proj_bwd),
// arguments checked.
int launch_gate_proj_bwd(const GateProj& G, int dtype, int tokens, int nout, const float* dz, void* dx,
                         float* dw1, float* dw2, float* db, const ProjBwdWs& W, void* stream);

// Spatial SwiGLU core (include/gla.h, gla_spatial_swiglu), arguments checked.
int launch_sswiglu(const void* a, const void* v, long long ld_in, const float* w, const float* bias,
                   void* out, long long ld_out, int B, int H, int W, int C, int dtype, void* stream);

// Backward (include/gla.h, gla_bwd): gradient of the outputs and the
// gradients written, plus the workspace parts.
struct BwdParams {
    const void* dout;   // [B, L, NH, DV]
    void* dq;           // [B, L, NH, DK]
    void* dk;           // [B, L, NH, DK]
    void* dv;           // [B, L, NH, DV]
    float* dz;          // [B, L, NH, DK] binary32
    float* ws_f;        // chunk local states, then the entering states [units][nchunks-1][D*D + D]
    float* ws_r;        // reverse aggregates, then the entering gradients [units][nchunks-1][D*D + D]
    float* ws_s;        // later chunks' part of dz per chunk [units][nchunks][D]
    int ld;             // row stride (elements) of q, k, v, z, dout and the gradients
    // A d = 128 call runs as four d = 64 quarters (key half x value half) whose
    // gradients add up in binary32 (mode 0: the quarter is the whole problem)
    float* pq;          // [rows][ldp] dq of one key half
    float* pk;          // [rows][ldp] dk of one key half
    float* pv;          // dv partials, row stride ld (at the value half's columns)
    int ldp;            // row stride of pq and pk
    int mode_qk;        // dq, dk, dz: 0 store, 1 keep as partial, 2 add the partial and store
    int mode_v;         // dv: the same
};

// Chunkwise backward, 64-position chunks (P describes the forward call).
int launch_bwd(const Params& P, const BwdParams& Q, int dtype, int d, void* stream);

// Zero-fills a workspace (counters, flags) on `stream`.
int launch_workspace_init(void* ws, size_t bytes, void* stream);

// Size of the library-owned scratch array of gla_fwd_noalloc (per device).
constexpr size_t kScratchBytes = GLA_NOALLOC_SCRATCH_BYTES;

// Device address of the scratch array on device `dev`, looked up (with `dev`
// current) and initialised on `stream` at the first call for that device.
int scratch_for_device(int dev, void* stream, void** ptr);

}  // namespace gla

#endif
