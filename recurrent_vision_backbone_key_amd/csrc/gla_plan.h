// gla_plan.h -- argument validation and work planning (no HIP dependency).
#ifndef GLA_PLAN_H
#define GLA_PLAN_H

#include <stddef.h>
#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

// Compute units and accelerator dies (XCDs, each with its own L2) of the
// device a call runs on.  A null pointer stands for one MI355X in its
// single-partition mode: 256 compute units in 8 XCDs.
typedef struct gla_geom {
    int cus;
    int xcds;
} gla_geom;

// Fixed prefix of every forward workspace: a 4096-byte header and room for
// GLA_FLAG_WORDS segment flags.  Header words (4 bytes each), every group on a
// 128-byte cache line of its own so that the loads of one never wait behind
// the atomics of another: the chip-wide ticket counter, the sticky error word
// with the initialisation mark beside it (read together), and the ticket
// counter of XCD x at GLA_HDR_XCD + 32 x.
#define GLA_HEADER_BYTES 4096
#define GLA_FLAG_WORDS 32768
#define GLA_PREFIX_BYTES (GLA_HEADER_BYTES + GLA_FLAG_WORDS * 4)
#define GLA_HDR_TICKET 0
#define GLA_HDR_ERR 32
#define GLA_HDR_MARK 33
#define GLA_HDR_XCD 128
// Initialisation mark gla_workspace_init writes at header word GLA_HDR_MARK.
#define GLA_WS_MARK 0x474c4131u
// Most XCDs the header's per-XCD ticket counters serve.
#define GLA_MAX_XCDS 16

typedef struct gla_plan {
    int L, nchunks, seg_chunks, nseg;
    int onepass;                 // 1: single-pass kernel, 0: three passes
    int xcd_local;               // single pass: every scan on one XCD (u mod xcds)
    int xcd_tasks;               // single pass, xcd_local: workgroups per XCD
    int xcds;                    // single pass: XCDs of the device
    int one_round;               // single pass: every workgroup of the call resident at once
    int group;                   // single pass, one round: segments per group of the
                                 // two-level exchange (nseg: one level)
    size_t workspace_bytes;
    size_t off_flags, off_agg, off_incl;  // single-pass workspace layout (bytes)
    size_t off_slots;                     // three-pass segment slots (bytes)
    int proj_fused;              // gate expansion (W2, b) inside the single pass
    size_t off_z;                // gate projection: x W1 (fused) or z staged here (bytes)
    float tau, scale, eps;
} gla_plan;

// Group size of the one-round exchange over nseg segments: nseg (one level)
// below 24 segments, else ceil(sqrt(nseg)), or one more when no segment then
// folds more transfers nor more than kFoldBatch (8) of them.
int gla_exchange_group(int nseg);

// Size-only checks and the work plan (segments, workspace bytes) for a
// device of geometry `geo` (null: the MI355X default).
int gla_make_plan(int dir, int H, int W, int chunk, const gla_opts* opts, int has_gate,
                  const gla_geom* geo, gla_plan* plan);

// Pure host check of every argument of gla_fwd (pointers are compared, never
// dereferenced).  Fills *plan on success.  Returns a gla_status.
int gla_validate(const void* q, const void* k, const void* v, const float* gate_logits,
                 int dir, int H, int W, int chunk, const void* out, const void* r,
                 const gla_opts* opts, const gla_geom* geo, gla_plan* plan);

// Plan of gla_fwd_gate_proj: the plan of gla_fwd plus whether the expansion
// by W2 and b is fused into the single pass.  The workspace grows by the
// staged x W1 (B*L*16 binary32 words, fused) or the staged logits
// (B*L*NH*dk binary32 words) at off_z (included in workspace_bytes).
int gla_make_plan_gate_proj(int dir, int H, int W, int chunk, const gla_gate_proj* gate,
                            const gla_opts* opts, int has_gate, const gla_geom* geo,
                            gla_plan* plan);

// Host check of every argument of gla_fwd_gate_proj.  Fills *plan on success.
int gla_validate_gate_proj(const void* q, const void* k, const void* v, const gla_gate_proj* gate,
                           int dir, int H, int W, int chunk, const void* out, const void* r,
                           const gla_opts* opts, const gla_geom* geo, gla_plan* plan);

// Host check of every argument of gla_gate_logits.
int gla_validate_gate_logits(const gla_gate_proj* gate, int batch, int tokens, int heads, int dk,
                             int dtype, const float* z);

// Host check of every argument of gla_spatial_swiglu.
int gla_validate_sswiglu(const void* gate, const void* value, int64_t ld_in, const float* conv_w,
                         const float* conv_b, int batch, int H, int W, int channels, int dtype,
                         const void* out, int64_t ld_out);

// Backward: sizes checks, workspace layout (bytes): forward states at
// *off_f (after the fixed forward prefix, which a backward never writes, so a
// workspace shared with gla_fwd keeps its counters, flags and mark), reverse
// states at *off_r, chunk sums at *off_s, for d = 128 the binary32 partial
// sums of its d = 64 quarters at *off_p (rows x 256 floats; else 0), total
// *bytes.  The state slots are those of the (quarter's) head size.
int gla_plan_bwd(int dir, int H, int W, const gla_opts* opts, int* nchunks, size_t* off_f,
                 size_t* off_r, size_t* off_s, size_t* off_p, size_t* bytes);

// Host check of every argument of gla_bwd.
int gla_validate_bwd(const void* q, const void* k, const void* v, const float* z, const void* dout,
                     int dir, int H, int W, const void* dq, const void* dk, const void* dv,
                     const float* dz, const gla_opts* opts, int* nchunks, size_t* off_f,
                     size_t* off_r, size_t* off_s, size_t* off_p);

// Gated backward: workspace layout (bytes) -- the backward's own part at 0
// (gla_plan_bwd), then dO (binary32, rows x d), the dw partial sums
// (units x nchunks x d binary32) and, for d = 128, the entering states of
// quarters 1 .. 3 at off_fq, fq_bytes apart (quarter 0 keeps off_f); total in
// bytes.
typedef struct gla_bwd_gated_layout {
    size_t bwd_bytes, off_f, off_r, off_s, off_p, off_do, off_dwp, off_fq, fq_bytes, bytes;
    int nchunks;
} gla_bwd_gated_layout;

int gla_plan_bwd_gated(int dir, int H, int W, const gla_opts* opts, gla_bwd_gated_layout* lay);

// Host check of every argument of gla_bwd_gated.
int gla_validate_bwd_gated(const void* q, const void* k, const void* v, const float* z,
                           const void* r, const void* dout, int dir, int H, int W, const void* dq,
                           const void* dk, const void* dv, const float* dz, const void* dr,
                           const float* dw, const gla_opts* opts, gla_bwd_gated_layout* lay);

// Gate projection backward: workspace layout (bytes, each part 256-byte
// aligned): hp [tokens][16 ceil(rank/16)], then the partial sums of dW1
// [nsplit][rank][d_model], dW2 [nsplit][nout][rank] and db [nsplit][nout]
// (binary32), nsplit = ceil(tokens / 64).
typedef struct gla_proj_bwd_layout {
    size_t off_hp, off_p1, off_p2, off_pb, bytes;
    int nsplit;
} gla_proj_bwd_layout;

int gla_plan_gate_proj_bwd(const gla_gate_proj* gate, int tokens, int nout, gla_proj_bwd_layout* lay);

// Host check of every argument of gla_gate_proj_bwd.
int gla_validate_gate_proj_bwd(const gla_gate_proj* gate, int tokens, int nout, int dtype,
                               const float* dz, const void* dx, const float* dw1, const float* dw2,
                               const float* db, const void* workspace, size_t workspace_bytes,
                               gla_proj_bwd_layout* lay);

// Whether a (dtype, d_k, d_v, chunk) instantiation is built (shared-memory
// footprint of one workgroup within the 160 KiB of a gfx950 CU; d_k != d_v
// with 64-token chunks only).
int gla_config_built(int dtype, int dk, int dv, int chunk);

#ifdef __cplusplus
}
#endif

#endif
