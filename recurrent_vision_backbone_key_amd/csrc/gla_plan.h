// gla_plan.h -- argument validation and work planning (no HIP dependency).
#ifndef GLA_PLAN_H
#define GLA_PLAN_H

#include <stddef.h>
#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gla_plan {
    int L, nchunks, seg_chunks, nseg;
    int onepass;                 // 1: single-pass kernel, 0: three passes
    int xcd_local;               // single pass: every scan on one XCD (u mod 8)
    int xcd_tasks;               // single pass, xcd_local: workgroups per XCD
    size_t workspace_bytes;
    size_t off_flags, off_agg, off_incl;  // single-pass workspace layout (bytes)
    size_t off_slots;                     // three-pass segment slots (bytes)
    int proj_fused;              // gate expansion (W2, b) inside the single pass
    size_t off_z;                // gate projection: x W1 (fused) or z staged here (bytes)
    float tau, scale, eps;
} gla_plan;

// Size-only checks and the work plan (segments, workspace bytes).
int gla_make_plan(int dir, int H, int W, int chunk, const gla_opts* opts, int has_gate,
                  gla_plan* plan);

// Pure host check of every argument of gla_fwd (pointers are compared, never
// dereferenced).  Fills *plan on success.  Returns a gla_status.
int gla_validate(const void* q, const void* k, const void* v, const float* gate_logits,
                 int dir, int H, int W, int chunk, const void* out, const void* r,
                 const gla_opts* opts, gla_plan* plan);

// Plan of gla_fwd_gate_proj: the plan of gla_fwd plus whether the expansion
// by W2 and b is fused into the single pass.  The workspace grows by the
// staged x W1 (B*L*16 binary32 words, fused) or the staged logits
// (B*L*NH*dk binary32 words) at off_z (included in workspace_bytes).
int gla_make_plan_gate_proj(int dir, int H, int W, int chunk, const gla_gate_proj* gate,
                            const gla_opts* opts, int has_gate, gla_plan* plan);

// Host check of every argument of gla_fwd_gate_proj.  Fills *plan on success.
int gla_validate_gate_proj(const void* q, const void* k, const void* v, const gla_gate_proj* gate,
                           int dir, int H, int W, int chunk, const void* out, const void* r,
                           const gla_opts* opts, gla_plan* plan);

// Host check of every argument of gla_gate_logits.
int gla_validate_gate_logits(const gla_gate_proj* gate, int batch, int tokens, int heads, int dk,
                             int dtype, const float* z);

// Host check of every argument of gla_spatial_swiglu.
int gla_validate_sswiglu(const void* gate, const void* value, int64_t ld_in, const float* conv_w,
                         const float* conv_b, int batch, int H, int W, int channels, int dtype,
                         const void* out, int64_t ld_out);

// Backward: sizes checks, workspace layout (bytes): forward states at 0,
// reverse states at *off_r, chunk sums at *off_s, total *bytes.
int gla_plan_bwd(int dir, int H, int W, const gla_opts* opts, int* nchunks, size_t* off_r,
                 size_t* off_s, size_t* bytes);

// Host check of every argument of gla_bwd.
int gla_validate_bwd(const void* q, const void* k, const void* v, const float* z, const void* dout,
                     int dir, int H, int W, const void* dq, const void* dk, const void* dv,
                     const float* dz, const gla_opts* opts, int* nchunks, size_t* off_r,
                     size_t* off_s);

// Gated backward: workspace layout (bytes) -- the backward's own part at 0
// (gla_plan_bwd), then dO (binary32, rows x d) and the dw partial sums
// (units x nchunks x d binary32); total in bytes.
typedef struct gla_bwd_gated_layout {
    size_t bwd_bytes, off_r, off_s, off_do, off_dwp, bytes;
    int nchunks;
} gla_bwd_gated_layout;

int gla_plan_bwd_gated(int dir, int H, int W, const gla_opts* opts, gla_bwd_gated_layout* lay);

// Host check of every argument of gla_bwd_gated.
int gla_validate_bwd_gated(const void* q, const void* k, const void* v, const float* z,
                           const void* r, const void* dout, int dir, int H, int W, const void* dq,
                           const void* dk, const void* dv, const float* dz, const void* dr,
                           const float* dw, const gla_opts* opts, gla_bwd_gated_layout* lay);

// Whether a (dtype, head dim, chunk) instantiation is built (shared-memory
// footprint of one workgroup within the 160 KiB of a gfx950 CU).
int gla_config_built(int dtype, int d, int chunk);

#ifdef __cplusplus
}
#endif

#endif
