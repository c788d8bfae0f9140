/*
 * gla.h -- C ABI of the MI355X (gfx950) chunkwise forward of key-only gated
 * linear attention (GLA), the token mixer of GTR ("GTR: Gated Token
 * Recurrence for Efficient Dense Prediction", paper Section 2.1).
 *
 * Operation (paper Section 2.1, key-only GLA paragraph and output-gate
 * paragraph).  For every batch b and head h, along the scan order of the
 * H x W patch grid:
 *     gamma_t = sigmoid(z_t)^(1/tau)            elementwise, 1 x d_k
 *     S_t     = Diag(gamma_t) S_{t-1} + k_t^T v_t,   S_0 = 0   (d_k x d_v)
 *     o_t     = scale * q_t S_t                 (scale = d_k^-1/2 by default)
 * and, when the output gate is requested (r != NULL),
 *     u_t     = SiLU(r_t) (.) w (.) o_t / sqrt(mean_{d_v}(o_t^2) + eps).
 * The value-side decay is fixed to one (no right-hand diagonal on S).
 *
 * Scan directions (paper Section 2.1, scan-direction paragraph; Figure 2 is
 * not available, so the orders below are this library's reading): token
 * index t = h*W + w on the row-major grid;
 *     GLA_L2R: raster order t = i;   GLA_R2L: raster order reversed;
 *     GLA_T2B: column-major order;   GLA_B2T: column-major order reversed.
 * One continuous scan covers all L = H*W tokens.  The output is always
 * written at each token's original grid position, so no caller-side
 * reordering is needed for any direction.
 *
 * Layout: q, k, gate_logits: [B, L, NH, d_k]; v, r, out: [B, L, NH, d_v];
 * all dense row-major, L = H*W.  d_k and d_v may differ (paper Section 2.1:
 * W_Q, W_K of d x d_k, W_V of d x d_v).  q, k, v, r, out share one storage type
 * (opts->dtype); gate_logits and norm_weight are binary32.
 *
 * Memory and ownership: every tensor pointer is a DEVICE pointer owned by the
 * caller and must be 16-byte aligned.  The library allocates nothing and
 * keeps no mutable global state.  Calls run asynchronously on opts->stream.
 *
 * Errors: every function returns a gla_status.  Argument checks run before
 * anything is launched; on any error nothing is launched and out is not
 * touched.  A launch failure is reported as GLA_EHIP.  Faults inside a kernel
 * surface at the caller's next synchronisation.  Non-finite inputs propagate
 * (a NaN gate logit yields NaN outputs downstream of it).
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_ABI_VERSION 7

#if defined(__GNUC__)
#define GLA_API __attribute__((visibility("default")))
#else
#define GLA_API
#endif

enum gla_dir { GLA_L2R = 0, GLA_R2L = 1, GLA_T2B = 2, GLA_B2T = 3 };
enum gla_dtype { GLA_F16 = 0, GLA_F32 = 1 };
enum gla_status {
    GLA_OK = 0,
    GLA_EINVAL = 1,       /* null or misaligned pointer, bad size or direction,
                             out overlapping an input                          */
    GLA_EUNSUPPORTED = 2, /* d_k, d_v, chunk, dtype or size outside the built set */
    GLA_EWORKSPACE = 3,   /* workspace missing or smaller than gla_workspace_size */
    GLA_EHIP = 4,         /* the HIP runtime reported an error at launch         */
    GLA_EKERNEL = 5,      /* a kernel reported a failure in the workspace's error
                             word (gla_workspace_status)                        */
    GLA_ESCRATCH = 6      /* gla_fwd_noalloc: the call needs more scratch than the
                             library's fixed array holds                        */
};

/* Bits of a workspace's error word (gla_workspace_status).  They are sticky:
 * once one is set, every later single-pass call on that workspace writes NaN
 * to all its outputs, until the workspace is initialised again.  Within a call,
 * a failure poisons every segment downstream of it in its scan (NaN rows). */
#define GLA_WS_ERR_WAIT 1u   /* a bounded wait for another workgroup's segment
                                exchange gave up; the affected rows hold NaN    */
#define GLA_WS_ERR_TICKET 2u /* a work ticket beyond the launch: the counters were
                                not clear (an earlier call did not complete)     */
#define GLA_WS_ERR_INIT 4u   /* the workspace was not initialised with
                                gla_workspace_init; every output row holds NaN  */

typedef struct gla_opts {
    int32_t batch;   /* B  >= 1 */
    int32_t heads;   /* NH >= 1 */
    int32_t dk;      /* key/query head dim d_k; supported: 16, 32, 64, 128    */
    int32_t dv;      /* value head dim d_v; supported: 16, 32, 64, 128; d_v !=
                        d_k with 64-token chunks (three passes)                 */
    int32_t dtype;   /* GLA_F16 or GLA_F32: storage of q, k, v, r and out      */
    float tau;       /* gate temperature; <= 0 selects 16 (paper Sec. 2.1)     */
    float scale;     /* output scale; <= 0 selects dk^-1/2 (paper Sec. 2.1)    */
    float eps;       /* RMSNorm epsilon, inside the square root; used iff r    */
    const float *norm_weight; /* [dv] device pointer, shared by all heads;
                                 NULL selects ones; used iff r                  */
    void *workspace;          /* device scratch, see gla_workspace_size         */
    size_t workspace_bytes;
    void *stream;             /* hipStream_t; NULL selects the null stream      */
    int32_t segment_chunks;   /* chunks per sequence segment; 0 lets the library
                                 choose; a value >= the chunk count runs one
                                 workgroup per (batch, head)                    */
    int32_t algorithm;        /* GLA_ALGO_AUTO, GLA_ALGO_SINGLE_PASS or
                                 GLA_ALGO_THREE_PASS (see below)                 */
} gla_opts;

/* Algorithms.  SINGLE_PASS (binary16, d_k = d_v = 64, chunk 64, segments of
 * at most 8 chunks, at most 65 segments per scan) reads every input once: one
 * workgroup per segment, segments exchange states through the workspace.
 * THREE_PASS (every built configuration) runs an aggregate pass, a fold pass
 * and an output pass.  AUTO picks SINGLE_PASS whenever it applies. */
enum gla_algorithm { GLA_ALGO_AUTO = 0, GLA_ALGO_SINGLE_PASS = 1, GLA_ALGO_THREE_PASS = 2 };

/*
 * gla_fwd -- chunkwise forward (paper Section 2.1, definition above).
 *   q, k         [B, L, NH, dk] queries and keys (opts->dtype)
 *   v            [B, L, NH, dv] values (opts->dtype)
 *   gate_logits  [B, L, NH, dk] binary32 pre-sigmoid gate logits z
 *   dir          GLA_L2R | GLA_R2L | GLA_T2B | GLA_B2T
 *   H, W         patch grid, H >= 1, W >= 1, H*W < 2^24
 *   chunk        tokens per chunk: 16, 32, 64 or 128; the result does not
 *                depend on it beyond rounding.  Combinations whose workgroup
 *                shared memory exceeds a gfx950 CU's 160 KiB return
 *                GLA_EUNSUPPORTED (binary16: d = 128 with chunk 128;
 *                binary32: d = 64 with chunk 128, d = 128 with chunk >= 32)
 *   out          [B, L, NH, dv] output (opts->dtype); must not overlap inputs
 *   r            [B, L, NH, dv] output-gate pre-activation x W_r, or NULL for
 *                out = o (no gate, no RMSNorm)
 *   opts         sizes, dtype, stream, workspace (must not be NULL)
 * The workspace must hold gla_workspace_size() bytes when that is nonzero.
 * It starts with a fixed 4096 + 131072-byte prefix (the single pass's ticket
 * counters, error word, initialisation mark and per-segment flags; nothing
 * else is ever written there), followed by per-segment fp32 states.  Before
 * its first use it must be initialised with gla_workspace_init(); every
 * completed call leaves the counters and flags cleared again, so calls and
 * graph replays need no reset in between.  A single-pass call on a workspace
 * that was not initialised writes NaN to every output row and sets
 * GLA_WS_ERR_INIT; a wait that gives up (bounded spin) writes NaN to the rows
 * it affects and sets GLA_WS_ERR_WAIT.  gla_workspace_status() reads these
 * bits.  Calls that share a workspace must be ordered on one stream; calls
 * that overlap on one workspace race.  The workspace size and the plan behind
 * it depend on the device current on the calling thread (its compute units
 * and XCDs; a host without a device plans for one MI355X).
 */
GLA_API int gla_fwd(const void *q, const void *k, const void *v, const float *gate_logits,
            int dir, int H, int W, int chunk, void *out, const void *r,
            const gla_opts *opts);

/*
 * gla_fwd_noalloc -- gla_fwd for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and kernels, with opts->workspace and
 * opts->workspace_bytes ignored.  The exchange area lives in a library-owned
 * device array of GLA_NOALLOC_SCRATCH_BYTES per GPU (allocated when the code
 * object loads, held until the process ends); a call whose
 * gla_workspace_size() exceeds it returns GLA_ESCRATCH and launches nothing.
 * Nothing is allocated per call.  The first call on a device looks the array
 * up and initialises it on opts->stream, ahead of its own kernels; every
 * completed call leaves it ready for the next.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, no
 * ordering between them) race and must not be issued.  gla_workspace_status
 * does not apply (the array is not addressable by the caller); a failure
 * still writes NaN to the affected rows.  Arguments, layout and the other
 * statuses as for gla_fwd.
 */
#define GLA_NOALLOC_SCRATCH_BYTES (64u << 20)
GLA_API int gla_fwd_noalloc(const void *q, const void *k, const void *v, const float *gate_logits,
                            int dir, int H, int W, int chunk, void *out, const void *r,
                            const gla_opts *opts);

/* Bytes of workspace gla_fwd needs for these arguments (0: none needed).
 * Returns 0 as well for arguments gla_fwd would reject. */
GLA_API size_t gla_workspace_size(int dir, int H, int W, int chunk, const gla_opts *opts);

/*
 * gla_workspace_init -- clears `bytes` bytes of a workspace (counters, flags,
 * error word) and, when bytes >= 4096, writes the initialisation mark, on
 * `stream` (hipStream_t, NULL selects the null stream) with a fill kernel.
 * Call once after allocating a workspace for gla_fwd, and again after
 * gla_workspace_status() reported an error.  workspace: device pointer,
 * 16-byte aligned; bytes: a multiple of 4 (0 does nothing).
 * GLA_EINVAL on a bad pointer or size, GLA_EHIP on a launch failure.
 */
GLA_API int gla_workspace_init(void *workspace, size_t bytes, void *stream);

/*
 * gla_workspace_status -- waits for the work queued on `stream` (hipStream_t,
 * NULL selects the null stream), then reads the error word of a workspace
 * used by gla_fwd / gla_fwd_gate_proj (bytes >= 4096, 16-byte aligned device
 * pointer) into *error_bits (GLA_WS_ERR_* bits; 0 when no kernel reported a
 * failure).  Returns GLA_OK when the word is zero.  When it is not, the
 * workspace is initialised again (gla_workspace_init over `bytes` bytes, on
 * `stream`) so that it can be reused, and GLA_EKERNEL is returned.
 * GLA_EINVAL on a bad pointer, size or a null error_bits, GLA_EHIP when the
 * runtime reports an error (for example a fault of the queued work).
 */
GLA_API int gla_workspace_status(void *workspace, size_t bytes, void *stream,
                                 uint32_t *error_bits);

/*
 * Low-rank retention-gate projection (paper Section 2.1, definition of the
 * retention gate: the gate logits are x_t W1 W2 + b with W1 of shape
 * d_model x rank, W2 of shape rank x d_k and rank 16).  This library reads
 * the formula for all heads at once, as in GLA's low-rank gate: W1 is shared
 * by the heads and W2, b hold the heads' d_k columns side by side, so head h
 * uses columns h*dk .. h*dk + dk - 1 of W2 and b:
 *     z[b, t, h, c] = bias[h*dk + c] + sum_j (sum_m x[b, t, m] W1[m][j]) W2[j][h*dk + c]
 * Both factors are passed transposed, the layout of a linear layer's weight.
 */
typedef struct gla_gate_proj {
    const void *x;       /* [B, L, d_model] block input, storage opts->dtype
                            (or the dtype argument of gla_gate_logits)         */
    const void *w1;      /* [rank, d_model] W1 transposed, same storage as x   */
    const float *w2;     /* [NH*dk, rank] W2 transposed, binary32             */
    const float *bias;   /* [NH*dk] binary32; NULL selects zeros              */
    /* every pointer above: device memory, 16-byte aligned                     */
    int32_t d_model;     /* >= 8, a multiple of 8                             */
    int32_t rank;        /* 1 .. 64 (the pages use 16)                        */
} gla_gate_proj;

/*
 * gla_gate_logits -- the projection alone: writes z [batch, tokens, heads, dk]
 * binary32 (the gate_logits operand of gla_fwd) on `stream` (hipStream_t,
 * NULL selects the null stream).  z is a 16-byte aligned device pointer that
 * must not overlap an input.
 * dtype: GLA_F16 or GLA_F32, the storage of x and w1; dk in {16, 32, 64, 128}.
 * GLA_EINVAL on a bad pointer, size or overlap, GLA_EUNSUPPORTED on a dtype
 * or dk outside the built set, GLA_EHIP on a launch failure.
 */
GLA_API int gla_gate_logits(const gla_gate_proj *gate, int batch, int tokens, int heads, int dk,
                            int dtype, float *z, void *stream);

/*
 * gla_gate_proj_bwd -- gradients of the projection above (chain rule of
 * z = x W1 W2 + b) for dz = dL/dz, written on the stored arrays (w1 [rank,
 * d_model], w2 [nout, rank]) with hp[t][j] = sum_m x[t][m] w1[j][m] (the rank
 * values of token t) and dhp[t][j] = sum_n dz[t][n] w2[n][j]:
 *     dx[t][m]  = sum_j dhp[t][j] w1[j][m]   [tokens, d_model]  storage dtype
 *     dw1[j][m] = sum_t dhp[t][j] x[t][m]    [rank, d_model]    binary32
 *     dw2[n][j] = sum_t dz[t][n] hp[t][j]    [nout, rank]       binary32
 *     db[n]     = sum_t dz[t][n]             [nout]             binary32
 * tokens = batch * sequence length and nout = heads * dk; dz [tokens, nout]
 * binary32 is the layout gla_bwd writes dz in ([B, L, NH, dk]).  x, w1 and
 * w2 are read from `gate` (bias unused); dtype: GLA_F16 or GLA_F32, the
 * storage of x, w1 and dx.  Accumulation in binary32; the sums over tokens
 * are formed per block of 64 tokens and the blocks added in order, so equal
 * inputs give equal bits.  The workspace (device, 16-byte aligned, no
 * initialisation) must hold gla_gate_proj_bwd_workspace_size() bytes; the
 * outputs must not overlap each other, an input or the workspace.
 * Asynchronous on `stream` (hipStream_t, NULL: the null stream).
 * GLA_EINVAL on a bad pointer, size or overlap, GLA_EUNSUPPORTED on a dtype
 * or size outside the built set (tokens <= 2^26, nout <= 65536, tokens *
 * nout and tokens * d_model below 2^29),
 * GLA_EWORKSPACE on a missing or small workspace, GLA_EHIP on a launch
 * failure.
 */
GLA_API int gla_gate_proj_bwd(const gla_gate_proj *gate, int tokens, int nout, int dtype,
                              const float *dz, void *dx, float *dw1, float *dw2, float *db,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace gla_gate_proj_bwd needs (0 for arguments it would reject). */
GLA_API size_t gla_gate_proj_bwd_workspace_size(const gla_gate_proj *gate, int tokens, int nout);

/*
 * gla_fwd_gate_proj -- gla_fwd with the gate logits computed from the block
 * input by the low-rank projection above instead of read from memory.
 * Arguments as for gla_fwd, with `gate` in place of gate_logits (x and w1
 * stored as opts->dtype).  For the single-pass configuration with rank 16
 * (any d_model), a first kernel writes x W1 (16 binary32 values per token,
 * shared by the heads) into the workspace and the single pass expands it
 * with each head's W2 columns and bias on the matrix cores in binary32, so
 * the logits never reach memory.  Every other configuration writes z into
 * the workspace with the kernel of gla_gate_logits first and then runs the
 * ordinary forward.  The workspace must hold gla_workspace_size_gate_proj()
 * bytes, cleared once with gla_workspace_init() as for gla_fwd.  Returns a
 * gla_status as gla_fwd.
 */
GLA_API int gla_fwd_gate_proj(const void *q, const void *k, const void *v,
                              const gla_gate_proj *gate, int dir, int H, int W, int chunk,
                              void *out, const void *r, const gla_opts *opts);

/* Bytes of workspace gla_fwd_gate_proj needs (0: none; also 0 for arguments
 * it would reject). */
GLA_API size_t gla_workspace_size_gate_proj(int dir, int H, int W, int chunk,
                                            const gla_gate_proj *gate, const gla_opts *opts);

/*
 * gla_spatial_swiglu -- the fused core of the Spatial SwiGLU block (paper
 * Section 2.1, Spatial SwiGLU paragraph; its equation is not available, so
 * the form below is this library's reading): the value branch is laid out on
 * the H x W patch grid (token t = h*W + w) and mixed by a 3x3 depthwise
 * convolution, the gating branch stays tokenwise:
 *     out[b, t, c] = SiLU(gate[b, t, c]) * (bias[c] + sum_{i,j = 0..2}
 *                    conv_w[c][i][j] * value[b, (h+i-1)*W + (w+j-1), c])
 * with zero padding outside the grid (cross-correlation, like a depthwise
 * Conv2d with padding 1) and SiLU(x) = x / (1 + e^-x), in binary32.
 *   gate, value  [batch, H*W, channels] rows of ld_in elements (the first
 *                `channels` used), storage dtype; a fused projection output
 *                [.., 2*channels] can be passed as gate = base,
 *                value = base + channels, ld_in = 2*channels
 *   conv_w       [channels, 3, 3] binary32 (a depthwise Conv2d weight)
 *   conv_b       [channels] binary32, NULL selects zeros
 *   out          [batch, H*W, channels] rows of ld_out elements, storage dtype;
 *                must not overlap an input
 *   dtype        GLA_F16 or GLA_F32; channels a multiple of 8; ld_in, ld_out
 *                multiples of 8 and >= channels; H, W, batch >= 1
 * gate, value and out are 16-byte aligned device pointers, conv_w and conv_b
 * 4-byte aligned.  Runs on `stream` (hipStream_t, NULL: the null stream); needs
 * no workspace.  GLA_EINVAL on a bad pointer, size or overlap,
 * GLA_EUNSUPPORTED on another dtype, GLA_EHIP on a launch failure.
 */
GLA_API int gla_spatial_swiglu(const void *gate, const void *value, int64_t ld_in,
                               const float *conv_w, const float *conv_b, int batch, int H, int W,
                               int channels, int dtype, void *out, int64_t ld_out, void *stream);

/*
 * gla_bwd -- gradients of the ungated forward (r == NULL in gla_fwd; paper
 * Section 2.1 recurrence, differentiated).  With dout = dL/do:
 *     dS_t = sum_{u >= t} Diag(prod_{t < j <= u} gamma_j) scale q_u^T dout_u
 *     dq_t = scale dout_t S_t^T,  dk_t = dS_t v_t^T,  dv_t = k_t dS_t
 *     dz_t = (1 - sigmoid(z_t)) / tau (.) sum_{u >= t} (q_u (.) dq_u - k_u (.) dk_u)
 * along the scan order of `dir`, results at the original token positions.
 *   q, k, gate_logits, dq, dk, dz  [B, L, NH, dk]; v, dout, dv [B, L, NH, dv]
 *   q, k, v, dout, dq, dk, dv in opts->dtype; gate_logits and dz binary32
 * Supported: dk == dv in {16, 32, 64, 128}, binary16 or binary32 storage;
 * 64-position chunks.  d = 128 runs as four d = 64 quarters (key half x value
 * half: the decay acts on each key channel alone and o is linear in v) whose
 * gradients add up in binary32 in the workspace.  opts->norm_weight, eps,
 * segment_chunks and algorithm are ignored.
 * The workspace must hold gla_bwd_workspace_size() bytes (no initialisation:
 * every call rewrites what it reads).  Its data starts after the same fixed
 * 4096 + 131072-byte prefix as gla_fwd's, which a backward never writes, so one
 * workspace can serve both.  All pointers are 16-byte aligned
 * device pointers; the four outputs must not overlap each other, an input or
 * the workspace.  Asynchronous on opts->stream.  Returns a gla_status.
 */
GLA_API int gla_bwd(const void *q, const void *k, const void *v, const float *gate_logits,
                    const void *dout, int dir, int H, int W, void *dq, void *dk, void *dv,
                    float *dz, const gla_opts *opts);

/* Bytes of workspace gla_bwd needs (0 for arguments it would reject). */
GLA_API size_t gla_bwd_workspace_size(int dir, int H, int W, const gla_opts *opts);

/*
 * gla_bwd_gated -- gradients of the gated forward (gla_fwd with r; paper
 * Section 2.1 output-gate paragraph): with dout = dL/du for
 *     u = SiLU(r) (.) w (.) o / sqrt(mean_{d_v}(o^2) + eps),
 * o the ungated output and rho = 1 / sqrt(mean(o^2) + eps), g = dout (.) SiLU(r) (.) w:
 *     do = rho g - (rho^3 / d_v) o sum(g (.) o)
 *     dr = dout (.) w (.) o rho (.) SiLU'(r)
 *     dw = sum over every (batch, token, head) row of dout (.) SiLU(r) (.) o rho
 * and dq, dk, dv, dz as gla_bwd for do.  o is recomputed chunk by chunk in
 * binary32 (never rounded to the storage type) and do stays binary32 in the
 * workspace; the same head sizes as gla_bwd.
 *   r, dout, dr [B, L, NH, dv] in opts->dtype; w = opts->norm_weight ([dv]
 *   binary32, NULL selects ones) and opts->eps as in gla_fwd; dw [dv] binary32,
 *   may be NULL (not computed); the rest as gla_bwd.
 * The workspace must hold gla_bwd_gated_workspace_size() bytes (no
 * initialisation).  16-byte aligned device pointers; outputs must not overlap
 * each other, an input or the workspace.  Asynchronous on opts->stream;
 * dw is the same for equal inputs (fixed summation order).  Returns a gla_status.
 */
GLA_API int gla_bwd_gated(const void *q, const void *k, const void *v, const float *gate_logits,
                          const void *r, const void *dout, int dir, int H, int W, void *dq,
                          void *dk, void *dv, float *dz, void *dr, float *dw,
                          const gla_opts *opts);

/* Bytes of workspace gla_bwd_gated needs (0 for arguments it would reject). */
GLA_API size_t gla_bwd_gated_workspace_size(int dir, int H, int W, const gla_opts *opts);

/* Static, NUL-terminated description of a gla_status value. */
GLA_API const char *gla_status_str(int status);

/* GLA_ABI_VERSION of the loaded library. */
GLA_API int gla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
