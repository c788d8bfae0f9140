// gla_api.cpp -- the C ABI (include/gla.h) over the HIP kernels.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "gla.h"
#include "gla_epi.h"
#include "gla_launch.h"
#include "gla_plan.h"

namespace {

// Geometry (compute units, XCDs) of the device `stream` belongs to (the
// current device for the null stream), read from the runtime once per device
// and kept: it never changes while the process runs.  A host with no device
// plans for one MI355X (the plan then only sizes workspaces).
constexpr int kMaxDevices = 64;
std::atomic<int> g_geom[kMaxDevices];  // (cus << 8) | xcds, 0 until read

// Device `stream` belongs to (the current device for the null stream), or -1.
int stream_device(void* stream)
{
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) dev = -1;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        dev = -1;
    }
    return dev;
}

gla_geom device_geom(void* stream)
{
    gla_geom g = {256, 8};
    const int dev = stream_device(stream);
    if (dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return g;
    }
    int packed = g_geom[dev].load(std::memory_order_relaxed);
    if (packed == 0) {
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
            xcds < 1 || xcds > 255)
            xcds = 1;
        (void)hipGetLastError();
        packed = (cus << 8) | xcds;
        g_geom[dev].store(packed, std::memory_order_relaxed);
    }
    g.cus = packed >> 8;
    g.xcds = packed & 255;
    return g;
}

// Launches the planned forward; P.z (or the fused projection operands) set.
int run_fwd(gla::Params& P, const void* q, const void* k, const void* v, int dir, int H, int W,
            int chunk, void* out, const void* r, const gla_opts* opts, const gla_plan& plan)
{
    P.q = q;
    P.k = k;
    P.v = v;
    P.r = r;
    P.w = r ? opts->norm_weight : nullptr;
    P.out = out;
    P.ws = plan.off_slots ? (float*)((char*)opts->workspace + plan.off_slots) : (float*)opts->workspace;
    P.B = opts->batch;
    P.NH = opts->heads;
    P.H = H;
    P.W = W;
    P.L = plan.L;
    P.dir = dir;
    P.nchunks = plan.nchunks;
    P.seg_chunks = plan.seg_chunks;
    P.nseg = plan.nseg;
    P.scale = plan.scale;
    P.inv_tau = 1.0f / plan.tau;
    P.eps = plan.eps;
    P.ticket = P.err = P.flags = nullptr;
    P.xcd_local = plan.xcd_local;
    P.xcd_tasks = plan.xcd_tasks;
    P.xcds = plan.xcds;
    P.one_round = plan.one_round;
    P.group = plan.group > 0 ? plan.group : plan.nseg;
    P.agg = P.incl = nullptr;
    if (plan.onepass) {
        char* ws = (char*)opts->workspace;
        P.ticket = (unsigned*)ws;
        P.err = (unsigned*)ws + GLA_HDR_ERR;
        P.flags = (unsigned*)(ws + plan.off_flags);
        P.agg = (float*)(ws + plan.off_agg);
        P.incl = (float*)(ws + plan.off_incl);
        return gla::launch_onepass(P, opts->stream);
    }
    return gla::launch_fwd(P, opts->dtype, opts->dk, opts->dv, chunk, opts->stream);
}

gla::GateProj gate_of(const gla_gate_proj* g)
{
    gla::GateProj G;
    G.x = g->x;
    G.w1 = g->w1;
    G.w2 = g->w2;
    G.bias = g->bias;
    G.d_model = g->d_model;
    G.rank = g->rank;
    return G;
}

void no_proj(gla::Params& P)
{
    P.ghp = P.gw2 = P.gb = nullptr;
}

}  // namespace

extern "C" int gla_fwd(const void* q, const void* k, const void* v, const float* gate_logits,
                       int dir, int H, int W, int chunk, void* out, const void* r,
                       const gla_opts* opts)
{
    gla_plan plan;
    const gla_geom geo = device_geom(opts ? opts->stream : nullptr);
    const int st = gla_validate(q, k, v, gate_logits, dir, H, W, chunk, out, r, opts, &geo, &plan);
    if (st != GLA_OK) return st;
    gla::Params P;
    P.z = gate_logits;
    no_proj(P);
    return run_fwd(P, q, k, v, dir, H, W, chunk, out, r, opts, plan);
}

extern "C" int gla_fwd_noalloc(const void* q, const void* k, const void* v,
                               const float* gate_logits, int dir, int H, int W, int chunk,
                               void* out, const void* r, const gla_opts* opts)
{
    if (!opts) return GLA_EINVAL;
    const gla_geom geo = device_geom(opts->stream);
    gla_opts o = *opts;
    o.workspace = nullptr;
    o.workspace_bytes = 0;
    gla_plan plan;
    int st = gla_make_plan(dir, H, W, chunk, &o, r != nullptr, &geo, &plan);
    if (st != GLA_OK) return st;
    if (plan.workspace_bytes > gla::kScratchBytes) return GLA_ESCRATCH;
    if (plan.workspace_bytes) {
        void* ptr = nullptr;
        st = gla::scratch_for_device(stream_device(opts->stream), opts->stream, &ptr);
        if (st != GLA_OK) return st;
        o.workspace = ptr;
        o.workspace_bytes = gla::kScratchBytes;
    }
    st = gla_validate(q, k, v, gate_logits, dir, H, W, chunk, out, r, &o, &geo, &plan);
    if (st != GLA_OK) return st;
    gla::Params P;
    P.z = gate_logits;
    no_proj(P);
    return run_fwd(P, q, k, v, dir, H, W, chunk, out, r, &o, plan);
}

extern "C" int gla_fwd_gate_proj(const void* q, const void* k, const void* v,
                                 const gla_gate_proj* gate, int dir, int H, int W, int chunk,
                                 void* out, const void* r, const gla_opts* opts)
{
    gla_plan plan;
    const gla_geom geo = device_geom(opts ? opts->stream : nullptr);
    const int st = gla_validate_gate_proj(q, k, v, gate, dir, H, W, chunk, out, r, opts, &geo, &plan);
    if (st != GLA_OK) return st;
    gla::Params P;
    no_proj(P);
    if (plan.proj_fused) {
        // x W1 (16 values per token) into the workspace; the single pass
        // expands it with W2 and b per head
        float* hp = (float*)((char*)opts->workspace + plan.off_z);
        const int ls = gla::launch_gate_rank(gate_of(gate), opts->dtype, opts->batch * plan.L, hp,
                                             opts->stream);
        if (ls != GLA_OK) return ls;
        P.z = nullptr;
        P.ghp = hp;
        P.gw2 = gate->w2;
        P.gb = gate->bias;
    } else {
        // z staged in the workspace by the projection kernel, then the
        // ordinary forward on the same stream
        float* z = (float*)((char*)opts->workspace + plan.off_z);
        const int ls = gla::launch_gate_logits(gate_of(gate), opts->dtype, opts->batch * plan.L,
                                               opts->heads * opts->dk, z, opts->stream);
        if (ls != GLA_OK) return ls;
        P.z = z;
    }
    return run_fwd(P, q, k, v, dir, H, W, chunk, out, r, opts, plan);
}

extern "C" size_t gla_workspace_size_gate_proj(int dir, int H, int W, int chunk,
                                               const gla_gate_proj* gate, const gla_opts* opts)
{
    gla_plan plan;
    const gla_geom geo = device_geom(opts ? opts->stream : nullptr);
    if (gla_make_plan_gate_proj(dir, H, W, chunk, gate, opts, 0, &geo, &plan) != GLA_OK) return 0;
    return plan.workspace_bytes;
}

extern "C" int gla_gate_logits(const gla_gate_proj* gate, int batch, int tokens, int heads, int dk,
                               int dtype, float* z, void* stream)
{
    const int st = gla_validate_gate_logits(gate, batch, tokens, heads, dk, dtype, z);
    if (st != GLA_OK) return st;
    return gla::launch_gate_logits(gate_of(gate), dtype, batch * tokens, heads * dk, z, stream);
}

extern "C" int gla_gate_proj_bwd(const gla_gate_proj* gate, int tokens, int nout, int dtype,
                                 const float* dz, void* dx, float* dw1, float* dw2, float* db,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    gla_proj_bwd_layout lay;
    const int st = gla_validate_gate_proj_bwd(gate, tokens, nout, dtype, dz, dx, dw1, dw2, db,
                                              workspace, workspace_bytes, &lay);
    if (st != GLA_OK) return st;
    char* ws = (char*)workspace;
    gla::ProjBwdWs W;
    W.hp = (float*)(ws + lay.off_hp);
    W.p1 = (float*)(ws + lay.off_p1);
    W.p2 = (float*)(ws + lay.off_p2);
    W.pb = (float*)(ws + lay.off_pb);
    return gla::launch_gate_proj_bwd(gate_of(gate), dtype, tokens, nout, dz, dx, dw1, dw2, db, W,
                                     stream);
}

extern "C" size_t gla_gate_proj_bwd_workspace_size(const gla_gate_proj* gate, int tokens, int nout)
{
    gla_proj_bwd_layout lay;
    if (gla_plan_gate_proj_bwd(gate, tokens, nout, &lay) != GLA_OK) return 0;
    return lay.bytes;
}

extern "C" size_t gla_workspace_size(int dir, int H, int W, int chunk, const gla_opts* opts)
{
    gla_plan plan;
    const gla_geom geo = device_geom(opts ? opts->stream : nullptr);
    if (gla_make_plan(dir, H, W, chunk, opts, 0, &geo, &plan) != GLA_OK) return 0;
    return plan.workspace_bytes;
}

extern "C" int gla_workspace_init(void* workspace, size_t bytes, void* stream)
{
    if (bytes == 0) return GLA_OK;
    if (!workspace || ((uintptr_t)workspace & 15u) != 0 || (bytes & 3u) != 0) return GLA_EINVAL;
    return gla::launch_workspace_init(workspace, bytes, stream);
}

extern "C" int gla_workspace_status(void* workspace, size_t bytes, void* stream,
                                    uint32_t* error_bits)
{
    if (!error_bits || !workspace || ((uintptr_t)workspace & 15u) != 0 || bytes < GLA_HEADER_BYTES ||
        (bytes & 3u) != 0)
        return GLA_EINVAL;
    *error_bits = 0;
    hipStream_t st = (hipStream_t)stream;
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, (const char*)workspace + 4 * GLA_HDR_ERR, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return GLA_EHIP;
    *error_bits = word;
    if (word == 0) return GLA_OK;
    const int ls = gla::launch_workspace_init(workspace, bytes, stream);
    return ls == GLA_OK ? GLA_EKERNEL : ls;
}

extern "C" int gla_spatial_swiglu(const void* gate, const void* value, int64_t ld_in,
                                  const float* conv_w, const float* conv_b, int batch, int H, int W,
                                  int channels, int dtype, void* out, int64_t ld_out, void* stream)
{
    const int st = gla_validate_sswiglu(gate, value, ld_in, conv_w, conv_b, batch, H, W, channels,
                                        dtype, out, ld_out);
    if (st != GLA_OK) return st;
    return gla::launch_sswiglu(gate, value, ld_in, conv_w, conv_b, out, ld_out, batch, H, W,
                               channels, dtype, stream);
}

namespace {

// Launch parameters of the backward for validated arguments.
void bwd_params(const void* q, const void* k, const void* v, const float* gate_logits,
                const void* dout, int dir, int H, int W, void* dq, void* dk, void* dv, float* dz,
                const gla_opts* opts, char* ws, int nchunks, size_t off_f, size_t off_r,
                size_t off_s, size_t off_p, gla::Params& P, gla::BwdParams& Q)
{
    P.q = q;
    P.k = k;
    P.v = v;
    P.z = gate_logits;
    P.r = nullptr;
    P.w = nullptr;
    P.out = nullptr;
    P.ws = (float*)ws;
    P.B = opts->batch;
    P.NH = opts->heads;
    P.H = H;
    P.W = W;
    P.L = H * W;
    P.dir = dir;
    P.nchunks = nchunks;
    P.seg_chunks = 1;
    P.nseg = nchunks;
    P.scale = opts->scale > 0.0f ? opts->scale : (float)(1.0 / sqrt((double)opts->dk));
    P.inv_tau = 1.0f / (opts->tau > 0.0f ? opts->tau : 16.0f);
    P.eps = 0.0f;
    P.ticket = P.err = P.flags = nullptr;
    P.agg = P.incl = nullptr;
    P.xcd_local = 0;
    P.xcd_tasks = 0;
    P.xcds = 1;
    P.one_round = 0;
    P.group = 1;
    no_proj(P);
    Q.dout = dout;
    Q.dq = dq;
    Q.dk = dk;
    Q.dv = dv;
    Q.dz = dz;
    Q.ws_f = (float*)(ws + off_f);
    Q.ws_r = (float*)(ws + off_r);
    Q.ws_s = (float*)(ws + off_s);
    Q.ld = opts->dk;
    // d = 128: binary32 partial sums of the d = 64 quarters (dq, dk of one key
    // half, dv of both value halves)
    const size_t rows = (size_t)opts->batch * H * W * opts->heads;
    Q.ldp = 64;
    Q.pq = off_p ? (float*)(ws + off_p) : nullptr;
    Q.pk = off_p ? Q.pq + rows * 64 : nullptr;
    Q.pv = off_p ? Q.pk + rows * 64 : nullptr;
    Q.mode_qk = Q.mode_v = 0;
}

}  // namespace

extern "C" int gla_bwd(const void* q, const void* k, const void* v, const float* gate_logits,
                       const void* dout, int dir, int H, int W, void* dq, void* dk, void* dv,
                       float* dz, const gla_opts* opts)
{
    int nchunks = 0;
    size_t off_f = 0, off_r = 0, off_s = 0, off_p = 0;
    const int st = gla_validate_bwd(q, k, v, gate_logits, dout, dir, H, W, dq, dk, dv, dz, opts,
                                    &nchunks, &off_f, &off_r, &off_s, &off_p);
    if (st != GLA_OK) return st;
    gla::Params P;
    gla::BwdParams Q;
    bwd_params(q, k, v, gate_logits, dout, dir, H, W, dq, dk, dv, dz, opts, (char*)opts->workspace,
               nchunks, off_f, off_r, off_s, off_p, P, Q);
    return gla::launch_bwd(P, Q, opts->dtype, opts->dk, opts->stream);
}

extern "C" size_t gla_bwd_workspace_size(int dir, int H, int W, const gla_opts* opts)
{
    int nchunks = 0;
    size_t off_f = 0, off_r = 0, off_s = 0, off_p = 0, bytes = 0;
    if (gla_plan_bwd(dir, H, W, opts, &nchunks, &off_f, &off_r, &off_s, &off_p, &bytes) != GLA_OK)
        return 0;
    return bytes;
}

extern "C" int gla_bwd_gated(const void* q, const void* k, const void* v,
                             const float* gate_logits, const void* r, const void* dout, int dir,
                             int H, int W, void* dq, void* dk, void* dv, float* dz, void* dr,
                             float* dw, const gla_opts* opts)
{
    gla_bwd_gated_layout lay;
    const int st = gla_validate_bwd_gated(q, k, v, gate_logits, r, dout, dir, H, W, dq, dk, dv,
                                          dz, dr, dw, opts, &lay);
    if (st != GLA_OK) return st;
    char* ws = (char*)opts->workspace;
    gla::Params P;
    gla::BwdParams Q;
    // dO (binary32) is produced inside the call, in the workspace
    bwd_params(q, k, v, gate_logits, ws + lay.off_do, dir, H, W, dq, dk, dv, dz, opts, ws,
               lay.nchunks, lay.off_f, lay.off_r, lay.off_s, lay.off_p, P, Q);
    gla::GatedBwd G;
    G.r = r;
    G.du = dout;
    G.w = opts->norm_weight;
    G.dr = dr;
    G.dwp = (float*)(ws + lay.off_dwp);
    G.dw = dw;
    G.eps = opts->eps;
    G.o_out = nullptr;
    G.o_acc = 0;
    G.fq = lay.off_fq ? (float*)(ws + lay.off_fq) : nullptr;
    G.fq_floats = lay.fq_bytes / 4;
    return gla::launch_bwd_gated(P, Q, G, opts->dtype, opts->dk, opts->stream);
}

extern "C" size_t gla_bwd_gated_workspace_size(int dir, int H, int W, const gla_opts* opts)
{
    gla_bwd_gated_layout lay;
    if (!opts || gla_plan_bwd_gated(dir, H, W, opts, &lay) != GLA_OK) return 0;
    return lay.bytes;
}

extern "C" const char* gla_status_str(int status)
{
    switch (status) {
    case GLA_OK: return "GLA_OK: success";
    case GLA_EINVAL: return "GLA_EINVAL: invalid argument (null or misaligned pointer, bad size or direction, or overlapping output)";
    case GLA_EUNSUPPORTED: return "GLA_EUNSUPPORTED: head dim, chunk, dtype or size outside the built set";
    case GLA_EWORKSPACE: return "GLA_EWORKSPACE: workspace missing, misaligned or smaller than gla_workspace_size()";
    case GLA_EHIP: return "GLA_EHIP: HIP runtime error at launch";
    case GLA_EKERNEL: return "GLA_EKERNEL: a kernel reported a failure in the workspace error word";
    case GLA_ESCRATCH: return "GLA_ESCRATCH: the call needs more scratch than gla_fwd_noalloc's fixed 64 MiB array (use gla_fwd with a workspace of gla_workspace_size() bytes)";
    default: return "unknown gla status";
    }
}

extern "C" int gla_abi_version(void) { return GLA_ABI_VERSION; }
