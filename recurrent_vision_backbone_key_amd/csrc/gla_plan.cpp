// gla_plan.cpp -- argument validation and work planning for gla_fwd.
// Compiled without HIP so that every error path can be exercised on a host
// without a GPU.
#include "gla_plan.h"

#include <math.h>
#include <stdint.h>

#include "gla_geometry.h"
#include "gla_launch.h"

namespace {

// Default geometry: one MI355X in its single-partition mode.
constexpr gla_geom kMi355x = {256, 8};
constexpr size_t kFlagWords = GLA_FLAG_WORDS;
// Every forward layout starts with the same fixed prefix (header and flag
// room; see gla_plan.h).  Data never lands there, so a workspace reused
// across shapes, algorithms or backward calls never finds another call's data
// where its own counters, flags and mark must be.
constexpr size_t kReserved = GLA_PREFIX_BYTES;

bool is_pow2_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// A usable geometry: the one given, else the default.
gla_geom geometry(const gla_geom* geo)
{
    gla_geom g = geo ? *geo : kMi355x;
    if (g.cus < 1) g.cus = kMi355x.cus;
    if (g.xcds < 1 || g.xcds > g.cus) g.xcds = 1;
    return g;
}

}  // namespace

extern "C" int gla_config_built(int dtype, int dk, int dv, int chunk)
{
    if (dtype != GLA_F16 && dtype != GLA_F32) return 0;
    if (!is_pow2_dim(dk) || !is_pow2_dim(dv) || !is_pow2_dim(chunk)) return 0;
    if (dk != dv && chunk != 64) return 0;
    return gla::config_fits(dtype == GLA_F16 ? 2 : 4, dk, dv, chunk) ? 1 : 0;
}

extern "C" // Two-level exchange of one-round single-pass plans: segment j of a scan folds
// j / G combined transfers (groups before its own) and j mod G aggregates
// (its own group's segments before it), at most
//     max((nseg-1) / G + (nseg-1) mod G,  nseg / G + G - 2)
// transfers.  Below 24 segments one level (G = nseg) is faster: the leaders'
// extra publish round trip costs more than it saves (5 segments: 34.1 ->
// 35.7 us per call).  From 24 on, G = ceil(sqrt(nseg)), or one more when that
// folds no more transfers at the worst segment and stays within one round of
// 8 loads: with 25 segments groups of 6 instead of 5 (the last segment folds
// 4 transfers instead of 8) measured 13.31 -> 13.16 us per call; with 28,
// groups of 7 would fold 9 (a second round of loads cost about 1 us).
int gla_exchange_group(int nseg)
{
    if (nseg < 24) return nseg;
    int g = 1;
    while (g * g < nseg) ++g;
    auto most = [nseg](int gs) {
        const int a = (nseg - 1) / gs + (nseg - 1) % gs;
        const int b = nseg / gs + gs - 2;
        return (nseg / gs >= 1 && b > a) ? b : a;
    };
    const int m0 = most(g), m1 = most(g + 1);
    return (m1 <= m0 && m1 <= 8) ? g + 1 : g;
}

int gla_make_plan(int dir, int H, int W, int chunk, const gla_opts* o,
                             int has_gate, const gla_geom* geo, gla_plan* plan)
{
    if (!o || !plan) return GLA_EINVAL;
    if (o->batch < 1 || o->heads < 1 || H < 1 || W < 1) return GLA_EINVAL;
    if (dir < GLA_L2R || dir > GLA_B2T) return GLA_EINVAL;
    if (o->dtype != GLA_F16 && o->dtype != GLA_F32) return GLA_EUNSUPPORTED;
    if (!is_pow2_dim(o->dk) || !is_pow2_dim(o->dv)) return GLA_EUNSUPPORTED;
    if (!is_pow2_dim(chunk) || !gla_config_built(o->dtype, o->dk, o->dv, chunk)) return GLA_EUNSUPPORTED;
    const int64_t L = (int64_t)H * W;
    if (L >= (int64_t)1 << 24) return GLA_EUNSUPPORTED;
    const int64_t rows = (int64_t)o->batch * L * o->heads;  // kernel row index is int32
    if (rows >= (int64_t)1 << 31) return GLA_EUNSUPPORTED;
    if (isnan(o->tau) || isnan(o->scale) || isinf(o->tau) || isinf(o->scale)) return GLA_EINVAL;
    if (has_gate && (isnan(o->eps) || o->eps < 0.0f || isinf(o->eps))) return GLA_EINVAL;

    const int nchunks = (int)((L + chunk - 1) / chunk);
    const int64_t units = (int64_t)o->batch * o->heads;
    if (o->algorithm < GLA_ALGO_AUTO || o->algorithm > GLA_ALGO_THREE_PASS) return GLA_EINVAL;
    const gla_geom gm = geometry(geo);
    const int cus = gm.cus, xcds = gm.xcds, cus_per_xcd = gm.cus / gm.xcds;
    plan->L = (int)L;
    plan->nchunks = nchunks;
    plan->onepass = 0;
    plan->xcds = xcds;
    plan->one_round = 0;
    plan->group = 0;
    plan->proj_fused = 0;
    plan->off_z = 0;
    plan->off_flags = plan->off_agg = plan->off_incl = plan->off_slots = 0;

    // Single pass: binary16, d = 64, 64-token chunks; segments of at most
    // kOnePassMaxChunks chunks, at most 65 segments per scan (one wavefront
    // of look-back), about one workgroup per compute unit.  When the scans
    // spread over the XCDs without costing a second round of workgroups on
    // any of them (or divide evenly), scan u runs on XCD u mod xcds and the
    // segment exchange stays in that XCD's L2.
    // (the kernel addresses its inputs with 32-bit buffer offsets: the fp32
    // gate logits, 256 bytes per row, stay below 2^31 bytes)
    const bool sp_shape = o->dtype == GLA_F16 && o->dk == 64 && o->dv == 64 && chunk == 64 &&
                          rows < ((int64_t)1 << 23);
    plan->xcd_local = 0;
    plan->xcd_tasks = 0;
    if (o->algorithm != GLA_ALGO_THREE_PASS && sp_shape) {
        const int min_seg = (nchunks + 64) / 65;
        const int64_t upx = (units + xcds - 1) / xcds;  // scans per XCD (most)
        const int max_seg = nchunks < gla::kOnePassMaxChunks ? nchunks : gla::kOnePassMaxChunks;
        // the shortest segment whose workgroups fit in one round, one per
        // compute unit, on `cu` compute units at `per` scans (the longest
        // allowed when none does: fewer workgroups and exchanges; 8 x 6 scans
        // of 256 chunks took 240 us per call in eight-chunk segments against
        // 260 us in five-chunk ones).  (The one-chunk instance could hold two
        // workgroups per CU, but plans that used them measured slower: a
        // 1.6K-token frame with 12 heads in one-chunk segments two per CU
        // took 19.3 us per call against 16.1 us in two-chunk segments.)
        auto fit_seg = [&](int64_t per, int64_t cu) {
            for (int sg = min_seg; sg <= max_seg; ++sg)
                if (per * ((nchunks + sg - 1) / sg) <= cu) return sg;
            return max_seg;
        };
        const int seg_g = fit_seg(units, cus);
        const int seg_l = fit_seg(upx, cus_per_xcd);
        int seg = o->segment_chunks;
        if (seg > nchunks) seg = nchunks;
        // XCD-local when it keeps segments as short as the chip-wide plan and
        // either fits one round per XCD or the scans divide evenly over XCDs
        const int seg_chk = seg > 0 ? seg : seg_l;
        const int64_t tasks = upx * ((nchunks + seg_chk - 1) / seg_chk);
        const bool local = xcds > 1 && xcds <= GLA_MAX_XCDS && (seg > 0 || seg_l <= seg_g) &&
                           (tasks <= cus_per_xcd || units % xcds == 0);
        if (seg <= 0) seg = local ? seg_l : seg_g;
        const size_t nflag = (size_t)units * ((nchunks + seg - 1) / (seg > 0 ? seg : 1));
        if (seg >= min_seg && seg <= gla::kOnePassMaxChunks && nflag <= kFlagWords) {
            const int nseg = (nchunks + seg - 1) / seg;
            plan->onepass = 1;
            plan->seg_chunks = seg;
            plan->nseg = nseg;
            plan->xcd_local = local ? 1 : 0;
            plan->xcd_tasks = local ? (int)(upx * nseg) : 0;
            plan->one_round = local ? (plan->xcd_tasks <= cus_per_xcd) : (units * nseg <= cus);
            plan->group = gla_exchange_group(nseg);
            plan->off_flags = GLA_HEADER_BYTES;
            plan->off_agg = kReserved;
            plan->off_incl = plan->off_agg + nflag * ((size_t)64 * 64 + 64) * 4;
            plan->workspace_bytes = plan->off_incl + nflag * ((size_t)64 * 64 + 64) * 4;
        }
    }
    if (!plan->onepass) {
        if (o->algorithm == GLA_ALGO_SINGLE_PASS) return GLA_EUNSUPPORTED;
        // Three passes: segments of seg_chunks chunks, enough workgroups for
        // the chip (the d = 128 binary16 chunk-64 kernels hold one workgroup
        // per compute unit: three full rounds).
        const bool wide = o->dtype == GLA_F16 && o->dk == 128 && o->dv == 128 && chunk == 64;
        const int64_t target = wide ? 3 * (int64_t)cus : 2 * (int64_t)cus;
        int seg = o->segment_chunks;
        if (seg <= 0) {
            const int64_t want = (units * nchunks + target - 1) / target;
            seg = (int)(want < 1 ? 1 : want);
        }
        if (seg > nchunks) seg = nchunks;
        const int nseg = (nchunks + seg - 1) / seg;
        plan->seg_chunks = seg;
        plan->nseg = nseg;
        plan->off_slots = nseg > 1 ? kReserved : 0;
        plan->workspace_bytes =
            nseg > 1 ? kReserved + (size_t)units * (nseg - 1) * ((size_t)o->dk * o->dv + o->dk) * 4 : 0;
    }
    plan->tau = o->tau > 0.0f ? o->tau : 16.0f;
    plan->scale = o->scale > 0.0f ? o->scale : (float)(1.0 / sqrt((double)o->dk));
    plan->eps = o->eps;
    return GLA_OK;
}

namespace {

// One input operand: pointer, bytes, required alignment.
struct Operand {
    const void* p;
    size_t bytes;
    uintptr_t align;
};

// Alignment of every operand and of out, no overlap of out with an input,
// and the workspace (size, alignment, no overlap with anything).
int check_operands(const Operand* ins, int n, const void* out, size_t out_bytes,
                   const gla_opts* o, const gla_plan* plan)
{
    for (int i = 0; i < n; ++i)
        if (ins[i].p && !aligned(ins[i].p, ins[i].align)) return GLA_EINVAL;
    if (!aligned(out, 16)) return GLA_EINVAL;
    for (int i = 0; i < n; ++i)
        if (overlaps(out, out_bytes, ins[i].p, ins[i].bytes)) return GLA_EINVAL;
    if (plan->workspace_bytes) {
        if (!o->workspace || o->workspace_bytes < plan->workspace_bytes ||
            !aligned(o->workspace, 16))
            return GLA_EWORKSPACE;
        if (overlaps(o->workspace, plan->workspace_bytes, out, out_bytes)) return GLA_EINVAL;
        for (int i = 0; i < n; ++i)
            if (overlaps(o->workspace, plan->workspace_bytes, ins[i].p, ins[i].bytes))
                return GLA_EINVAL;
    }
    return GLA_OK;
}

// Sizes of the gate projection operands.
int check_gate_sizes(const gla_gate_proj* gate)
{
    if (!gate || !gate->x || !gate->w1 || !gate->w2) return GLA_EINVAL;
    if (gate->d_model < 8 || gate->d_model > (1 << 16) || gate->d_model % 8 != 0) return GLA_EINVAL;
    if (gate->rank < 1 || gate->rank > 64) return GLA_EINVAL;
    return GLA_OK;
}

// The gate projection operands as a list (x, w1, w2, bias).
void gate_operands(const gla_gate_proj* gate, size_t tokens, int heads, int dk, size_t es,
                   Operand* ops)
{
    const size_t nout = (size_t)heads * dk;
    ops[0] = Operand{gate->x, tokens * gate->d_model * es, 16};
    ops[1] = Operand{gate->w1, (size_t)gate->rank * gate->d_model * es, 16};
    ops[2] = Operand{gate->w2, nout * gate->rank * 4, 16};
    ops[3] = Operand{gate->bias, nout * 4, 16};
}

}  // namespace

extern "C" int gla_validate(const void* q, const void* k, const void* v, const float* z,
                            int dir, int H, int W, int chunk, const void* out, const void* r,
                            const gla_opts* o, const gla_geom* geo, gla_plan* plan)
{
    if (!o || !plan) return GLA_EINVAL;
    if (!q || !k || !v || !z || !out) return GLA_EINVAL;
    const int st = gla_make_plan(dir, H, W, chunk, o, r != nullptr, geo, plan);
    if (st != GLA_OK) return st;

    const size_t es = o->dtype == GLA_F16 ? 2 : 4;
    const size_t rows = (size_t)o->batch * plan->L * o->heads;
    const size_t nk = rows * o->dk, nv = rows * o->dv;
    const Operand ins[6] = {{q, nk * es, 16}, {k, nk * es, 16}, {v, nv * es, 16}, {z, nk * 4, 16},
                            {r, nv * es, 16}, {r ? o->norm_weight : nullptr, (size_t)o->dv * 4, 4}};
    return check_operands(ins, 6, out, nv * es, o, plan);
}

extern "C" int gla_make_plan_gate_proj(int dir, int H, int W, int chunk, const gla_gate_proj* gate,
                                       const gla_opts* o, int has_gate, const gla_geom* geo,
                                       gla_plan* plan)
{
    int st = check_gate_sizes(gate);
    if (st != GLA_OK) return st;
    st = gla_make_plan(dir, H, W, chunk, o, has_gate, geo, plan);
    if (st != GLA_OK) return st;
    // fused (single pass, rank 16): x W1 staged, 16 binary32 values per
    // token; otherwise the logits themselves, NH*dk per token.  Either sits
    // after the fixed prefix even when the forward itself needs no workspace,
    // so it never overwrites the counters, flags or mark.
    plan->off_z = align256(plan->workspace_bytes > kReserved ? plan->workspace_bytes : kReserved);
    const size_t tokens = (size_t)o->batch * plan->L;
    if (plan->onepass && gate->rank == gla::kFusedProjRank) {
        plan->proj_fused = 1;
        plan->workspace_bytes = plan->off_z + tokens * gla::kFusedProjRank * 4;
    } else {
        plan->workspace_bytes = plan->off_z + tokens * o->heads * o->dk * 4;
    }
    return GLA_OK;
}

extern "C" int gla_validate_gate_proj(const void* q, const void* k, const void* v,
                                      const gla_gate_proj* gate, int dir, int H, int W, int chunk,
                                      const void* out, const void* r, const gla_opts* o,
                                      const gla_geom* geo, gla_plan* plan)
{
    if (!o || !plan || !gate) return GLA_EINVAL;
    if (!q || !k || !v || !out) return GLA_EINVAL;
    const int st = gla_make_plan_gate_proj(dir, H, W, chunk, gate, o, r != nullptr, geo, plan);
    if (st != GLA_OK) return st;
    const size_t es = o->dtype == GLA_F16 ? 2 : 4;
    const size_t tokens = (size_t)o->batch * plan->L;
    const size_t rows = tokens * o->heads;
    const size_t nk = rows * o->dk, nv = rows * o->dv;
    Operand ins[9] = {{q, nk * es, 16}, {k, nk * es, 16}, {v, nv * es, 16}, {r, nv * es, 16},
                      {r ? o->norm_weight : nullptr, (size_t)o->dv * 4, 4}};
    gate_operands(gate, tokens, o->heads, o->dk, es, ins + 5);
    return check_operands(ins, 9, out, nv * es, o, plan);
}

extern "C" int gla_validate_gate_logits(const gla_gate_proj* gate, int batch, int tokens, int heads,
                                        int dk, int dtype, const float* z)
{
    int st = check_gate_sizes(gate);
    if (st != GLA_OK) return st;
    if (!z || batch < 1 || tokens < 1 || heads < 1) return GLA_EINVAL;
    if (dtype != GLA_F16 && dtype != GLA_F32) return GLA_EUNSUPPORTED;
    if (!is_pow2_dim(dk)) return GLA_EUNSUPPORTED;
    const int64_t ntok = (int64_t)batch * tokens;
    if (ntok >= (int64_t)1 << 31 || ntok * heads >= (int64_t)1 << 31) return GLA_EUNSUPPORTED;
    const size_t es = dtype == GLA_F16 ? 2 : 4;
    Operand ins[4];
    gate_operands(gate, (size_t)ntok, heads, dk, es, ins);
    for (int i = 0; i < 4; ++i)
        if (ins[i].p && !aligned(ins[i].p, ins[i].align)) return GLA_EINVAL;
    const size_t zb = (size_t)ntok * heads * dk * 4;
    if (!aligned(z, 16)) return GLA_EINVAL;
    for (int i = 0; i < 4; ++i)
        if (overlaps(z, zb, ins[i].p, ins[i].bytes)) return GLA_EINVAL;
    return GLA_OK;
}

extern "C" int gla_plan_gate_proj_bwd(const gla_gate_proj* gate, int tokens, int nout,
                                      gla_proj_bwd_layout* lay)
{
    const int st = check_gate_sizes(gate);
    if (st != GLA_OK) return st;
    if (!lay || tokens < 1 || nout < 1) return GLA_EINVAL;
    if (tokens > (1 << 26) || nout > (1 << 16)) return GLA_EUNSUPPORTED;
    const int64_t R = gate->rank, RP = 16 * ((R + 15) / 16), DM = gate->d_model;
    const int64_t ns = ((int64_t)tokens + gla::kProjBwdSplit - 1) / gla::kProjBwdSplit;
    // the fused kernel addresses dz and x with 32-bit buffer offsets
    if ((int64_t)tokens * nout * 4 >= ((int64_t)1 << 31) || (int64_t)tokens * DM * 4 >= ((int64_t)1 << 31))
        return GLA_EUNSUPPORTED;
    // one workgroup per token block; the reduction's grid (64 outputs per
    // workgroup over the three arrays) stays far below 2^31 at these bounds
    lay->nsplit = (int)ns;
    lay->off_hp = 0;
    lay->off_p1 = align256(lay->off_hp + (size_t)tokens * RP * 4);
    lay->off_p2 = align256(lay->off_p1 + (size_t)ns * R * DM * 4);
    lay->off_pb = align256(lay->off_p2 + (size_t)ns * nout * R * 4);
    lay->bytes = lay->off_pb + (size_t)ns * nout * 4;
    return GLA_OK;
}

extern "C" int gla_validate_gate_proj_bwd(const gla_gate_proj* gate, int tokens, int nout, int dtype,
                                          const float* dz, const void* dx, const float* dw1,
                                          const float* dw2, const float* db, const void* workspace,
                                          size_t workspace_bytes, gla_proj_bwd_layout* lay)
{
    const int st = gla_plan_gate_proj_bwd(gate, tokens, nout, lay);
    if (st != GLA_OK) return st;
    if (!dz || !dx || !dw1 || !dw2 || !db) return GLA_EINVAL;
    if (dtype != GLA_F16 && dtype != GLA_F32) return GLA_EUNSUPPORTED;
    const size_t es = dtype == GLA_F16 ? 2 : 4;
    const size_t R = gate->rank, DM = gate->d_model;
    const Operand ins[5] = {{gate->x, (size_t)tokens * DM * es, 16},
                            {gate->w1, R * DM * es, 16},
                            {gate->w2, (size_t)nout * R * 4, 16},
                            {gate->bias, (size_t)nout * 4, 16},
                            {dz, (size_t)tokens * nout * 4, 16}};
    const Operand outs[4] = {{dx, (size_t)tokens * DM * es, 16},
                             {dw1, R * DM * 4, 16},
                             {dw2, (size_t)nout * R * 4, 16},
                             {db, (size_t)nout * 4, 16}};
    for (int i = 0; i < 5; ++i)
        if (ins[i].p && !aligned(ins[i].p, 16)) return GLA_EINVAL;
    for (int i = 0; i < 4; ++i) {
        if (!aligned(outs[i].p, 16)) return GLA_EINVAL;
        for (int j = 0; j < 5; ++j)
            if (ins[j].p && overlaps(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes)) return GLA_EINVAL;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return GLA_EINVAL;
    }
    if (!workspace || workspace_bytes < lay->bytes || !aligned(workspace, 16)) return GLA_EWORKSPACE;
    for (int i = 0; i < 5; ++i)
        if (ins[i].p && overlaps(workspace, lay->bytes, ins[i].p, ins[i].bytes)) return GLA_EINVAL;
    for (int i = 0; i < 4; ++i)
        if (overlaps(workspace, lay->bytes, outs[i].p, outs[i].bytes)) return GLA_EINVAL;
    return GLA_OK;
}

extern "C" int gla_validate_sswiglu(const void* gate, const void* value, int64_t ld_in,
                                    const float* conv_w, const float* conv_b, int batch, int H,
                                    int W, int channels, int dtype, const void* out, int64_t ld_out)
{
    if (!gate || !value || !conv_w || !out) return GLA_EINVAL;
    if (batch < 1 || H < 1 || W < 1 || channels < 8 || channels % 8 != 0) return GLA_EINVAL;
    if (ld_in < channels || ld_out < channels || ld_in % 8 != 0 || ld_out % 8 != 0) return GLA_EINVAL;
    if (dtype != GLA_F16 && dtype != GLA_F32) return GLA_EUNSUPPORTED;
    const int64_t tokens = (int64_t)batch * H * W;
    if ((int64_t)H * W >= ((int64_t)1 << 31) || tokens >= ((int64_t)1 << 40)) return GLA_EINVAL;
    // one workgroup per 8 x 8 tile and 64 channels (grid below 2^31)
    const int64_t planes = (int64_t)batch * ((channels + 63) / 64);
    const int64_t tiles = (int64_t)((H + 7) / 8) * ((W + 7) / 8);
    if (8 * ((planes + 7) / 8) * tiles >= ((int64_t)1 << 31)) return GLA_EINVAL;
    const size_t es = dtype == GLA_F16 ? 2 : 4;
    const size_t in_b = ((size_t)(tokens - 1) * ld_in + channels) * es;
    const size_t out_b = ((size_t)(tokens - 1) * ld_out + channels) * es;
    const Operand ins[4] = {{gate, in_b, 16}, {value, in_b, 16}, {conv_w, (size_t)channels * 36, 4},
                            {conv_b, (size_t)channels * 4, 4}};
    for (int i = 0; i < 4; ++i)
        if (ins[i].p && !aligned(ins[i].p, ins[i].align)) return GLA_EINVAL;
    if (!aligned(out, 16)) return GLA_EINVAL;
    for (int i = 0; i < 4; ++i)
        if (overlaps(out, out_b, ins[i].p, ins[i].bytes)) return GLA_EINVAL;
    return GLA_OK;
}

extern "C" int gla_plan_bwd(int dir, int H, int W, const gla_opts* o, int* nchunks, size_t* off_f,
                            size_t* off_r, size_t* off_s, size_t* off_p, size_t* bytes)
{
    if (!o) return GLA_EINVAL;
    if (o->batch < 1 || o->heads < 1 || H < 1 || W < 1) return GLA_EINVAL;
    if (dir < GLA_L2R || dir > GLA_B2T) return GLA_EINVAL;
    if (o->dtype != GLA_F16 && o->dtype != GLA_F32) return GLA_EUNSUPPORTED;
    if (o->dk != o->dv || (o->dk != 16 && o->dk != 32 && o->dk != 64 && o->dk != 128))
        return GLA_EUNSUPPORTED;
    const int64_t L = (int64_t)H * W;
    if (L >= (int64_t)1 << 24) return GLA_EUNSUPPORTED;
    const int64_t rows = (int64_t)o->batch * L * o->heads;
    if (rows >= (int64_t)1 << 31) return GLA_EUNSUPPORTED;
    if (isnan(o->tau) || isnan(o->scale) || isinf(o->tau) || isinf(o->scale)) return GLA_EINVAL;
    const int64_t nc = (L + 63) / 64;
    const int64_t units = (int64_t)o->batch * o->heads;
    const int dq = o->dk == 128 ? 64 : o->dk;  // d = 128 runs as four d = 64 quarters
    const size_t slot = ((size_t)dq * dq + dq) * 4;
    const size_t part = (size_t)units * (nc - 1) * slot;
    *nchunks = (int)nc;
    *off_f = kReserved;
    *off_r = *off_f + align256(part);
    *off_s = *off_r + align256(part);
    *bytes = *off_s + (size_t)units * nc * dq * 4;
    *off_p = 0;
    if (o->dk == 128) {
        *off_p = align256(*bytes);
        *bytes = *off_p + (size_t)rows * 256 * 4;
    }
    return GLA_OK;
}

extern "C" int gla_validate_bwd(const void* q, const void* k, const void* v, const float* z,
                                const void* dout, int dir, int H, int W, const void* dq,
                                const void* dk, const void* dv, const float* dz, const gla_opts* o,
                                int* nchunks, size_t* off_f, size_t* off_r, size_t* off_s,
                                size_t* off_p)
{
    if (!o || !q || !k || !v || !z || !dout || !dq || !dk || !dv || !dz) return GLA_EINVAL;
    size_t bytes = 0;
    const int st = gla_plan_bwd(dir, H, W, o, nchunks, off_f, off_r, off_s, off_p, &bytes);
    if (st != GLA_OK) return st;
    const size_t es = o->dtype == GLA_F16 ? 2 : 4;
    const size_t n = (size_t)o->batch * H * W * o->heads * o->dk;
    const Operand ins[5] = {{q, n * es, 16}, {k, n * es, 16}, {v, n * es, 16}, {z, n * 4, 16},
                            {dout, n * es, 16}};
    const Operand outs[4] = {{dq, n * es, 16}, {dk, n * es, 16}, {dv, n * es, 16}, {dz, n * 4, 16}};
    for (int i = 0; i < 5; ++i)
        if (!aligned(ins[i].p, 16)) return GLA_EINVAL;
    for (int i = 0; i < 4; ++i) {
        if (!aligned(outs[i].p, 16)) return GLA_EINVAL;
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes)) return GLA_EINVAL;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return GLA_EINVAL;
    }
    if (!o->workspace || o->workspace_bytes < bytes || !aligned(o->workspace, 16)) return GLA_EWORKSPACE;
    for (int i = 0; i < 5; ++i)
        if (overlaps(o->workspace, bytes, ins[i].p, ins[i].bytes)) return GLA_EINVAL;
    for (int i = 0; i < 4; ++i)
        if (overlaps(o->workspace, bytes, outs[i].p, outs[i].bytes)) return GLA_EINVAL;
    return GLA_OK;
}

extern "C" int gla_plan_bwd_gated(int dir, int H, int W, const gla_opts* o, gla_bwd_gated_layout* lay)
{
    int nchunks = 0;
    size_t off_f = 0, off_r = 0, off_s = 0, off_p = 0, bwd_bytes = 0;
    const int st = gla_plan_bwd(dir, H, W, o, &nchunks, &off_f, &off_r, &off_s, &off_p, &bwd_bytes);
    if (st != GLA_OK) return st;
    if (isnan(o->eps) || isinf(o->eps) || o->eps < 0.0f) return GLA_EINVAL;
    const size_t rows = (size_t)o->batch * H * W * o->heads;
    const size_t units = (size_t)o->batch * o->heads;
    lay->nchunks = nchunks;
    lay->off_f = off_f;
    lay->off_r = off_r;
    lay->off_s = off_s;
    lay->off_p = off_p;
    lay->bwd_bytes = bwd_bytes;
    lay->off_do = align256(bwd_bytes);
    lay->off_dwp = align256(lay->off_do + rows * o->dk * 4);
    lay->bytes = lay->off_dwp + units * nchunks * o->dk * 4;
    // d = 128: each quarter keeps its entering states from the o phase for
    // the gradient phase (three more arrays of the off_f part's size)
    lay->off_fq = 0;
    lay->fq_bytes = off_r - off_f;
    if (o->dk == 128) {
        lay->off_fq = align256(lay->bytes);
        lay->bytes = lay->off_fq + 3 * lay->fq_bytes;
    }
    return GLA_OK;
}

extern "C" int gla_validate_bwd_gated(const void* q, const void* k, const void* v, const float* z,
                                      const void* r, const void* dout, int dir, int H, int W,
                                      const void* dq, const void* dk, const void* dv, const float* dz,
                                      const void* dr, const float* dw, const gla_opts* o,
                                      gla_bwd_gated_layout* lay)
{
    if (!o || !q || !k || !v || !z || !r || !dout || !dq || !dk || !dv || !dz || !dr) return GLA_EINVAL;
    const int st = gla_plan_bwd_gated(dir, H, W, o, lay);
    if (st != GLA_OK) return st;
    const size_t es = o->dtype == GLA_F16 ? 2 : 4;
    const size_t n = (size_t)o->batch * H * W * o->heads * o->dk;
    const size_t wb = (size_t)o->dk * 4;
    const Operand ins[7] = {{q, n * es, 16},  {k, n * es, 16},    {v, n * es, 16},
                            {z, n * 4, 16},   {r, n * es, 16},    {dout, n * es, 16},
                            {o->norm_weight, wb, 16}};
    const Operand outs[6] = {{dq, n * es, 16}, {dk, n * es, 16}, {dv, n * es, 16},
                             {dz, n * 4, 16},  {dr, n * es, 16}, {dw, wb, 16}};
    for (int i = 0; i < 7; ++i)
        if (ins[i].p && !aligned(ins[i].p, 16)) return GLA_EINVAL;
    for (int i = 0; i < 6; ++i) {
        if (!outs[i].p) continue;
        if (!aligned(outs[i].p, 16)) return GLA_EINVAL;
        for (int j = 0; j < 7; ++j)
            if (ins[j].p && overlaps(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes)) return GLA_EINVAL;
        for (int j = 0; j < i; ++j)
            if (outs[j].p && overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return GLA_EINVAL;
    }
    if (!o->workspace || o->workspace_bytes < lay->bytes || !aligned(o->workspace, 16)) return GLA_EWORKSPACE;
    for (int i = 0; i < 7; ++i)
        if (ins[i].p && overlaps(o->workspace, lay->bytes, ins[i].p, ins[i].bytes)) return GLA_EINVAL;
    for (int i = 0; i < 6; ++i)
        if (outs[i].p && overlaps(o->workspace, lay->bytes, outs[i].p, outs[i].bytes)) return GLA_EINVAL;
    return GLA_OK;
}
