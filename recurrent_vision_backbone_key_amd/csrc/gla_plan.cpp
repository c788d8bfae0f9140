// gla_plan.cpp -- argument validation and work planning for gla_fwd.
// Compiled without HIP so that every error path can be exercised on a host
// without a GPU.
#include "gla_plan.h"

#include <math.h>
#include <stdint.h>

#include "gla_geometry.h"
#include "gla_launch.h"

namespace {

constexpr int kCUs = 256;          // compute units of one MI355X
constexpr int kXcds = 8;           // accelerator dies (XCDs), each with its own L2
constexpr int kCUsPerXcd = kCUs / kXcds;
// Single-pass workspace header: word 0 ticket counter, word 1 error word,
// word 16 (1 + x) ticket counter of XCD x.
constexpr size_t kOnePassHeader = 1024;
constexpr int kTargetGroups = 2 * kCUs;

bool is_pow2_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

extern "C" int gla_config_built(int dtype, int d, int chunk)
{
    if (dtype != GLA_F16 && dtype != GLA_F32) return 0;
    if (!is_pow2_dim(d) || !is_pow2_dim(chunk)) return 0;
    return gla::config_fits(dtype == GLA_F16 ? 2 : 4, d, chunk) ? 1 : 0;
}

extern "C" int gla_make_plan(int dir, int H, int W, int chunk, const gla_opts* o,
                             int has_gate, gla_plan* plan)
{
    if (!o || !plan) return GLA_EINVAL;
    if (o->batch < 1 || o->heads < 1 || H < 1 || W < 1) return GLA_EINVAL;
    if (dir < GLA_L2R || dir > GLA_B2T) return GLA_EINVAL;
    if (o->dtype != GLA_F16 && o->dtype != GLA_F32) return GLA_EUNSUPPORTED;
    if (!is_pow2_dim(o->dk) || !is_pow2_dim(o->dv) || o->dk != o->dv) return GLA_EUNSUPPORTED;
    if (!is_pow2_dim(chunk) || !gla_config_built(o->dtype, o->dk, chunk)) return GLA_EUNSUPPORTED;
    const int64_t L = (int64_t)H * W;
    if (L >= (int64_t)1 << 24) return GLA_EUNSUPPORTED;
    const int64_t rows = (int64_t)o->batch * L * o->heads;  // kernel row index is int32
    if (rows >= (int64_t)1 << 31) return GLA_EUNSUPPORTED;
    if (isnan(o->tau) || isnan(o->scale) || isinf(o->tau) || isinf(o->scale)) return GLA_EINVAL;
    if (has_gate && (isnan(o->eps) || o->eps < 0.0f || isinf(o->eps))) return GLA_EINVAL;

    const int nchunks = (int)((L + chunk - 1) / chunk);
    const int64_t units = (int64_t)o->batch * o->heads;
    if (o->algorithm < GLA_ALGO_AUTO || o->algorithm > GLA_ALGO_THREE_PASS) return GLA_EINVAL;
    plan->L = (int)L;
    plan->nchunks = nchunks;
    plan->onepass = 0;
    plan->off_done = plan->off_flags = plan->off_agg = plan->off_incl = 0;

    // Single pass: binary16, d = 64, 64-token chunks; segments of at most
    // kOnePassMaxChunks chunks, at most 65 segments per scan (one wavefront
    // of look-back), about one workgroup per compute unit.  When the scans
    // spread over the 8 XCDs without costing a second round of workgroups on
    // any of them (or divide evenly), scan u runs on XCD u mod 8 and the
    // segment exchange stays in that XCD's L2.
    const bool sp_shape = o->dtype == GLA_F16 && o->dk == 64 && o->dv == 64 && chunk == 64;
    plan->xcd_local = 0;
    plan->xcd_tasks = 0;
    if (o->algorithm != GLA_ALGO_THREE_PASS && sp_shape) {
        const int min_seg = (nchunks + 64) / 65;
        const int64_t upx = (units + kXcds - 1) / kXcds;  // scans per XCD (most)
        const int max_seg = nchunks < gla::kOnePassMaxChunks ? nchunks : gla::kOnePassMaxChunks;
        // the shortest segment whose workgroups fit in `slots` at `per` scans
        // (the longest allowed when none does)
        auto fit_seg = [&](int64_t per, int64_t slots) {
            for (int sg = min_seg; sg <= max_seg; ++sg)
                if (per * ((nchunks + sg - 1) / sg) <= slots) return sg;
            return max_seg;
        };
        const int seg_g = fit_seg(units, kCUs);
        const int seg_l = fit_seg(upx, kCUsPerXcd);
        int seg = o->segment_chunks;
        if (seg > nchunks) seg = nchunks;
        // XCD-local when it keeps segments as short as the chip-wide plan and
        // either fits one round per XCD or the scans divide evenly over XCDs
        const int seg_chk = seg > 0 ? seg : seg_l;
        const int64_t tasks = upx * ((nchunks + seg_chk - 1) / seg_chk);
        const bool local = (seg > 0 || seg_l <= seg_g) &&
                           (tasks <= kCUsPerXcd || units % kXcds == 0);
        if (seg <= 0) seg = local ? seg_l : seg_g;
        if (seg >= min_seg && seg <= gla::kOnePassMaxChunks) {
            const int nseg = (nchunks + seg - 1) / seg;
            const size_t nflag = (size_t)units * nseg;
            plan->onepass = 1;
            plan->seg_chunks = seg;
            plan->nseg = nseg;
            plan->xcd_local = local ? 1 : 0;
            plan->xcd_tasks = local ? (int)(upx * nseg) : 0;
            plan->off_done = kOnePassHeader;
            plan->off_flags = plan->off_done + (((size_t)units * 4 + 255) / 256) * 256;
            plan->off_agg = plan->off_flags + ((nflag * 4 + 255) / 256) * 256;
            plan->off_incl = plan->off_agg + nflag * ((size_t)64 * 64 + 64) * 4;
            plan->workspace_bytes = plan->off_incl + nflag * (size_t)64 * 64 * 4;
        }
    }
    if (!plan->onepass) {
        if (o->algorithm == GLA_ALGO_SINGLE_PASS) return GLA_EUNSUPPORTED;
        // Three passes: segments of seg_chunks chunks, enough workgroups for
        // the chip (the d = 128 binary16 chunk-64 kernels hold one workgroup
        // per compute unit: three full rounds).
        const bool wide = o->dtype == GLA_F16 && o->dk == 128 && chunk == 64;
        const int64_t target = wide ? 3 * kCUs : kTargetGroups;
        int seg = o->segment_chunks;
        if (seg <= 0) {
            const int64_t want = (units * nchunks + target - 1) / target;
            seg = (int)(want < 1 ? 1 : want);
        }
        if (seg > nchunks) seg = nchunks;
        const int nseg = (nchunks + seg - 1) / seg;
        plan->seg_chunks = seg;
        plan->nseg = nseg;
        plan->workspace_bytes =
            nseg > 1 ? (size_t)units * (nseg - 1) * ((size_t)o->dk * o->dv + o->dk) * 4 : 0;
    }
    plan->tau = o->tau > 0.0f ? o->tau : 16.0f;
    plan->scale = o->scale > 0.0f ? o->scale : (float)(1.0 / sqrt((double)o->dk));
    plan->eps = o->eps;
    return GLA_OK;
}

extern "C" int gla_validate(const void* q, const void* k, const void* v, const float* z,
                            int dir, int H, int W, int chunk, const void* out, const void* r,
                            const gla_opts* o, gla_plan* plan)
{
    if (!o || !plan) return GLA_EINVAL;
    if (!q || !k || !v || !z || !out) return GLA_EINVAL;
    const int st = gla_make_plan(dir, H, W, chunk, o, r != nullptr, plan);
    if (st != GLA_OK) return st;

    const size_t es = o->dtype == GLA_F16 ? 2 : 4;
    const size_t rows = (size_t)o->batch * plan->L * o->heads;
    const size_t nk = rows * o->dk, nv = rows * o->dv;
    const void* ins[6] = {q, k, v, z, r, r ? o->norm_weight : nullptr};
    const size_t insz[6] = {nk * es, nk * es, nv * es, nk * 4, nv * es, (size_t)o->dv * 4};
    for (int i = 0; i < 5; ++i)
        if (ins[i] && !aligned(ins[i], 16)) return GLA_EINVAL;
    if (!aligned(out, 16)) return GLA_EINVAL;
    if (ins[5] && !aligned(ins[5], 4)) return GLA_EINVAL;
    for (int i = 0; i < 6; ++i)
        if (overlaps(out, nv * es, ins[i], insz[i])) return GLA_EINVAL;

    if (plan->workspace_bytes) {
        if (!o->workspace || o->workspace_bytes < plan->workspace_bytes ||
            !aligned(o->workspace, 16))
            return GLA_EWORKSPACE;
        if (overlaps(o->workspace, plan->workspace_bytes, out, nv * es)) return GLA_EINVAL;
        for (int i = 0; i < 6; ++i)
            if (overlaps(o->workspace, plan->workspace_bytes, ins[i], insz[i])) return GLA_EINVAL;
    }
    return GLA_OK;
}
