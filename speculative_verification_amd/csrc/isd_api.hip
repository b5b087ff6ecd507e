// C-ABI entry points of libisd: argument validation, workspace layout, work
// decomposition and kernel launches.  Declarations and the contract are in
// include/isd.h.

#include "isd.h"
#include "isd_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

namespace isd {
namespace {

thread_local char g_err[512] = "";

isd_status_t fail(isd_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

std::atomic<int> g_segments{0};
std::atomic<int> g_propose_segments{0};
std::atomic<int> g_resid_segments{0};
std::atomic<int> g_trunc_segments{0};
// default decomposition (tiles of 2048 elements per workgroup segment)
// Verify rows are taken whole up to this many tiles, and cut further only
// while there are fewer than kMinVerifyItems verify items (so that a small
// batch still spreads over the chip).
constexpr int kVerifyTilesPerSeg = 96;
constexpr int kMinVerifyItems = 1024;
constexpr int kProposeTilesPerSeg = 19;
constexpr int kResidTilesPerSeg = 8;
// truncated path: split rows only as far as needed for about this many items
// (each item's warm-up costs more than a longer stream)
constexpr int kTruncTargetItems = 1024;
constexpr int kItemOrder = 0;
std::atomic<long long> g_spin_limit{0};
// Launch epochs: every launch that publishes decisions takes the next nonzero
// value, so decisions of two launches that share a workspace never match.
std::atomic<uint32_t> g_epoch{0};

uint32_t next_epoch() {
    uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    while (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    return e;
}
constexpr uint32_t kDefaultSpinLimit = 1u << 22;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

isd_status_t check_shape(const isd_shape_t *s, bool need_temperature) {
    if (!s) return fail(ISD_ERR_ARG, "shape pointer is NULL");
    if (s->dtype != ISD_DTYPE_BF16 && s->dtype != ISD_DTYPE_F32)
        return fail(ISD_ERR_UNSUPPORTED, "unknown dtype %d", (int)s->dtype);
    if (s->mode != ISD_MODE_SAMPLE && s->mode != ISD_MODE_GREEDY)
        return fail(ISD_ERR_UNSUPPORTED, "unknown mode %d", (int)s->mode);
    if (s->C < 1) return fail(ISD_ERR_ARG, "C must be >= 1 (got %d)", (int)s->C);
    if (s->L < 1 || s->L > kMaxL) return fail(ISD_ERR_ARG, "L must be in [1, 64] (got %d)", (int)s->L);
    if (s->V < 1) return fail(ISD_ERR_ARG, "V must be >= 1 (got %d)", (int)s->V);
    if (s->ld < (int64_t)s->V) return fail(ISD_ERR_ARG, "ld (%lld) must be >= V (%d)", (long long)s->ld, (int)s->V);
    if (s->ldc != 0 && s->ldc < (int64_t)s->L * s->ld)
        return fail(ISD_ERR_ARG, "ldc (%lld) must be 0 or >= L*ld (%lld)", (long long)s->ldc,
                    (long long)s->L * (long long)s->ld);
    const long long rows = (long long)s->C * s->L;
    if (rows > (1LL << 24)) return fail(ISD_ERR_ARG, "C*L too large (%lld)", rows);
    if (need_temperature && s->mode == ISD_MODE_SAMPLE &&
        !(isfinite(s->temperature) && s->temperature > 0.0f))
        return fail(ISD_ERR_ARG, "temperature must be finite and > 0 in sample mode");
    if (!(isfinite(s->relax) && s->relax >= 0.0f))
        return fail(ISD_ERR_ARG, "relax must be finite and >= 0");
    if (s->q_onehot != 0 && s->q_onehot != 1) return fail(ISD_ERR_ARG, "q_onehot must be 0 or 1");
    if (s->sampler != ISD_SAMPLER_CDF && s->sampler != ISD_SAMPLER_GUMBEL)
        return fail(ISD_ERR_ARG, "sampler must be 0 (inverse CDF) or 1 (Gumbel-max), got %d",
                    (int)s->sampler);
    if (s->top_k < 0) return fail(ISD_ERR_ARG, "top_k must be >= 0 (got %d)", (int)s->top_k);
    if (s->top_k > kMaxTopK)
        return fail(ISD_ERR_UNSUPPORTED, "top_k must be at most %d (got %d)", kMaxTopK, (int)s->top_k);
    if (!(isfinite(s->top_p) && s->top_p >= 0.0f))
        return fail(ISD_ERR_ARG, "top_p must be finite and >= 0 (0 or >= 1: off)");
    if (s->top_p > 0.0f && s->top_p < 1.0f && s->top_k == 0)
        return fail(ISD_ERR_UNSUPPORTED, "top_p needs top_k in [1, %d]", kMaxTopK);
    return ISD_OK;
}

size_t elem_size(const isd_shape_t *s) { return s->dtype == ISD_DTYPE_BF16 ? 2 : 4; }

// Sample-mode calls with top-k (and possibly top-p) take the truncated path.
bool truncated(const isd_shape_t *s) { return s->mode == ISD_MODE_SAMPLE && s->top_k > 0; }

isd_status_t check_ptr(const void *p, const char *name, size_t align) {
    if (!p) return fail(ISD_ERR_ARG, "%s is NULL", name);
    if (((uintptr_t)p) % align) return fail(ISD_ERR_ARG, "%s is not %zu-byte aligned", name, align);
    return ISD_OK;
}

#define ISD_TRY(expr)                      \
    do {                                   \
        isd_status_t st_ = (expr);         \
        if (st_ != ISD_OK) return st_;     \
    } while (0)

int64_t seq_stride(const isd_shape_t *s) { return s->ldc ? s->ldc : (int64_t)s->L * s->ld; }

bool vec_ok(const isd_shape_t *s, const void *a, const void *b, const void *c) {
    const size_t es = elem_size(s);
    if (s->V % kGroupElems) return false;   // the vector path takes whole 8-element groups only
    if (((size_t)s->ld * es) % 16) return false;
    if (((size_t)seq_stride(s) * es) % 16) return false;
    for (const void *p : {a, b, c})
        if (p && ((uintptr_t)p) % 16) return false;
    return true;
}

struct Plan {
    bool verify = false, propose = false, residual = false, verify_outputs = false;
    bool fused = false;   // statistics from the LM head: decide, residual items, propose
};

isd_status_t run(const isd_shape_t *s, const Plan &plan, StepArgs a, void *workspace,
                 size_t ws_bytes, void *stream) {
    const bool trunc = truncated(s);
    const WorkspaceLayout lay = workspace_layout(s->C, s->L, s->V, trunc);
    if (!workspace) return fail(ISD_ERR_ARG, "workspace is NULL");
    if (((uintptr_t)workspace) % 256) return fail(ISD_ERR_ARG, "workspace is not 256-byte aligned");
    if (ws_bytes < lay.total)
        return fail(ISD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, lay.total);

    const int C = s->C, L = s->L, V = s->V;
    const bool greedy = s->mode == ISD_MODE_GREEDY;
    a.C = C;
    a.L = L;
    a.V = V;
    a.ld = (long long)s->ld;
    a.ldc = (long long)seq_stride(s);
    a.k2 = greedy ? 1.0f : (float)(1.4426950408889634 / (double)s->temperature);
    a.ws = workspace_at(workspace, lay);
    a.tws = trunc_workspace_at(workspace, lay);
    a.tiles_row = ceil_div(V, kTileElems);

    // Segments per row.  Verify rows are dispatched first and can be large;
    // mask rows and residual rows come later and are cut finer so that the
    // last workgroups of the launch are short.
    a.smax = lay.smax;
    auto segs = [&](int want, int tiles_per_seg_target) {
        int S = want > 0 ? want : ceil_div(a.tiles_row, tiles_per_seg_target);
        return max(1, min(S, min(lay.smax, a.tiles_row)));
    };
    int Sv = segs(g_segments.load(), kVerifyTilesPerSeg);
    if (g_segments.load() <= 0) {
        const long long vrows = (long long)C * ((greedy || s->q_onehot) ? L : 2 * L);
        if (vrows * Sv < kMinVerifyItems)
            Sv = segs((int)((kMinVerifyItems + vrows - 1) / vrows), 0);
    }
    a.tps = ceil_div(a.tiles_row, Sv);
    a.S = ceil_div(a.tiles_row, a.tps);
    const int Sq = segs(g_propose_segments.load(), kProposeTilesPerSeg);
    a.tpsq = ceil_div(a.tiles_row, Sq);
    a.Sq = ceil_div(a.tiles_row, a.tpsq);
    int Sr = g_resid_segments.load();
    if (Sr <= 0) Sr = ceil_div(a.tiles_row, kResidTilesPerSeg);
    Sr = max(1, min(Sr, min(kMaxResidSegments, a.tiles_row)));
    a.tpsr = ceil_div(a.tiles_row, Sr);
    a.Sr = ceil_div(a.tiles_row, a.tpsr);
    a.order = kItemOrder;

    if (trunc) {
        // truncated path: every row is cut into St segments; no residual items
        a.q_onehot = s->q_onehot ? 1 : 0;
        a.relax1p = 1.0 + (double)s->relax;
        a.sampler = s->sampler == ISD_SAMPLER_GUMBEL ? 1 : 0;
        a.top_k = min((int)s->top_k, V);
        a.top_p = (s->top_p > 0.0f && s->top_p < 1.0f) ? (double)s->top_p : 1.0;
        a.temp = (double)s->temperature;
        a.rows_pq = plan.verify ? (s->q_onehot ? L : 2 * L) : 0;
        const int rows = C * (a.rows_pq + (plan.propose ? L : 0));
        int St = g_trunc_segments.load();
        if (St <= 0) St = ceil_div(kTruncTargetItems, max(rows, 1));
        St = max(1, min(St, min(kMaxTruncSegments, a.tiles_row)));
        a.tpst = ceil_div(a.tiles_row, St);
        a.St = ceil_div(a.tiles_row, a.tpst);
        const long long n_items =
            (long long)C * a.rows_pq * a.St + (plan.propose ? (long long)C * L * a.St : 0);
        if (n_items <= 0 || n_items >= (1LL << 31))
            return fail(ISD_ERR_ARG, "work decomposition out of range (%lld items)", n_items);
        a.n_items = (int)n_items;
        a.verify_outputs = plan.verify_outputs ? 1 : 0;
        const bool vec = vec_ok(s, a.p, a.q, a.qn);
        const hipError_t e = launch_trunc(a, s->dtype, vec, (hipStream_t)stream);
        if (e != hipSuccess)
            return fail(ISD_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
        return ISD_OK;
    }

    a.q_onehot = (!greedy && s->q_onehot) ? 1 : 0;
    a.relax1p = greedy ? 1.0 : 1.0 + (double)s->relax;
    a.sampler = (!greedy && s->sampler == ISD_SAMPLER_GUMBEL) ? 1 : 0;
    a.rows_pq = plan.fused ? 0 : plan.verify ? ((greedy || a.q_onehot) ? L : 2 * L) : 0;
    a.n_pq = C * a.rows_pq * a.S;
    a.q_blk = (plan.propose && !plan.fused) ? L * a.Sq : 0;
    a.r_blk = (plan.residual && !greedy) ? a.Sr : 0;
    const long long n_items = (long long)a.n_pq + (long long)C * (a.q_blk + a.r_blk);
    if (n_items <= 0 || n_items >= (1LL << 31))
        return fail(ISD_ERR_ARG, "work decomposition out of range (%lld items)", n_items);
    a.n_items = (int)n_items;
    a.verify_outputs = plan.verify_outputs ? 1 : 0;
    const long long spin = g_spin_limit.load();
    a.spin_limit = spin > 0 ? (uint32_t)(spin < (long long)UINT32_MAX ? spin : (long long)UINT32_MAX)
                            : kDefaultSpinLimit;
    a.epoch = next_epoch();

    const bool vec = vec_ok(s, a.p, a.q, a.qn);
    hipError_t e = hipSuccess;
    // the statistics path: decisions (and proposals, in the same launch when
    // it fits) before the residual items, which read the decisions
    const bool front = plan.fused && fused_front_fits(a);
    if (front) e = launch_fused_front(a, s->dtype, (hipStream_t)stream);
    else if (plan.fused) e = launch_fused_decide(a, s->dtype, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_step(a, s->dtype, s->mode, vec, (hipStream_t)stream);
    if (e == hipSuccess && plan.fused && !front) e = launch_fused_propose(a, s->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

StepArgs blank_args() {
    StepArgs a;
    memset(&a, 0, sizeof(a));
    return a;
}

}  // namespace

WorkspaceLayout workspace_layout(int C, int L, int V, bool trunc) {
    WorkspaceLayout lay;
    const size_t CL = (size_t)C * L;
    const int tiles_row = ceil_div(V, kTileElems);
    lay.smax = min(kMaxSegments, tiles_row);
    size_t off = align256(sizeof(Control));
    const size_t cs = sizeof(uint32_t) * kCounterStride;
    lay.off_seq_cnt = off;
    off = align256(off + cs * C);
    lay.off_res_cnt = off;
    off = align256(off + cs * C);
    lay.off_flag = off;
    off = align256(off + cs * C);
    lay.off_row_cnt = off;
    off = align256(off + cs * CL);
    lay.off_seg = off;
    off = align256(off + sizeof(SegRec) * 2 * CL * lay.smax);
    lay.off_tiles = off;
    off = align256(off + sizeof(TileRec) * CL * tiles_row);
    lay.off_rtiles = off;
    off = align256(off + sizeof(ResTile) * (size_t)C * tiles_row);
    lay.off_info = off;
    off = align256(off + sizeof(SeqInfo) * C);
    lay.off_garg = off;
    off = align256(off + sizeof(ArgRec) * 2 * (size_t)C * kMaxResidSegments);
    lay.trunc = trunc;
    lay.off_trow_cnt = lay.off_tseq_cnt = lay.off_tkeys = lay.off_tlists = lay.off_tpxq =
        lay.off_talpha = 0;
    if (trunc) {
        const int St = min(kMaxTruncSegments, tiles_row);
        lay.off_trow_cnt = off;
        off = align256(off + cs * 3 * CL);
        lay.off_tseq_cnt = off;
        off = align256(off + cs * C);
        lay.off_tkeys = off;
        off = align256(off + sizeof(uint64_t) * 3 * CL * St * kWave);
        lay.off_tlists = off;
        off = align256(off + sizeof(uint64_t) * 2 * CL * kWave * 2);
        lay.off_tpxq = off;
        off = align256(off + sizeof(uint64_t) * 2 * CL);
        lay.off_talpha = off;
        off = align256(off + sizeof(uint32_t) * C);
    }
    lay.total = off;
    return lay;
}

Workspace workspace_at(void *base, const WorkspaceLayout &lay) {
    char *b = static_cast<char *>(base);
    Workspace w;
    w.ctl = reinterpret_cast<Control *>(b);
    w.seq_cnt = reinterpret_cast<uint32_t *>(b + lay.off_seq_cnt);
    w.res_cnt = reinterpret_cast<uint32_t *>(b + lay.off_res_cnt);
    w.flag = reinterpret_cast<uint32_t *>(b + lay.off_flag);
    w.row_cnt = reinterpret_cast<uint32_t *>(b + lay.off_row_cnt);
    w.seg = reinterpret_cast<SegRec *>(b + lay.off_seg);
    w.arg = reinterpret_cast<ArgRec *>(b + lay.off_seg);
    w.tiles = reinterpret_cast<TileRec *>(b + lay.off_tiles);
    w.rtiles = reinterpret_cast<ResTile *>(b + lay.off_rtiles);
    w.info = reinterpret_cast<SeqInfo *>(b + lay.off_info);
    w.garg = reinterpret_cast<ArgRec *>(b + lay.off_garg);
    return w;
}

TruncWorkspace trunc_workspace_at(void *base, const WorkspaceLayout &lay) {
    char *b = static_cast<char *>(base);
    TruncWorkspace t;
    memset(&t, 0, sizeof(t));
    if (!lay.trunc) return t;
    t.row_cnt = reinterpret_cast<uint32_t *>(b + lay.off_trow_cnt);
    t.seq_cnt = reinterpret_cast<uint32_t *>(b + lay.off_tseq_cnt);
    t.keys = reinterpret_cast<uint64_t *>(b + lay.off_tkeys);
    t.lists = reinterpret_cast<uint64_t *>(b + lay.off_tlists);
    t.pxq = reinterpret_cast<uint64_t *>(b + lay.off_tpxq);
    t.alpha = reinterpret_cast<uint32_t *>(b + lay.off_talpha);
    return t;
}

}  // namespace isd

using namespace isd;

extern "C" {

size_t isd_workspace_bytes(const isd_shape_t *s) {
    if (check_shape(s, false) != ISD_OK) return 0;
    return workspace_layout(s->C, s->L, s->V, truncated(s)).total;
}

isd_status_t isd_verify_step(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                             const int32_t *proposals, const float *u_accept, const float *u_resid,
                             int32_t *accept_len, int32_t *out_tokens, int32_t *n_emitted,
                             float *p_x, float *q_x, float *alpha, void *workspace,
                             size_t ws_bytes, void *stream) {
    ISD_TRY(check_shape(s, true));
    const size_t es = elem_size(s);
    const bool sample = s->mode == ISD_MODE_SAMPLE;
    ISD_TRY(check_ptr(p_logits, "p_logits", es));
    if (sample) {
        if (!s->q_onehot) ISD_TRY(check_ptr(q_logits, "q_logits", es));
        ISD_TRY(check_ptr(u_accept, "u_accept", 4));
        ISD_TRY(check_ptr(u_resid, "u_resid", 4));
    }
    ISD_TRY(check_ptr(proposals, "proposals", 4));
    ISD_TRY(check_ptr(accept_len, "accept_len", 4));
    ISD_TRY(check_ptr(out_tokens, "out_tokens", 4));
    ISD_TRY(check_ptr(n_emitted, "n_emitted", 4));
    StepArgs a = blank_args();
    a.p = p_logits;
    a.q = (sample && !s->q_onehot) ? q_logits : nullptr;
    a.x = proposals;
    a.ua = sample ? u_accept : nullptr;
    a.ur = sample ? u_resid : nullptr;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.n_emitted = n_emitted;
    a.p_x = p_x;
    a.q_x = q_x;
    a.alpha = alpha;
    Plan plan;
    plan.verify = plan.residual = plan.verify_outputs = true;
    return run(s, plan, a, workspace, ws_bytes, stream);
}

isd_status_t isd_propose(const isd_shape_t *s, const void *qnext_logits, const float *u_propose,
                         int32_t *next_tokens, float *qnext_x, void *workspace, size_t ws_bytes,
                         void *stream) {
    return isd_propose_masked(s, qnext_logits, u_propose, nullptr, next_tokens, qnext_x, workspace,
                              ws_bytes, stream);
}

isd_status_t isd_propose_masked(const isd_shape_t *s, const void *qnext_logits,
                                const float *u_propose, const int32_t *mask,
                                int32_t *next_tokens, float *qnext_x, void *workspace,
                                size_t ws_bytes, void *stream) {
    ISD_TRY(check_shape(s, true));
    if (mask) ISD_TRY(check_ptr(mask, "mask", 4));
    const bool sample = s->mode == ISD_MODE_SAMPLE;
    ISD_TRY(check_ptr(qnext_logits, "qnext_logits", elem_size(s)));
    if (sample) ISD_TRY(check_ptr(u_propose, "u_propose", 4));
    ISD_TRY(check_ptr(next_tokens, "next_tokens", 4));
    StepArgs a = blank_args();
    a.qn = qnext_logits;
    a.up = sample ? u_propose : nullptr;
    a.next_tokens = next_tokens;
    a.qnext_x = qnext_x;
    a.pmask = mask;
    Plan plan;
    plan.propose = true;
    return run(s, plan, a, workspace, ws_bytes, stream);
}

isd_status_t isd_alpha(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                       const int32_t *proposals, float *alpha, float *alpha_mean, void *workspace,
                       size_t ws_bytes, void *stream) {
    ISD_TRY(check_shape(s, true));
    const bool sample = s->mode == ISD_MODE_SAMPLE;
    ISD_TRY(check_ptr(p_logits, "p_logits", elem_size(s)));
    if (sample && !s->q_onehot) ISD_TRY(check_ptr(q_logits, "q_logits", elem_size(s)));
    ISD_TRY(check_ptr(proposals, "proposals", 4));
    ISD_TRY(check_ptr(alpha, "alpha", 4));
    StepArgs a = blank_args();
    a.p = p_logits;
    a.q = (sample && !s->q_onehot) ? q_logits : nullptr;
    a.x = proposals;
    a.alpha = alpha;
    a.alpha_mean = alpha_mean;
    Plan plan;
    plan.verify = true;
    return run(s, plan, a, workspace, ws_bytes, stream);
}

isd_status_t isd_step(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                      const int32_t *proposals, const float *u_accept, const float *u_resid,
                      const void *qnext_logits, const float *u_propose, int32_t *accept_len,
                      int32_t *out_tokens, int32_t *n_emitted, float *p_x, float *q_x,
                      float *alpha, int32_t *next_tokens, float *qnext_x, void *workspace,
                      size_t ws_bytes, void *stream) {
    return isd_step_masked(s, p_logits, q_logits, proposals, u_accept, u_resid, qnext_logits,
                           u_propose, nullptr, nullptr, accept_len, out_tokens, n_emitted, p_x,
                           q_x, alpha, next_tokens, qnext_x, workspace, ws_bytes, stream);
}

}  // extern "C"

namespace isd {
namespace {

// Validates the arguments of a fused step and fills `a` with them.
isd_status_t step_args(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                       const int32_t *proposals, const float *u_accept, const float *u_resid,
                       const void *qnext_logits, const float *u_propose,
                       const int32_t *verify_mask, const int32_t *propose_mask,
                       int32_t *accept_len, int32_t *out_tokens, int32_t *n_emitted, float *p_x,
                       float *q_x, float *alpha, int32_t *next_tokens, float *qnext_x,
                       StepArgs &a) {
    ISD_TRY(check_shape(s, true));
    if (verify_mask) ISD_TRY(check_ptr(verify_mask, "verify_mask", 4));
    if (propose_mask) ISD_TRY(check_ptr(propose_mask, "propose_mask", 4));
    const size_t es = elem_size(s);
    const bool sample = s->mode == ISD_MODE_SAMPLE;
    ISD_TRY(check_ptr(p_logits, "p_logits", es));
    ISD_TRY(check_ptr(qnext_logits, "qnext_logits", es));
    if (sample) {
        if (!s->q_onehot) ISD_TRY(check_ptr(q_logits, "q_logits", es));
        ISD_TRY(check_ptr(u_accept, "u_accept", 4));
        ISD_TRY(check_ptr(u_resid, "u_resid", 4));
        ISD_TRY(check_ptr(u_propose, "u_propose", 4));
    }
    ISD_TRY(check_ptr(proposals, "proposals", 4));
    ISD_TRY(check_ptr(accept_len, "accept_len", 4));
    ISD_TRY(check_ptr(out_tokens, "out_tokens", 4));
    ISD_TRY(check_ptr(n_emitted, "n_emitted", 4));
    ISD_TRY(check_ptr(next_tokens, "next_tokens", 4));
    a = blank_args();
    a.p = p_logits;
    a.q = (sample && !s->q_onehot) ? q_logits : nullptr;
    a.qn = qnext_logits;
    a.x = proposals;
    a.ua = sample ? u_accept : nullptr;
    a.ur = sample ? u_resid : nullptr;
    a.up = sample ? u_propose : nullptr;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.n_emitted = n_emitted;
    a.p_x = p_x;
    a.q_x = q_x;
    a.alpha = alpha;
    a.next_tokens = next_tokens;
    a.qnext_x = qnext_x;
    a.vmask = verify_mask;
    a.pmask = propose_mask;
    return ISD_OK;
}

Plan step_plan() {
    Plan plan;
    plan.verify = plan.propose = plan.residual = plan.verify_outputs = true;
    return plan;
}

}  // namespace
}  // namespace isd

extern "C" {

isd_status_t isd_step_masked(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                             const int32_t *proposals, const float *u_accept,
                             const float *u_resid, const void *qnext_logits,
                             const float *u_propose, const int32_t *verify_mask,
                             const int32_t *propose_mask, int32_t *accept_len,
                             int32_t *out_tokens, int32_t *n_emitted, float *p_x, float *q_x,
                             float *alpha, int32_t *next_tokens, float *qnext_x, void *workspace,
                             size_t ws_bytes, void *stream) {
    StepArgs a;
    ISD_TRY(step_args(s, p_logits, q_logits, proposals, u_accept, u_resid, qnext_logits,
                      u_propose, verify_mask, propose_mask, accept_len, out_tokens, n_emitted,
                      p_x, q_x, alpha, next_tokens, qnext_x, a));
    return run(s, step_plan(), a, workspace, ws_bytes, stream);
}

isd_status_t isd_step_fused(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                            const int32_t *proposals, const float *u_accept, const float *u_resid,
                            const void *qnext_logits, const float *u_propose,
                            const float *p_stats, const float *q_stats, const float *qn_stats,
                            int64_t stats_ld, int64_t stats_ldc, int32_t *accept_len,
                            int32_t *out_tokens, int32_t *n_emitted, float *p_x, float *q_x,
                            float *alpha, int32_t *next_tokens, float *qnext_x, void *workspace,
                            size_t ws_bytes, void *stream) {
    ISD_TRY(check_shape(s, true));
    if (s->mode != ISD_MODE_SAMPLE)
        return fail(ISD_ERR_UNSUPPORTED, "the statistics path is for sample mode");
    if (s->top_k != 0) return fail(ISD_ERR_UNSUPPORTED, "the statistics path takes no top-k");
    const size_t es = elem_size(s);
    ISD_TRY(check_ptr(p_logits, "p_logits", es));
    ISD_TRY(check_ptr(qnext_logits, "qnext_logits", es));
    if (!s->q_onehot) {
        ISD_TRY(check_ptr(q_logits, "q_logits", es));
        ISD_TRY(check_ptr(q_stats, "q_stats", 8));
    }
    ISD_TRY(check_ptr(p_stats, "p_stats", 8));
    ISD_TRY(check_ptr(qn_stats, "qn_stats", 8));
    ISD_TRY(check_ptr(u_accept, "u_accept", 4));
    ISD_TRY(check_ptr(u_resid, "u_resid", 4));
    ISD_TRY(check_ptr(u_propose, "u_propose", 4));
    ISD_TRY(check_ptr(proposals, "proposals", 4));
    ISD_TRY(check_ptr(accept_len, "accept_len", 4));
    ISD_TRY(check_ptr(out_tokens, "out_tokens", 4));
    ISD_TRY(check_ptr(n_emitted, "n_emitted", 4));
    ISD_TRY(check_ptr(next_tokens, "next_tokens", 4));
    const int n_st = ceil_div(s->V, kStatsTile);
    if (stats_ld < n_st)
        return fail(ISD_ERR_ARG, "stats_ld (%lld) must be >= ceil(V / %d) = %d", (long long)stats_ld,
                    kStatsTile, n_st);
    if (stats_ldc == 0) stats_ldc = (int64_t)s->L * stats_ld;
    if (stats_ldc < (int64_t)s->L * stats_ld)
        return fail(ISD_ERR_ARG, "stats_ldc must be 0 or >= L * stats_ld");
    StepArgs a = blank_args();
    a.p = p_logits;
    a.q = s->q_onehot ? nullptr : q_logits;
    a.qn = qnext_logits;
    a.x = proposals;
    a.ua = u_accept;
    a.ur = u_resid;
    a.up = u_propose;
    a.p_stats = p_stats;
    a.q_stats = s->q_onehot ? nullptr : q_stats;
    a.qn_stats = qn_stats;
    a.s_ld = stats_ld;
    a.s_ldc = stats_ldc;
    a.n_stiles = n_st;
    a.accept_len = accept_len;
    a.out_tokens = out_tokens;
    a.n_emitted = n_emitted;
    a.p_x = p_x;
    a.q_x = q_x;
    a.alpha = alpha;
    a.next_tokens = next_tokens;
    a.qnext_x = qnext_x;
    Plan plan;
    plan.verify = plan.propose = plan.residual = plan.verify_outputs = plan.fused = true;
    return run(s, plan, a, workspace, ws_bytes, stream);
}

isd_status_t isd_lm_head_stats(const void *h, const void *wt, int32_t M, int32_t K, int32_t N,
                               float temperature, void *logits, float *stats, void *workspace,
                               size_t ws_bytes, void *stream) {
    ISD_TRY(check_ptr(h, "h", 16));
    ISD_TRY(check_ptr(wt, "wt", 16));
    ISD_TRY(check_ptr(logits, "logits", 2));
    ISD_TRY(check_ptr(stats, "stats", 8));
    if (workspace) ISD_TRY(check_ptr(workspace, "workspace", 256));
    if (M < 1 || N < 1 || K < 1) return fail(ISD_ERR_ARG, "M, K, N must be >= 1");
    if (K % 64) return fail(ISD_ERR_ARG, "K must be a multiple of 64 (got %d)", (int)K);
    if (!(isfinite(temperature) && temperature > 0.0f))
        return fail(ISD_ERR_ARG, "temperature must be finite and > 0");
    const float k2 = (float)(1.4426950408889634 / (double)temperature);
    const hipError_t e = launch_lm_head_stats(static_cast<const uint16_t *>(h),
                                              static_cast<const uint16_t *>(wt), M, K, N, k2,
                                              static_cast<uint16_t *>(logits), stats, workspace,
                                              workspace ? ws_bytes : 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "lm_head launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_lm_head(const void *h, const void *w, int32_t M, int32_t K, int32_t N,
                         void *logits, void *workspace, size_t ws_bytes, void *stream) {
    (void)workspace;
    (void)ws_bytes;
    ISD_TRY(check_ptr(h, "h", 16));
    ISD_TRY(check_ptr(w, "w", 16));
    ISD_TRY(check_ptr(logits, "logits", 16));
    if (M < 1 || N < 1 || K < 1) return fail(ISD_ERR_ARG, "M, K, N must be >= 1");
    if (K % 64) return fail(ISD_ERR_ARG, "K must be a multiple of 64 (got %d)", (int)K);
    if (N % 8) return fail(ISD_ERR_ARG, "N must be a multiple of 8 (got %d)", (int)N);
    const hipError_t e = launch_lm_head(static_cast<const uint16_t *>(h),
                                        static_cast<const uint16_t *>(w), M, K, N,
                                        static_cast<uint16_t *>(logits), (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "lm_head launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_lm_head_pack(const void *w, int32_t K, int32_t N, void *wt, void *stream) {
    ISD_TRY(check_ptr(w, "w", 2));
    ISD_TRY(check_ptr(wt, "wt", 16));
    if (K < 1 || N < 1) return fail(ISD_ERR_ARG, "K, N must be >= 1");
    const hipError_t e = launch_pack_wt(static_cast<const uint16_t *>(w), static_cast<uint16_t *>(wt),
                                        K, N, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "pack launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

size_t isd_gemm_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    if (M < 1 || N < 1 || K < 64 || K % 64) return 0;
    return gemm_workspace_bytes(M, K, N);
}

isd_status_t isd_lm_head_packed(const void *h, const void *wt, int32_t M, int32_t K, int32_t N,
                                void *logits, void *workspace, size_t ws_bytes, void *stream) {
    ISD_TRY(check_ptr(h, "h", 16));
    ISD_TRY(check_ptr(wt, "wt", 16));
    ISD_TRY(check_ptr(logits, "logits", 2));
    if (workspace) ISD_TRY(check_ptr(workspace, "workspace", 256));
    if (M < 1 || N < 1 || K < 1) return fail(ISD_ERR_ARG, "M, K, N must be >= 1");
    if (K % 64) return fail(ISD_ERR_ARG, "K must be a multiple of 64 (got %d)", (int)K);
    const hipError_t e = launch_lm_head_packed(static_cast<const uint16_t *>(h),
                                               static_cast<const uint16_t *>(wt), M, K, N,
                                               static_cast<uint16_t *>(logits), workspace,
                                               workspace ? ws_bytes : 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "lm_head launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_decode_masks(int32_t C, int32_t L, const int32_t *state,
                              const int32_t *accept_len, int32_t *bonus_mask,
                              int32_t *anchor_mask, void *stream) {
    if (C < 1) return fail(ISD_ERR_ARG, "C must be >= 1 (got %d)", (int)C);
    if (L < 1 || L > kMaxL) return fail(ISD_ERR_ARG, "L must be in [1, 64] (got %d)", (int)L);
    ISD_TRY(check_ptr(state, "state", 4));
    ISD_TRY(check_ptr(accept_len, "accept_len", 4));
    ISD_TRY(check_ptr(bonus_mask, "bonus_mask", 4));
    ISD_TRY(check_ptr(anchor_mask, "anchor_mask", 4));
    const hipError_t e = launch_decode_masks(C, L, state, accept_len, bonus_mask, anchor_mask,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_decode_commit(int32_t C, int32_t L, int32_t *state, const int32_t *accept_len,
                               const int32_t *out_tokens, const int32_t *bonus,
                               const int32_t *anchor, int32_t *history, int64_t hist_cap,
                               int64_t *tokens, int64_t *forwards, void *stream) {
    if (C < 1) return fail(ISD_ERR_ARG, "C must be >= 1 (got %d)", (int)C);
    if (L < 1 || L > kMaxL) return fail(ISD_ERR_ARG, "L must be in [1, 64] (got %d)", (int)L);
    ISD_TRY(check_ptr(state, "state", 4));
    ISD_TRY(check_ptr(accept_len, "accept_len", 4));
    ISD_TRY(check_ptr(out_tokens, "out_tokens", 4));
    ISD_TRY(check_ptr(bonus, "bonus", 4));
    ISD_TRY(check_ptr(anchor, "anchor", 4));
    ISD_TRY(check_ptr(tokens, "tokens", 8));
    ISD_TRY(check_ptr(forwards, "forwards", 8));
    if (hist_cap < 0) return fail(ISD_ERR_ARG, "hist_cap must be >= 0");
    if (hist_cap > 0) ISD_TRY(check_ptr(history, "history", 4));
    const hipError_t e = launch_decode_commit(C, L, state, accept_len, out_tokens, bonus, anchor,
                                              hist_cap > 0 ? history : nullptr, hist_cap, tokens,
                                              forwards, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_check_device_error(void *workspace, size_t ws_bytes, void *stream) {
    if (!workspace) return fail(ISD_ERR_ARG, "workspace is NULL");
    if (ws_bytes < sizeof(Control)) return fail(ISD_ERR_WORKSPACE, "workspace too small");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "stream sync failed: %s", hipGetErrorString(e));
    Control *ctl = static_cast<Control *>(workspace);
    uint32_t err = 0;
    e = hipMemcpy(&err, &ctl->error, sizeof(err), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "reading the error word failed: %s", hipGetErrorString(e));
    if (!err) return ISD_OK;
    const uint32_t zero = 0;
    e = hipMemcpy(&ctl->error, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "clearing the error word failed: %s", hipGetErrorString(e));
    return fail(ISD_ERR_DEVICE, "device error word 0x%x:%s%s%s", err,
                (err & kErrBadToken) ? " proposal id out of range;" : "",
                (err & kErrEmptyRow) ? " logits row without a finite value;" : "",
                (err & kErrWaitExpired) ? " cross-workgroup wait expired;" : "");
}

isd_status_t isd_set_tuning(int32_t segments, int32_t propose_segments, int32_t resid_segments,
                            int64_t spin_limit) {
    if (segments < 0 || segments > kMaxSegments)
        return fail(ISD_ERR_ARG, "segments must be in [0, %d]", kMaxSegments);
    if (propose_segments < 0 || propose_segments > kMaxSegments)
        return fail(ISD_ERR_ARG, "propose_segments must be in [0, %d]", kMaxSegments);
    if (resid_segments < 0 || resid_segments > kMaxResidSegments)
        return fail(ISD_ERR_ARG, "resid_segments must be in [0, %d]", kMaxResidSegments);
    if (spin_limit < 0) return fail(ISD_ERR_ARG, "spin_limit must be >= 0");
    g_segments.store(segments);
    g_propose_segments.store(propose_segments);
    g_resid_segments.store(resid_segments);
    g_spin_limit.store(spin_limit);
    return ISD_OK;
}

isd_status_t isd_lora_pack(const void *w, const void *b, int32_t N, int32_t K, int32_t r,
                           void *wcat, void *stream) {
    ISD_TRY(check_ptr(w, "w", 2));
    ISD_TRY(check_ptr(b, "b", 2));
    ISD_TRY(check_ptr(wcat, "wcat", 2));
    if (N < 1 || K < 1 || r < 1) return fail(ISD_ERR_ARG, "N, K, r must be >= 1");
    const size_t pitch = (size_t)(K + r) * 2;
    hipError_t e = hipMemcpy2DAsync(wcat, pitch, w, (size_t)K * 2, (size_t)K * 2, (size_t)N,
                                    hipMemcpyDeviceToDevice, (hipStream_t)stream);
    if (e == hipSuccess)
        e = hipMemcpy2DAsync(static_cast<char *>(wcat) + (size_t)K * 2, pitch, b, (size_t)r * 2,
                             (size_t)r * 2, (size_t)N, hipMemcpyDeviceToDevice,
                             (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "lora pack copy failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_lora_gemm(const void *x, const void *a, const void *wcat, const int32_t *mask,
                           int32_t M, int32_t K, int32_t N, int32_t r, void *t, void *out,
                           void *workspace, size_t ws_bytes, void *stream) {
    ISD_TRY(check_ptr(x, "x", 16));
    ISD_TRY(check_ptr(a, "a", 16));
    ISD_TRY(check_ptr(wcat, "wcat", 16));
    ISD_TRY(check_ptr(t, "t", 16));
    ISD_TRY(check_ptr(out, "out", 2));
    if (mask) ISD_TRY(check_ptr(mask, "mask", 4));
    if (workspace) ISD_TRY(check_ptr(workspace, "workspace", 256));
    if (M < 1 || N < 1 || K < 1 || r < 1) return fail(ISD_ERR_ARG, "M, K, N, r must be >= 1");
    if (K % 64) return fail(ISD_ERR_ARG, "K must be a multiple of 64 (got %d)", (int)K);
    if (r % 64) return fail(ISD_ERR_ARG, "r must be a multiple of 64 (got %d)", (int)r);
    const hipError_t e = launch_lora_gemm(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(a),
        static_cast<const uint16_t *>(wcat), mask, M, K, N, r, static_cast<uint16_t *>(t),
        static_cast<uint16_t *>(out), workspace, workspace ? ws_bytes : 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "lora launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

isd_status_t isd_set_trunc_tuning(int32_t segments) {
    if (segments < 0 || segments > kMaxTruncSegments)
        return fail(ISD_ERR_ARG, "segments must be in [0, %d]", kMaxTruncSegments);
    g_trunc_segments.store(segments);
    return ISD_OK;
}

isd_status_t isd_read_probe(const void *buf, size_t bytes, int32_t tiles_per_group,
                            uint32_t *sink, void *stream) {
    ISD_TRY(check_ptr(buf, "buf", 16));
    ISD_TRY(check_ptr(sink, "sink", 4));
    const size_t tile_bytes = (size_t)kTileElems * 2;
    if (bytes == 0 || bytes % tile_bytes)
        return fail(ISD_ERR_ARG, "bytes must be a positive multiple of %zu", tile_bytes);
    if (bytes / tile_bytes > (size_t)INT32_MAX / kTileElems)
        return fail(ISD_ERR_ARG, "bytes too large (%zu)", bytes);
    if (tiles_per_group < 1 || tiles_per_group > 4096)
        return fail(ISD_ERR_ARG, "tiles_per_group must be in [1, 4096]");
    const hipError_t e = launch_read_probe(buf, (long long)(bytes / tile_bytes), tiles_per_group,
                                           sink, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "probe launch failed: %s", hipGetErrorString(e));
    return ISD_OK;
}

const char *isd_last_error(void) { return g_err; }

}  // extern "C"

// ---------------------------------------------------------------------------
// The fused step without a caller workspace
// ---------------------------------------------------------------------------
//
// Its kernels keep their counters and partial results in `scratch`, a
// file-scope device array of fixed size instead of a workspace argument.
// Each device that runs the library holds its own copy until the process
// ends.  In host code the array's name only stands for the symbol: the
// device address comes from hipGetSymbolAddress, taken once per device at
// that device's first call and kept in scratch_ptr; every kernel argument
// and copy uses that address.

namespace isd {
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxScratchDevices = 64;
}  // namespace isd

static __device__ __align__(256) unsigned char scratch[isd::kScratchBytes];

namespace isd {
namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

__global__ void scratch_clear_kernel(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Moves the device error word of the scratch to *out and clears it.
__global__ void scratch_take_error_kernel(Control *ctl, uint32_t *out) {
    if (threadIdx.x == 0) {
        const uint32_t e = __hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl->error, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *out = e;
    }
}

// The current device's scratch address.  The first call on a device takes
// the symbol's address and zero-fills the array (a kernel on the null
// stream, waited for, so that every later launch on any stream sees zeros).
isd_status_t current_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ISD_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(ISD_ERR_UNSUPPORTED, "device %d: the allocation-free step serves devices 0..%d",
                    dev, kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(ISD_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(1024), dim3(256), 0, (hipStream_t)0,
                           static_cast<uint4 *>(ptr), kScratchBytes / 16);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)0);
        if (e != hipSuccess)
            return fail(ISD_ERR_DEVICE, "clearing the scratch failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ISD_OK;
}

}  // namespace
}  // namespace isd

extern "C" isd_status_t isd_step_noalloc(const isd_shape_t *s, const void *p_logits,
                                         const void *q_logits, const int32_t *proposals,
                                         const float *u_accept, const float *u_resid,
                                         const void *qnext_logits, const float *u_propose,
                                         int32_t *accept_len, int32_t *out_tokens,
                                         int32_t *n_emitted, float *p_x, float *q_x, float *alpha,
                                         int32_t *next_tokens, float *qnext_x,
                                         uint32_t *device_error, void *stream) {
    StepArgs a;
    ISD_TRY(step_args(s, p_logits, q_logits, proposals, u_accept, u_resid, qnext_logits,
                      u_propose, nullptr, nullptr, accept_len, out_tokens, n_emitted, p_x, q_x,
                      alpha, next_tokens, qnext_x, a));
    if (device_error) ISD_TRY(check_ptr(device_error, "device_error", 4));
    const size_t need = workspace_layout(s->C, s->L, s->V, truncated(s)).total;
    if (need > kScratchBytes)
        return fail(ISD_ERR_WORKSPACE,
                    "this shape needs %zu bytes of scratch; the allocation-free step holds %zu "
                    "(use isd_step with a workspace)", need, kScratchBytes);
    void *ws = nullptr;
    ISD_TRY(current_scratch(&ws));
    ISD_TRY(run(s, step_plan(), a, ws, kScratchBytes, stream));
    if (device_error) {
        hipLaunchKernelGGL(scratch_take_error_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                           static_cast<Control *>(ws), device_error);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(ISD_ERR_DEVICE, "error-word launch failed: %s", hipGetErrorString(e));
    }
    return ISD_OK;
}
