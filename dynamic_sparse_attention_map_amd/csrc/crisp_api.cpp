// C ABI of the CRISP sparse-prefill library: argument validation, workspace
// carving and kernel launches.  Declared in include/crisp.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <vector>

#include "crisp.h"
#include "crisp_kernels.h"

using namespace crisp;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Shape {
    int n, hq, hkv, nb, G;
};

// Workspace layout.  The scratch region S is shared by the route partials,
// the select scratch and the transposed V (stages run in that order on one
// stream); region P after it holds crisp_prefill's intermediates.  Up to
// kSelectSmall key blocks crisp_prefill lays V^T out during the selection
// launch, so its V^T (vt_pf, queue_pf) then follows the selection scratch;
// the attention-only calls keep theirs at the start of S.
struct Layout {
    size_t part_m, part_lo, part_up, jsd_kbar, jsd_qbar;   // route (in S)
    size_t seg_m, seg_l, row_mx, row_inv, tile_sums;       // route reduction (in S)
    size_t qbar, kbar, abar, hist_mass, hist_count, pass_ctr, state, bitmap, rowmask;   // select (in S)
    size_t vt, queue;                                      // attend (in S)
    size_t vt_pf, queue_pf;                                // crisp_prefill's attend (in S)
    size_t route_end, select_end, attend_end;              // bytes of S each stage needs
    size_t pattern, c_struct, p_v, p_s, sel_v, sel_s, counts, row_ptr, col_idx;  // P
    size_t total;
    int64_t csr_capacity;
};

Layout make_layout(const Shape& s)
{
    Layout L{};
    const size_t hq = s.hq, hkv = s.hkv, nb = s.nb;
    const size_t tri = nb * (nb + 1) / 2;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    const size_t part = hq * nb * kB * sizeof(float);
    L.part_m = take(part);
    L.part_lo = take(part);
    L.part_up = take(part);
    L.jsd_kbar = take(hkv * nb * kD * sizeof(float));      // JSD router only
    L.jsd_qbar = take(hq * kD * sizeof(float));
    // the multi-launch route reductions' scratch (unused up to kRouteSmall blocks)
    const size_t rs = nb > (size_t)kRouteSmall ? 1 : 0;
    L.seg_m = take(rs * hq * kRouteSegs * kB * sizeof(float));
    L.seg_l = take(rs * hq * kRouteSegs * kB * sizeof(double));
    L.row_mx = take(rs * hq * kB * sizeof(float));
    L.row_inv = take(rs * hq * kB * sizeof(float));
    L.tile_sums = take(rs * hq * 4 * nb * sizeof(float));
    L.route_end = o;
    o = 0;
    L.qbar = take(hq * nb * kD * sizeof(float));
    L.kbar = take(hkv * nb * kD * sizeof(float));
    L.abar = take(hq * tri * sizeof(float));
    // the multi-launch radix select's histograms and the expansion's
    // membership ballots (unused for small maps)
    const size_t rx = tri > (size_t)kRadixSmall ? 1 : 0;
    L.hist_mass = take(rx * hq * kValPasses * kValBins * sizeof(unsigned long long));
    L.hist_count = take(rx * hq * kRadixPasses * kFlatBins * sizeof(uint32_t));
    L.pass_ctr = take(rx * hq * kRadixPasses * sizeof(uint32_t));
    L.state = take(hq * sizeof(PeState));
    L.bitmap = take(hq * 2 * nb);
    L.rowmask = take(rx * hq * nb * ((nb + 63) / 64) * sizeof(unsigned long long));
    L.select_end = o;
    o = 0;
    L.vt = take(hkv * kD * (nb * kB) * sizeof(uint16_t));     // V^T padded to N_b blocks
    L.queue = take(8 * sizeof(int));
    L.attend_end = o;
    if (select_lays_out_v(s.nb)) {
        o = L.select_end;
        L.vt_pf = take(hkv * kD * (nb * kB) * sizeof(uint16_t));
        L.queue_pf = take(8 * sizeof(int));
    } else {
        L.vt_pf = L.vt;
        L.queue_pf = L.queue;
    }
    o = std::max(o, L.route_end);
    if (L.select_end > o) o = L.select_end;
    if (L.attend_end > o) o = L.attend_end;
    if (s.nb > kSelectSmall) {
        // never less than a shorter layer needs (a workspace sized for the
        // longest sequence serves every shorter one): at least S of N_b =
        // kSelectSmall, where V^T follows the selection scratch
        Shape t = s;
        t.nb = kSelectSmall;
        t.n = kSelectSmall * kB;
        o = std::max(o, make_layout(t).pattern);
    }
    L.pattern = take(hq);
    L.c_struct = take(hq * sizeof(float));
    L.p_v = take(hq * nb * sizeof(float));
    L.p_s = take(hq * nb * sizeof(float));
    L.sel_v = take(hq * nb * sizeof(int32_t));
    L.sel_s = take(hq * nb * sizeof(int32_t));
    L.counts = take(hq * 3 * sizeof(int32_t));
    L.row_ptr = take(hq * (nb + 1) * sizeof(int32_t));
    L.csr_capacity = (int64_t)(hq * tri);
    L.col_idx = take(hq * tri * sizeof(int32_t));
    L.total = o;
    return L;
}

int check_shape(int seq_len, int n_heads, int n_kv_heads, int head_dim, int block_size, Shape* s)
{
    if (head_dim != kD || block_size != kB) return CRISP_ERR_UNSUPPORTED;
    if (seq_len < 0 || n_heads <= 0 || n_kv_heads <= 0) return CRISP_ERR_SHAPE;
    if (n_heads % n_kv_heads != 0) return CRISP_ERR_SHAPE;
    // N_b = ceil(n / B): the last block may be partial; n = 0 is an empty call
    const int nb = (int)(((long long)seq_len + block_size - 1) / block_size);
    if (nb > kMaxBlocks) return CRISP_ERR_UNSUPPORTED;
    const long long tri = (long long)nb * (nb + 1) / 2;
    if ((long long)n_heads * tri >= (1LL << 31)) return CRISP_ERR_UNSUPPORTED;
    s->n = seq_len;
    s->hq = n_heads;
    s->hkv = n_kv_heads;
    s->nb = nb;
    s->G = n_heads / n_kv_heads;
    return CRISP_OK;
}

bool bad_ptr(const void* p, size_t align = 16)
{
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) % align) != 0;
}

struct Opts {
    float tau, gamma, tau_jsd, gamma_vs;
    int kmin_blocks, router, vs_rule, dense_below;
};

constexpr crisp_opts kDefaults = {0.2f, 0.95f, 1024, kB, kB, CRISP_ROUTER_CSTRUCT, 0.1f,
                                  CRISP_VS_NOISE_MEAN, 0.95f, 0};

int check_opts(const crisp_opts* o, Opts* out)
{
    const crisp_opts d = o ? *o : kDefaults;
    if (!std::isfinite(d.tau_proxy) || !std::isfinite(d.tau_jsd)) return CRISP_ERR_INVALID_ARG;
    if (!(d.gamma > 0.0f && d.gamma <= 1.0f)) return CRISP_ERR_INVALID_ARG;
    if (!(d.gamma_vs > 0.0f && d.gamma_vs <= 1.0f)) return CRISP_ERR_INVALID_ARG;
    if (d.k_min_tokens < 0 || d.k_min_tokens % kB != 0) return CRISP_ERR_INVALID_ARG;
    if (d.router != CRISP_ROUTER_CSTRUCT && d.router != CRISP_ROUTER_JSD) return CRISP_ERR_INVALID_ARG;
    if (d.vs_rule < CRISP_VS_NOISE_MEAN || d.vs_rule > CRISP_VS_GAMMA) return CRISP_ERR_INVALID_ARG;
    if (d.dense_below_tokens < 0) return CRISP_ERR_INVALID_ARG;
    if (d.w_sink != kB || d.w_local != kB) return CRISP_ERR_UNSUPPORTED;
    out->tau = d.tau_proxy;
    out->gamma = d.gamma;
    out->tau_jsd = d.tau_jsd;
    out->gamma_vs = d.gamma_vs;
    out->kmin_blocks = d.k_min_tokens / kB;
    out->router = d.router;
    out->vs_rule = d.vs_rule;
    out->dense_below = d.dense_below_tokens;
    return CRISP_OK;
}

// Q, K, V and the output of one sequence with their strides.
struct Operands {
    Rows q, k, v;
    OutRows out;
};

// [H][n][128] contiguous
Rows packed(const void* p, int n)
{
    return Rows{static_cast<const uint16_t*>(p), (long long)n * kD, kD};
}
OutRows packed_out(void* p, int n)
{
    return OutRows{static_cast<uint16_t*>(p), (long long)n * kD, kD};
}

thread_local hipEvent_t g_events[5];
thread_local bool g_events_on = false;

void mark(int i, hipStream_t stream)
{
    if (g_events_on) (void)hipEventRecord(g_events[i], stream);
}

int hip_status(hipError_t e) { return e == hipSuccess ? CRISP_OK : CRISP_ERR_HIP; }

template <typename T>
T* at(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

template <class R>
int do_route(const Shape& s, const Opts& op, R q, R k, void* ws,
             const Layout& L, uint8_t* pattern, float* c_struct, float* p_v, float* p_s,
             hipStream_t stream)
{
    RouteArgs ra;
    ra.router = op.router;
    ra.tau = op.router == CRISP_ROUTER_JSD ? op.tau_jsd : op.tau;
    ra.part_m = at<float>(ws, L.part_m);
    ra.part_lo = at<float>(ws, L.part_lo);
    ra.part_up = at<float>(ws, L.part_up);
    ra.jsd_kbar = at<float>(ws, L.jsd_kbar);
    ra.jsd_qbar = at<float>(ws, L.jsd_qbar);
    ra.seg_m = at<float>(ws, L.seg_m);
    ra.seg_l = at<double>(ws, L.seg_l);
    ra.row_mx = at<float>(ws, L.row_mx);
    ra.row_inv = at<float>(ws, L.row_inv);
    ra.tile_sums = at<float>(ws, L.tile_sums);
    return hip_status(launch_route(q, k, s.n, s.hq, s.hkv, ra, p_v, p_s, c_struct, pattern, stream));
}

template <class R>
int do_select(const Shape& s, const Opts& op, float alpha, R q, R k,
              const uint8_t* pattern, const float* p_v, const float* p_s, void* ws,
              const Layout& L, int32_t* sel_v, int32_t* sel_s, int32_t* counts,
              int32_t* row_ptr, int32_t* col_idx, const VtJob<R>& vt, hipStream_t stream)
{
    SelectScratch sc;
    sc.qbar = at<float>(ws, L.qbar);
    sc.kbar = at<float>(ws, L.kbar);
    sc.abar = at<float>(ws, L.abar);
    sc.hist_mass = at<unsigned long long>(ws, L.hist_mass);
    sc.hist_count = at<uint32_t>(ws, L.hist_count);
    sc.pass_ctr = at<uint32_t>(ws, L.pass_ctr);
    sc.state = at<PeState>(ws, L.state);
    sc.bitmap = at<uint8_t>(ws, L.bitmap);
    sc.rowmask = at<unsigned long long>(ws, L.rowmask);
    VsRule vr;
    vr.rule = op.vs_rule;
    vr.alpha = alpha;
    vr.gamma_vs = op.gamma_vs;
    vr.kmin_blocks = op.kmin_blocks;
    return hip_status(launch_select(q, k, pattern, p_v, p_s, s.n, s.hq, s.hkv, vr, op.gamma, sc,
                                    sel_v, sel_s, counts, row_ptr, col_idx, vt, stream));
}

// vt_ready: V^T and the cleared queue are already in place (the selection
// launch laid them out).
int do_attend(const Shape& s, const Operands& x, const int32_t* row_ptr, const int32_t* col_idx,
              uint16_t* vt, int* queue, bool vt_ready, hipStream_t stream)
{
    mark(2, stream);
    hipError_t e = hipSuccess;
    if (!vt_ready && (e = launch_v_transpose(x.v, s.n, s.hkv, vt, queue, stream)) != hipSuccess)
        return CRISP_ERR_HIP;
    mark(3, stream);
    e = launch_attend(x.q, x.k, vt, row_ptr, col_idx, s.n, s.hq, s.hkv, queue, x.out, stream);
    mark(4, stream);
    return hip_status(e);
}

int do_attend(const Shape& s, const Operands& x, const int32_t* row_ptr, const int32_t* col_idx,
              void* ws, const Layout& L, hipStream_t stream)
{
    return do_attend(s, x, row_ptr, col_idx, at<uint16_t>(ws, L.vt), at<int>(ws, L.queue), false,
                     stream);
}

// Alg. 1 for one sequence: route, select, attend; or, below the gating
// length, dense causal attention alone.
int run_prefill(const Shape& s, const Opts& op, float alpha, const Operands& x, void* ws,
                const Layout& L, hipStream_t st)
{
    if (s.n < op.dense_below) {
        mark(0, st);
        mark(1, st);
        return do_attend(s, x, nullptr, nullptr, ws, L, st);
    }
    uint8_t* pattern = at<uint8_t>(ws, L.pattern);
    float* p_v = at<float>(ws, L.p_v);
    float* p_s = at<float>(ws, L.p_s);
    int32_t* row_ptr = at<int32_t>(ws, L.row_ptr);
    int32_t* col_idx = at<int32_t>(ws, L.col_idx);
    mark(0, st);
    int rc = do_route(s, op, x.q, x.k, ws, L, pattern, at<float>(ws, L.c_struct), p_v, p_s, st);
    if (rc) return rc;
    mark(1, st);
    uint16_t* vt = at<uint16_t>(ws, L.vt_pf);
    int* queue = at<int>(ws, L.queue_pf);
    const bool fused = select_lays_out_v(s.nb);
    const VtJob<Rows> job{x.v, fused ? vt : nullptr, queue};
    rc = do_select(s, op, alpha, x.q, x.k, pattern, p_v, p_s, ws, L, at<int32_t>(ws, L.sel_v),
                   at<int32_t>(ws, L.sel_s), at<int32_t>(ws, L.counts), row_ptr, col_idx, job, st);
    if (rc) return rc;
    return do_attend(s, x, row_ptr, col_idx, vt, queue, fused, st);
}

// element strides: positive, rows 16-byte aligned
bool bad_strides(long long sh, long long st)
{
    return sh <= 0 || st <= 0 || sh % 8 != 0 || st % 8 != 0;
}

// crisp_prefill_batch's single-launch path works on groups: the sequences
// of one length form a group, routed, selected and re-laid out as one layer
// of count * n_heads query and count * n_kv_heads KV heads (sequence i of
// the group owns heads i * n_heads .. and i * n_kv_heads ..), reading its
// rows through per-sequence base pointers; then one attention launch covers
// every sequence.  Workspace: the routing / selection scratch region S at
// offset 0 (one group at a time), then per group its intermediates (region
// P of the group's layout), its V^T images and three pointer tables, then
// the sequence table, the queue-slot map and the queue counters.
struct BatchGroup {
    int n;
    std::vector<int> seqs;        // indices into the batch, in batch order
    size_t p_base, vt_base, qtab, ktab, vtab;
};
struct BatchLayout {
    std::vector<BatchGroup> groups;
    std::vector<int> run, per_xcd, slot0, pair_major;   // per batch entry
    size_t table = 0, slot_seq = 0, counters = 0, total = 0;
    int total_per_xcd = 0;
};

// the group's layer shape (validated lengths)
Shape group_shape(const BatchGroup& g, int hq, int hkv)
{
    Shape s;
    const int c = (int)g.seqs.size();
    (void)check_shape(g.n, hq * c, hkv * c, kD, kB, &s);
    return s;
}

template <typename LenOf>
BatchLayout make_batch_layout(int batch, LenOf len_of, int hq, int hkv)
{
    BatchLayout B;
    for (int b = 0; b < batch; ++b) {
        const int n = len_of(b);
        if (n == 0) continue;
        // a group's layer must stay within the shape limits of one call
        // (n_heads * N_b (N_b + 1) / 2 list entries below 2^31)
        const long long nb = (n + kB - 1) / kB;
        const long long cap = std::max(1LL, ((1LL << 31) - 1) / ((long long)hq * (nb * (nb + 1) / 2)));
        auto it = std::find_if(B.groups.begin(), B.groups.end(), [&](const BatchGroup& g) {
            return g.n == n && (long long)g.seqs.size() < cap;
        });
        if (it == B.groups.end()) {
            B.groups.push_back(BatchGroup{n, {}, 0, 0, 0, 0, 0});
            it = B.groups.end() - 1;
        }
        it->seqs.push_back(b);
    }
    size_t S = 0;
    for (const BatchGroup& g : B.groups) {
        const Layout L = make_layout(group_shape(g, hq, hkv));
        S = std::max(S, std::max(L.route_end, L.select_end));
    }
    size_t o = align_up(S);
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    for (BatchGroup& g : B.groups) {
        const Shape s = group_shape(g, hq, hkv);
        const Layout L = make_layout(s);
        g.p_base = take(L.total - L.pattern);
        g.vt_base = take((size_t)s.hkv * kD * s.nb * kB * sizeof(uint16_t));
        g.qtab = take(g.seqs.size() * sizeof(void*));
        g.ktab = take(g.seqs.size() * sizeof(void*));
        g.vtab = take(g.seqs.size() * sizeof(void*));
    }
    B.run.assign(batch, 0);
    B.per_xcd.assign(batch, 0);
    B.slot0.assign(batch, 0);
    B.pair_major.assign(batch, 0);
    for (int b = 0; b < batch; ++b) {
        const int n = len_of(b);
        if (n == 0) continue;
        attend_plan(n, hq, hkv, &B.run[b], &B.per_xcd[b], &B.pair_major[b]);
        B.slot0[b] = B.total_per_xcd;
        B.total_per_xcd += B.per_xcd[b];
    }
    B.table = take((size_t)batch * sizeof(SeqDesc));
    B.slot_seq = take((size_t)B.total_per_xcd * sizeof(int));
    B.counters = take(8 * sizeof(int));
    B.total = o;
    return B;
}

// Alg. 1 over every sequence of a batch: route every group (stage 0 -> 1),
// select every group (1 -> 2), lay out V and build the sequence table
// (2 -> 3), attend all in one launch (3 -> 4).  Groups below the gating
// length keep dense lists.
int run_prefill_batch_fused(const crisp_seq* seqs, int batch, const crisp_strides* strides,
                            int hq, int hkv, const Opts& op, float alpha, void* ws,
                            const BatchLayout& B, hipStream_t st)
{
    const size_t ng = B.groups.size();
    std::vector<Shape> gs(ng);
    std::vector<Layout> gl(ng);
    std::vector<SeqRows> gq(ng), gk(ng), gv(ng);
    for (size_t i = 0; i < ng; ++i) {
        const BatchGroup& g = B.groups[i];
        gs[i] = group_shape(g, hq, hkv);
        gl[i] = make_layout(gs[i]);
        // rows of every sequence of the group share their strides
        long long qsh, qst, ksh, kst, vsh, vst;
        if (strides) {
            qsh = strides->q_head, qst = strides->q_token;
            ksh = strides->k_head, kst = strides->k_token;
            vsh = strides->v_head, vst = strides->v_token;
        } else {
            qsh = ksh = vsh = (long long)g.n * kD;
            qst = kst = vst = kD;
        }
        gq[i] = SeqRows{at<const uint16_t*>(ws, g.qtab), hq, qsh, qst};
        gk[i] = SeqRows{at<const uint16_t*>(ws, g.ktab), hkv, ksh, kst};
        gv[i] = SeqRows{at<const uint16_t*>(ws, g.vtab), hkv, vsh, vst};
        // the three pointer tables, written from kernel arguments
        std::vector<const void*> qp, kp, vp;
        for (int b : g.seqs) {
            qp.push_back(seqs[b].q);
            kp.push_back(seqs[b].k);
            vp.push_back(seqs[b].v);
        }
        if (launch_ptr_table(qp.data(), (int)qp.size(), at<const void*>(ws, g.qtab), st) != hipSuccess ||
            launch_ptr_table(kp.data(), (int)kp.size(), at<const void*>(ws, g.ktab), st) != hipSuccess ||
            launch_ptr_table(vp.data(), (int)vp.size(), at<const void*>(ws, g.vtab), st) != hipSuccess)
            return CRISP_ERR_HIP;
    }
    auto pp = [&](size_t i, size_t off) { return B.groups[i].p_base + (off - gl[i].pattern); };
    auto sparse = [&](size_t i) { return B.groups[i].n >= op.dense_below; };
    int rc;
    mark(0, st);
    for (size_t i = 0; i < ng; ++i) {
        if (!sparse(i)) continue;
        const Layout& L = gl[i];
        if ((rc = do_route(gs[i], op, gq[i], gk[i], ws, L, at<uint8_t>(ws, pp(i, L.pattern)),
                           at<float>(ws, pp(i, L.c_struct)), at<float>(ws, pp(i, L.p_v)),
                           at<float>(ws, pp(i, L.p_s)), st)))
            return rc;
    }
    int* counters = at<int>(ws, B.counters);
    // small sparse groups lay out V^T (and clear the counters) in their selection launch
    auto fused = [&](size_t i) { return sparse(i) && select_lays_out_v(gs[i].nb); };
    mark(1, st);
    for (size_t i = 0; i < ng; ++i) {
        if (!sparse(i)) continue;
        const Layout& L = gl[i];
        const VtJob<SeqRows> job{gv[i], fused(i) ? at<uint16_t>(ws, B.groups[i].vt_base) : nullptr,
                                 counters};
        if ((rc = do_select(gs[i], op, alpha, gq[i], gk[i], at<uint8_t>(ws, pp(i, L.pattern)),
                            at<float>(ws, pp(i, L.p_v)), at<float>(ws, pp(i, L.p_s)), ws, L,
                            at<int32_t>(ws, pp(i, L.sel_v)), at<int32_t>(ws, pp(i, L.sel_s)),
                            at<int32_t>(ws, pp(i, L.counts)), at<int32_t>(ws, pp(i, L.row_ptr)),
                            at<int32_t>(ws, pp(i, L.col_idx)), job, st)))
            return rc;
    }
    mark(2, st);
    std::vector<SeqDesc> descs(batch);
    std::vector<int> live(batch, 0);
    for (size_t i = 0; i < ng; ++i) {
        const BatchGroup& g = B.groups[i];
        uint16_t* vt = at<uint16_t>(ws, g.vt_base);
        if (!fused(i) && launch_v_transpose(gv[i], g.n, gs[i].hkv, vt, counters, st) != hipSuccess)
            return CRISP_ERR_HIP;
        const int nb = gs[i].nb;
        for (size_t j = 0; j < g.seqs.size(); ++j) {
            const int b = g.seqs[j];
            SeqDesc& d = descs[b];
            d.q = static_cast<const uint16_t*>(seqs[b].q);
            d.k = static_cast<const uint16_t*>(seqs[b].k);
            d.out = static_cast<uint16_t*>(seqs[b].out);
            d.vt = vt + j * (size_t)hkv * nb * kB * kD;     // its KV heads' images
            const bool sp = sparse(i);
            d.row_ptr = sp ? at<int32_t>(ws, pp(i, gl[i].row_ptr)) + j * (size_t)hq * (nb + 1) : nullptr;
            d.col_idx = sp ? at<int32_t>(ws, pp(i, gl[i].col_idx)) : nullptr;
            d.q_sh = gq[i].sh;
            d.q_st = gq[i].st;
            d.k_sh = gk[i].sh;
            d.k_st = gk[i].st;
            if (strides) {
                d.o_sh = strides->out_head;
                d.o_st = strides->out_token;
            } else {
                d.o_sh = (long long)g.n * kD;
                d.o_st = kD;
            }
            d.n = g.n;
            d.run = B.run[b];
            d.slot0 = B.slot0[b];
            d.per_xcd = B.per_xcd[b];
            d.pair_major = B.pair_major[b];
            live[b] = 1;
        }
    }
    std::vector<SeqDesc> packed_descs;
    for (int b = 0; b < batch; ++b)
        if (live[b]) packed_descs.push_back(descs[b]);
    if (packed_descs.empty()) return CRISP_OK;
    SeqDesc* table = at<SeqDesc>(ws, B.table);
    int* slot_seq = at<int>(ws, B.slot_seq);
    if (launch_seq_table(packed_descs.data(), 0, (int)packed_descs.size(), table, slot_seq, st) !=
        hipSuccess)
        return CRISP_ERR_HIP;
    mark(3, st);
    const hipError_t e = launch_attend_batch(table, slot_seq, B.total_per_xcd, hq, hkv, counters, st);
    mark(4, st);
    return hip_status(e);
}

}  // namespace

namespace crisp {

int validate_prefill(const void* q, const void* k, const void* v, int seq_len, int n_heads,
                     int n_kv_heads, int head_dim, int block_size, float alpha,
                     const crisp_opts* opts, const void* out, size_t* ws_need)
{
    Shape s;
    int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    Opts op;
    if ((rc = check_opts(opts, &op))) return rc;
    if (!std::isfinite(alpha) || alpha < 0.0f) return CRISP_ERR_INVALID_ARG;
    *ws_need = 0;
    if (s.n == 0) return CRISP_OK;
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(out)) return CRISP_ERR_INVALID_ARG;
    *ws_need = make_layout(s).total;
    return CRISP_OK;
}

}  // namespace crisp

extern "C" {

void crisp_default_opts(crisp_opts* opts)
{
    if (opts) *opts = kDefaults;
}

const char* crisp_status_string(int code)
{
    switch (code) {
    case CRISP_OK: return "ok";
    case CRISP_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, or bad option)";
    case CRISP_ERR_SHAPE: return "bad shape (negative seq_len, n_heads % n_kv_heads != 0, or non-positive head count)";
    case CRISP_ERR_UNSUPPORTED: return "unsupported (head_dim, block_size and anchor windows must be 128; N_b <= 4096)";
    case CRISP_ERR_WORKSPACE: return "workspace or CSR capacity too small (crisp_prefill_noalloc: the layer needs more than its CRISP_NOALLOC_SCRATCH_BYTES)";
    case CRISP_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int crisp_workspace_size(int seq_len, int n_heads, int n_kv_heads, int head_dim, int block_size,
                         size_t* ws_bytes, int64_t* csr_capacity)
{
    Shape s;
    const int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    if (!ws_bytes || !csr_capacity) return CRISP_ERR_INVALID_ARG;
    const Layout L = make_layout(s);
    *ws_bytes = L.total;
    *csr_capacity = L.csr_capacity;
    return CRISP_OK;
}

int crisp_workspace_size_batch(const int* seq_lens, int batch, int n_heads, int n_kv_heads,
                               int head_dim, int block_size, size_t* ws_bytes)
{
    if (batch < 0 || (batch > 0 && seq_lens == nullptr) || ws_bytes == nullptr)
        return CRISP_ERR_INVALID_ARG;
    for (int b = 0; b < batch; ++b) {
        Shape s;
        const int rc = check_shape(seq_lens[b], n_heads, n_kv_heads, head_dim, block_size, &s);
        if (rc) return rc;
    }
    if (batch == 0) {
        Shape s;
        const int rc = check_shape(0, n_heads, n_kv_heads, head_dim, block_size, &s);
        if (rc) return rc;
    }
    *ws_bytes = make_batch_layout(batch, [&](int b) { return seq_lens[b]; }, n_heads, n_kv_heads).total;
    return CRISP_OK;
}

int crisp_set_stage_events(void* const* events, int count)
{
    if (events == nullptr) {
        g_events_on = false;
        return CRISP_OK;
    }
    if (count != 5) return CRISP_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i) {
        if (!events[i]) return CRISP_ERR_INVALID_ARG;
        g_events[i] = static_cast<hipEvent_t>(events[i]);
    }
    g_events_on = true;
    return CRISP_OK;
}

int crisp_route(const void* q, const void* k, int seq_len, int n_heads, int n_kv_heads,
                int head_dim, int block_size, const crisp_opts* opts, void* ws, size_t ws_bytes,
                uint8_t* pattern, float* c_struct, float* p_v, float* p_s, void* stream)
{
    Shape s;
    int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    Opts op;
    if ((rc = check_opts(opts, &op))) return rc;
    if (s.n == 0) return CRISP_OK;
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(ws, kAlign) || !pattern || bad_ptr(c_struct, 4) ||
        bad_ptr(p_v, 4) || bad_ptr(p_s, 4))
        return CRISP_ERR_INVALID_ARG;
    const Layout L = make_layout(s);
    if (ws_bytes < L.route_end) return CRISP_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    mark(0, st);
    rc = do_route(s, op, packed(q, s.n), packed(k, s.n), ws, L, pattern, c_struct, p_v, p_s, st);
    mark(1, st);
    return rc;
}

int crisp_select(const void* q, const void* k, const uint8_t* pattern, const float* p_v,
                 const float* p_s, int seq_len, int n_heads, int n_kv_heads, int head_dim,
                 int block_size, float alpha, const crisp_opts* opts, void* ws, size_t ws_bytes,
                 int32_t* sel_v, int32_t* sel_s, int32_t* sel_counts, int32_t* row_ptr,
                 int32_t* col_idx, int64_t csr_capacity, void* stream)
{
    Shape s;
    int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    Opts op;
    if ((rc = check_opts(opts, &op))) return rc;
    if (!std::isfinite(alpha) || alpha < 0.0f) return CRISP_ERR_INVALID_ARG;
    if (s.n == 0) return CRISP_OK;
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(ws, kAlign) || !pattern || bad_ptr(p_v, 4) ||
        bad_ptr(p_s, 4) || bad_ptr(sel_v, 4) || bad_ptr(sel_s, 4) || bad_ptr(sel_counts, 4) ||
        bad_ptr(row_ptr, 4) || bad_ptr(col_idx, 4))
        return CRISP_ERR_INVALID_ARG;
    const Layout L = make_layout(s);
    if (ws_bytes < L.select_end || csr_capacity < L.csr_capacity) return CRISP_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    mark(1, st);
    rc = do_select(s, op, alpha, packed(q, s.n), packed(k, s.n), pattern, p_v, p_s, ws, L, sel_v,
                   sel_s, sel_counts, row_ptr, col_idx, VtJob<Rows>{}, st);
    mark(2, st);
    return rc;
}

int crisp_attend(const void* q, const void* k, const void* v, const int32_t* row_ptr,
                 const int32_t* col_idx, int seq_len, int n_heads, int n_kv_heads, int head_dim,
                 int block_size, void* ws, size_t ws_bytes, void* out, void* stream)
{
    Shape s;
    const int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    if (s.n == 0) return CRISP_OK;
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(out) || bad_ptr(ws, kAlign) ||
        bad_ptr(row_ptr, 4) || bad_ptr(col_idx, 4))
        return CRISP_ERR_INVALID_ARG;
    const Layout L = make_layout(s);
    if (ws_bytes < L.attend_end) return CRISP_ERR_WORKSPACE;
    const Operands x{packed(q, s.n), packed(k, s.n), packed(v, s.n), packed_out(out, s.n)};
    return do_attend(s, x, row_ptr, col_idx, ws, L, static_cast<hipStream_t>(stream));
}

int crisp_attend_dense(const void* q, const void* k, const void* v, int seq_len, int n_heads,
                       int n_kv_heads, int head_dim, int block_size, void* ws, size_t ws_bytes,
                       void* out, void* stream)
{
    Shape s;
    const int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    if (s.n == 0) return CRISP_OK;
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(out) || bad_ptr(ws, kAlign))
        return CRISP_ERR_INVALID_ARG;
    const Layout L = make_layout(s);
    if (ws_bytes < L.attend_end) return CRISP_ERR_WORKSPACE;
    const Operands x{packed(q, s.n), packed(k, s.n), packed(v, s.n), packed_out(out, s.n)};
    return do_attend(s, x, nullptr, nullptr, ws, L, static_cast<hipStream_t>(stream));
}

int crisp_prefill(const void* q, const void* k, const void* v, int seq_len, int n_heads,
                  int n_kv_heads, int head_dim, int block_size, float alpha,
                  const crisp_opts* opts, void* ws, size_t ws_bytes, void* out, void* stream)
{
    Shape s;
    int rc = check_shape(seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
    if (rc) return rc;
    Opts op;
    if ((rc = check_opts(opts, &op))) return rc;
    if (!std::isfinite(alpha) || alpha < 0.0f) return CRISP_ERR_INVALID_ARG;
    if (s.n == 0) return CRISP_OK;
    if (bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(out) || bad_ptr(ws, kAlign))
        return CRISP_ERR_INVALID_ARG;
    const Layout L = make_layout(s);
    if (ws_bytes < L.total) return CRISP_ERR_WORKSPACE;
    const Operands x{packed(q, s.n), packed(k, s.n), packed(v, s.n), packed_out(out, s.n)};
    return run_prefill(s, op, alpha, x, ws, L, static_cast<hipStream_t>(stream));
}

int crisp_prefill_batch(const crisp_seq* seqs, int batch, const crisp_strides* strides,
                        int n_heads, int n_kv_heads, int head_dim, int block_size, float alpha,
                        const crisp_opts* opts, void* ws, size_t ws_bytes, void* stream)
{
    if (batch < 0 || (batch > 0 && seqs == nullptr)) return CRISP_ERR_INVALID_ARG;
    Opts op;
    int rc = check_opts(opts, &op);
    if (rc) return rc;
    if (!std::isfinite(alpha) || alpha < 0.0f) return CRISP_ERR_INVALID_ARG;
    if (strides && (bad_strides(strides->q_head, strides->q_token) ||
                    bad_strides(strides->k_head, strides->k_token) ||
                    bad_strides(strides->v_head, strides->v_token) ||
                    bad_strides(strides->out_head, strides->out_token)))
        return CRISP_ERR_INVALID_ARG;
    // validate every sequence before the first launch
    for (int b = 0; b < batch; ++b) {
        Shape s;
        if ((rc = check_shape(seqs[b].seq_len, n_heads, n_kv_heads, head_dim, block_size, &s)))
            return rc;
        if (s.n == 0) continue;
        if (bad_ptr(seqs[b].q) || bad_ptr(seqs[b].k) || bad_ptr(seqs[b].v) || bad_ptr(seqs[b].out) ||
            bad_ptr(ws, kAlign))
            return CRISP_ERR_INVALID_ARG;
        if (ws_bytes < make_layout(s).total) return CRISP_ERR_WORKSPACE;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (batch > 0) {
        const BatchLayout BL = make_batch_layout(
            batch, [&](int b) { return seqs[b].seq_len; }, n_heads, n_kv_heads);
        if (BL.total_per_xcd > 0 && ws_bytes >= BL.total)
            return run_prefill_batch_fused(seqs, batch, strides, n_heads, n_kv_heads, op, alpha, ws,
                                           BL, st);
    }
    for (int b = 0; b < batch; ++b) {
        Shape s;
        (void)check_shape(seqs[b].seq_len, n_heads, n_kv_heads, head_dim, block_size, &s);
        if (s.n == 0) continue;
        Operands x;
        if (strides) {
            x.q = Rows{static_cast<const uint16_t*>(seqs[b].q), strides->q_head, strides->q_token};
            x.k = Rows{static_cast<const uint16_t*>(seqs[b].k), strides->k_head, strides->k_token};
            x.v = Rows{static_cast<const uint16_t*>(seqs[b].v), strides->v_head, strides->v_token};
            x.out = OutRows{static_cast<uint16_t*>(seqs[b].out), strides->out_head, strides->out_token};
        } else {
            x = Operands{packed(seqs[b].q, s.n), packed(seqs[b].k, s.n), packed(seqs[b].v, s.n),
                         packed_out(seqs[b].out, s.n)};
        }
        if ((rc = run_prefill(s, op, alpha, x, ws, make_layout(s), st))) return rc;
    }
    return CRISP_OK;
}

}  // extern "C"
