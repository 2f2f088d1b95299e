// Index selection and block-list expansion kernels.
//
//   vs_select_*        VS budget per direction: the sink-aware noise floor
//                      (Alg. 3; Eq. 3-4), the median floor
//                      (Appendix H) or FlexPrefill's cumulative rule (Alg. 6),
//                      with stream compaction
//   pe_*_kernel        pooled estimation for PE heads (Alg. 4): block-mean
//                      pooling of Q and K, the causal pooled softmax map,
//                      normalisation, and the gamma-cumsum cut-off found by a
//                      mass-weighted radix select on the float bits instead
//                      of a full sort
//   expand_*_kernel    per-(head, query block) key-block lists (the block
//                      mask M_S of Eq. 1), CSR with per-head worst-case bases:
//                      row lengths, per-head scan, fill
//   select_small_kernel  for N_b <= 128, everything after pooling in one
//                      work-group per head: a VS head's budgets, or a PE
//                      head's map (built here for N_b <= 64) and cut-off,
//                      then its lists; extra work-groups lay out the
//                      attention's V^T meanwhile
//
// Decisions are taken in float in the order the paper writes them; the
// pooled masses are summed in 2^-62 fixed point, which is exact and
// independent of summation order for every value >= 2^-38.
#include "crisp_common.h"
#include "crisp_kernels.h"

namespace crisp {

namespace {

__device__ __forceinline__ unsigned long long to_fix(float v)
{
    return (unsigned long long)((double)v * kFix);
}

__device__ __forceinline__ size_t tri(int qb) { return (size_t)qb * (qb + 1) / 2; }

// Exclusive prefix sum over a 1024-thread block; also returns the total.
__device__ int block_scan_1024(int v, int* wsum, int* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = (int)wave_scan_incl((uint32_t)v);
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        const int s = (int)wave_scan_incl((uint32_t)((lane < 16) ? wsum[lane] : 0));
        if (lane < 16) wsum[lane] = s;
    }
    __syncthreads();
    const int excl = (w > 0 ? wsum[w - 1] : 0) + x - v;
    *total = wsum[15];
    __syncthreads();
    return excl;
}

// Exclusive prefix sum of doubles over a 1024-thread block; also the total.
__device__ double block_scan_1024(double v, double* wsum, double* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        double s = (lane < 16) ? wsum[lane] : 0.0;
        for (int o = 1; o < 16; o <<= 1) {
            const double y = __shfl_up(s, o);
            if (lane >= o) s += y;
        }
        if (lane < 16) wsum[lane] = s;
    }
    __syncthreads();
    const double excl = (w > 0 ? wsum[w - 1] : 0.0) + x - v;
    *total = wsum[15];
    __syncthreads();
    return excl;
}

// Ascending bitonic sort of keys[0 .. np2) in LDS (np2 a power of two
// <= kMaxBlocks), 1024 threads.
__device__ void bitonic_sort(unsigned long long* keys, int np2)
{
    for (int k = 2; k <= np2; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < np2; i += 1024) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long a = keys[i], b = keys[ixj];
                    if ((a > b) == ((i & k) == 0)) {
                        keys[i] = b;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
}

constexpr int kRankClip = 256;      // largest N_b whose k_min clip ranks all entries

// LDS of one direction's budget selection; keys hold at least the power
// of two at or above N_b.
template <int KeyCap>
struct VsLds {
    int wsum[16];
    double wsum_d[16];
    float best_v[2][16];
    int best_i[2][16];
    int kk;
    uint8_t flag[kMaxBlocks];
    unsigned long long keys[KeyCap];
};

// One direction of VS head h (p: its p_v or p_s row), by every thread of a
// 1024-thread block: the kept blocks, ascending, into sel, their number into
// counts[h * 3 + dir], and a 0/1 flag per block into bm (global or LDS).
// Budget rule:
//   0  p_j > alpha * r / (N_b - 2), r = max(1 - p_0 - p_{N_b-1}, 0)   (Eq. 3-4)
//   1  p_j > alpha * median(p_1 .. p_{N_b-2})                          (App. H)
//   2  the shortest prefix of (p desc, j asc) whose running sum, in
//      double, reaches gamma_vs                                        (Alg. 6)
// then clip(k, k_min, N_b) with top-k by (p desc, j asc) for rules 0 and 1
// (N_b <= 2 keeps every block under them) and, for rule 2, at least k_min
// entries of the same order.  Values are compared in float.
template <int KeyCap>
__device__ void vs_select_dir(VsLds<KeyCap>& L, int h, int dir, const float* __restrict__ p, int nb,
                              const VsRule& vr, int32_t* __restrict__ sel,
                              int32_t* __restrict__ counts, uint8_t* bm)
{
    int* wsum = L.wsum;
    double* wsum_d = L.wsum_d;
    auto& best_v = L.best_v;
    auto& best_i = L.best_i;
    int& s_kk = L.kk;
    uint8_t* flag = L.flag;
    unsigned long long* keys = L.keys;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    int np2 = 1;
    while (np2 < nb) np2 <<= 1;

    float pv[4];
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        pv[e] = (j < nb) ? p[j] : -INFINITY;
    }
    int cnt = 0;
    if (vr.rule == 2) {
        // order (p desc, j asc): the complemented float bits of p >= 0
        // descend as p grows
        for (int i = tid; i < np2; i += 1024)
            keys[i] = (i < nb) ? ((unsigned long long)(~__float_as_uint(p[i])) << 32) | (unsigned)i
                               : ~0ull;
        __syncthreads();
        bitonic_sort(keys, np2);
        double part = 0.0, vals[4];
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * tid + e;
            vals[e] = (t < nb) ? (double)__uint_as_float(~(uint32_t)(keys[t] >> 32)) : 0.0;
            part += vals[e];
        }
        if (tid == 0) s_kk = nb;
        double total;
        double run = block_scan_1024(part, wsum_d, &total);
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * tid + e;
            run += vals[e];
            if (t < nb && run >= (double)vr.gamma_vs) {
                atomicMin(&s_kk, t + 1);
                break;
            }
        }
        __syncthreads();
        const int kk = min(max(s_kk, vr.kmin_blocks), nb);
        for (int e = 0; e < 4; ++e) flag[4 * tid + e] = 0;
        __syncthreads();
        for (int t = tid; t < kk; t += 1024) flag[(uint32_t)keys[t]] = 1;
        __syncthreads();
        for (int e = 0; e < 4; ++e) cnt += flag[4 * tid + e];
    } else {
        float theta = -INFINITY;
        if (nb > 2 && vr.rule == 0) {
            // Eq. 3: mu over the N_b - 2 non-retained blocks
            float r = 1.0f - p[0];
            r = r - p[nb - 1];
            r = fmaxf(r, 0.0f);
            const float mu = r / (float)(nb - 2);
            theta = vr.alpha * mu;
        } else if (nb > 2) {
            // Appendix H: median of blocks 1 .. N_b-2 (ascending float bits)
            for (int i = tid; i < np2; i += 1024)
                keys[i] = (i >= 1 && i <= nb - 2)
                              ? ((unsigned long long)__float_as_uint(p[i]) << 32) | (unsigned)i
                              : ~0ull;
            __syncthreads();
            bitonic_sort(keys, np2);
            const int m = nb - 2;
            const float hi_v = __uint_as_float((uint32_t)(keys[m / 2] >> 32));
            const float med = (m & 1) ? hi_v
                                      : (__uint_as_float((uint32_t)(keys[m / 2 - 1] >> 32)) + hi_v) * 0.5f;
            theta = vr.alpha * med;
        }
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * tid + e;
            const bool f = (j < nb) && (pv[e] > theta);
            flag[j] = f;
            cnt += f;
        }
        int total;
        block_scan_1024(cnt, wsum, &total);
        if (total < vr.kmin_blocks && total < nb) {
            // clip to k_min: top-k_min by (p desc, index asc)
            const int kk = min(vr.kmin_blocks, nb);
            for (int e = 0; e < 4; ++e) flag[4 * tid + e] = 0;
            __syncthreads();
            if (nb <= kRankClip) {
                // small N_b: entry j is kept iff fewer than kk entries precede it
                // in the order (p desc, j asc); the same kk entries as the picks
                float* pl = reinterpret_cast<float*>(keys);     // free under rules 0 and 1
                for (int i = tid; i < nb; i += 1024) pl[i] = p[i];
                __syncthreads();
                if (4 * tid < nb) {
                    int rank[4] = {0, 0, 0, 0};
                    for (int i = 0; i < nb; ++i) {
                        const float x = pl[i];
                        for (int e = 0; e < 4; ++e)
                            rank[e] += (x > pv[e] || (x == pv[e] && i < 4 * tid + e)) ? 1 : 0;
                    }
                    for (int e = 0; e < 4; ++e)
                        if (4 * tid + e < nb) flag[4 * tid + e] = rank[e] < kk;
                }
            } else {
                // one round per pick: each wavefront's best candidate, then every
                // thread finds the overall best and its owner flags it (flags
                // are only read by their owner); the per-wave slots alternate
                // between rounds, so one barrier per round suffices
                for (int round = 0; round < kk; ++round) {
                    float bv = -INFINITY;
                    int bi = 0x7fffffff;
                    for (int e = 0; e < 4; ++e) {
                        const int j = 4 * tid + e;
                        if (j < nb && !flag[j] && (pv[e] > bv || (pv[e] == bv && j < bi))) { bv = pv[e]; bi = j; }
                    }
                    for (int o = 32; o > 0; o >>= 1) {
                        const float ov = __shfl_xor(bv, o);
                        const int oi = __shfl_xor(bi, o);
                        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
                    }
                    const int slot = round & 1;
                    if (lane == 0) { best_v[slot][w] = bv; best_i[slot][w] = bi; }
                    __syncthreads();
                    float v = best_v[slot][0];
                    int i = best_i[slot][0];
                    for (int x = 1; x < 16; ++x)
                        if (best_v[slot][x] > v || (best_v[slot][x] == v && best_i[slot][x] < i)) {
                            v = best_v[slot][x];
                            i = best_i[slot][x];
                        }
                    if ((i >> 2) == tid) flag[i] = 1;
                }
            }
            __syncthreads();
            cnt = 0;
            for (int e = 0; e < 4; ++e) cnt += flag[4 * tid + e];
        }
    }
    int kept;
    int pos = block_scan_1024(cnt, wsum, &kept);
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        if (j >= nb) break;
        bm[j] = flag[j];
        if (flag[j]) sel[pos++] = j;
    }
    if (tid == 0) counts[h * 3 + dir] = kept;
}

// grid (hq, 2): direction 0 = vertical (p_v), 1 = slash (p_s); a PE head's
// work-groups only zero its two counts.
__global__ void __launch_bounds__(1024)
vs_select_kernel(const uint8_t* __restrict__ pattern, const float* __restrict__ p_v,
                 const float* __restrict__ p_s, int nb, VsRule vr,
                 int32_t* __restrict__ sel_v, int32_t* __restrict__ sel_s,
                 int32_t* __restrict__ counts, uint8_t* __restrict__ bitmap)
{
    __shared__ VsLds<kMaxBlocks> L;
    const int h = blockIdx.x, dir = blockIdx.y;
    if (!pattern[h]) {
        if (threadIdx.x == 0) counts[h * 3 + dir] = 0;
        return;
    }
    vs_select_dir(L, h, dir, (dir ? p_s : p_v) + (size_t)h * nb, nb, vr,
                  (dir ? sel_s : sel_v) + (size_t)h * nb, counts,
                  bitmap + ((size_t)h * 2 + dir) * nb);
}

// grid (hq), 1024 threads: clear the head's radix histograms and pass
// counters, and seed its cut-off state.
__global__ void __launch_bounds__(1024)
pe_init_kernel(const uint8_t* __restrict__ pattern, float gamma,
               unsigned long long* __restrict__ hist_mass, uint32_t* __restrict__ hist_count,
               uint32_t* __restrict__ pass_ctr, PeState* __restrict__ state)
{
    const int h = blockIdx.x, tid = threadIdx.x;
    if (pattern[h] == 0) {
        for (int i = tid; i < kValPasses * kValBins; i += 1024)
            hist_mass[(size_t)h * kValPasses * kValBins + i] = 0ull;
        for (int i = tid; i < kRadixPasses * kFlatBins; i += 1024)
            hist_count[(size_t)h * kRadixPasses * kFlatBins + i] = 0u;
        if (tid < kRadixPasses) pass_ctr[h * kRadixPasses + tid] = 0u;
    }
    if (tid == 0) {
        PeState st = {};
        st.need = (unsigned long long)((double)gamma * kFix);
        st.done = pattern[h] ? 1u : 0u;
        state[h] = st;
    }
}

__device__ __forceinline__ bool group_has_pe(const uint8_t* pattern, int g, int G)
{
    for (int x = 0; x < G; ++x)
        if (!pattern[g * G + x]) return true;
    return false;
}

// grid (Nb, hq + hkv): block means of Q (PE heads) and K (groups with a PE
// head), over the tokens each block holds (the last block may be partial).
template <class R>
__global__ void __launch_bounds__(256)
pe_pool_kernel(R q, R k,
               const uint8_t* __restrict__ pattern, int n, int hq, int G,
               float* __restrict__ qbar, float* __restrict__ kbar)
{
    __shared__ float red[16][kD];
    const int qb = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
    const int nb = (n + kB - 1) / kB;
    const int len = min(kB, n - qb * kB);           // tokens in block qb
    const uint16_t* src;
    long long st;
    float* dst;
    if (y < hq) {
        if (pattern[y]) return;
        src = q.row(y, (long long)qb * kB);
        st = q.st;
        dst = qbar + ((size_t)y * nb + qb) * kD;
    } else {
        const int g = y - hq;
        if (!group_has_pe(pattern, g, G)) return;
        src = k.row(g, (long long)qb * kB);
        st = k.st;
        dst = kbar + ((size_t)g * nb + qb) * kD;
    }
    const int dc = tid & 15, tg = tid >> 4;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = tg * 8; t < min(tg * 8 + 8, len); ++t) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(src + t * st + 8 * dc);
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(raw[e] << 16);
            acc[2 * e + 1] += __uint_as_float(raw[e] & 0xffff0000u);
        }
    }
    for (int e = 0; e < 8; ++e) red[tg][8 * dc + e] = acc[e];
    __syncthreads();
    if (tid < kD) {
        float s = 0.f;
        for (int x = 0; x < 16; ++x) s += red[x][tid];
        dst[tid] = s / (float)len;
    }
}

// grid (ceil(Nb/32), ceil(Nb/128), hq), 256 threads: scaled pooled logits
// Q̄ K̄^T of a 32-query-block tile against four 32-key-block tiles, one per
// wavefront, on the fp32 matrix cores (v_mfma_f32_32x32x2_f32, 64 steps
// over d), log2 domain, triangular row layout; tiles above the diagonal
// are skipped.
__global__ void __launch_bounds__(256)
pe_logits_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                 const uint8_t* __restrict__ pattern, int nb, int G, float scale_log2,
                 int fuse_softmax, float* __restrict__ abar)
{
    constexpr int kP = kD + 1;                   // LDS pitch (floats)
    __shared__ float qs[32 * kP];
    __shared__ float kst[128 * kP];
    const int h = blockIdx.z, tid = threadIdx.x;
    if (pattern[h]) return;
    const int qt = blockIdx.x, kt0 = 4 * blockIdx.y;
    if (kt0 > qt) return;                        // every tile above the diagonal
    const int g = h / G;
    // stage both operands with every load in flight at once: 4 + 16 float4
    // per thread, then the LDS stores
    f32x4 qv[4], kv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + 256 * j, r = e >> 5, qb = 32 * qt + r;
        qv[j] = (qb < nb) ? *reinterpret_cast<const f32x4*>(qbar + ((size_t)h * nb + qb) * kD + 4 * (e & 31))
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = tid + 256 * j, r = e >> 5, kb = 32 * kt0 + r;
        kv[j] = (kb < nb) ? *reinterpret_cast<const f32x4*>(kbar + ((size_t)g * nb + kb) * kD + 4 * (e & 31))
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + 256 * j;
        for (int x = 0; x < 4; ++x) qs[(e >> 5) * kP + 4 * (e & 31) + x] = qv[j][x];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = tid + 256 * j;
        for (int x = 0; x < 4; ++x) kst[(e >> 5) * kP + 4 * (e & 31) + x] = kv[j][x];
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int kt = kt0 + w;
    const bool live = kt <= qt;
    if (!live && !fuse_softmax) return;
    // D[m][n] = sum_d Q̄[32 qt + m][d] K̄[32 kt + n][d]; step s covers d = 2s, 2s+1
    // (A: lane l holds row l % 32, d = 2s + l / 32; B likewise for keys)
    // (two independent accumulation chains over alternate steps)
    f32x16 acc = f32x16{}, acc1 = f32x16{};
    if (live) {
        const float* qa = qs + l32 * kP + hi;
        const float* kb_ = kst + (32 * w + l32) * kP + hi;
        for (int s = 0; s < kD / 2; s += 2) {
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[2 * s], kb_[2 * s], acc, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[2 * s + 2], kb_[2 * s + 2], acc1, 0, 0, 0);
        }
        acc += acc1;
    }
    const size_t base = (size_t)h * tri(nb);
    const int kb = 32 * kt + l32;
    if (!fuse_softmax) {
        for (int r = 0; r < 16; ++r) {
            const int qb = 32 * qt + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (qb < nb && kb <= qb) abar[base + tri(qb) + kb] = acc[r] * scale_log2;
        }
        return;
    }
    // N_b <= 128: this work-group holds whole rows (every key tile of query
    // blocks 32 qt .. 32 qt + 31), so it also runs pe_softmax_kernel's row
    // normalisation on them, in the same order, from an LDS copy
    __syncthreads();                              // kst is free
    float* rows = kst;                            // [32][kP]
    if (live)
        for (int r = 0; r < 16; ++r) rows[(8 * (r >> 2) + 4 * hi + (r & 3)) * kP + kb] = acc[r] * scale_log2;
    __syncthreads();
    // the wavefront's eight rows (rl = w, w + 4, ..) with their wave
    // reductions interleaved: each row's max and sum use the butterflies of
    // wave_max / wave_sum, so the bits match pe_softmax_kernel's
    float m8[8];
    double l8[8];
    for (int j = 0; j < 8; ++j) {
        const int qb = 32 * qt + w + 4 * j;
        const float* row = rows + (w + 4 * j) * kP;
        float m = -INFINITY;
        if (qb < nb)
            for (int k2 = lane; k2 <= qb; k2 += 64) m = fmaxf(m, row[k2]);
        m8[j] = m;
    }
    for (int o = 32; o > 0; o >>= 1) {
        float y[8];
        for (int j = 0; j < 8; ++j) y[j] = __shfl_xor(m8[j], o);
        for (int j = 0; j < 8; ++j) m8[j] = fmaxf(m8[j], y[j]);
    }
    for (int j = 0; j < 8; ++j) {
        const int qb = 32 * qt + w + 4 * j;
        const float* row = rows + (w + 4 * j) * kP;
        double l = 0.0;
        if (qb < nb)
            for (int k2 = lane; k2 <= qb; k2 += 64) l += (double)exp2f(row[k2] - m8[j]);
        l8[j] = l;
    }
    wave_sum_n(l8);
    for (int j = 0; j < 8; ++j) {
        const int qb = 32 * qt + w + 4 * j;
        if (qb >= nb) break;
        const float* row = rows + (w + 4 * j) * kP;
        const double inv = 1.0 / (l8[j] * (double)nb);
        float* out = abar + base + tri(qb);
        for (int k2 = lane; k2 <= qb; k2 += 64) out[k2] = (float)((double)exp2f(row[k2] - m8[j]) * inv);
    }
}

// grid (ceil(Nb/4), hq): row softmax over kb <= qb, then divide by the total
// mass (each row sums to one, so the total is N_b).
__global__ void __launch_bounds__(256)
pe_softmax_kernel(const uint8_t* __restrict__ pattern, int nb, float* __restrict__ abar)
{
    const int h = blockIdx.y, lane = threadIdx.x & 63;
    const int qb = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pattern[h] || qb >= nb) return;
    float* row = abar + (size_t)h * tri(nb) + tri(qb);
    float m = -INFINITY;
    for (int kb = lane; kb <= qb; kb += 64) m = fmaxf(m, row[kb]);
    m = wave_max(m);
    double l = 0.0;
    for (int kb = lane; kb <= qb; kb += 64) l += (double)exp2f(row[kb] - m);
    l = wave_sum(l);
    const double inv = 1.0 / (l * (double)nb);
    for (int kb = lane; kb <= qb; kb += 64) row[kb] = (float)((double)exp2f(row[kb] - m) * inv);
}

// The gamma cut-off of a PE head (Alg. 4: the shortest prefix of the map
// sorted by value, descending, ties by flat index qb*Nb+kb ascending, whose
// mass reaches gamma) as a mass-weighted radix select in five passes.  Keys
// are key = ~bits(value), ascending in value-descending order.  Passes 0-2
// histogram the key 11, 11 and 10 bits at a time (count and fixed-point
// mass per digit) among the entries that match the digits resolved so far;
// passes 3-4 histogram the flat index (12 + 12 bits) of the entries whose
// key equals the cut-off key, by count.  Each work-group takes a contiguous
// range of the head's triangular map; the last work-group of a pass to
// finish (a per-head counter) scans the global histogram and resolves the
// pass's digit into the head's state.
constexpr int kRadixChunk = 4096;          // map entries per work-group

__device__ __forceinline__ int pass_shift(int pass)
{
    return pass == 0 ? 21 : pass == 1 ? 10 : pass == 2 ? 0 : pass == 3 ? 12 : 0;
}
__device__ __forceinline__ int pass_bits(int pass)
{
    return pass < 2 ? 11 : pass == 2 ? 10 : 12;
}

// Exclusive scan of one value per thread over a 256-thread block; total too.
template <typename T>
__device__ T block_scan_256(T v, T* wsum, T* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    T x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const T y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    T before = 0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    return before + x - v;
}

// One map entry's contribution to pass `pass`'s LDS histogram: entry e
// (flat position in the head's triangular map) with value v.
__device__ __forceinline__ void radix_add(int pass, int nb, const PeState& st, size_t e, float v,
                                          uint32_t* cnt, unsigned long long* mass)
{
    const int shift = pass_shift(pass), bits = pass_bits(pass);
    const uint32_t mask = (1u << bits) - 1u;
    const uint32_t key = ~__float_as_uint(v);
    if (pass < kValPasses) {
        if (pass > 0 && (key >> (shift + bits)) != st.key_prefix) return;
        const uint32_t d = (key >> shift) & mask;
        atomicAdd(&cnt[d], 1u);
        atomicAdd(&mass[d], to_fix(v));
    } else {
        if (key != st.key_star) return;
        // row of entry e: the largest qb with qb (qb + 1) / 2 <= e
        int qb = (int)((sqrt(8.0 * (double)e + 1.0) - 1.0) * 0.5);
        while (tri(qb + 1) <= e) ++qb;
        while (tri(qb) > e) --qb;
        const uint32_t flat = (uint32_t)qb * (uint32_t)nb + (uint32_t)(e - tri(qb));
        if (pass > kValPasses && (flat >> (shift + bits)) != st.flat_prefix) return;
        atomicAdd(&cnt[(flat >> shift) & mask], 1u);
    }
}

// Resolve pass `pass` of a PE head from its complete histogram (cnt, and
// mass for the value passes; LDS, 1 << pass_bits(pass) digits), 256
// threads: the digit at which the kept mass (value passes) or the tie count
// (index passes) is reached.  The thread that finds it writes the head's
// next state to *out; every thread must call this (it holds barriers).
__device__ void radix_resolve(int pass, size_t total, const PeState& st, const uint32_t* cnt,
                              const unsigned long long* mass, uint32_t* wsum_c,
                              unsigned long long* wsum_m, PeState* out)
{
    const int tid = threadIdx.x;
    const bool val = pass < kValPasses;
    const int bits = pass_bits(pass);
    const int per = (1 << bits) / 256;                // consecutive digits per thread
    uint32_t c_loc = 0;
    unsigned long long m_loc = 0;
    for (int j = 0; j < per; ++j) {
        const int i = tid * per + j;
        c_loc += cnt[i];
        if (val) m_loc += mass[i];
    }
    uint32_t c_all;
    unsigned long long m_all;
    uint32_t c_before = block_scan_256(c_loc, wsum_c, &c_all);
    unsigned long long m_before = val ? block_scan_256(m_loc, wsum_m, &m_all) : 0ull;
    if (val) {
        const unsigned long long need = st.need;
        if (m_all < need) {
            // the kept mass never reaches gamma: keep every causal entry
            if (tid == 0) {
                PeState nx = st;
                nx.key_star = 0xffffffffu;
                nx.flat_star = 0xffffffffu;
                nx.kstar = (uint32_t)total;
                nx.done = 1u;
                *out = nx;
            }
            return;
        }
        for (int j = 0; j < per; ++j) {
            const int i = tid * per + j;
            const unsigned long long incl = m_before + mass[i];
            if (m_before < need && incl >= need) {
                PeState nx = st;
                nx.need = need - m_before;
                nx.before = st.before + c_before;
                nx.key_prefix = (st.key_prefix << bits) | (uint32_t)i;
                if (pass == kValPasses - 1) {
                    nx.key_star = nx.key_prefix;
                    const float tv = __uint_as_float(~nx.key_star);
                    const unsigned long long tf = to_fix(tv);
                    const unsigned long long ties = (nx.need + tf - 1) / tf;
                    nx.tfix = tf;
                    if (ties >= cnt[i]) {
                        nx.flat_star = 0xffffffffu;
                        nx.kstar = nx.before + cnt[i];
                        nx.done = 1u;
                    } else {
                        nx.tie_need = (uint32_t)ties;
                        nx.kstar = nx.before + (uint32_t)ties;
                    }
                }
                *out = nx;
            }
            m_before = incl;
            c_before += cnt[i];
        }
    } else {
        const uint32_t need = st.tie_need;
        for (int j = 0; j < per; ++j) {
            const int i = tid * per + j;
            const uint32_t incl = c_before + cnt[i];
            if (c_before < need && incl >= need) {
                PeState nx = st;
                nx.tie_need = need - c_before;
                nx.flat_prefix = (st.flat_prefix << bits) | (uint32_t)i;
                if (pass == kRadixPasses - 1) {
                    nx.flat_star = nx.flat_prefix;
                    nx.done = 1u;
                }
                *out = nx;
            }
            c_before = incl;
        }
    }
}

// The gamma cut-off of one PE head whose triangular map (at most
// kRadixSmall entries, N_b <= 128) starts at `base`, by one 1024-thread
// block over an LDS copy of the map.  The sorted order, the fixed-point
// masses and the tie rule define the cut-off uniquely, so this finds the
// same (key_star, flat_star, K*) as the multi-launch passes, by a cheaper
// route for small maps: four passes over 8-bit digits of the key, each
// wavefront counting into its own LDS copy of the 256-bin histogram (so
// atomics contend only inside a wavefront), and, only when the cut-off key
// is shared by entries that are not all kept, one block scan for the tie
// (entry order in the triangular map is flat order).  Every thread calls it
// and gets the final state; the map stays in L.vals (base == nullptr: it is
// there already).
constexpr int kSmallBins = 256;               // 8-bit digits
constexpr int kSmallPasses = 4;
constexpr int kFoldRounds = 4;

constexpr int kMapSmall = 64;                 // N_b up to which the map is built here too
constexpr int kMapPitch = kD + 1;             // LDS pitch of a pooled row (floats)

struct SmallCutLds {
    float vals[kRadixSmall];
    union {
        struct {                                // the cut-off's histograms
            uint32_t wcnt[16][kSmallBins];      // per wavefront
            unsigned long long wmass[16][kSmallBins];
            uint32_t pcnt[4][kSmallBins];       // sums of four copies each
            unsigned long long pmass[4][kSmallBins];
        } h;
        struct {                                // pe_map_small's pooled rows
            float q[kMapSmall * kMapPitch];
            float k[kMapSmall * kMapPitch];     // then the scaled logits rows
        } m;
    } x;
    PeState st;
    uint32_t bin_count;                         // entries in the resolved bin
    int scan[16];
};

// The normalised pooled map of one PE head for N_b <= kMapSmall, built in
// LDS (L.vals, triangular rows) by one 1024-thread block from its pooled
// query rows and its KV head's pooled key rows: the same tiles, MFMA steps
// and row reductions as pe_logits_kernel with its fused softmax, so the
// same bits, without the map's round trip through memory or a launch of
// its own.  Ends with a barrier.
__device__ void pe_map_small(SmallCutLds& L, const float* __restrict__ qrows,
                             const float* __restrict__ krows, int nb, float scale_log2)
{
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    constexpr int kP = kMapPitch;
    float* qs = L.x.m.q;
    float* ks = L.x.m.k;
    for (int j = 0; j < 2; ++j) {               // 64 rows x 32 float4 per operand
        const int e = tid + 1024 * j, r = e >> 5, c = 4 * (e & 31);
        const f32x4 qv = (r < nb) ? *reinterpret_cast<const f32x4*>(qrows + (size_t)r * kD + c)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 kv = (r < nb) ? *reinterpret_cast<const f32x4*>(krows + (size_t)r * kD + c)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        for (int x = 0; x < 4; ++x) {
            qs[r * kP + c + x] = qv[x];
            ks[r * kP + c + x] = kv[x];
        }
    }
    __syncthreads();
    // the causal 32 x 32 tiles (qt, kt), kt <= qt: wavefronts 0, 1, 2
    const int tiles = nb > 32 ? 3 : 1;
    const int qt = w == 0 ? 0 : 1, kt = w == 2 ? 1 : 0;
    f32x16 acc = f32x16{}, acc1 = f32x16{};
    if (w < tiles) {
        const float* qa = qs + (32 * qt + l32) * kP + hi;
        const float* kb_ = ks + (32 * kt + l32) * kP + hi;
        for (int s = 0; s < kD / 2; s += 2) {
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[2 * s], kb_[2 * s], acc, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[2 * s + 2], kb_[2 * s + 2], acc1, 0, 0, 0);
        }
        acc += acc1;
    }
    __syncthreads();                              // ks is free: the logits rows
    float* rows = ks;
    if (w < tiles)
        for (int r = 0; r < 16; ++r)
            rows[(32 * qt + 8 * (r >> 2) + 4 * hi + (r & 3)) * kP + 32 * kt + l32] = acc[r] * scale_log2;
    __syncthreads();
    // rows w, w + 16, w + 32, w + 48, each reduced as pe_logits_kernel does
    float m4[4];
    double l4[4];
    for (int j = 0; j < 4; ++j) {
        const int qb = w + 16 * j;
        const float* row = rows + qb * kP;
        float m = -INFINITY;
        if (qb < nb)
            for (int k2 = lane; k2 <= qb; k2 += 64) m = fmaxf(m, row[k2]);
        m4[j] = m;
    }
    for (int o = 32; o > 0; o >>= 1) {
        float y[4];
        for (int j = 0; j < 4; ++j) y[j] = __shfl_xor(m4[j], o);
        for (int j = 0; j < 4; ++j) m4[j] = fmaxf(m4[j], y[j]);
    }
    for (int j = 0; j < 4; ++j) {
        const int qb = w + 16 * j;
        const float* row = rows + qb * kP;
        double l = 0.0;
        if (qb < nb)
            for (int k2 = lane; k2 <= qb; k2 += 64) l += (double)exp2f(row[k2] - m4[j]);
        l4[j] = l;
    }
    wave_sum_n(l4);
    for (int j = 0; j < 4; ++j) {
        const int qb = w + 16 * j;
        if (qb >= nb) break;
        const float* row = rows + qb * kP;
        const double inv = 1.0 / (l4[j] * (double)nb);
        float* out = L.vals + tri(qb);
        for (int k2 = lane; k2 <= qb; k2 += 64) out[k2] = (float)((double)exp2f(row[k2] - m4[j]) * inv);
    }
    __syncthreads();                              // the histograms reuse qs / ks
}

__device__ PeState pe_cut_small(SmallCutLds& L, const float* __restrict__ base, int nb, float gamma)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int total = nb * (nb + 1) / 2;
    if (base)                                   // else the map is in L.vals already
        for (int e = tid; e < total; e += 1024) L.vals[e] = base[e];
    PeState st = {};
    st.need = (unsigned long long)((double)gamma * kFix);
    // nothing reaches a zero need: only the always-kept blocks (K* = 0)
    if (st.need == 0) return st;
    if (tid == 0) L.st = st;
    for (int pass = 0; pass < kSmallPasses; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = lane; i < kSmallBins; i += 64) {
            L.x.h.wcnt[w][i] = 0u;
            L.x.h.wmass[w][i] = 0ull;
        }
        __syncthreads();
        st = L.st;
        if (st.done) break;
        // The entries whose higher digits match the ones resolved so far.
        // The values of a map span few binades, so in the first pass most
        // lanes of a wavefront share one of a few digits: there the
        // wavefront first folds up to kFoldRounds groups of lanes with equal
        // digits, one lane adding each group's count and mass (its own
        // histogram copy, so a plain update), and only the remaining lanes
        // add atomically.  (The later passes' digits are mantissa bits,
        // rarely shared: folding there cost more than it saved.)  Integer
        // sums: the same totals in any order.
        for (int e0 = 64 * w; e0 < total; e0 += 1024) {
            const int e = e0 + lane;
            bool act = false;
            uint32_t d = 0;
            unsigned long long fx = 0;
            if (e < total) {
                const float v = L.vals[e];
                const uint32_t key = ~__float_as_uint(v);
                act = pass == 0 || (key >> (shift + 8)) == st.key_prefix;
                d = (key >> shift) & (kSmallBins - 1);
                fx = to_fix(v);
            }
            unsigned long long pend = pass == 0 ? __ballot(act) : 0ull;
            for (int r = 0; r < kFoldRounds && pend; ++r) {
                const int leader = __builtin_ctzll(pend);
                const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
                const bool mt = act && d == ld;
                const unsigned long long mm = __ballot(mt);
                const unsigned long long sum = last_lane(wave_scan_incl(mt ? fx : 0ull));
                if (lane == leader) {
                    L.x.h.wcnt[w][ld] += (uint32_t)__popcll(mm);
                    L.x.h.wmass[w][ld] += sum;
                }
                act = act && !mt;
                pend &= ~mm;
            }
            if (act) {
                atomicAdd(&L.x.h.wcnt[w][d], 1u);
                atomicAdd(&L.x.h.wmass[w][d], fx);
            }
        }
        __syncthreads();
        {
            const int bin = tid & (kSmallBins - 1), part = tid >> 8;
            uint32_t c = 0;
            unsigned long long m = 0;
            for (int x = 4 * part; x < 4 * part + 4; ++x) {
                c += L.x.h.wcnt[x][bin];
                m += L.x.h.wmass[x][bin];
            }
            L.x.h.pcnt[part][bin] = c;
            L.x.h.pmass[part][bin] = m;
        }
        __syncthreads();
        if (w == 0) {
            // lane l holds bins 4l .. 4l + 3; scan the lanes' totals
            uint32_t c[4], c_lane = 0;
            unsigned long long m[4], m_lane = 0;
            for (int j = 0; j < 4; ++j) {
                const int bin = 4 * lane + j;
                c[j] = (L.x.h.pcnt[0][bin] + L.x.h.pcnt[1][bin]) + (L.x.h.pcnt[2][bin] + L.x.h.pcnt[3][bin]);
                m[j] = (L.x.h.pmass[0][bin] + L.x.h.pmass[1][bin]) + (L.x.h.pmass[2][bin] + L.x.h.pmass[3][bin]);
                c_lane += c[j];
                m_lane += m[j];
            }
            const uint32_t c_incl = wave_scan_incl(c_lane);
            const unsigned long long m_incl = wave_scan_incl(m_lane);
            const unsigned long long m_all = last_lane(m_incl);
            uint32_t c_before = c_incl - c_lane;
            unsigned long long m_before = m_incl - m_lane;
            if (m_all < st.need) {
                // (first pass only) the whole map never reaches gamma: keep
                // every causal entry
                if (lane == 0) {
                    PeState nx = st;
                    nx.key_star = 0xffffffffu;
                    nx.flat_star = 0xffffffffu;
                    nx.kstar = (uint32_t)total;
                    nx.done = 1u;
                    L.st = nx;
                }
            } else if (m_before < st.need && m_incl >= st.need) {
                for (int j = 0; j < 4; ++j) {
                    const unsigned long long incl = m_before + m[j];
                    if (m_before < st.need && incl >= st.need) {
                        PeState nx = st;
                        nx.need = st.need - m_before;
                        nx.before = st.before + c_before;
                        nx.key_prefix = (st.key_prefix << 8) | (uint32_t)(4 * lane + j);
                        L.st = nx;
                        L.bin_count = c[j];
                    }
                    m_before = incl;
                    c_before += c[j];
                }
            }
        }
    }
    __syncthreads();
    st = L.st;
    if (st.done) return st;
    // key_prefix is now the whole cut-off key: take just enough of its
    // equal-valued entries, in flat order
    const uint32_t key_star = st.key_prefix;
    const unsigned long long tf = to_fix(__uint_as_float(~key_star));
    const unsigned long long ties = (st.need + tf - 1) / tf;
    const uint32_t cnt = L.bin_count;
    st.key_star = key_star;
    st.tfix = tf;
    st.done = 1u;
    if (ties >= cnt) {
        st.flat_star = 0xffffffffu;
        st.kstar = st.before + cnt;
        return st;
    }
    st.tie_need = (uint32_t)ties;
    st.kstar = st.before + (uint32_t)ties;
    const int per = (total + 1023) / 1024;
    const int e0 = min(total, tid * per), e1 = min(total, e0 + per);
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += ~__float_as_uint(L.vals[e]) == key_star;
    int all;
    const int excl = block_scan_1024(mine, L.scan, &all);    // ends with a barrier
    if (excl < (int)ties && excl + mine >= (int)ties) {
        int seen = excl;
        for (int e = e0; e < e1; ++e) {
            if (~__float_as_uint(L.vals[e]) != key_star || ++seen < (int)ties) continue;
            int qb = (int)((sqrtf(8.0f * (float)e + 1.0f) - 1.0f) * 0.5f);
            while (tri(qb + 1) <= (size_t)e) ++qb;
            while (tri(qb) > (size_t)e) --qb;
            L.st.flat_star = (uint32_t)qb * (uint32_t)nb + (uint32_t)(e - (int)tri(qb));
            break;
        }
    }
    __syncthreads();
    st.flat_star = st.flat_prefix = L.st.flat_star;
    return st;
}

// grid (ceil(tri(Nb) / kRadixChunk), hq), 256 threads
__global__ void __launch_bounds__(256)
pe_radix_kernel(int nb, int pass,
                const float* __restrict__ abar, PeState* __restrict__ state,
                unsigned long long* __restrict__ hist_mass, uint32_t* __restrict__ hist_count,
                uint32_t* __restrict__ pass_ctr)
{
    __shared__ uint32_t cnt[kFlatBins];
    __shared__ unsigned long long mass[kValBins];
    __shared__ unsigned long long wsum_m[4];
    __shared__ uint32_t wsum_c[4];
    __shared__ int s_last;
    const int h = blockIdx.y, tid = threadIdx.x;
    const PeState st = state[h];
    if (st.done) return;                // VS heads start done (pe_init_kernel)
    const bool val = pass < kValPasses;
    const int bins = 1 << pass_bits(pass);
    for (int i = tid; i < bins; i += 256) {
        cnt[i] = 0u;
        if (val) mass[i] = 0ull;
    }
    __syncthreads();
    const size_t total = tri(nb);
    const float* base = abar + (size_t)h * total;
    const size_t e0 = (size_t)blockIdx.x * kRadixChunk;
    const size_t e1 = min(total, e0 + kRadixChunk);
    // all of this thread's entries in flight at once
    constexpr int kPer = kRadixChunk / 256;
    float vals[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const size_t e = e0 + tid + 256 * j;
        vals[j] = (e < e1) ? base[e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const size_t e = e0 + tid + 256 * j;
        if (e >= e1) break;
        radix_add(pass, nb, st, e, vals[j], cnt, mass);
    }
    __syncthreads();
    uint32_t* gc = hist_count + ((size_t)h * kRadixPasses + pass) * kFlatBins;
    unsigned long long* gm = hist_mass + ((size_t)h * kValPasses + (val ? pass : 0)) * kValBins;
    for (int i = tid; i < bins; i += 256) {
        if (cnt[i]) {
            atomicAdd(&gc[i], cnt[i]);
            if (val) atomicAdd(&gm[i], mass[i]);
        }
    }
    // The histogram atomics are performed at the device's coherence point;
    // waiting for them to complete (vmcnt) before the counter increment
    // orders them without a cache write-back (a __threadfence() writes back
    // and invalidates the XCD's L2, which costs more than the pass itself).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t nwg = gridDim.x;
        s_last = atomicAdd(&pass_ctr[h * kRadixPasses + pass], 1u) == nwg - 1;
    }
    __syncthreads();
    if (!s_last) return;
    // every other work-group's atomics are complete: read them coherently

    // ---- resolve: this work-group saw every other one finish the pass ----
    const int per = bins / 256;                       // consecutive bins per thread
    for (int j = 0; j < per; ++j) {
        const int i = tid * per + j;
        cnt[i] = __hip_atomic_load(&gc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (val) mass[i] = __hip_atomic_load(&gm[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    radix_resolve(pass, total, st, cnt, mass, wsum_c, wsum_m, &state[h]);
}

// Block-list membership of (qb, kb) for one head: VS rows from the two
// direction bitmaps, PE rows from the gamma cut-off (key_star, flat_star).
struct RowRule {
    bool vs;
    int nb;
    const uint8_t* bmv;       // LDS copies of the head's bitmaps (VS)
    const uint8_t* bms;
    const float* arow;        // head's triangular pooled map (PE)
    uint32_t key_star, flat_star;

    __device__ bool member(int qb, int kb) const
    {
        if (kb > qb) return false;
        if (kb == 0 || kb == qb) return true;
        if (vs) return bmv[kb] || bms[nb - 1 - (qb - kb)];
        const uint32_t key = ~__float_as_uint(arow[tri(qb) + kb]);
        return key < key_star ||
               (key == key_star && (uint32_t)qb * (uint32_t)nb + (uint32_t)kb <= flat_star);
    }
};

constexpr int kRowsPerGroup = 64;   // query blocks per work-group of the expansion

__device__ RowRule load_rule(const uint8_t* __restrict__ pattern, int nb, int h,
                             const uint8_t* __restrict__ bitmap, const float* __restrict__ abar,
                             const PeState* __restrict__ state, uint8_t* bmv, uint8_t* bms)
{
    RowRule r;
    r.vs = pattern[h] != 0;
    r.nb = nb;
    r.bmv = bmv;
    r.bms = bms;
    r.arow = abar + (size_t)h * tri(nb);
    r.key_star = r.flat_star = 0;
    if (r.vs) {
        for (int j = threadIdx.x; j < nb; j += blockDim.x) {
            bmv[j] = bitmap[((size_t)h * 2) * nb + j];
            bms[j] = bitmap[((size_t)h * 2 + 1) * nb + j];
        }
    } else {
        r.key_star = state[h].key_star;
        r.flat_star = state[h].flat_star;
    }
    __syncthreads();
    return r;
}

// grid (ceil(Nb / 64), hq), 1024 threads: the length of each row, written
// into row_ptr[h][qb] (scanned in place by expand_scan_kernel), and the
// row's membership ballots, one 64-bit word per 64 key blocks, into
// rowmask[h][qb][0 .. ceil((qb + 1) / 64)), so that expand_fill_kernel
// neither reads the pooled map again nor re-evaluates the rule.
__global__ void __launch_bounds__(1024)
expand_count_kernel(const uint8_t* __restrict__ pattern, int nb, const uint8_t* __restrict__ bitmap,
                    const float* __restrict__ abar, const PeState* __restrict__ state,
                    int32_t* __restrict__ row_ptr, unsigned long long* __restrict__ rowmask)
{
    __shared__ uint8_t bmv[kMaxBlocks];
    __shared__ uint8_t bms[kMaxBlocks];
    const int h = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const RowRule rule = load_rule(pattern, nb, h, bitmap, abar, state, bmv, bms);
    const int nw = (nb + 63) / 64;
    const int q0 = blockIdx.x * kRowsPerGroup, q1 = min(nb, q0 + kRowsPerGroup);
    for (int qb = q0 + w; qb < q1; qb += 16) {
        unsigned long long* m = rowmask + ((size_t)h * nb + qb) * nw;
        const int chunks = (qb >> 6) + 1;
        int c = 0;
        // eight chunks' tests (map reads for PE heads) in flight before the
        // ballots consume them
        for (int c0 = 0; c0 < chunks; c0 += 8) {
            bool mb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) mb[j] = c0 + j < chunks && rule.member(qb, 64 * (c0 + j) + lane);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + j >= chunks) break;
                const unsigned long long bal = __ballot(mb[j]);
                c += __popcll(bal);
                if (lane == 0) m[c0 + j] = bal;
            }
        }
        if (lane == 0) row_ptr[(size_t)h * (nb + 1) + qb] = c;
    }
}

// grid hq, 1024 threads: exclusive scan of the row lengths into absolute
// offsets (head h's lists start at h * Nb (Nb + 1) / 2), and K*.
__global__ void __launch_bounds__(1024)
expand_scan_kernel(const uint8_t* __restrict__ pattern, int nb, const PeState* __restrict__ state,
                   int32_t* __restrict__ row_ptr, int32_t* __restrict__ counts)
{
    __shared__ int wsum[16];
    const int h = blockIdx.x, tid = threadIdx.x;
    const size_t base = (size_t)h * tri(nb);
    int32_t* rp = row_ptr + (size_t)h * (nb + 1);
    int len[4], mine = 0;
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        len[e] = (j < nb) ? rp[j] : 0;
        mine += len[e];
    }
    int total;
    int start = block_scan_1024(mine, wsum, &total);
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        if (j >= nb) break;
        rp[j] = (int32_t)(base + start);
        start += len[e];
    }
    if (tid == 0) {
        rp[nb] = (int32_t)(base + total);
        counts[h * 3 + 2] = pattern[h] ? 0 : (int32_t)state[h].kstar;
    }
}

// grid (ceil(Nb / 64), hq), 1024 threads: ascending key blocks of each row,
// from the membership ballots expand_count_kernel stored.
__global__ void __launch_bounds__(1024)
expand_fill_kernel(int nb, const unsigned long long* __restrict__ rowmask,
                   const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx)
{
    const int h = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nw = (nb + 63) / 64;
    const int q0 = blockIdx.x * kRowsPerGroup, q1 = min(nb, q0 + kRowsPerGroup);
    for (int qb = q0 + w; qb < q1; qb += 16) {
        const unsigned long long* m = rowmask + ((size_t)h * nb + qb) * nw;
        const int chunks = (qb >> 6) + 1;                 // at most 64 (N_b <= 4096)
        // lane j holds the row's ballot word j: one load for the whole row
        const unsigned long long word = lane < chunks ? m[lane] : 0ull;
        size_t pos = (size_t)row_ptr[(size_t)h * (nb + 1) + qb];
        for (int j = 0; j < chunks; ++j) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)word, j);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(word >> 32), j);
            const unsigned long long bal = ((unsigned long long)hi << 32) | lo;
            if ((bal >> lane) & 1ull) col_idx[pos + __popcll(bal & below)] = 64 * j + lane;
            pos += __popcll(bal);
        }
    }
}

// The block lists of head h under `rule` by one 1024-thread block
// (N_b <= kSelectSmall): the row lengths, their exclusive scan into
// absolute offsets (head h's lists start at h N_b (N_b + 1) / 2), then the
// ascending key blocks of every row; K* (0 for VS heads) into counts.  The
// same rows, offsets and K* as expand_count, expand_scan and expand_fill.
static_assert(kSelectSmall * (kSelectSmall + 1) / 2 == kRadixSmall, "one small-map bound");

__device__ void expand_head(const RowRule& rule, int h, int nb, uint32_t kstar,
                            int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                            int32_t* __restrict__ counts, int* start, int* wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int qb = w; qb < nb; qb += 16) {
        int c = 0;
        for (int kb0 = 0; kb0 <= qb; kb0 += 64) c += __popcll(__ballot(rule.member(qb, kb0 + lane)));
        if (lane == 0) start[qb] = c;
    }
    __syncthreads();
    const size_t base = (size_t)h * tri(nb);
    int32_t* rp = row_ptr + (size_t)h * (nb + 1);
    int len[4], mine = 0;
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        len[e] = (j < nb) ? start[j] : 0;
        mine += len[e];
    }
    int total;
    int at = block_scan_1024(mine, wsum, &total);    // ends with a barrier
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        if (j >= nb) break;
        start[j] = (int)base + at;
        rp[j] = (int32_t)(base + at);
        at += len[e];
    }
    if (tid == 0) {
        rp[nb] = (int32_t)(base + total);
        counts[h * 3 + 2] = rule.vs ? 0 : (int32_t)kstar;
    }
    __syncthreads();
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int qb = w; qb < nb; qb += 16) {
        size_t pos = (size_t)start[qb];
        for (int kb0 = 0; kb0 <= qb; kb0 += 64) {
            const bool mbr = rule.member(qb, kb0 + lane);
            const unsigned long long bal = __ballot(mbr);
            if (mbr) col_idx[pos + __popcll(bal & below)] = kb0 + lane;
            pos += __popcll(bal);
        }
    }
}

struct SelectSmallLds {
    union {
        SmallCutLds cut;
        VsLds<kSelectSmall> vs;
    } u;
    uint8_t bmv[kSelectSmall];
    uint8_t bms[kSelectSmall];
    int start[kSelectSmall];
    int wsum[16];
};

// V^T images per work-group of select_small_kernel's layout part: one per
// 256 threads, staged in the selection's LDS.
constexpr int kVtPerGroup = 4;
static_assert(kVtPerGroup * 64 * kVPitch * sizeof(uint16_t) <= sizeof(SelectSmallLds), "V^T tiles fit");

// grid hq (+ the V^T layout's work-groups), 1024 threads, N_b <=
// kSelectSmall: the whole selection of one head in one work-group, after
// routing and pooling (and, for N_b > kMapSmall, the pooled map from
// pe_logits_kernel): a VS head's two budget selections (as
// vs_select_kernel), or a PE head's pooled map (built here for N_b <=
// kMapSmall, pe_map_small) and gamma cut-off (pe_cut_small; its state also
// goes to state[h]), then the head's block lists (expand_head) from the
// LDS copies of the bitmaps or of the map.  The same outputs as the
// multi-launch path.  The hq selection work-groups occupy hq compute
// units for the launch's whole length; work-groups hq onward lay out V^T
// meanwhile on the rest of the chip (the images v_transpose_kernel writes,
// kVtPerGroup each; the first also clears queue), so that layout costs no
// launch of its own.
template <class R>
__global__ void __launch_bounds__(1024)
select_small_kernel(const uint8_t* __restrict__ pattern, const float* __restrict__ p_v,
                    const float* __restrict__ p_s, int nb, VsRule vr, float gamma,
                    const float* __restrict__ qbar, const float* __restrict__ kbar, int G,
                    float scale_log2, const float* __restrict__ abar, int32_t* __restrict__ sel_v,
                    int32_t* __restrict__ sel_s, int32_t* __restrict__ counts,
                    PeState* __restrict__ state, int32_t* __restrict__ row_ptr,
                    int32_t* __restrict__ col_idx, int hq, R v, int n, int hkv,
                    uint16_t* __restrict__ vt, int* __restrict__ queue)
{
    __shared__ SelectSmallLds L;
    if ((int)blockIdx.x >= hq) {                 // V^T layout work-group
        const int tid = threadIdx.x & 255, part = threadIdx.x >> 8;
        const int n_img = 2 * nb;
        const int img = ((int)blockIdx.x - hq) * kVtPerGroup + part;    // g n_img + i
        uint16_t (*tile)[kVPitch] = reinterpret_cast<uint16_t (*)[kVPitch]>(&L) + 64 * part;
        if (blockIdx.x == (unsigned)hq && threadIdx.x < 8) queue[threadIdx.x] = 0;
        const bool live = img < hkv * n_img;
        if (live) v_image_stage(v, n, img / n_img, img % n_img, tile, tid);
        __syncthreads();
        if (live) v_image_write(tile, vt + (size_t)img * kVImage, tid);
        return;
    }
    const int h = blockIdx.x;
    RowRule rule;
    rule.vs = pattern[h] != 0;
    rule.nb = nb;
    rule.bmv = L.bmv;
    rule.bms = L.bms;
    rule.arow = L.u.cut.vals;
    rule.key_star = rule.flat_star = 0;
    uint32_t kstar = 0;
    if (rule.vs) {
        vs_select_dir(L.u.vs, h, 0, p_v + (size_t)h * nb, nb, vr, sel_v + (size_t)h * nb, counts,
                      L.bmv);
        __syncthreads();
        vs_select_dir(L.u.vs, h, 1, p_s + (size_t)h * nb, nb, vr, sel_s + (size_t)h * nb, counts,
                      L.bms);
    } else {
        const float* map = abar + (size_t)h * tri(nb);
        if (nb <= kMapSmall) {
            pe_map_small(L.u.cut, qbar + (size_t)h * nb * kD, kbar + (size_t)(h / G) * nb * kD, nb,
                         scale_log2);
            map = nullptr;
        }
        const PeState st = pe_cut_small(L.u.cut, map, nb, gamma);
        if (threadIdx.x == 0) {
            state[h] = st;
            counts[h * 3] = 0;
            counts[h * 3 + 1] = 0;
        }
        rule.key_star = st.key_star;
        rule.flat_star = st.flat_star;
        kstar = st.kstar;
    }
    __syncthreads();
    expand_head(rule, h, nb, kstar, row_ptr, col_idx, counts, L.start, L.wsum);
}

}  // namespace

template <class R>
hipError_t launch_select(R q, R k, const uint8_t* pattern,
                         const float* p_v, const float* p_s, int n, int hq, int hkv,
                         const VsRule& vs, float gamma, const SelectScratch& s, int32_t* sel_v,
                         int32_t* sel_s, int32_t* sel_counts, int32_t* row_ptr, int32_t* col_idx,
                         const VtJob<R>& vt, hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv;
    hipError_t e;
#define CRISP_CHECK_LAUNCH() \
    if ((e = hipGetLastError()) != hipSuccess) return e
    const bool small = nb <= kSelectSmall;
    if (!small) {
        hipLaunchKernelGGL(vs_select_kernel, dim3(hq, 2), dim3(1024), 0, stream, pattern, p_v, p_s,
                           nb, vs, sel_v, sel_s, sel_counts, s.bitmap);
        CRISP_CHECK_LAUNCH();
        hipLaunchKernelGGL(pe_init_kernel, dim3(hq), dim3(1024), 0, stream, pattern, gamma,
                           s.hist_mass, s.hist_count, s.pass_ctr, s.state);
        CRISP_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(HIP_KERNEL_NAME(pe_pool_kernel<R>), dim3(nb, hq + hkv), dim3(256), 0, stream, q, k, pattern, n,
                       hq, G, s.qbar, s.kbar);
    CRISP_CHECK_LAUNCH();
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    const int fuse_softmax = small;              // one work-group per 32 whole rows
    if (nb > kMapSmall) {                        // else select_small_kernel builds the map
        hipLaunchKernelGGL(pe_logits_kernel, dim3((nb + 31) / 32, (nb + 127) / 128, hq), dim3(256), 0,
                           stream, s.qbar, s.kbar, pattern, nb, G, scale_log2, fuse_softmax, s.abar);
        CRISP_CHECK_LAUNCH();
    }
    if (small) {
        const int vt_groups = vt.vt ? (hkv * 2 * nb + kVtPerGroup - 1) / kVtPerGroup : 0;
        hipLaunchKernelGGL(HIP_KERNEL_NAME(select_small_kernel<R>), dim3(hq + vt_groups), dim3(1024), 0,
                           stream, pattern, p_v, p_s, nb, vs, gamma, s.qbar, s.kbar, G, scale_log2,
                           s.abar, sel_v, sel_s, sel_counts, s.state, row_ptr, col_idx, hq, vt.v, n,
                           hkv, vt.vt, vt.queue);
        CRISP_CHECK_LAUNCH();
        return hipSuccess;
    }
    hipLaunchKernelGGL(pe_softmax_kernel, dim3((nb + 3) / 4, hq), dim3(256), 0, stream, pattern, nb,
                       s.abar);
    CRISP_CHECK_LAUNCH();
    const long long tri_nb = (long long)nb * (nb + 1) / 2;
    const dim3 radix_grid((unsigned)((tri_nb + kRadixChunk - 1) / kRadixChunk), hq);
    for (int pass = 0; pass < kRadixPasses; ++pass) {
        hipLaunchKernelGGL(pe_radix_kernel, radix_grid, dim3(256), 0, stream, nb, pass, s.abar,
                           s.state, s.hist_mass, s.hist_count, s.pass_ctr);
        CRISP_CHECK_LAUNCH();
    }
    const dim3 rows_grid((nb + kRowsPerGroup - 1) / kRowsPerGroup, hq);
    hipLaunchKernelGGL(expand_count_kernel, rows_grid, dim3(1024), 0, stream, pattern, nb, s.bitmap,
                       s.abar, s.state, row_ptr, s.rowmask);
    CRISP_CHECK_LAUNCH();
    hipLaunchKernelGGL(expand_scan_kernel, dim3(hq), dim3(1024), 0, stream, pattern, nb, s.state,
                       row_ptr, sel_counts);
    CRISP_CHECK_LAUNCH();
    hipLaunchKernelGGL(expand_fill_kernel, rows_grid, dim3(1024), 0, stream, nb, s.rowmask, row_ptr,
                       col_idx);
    CRISP_CHECK_LAUNCH();
#undef CRISP_CHECK_LAUNCH
    return hipSuccess;
}

template hipError_t launch_select<Rows>(Rows, Rows, const uint8_t*, const float*, const float*, int,
                                        int, int, const VsRule&, float, const SelectScratch&, int32_t*,
                                        int32_t*, int32_t*, int32_t*, int32_t*, const VtJob<Rows>&,
                                        hipStream_t);
template hipError_t launch_select<SeqRows>(SeqRows, SeqRows, const uint8_t*, const float*,
                                           const float*, int, int, int, const VsRule&, float,
                                           const SelectScratch&, int32_t*, int32_t*, int32_t*,
                                           int32_t*, int32_t*, const VtJob<SeqRows>&, hipStream_t);

}  // namespace crisp
