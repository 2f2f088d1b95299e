// Index selection and block-list expansion kernels.
//
//   vs_select_kernel   sink-aware noise floor per VS direction (Alg. 3,
//                      lines 7-12; Eq. 3-4) with stream compaction
//   pe_*_kernel        pooled estimation for PE heads (Alg. 4): block-mean
//                      pooling of Q and K, the causal pooled softmax map,
//                      normalisation, and the gamma-cumsum cut-off found by a
//                      mass-weighted radix select on the float bits instead
//                      of a full sort
//   expand_kernel      per-(head, query block) key-block lists (the block
//                      mask M_S of Eq. 1), CSR with per-head worst-case bases
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
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        int s = (lane < 16) ? wsum[lane] : 0;
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(s, o);
            if (lane >= o) s += y;
        }
        if (lane < 16) wsum[lane] = s;
    }
    __syncthreads();
    const int excl = (w > 0 ? wsum[w - 1] : 0) + x - v;
    *total = wsum[15];
    __syncthreads();
    return excl;
}

// grid (hq, 2): direction 0 = vertical (p_v), 1 = slash (p_s).
__global__ void __launch_bounds__(1024)
vs_select_kernel(const uint8_t* __restrict__ pattern, const float* __restrict__ p_v,
                 const float* __restrict__ p_s, int nb, float alpha, int kmin,
                 int32_t* __restrict__ sel_v, int32_t* __restrict__ sel_s,
                 int32_t* __restrict__ counts, uint8_t* __restrict__ bitmap)
{
    __shared__ int wsum[16];
    __shared__ float best_v[16];
    __shared__ int best_i[16];
    __shared__ uint8_t flag[kMaxBlocks];

    const int h = blockIdx.x, dir = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    if (!pattern[h]) {
        if (tid == 0) counts[h * 3 + dir] = 0;
        return;
    }
    const float* p = (dir ? p_s : p_v) + (size_t)h * nb;
    int32_t* sel = (dir ? sel_s : sel_v) + (size_t)h * nb;
    uint8_t* bm = bitmap + ((size_t)h * 2 + dir) * nb;

    // Eq. 3: mu over the N_b - 2 non-retained blocks; Eq. 4: p_j > alpha * mu
    float theta = -INFINITY;
    if (nb > 2) {
        float r = 1.0f - p[0];
        r = r - p[nb - 1];
        r = fmaxf(r, 0.0f);
        const float mu = r / (float)(nb - 2);
        theta = alpha * mu;
    }
    float pv[4];
    int cnt = 0;
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        pv[e] = (j < nb) ? p[j] : -INFINITY;
        const bool f = (j < nb) && (pv[e] > theta);
        flag[j] = f;
        cnt += f;
    }
    int total;
    block_scan_1024(cnt, wsum, &total);
    if (total < kmin && total < nb) {
        // clip to k_min: top-k_min by (p desc, index asc)
        const int kk = min(kmin, nb);
        for (int e = 0; e < 4; ++e) flag[4 * tid + e] = 0;
        __syncthreads();
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
            if (lane == 0) { best_v[w] = bv; best_i[w] = bi; }
            __syncthreads();
            if (tid == 0) {
                float v = best_v[0];
                int i = best_i[0];
                for (int x = 1; x < 16; ++x)
                    if (best_v[x] > v || (best_v[x] == v && best_i[x] < i)) { v = best_v[x]; i = best_i[x]; }
                flag[i] = 1;
            }
            __syncthreads();
        }
        cnt = 0;
        for (int e = 0; e < 4; ++e) cnt += flag[4 * tid + e];
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

__global__ void pe_init_kernel(const uint8_t* __restrict__ pattern, float gamma,
                               unsigned long long* __restrict__ hist_mass,
                               uint32_t* __restrict__ hist_count, PeState* __restrict__ state)
{
    const int h = blockIdx.x, tid = threadIdx.x;
    hist_mass[h * 256 + tid] = 0ull;
    hist_count[h * 256 + tid] = 0u;
    if (tid == 0) {
        PeState s = {};
        s.need = (unsigned long long)((double)gamma * kFix);
        s.done = pattern[h] ? 1u : 0u;
        state[h] = s;
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
__global__ void __launch_bounds__(256)
pe_pool_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint8_t* __restrict__ pattern, int n, int hq, int G,
               float* __restrict__ qbar, float* __restrict__ kbar)
{
    __shared__ float red[16][kD];
    const int qb = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
    const int nb = (n + kB - 1) / kB;
    const int len = min(kB, n - qb * kB);           // tokens in block qb
    const uint16_t* src;
    float* dst;
    if (y < hq) {
        if (pattern[y]) return;
        src = q + ((size_t)y * n + (size_t)qb * kB) * kD;
        dst = qbar + ((size_t)y * nb + qb) * kD;
    } else {
        const int g = y - hq;
        if (!group_has_pe(pattern, g, G)) return;
        src = k + ((size_t)g * n + (size_t)qb * kB) * kD;
        dst = kbar + ((size_t)g * nb + qb) * kD;
    }
    const int dc = tid & 15, tg = tid >> 4;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = tg * 8; t < min(tg * 8 + 8, len); ++t) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (size_t)t * kD + 8 * dc);
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

// grid (ceil(Nb/16), hq): scaled pooled logits of 16 query blocks against
// every causal key block, log2 domain, triangular row layout.
__global__ void __launch_bounds__(256)
pe_logits_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                 const uint8_t* __restrict__ pattern, int nb, int G, float scale_log2,
                 float* __restrict__ abar)
{
    __shared__ float qs[16][kD];
    __shared__ float kst[64][kD + 1];
    const int h = blockIdx.y, tid = threadIdx.x;
    if (pattern[h]) return;
    const int g = h / G;
    const int r0 = blockIdx.x * 16;
    const size_t tri_total = tri(nb);
    for (int e = tid; e < 16 * kD; e += 256) {
        const int r = e / kD, c = e % kD;
        qs[r][c] = (r0 + r < nb) ? qbar[((size_t)h * nb + r0 + r) * kD + c] : 0.f;
    }
    const int row = tid >> 4, c4 = (tid & 15) * 4;
    const int qb = r0 + row;
    const int kb_end = min(nb, r0 + 16);
    for (int kb0 = 0; kb0 < kb_end; kb0 += 64) {
        __syncthreads();
        for (int e = tid; e < 64 * kD; e += 256) {
            const int r = e / kD, c = e % kD;
            kst[r][c] = (kb0 + r < nb) ? kbar[((size_t)g * nb + kb0 + r) * kD + c] : 0.f;
        }
        __syncthreads();
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < kD; ++c) {
            const float x = qs[row][c];
            for (int j = 0; j < 4; ++j) acc[j] += x * kst[c4 + j][c];
        }
        for (int j = 0; j < 4; ++j) {
            const int kb = kb0 + c4 + j;
            if (qb < nb && kb <= qb) abar[(size_t)h * tri_total + tri(qb) + kb] = acc[j] * scale_log2;
        }
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

// One radix digit of the cut-off: pass 0..3 histogram the value key (value
// descending == key ascending) 8 bits at a time, weighting by mass; pass
// 4..6 histogram the flat index qb*Nb+kb of the entries equal to the cut-off
// value, by count.  grid (ceil(Nb/8), hq).
__global__ void __launch_bounds__(256)
pe_hist_kernel(const uint8_t* __restrict__ pattern, int nb, int pass,
               const float* __restrict__ abar, const PeState* __restrict__ state,
               unsigned long long* __restrict__ hist_mass, uint32_t* __restrict__ hist_count)
{
    __shared__ uint32_t cnt[256];
    __shared__ unsigned long long mass[256];
    const int h = blockIdx.y, tid = threadIdx.x;
    if (pattern[h]) return;
    const PeState st = state[h];
    if (st.done) return;
    cnt[tid] = 0u;
    mass[tid] = 0ull;
    __syncthreads();
    const float* base = abar + (size_t)h * tri(nb);
    const int r0 = blockIdx.x * 8, r1 = min(nb, r0 + 8);
    for (int qb = r0; qb < r1; ++qb) {
        const float* row = base + tri(qb);
        for (int kb = tid; kb <= qb; kb += 256) {
            const float v = row[kb];
            const uint32_t key = ~__float_as_uint(v);
            if (pass < 4) {
                const int shift = 24 - 8 * pass;
                if (pass > 0 && (key >> (shift + 8)) != st.key_prefix) continue;
                const int dgt = (key >> shift) & 255;
                atomicAdd(&cnt[dgt], 1u);
                atomicAdd(&mass[dgt], to_fix(v));
            } else {
                if (key != st.key_star) continue;
                const uint32_t flat = (uint32_t)qb * (uint32_t)nb + (uint32_t)kb;
                const int shift = 16 - 8 * (pass - 4);
                if (pass > 4 && (flat >> (shift + 8)) != st.flat_prefix) continue;
                atomicAdd(&cnt[(flat >> shift) & 255], 1u);
            }
        }
    }
    __syncthreads();
    if (cnt[tid]) {
        atomicAdd(&hist_count[h * 256 + tid], cnt[tid]);
        if (pass < 4) atomicAdd(&hist_mass[h * 256 + tid], mass[tid]);
    }
}

// grid hq, 256 threads (one per digit): pick the digit where the running
// mass (count, for flat passes) reaches what is still needed.
__global__ void __launch_bounds__(256)
pe_resolve_kernel(const uint8_t* __restrict__ pattern, int nb, int pass,
                  unsigned long long* __restrict__ hist_mass, uint32_t* __restrict__ hist_count,
                  PeState* __restrict__ state)
{
    __shared__ unsigned long long smass[256];
    __shared__ uint32_t scnt[256];
    __shared__ PeState cur;
    const int h = blockIdx.x, tid = threadIdx.x;
    if (pattern[h]) return;
    if (tid == 0) cur = state[h];
    __syncthreads();
    if (cur.done) return;
    const uint32_t c = hist_count[h * 256 + tid];
    const unsigned long long m = hist_mass[h * 256 + tid];
    scnt[tid] = c;
    smass[tid] = m;
    __syncthreads();
    // inclusive scans (Hillis-Steele; 256 entries)
    for (int o = 1; o < 256; o <<= 1) {
        const uint32_t yc = (tid >= o) ? scnt[tid - o] : 0u;
        const unsigned long long ym = (tid >= o) ? smass[tid - o] : 0ull;
        __syncthreads();
        scnt[tid] += yc;
        smass[tid] += ym;
        __syncthreads();
    }
    hist_count[h * 256 + tid] = 0u;
    hist_mass[h * 256 + tid] = 0ull;
    const uint32_t incl_c = scnt[tid], excl_c = incl_c - c;
    const unsigned long long incl_m = smass[tid], excl_m = incl_m - m;
    PeState& st = state[h];   // written by exactly one thread below
    if (pass < 4) {
        const unsigned long long need = cur.need;
        if (smass[255] < need) {
            // the kept mass never reaches gamma: keep every causal entry
            if (tid == 0) {
                PeState nx = cur;
                nx.key_star = 0xffffffffu;
                nx.flat_star = 0xffffffffu;
                nx.kstar = (uint32_t)tri(nb);
                nx.done = 1u;
                st = nx;
            }
            return;
        }
        if (incl_m >= need && excl_m < need) {
            PeState nx = cur;
            nx.need = need - excl_m;
            nx.before = cur.before + excl_c;
            nx.key_prefix = (cur.key_prefix << 8) | (uint32_t)tid;
            if (pass == 3) {
                nx.key_star = nx.key_prefix;
                const float tv = __uint_as_float(~nx.key_star);
                const unsigned long long tf = to_fix(tv);
                const unsigned long long ties = (nx.need + tf - 1) / tf;
                nx.tfix = tf;
                if (ties >= c) {
                    nx.flat_star = 0xffffffffu;
                    nx.kstar = nx.before + c;
                    nx.done = 1u;
                } else {
                    nx.tie_need = (uint32_t)ties;
                    nx.kstar = nx.before + (uint32_t)ties;
                }
            }
            st = nx;
        }
    } else {
        const uint32_t need = cur.tie_need;
        if (incl_c >= need && excl_c < need) {
            PeState nx = cur;
            nx.tie_need = need - excl_c;
            nx.flat_prefix = (cur.flat_prefix << 8) | (uint32_t)tid;
            if (pass == 6) {
                nx.flat_star = nx.flat_prefix;
                nx.done = 1u;
            }
            st = nx;
        }
    }
}

// grid hq, 1024 threads: row lengths, per-head scan, fill.
__global__ void __launch_bounds__(1024)
expand_kernel(const uint8_t* __restrict__ pattern, int nb, const uint8_t* __restrict__ bitmap,
              const float* __restrict__ abar, const PeState* __restrict__ state,
              int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
              int32_t* __restrict__ counts)
{
    __shared__ int len[kMaxBlocks];
    __shared__ uint8_t bmv[kMaxBlocks];
    __shared__ uint8_t bms[kMaxBlocks];
    __shared__ int wsum[16];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const bool vs = pattern[h] != 0;
    const size_t tri_total = tri(nb);
    const size_t base = (size_t)h * tri_total;
    const float* arow = abar + base;
    uint32_t key_star = 0, flat_star = 0;
    if (vs) {
        for (int j = tid; j < nb; j += 1024) {
            bmv[j] = bitmap[((size_t)h * 2) * nb + j];
            bms[j] = bitmap[((size_t)h * 2 + 1) * nb + j];
        }
    } else {
        key_star = state[h].key_star;
        flat_star = state[h].flat_star;
    }
    __syncthreads();

    auto member = [&](int qb, int kb) -> bool {
        if (kb > qb) return false;
        if (kb == 0 || kb == qb) return true;
        if (vs) return bmv[kb] || bms[nb - 1 - (qb - kb)];
        const uint32_t key = ~__float_as_uint(arow[tri(qb) + kb]);
        return key < key_star ||
               (key == key_star && (uint32_t)qb * (uint32_t)nb + (uint32_t)kb <= flat_star);
    };

    for (int qb = w; qb < nb; qb += 16) {
        int c = 0;
        for (int kb0 = 0; kb0 <= qb; kb0 += 64) c += __popcll(__ballot(member(qb, kb0 + lane)));
        if (lane == 0) len[qb] = c;
    }
    __syncthreads();
    int mine = 0;
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        mine += (j < nb) ? len[j] : 0;
    }
    int total;
    int start = block_scan_1024(mine, wsum, &total);
    for (int e = 0; e < 4; ++e) {
        const int j = 4 * tid + e;
        if (j >= nb) break;
        const int l = len[j];
        len[j] = start;
        row_ptr[(size_t)h * (nb + 1) + j] = (int32_t)(base + start);
        start += l;
    }
    if (tid == 0) {
        row_ptr[(size_t)h * (nb + 1) + nb] = (int32_t)(base + total);
        counts[h * 3 + 2] = vs ? 0 : (int32_t)state[h].kstar;
    }
    __syncthreads();
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int qb = w; qb < nb; qb += 16) {
        size_t pos = base + len[qb];
        for (int kb0 = 0; kb0 <= qb; kb0 += 64) {
            const bool mbr = member(qb, kb0 + lane);
            const unsigned long long bal = __ballot(mbr);
            if (mbr) col_idx[pos + __popcll(bal & below)] = kb0 + lane;
            pos += __popcll(bal);
        }
    }
}

}  // namespace

hipError_t launch_select(const uint16_t* q, const uint16_t* k, const uint8_t* pattern,
                         const float* p_v, const float* p_s, int n, int hq, int hkv, float alpha,
                         int kmin_blocks, float gamma, const SelectScratch& s, int32_t* sel_v,
                         int32_t* sel_s, int32_t* sel_counts, int32_t* row_ptr, int32_t* col_idx,
                         hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv;
    hipError_t e;
#define CRISP_CHECK_LAUNCH() \
    if ((e = hipGetLastError()) != hipSuccess) return e
    hipLaunchKernelGGL(vs_select_kernel, dim3(hq, 2), dim3(1024), 0, stream, pattern, p_v, p_s, nb,
                       alpha, kmin_blocks, sel_v, sel_s, sel_counts, s.bitmap);
    CRISP_CHECK_LAUNCH();
    hipLaunchKernelGGL(pe_init_kernel, dim3(hq), dim3(256), 0, stream, pattern, gamma, s.hist_mass,
                       s.hist_count, s.state);
    CRISP_CHECK_LAUNCH();
    hipLaunchKernelGGL(pe_pool_kernel, dim3(nb, hq + hkv), dim3(256), 0, stream, q, k, pattern, n,
                       hq, G, s.qbar, s.kbar);
    CRISP_CHECK_LAUNCH();
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    hipLaunchKernelGGL(pe_logits_kernel, dim3((nb + 15) / 16, hq), dim3(256), 0, stream, s.qbar,
                       s.kbar, pattern, nb, G, scale_log2, s.abar);
    CRISP_CHECK_LAUNCH();
    hipLaunchKernelGGL(pe_softmax_kernel, dim3((nb + 3) / 4, hq), dim3(256), 0, stream, pattern, nb,
                       s.abar);
    CRISP_CHECK_LAUNCH();
    for (int pass = 0; pass < 7; ++pass) {
        hipLaunchKernelGGL(pe_hist_kernel, dim3((nb + 7) / 8, hq), dim3(256), 0, stream, pattern, nb,
                           pass, s.abar, s.state, s.hist_mass, s.hist_count);
        CRISP_CHECK_LAUNCH();
        hipLaunchKernelGGL(pe_resolve_kernel, dim3(hq), dim3(256), 0, stream, pattern, nb, pass,
                           s.hist_mass, s.hist_count, s.state);
        CRISP_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(expand_kernel, dim3(hq), dim3(1024), 0, stream, pattern, nb, s.bitmap, s.abar,
                       s.state, row_ptr, col_idx, sel_counts);
    CRISP_CHECK_LAUNCH();
#undef CRISP_CHECK_LAUNCH
    return hipSuccess;
}

}  // namespace crisp
