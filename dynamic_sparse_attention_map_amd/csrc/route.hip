// Routing kernels: proxy map (Alg. 2) and the block-mass
// reduction that yields the vertical / slash scores (Alg. 3),
// C_struct (Eq. 2) and the routing bit (Alg. 2).
//
// The proxy map A^ = Softmax(Q^ K^T / sqrt(d)) over the last R = min(B, n)
// query rows is never stored.  proxy_map_kernel splits the keys into 128-key
// tiles and emits, per (query row i, tile t): the row's maximum scaled logit
// on the tile and the exp-sums of the tile's keys with in-tile column
// c <= b_i ("lower") and c > b_i ("upper"), b_i = q_i mod B for the row's
// position q_i = n - R + i.  A key at column c of tile t sits at offset
// o = q_i - tB - c from the row's diagonal; with q_i = B floor(q_i / B) + b_i
// its offset block is floor(q_i / B) - t for c <= b_i and one less for
// c > b_i, i.e. slash block t + e_i and t + e_i + 1 with
// e_i = N_b - 1 - floor(q_i / B) (0 or 1; always 0 when B divides n).  So
// lower + upper pools the tile's column mass (vertical score) and lower /
// upper split it between two slash blocks.  Four reduction kernels rescale the
// partials with the global row maxima and normalisers.  Under the JSD router
// (FlexPrefill's Alg. 5, kept as the baseline) two more kernels pool the
// keys and the representative queries and compare the pooled estimate with
// p_v.
#include "crisp_common.h"
#include "crisp_kernels.h"

namespace crisp {

namespace {

constexpr int kTileKeys = 128;

// grid: (ceil(Nb / tiles_per_wg), n_kv_heads * ceil(G / 4)); block: 16
// wavefronts sharing one K tile, double-buffered in LDS.  Wave w handles proxy
// rows 32 (w % 4) .. +31 of query head kv*G + 4*sub + w / 4 (idle when that
// head is >= G; it still copies its share of K).
// Each K tile (128 keys x 256 bytes) is copied from HBM straight into LDS
// (two 1 KiB copies per wavefront), one tile ahead: the copies of tile t+1
// are issued when tile t's products start and awaited at the barrier that
// opens iteration t+1, so their latency hides behind a whole tile of work.
// The 16-byte chunk c of key r sits at slot c ^ (r & 15) of the key's row, so
// the fragment reads below are free of bank conflicts without padding.  The
// per-(row, tile) partials of a tile are stored one iteration later, so that
// the wait for the copies never waits on fresh stores.
// Aligned (B divides n): row i sits at column i of the last tile, so the
// split column and the causal cut are compile-time per (chunk, key group).
template <bool Aligned, class QK>
__global__ void __launch_bounds__(1024)
proxy_map_kernel(QK q, QK k, int n, int nb,
                 int G, int tiles_per_wg, float scale_log2,
                 float* __restrict__ part_m, float* __restrict__ part_lo,
                 float* __restrict__ part_up)
{
    __shared__ __attribute__((aligned(1024))) uint16_t ks[2][kTileKeys * kD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int c = __builtin_amdgcn_readfirstlane(w & 3);   // row chunk (uniform)
    const int subs = (G + 3) / 4;
    const int kv = blockIdx.y / subs;
    const int hg = 4 * (blockIdx.y % subs) + (w >> 2);   // head within the KV group
    const bool active = hg < G;
    const int h = kv * G + (active ? hg : 0);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int R = min(kB, n);                       // proxy rows
    const int q0 = n - R;                           // position of proxy row 0

    const uint16_t* kg = k.row(kv, 0);
    const int t0 = blockIdx.x * tiles_per_wg;
    const int t1 = min(nb, t0 + tiles_per_wg);
    // copy j of this wavefront fills LDS bytes 1024 (2w + j) .. +1023 of the
    // tile: keys 4 (2w + j) .. +3, lane l at key 4 (2w + j) + l / 16, slot
    // l % 16, which holds chunk (l % 16) ^ (key & 15).  Keys past the end of
    // the sequence repeat the last key (masked below: they lie after every
    // proxy row).
    const uint32_t lds0 = lds_address(&ks[0][0]) + 2048u * w;
    auto issue = [&](int t, int buf) {
        const long long key0 = (long long)t * kTileKeys;
        const uint16_t* base = kg + key0 * k.st;                 // wave-uniform
        for (int j = 0; j < 2; ++j) {
            const int r = 4 * (2 * w + j) + (lane >> 4);          // key in the tile
            const int rr = (int)min((long long)r, (long long)n - 1 - key0);
            const uint32_t off = (uint32_t)(rr * k.st + 8 * ((lane & 15) ^ (r & 15))) * 2u;
            copy16_to_lds(base, off, lds0 + (uint32_t)buf * (kTileKeys * kD * 2) + 1024u * j);
        }
    };
    if (t0 < t1) issue(t0, 0);

    // rows 32c .. 32c+31 of the representative block Q^ as MFMA B-operands,
    // step s holding d = 16s .. 16s+15 (rows past R, which exist only when
    // n < B, repeat the last row)
    bf16x8 qf[8];
    {
        const uint16_t* qr = q.row(h, q0) + min(32 * c + l32, R - 1) * q.st;
        for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s + 8 * hi);
    }

    const int i = 32 * c + l32;
    const int qi = q0 + i;
    const int kx = l32 & 15;                        // this lane's key swizzle
    // partials of the previous tile, stored one iteration late
    bool pend = false;
    float pms = 0.f, plo = 0.f, pup = 0.f;
    auto store_prev = [&](int tp) {
        const size_t o = ((size_t)h * nb + tp) * kB + i;
        part_m[o] = pms;
        part_lo[o] = plo;
        part_up[o] = pup;
    };
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        wait_copies<0>();
        __syncthreads();                            // tile t landed, buffer buf ^ 1 free
        if (t + 1 < t1) issue(t + 1, buf ^ 1);
        if (pend) {
            store_prev(t - 1);
            pend = false;
        }
        if (!active) continue;

        // S^T of this wave's rows against key group (a + c) % 4 of the tile
        // (keys 32 g .. 32 g + 31) in acc[a]: acc[0] holds the group of the
        // wave's own rows' columns
        f32x16 acc[4];
        for (int a = 0; a < 4; ++a) acc[a] = f32x16{};
        const uint16_t* kb = &ks[buf][l32 * kD];
        for (int s = 0; s < 8; ++s)
            for (int a = 0; a < 4; ++a) {
                const int g = (a + c) & 3;
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + 32 * g * kD + 8 * ((2 * s + hi) ^ kx));
                acc[a] = mfma32(kf, qf[s], acc[a]);
            }

        // this lane: query row i at position qi, 64 of the tile's 128 keys;
        // element r of acc[a] is column 32 g + off(r), g = (a + c) % 4.
        // Aligned: row i = 32 c + l32 is column i of the last tile, so acc[0]
        // (g = c) needs a per-element test at offset l32, and acc[a], a > 0,
        // lies wholly after column i when a + c < 4 (g > c) and wholly
        // before it otherwise.
        float m;
        if (Aligned) {
            if (t == nb - 1) {                                // causal cut
                for (int r = 0; r < 16; ++r)
                    if (8 * (r >> 2) + 4 * hi + (r & 3) > l32) acc[0][r] = -INFINITY;
                for (int a = 1; a < 4; ++a)
                    if (a + c < 4)
                        for (int r = 0; r < 16; ++r) acc[a][r] = -INFINITY;
            }
            float t4[4];
            for (int a = 0; a < 4; ++a) {
                float x[5];
                for (int j = 0; j < 5; ++j)
                    x[j] = fmaxf(fmaxf(acc[a][3 * j], acc[a][3 * j + 1]), acc[a][3 * j + 2]);
                t4[a] = fmaxf(fmaxf(fmaxf(x[0], x[1]), x[2]), fmaxf(fmaxf(x[3], x[4]), acc[a][15]));
            }
            m = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
        } else {
            const int rel = qi - t * kTileKeys;               // last visible column
            const bool cut = t * kTileKeys + kTileKeys - 1 > q0;
            m = -INFINITY;
            for (int a = 0; a < 4; ++a)
                for (int r = 0; r < 16; ++r) {
                    const int col = 32 * ((a + c) & 3) + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (cut && col > rel) acc[a][r] = -INFINITY;   // causal
                    m = fmaxf(m, acc[a][r]);
                }
        }
        m = fmaxf(m, swap_half(m));
        // scaled logits in the exp2 domain; a tile wholly in the row's future
        // keeps m = -inf and sums 0
        const float ms = m * scale_log2;
        const float nref = (m == -INFINITY) ? 0.f : -ms;
        float lo = 0.f, up = 0.f;
        if (Aligned) {
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(fmaf(acc[0][r], scale_log2, nref));
                if (8 * (r >> 2) + 4 * hi + (r & 3) <= l32) lo += e;
                else up += e;
            }
            for (int a = 1; a < 4; ++a) {
                // exponentials in place (the accumulator is dead after this)
                for (int r = 0; r < 16; ++r)
                    acc[a][r] = __builtin_amdgcn_exp2f(fmaf(acc[a][r], scale_log2, nref));
                float s4[4];
                for (int j = 0; j < 4; ++j)
                    s4[j] = (acc[a][j] + acc[a][4 + j]) + (acc[a][8 + j] + acc[a][12 + j]);
                const float sa = (s4[0] + s4[1]) + (s4[2] + s4[3]);
                if (a + c < 4) up += sa;
                else lo += sa;
            }
        } else {
            const int bi = qi & (kB - 1);
            for (int a = 0; a < 4; ++a)
                for (int r = 0; r < 16; ++r) {
                    const int col = 32 * ((a + c) & 3) + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const float e = __builtin_amdgcn_exp2f(fmaf(acc[a][r], scale_log2, nref));
                    if (col <= bi) lo += e; else up += e;
                }
        }
        lo += swap_half(lo);
        up += swap_half(up);
        if (hi == 0 && i < R) {
            pend = true;
            pms = ms;
            plo = lo;
            pup = up;
        }
    }
    if (pend) store_prev(t1 - 1);
}

// The block-mass reduction runs in four small kernels so that it spreads over
// the whole chip:
//   row_part_kernel   per (head, segment of tiles, row): online max m and
//                     normaliser l = sum_t e^(m_t - m) (lo_t + up_t)
//   row_norm_kernel   per (head, row): combine the segments into the row's
//                     max m_i and 1 / l_i
//   tile_mass_kernel  per (head, tile): weights w_{i,t} = e^(m_{i,t} - m_i) / l_i,
//                     p_v[t] and the lower / upper slash sums of the tile,
//                     split by e_i
//   finalize_kernel   per head: p_s from the tile sums; C_struct and the
//                     routing bit (Eq. 2, Alg. 2) under the C_struct router
constexpr int kSegs = kRouteSegs;

// grid (kSegs, hq), kB threads: thread i = proxy row i, tiles t = seg (mod kSegs)
__global__ void __launch_bounds__(kB)
row_part_kernel(const float* __restrict__ part_m, const float* __restrict__ part_lo,
                const float* __restrict__ part_up, int n, int nb, float* __restrict__ seg_m,
                double* __restrict__ seg_l)
{
    const int seg = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
    const int R = min(kB, n);
    const size_t base = (size_t)h * nb * kB;
    float m = -INFINITY;
    double l = 0.0;
    if (i < R) {
        for (int t = seg; t < nb; t += kSegs) {
            const size_t o = base + (size_t)t * kB + i;
            const float mt = part_m[o];
            if (mt == -INFINITY) continue;
            const double sum = (double)part_lo[o] + (double)part_up[o];
            if (mt > m) {
                l = l * (double)exp2f(m - mt) + sum;
                m = mt;
            } else {
                l += sum * (double)exp2f(mt - m);
            }
        }
    }
    const size_t o = ((size_t)h * kSegs + seg) * kB + i;
    seg_m[o] = m;
    seg_l[o] = l;
}

// grid hq, 1024 threads: eight threads per row, each over every eighth segment
__global__ void __launch_bounds__(1024)
row_norm_kernel(const float* __restrict__ seg_m, const double* __restrict__ seg_l, int n,
                float* __restrict__ row_mx, float* __restrict__ row_inv)
{
    __shared__ float pm[8][kB];
    __shared__ double pl[8][kB];
    const int h = blockIdx.x, i = threadIdx.x & (kB - 1), part = threadIdx.x >> 7;
    const size_t b = (size_t)h * kSegs * kB + i;
    float m = -INFINITY;
    for (int x = part; x < kSegs; x += 8) m = fmaxf(m, seg_m[b + (size_t)x * kB]);
    double l = 0.0;
    for (int x = part; x < kSegs; x += 8) {
        const float mx = seg_m[b + (size_t)x * kB];
        if (mx > -INFINITY) l += seg_l[b + (size_t)x * kB] * (double)exp2f(mx - m);
    }
    pm[part][i] = m;
    pl[part][i] = l;
    __syncthreads();
    if (part != 0 || i >= min(kB, n)) return;
    float mt = -INFINITY;
    for (int x = 0; x < 8; ++x) mt = fmaxf(mt, pm[x][i]);
    double lt = 0.0;
    for (int x = 0; x < 8; ++x)
        if (pm[x][i] > -INFINITY) lt += pl[x][i] * (double)exp2f(pm[x][i] - mt);
    row_mx[(size_t)h * kB + i] = mt;
    row_inv[(size_t)h * kB + i] = (float)(1.0 / lt);
}

// grid (ceil(Nb / 16), hq), 1024 threads: one wavefront per tile, lanes over
// the R rows.  tile_sums[h][4][Nb] = lower / upper sums for rows with e_i = 0,
// then for rows with e_i = 1, each divided by R.
__global__ void __launch_bounds__(1024)
tile_mass_kernel(const float* __restrict__ part_m, const float* __restrict__ part_lo,
                 const float* __restrict__ part_up, const float* __restrict__ row_mx,
                 const float* __restrict__ row_inv, int n, int nb, float* __restrict__ p_v,
                 float* __restrict__ tile_sums)
{
    __shared__ float mx[kB], inv[kB];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int R = min(kB, n), q0 = n - R;
    if (tid < R) {
        mx[tid] = row_mx[(size_t)h * kB + tid];
        inv[tid] = row_inv[(size_t)h * kB + tid];
    }
    __syncthreads();
    const int lane = tid & 63;
    const int t = blockIdx.x * 16 + (tid >> 6);
    if (t >= nb) return;
    float sv = 0.f, slo0 = 0.f, sup0 = 0.f, slo1 = 0.f, sup1 = 0.f;
    for (int i = lane; i < R; i += 64) {
        const size_t o = ((size_t)h * nb + t) * kB + i;
        const float mt = part_m[o];
        if (mt == -INFINITY) continue;
        const float wt = exp2f(mt - mx[i]) * inv[i];
        const float lo = part_lo[o] * wt, up = part_up[o] * wt;
        sv += lo + up;
        const int ei = nb - 1 - (q0 + i) / kB;
        if (ei == 0) { slo0 += lo; sup0 += up; }
        else { slo1 += lo; sup1 += up; }
    }
    // 128-term sums: float, reduced without the LDS crossbar
    float r5[5] = {sv, slo0, sup0, slo1, sup1};
    wave_sum_fast_n(r5);
    if (lane == 0) {
        p_v[(size_t)h * nb + t] = (float)(r5[0] / R);
        float* ts = tile_sums + (size_t)h * 4 * nb;
        ts[t] = (float)(r5[1] / R);
        ts[nb + t] = (float)(r5[2] / R);
        ts[2 * nb + t] = (float)(r5[3] / R);
        ts[3 * nb + t] = (float)(r5[4] / R);
    }
}

// grid (ceil(Nb / 256), hq), 256 threads.  Slash block t collects the lower
// parts of tile t (rows with e = 0) and t-1 (e = 1) and the upper parts of
// tile t-1 (e = 0) and t-2 (e = 1).
__global__ void __launch_bounds__(256)
finalize_kernel(const float* __restrict__ tile_sums, const float* __restrict__ p_v, int nb,
                float tau, int route_here, float* __restrict__ p_s, float* __restrict__ c_struct,
                uint8_t* __restrict__ pattern)
{
    const int h = blockIdx.y;
    const int t = blockIdx.x * 256 + threadIdx.x;
    const float* ts = tile_sums + (size_t)h * 4 * nb;
    if (t < nb) {
        float ps = ts[t];
        if (t >= 1) ps += ts[nb + t - 1] + ts[2 * nb + t - 1];
        if (t >= 2) ps += ts[3 * nb + t - 2];
        p_s[(size_t)h * nb + t] = ps;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && route_here) {
        // Eq. 2 with w_sink = w_local = B: the first and the last key block
        const float* pv = p_v + (size_t)h * nb;
        const float cs = (nb > 1) ? pv[0] + pv[nb - 1] : pv[0];
        c_struct[h] = cs;
        pattern[h] = (cs >= tau) ? 1 : 0;
    }
}

// grid hq, 1024 threads, N_b <= kRouteSmall: the four kernels above for one
// head in one work-group (beyond that, one work-group per head is slower
// than the four launches).  Every sum runs in the same order as there (thread
// (row i, part p) walks segments p, p+8, .. and, within each, tiles
// seg, seg+64, ..; wave w takes tiles w, w+16, ..), so p_v, p_s, C_struct
// and the routing bit are the same bits.

__global__ void __launch_bounds__(1024)
route_small_kernel(const float* __restrict__ part_m, const float* __restrict__ part_lo,
                   const float* __restrict__ part_up, int n, int nb, float tau, int route_here,
                   float* __restrict__ p_v, float* __restrict__ p_s, float* __restrict__ c_struct,
                   uint8_t* __restrict__ pattern)
{
    __shared__ float pm[8][kB];
    __shared__ double pl[8][kB];
    __shared__ float mx[kB], inv[kB];
    __shared__ float ts[4 * kRouteSmall];
    __shared__ float pv_l[kRouteSmall];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int R = min(kB, n), q0 = n - R;
    {
        // row statistics: row_part_kernel per segment, row_norm_kernel per part
        const int i = tid & (kB - 1), part = tid >> 7;
        const size_t base = (size_t)h * nb * kB;
        // segment j = part + 8 jj visits tiles seg, seg + 64, .. in order;
        // round rr loads tile seg + 64 rr of all eight segments at once
        float sm[kSegs / 8];
        double sl[kSegs / 8];
        for (int j = 0; j < kSegs / 8; ++j) {
            sm[j] = -INFINITY;
            sl[j] = 0.0;
        }
        if (i < R) {
            for (int t0 = 0; t0 < nb; t0 += kSegs) {
                float mt[kSegs / 8], lo[kSegs / 8], up[kSegs / 8];
                for (int j = 0; j < kSegs / 8; ++j) {
                    const int t = t0 + part + 8 * j;
                    mt[j] = -INFINITY;
                    if (t < nb) {
                        const size_t o = base + (size_t)t * kB + i;
                        mt[j] = part_m[o];
                        lo[j] = part_lo[o];
                        up[j] = part_up[o];
                    }
                }
                for (int j = 0; j < kSegs / 8; ++j) {
                    if (mt[j] == -INFINITY) continue;
                    const double sum = (double)lo[j] + (double)up[j];
                    if (mt[j] > sm[j]) {
                        sl[j] = sl[j] * (double)exp2f(sm[j] - mt[j]) + sum;
                        sm[j] = mt[j];
                    } else {
                        sl[j] += sum * (double)exp2f(mt[j] - sm[j]);
                    }
                }
            }
        }
        float m = -INFINITY;
        for (int j = 0; j < kSegs / 8; ++j) m = fmaxf(m, sm[j]);
        double l = 0.0;
        for (int j = 0; j < kSegs / 8; ++j)
            if (sm[j] > -INFINITY) l += sl[j] * (double)exp2f(sm[j] - m);
        pm[part][i] = m;
        pl[part][i] = l;
        __syncthreads();
        if (part == 0 && i < R) {
            float mt = -INFINITY;
            for (int x = 0; x < 8; ++x) mt = fmaxf(mt, pm[x][i]);
            double lt = 0.0;
            for (int x = 0; x < 8; ++x)
                if (pm[x][i] > -INFINITY) lt += pl[x][i] * (double)exp2f(pm[x][i] - mt);
            mx[i] = mt;
            inv[i] = (float)(1.0 / lt);
        }
        __syncthreads();
    }
    // tile masses: tile_mass_kernel, one wavefront per tile; a wavefront
    // loads four of its tiles (t, t + 16, ..) at a time
    const int lane = tid & 63;
    for (int t4 = tid >> 6; t4 < nb; t4 += 64) {
        float vm[4][2], vlo[4][2], vup[4][2];
        for (int b = 0; b < 4; ++b)
            for (int x = 0; x < 2; ++x) {
                const int t = t4 + 16 * b, i = lane + 64 * x;
                vm[b][x] = -INFINITY;
                if (t < nb && i < R) {
                    const size_t o = ((size_t)h * nb + t) * kB + i;
                    vm[b][x] = part_m[o];
                    vlo[b][x] = part_lo[o];
                    vup[b][x] = part_up[o];
                }
            }
        // the five sums of each of the four tiles, reduced together (as
        // tile_mass_kernel: float, the same order)
        float r[20];
        for (int b = 0; b < 4; ++b) {
            float sv = 0.f, slo0 = 0.f, sup0 = 0.f, slo1 = 0.f, sup1 = 0.f;
            for (int x = 0; x < 2; ++x) {
                const int i = lane + 64 * x;
                const float mt = vm[b][x];
                if (i >= R || mt == -INFINITY) continue;
                const float wt = exp2f(mt - mx[i]) * inv[i];
                const float lo = vlo[b][x] * wt, up = vup[b][x] * wt;
                sv += lo + up;
                const int ei = nb - 1 - (q0 + i) / kB;
                if (ei == 0) { slo0 += lo; sup0 += up; }
                else { slo1 += lo; sup1 += up; }
            }
            r[5 * b] = sv;
            r[5 * b + 1] = slo0;
            r[5 * b + 2] = sup0;
            r[5 * b + 3] = slo1;
            r[5 * b + 4] = sup1;
        }
        wave_sum_fast_n(r);
        for (int b = 0; b < 4; ++b) {
            const int t = t4 + 16 * b;
            if (t >= nb) break;
            if (lane == 0) {
                const float v = (float)(r[5 * b] / R);
                p_v[(size_t)h * nb + t] = v;
                pv_l[t] = v;
                ts[t] = (float)(r[5 * b + 1] / R);
                ts[nb + t] = (float)(r[5 * b + 2] / R);
                ts[2 * nb + t] = (float)(r[5 * b + 3] / R);
                ts[3 * nb + t] = (float)(r[5 * b + 4] / R);
            }
        }
    }
    __syncthreads();
    // finalize_kernel
    for (int t = tid; t < nb; t += 1024) {
        float ps = ts[t];
        if (t >= 1) ps += ts[nb + t - 1] + ts[2 * nb + t - 1];
        if (t >= 2) ps += ts[3 * nb + t - 2];
        p_s[(size_t)h * nb + t] = ps;
    }
    if (tid == 0 && route_here) {
        const float cs = (nb > 1) ? pv_l[0] + pv_l[nb - 1] : pv_l[0];
        c_struct[h] = cs;
        pattern[h] = (cs >= tau) ? 1 : 0;
    }
}

// FlexPrefill's router (Alg. 5), the baseline CRISP replaces.
// grid (Nb, hkv + hq), 256 threads: y < hkv: mean of key block x of KV head
// y over the tokens it holds; y >= hkv (x == 0 only): mean of the R
// representative query rows of head y - hkv.
template <class QK>
__global__ void __launch_bounds__(256)
jsd_pool_kernel(QK q, QK k, int n, int nb,
                int hkv, float* __restrict__ kbar, float* __restrict__ qbar)
{
    __shared__ float red[16][kD];
    const int x = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
    const uint16_t* src;
    long long st;
    float* dst;
    int len;
    if (y < hkv) {
        len = min(kB, n - x * kB);
        src = k.row(y, (long long)x * kB);
        st = k.st;
        dst = kbar + ((size_t)y * nb + x) * kD;
    } else {
        if (x != 0) return;
        len = min(kB, n);
        src = q.row(y - hkv, n - len);
        st = q.st;
        dst = qbar + (size_t)(y - hkv) * kD;
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
        float sum = 0.f;
        for (int r = 0; r < 16; ++r) sum += red[r][tid];
        dst[tid] = sum / (float)len;
    }
}

// One work-group per query head:
//   abar_j = softmax_j(qbar . kbar_j / sqrt(d)) over the N_b blocks,
//   D_JS = sqrt(KL(p_v||m) / 2 + KL(abar||m) / 2), m = (p_v + abar) / 2,
// natural logarithms, sums in double; VS iff D_JS >= tau (in float).
__global__ void __launch_bounds__(256)
jsd_route_kernel(const float* __restrict__ kbar, const float* __restrict__ qbar,
                 const float* __restrict__ p_v, int nb, int G, float tau,
                 float* __restrict__ c_struct, uint8_t* __restrict__ pattern)
{
    __shared__ float qs[kD];
    __shared__ float z[kMaxBlocks];
    __shared__ float red_f[4];
    __shared__ double red_d[3][4];
    const int h = blockIdx.x, g = h / G, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    if (tid < kD) qs[tid] = qbar[(size_t)h * kD + tid];
    __syncthreads();
    const float scale = 1.0f / sqrtf((float)kD);
    float mx = -INFINITY;
    for (int j = tid; j < nb; j += 256) {
        const float* kr = kbar + ((size_t)g * nb + j) * kD;
        float dot = 0.f;
        for (int c = 0; c < kD; ++c) dot = fmaf(qs[c], kr[c], dot);
        z[j] = dot * scale;
        mx = fmaxf(mx, z[j]);
    }
    mx = wave_max(mx);
    if (lane == 0) red_f[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
    double l = 0.0;
    for (int j = tid; j < nb; j += 256) {
        const float e = expf(z[j] - mx);
        z[j] = e;
        l += (double)e;
    }
    l = wave_sum(l);
    if (lane == 0) red_d[0][w] = l;
    __syncthreads();
    l = red_d[0][0] + red_d[0][1] + red_d[0][2] + red_d[0][3];
    const double inv = 1.0 / l;
    double kl_hat = 0.0, kl_bar = 0.0;
    for (int j = tid; j < nb; j += 256) {
        const double a = (double)p_v[(size_t)h * nb + j], b = (double)z[j] * inv;
        const double m = 0.5 * (a + b);
        if (a > 0.0) kl_hat += a * log(a / m);
        if (b > 0.0) kl_bar += b * log(b / m);
    }
    kl_hat = wave_sum(kl_hat);
    kl_bar = wave_sum(kl_bar);
    if (lane == 0) {
        red_d[1][w] = kl_hat;
        red_d[2][w] = kl_bar;
    }
    __syncthreads();
    if (tid == 0) {
        const double js = 0.5 * (red_d[1][0] + red_d[1][1] + red_d[1][2] + red_d[1][3]) +
                          0.5 * (red_d[2][0] + red_d[2][1] + red_d[2][2] + red_d[2][3]);
        const float d = (float)sqrt(js > 0.0 ? js : 0.0);
        c_struct[h] = d;
        pattern[h] = (d >= tau) ? 1 : 0;
    }
}

}  // namespace

template <class QK>
hipError_t launch_route(QK q, QK k, int n, int hq, int hkv,
                        const RouteArgs& a, float* p_v, float* p_s, float* c_struct,
                        uint8_t* pattern, hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB;
    const int G = hq / hkv;
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    // about one work-group per CU, each walking its tiles with the next
    // tile's copy in flight (at 131072 tokens 32 tiles per work-group,
    // 0.210 against 0.225 ms with a quarter of that; at 8192 tokens two
    // tiles, 0.030 against 0.034 ms)
    int tiles_per_wg = 1;
    while (tiles_per_wg < 64 && (size_t)((nb + 2 * tiles_per_wg - 1) / (2 * tiles_per_wg)) * hkv * ((G + 3) / 4) >= 256)
        tiles_per_wg *= 2;
    dim3 grid((nb + tiles_per_wg - 1) / tiles_per_wg, hkv * ((G + 3) / 4));
    if (n % kB == 0)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(proxy_map_kernel<true, QK>), grid, dim3(1024), 0, stream, q, k, n, nb, G,
                           tiles_per_wg, scale_log2, a.part_m, a.part_lo, a.part_up);
    else
        hipLaunchKernelGGL(HIP_KERNEL_NAME(proxy_map_kernel<false, QK>), grid, dim3(1024), 0, stream, q, k, n, nb, G,
                           tiles_per_wg, scale_log2, a.part_m, a.part_lo, a.part_up);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int route_here = a.router == 0;
    if (nb <= kRouteSmall) {
        hipLaunchKernelGGL(route_small_kernel, dim3(hq), dim3(1024), 0, stream, a.part_m, a.part_lo,
                           a.part_up, n, nb, a.tau, route_here, p_v, p_s, c_struct, pattern);
    } else {
        hipLaunchKernelGGL(row_part_kernel, dim3(kSegs, hq), dim3(kB), 0, stream, a.part_m,
                           a.part_lo, a.part_up, n, nb, a.seg_m, a.seg_l);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(row_norm_kernel, dim3(hq), dim3(1024), 0, stream, a.seg_m, a.seg_l, n,
                           a.row_mx, a.row_inv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(tile_mass_kernel, dim3((nb + 15) / 16, hq), dim3(1024), 0, stream,
                           a.part_m, a.part_lo, a.part_up, a.row_mx, a.row_inv, n, nb, p_v,
                           a.tile_sums);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(finalize_kernel, dim3((nb + 255) / 256, hq), dim3(256), 0, stream,
                           a.tile_sums, p_v, nb, a.tau, route_here, p_s, c_struct, pattern);
    }
    if ((e = hipGetLastError()) != hipSuccess || route_here) return e;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(jsd_pool_kernel<QK>), dim3(nb, hkv + hq), dim3(256), 0, stream, q, k, n, nb, hkv,
                       a.jsd_kbar, a.jsd_qbar);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(jsd_route_kernel, dim3(hq), dim3(256), 0, stream, a.jsd_kbar, a.jsd_qbar, p_v,
                       nb, G, a.tau, c_struct, pattern);
    return hipGetLastError();
}

template hipError_t launch_route<Rows>(Rows, Rows, int, int, int, const RouteArgs&, float*, float*,
                                       float*, uint8_t*, hipStream_t);
template hipError_t launch_route<SeqRows>(SeqRows, SeqRows, int, int, int, const RouteArgs&, float*,
                                          float*, float*, uint8_t*, hipStream_t);

}  // namespace crisp
