// Routing kernels: proxy map (Alg. 2, lines 3-5) and the block-mass
// reduction that yields the vertical / slash scores (Alg. 3, lines 3-5),
// C_struct (Eq. 2) and the routing bit (Alg. 2, lines 9-13).
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
// upper split it between two slash blocks.  mass_reduce_kernel rescales the
// partials with the global row maxima and normalisers.
#include "crisp_common.h"
#include "crisp_kernels.h"

namespace crisp {

namespace {

constexpr int kTileKeys = 128;
constexpr int kKRow = kD + 8;   // LDS row pitch of a K tile (bf16): 272 bytes

// grid: (ceil(Nb / tiles_per_wg), n_kv_heads * ceil(G / 4)); block: 4
// wavefronts sharing one staged K tile.  Wave w handles query head
// kv*G + 4*sub + w (idle when that is >= G; it still helps stage K).
__global__ void __launch_bounds__(256)
proxy_map_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int n, int nb,
                 int G, int tiles_per_wg, float scale_log2,
                 float* __restrict__ part_m, float* __restrict__ part_lo,
                 float* __restrict__ part_up)
{
    __shared__ __attribute__((aligned(16))) uint16_t ks[kTileKeys * kKRow];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int subs = (G + 3) / 4;
    const int kv = blockIdx.y / subs;
    const int hg = 4 * (blockIdx.y % subs) + w;     // head within the KV group
    const bool active = hg < G;
    const int h = kv * G + (active ? hg : 0);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int R = min(kB, n);                       // proxy rows
    const int q0 = n - R;                           // position of proxy row 0

    // representative query block Q^ of head h as MFMA B-operands:
    // chunk c holds rows 32c .. 32c+31, step s holds d = 16s .. 16s+15
    // (rows past R, which exist only when n < B, repeat the last row)
    bf16x8 qf[4][8];
    {
        const uint16_t* qh = q + ((size_t)h * n + q0) * kD;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int s = 0; s < 8; ++s)
                qf[c][s] = *reinterpret_cast<const bf16x8*>(
                    qh + (size_t)min(32 * c + l32, R - 1) * kD + 16 * s + 8 * hi);
    }

    const uint16_t* kg = k + (size_t)kv * n * kD;
    const int t0 = blockIdx.x * tiles_per_wg;
    const int t1 = min(nb, t0 + tiles_per_wg);
    for (int t = t0; t < t1; ++t) {
        // stage K tile t: 128 rows x 256 bytes as 16-byte chunks; rows past
        // the end of the sequence are zero (and masked below)
        __syncthreads();
        for (int e = threadIdx.x; e < kTileKeys * (kD / 8); e += 256) {
            const int row = e >> 4, ch = e & 15;
            const size_t key = (size_t)t * kTileKeys + row;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (key < (size_t)n) val = *reinterpret_cast<const u32x4*>(kg + key * kD + 8 * ch);
            *reinterpret_cast<u32x4*>(&ks[row * kKRow + 8 * ch]) = val;
        }
        __syncthreads();
        if (!active) continue;

        // the tile holds keys after some proxy row's position
        const bool maybe_future = t * kTileKeys + kTileKeys - 1 > q0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // S^T for keys 32a.. of the tile against query rows 32c..
            f32x16 acc[4];
            for (int a = 0; a < 4; ++a) acc[a] = f32x16{};
            for (int s = 0; s < 8; ++s)
                for (int a = 0; a < 4; ++a) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[(32 * a + l32) * kKRow + 16 * s + 8 * hi]);
                    acc[a] = mfma32(kf, qf[c][s], acc[a]);
                }

            // this lane: query row i at position qi, 64 of the tile's 128 keys
            const int i = 32 * c + l32;
            const int qi = q0 + i;
            const int bi = qi & (kB - 1);
            const int rel = qi - t * kTileKeys;     // last visible column
            float m = -INFINITY;
            for (int a = 0; a < 4; ++a)
                for (int r = 0; r < 16; ++r) {
                    const int col = 32 * a + 8 * (r >> 2) + 4 * hi + (r & 3);
                    float x = acc[a][r] * scale_log2;
                    if (maybe_future && col > rel) x = -INFINITY;   // causal
                    acc[a][r] = x;
                    m = fmaxf(m, x);
                }
            m = fmaxf(m, swap_half(m));
            float lo = 0.f, up = 0.f;
            if (m > -INFINITY) {                    // else: the whole tile is in the row's future
                for (int a = 0; a < 4; ++a)
                    for (int r = 0; r < 16; ++r) {
                        const int col = 32 * a + 8 * (r >> 2) + 4 * hi + (r & 3);
                        const float e = exp2f(acc[a][r] - m);
                        if (col <= bi) lo += e; else up += e;
                    }
            }
            lo += swap_half(lo);
            up += swap_half(up);
            if (hi == 0 && i < R) {
                const size_t o = ((size_t)h * nb + t) * kB + i;
                part_m[o] = m;
                part_lo[o] = lo;
                part_up[o] = up;
            }
        }
    }
}

// One work-group (256 threads) per query head; rows i < R = min(B, n).
//   m_i   = max_t M[t][i],  l_i = sum_t exp2(M[t][i] - m_i) (LO + UP)[t][i]
//   w_ti  = exp2(M[t][i] - m_i) / l_i
//   p_v[t] = (1/R) sum_i w_ti (LO + UP)[t][i]
//   p_s[t] = (1/R) sum_i (w_(t-e_i)i LO[t-e_i][i] + w_(t-e_i-1)i UP[t-e_i-1][i])
// Tiles wholly in a row's future carry M = -inf and are skipped.
__global__ void __launch_bounds__(256)
mass_reduce_kernel(const float* __restrict__ part_m, const float* __restrict__ part_lo,
                   const float* __restrict__ part_up, int n, int nb, float tau,
                   float* __restrict__ p_v, float* __restrict__ p_s,
                   float* __restrict__ c_struct, uint8_t* __restrict__ pattern)
{
    __shared__ float row_m[2][kB];
    __shared__ double row_l[2][kB];
    __shared__ float row_inv[kB];
    __shared__ float row_mx[kB];
    // lower / upper slash sums of each tile, for rows with e_i = 0 and 1
    __shared__ float lo_sum[2][kMaxBlocks];
    __shared__ float up_sum[2][kMaxBlocks];
    __shared__ float pv_ends[2];

    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t base = (size_t)h * nb * kB;
    const int R = min(kB, n), q0 = n - R;

    // phase 1: per-row online max / normaliser, two threads per row
    {
        const int i = tid & (kB - 1), part = tid >> 7;
        float m = -INFINITY;
        double l = 0.0;
        if (i < R) {
            for (int t = part; t < nb; t += 2) {
                const size_t o = base + (size_t)t * kB + i;
                const float mt = part_m[o];
                if (mt == -INFINITY) continue;
                const double s = (double)part_lo[o] + (double)part_up[o];
                if (mt > m) {
                    l = l * (double)exp2f(m - mt) + s;
                    m = mt;
                } else {
                    l += s * (double)exp2f(mt - m);
                }
            }
        }
        row_m[part][i] = m;
        row_l[part][i] = l;
    }
    __syncthreads();
    if (tid < R) {
        const float m0 = row_m[0][tid], m1 = row_m[1][tid];
        const float m = fmaxf(m0, m1);
        double l = 0.0;
        if (m0 > -INFINITY) l += row_l[0][tid] * (double)exp2f(m0 - m);
        if (m1 > -INFINITY) l += row_l[1][tid] * (double)exp2f(m1 - m);
        row_mx[tid] = m;
        row_inv[tid] = (float)(1.0 / l);
    }
    __syncthreads();

    // phase 2: one wavefront per tile, lanes over the R rows
    const int lane = tid & 63, w = tid >> 6;
    for (int t = w; t < nb; t += 4) {
        double sv = 0.0, slo0 = 0.0, sup0 = 0.0, slo1 = 0.0, sup1 = 0.0;
        for (int i = lane; i < R; i += 64) {
            const size_t o = base + (size_t)t * kB + i;
            const float mt = part_m[o];
            if (mt == -INFINITY) continue;
            const float wt = exp2f(mt - row_mx[i]) * row_inv[i];
            const float lo = part_lo[o] * wt, up = part_up[o] * wt;
            sv += (double)lo + (double)up;
            const int ei = nb - 1 - (q0 + i) / kB;
            if (ei == 0) { slo0 += lo; sup0 += up; }
            else { slo1 += lo; sup1 += up; }
        }
        sv = wave_sum(sv);
        slo0 = wave_sum(slo0);
        sup0 = wave_sum(sup0);
        slo1 = wave_sum(slo1);
        sup1 = wave_sum(sup1);
        if (lane == 0) {
            const float pv = (float)(sv / R);
            p_v[(size_t)h * nb + t] = pv;
            if (t == 0) pv_ends[0] = pv;
            if (t == nb - 1) pv_ends[1] = pv;
            lo_sum[0][t] = (float)(slo0 / R);
            up_sum[0][t] = (float)(sup0 / R);
            lo_sum[1][t] = (float)(slo1 / R);
            up_sum[1][t] = (float)(sup1 / R);
        }
    }
    __syncthreads();
    // slash block t: lower parts of tile t (e = 0) and t-1 (e = 1), upper
    // parts of tile t-1 (e = 0) and t-2 (e = 1)
    for (int t = tid; t < nb; t += 256) {
        float ps = lo_sum[0][t];
        if (t >= 1) ps += up_sum[0][t - 1] + lo_sum[1][t - 1];
        if (t >= 2) ps += up_sum[1][t - 2];
        p_s[(size_t)h * nb + t] = ps;
    }
    if (tid == 0) {
        // Eq. 2 with w_sink = w_local = B: the first and the last key block
        const float cs = (nb > 1) ? pv_ends[0] + pv_ends[1] : pv_ends[0];
        c_struct[h] = cs;
        pattern[h] = (cs >= tau) ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_route(const uint16_t* q, const uint16_t* k, int n, int hq, int hkv,
                        float tau, float* part_m, float* part_lo, float* part_up,
                        float* p_v, float* p_s, float* c_struct, uint8_t* pattern,
                        hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB;
    const int G = hq / hkv;
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    // enough work-groups to fill 256 CUs several times over
    int tiles_per_wg = 1;
    while (tiles_per_wg < 8 && (size_t)((nb + 2 * tiles_per_wg - 1) / (2 * tiles_per_wg)) * hkv >= 1024)
        tiles_per_wg *= 2;
    dim3 grid((nb + tiles_per_wg - 1) / tiles_per_wg, hkv * ((G + 3) / 4));
    hipLaunchKernelGGL(proxy_map_kernel, grid, dim3(256), 0, stream, q, k, n, nb, G,
                       tiles_per_wg, scale_log2, part_m, part_lo, part_up);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mass_reduce_kernel, dim3(hq), dim3(256), 0, stream, part_m, part_lo, part_up,
                       n, nb, tau, p_v, p_s, c_struct, pattern);
    return hipGetLastError();
}

}  // namespace crisp
