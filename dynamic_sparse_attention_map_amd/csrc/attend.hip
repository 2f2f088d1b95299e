// Block-sparse causal GQA attention (Eq. 1) on bf16 matrix cores.
//
// One work-group of 8 wavefronts computes two adjacent query blocks of one
// query head (256 queries, 32 per wavefront).  It walks the merged union of
// the two blocks' key-block lists, so every K/V tile is fetched once for both
// blocks; the listed blocks are streamed as 64-key sub-tiles through
// double-buffered LDS (K row-major; V transposed, keys permuted so that each
// operand fragment is one 16-byte read), and each wavefront whose block
// lists the tile runs
//     S^T = K Q^T          (32x32x16 bf16 MFMA, fp32 accumulate)
//     online softmax       (exp2 domain, fp32 running max / sum)
//     O^T += V^T P^T       (P rounded to bf16, fp32 accumulate)
// Computing S^T rather than S leaves each lane holding one query's scores
// in exactly the register order the P^T operand of the second product
// needs, so P never leaves registers.  The causal mask is applied only on
// the diagonal key block; sub-tiles that lie entirely in a wavefront's
// future are skipped.  Fragment reads are issued several products ahead
// of the matrix cores (scheduling-group hints), and the exponentials of
// key group u+1 are interleaved with the PV products of group u.
#include "crisp_common.h"
#include "crisp_kernels.h"

namespace crisp {

namespace {

constexpr int kKT = 64;                   // keys per sub-tile
constexpr int kKPitch = kD + 8;           // K tile row pitch (bf16), 272 bytes
constexpr int kVPitch = kKT + 8;          // V^T tile row pitch (bf16), 144 bytes
constexpr int kKStage = kKT * kKPitch;    // bf16 elements
constexpr int kVStage = kD * kVPitch;
constexpr int kStage = kKStage + kVStage;

constexpr int kThreads = 512;             // 8 wavefronts: two query blocks x 4
constexpr int kEnd = 0x7fffffff;           // list exhausted

// Register cache of one row's key-block list: lane x of cur holds entry
// 64*chunk + x and nxt the next 64 (loaded a whole chunk ahead), so entries
// are read with wave-uniform readlanes and no tile load waits on the list.
struct ListCursor {
    int lbase, len, pos, chunk, cur, nxt;
    bool dense;                            // implicit list 0 .. len-1
};

__device__ __forceinline__ void cursor_init(ListCursor& c, const int32_t* __restrict__ col_idx,
                                            int lbase, int len, bool dense, int lane)
{
    c.lbase = lbase;
    c.len = len;
    c.pos = 0;
    c.chunk = 0;
    c.dense = dense;
    c.cur = c.nxt = -1;
    if (!dense) {
        c.cur = (lane < len) ? col_idx[lbase + lane] : -1;
        c.nxt = (64 + lane < len) ? col_idx[lbase + 64 + lane] : -1;
    }
}

__device__ __forceinline__ int cursor_peek(const ListCursor& c)
{
    if (c.pos >= c.len) return kEnd;
    if (c.dense) return c.pos;
    const int src = ((c.pos >> 6) == c.chunk) ? c.cur : c.nxt;
    return __builtin_amdgcn_readlane(src, c.pos & 63);
}

__device__ __forceinline__ void cursor_advance(ListCursor& c, const int32_t* __restrict__ col_idx,
                                               int lane)
{
    ++c.pos;
    if (!c.dense && (c.pos >> 6) != c.chunk) {
        c.chunk = c.pos >> 6;
        c.cur = c.nxt;
        // lanes past the end keep stale values, which are never read
        const int e = 64 * (c.chunk + 1) + lane;
        if (e < c.len) c.nxt = col_idx[c.lbase + e];
    }
}

// One step of the merged walk over the two rows' lists: the smallest next
// key block and which of the two rows lists it.
struct Entry {
    int kb;            // kEnd when both lists are exhausted
    bool hi, lo;
};

__device__ __forceinline__ Entry next_entry(ListCursor& chi, ListCursor& clo,
                                            const int32_t* __restrict__ col_idx, int lane)
{
    const int a = cursor_peek(chi), b = cursor_peek(clo);
    Entry e;
    e.kb = min(a, b);
    e.hi = (a == e.kb) && a != kEnd;
    e.lo = (b == e.kb) && b != kEnd;
    if (e.hi) cursor_advance(chi, col_idx, lane);
    if (e.lo) cursor_advance(clo, col_idx, lane);
    return e;
}

// Work items: like a grid of ceil(npairs*hkv / 8) * 8 * G items whose item b
// belongs to XCD b % 8: its j = b / 8-th slot there takes chunk
// (j / G) * 8 + b % 8 and head j % G of that chunk, where chunk c covers the G
// query heads of KV head c % hkv at query-block pair c / hkv, the pair p
// being blocks Nb-1-2p and Nb-2-2p.  Each XCD keeps whole GQA groups (sharing
// K/V in its L2) and walks the pairs from the longest causal rows down.
__device__ __forceinline__ void
attend_pair(int b, uint16_t* lds, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr,
            const int32_t* __restrict__ col_idx, int n, int nb, int hkv, int G,
            float scale_log2, uint16_t* __restrict__ out)
{
    const int npairs = (nb + 1) >> 1;
    const int slot = b >> 3;
    const int chunk = (slot / G) * 8 + (b & 7);
    if (chunk >= npairs * hkv) return;
    const int pair = chunk / hkv;
    const int g = chunk % hkv;
    const int h = g * G + slot % G;
    const int qb_hi = nb - 1 - 2 * pair;
    const int qb_lo = qb_hi - 1;                   // -1: no second block

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int half = w >> 2, wq = w & 3;           // half 0: qb_hi, half 1: qb_lo
    const int l32 = lane & 31, hi = lane >> 5;
    const int myqb = half ? qb_lo : qb_hi;
    const bool active = myqb >= 0;

    ListCursor chi, clo;
    if (row_ptr) {
        const int b_hi = row_ptr[h * (nb + 1) + qb_hi];
        cursor_init(chi, col_idx, b_hi, row_ptr[h * (nb + 1) + qb_hi + 1] - b_hi, false, lane);
        if (qb_lo >= 0) {
            const int b_lo = row_ptr[h * (nb + 1) + qb_lo];
            cursor_init(clo, col_idx, b_lo, row_ptr[h * (nb + 1) + qb_lo + 1] - b_lo, false, lane);
        } else {
            cursor_init(clo, col_idx, 0, 0, true, lane);
        }
    } else {
        cursor_init(chi, col_idx, 0, qb_hi + 1, true, lane);
        cursor_init(clo, col_idx, 0, qb_lo + 1, true, lane);
    }

    const int qc = 32 * wq + l32;                         // query within its block
    // a partial last block has rows past the end: they load the last row
    // (their results are never stored)
    const int qpos = (active ? myqb : 0) * kB + qc;
    const bool q_valid = active && qpos < n;
    const size_t qrow = (size_t)h * n + min(qpos, n - 1);
    bf16x8 qf[8];
    for (int s = 0; s < 8; ++s)
        qf[s] = *reinterpret_cast<const bf16x8*>(q + qrow * kD + 16 * s + 8 * hi);

    f32x16 o[4];
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float rescale_gap = 8.0f / scale_log2;   // 2^8 in probability

    const uint16_t* kg = k + (size_t)g * n * kD;
    const size_t n_pad = (size_t)nb * kB;                 // V^T row length
    const uint16_t* vg = vt + (size_t)g * kD * n_pad;

    // staging: 2 x 16 bytes of K and 2 x 16 bytes of V^T per thread
    u32x4 pk[2], pv[2];
    auto load_tile = [&](int kb, int sub) {
        const size_t key0 = (size_t)kb * kB + sub * kKT;
        for (int i = 0; i < 2; ++i) {
            const int e = tid + kThreads * i;
            const int row = e >> 4, ch = e & 15;              // 64 keys x 16 chunks
            // keys past the end of a partial last block read as zero (every
            // query that exists masks them: they lie in its future)
            pk[i] = u32x4{0u, 0u, 0u, 0u};
            if (key0 + row < (size_t)n)
                pk[i] = *reinterpret_cast<const u32x4*>(kg + (key0 + row) * kD + 8 * ch);
            const int dr = e >> 3, vc = e & 7;                // 128 d-rows x 8 chunks
            pv[i] = *reinterpret_cast<const u32x4*>(vg + (size_t)dr * n_pad + key0 + 8 * vc);
        }
    };
    auto store_tile = [&](int stage) {
        uint16_t* ks = lds + stage * kStage;
        uint16_t* vs = ks + kKStage;
        for (int i = 0; i < 2; ++i) {
            const int e = tid + kThreads * i;
            *reinterpret_cast<u32x4*>(ks + (e >> 4) * kKPitch + 8 * (e & 15)) = pk[i];
            *reinterpret_cast<u32x4*>(vs + (e >> 3) * kVPitch + 8 * (e & 7)) = pv[i];
        }
    };

    // ---- tile stream: two 64-key sub-tiles per merged list entry ----
    struct Tile {
        int kb, sub;
        bool act;      // this wavefront computes the tile
        bool diag;     // the tile is in this wavefront's diagonal block
    };
    Entry ent = next_entry(chi, clo, col_idx, lane);
    int ent_sub = 0;
    auto pull = [&](Tile& d) -> bool {
        if (ent.kb == kEnd) return false;
        const bool uh = ent.hi && ent.kb >= 0 && ent.kb <= qb_hi;
        const bool ul = ent.lo && ent.kb >= 0 && ent.kb <= qb_lo;
        const bool mine = half ? ul : uh;
        // a block no row can use is never addressed: block 0 is loaded instead
        d.kb = (uh || ul) ? ent.kb : 0;
        d.sub = ent_sub;
        d.diag = mine && ent.kb == myqb;
        // keys 64..127 of the diagonal block lie after every query < 64
        d.act = mine && !(d.diag && ent_sub == 1 && wq < 2);
        if (ent_sub == 0) {
            ent_sub = 1;
        } else {
            ent_sub = 0;
            ent = next_entry(chi, clo, col_idx, lane);
        }
        return true;
    };

    // Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
    constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

    f32x16 s[2];
    // S^T = K Q^T for the tile in `stage`.  The 16 K fragments are read in
    // the order the matrix cores consume them, six reads ahead.
    auto qk = [&](int stage) {
        const uint16_t* kbase = lds + stage * kStage + l32 * kKPitch + 8 * hi;
        bf16x8 kf[16];
        for (int i = 0; i < 16; ++i) {      // i = 2 st + a
            const int st = i >> 1, a = i & 1;
            kf[i] = *reinterpret_cast<const bf16x8*>(kbase + 32 * a * kKPitch + 16 * st);
        }
        s[0] = f32x16{};
        s[1] = f32x16{};
        for (int i = 0; i < 16; ++i) s[i & 1] = mfma32(kf[i], qf[i >> 1], s[i & 1]);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
        for (int i = 0; i < 10; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 6, 0);
    };
    // causal mask on the diagonal block (wave-uniform branch around it)
    auto mask = [&](int sub) {
        for (int a = 0; a < 2; ++a)
            for (int r = 0; r < 16; ++r) {
                const int kc = kKT * sub + 32 * a + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (kc > qc) s[a][r] = -INFINITY;
            }
    };
    // Running max in raw-score units (tree reduction); the accumulator is
    // rescaled only when the max grows by more than 2^8 in probability
    // (exact: the final normalisation uses the same reference max).
    auto update_max = [&]() {
        float t[11];
        for (int i = 0; i < 5; ++i) t[i] = fmaxf(fmaxf(s[0][3 * i], s[0][3 * i + 1]), s[0][3 * i + 2]);
        for (int i = 0; i < 5; ++i) t[5 + i] = fmaxf(fmaxf(s[1][3 * i], s[1][3 * i + 1]), s[1][3 * i + 2]);
        t[10] = fmaxf(s[0][15], s[1][15]);
        const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
        const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(t[9], t[10]);
        float tmax = fmaxf(fmaxf(u0, u1), fmaxf(u2, u3));
        tmax = fmaxf(tmax, swap_half(tmax));
        const bool grow = tmax > m_run + rescale_gap;
        if (__ballot(grow)) {
            asm volatile("; rescale");
            const float m_new = grow ? tmax : m_run;
            const float alpha = (m_run == -INFINITY) ? 0.f
                              : __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
            m_run = m_new;
            l_run *= alpha;
            for (int dt = 0; dt < 4; ++dt)
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
    };
    // p = 2^(c s - c m) (one FMA and one v_exp), rounded to bf16 into the
    // P^T operand, then O^T += V^T P^T.  Probabilities of key group u + 1
    // are computed while the matrix cores run group u; a lane whose keys
    // are all masked so far keeps m = -inf and uses 0 as its reference.
    auto exp_pv = [&](int stage) {
        const uint16_t* vbase = lds + stage * kStage + kKStage + l32 * kVPitch + 8 * hi;
        const float neg_mc = (m_run == -INFINITY) ? 0.f : -m_run * scale_log2;
        bf16x8 vf[16];                       // vf[4 u + dt]
        for (int u = 0; u < 4; ++u)
            for (int dt = 0; dt < 4; ++dt) {
                vf[4 * u + dt] = *reinterpret_cast<const bf16x8*>(vbase + 32 * dt * kVPitch + 16 * u);
            }
        bf16x8 pf[4];
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int u = 0; u < 4; ++u) {        // key group u: s[u >> 1][8 (u & 1) .. +7]
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + j], scale_log2, neg_mc));
                acc[j & 3] += p;
                pf[u][j] = (__bf16)p;
            }
        }
        for (int u = 0; u < 4; ++u)
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vf[4 * u + dt], pf[u], o[dt]);
        l_run += (acc[0] + acc[1]) + (acc[2] + acc[3]);
        // schedule: V reads for groups 0, 1 and the probabilities of group
        // 0 first; then each group's 4 products interleaved with the next
        // group's probabilities and V reads
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 30, 0);
        for (int u = 0; u < 3; ++u)
            for (int dt = 0; dt < 4; ++dt) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 7, 0);
                if (u < 2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
    };

    // Sequential schedule: tile t+1 is fetched into registers while tile t
    // is computed, then stored into the other LDS stage.
    Tile cur{0, 0, false, false}, nxt{0, 0, false, false};
    if (pull(cur)) {
        load_tile(cur.kb, cur.sub);
        store_tile(0);
        int stage = 0;
        for (;;) {
            const bool has_next = pull(nxt);
            if (has_next) load_tile(nxt.kb, nxt.sub);
            __syncthreads();
            if (cur.act) {
                qk(stage);
                if (cur.diag) mask(cur.sub);
                update_max();
                exp_pv(stage);
            }
            if (!has_next) break;
            store_tile(stage ^ 1);
            stage ^= 1;
            cur = nxt;
        }
    }

    if (!active) return;
    const float l = l_run + swap_half(l_run);
    if (!q_valid) return;             // after the wave-wide exchange above
    const float inv = (l > 0.f) ? 1.0f / l : 0.f;
    uint16_t* orow = out + qrow * kD;
    for (int dt = 0; dt < 4; ++dt)
        for (int j = 0; j < 4; ++j) {
            bf16x4 v4;
            for (int r = 0; r < 4; ++r) v4[r] = (__bf16)(o[dt][4 * j + r] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * j + 4 * hi) = v4;
        }
}

// Persistent work-groups (one per CU) drain eight per-XCD queues of work
// items; a group starts on the queue of its own XCD (work-group b is placed
// on XCD b % 8) and moves to the others once that one is empty.  ctr[x]
// counts items taken from queue x and must be zero at launch.
__global__ void __launch_bounds__(kThreads)
attend_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr,
              const int32_t* __restrict__ col_idx, int n, int nb, int hkv, int G,
              float scale_log2, int per_xcd, int* __restrict__ ctr, uint16_t* __restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];
    __shared__ int s_item;
    const int home = blockIdx.x & 7;
    int next_q = 0;   // queues home+0 .. home+7 in turn; only thread 0 uses it
    for (;;) {
        if (threadIdx.x == 0) {
            int item = -1;
            while (next_q < 8) {
                const int x = (home + next_q) & 7;
                const int j = atomicAdd(&ctr[x], 1);
                if (j < per_xcd) { item = 8 * j + x; break; }
                ++next_q;
            }
            s_item = item;
        }
        __syncthreads();
        const int item = s_item;
        __syncthreads();
        if (item < 0) break;
        attend_pair(item, lds, q, k, vt, row_ptr, col_idx, n, nb, hkv, G, scale_log2, out);
    }
}

__global__ void zero_counters_kernel(int* __restrict__ ctr)
{
    if (threadIdx.x < 8) ctr[threadIdx.x] = 0;
}

// V^T with keys permuted inside every group of 16 (bits 2 and 3 of the key
// index swapped): vt[g][d][16 j + pi(c)] = v[g][16 j + c][d].  A lane's 8 keys
// of a PV operand fragment, {4h .. 4h+3, 8+4h .. 8+4h+3} for lane half h (the
// order the S^T accumulator holds them in), are then 16 contiguous bytes.
// Rows have n_pad = N_b * B keys; keys past n are zero.
// grid (n_pad/64, hkv), 256 threads.
__global__ void __launch_bounds__(256)
v_transpose_kernel(const uint16_t* __restrict__ v, int n, int n_pad, uint16_t* __restrict__ vt)
{
    __shared__ uint16_t tile[64][kD + 8];
    const int g = blockIdx.y, key0 = blockIdx.x * 64, tid = threadIdx.x;
    const uint16_t* src = v + ((size_t)g * n + key0) * kD;
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 4, ch = e & 15;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (key0 + row < n) val = *reinterpret_cast<const u32x4*>(src + (size_t)row * kD + 8 * ch);
        *reinterpret_cast<u32x4*>(&tile[row][8 * ch]) = val;
    }
    __syncthreads();
    uint16_t* dst = vt + (size_t)g * kD * n_pad + key0;
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        const int d = e >> 3, c8 = e & 7;
        u32x4 val;
        for (int x = 0; x < 4; ++x) {
            const int p0 = 8 * c8 + 2 * x;              // positions p0, p0 + 1
            const int k0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);
            val[x] = (uint32_t)tile[k0][d] | ((uint32_t)tile[k0 + 1][d] << 16);
        }
        *reinterpret_cast<u32x4*>(dst + (size_t)d * n_pad + 8 * c8) = val;
    }
}

}  // namespace

hipError_t launch_v_transpose(const uint16_t* v, int n, int hkv, uint16_t* vt, hipStream_t stream)
{
    const int n_pad = (n + kB - 1) / kB * kB;
    hipLaunchKernelGGL(v_transpose_kernel, dim3(n_pad / 64, hkv), dim3(256), 0, stream, v, n, n_pad,
                       vt);
    return hipGetLastError();
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                         const int32_t* row_ptr, const int32_t* col_idx, int n, int hq, int hkv,
                         int* counters, uint16_t* out, hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv;
    const long long chunks = (long long)((nb + 1) / 2) * hkv;
    const long long items = ((chunks + 7) / 8) * 8 * G;
    const int per_xcd = (int)(items / 8);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int groups = cus;   // one resident work-group of 8 wavefronts per CU
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, stream, counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_kernel, dim3(groups), dim3(kThreads), 0, stream, q, k, vt, row_ptr, col_idx,
                       n, nb, hkv, G, scale_log2, per_xcd, counters, out);
    return hipGetLastError();
}

}  // namespace crisp
