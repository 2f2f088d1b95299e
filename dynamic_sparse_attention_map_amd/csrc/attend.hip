// Block-sparse causal GQA attention (Eq. 1) on bf16 matrix cores.
//
// One work-group of 8 wavefronts computes two adjacent query blocks of one
// query head (256 queries, 32 per wavefront).  It walks the merged union of
// the two blocks' key-block lists, so every K/V tile is fetched once for both
// blocks; the listed blocks are streamed as 64-key sub-tiles, copied from
// HBM straight into a 4-stage LDS ring (K row-major, V transposed with keys
// permuted so that each operand fragment is one 16-byte read; both with
// XOR-swizzled chunks), and each wavefront whose block lists the tile runs
//     S^T = K Q^T          (32x32x16 bf16 MFMA, fp32 accumulate)
//     online softmax       (exp2 domain, fp32 running max / sum)
//     O^T += V^T P^T       (P rounded to bf16, fp32 accumulate)
// Computing S^T rather than S leaves each lane holding one query's scores
// in exactly the register order the P^T operand of the second product
// needs, so P never leaves registers.  The causal mask is applied only on
// the diagonal key block; sub-tiles that lie entirely in a wavefront's
// future are skipped.  Fragment reads are issued several products ahead
// of the matrix cores (scheduling-group hints), and the two wavefronts on
// each SIMD run the matrix and vector phases of a tile in opposite order,
// the one in its matrix phase with the higher issue priority (schedule
// below).
#include "crisp_common.h"
#include "crisp_kernels.h"

namespace crisp {

namespace {

constexpr int kKT = 64;                   // keys per sub-tile
constexpr int kImg = kKT * kD;            // one K or V^T sub-tile image, bf16 elements (16 KiB)
constexpr int kStageBytes = 4 * kImg;     // K image, then V^T image
constexpr int kStages = 4;                // LDS ring depth

constexpr int kThreads = 512;             // 8 wavefronts: two query blocks x 4

constexpr int kListWords = kMaxBlocks / 32;   // bitmap words per row
// Run length of one head's pairs on an XCD: a whole head when it has at most
// kWholeHeadPairs pairs, else kPairRun; never so long that an XCD is left
// without a chunk of its own (fewer KV heads than XCDs).  Measured at 1024
// and 4096 blocks: whole heads were 0.9% faster at 1024, runs of 256 0.2%
// faster than 512 or 1024 at 4096.
constexpr int kPairRun = 256;
constexpr int kWholeHeadPairs = 512;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_addr + 16 l (lds_addr wave-uniform).  Written as inline asm so
// that the compiler, which cannot tell the ring's stages apart, does not put
// a full vmcnt(0) before every LDS read; completion is awaited explicitly
// (wait_copies) before the barrier that publishes a tile.  M0 is set here
// and declared clobbered; the s_nop covers the M0 -> LDS-DMA hazard.
// (M0 is otherwise unused by this code, so its clobber is harmless.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_copies()
{
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8));
}

// Work items.  Pair p is query blocks Nb-1-2p and Nb-2-2p.  A chunk is `run`
// consecutive pairs of the G query heads of one KV head: chunk c covers KV
// head c % hkv and pairs run * (c / hkv) onward, and holds its G x run items
// head-major (one head's run of pairs, then the next head's).  Item b belongs
// to XCD b % 8; its j = b / 8-th slot there is item j % (G run) of chunk
// (j / (G run)) * 8 + b % 8.  So each XCD keeps whole GQA groups and walks
// the pairs from the longest causal rows down in runs, and the work-groups of
// an XCD start one head's adjacent pairs close together in time: their lists
// are alike, they walk them in step, and all but the first find most K/V
// tiles in L2.  (Interleaving the heads instead, pair by pair, leaves almost
// no reuse: the long rows of diffuse heads start far apart in time.)  XCD x
// starts its chunks' heads at head x % G: vertical-slash heads, with short,
// scattered lists, miss L2 far more often than diffuse heads, and this keeps
// the XCDs from all running them at the same time.  (Runs inside a chunk are
// rotated, never reordered across chunks, so the walk from the longest rows
// down is kept.)
__device__ __forceinline__ void
attend_pair(int b, uint16_t* lds, uint32_t* list, Rows q, Rows k,
            const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr,
            const int32_t* __restrict__ col_idx, int n, int nb, int hkv, int G, int run,
            float scale_log2, OutRows out)
{
    const int npairs = (nb + 1) >> 1;
    const int slot = b >> 3;
    const int per_chunk = G * run;
    const int chunk = (slot / per_chunk) * 8 + (b & 7);
    const int r = slot % per_chunk;
    const int pair = (chunk / hkv) * run + r % run;
    if (pair >= npairs) return;
    const int g = chunk % hkv;
    const int h = g * G + (r / run + (b & 7)) % G;
    const int qb_hi = nb - 1 - 2 * pair;
    const int qb_lo = qb_hi - 1;                   // -1: no second block

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int half = w >> 2, wq = w & 3;           // half 0: qb_hi, half 1: qb_lo
    const int l32 = lane & 31, hi = lane >> 5;
    const int myqb = half ? qb_lo : qb_hi;
    const bool active = myqb >= 0;

    // ---- the merged key-block list of the two rows, built in LDS ----
    // bits[r][kb / 32] bit kb % 32: row r (0 = qb_hi, 1 = qb_lo) lists key
    // block kb (blocks outside [0, qb] are ignored); then one wavefront
    // compacts the union into desc[] = kb | hi << 16 | lo << 17, ascending.
    uint32_t* bits = list;                       // [2][kListWords]
    uint32_t* desc = list + 2 * kListWords;      // [kMaxBlocks], then the count
    for (int i = tid; i < 2 * kListWords; i += kThreads) bits[i] = 0u;
    __syncthreads();
    if (row_ptr) {
        for (int r = 0; r < 2; ++r) {
            const int qb = r ? qb_lo : qb_hi;
            if (qb < 0) continue;
            const int e0 = row_ptr[h * (nb + 1) + qb], e1 = row_ptr[h * (nb + 1) + qb + 1];
            for (int e = e0 + tid; e < e1; e += kThreads) {
                const int kb = col_idx[e];
                if (kb >= 0 && kb <= qb) atomicOr(&bits[r * kListWords + (kb >> 5)], 1u << (kb & 31));
            }
        }
    } else {
        for (int i = tid; i < 2 * kListWords; i += kThreads) {
            const int r = i / kListWords, wd = i % kListWords;
            const int qb = r ? qb_lo : qb_hi;          // blocks 0 .. qb
            const int lo = 32 * wd;
            bits[i] = (qb < lo) ? 0u : (qb >= lo + 31) ? ~0u : ((2u << (qb - lo)) - 1u);
        }
    }
    __syncthreads();
    if (w == 0) {
        uint32_t wa[2], wb[2];
        int c = 0;
        for (int x = 0; x < 2; ++x) {
            wa[x] = bits[2 * lane + x];
            wb[x] = bits[kListWords + 2 * lane + x];
            c += __popc(wa[x] | wb[x]);
        }
        int incl = c;
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        int pos = incl - c;
        for (int x = 0; x < 2; ++x) {
            uint32_t u = wa[x] | wb[x];
            while (u) {
                const int bit = __ffs(u) - 1;
                u &= u - 1;
                const int kb = 32 * (2 * lane + x) + bit;
                desc[pos++] = (uint32_t)kb | (((wa[x] >> bit) & 1u) << 16) | (((wb[x] >> bit) & 1u) << 17);
            }
        }
        if (lane == 63) desc[kMaxBlocks] = (uint32_t)incl;
    }
    __syncthreads();
    const int n_entries = __builtin_amdgcn_readfirstlane((int)desc[kMaxBlocks]);

    const int qc = 32 * wq + l32;                         // query within its block
    // a partial last block has rows past the end: they load the last row
    // (their results are never stored)
    const int qpos = (active ? myqb : 0) * kB + qc;
    const bool q_valid = active && qpos < n;
    const uint16_t* qrow = q.row(h, min(qpos, n - 1));
    bf16x8 qf[8];
    for (int s = 0; s < 8; ++s)
        qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hi);

    f32x16 o[4];
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float rescale_gap = 8.0f / scale_log2;   // 2^8 in probability

    const uint16_t* kg = k.row(g, 0);
    // V^T sub-tile images of this KV head, 2 per key block
    const uint16_t* vg = vt + (size_t)g * nb * (2 * kImg);

    // Staging.  Every wavefront copies 2 KiB of K and 2 KiB of V^T per tile,
    // 1 KiB per copy instruction.  LDS images carry an XOR swizzle of the
    // 16-byte chunks so that the operand reads below are free of bank
    // conflicts without padding:
    //   K    [64 keys][16 chunks]:  chunk c of key r at slot c ^ (r & 15)
    //   V^T  [128 d][8 chunks]:     chunk c of row d at slot c ^ ((d >> 1) & 7)
    // K is swizzled by the per-lane source address; V^T is stored in HBM as
    // these images already (v_transpose_kernel), so its copy is contiguous.
    int k_row[2], k_col[2];
    long long k_src[2];
    for (int j = 0; j < 2; ++j) {
        const int ci = 2 * w + j;                       // 1 KiB chunk of the image
        k_row[j] = 4 * ci + (lane >> 4);
        k_col[j] = 8 * ((lane & 15) ^ (k_row[j] & 15));
        k_src[j] = k_row[j] * k.st + k_col[j];
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) uint16_t*)lds);
    auto issue_tile = [&](int t, uint32_t dsc) {        // tile t into stage t % 4
        const int kb = (int)(dsc & 0xffffu), sub = t & 1;
        const int key0 = kb * kB + sub * kKT;
        const uint32_t sb = lds_base + (uint32_t)((t & 3) * kStageBytes) + 2048u * w;
        const uint16_t* kt = kg + key0 * k.st;
        const bool full = key0 + kKT <= n;
        for (int j = 0; j < 2; ++j) {
            // keys past the end of a partial last block repeat the last key
            // (every query that exists masks them: they lie in its future)
            const uint16_t* src = full ? kt + k_src[j]
                                       : kg + min(key0 + k_row[j], n - 1) * k.st + k_col[j];
            copy16_to_lds(src, sb + 1024u * j);
        }
        const uint16_t* vimg = vg + (size_t)(2 * kb + sub) * kImg + 1024 * w + 8 * lane;
        for (int j = 0; j < 2; ++j) copy16_to_lds(vimg + 512 * j, sb + 2 * kImg + 1024u * j);
    };

    // ---- tile stream: two 64-key sub-tiles per merged list entry ----
    struct Tile {
        int kb, sub;
        bool act;      // this wavefront computes the tile
        bool diag;     // the tile is in this wavefront's diagonal block
    };
    const int n_tiles = 2 * n_entries;
    auto tile_of = [&](int t, uint32_t dsc) {
        Tile d;
        d.kb = (int)(dsc & 0xffffu);
        d.sub = t & 1;
        const bool mine = half ? ((dsc >> 17) & 1u) : ((dsc >> 16) & 1u);
        d.diag = mine && d.kb == myqb;
        // keys 64..127 of the diagonal block lie after every query < 64
        d.act = mine && !(d.diag && d.sub == 1 && wq < 2);
        return d;
    };
    auto desc_at = [&](int t) -> uint32_t {
        return __builtin_amdgcn_readfirstlane(desc[min(t, n_tiles - 1) >> 1]);
    };

    // Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
    constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

    const int kx = l32 & 15, vx = (l32 >> 1) & 7;   // this lane's swizzles
    f32x16 s[2];
    // S^T = K Q^T for the tile in `stage`.  The 16 K fragments are read in
    // the order the matrix cores consume them, six reads ahead.
    auto qk = [&](int stage) {
        const uint16_t* kbase = lds + stage * (kStageBytes / 2) + l32 * kD;
        bf16x8 kf[16];
        for (int i = 0; i < 16; ++i) {      // i = 2 st + a
            const int st = i >> 1, a = i & 1;
            kf[i] = *reinterpret_cast<const bf16x8*>(kbase + 32 * a * kD + 8 * ((2 * st + hi) ^ kx));
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
    // P^T operand; a lane whose keys are all masked so far keeps m = -inf
    // and uses 0 as its reference
    bf16x8 pf[4];
    auto probs = [&]() {
        const float neg_mc = (m_run == -INFINITY) ? 0.f : -m_run * scale_log2;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int u = 0; u < 4; ++u)            // key group u: s[u >> 1][8 (u & 1) .. +7]
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + j], scale_log2, neg_mc));
                acc[j & 3] += p;
                pf[u][j] = (__bf16)p;
            }
        l_run += (acc[0] + acc[1]) + (acc[2] + acc[3]);
    };
    // O^T += V^T P^T for the tile in `stage`
    auto pv_mfma = [&](int stage) {
        const uint16_t* vbase = lds + stage * (kStageBytes / 2) + kImg + l32 * kKT;
        bf16x8 vf[16];                       // vf[4 u + dt]
        for (int u = 0; u < 4; ++u)
            for (int dt = 0; dt < 4; ++dt)
                vf[4 * u + dt] = *reinterpret_cast<const bf16x8*>(vbase + 32 * dt * kKT + 8 * ((2 * u + hi) ^ vx));
        for (int u = 0; u < 4; ++u)
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vf[4 * u + dt], pf[u], o[dt]);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
        for (int i = 0; i < 10; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 6, 0);
    };

    // Schedule.  Per tile t every wavefront runs a matrix phase M_t = PV(t-1)
    // + QK(t) and a vector phase V_t = softmax(t); one barrier ends each
    // iteration.  Half 0 runs M_t then V_t; half 1 runs V_{t-1} then M_t, so
    // the two wavefronts sharing a SIMD start each iteration on different
    // units and stay out of each other's way without a barrier in between.
    // Tiles rotate through 4 LDS stages: tile t is read in iterations t (K)
    // and t+1 (V^T).  Each wavefront issues its copies of tile t+2 at the
    // start of iteration t, into the stage of tile t-2 (last read in
    // iteration t-1), and waits for those of tile t+1 before the barrier
    // that ends iteration t.
    if (n_tiles > 0) {
        uint32_t d0 = desc_at(0), d1 = desc_at(1), d2 = desc_at(2);
        issue_tile(0, d0);
        if (n_tiles > 1) issue_tile(1, d1);
        wait_copies<0>();
        __syncthreads();
        Tile prev{0, 0, false, false};
        for (int t = 0; t < n_tiles; ++t) {
            const Tile cur = tile_of(t, d0);
            const bool more = t + 2 < n_tiles;
            if (more) issue_tile(t + 2, d2);
            if (half == 1 && t >= 1 && prev.act) {          // V_{t-1}
                if (prev.diag) mask(prev.sub);
                update_max();
                probs();
            }
            // the wavefront in its matrix phase issues first, so the matrix
            // core stays fed and the other wavefront's vector work fills the
            // gaps (raising the vector phase instead was 2% slower)
            __builtin_amdgcn_s_setprio(1);
            if (t >= 1 && prev.act) pv_mfma((t - 1) & 3);   // M_t
            if (cur.act) qk(t & 3);
            __builtin_amdgcn_s_setprio(0);
            if (half == 0 && cur.act) {                     // V_t
                if (cur.diag) mask(cur.sub);
                update_max();
                probs();
            }
            d0 = d1;
            d1 = d2;
            d2 = desc_at(t + 3);
            if (more) wait_copies<4>(); else wait_copies<0>();
            __syncthreads();
            prev = cur;
        }
        if (half == 1 && prev.act) {                        // V of the last tile
            if (prev.diag) mask(prev.sub);
            update_max();
            probs();
        }
        if (prev.act) pv_mfma((n_tiles - 1) & 3);           // PV of the last tile
    }

    if (!active) return;
    const float l = l_run + swap_half(l_run);
    if (!q_valid) return;             // after the wave-wide exchange above
    const float inv = (l > 0.f) ? 1.0f / l : 0.f;
    uint16_t* orow = out.row(h, qpos);
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
attend_kernel(Rows q, Rows k,
              const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr,
              const int32_t* __restrict__ col_idx, int n, int nb, int hkv, int G, int run,
              float scale_log2, int per_xcd, int* __restrict__ ctr, OutRows out)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages * kStageBytes / 2];
    __shared__ uint32_t list[2 * kListWords + kMaxBlocks + 1];
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
        attend_pair(item, lds, list, q, k, vt, row_ptr, col_idx, n, nb, hkv, G, run, scale_log2,
                    out);
    }
}

// V^T as LDS-ready images, one per 64-key sub-tile: image i of KV head g
// (keys 64 i .. 64 i + 63) holds row d (the 64 keys' values
// of head dimension d) as 8 chunks of 8 keys, chunk c at slot c ^ ((d >> 1) & 7), and inside
// every group of 16 keys bits 2 and 3 of the key index are swapped.  A
// lane's 8 keys of a PV operand fragment, {4h .. 4h+3, 8+4h .. 8+4h+3} of a
// group for lane half h (the order the S^T accumulator holds them in), are
// then one 16-byte chunk.  Keys past n are zero.  The first work-group also
// clears the attention kernel's eight per-XCD queue counters.
// grid (N_b * 2, hkv), 256 threads.
__global__ void __launch_bounds__(256)
v_transpose_kernel(Rows v, int n, int n_img, uint16_t* __restrict__ vt, int* __restrict__ queue)
{
    __shared__ uint16_t tile[64][kD + 8];
    const int g = blockIdx.y, key0 = blockIdx.x * 64, tid = threadIdx.x;
    if (blockIdx.x == 0 && g == 0 && tid < 8) queue[tid] = 0;
    const uint16_t* src = v.row(g, key0);
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 4, ch = e & 15;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (key0 + row < n) val = *reinterpret_cast<const u32x4*>(src + row * v.st + 8 * ch);
        *reinterpret_cast<u32x4*>(&tile[row][8 * ch]) = val;
    }
    __syncthreads();
    uint16_t* dst = vt + ((size_t)g * n_img + blockIdx.x) * kImg;
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;                    // slot e & 7 of row d
        const int d = e >> 3, c = (e & 7) ^ ((d >> 1) & 7);
        u32x4 val;
        for (int x = 0; x < 4; ++x) {
            const int p0 = 8 * c + 2 * x;               // positions p0, p0 + 1
            const int k0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);
            val[x] = (uint32_t)tile[k0][d] | ((uint32_t)tile[k0 + 1][d] << 16);
        }
        *reinterpret_cast<u32x4*>(dst + 8 * e) = val;
    }
}

}  // namespace

hipError_t launch_v_transpose(Rows v, int n, int hkv, uint16_t* vt, int* queue,
                              hipStream_t stream)
{
    const int n_img = (n + kB - 1) / kB * 2;
    hipLaunchKernelGGL(v_transpose_kernel, dim3(n_img, hkv), dim3(256), 0, stream, v, n, n_img, vt,
                       queue);
    return hipGetLastError();
}

hipError_t launch_attend(Rows q, Rows k, const uint16_t* vt,
                         const int32_t* row_ptr, const int32_t* col_idx, int n, int hq, int hkv,
                         int* counters, OutRows out, hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv;
    const int npairs = (nb + 1) / 2;
    int run = npairs <= kWholeHeadPairs ? npairs : kPairRun;
    if (run > npairs * hkv / 8) run = npairs * hkv / 8;
    if (run < 1) run = 1;
    const long long chunks = (long long)((npairs + run - 1) / run) * hkv;
    const long long items = ((chunks + 7) / 8) * 8 * G * run;
    const int per_xcd = (int)(items / 8);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int groups = cus;   // one resident work-group of 8 wavefronts per CU
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    hipLaunchKernelGGL(attend_kernel, dim3(groups), dim3(kThreads), 0, stream, q, k, vt, row_ptr, col_idx,
                       n, nb, hkv, G, run, scale_log2, per_xcd, counters, out);
    return hipGetLastError();
}

}  // namespace crisp
