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
//     online softmax       (exp2 domain, fp32 running max)
//     O^T += V^T P^T       (P rounded to bf16, fp32 accumulate)
//     l   += SEL P^T       (row sums of the same bf16 P, 16x16x32 MFMA)
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
#include "work_order.h"

namespace crisp {

namespace {

constexpr int kKT = 64;                   // keys per sub-tile
constexpr int kImg = kKT * kD;            // one K or V^T sub-tile image, bf16 elements (16 KiB)
static_assert(kImg == kVImage, "V^T image size");
constexpr int kStageBytes = 4 * kImg;     // K image, then V^T image
constexpr int kStages = 4;                // LDS ring depth

constexpr int kThreads = 512;             // 8 wavefronts: two query blocks x 4

constexpr int kListWords = kMaxBlocks / 32;   // bitmap words per row

// One work item: the two query blocks of pair it.pair of head it.h (the
// order is in work_order.h).
__device__ __forceinline__ void
attend_pair(int b, uint16_t* lds, uint32_t* list, Rows q, Rows k,
            const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr,
            const int32_t* __restrict__ col_idx, int n, int nb, int hkv, int G, int run,
            bool pair_major, float scale_log2, OutRows out)
{
    WorkItem it;
    if (!work_item(b, nb, hkv, G, run, pair_major, &it)) return;
    const int pair = it.pair, g = it.g, h = it.h;
    const int qb_hi = nb - 1 - 2 * pair;
    const int qb_lo = qb_hi - 1;                   // -1: no second block

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int half = w >> 2, wq = w & 3;           // half 0: qb_hi, half 1: qb_lo
    const int l32 = lane & 31, hi = lane >> 5;
    const int myqb = half ? qb_lo : qb_hi;
    const bool active = myqb >= 0;

    // this wavefront's queries, loaded first so that their latency overlaps
    // the list build below (a partial last block has rows past the end:
    // they load the last row and their results are never stored)
    const int qc = 32 * wq + l32;                         // query within its block
    const int qpos = (active ? myqb : 0) * kB + qc;
    const bool q_valid = active && qpos < n;
    bf16x8 qf[8];
    {
        const uint16_t* qrow = q.row(h, min(qpos, n - 1));
        for (int s = 0; s < 8; ++s)
            qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hi);
    }

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


    f32x16 o[4];
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY;
    // Row sums on the matrix cores, so that the vector phase (the co-bound
    // with the products) has no additions: lsum += SEL P^T with P^T[u] as a
    // 32x16 operand of a 16x16x32 product.  Its k-slots 8 (l / 16) .. +7 are
    // lane l's eight probabilities of query l % 32, so the k-groups 0 and 2
    // hold queries 0-15 (both key halves) and the groups 1 and 3 queries
    // 16-31.  SEL row 0 is 1 on groups 0 and 2, row 1 on groups 1 and 3 and
    // every other row 0: lane q < 16 then holds the sum of query q in
    // lsum[0] and of query q + 16 in lsum[1], and every other element stays
    // 0.  These are sums of the bf16 probabilities the PV product uses, so
    // the weights of a row sum to one exactly as the products see them.
    f32x4 lsum = f32x4{};
    bf16x8 sel;
    {
        const int m = lane & 15, par = (lane >> 4) & 1;
        const __bf16 one = (__bf16)(((m == 0 && par == 0) || (m == 1 && par == 1)) ? 1.0f : 0.0f);
        for (int j = 0; j < 8; ++j) sel[j] = one;
    }
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
    // these images already (v_image_write), so its copy is contiguous.
    // Copies take a wave-uniform base (scalar registers) and a 32-bit byte
    // offset per lane.  K: lane l of copy j holds key 4 (2w + j) + l / 16 of
    // the sub-tile, chunk (l % 16) ^ (key & 15).
    uint32_t k_off[2];
    for (int j = 0; j < 2; ++j) {
        const int row = 4 * (2 * w + j) + (lane >> 4);
        k_off[j] = (uint32_t)(row * k.st + 8 * ((lane & 15) ^ (row & 15))) * 2u;
    }
    const uint32_t v_off = (uint32_t)(1024 * w + 8 * lane) * 2u;
    const uint32_t lds_base = lds_address(lds);
    auto issue_tile = [&](int t, uint32_t dsc) {        // tile t into stage t % 4
        const int kb = (int)(dsc & 0xffffu), sub = t & 1;
        const int key0 = kb * kB + sub * kKT;
        const uint32_t sb = lds_base + (uint32_t)((t & 3) * kStageBytes) + 2048u * w;
        const bool full = key0 + kKT <= n;
        // keys past the end of a partial last block repeat the last key
        // (every query that exists masks them: they lie in its future); the
        // base then sits at the sub-tile's first existing key, or at the last
        // key when none exists, so every offset stays non-negative
        const int kfirst = min(key0, n - 1);
        const uint16_t* kt = kg + (long long)kfirst * k.st;
        for (int j = 0; j < 2; ++j) {
            uint32_t off = k_off[j];
            if (!full) {
                const int r = 4 * (2 * w + j) + (lane >> 4);
                const int row = min(key0 + r, n - 1) - kfirst;
                off = (uint32_t)(row * k.st + 8 * ((lane & 15) ^ (r & 15))) * 2u;
            }
            copy16_to_lds(kt, off, sb + 1024u * j);
        }
        const uint16_t* vimg = vg + (size_t)(2 * kb + sub) * kImg;
        for (int j = 0; j < 2; ++j) copy16_to_lds(vimg, v_off + 1024u * j, sb + 2 * kImg + 1024u * j);
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
    // the order the matrix cores consume them, four reads ahead.
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
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
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
            lsum[0] *= alpha;                          // query l32 (lanes < 16)
            lsum[1] *= __shfl_down(alpha, 16);         // query l32 + 16
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
        for (int u = 0; u < 4; ++u)            // key group u: s[u >> 1][8 (u & 1) .. +7]
            for (int j = 0; j < 8; ++j)
                pf[u][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + j], scale_log2, neg_mc));
    };
    // O^T += V^T P^T for the tile in `stage`, and the row sums.  The four
    // row-sum products need no LDS operand, so they go first and cover the
    // latency of the first V^T fragment reads (then four reads ahead).
    auto pv_mfma = [&](int stage) {
        const uint16_t* vbase = lds + stage * (kStageBytes / 2) + kImg + l32 * kKT;
        bf16x8 vf[16];                       // vf[4 u + dt]
        for (int u = 0; u < 4; ++u)
            for (int dt = 0; dt < 4; ++dt)
                vf[4 * u + dt] = *reinterpret_cast<const bf16x8*>(vbase + 32 * dt * kKT + 8 * ((2 * u + hi) ^ vx));
        for (int u = 0; u < 4; ++u) lsum = mfma16(sel, pf[u], lsum);
        for (int u = 0; u < 4; ++u)
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vf[4 * u + dt], pf[u], o[dt]);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
    };

    // Schedule.  Per tile t every wavefront runs a matrix phase M_t = PV(t-1)
    // + QK(t) and a vector phase V_t = softmax(t); one barrier ends each
    // iteration.  Half 0 runs M_t then V_t; half 1 runs V_{t-1} then M_t, so
    // the two wavefronts sharing a SIMD start each iteration on different
    // units and stay out of each other's way without a barrier in between.
    // Tiles rotate through 4 LDS stages: tile t is read in iterations t (K)
    // and t+1 (V^T).  Each wavefront issues its copies of tile t+2 during
    // iteration t, into the stage of tile t-2 (last read in iteration t-1),
    // and waits for those of tile t+1 before the barrier that ends iteration
    // t.  Half 1 issues them before its vector phase, half 0 after its
    // matrix phase: so half 0's products start right after the barrier, and
    // the two halves' copies do not queue for the address unit at the same
    // moment (issuing four copies costs a wavefront about 300 cycles; with
    // every wavefront issuing at the start of the iteration, the kernel was
    // 0.5-1.1% slower at 131072 tokens).
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
            if (half == 1 && more) issue_tile(t + 2, d2);
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
            if (half == 0 && more) issue_tile(t + 2, d2);
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
    // the row sum of query l32 from the lane that holds it
    const float l0 = __shfl(lsum[0], l32 & 15), l1 = __shfl(lsum[1], l32 & 15);
    const float l = (l32 < 16) ? l0 : l1;
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
// (The item order is a template parameter here, so that each order compiles
// to its own loop: a run-time flag cost 0.4% at 131072 tokens.)
template <bool PairMajor>
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
        const int item = __builtin_amdgcn_readfirstlane(s_item);
        __syncthreads();
        if (item < 0) break;
        attend_pair(item, lds, list, q, k, vt, row_ptr, col_idx, n, nb, hkv, G, run, PairMajor,
                    scale_log2, out);
    }
}

// The same for several sequences in one launch: queue slot j (every queue
// has the same layout) belongs to sequence slot_seq[j], whose items occupy
// slots slot0 .. slot0 + per_xcd - 1; within it the item is decoded exactly
// as in a launch of that sequence alone, so each sequence's output is the
// same bits.
__global__ void __launch_bounds__(kThreads)
attend_batch_kernel(const SeqDesc* __restrict__ seqs, const int* __restrict__ slot_seq, int hkv,
                    int G, float scale_log2, int per_xcd, int* __restrict__ ctr)
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
        const int item = __builtin_amdgcn_readfirstlane(s_item);
        __syncthreads();
        if (item < 0) break;
        const int j = item >> 3;
        const SeqDesc& d = seqs[__builtin_amdgcn_readfirstlane(slot_seq[j])];
        const int n = d.n;
        attend_pair(8 * (j - d.slot0) + (item & 7), lds, list, Rows{d.q, d.q_sh, d.q_st},
                    Rows{d.k, d.k_sh, d.k_st}, d.vt, d.row_ptr, d.col_idx, n, (n + kB - 1) / kB, hkv,
                    G, d.run, d.pair_major != 0, scale_log2, OutRows{d.out, d.o_sh, d.o_st});
    }
}

// Up to 16 descriptors per launch, passed by value.
struct SeqChunk {
    SeqDesc d[16];
    int first, count;
};

// Up to 64 pointers per launch, passed by value.
struct PtrChunk {
    const void* p[64];
    int count;
};

// one work-group of 64 threads
__global__ void __launch_bounds__(64)
ptr_table_kernel(PtrChunk c, const void** __restrict__ dst)
{
    if ((int)threadIdx.x < c.count) dst[threadIdx.x] = c.p[threadIdx.x];
}

// grid (ceil(max per_xcd / 256), count), 256 threads
__global__ void __launch_bounds__(256)
seq_table_kernel(SeqChunk c, SeqDesc* __restrict__ table, int* __restrict__ slot_seq)
{
    const int i = blockIdx.y;
    const SeqDesc& d = c.d[i];
    if (blockIdx.x == 0 && threadIdx.x == 0) table[c.first + i] = d;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j < d.per_xcd) slot_seq[d.slot0 + j] = c.first + i;
}

// The V^T images (layout at v_image_stage), one per work-group.  The first
// work-group also clears the attention kernel's eight per-XCD queue
// counters.  grid (N_b * 2, hkv), 256 threads.
template <class R>
__global__ void __launch_bounds__(256)
v_transpose_kernel(R v, int n, int n_img, uint16_t* __restrict__ vt, int* __restrict__ queue)
{
    __shared__ uint16_t tile[64][kVPitch];
    const int g = blockIdx.y, i = blockIdx.x, tid = threadIdx.x;
    if (i == 0 && g == 0 && tid < 8) queue[tid] = 0;
    v_image_stage(v, n, g, i, tile, tid);
    __syncthreads();
    v_image_write(tile, vt + ((size_t)g * n_img + i) * kVImage, tid);
}

}  // namespace

template <class R>
hipError_t launch_v_transpose(R v, int n, int hkv, uint16_t* vt, int* queue, hipStream_t stream)
{
    const int n_img = (n + kB - 1) / kB * 2;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(v_transpose_kernel<R>), dim3(n_img, hkv), dim3(256), 0, stream, v, n, n_img, vt,
                       queue);
    return hipGetLastError();
}

void attend_plan(int n, int hq, int hkv, int* run_out, int* per_xcd_out, int* pair_major_out)
{
    const WorkPlan w = work_plan(n, hq, hkv);
    *run_out = w.run;
    *per_xcd_out = w.per_xcd;
    *pair_major_out = w.pair_major;
}

namespace {
int resident_groups()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus;   // one resident work-group of 8 wavefronts per CU
}
}  // namespace

hipError_t launch_attend(Rows q, Rows k, const uint16_t* vt,
                         const int32_t* row_ptr, const int32_t* col_idx, int n, int hq, int hkv,
                         int* counters, OutRows out, hipStream_t stream)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv;
    int run, per_xcd, pair_major;
    attend_plan(n, hq, hkv, &run, &per_xcd, &pair_major);
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    if (pair_major)
        hipLaunchKernelGGL(attend_kernel<true>, dim3(resident_groups()), dim3(kThreads), 0, stream,
                           q, k, vt, row_ptr, col_idx, n, nb, hkv, G, run, scale_log2, per_xcd,
                           counters, out);
    else
        hipLaunchKernelGGL(attend_kernel<false>, dim3(resident_groups()), dim3(kThreads), 0, stream,
                           q, k, vt, row_ptr, col_idx, n, nb, hkv, G, run, scale_log2, per_xcd,
                           counters, out);
    return hipGetLastError();
}

hipError_t launch_seq_table(const SeqDesc* descs, int first, int count, SeqDesc* table,
                            int* slot_seq, hipStream_t stream)
{
    for (int at = 0; at < count; at += 16) {
        SeqChunk c{};
        c.first = first + at;
        c.count = count - at < 16 ? count - at : 16;
        int most = 1;
        for (int i = 0; i < c.count; ++i) {
            c.d[i] = descs[at + i];
            if (c.d[i].per_xcd > most) most = c.d[i].per_xcd;
        }
        hipLaunchKernelGGL(seq_table_kernel, dim3((most + 255) / 256, c.count), dim3(256), 0, stream,
                           c, table, slot_seq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_ptr_table(const void* const* ptrs, int count, const void** dst,
                            hipStream_t stream)
{
    for (int at = 0; at < count; at += 64) {
        PtrChunk c{};
        c.count = count - at < 64 ? count - at : 64;
        for (int i = 0; i < c.count; ++i) c.p[i] = ptrs[at + i];
        hipLaunchKernelGGL(ptr_table_kernel, dim3(1), dim3(64), 0, stream, c, dst + at);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_attend_batch(const SeqDesc* table, const int* slot_seq, int total_per_xcd,
                               int hq, int hkv, int* counters, hipStream_t stream)
{
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    hipLaunchKernelGGL(attend_batch_kernel, dim3(resident_groups()), dim3(kThreads), 0, stream, table,
                       slot_seq, hkv, hq / hkv, scale_log2, total_per_xcd, counters);
    return hipGetLastError();
}

template hipError_t launch_v_transpose<Rows>(Rows, int, int, uint16_t*, int*, hipStream_t);
template hipError_t launch_v_transpose<SeqRows>(SeqRows, int, int, uint16_t*, int*, hipStream_t);

}  // namespace crisp
