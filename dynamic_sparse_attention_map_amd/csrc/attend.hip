// Block-sparse causal GQA attention (Eq. 1) on bf16 matrix cores.
//
// One work-group of 4 wavefronts computes one (query head, query block):
// 128 queries, 32 per wavefront.  The listed key blocks are streamed as
// 64-key sub-tiles through double-buffered LDS (K row-major, V transposed),
// and each wavefront runs
//     S^T = K Q^T          (32x32x16 bf16 MFMA, fp32 accumulate)
//     online softmax       (exp2 domain, fp32 running max / sum)
//     O^T += V^T P^T       (P rounded to bf16, fp32 accumulate)
// Computing S^T rather than S leaves each lane holding one query's scores
// in exactly the register order the P^T operand of the second product
// needs, so P never leaves registers.  The causal mask is applied only on
// the diagonal key block; sub-tiles that lie entirely in a wavefront's
// future are skipped.
#include "crisp_common.h"
#include "crisp_kernels.h"

namespace crisp {

namespace {

constexpr int kKT = 64;                   // keys per sub-tile
constexpr int kKPitch = kD + 8;           // K tile row pitch (bf16), 272 bytes
constexpr int kVPitch = kKT + 4;          // V^T tile row pitch (bf16), 136 bytes
constexpr int kKStage = kKT * kKPitch;    // bf16 elements
constexpr int kVStage = kD * kVPitch;
constexpr int kStage = kKStage + kVStage;

// One query block of one head.  Work items are numbered like a grid of
// ceil(Nb*hkv / 8) * 8 * G work-groups whose item b belongs to XCD b % 8:
// its j = b / 8-th slot there takes chunk (j / G) * 8 + b % 8 and head j % G
// of that chunk, where chunk c covers the G query heads of KV head c % hkv at
// query block Nb-1-c/hkv.  Each XCD thus keeps whole GQA groups (sharing K/V
// in its L2) and walks the query blocks from the longest causal row down.
__device__ __forceinline__ void
attend_row(int b, uint16_t* lds, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
           const uint16_t* __restrict__ vt, const int32_t* __restrict__ row_ptr,
           const int32_t* __restrict__ col_idx, int n, int nb, int hkv, int G,
           float scale_log2, uint16_t* __restrict__ out)
{
    const int slot = b >> 3;
    const int chunk = (slot / G) * 8 + (b & 7);
    if (chunk >= nb * hkv) return;
    const int qb = nb - 1 - chunk / hkv;
    const int g = chunk % hkv;
    const int h = g * G + slot % G;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int len, lbase = 0;
    if (row_ptr) {
        lbase = row_ptr[h * (nb + 1) + qb];
        len = row_ptr[h * (nb + 1) + qb + 1] - lbase;
    } else {
        len = qb + 1;
    }

    const int qc = 32 * w + l32;                       // query within the block
    const size_t qrow = (size_t)h * n + (size_t)qb * kB + qc;
    bf16x8 qf[8];
    for (int s = 0; s < 8; ++s)
        qf[s] = *reinterpret_cast<const bf16x8*>(q + qrow * kD + 16 * s + 8 * hi);

    f32x16 o[4];
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float rescale_gap = 8.0f / scale_log2;   // 2^8 in probability

    const uint16_t* kg = k + (size_t)g * n * kD;
    const uint16_t* vg = vt + (size_t)g * kD * n;
    const int ntiles = 2 * len;

    // The row's key-block list is held in registers, 64 entries per chunk:
    // lane x of idx_cur holds entry 64*chunk + x, idx_nxt the next chunk
    // (prefetched a whole chunk ahead).  Tile t reads entry t/2 with a
    // wave-uniform readlane, so no K/V load waits on a list load.
    int lchunk = 0, idx_cur = -1, idx_nxt = -1;
    if (row_ptr) {
        idx_cur = (lane < len) ? col_idx[lbase + lane] : -1;
        idx_nxt = (64 + lane < len) ? col_idx[lbase + 64 + lane] : -1;
    }
    // a listed block outside [0, qb] is ignored (never addressed)
    auto block_of = [&](int t) {
        const int e = t >> 1;
        int kb = e;
        if (row_ptr) {
            const int src = ((e >> 6) == lchunk) ? idx_cur : idx_nxt;
            kb = __builtin_amdgcn_readlane(src, e & 63);
        }
        return (kb >= 0 && kb <= qb) ? kb : -1;
    };

    // staging: 4 x 16 bytes of K and 4 x 16 bytes of V^T per thread
    u32x4 pk[4], pv[4];
    auto load_tile = [&](int t) {
        const int kb = max(block_of(t), 0);
        const size_t key0 = (size_t)kb * kB + (t & 1) * kKT;
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            const int row = e >> 4, ch = e & 15;              // 64 keys x 16 chunks
            pk[i] = *reinterpret_cast<const u32x4*>(kg + (key0 + row) * kD + 8 * ch);
            const int dr = e >> 3, vc = e & 7;                // 128 d-rows x 8 chunks
            pv[i] = *reinterpret_cast<const u32x4*>(vg + (size_t)dr * n + key0 + 8 * vc);
        }
    };
    auto store_tile = [&](int stage) {
        uint16_t* ks = lds + stage * kStage;
        uint16_t* vs = ks + kKStage;
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            *reinterpret_cast<u32x4*>(ks + (e >> 4) * kKPitch + 8 * (e & 15)) = pk[i];
            *reinterpret_cast<u32x2*>(vs + (e >> 3) * kVPitch + 8 * (e & 7)) = u32x2{pv[i][0], pv[i][1]};
            *reinterpret_cast<u32x2*>(vs + (e >> 3) * kVPitch + 8 * (e & 7) + 4) = u32x2{pv[i][2], pv[i][3]};
        }
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    for (int t = 0; t < ntiles; ++t) {
        if (row_ptr && ((t >> 1) >> 6) != lchunk) {
            // entering the next 64-entry chunk: rotate, prefetch the one after
            lchunk = (t >> 1) >> 6;
            idx_cur = idx_nxt;
            const int nxt = 64 * (lchunk + 1) + lane;
            idx_nxt = (nxt < len) ? col_idx[lbase + nxt] : -1;
        }
        if (t + 1 < ntiles) load_tile(t + 1);
        __syncthreads();
        const int kb = block_of(t);
        const int sub = t & 1;
        const bool diag = (kb == qb);
        // keys 64..127 of the diagonal block lie after every query < 64
        const bool skip = kb < 0 || (diag && sub == 1 && w < 2);
        if (!skip) {
            const uint16_t* ks = lds + (t & 1) * kStage;
            const uint16_t* vs = ks + kKStage;
            f32x16 s[2];
            s[0] = f32x16{};
            s[1] = f32x16{};
            for (int st = 0; st < 8; ++st)
                for (int a = 0; a < 2; ++a) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (32 * a + l32) * kKPitch + 16 * st + 8 * hi);
                    s[a] = mfma32(kf, qf[st], s[a]);
                }
            if (diag) {
                // causal mask on the diagonal block only (wave-uniform branch;
                // the empty asm keeps the compiler from if-converting it)
                asm volatile("; diagonal mask");
                for (int a = 0; a < 2; ++a)
                    for (int r = 0; r < 16; ++r) {
                        const int kc = kKT * sub + 32 * a + 8 * (r >> 2) + 4 * hi + (r & 3);
                        if (kc > qc) s[a][r] = -INFINITY;
                    }
            }
            // running max in raw-score units; the accumulator is rescaled only
            // when the max grows by more than 2^8 in probability (exact: the
            // final normalisation uses the same reference max)
            float tmax = -INFINITY;
            for (int a = 0; a < 2; ++a)
                for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[a][r]);
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
            // p = 2^(c (s - m)) as one FMA and one v_exp; a lane whose keys are
            // all masked so far keeps m = -inf and uses 0 as its reference
            const float neg_mc = (m_run == -INFINITY) ? 0.f : -m_run * scale_log2;
            bf16x8 pf[4];
            for (int a = 0; a < 2; ++a)
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[a][r], scale_log2, neg_mc));
                    l_run += p;
                    pf[2 * a + (r >> 3)][r & 7] = (__bf16)p;
                }
            for (int dt = 0; dt < 4; ++dt) {
                const uint16_t* vrow = vs + (32 * dt + l32) * kVPitch;
                for (int u = 0; u < 4; ++u) {
                    const int kk = 32 * (u >> 1) + 16 * (u & 1) + 4 * hi;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kk);
                    const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vrow + kk + 8);
                    const u32x4 vv = {lo[0], lo[1], hi2[0], hi2[1]};
                    o[dt] = mfma32(__builtin_bit_cast(bf16x8, vv), pf[u], o[dt]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile((t + 1) & 1);
    }

    const float l = l_run + swap_half(l_run);
    const float inv = (l > 0.f) ? 1.0f / l : 0.f;
    uint16_t* orow = out + qrow * kD;
    for (int dt = 0; dt < 4; ++dt)
        for (int j = 0; j < 4; ++j) {
            bf16x4 v4;
            for (int r = 0; r < 4; ++r) v4[r] = (__bf16)(o[dt][4 * j + r] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * j + 4 * hi) = v4;
        }
}

// Persistent work-groups (two per CU) drain eight per-XCD queues of work
// items; a group starts on the queue of its own XCD (work-group b is placed
// on XCD b % 8) and moves to the others once that one is empty.  ctr[x]
// counts items taken from queue x and must be zero at launch.
__global__ void __launch_bounds__(256, 2)
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
        attend_row(item, lds, q, k, vt, row_ptr, col_idx, n, nb, hkv, G, scale_log2, out);
    }
}

__global__ void zero_counters_kernel(int* __restrict__ ctr)
{
    if (threadIdx.x < 8) ctr[threadIdx.x] = 0;
}

// vt[g][d][key] = v[g][key][d]; grid (n/64, hkv), 256 threads.
__global__ void __launch_bounds__(256)
v_transpose_kernel(const uint16_t* __restrict__ v, int n, uint16_t* __restrict__ vt)
{
    __shared__ uint16_t tile[64][kD + 8];
    const int g = blockIdx.y, key0 = blockIdx.x * 64, tid = threadIdx.x;
    const uint16_t* src = v + ((size_t)g * n + key0) * kD;
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 4, ch = e & 15;
        *reinterpret_cast<u32x4*>(&tile[row][8 * ch]) =
            *reinterpret_cast<const u32x4*>(src + (size_t)row * kD + 8 * ch);
    }
    __syncthreads();
    uint16_t* dst = vt + (size_t)g * kD * n + key0;
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        const int d = e >> 3, c8 = e & 7;
        u32x4 val;
        for (int x = 0; x < 4; ++x)
            val[x] = (uint32_t)tile[8 * c8 + 2 * x][d] | ((uint32_t)tile[8 * c8 + 2 * x + 1][d] << 16);
        *reinterpret_cast<u32x4*>(dst + (size_t)d * n + 8 * c8) = val;
    }
}

}  // namespace

hipError_t launch_v_transpose(const uint16_t* v, int n, int hkv, uint16_t* vt, hipStream_t stream)
{
    hipLaunchKernelGGL(v_transpose_kernel, dim3(n / 64, hkv), dim3(256), 0, stream, v, n, vt);
    return hipGetLastError();
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                         const int32_t* row_ptr, const int32_t* col_idx, int n, int hq, int hkv,
                         int* counters, uint16_t* out, hipStream_t stream)
{
    const int nb = n / kB, G = hq / hkv;
    const long long chunks = (long long)nb * hkv;
    const long long items = ((chunks + 7) / 8) * 8 * G;
    const int per_xcd = (int)(items / 8);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int groups = 2 * cus;   // two resident work-groups per CU
    const float scale_log2 = kLog2e / sqrtf((float)kD);
    hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, stream, counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_kernel, dim3(groups), dim3(256), 0, stream, q, k, vt, row_ptr, col_idx,
                       n, nb, hkv, G, scale_log2, per_xcd, counters, out);
    return hipGetLastError();
}

}  // namespace crisp
