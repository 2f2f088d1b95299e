// Internal launchers of the CRISP HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct crisp_opts;   // include/crisp.h

namespace crisp {

constexpr int kD = 128;            // head_dim
constexpr int kB = 128;            // block size B (tokens per block)
constexpr int kMaxBlocks = 4096;   // largest N_b (seq_len 524288 at B = 128)
constexpr int kRouteSegs = 64;     // tile segments per head in the routing row reduction
// Up to these sizes a kernel runs one work-group per head over the whole
// head (bit-identical to the multi-launch path used beyond): the route
// reductions up to kRouteSmall key blocks, the PE cut-off up to kRadixSmall
// map entries (N_b <= 128).  The multi-launch scratch is not needed below.
constexpr int kRouteSmall = 64;
constexpr int kRadixSmall = 128 * 129 / 2;
// Up to kSelectSmall key blocks the selection after pooling is one launch
// of one work-group per head, which leaves most of the chip idle; that
// launch also lays out V^T (launch_select's vt job) in work-groups of its
// own, so the V^T images must not overlap the selection scratch there.
constexpr int kSelectSmall = 128;
inline bool select_lays_out_v(int nb) { return nb > 0 && nb <= kSelectSmall; }
// V^T image of 64 keys of one KV head (bf16 elements); N_b blocks take 2 N_b.
constexpr int kVImage = 64 * kD;

// A bf16 operand [heads][tokens][128] with arbitrary head and token strides
// in elements; the 128 head-dimension values of one row are contiguous.
struct Rows {
    const uint16_t* p;
    long long sh, st;               // head stride, token stride
    __host__ __device__ const uint16_t* row(int h, long long i) const { return p + h * sh + i * st; }
};
// The same rows for a group of sequences of one length seen as one layer of
// count * hper heads: head h is head h % hper of sequence h / hper, whose
// rows start at base[h / hper] (a device array); the strides are shared.
struct SeqRows {
    const uint16_t* const* base;
    int hper;
    long long sh, st;
    __device__ const uint16_t* row(int h, long long i) const
    {
        return base[h / hper] + (long long)(h % hper) * sh + i * st;
    }
};
struct OutRows {
    uint16_t* p;
    long long sh, st;
    __host__ __device__ uint16_t* row(int h, long long i) const { return p + h * sh + i * st; }
};

// Per-head state of the PE radix select (device memory, 64 bytes).
struct PeState {
    unsigned long long need;        // fixed-point mass still to cover
    unsigned long long tfix;        // fixed-point value of the cut-off entry
    uint32_t key_prefix;            // resolved high digits of the cut-off key
    uint32_t flat_prefix;           // resolved high digits of the cut-off flat index
    uint32_t before;                // entries strictly before the cut-off key
    uint32_t tie_need;              // cut-off-valued entries still to take
    uint32_t key_star;              // cut-off key (ascending order = value desc)
    uint32_t flat_star;             // last kept flat index among key_star entries
    uint32_t kstar;                 // K*
    uint32_t done;
    uint32_t pad[4];
};

// Radix select of the PE cut-off: value-key passes and flat-index passes.
constexpr int kValPasses = 3;      // 11 + 11 + 10 bits of the 32-bit key
constexpr int kRadixPasses = 5;    // then 12 + 12 bits of the 24-bit flat index
constexpr int kValBins = 2048;
constexpr int kFlatBins = 4096;

// Fixed point used for masses: value * 2^62 truncated (values are <= 1).
constexpr double kFix = 4611686018427387904.0;

struct RouteArgs {
    int router;                     // 0: C_struct >= tau (Alg. 2); 1: D_JS >= tau (Alg. 5)
    float tau;
    float* part_m;                  // [hq][Nb][128] per (tile, row) partials
    float* part_lo;
    float* part_up;
    float* jsd_kbar;                // [hkv][Nb][128] block key means (router 1)
    float* jsd_qbar;                // [hq][128] mean representative query (router 1)
    float* seg_m;                   // [hq][kRouteSegs][128] per (tile segment, row) max
    double* seg_l;                  //                and normaliser
    float* row_mx;                  // [hq][128] row max
    float* row_inv;                 // [hq][128] 1 / row normaliser
    float* tile_sums;               // [hq][4][Nb] slash-part sums per tile
};

template <class R>
hipError_t launch_route(R q, R k, int n, int hq, int hkv,
                        const RouteArgs& a, float* p_v, float* p_s, float* c_struct,
                        uint8_t* pattern, hipStream_t stream);

struct VsRule {
    int rule;                       // 0: mean floor, 1: median floor, 2: cumulative gamma
    float alpha;                    // floor multiplier (rules 0, 1)
    float gamma_vs;                 // coverage target (rule 2)
    int kmin_blocks;                // every rule clips to at least this many blocks
};

struct SelectScratch {
    float* qbar;                    // [hq][Nb][128]
    float* kbar;                    // [hkv][Nb][128]
    float* abar;                    // [hq][Nb(Nb+1)/2] triangular rows
    unsigned long long* hist_mass;  // [hq][kValPasses][kValBins]
    uint32_t* hist_count;           // [hq][kRadixPasses][kFlatBins]
    uint32_t* pass_ctr;             // [hq][kRadixPasses]
    PeState* state;                 // [hq]
    uint8_t* bitmap;                // [hq][2][Nb]
    unsigned long long* rowmask;    // [hq][Nb][ceil(Nb/64)] list membership ballots
};

// V^T layout for the attention kernel riding on the selection launch
// (vt == nullptr: none).  Done only when select_lays_out_v(N_b); it then
// also clears queue (the attention kernel's 8 ints), as launch_v_transpose.
template <class R>
struct VtJob {
    R v;
    uint16_t* vt;
    int* queue;
};

template <class R>
hipError_t launch_select(R q, R k, const uint8_t* pattern,
                         const float* p_v, const float* p_s, int n, int hq, int hkv,
                         const VsRule& vs, float gamma, const SelectScratch& s, int32_t* sel_v,
                         int32_t* sel_s, int32_t* sel_counts, int32_t* row_ptr, int32_t* col_idx,
                         const VtJob<R>& vt, hipStream_t stream);

// queue: the attention kernel's 8 ints of device scratch, cleared here.
template <class R>
hipError_t launch_v_transpose(R v, int n, int hkv, uint16_t* vt, int* queue,
                              hipStream_t stream);

// row_ptr / col_idx == nullptr: dense causal lists.
// counters: 8 ints of device scratch, zero on entry (launch_v_transpose, or
// launch_select's V^T job, clears them on the same stream).
hipError_t launch_attend(Rows q, Rows k, const uint16_t* vt,
                         const int32_t* row_ptr, const int32_t* col_idx, int n, int hq, int hkv,
                         int* counters, OutRows out, hipStream_t stream);

// One sequence of a batched attention launch (an entry of a device table):
// its operands with their strides, its V^T images and block lists, and its
// share of the eight per-XCD work queues (slots slot0 .. slot0 + per_xcd - 1
// of every queue).  row_ptr == nullptr: dense causal lists.
struct SeqDesc {
    const uint16_t* q;
    const uint16_t* k;
    uint16_t* out;
    const uint16_t* vt;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    long long q_sh, q_st, k_sh, k_st, o_sh, o_st;
    int n, run, slot0, per_xcd, pair_major;
};

// Work-queue plan of one sequence's attention: pair-run length, slots per
// XCD queue, and the order of a chunk's items (1: pair-major, 0: head-major).
void attend_plan(int n, int hq, int hkv, int* run, int* per_xcd, int* pair_major);

// Copies `count` host descriptors into the device table at table[first ..]
// and marks their queue slots in slot_seq (kernel arguments only: no host
// copy), in launches of up to 16 descriptors.
hipError_t launch_seq_table(const SeqDesc* descs, int first, int count, SeqDesc* table,
                            int* slot_seq, hipStream_t stream);

// Writes `count` host pointers into the device array dst (kernel arguments
// only), in launches of up to 64.
hipError_t launch_ptr_table(const void* const* ptrs, int count, const void** dst,
                            hipStream_t stream);

// Attention of every sequence in `table` in one launch; total_per_xcd is the
// sum of their per_xcd, slot_seq maps a queue slot to its sequence and
// counters are 8 ints at zero (launch_v_transpose clears them).
hipError_t launch_attend_batch(const SeqDesc* table, const int* slot_seq, int total_per_xcd,
                               int hq, int hkv, int* counters, hipStream_t stream);

// crisp_prefill's argument checks without a workspace: shape, options,
// alpha and the q/k/v/out pointers.  On CRISP_OK, *ws_need is the workspace
// the call needs (0 for an empty call, which then needs nothing else).
int validate_prefill(const void* q, const void* k, const void* v, int seq_len, int n_heads,
                     int n_kv_heads, int head_dim, int block_size, float alpha,
                     const ::crisp_opts* opts, const void* out, size_t* ws_need);

}  // namespace crisp
