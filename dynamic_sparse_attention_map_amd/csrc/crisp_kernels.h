// Internal launchers of the CRISP HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crisp {

constexpr int kD = 128;            // head_dim
constexpr int kB = 128;            // block size B (tokens per block)
constexpr int kMaxBlocks = 4096;   // largest N_b (seq_len 524288 at B = 128)
constexpr int kRouteSegs = 64;     // tile segments per head in the routing row reduction

// A bf16 operand [heads][tokens][128] with arbitrary head and token strides
// in elements; the 128 head-dimension values of one row are contiguous.
struct Rows {
    const uint16_t* p;
    long long sh, st;               // head stride, token stride
    __host__ __device__ const uint16_t* row(int h, long long i) const { return p + h * sh + i * st; }
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

hipError_t launch_route(Rows q, Rows k, int n, int hq, int hkv,
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
};

hipError_t launch_select(Rows q, Rows k, const uint8_t* pattern,
                         const float* p_v, const float* p_s, int n, int hq, int hkv,
                         const VsRule& vs, float gamma, const SelectScratch& s, int32_t* sel_v,
                         int32_t* sel_s, int32_t* sel_counts, int32_t* row_ptr, int32_t* col_idx,
                         hipStream_t stream);

// queue: the attention kernel's 8 ints of device scratch, cleared here.
hipError_t launch_v_transpose(Rows v, int n, int hkv, uint16_t* vt, int* queue,
                              hipStream_t stream);

// row_ptr / col_idx == nullptr: dense causal lists.
// counters: 8 ints of device scratch, zero on entry (launch_v_transpose
// clears them on the same stream).
hipError_t launch_attend(Rows q, Rows k, const uint16_t* vt,
                         const int32_t* row_ptr, const int32_t* col_idx, int n, int hq, int hkv,
                         int* counters, OutRows out, hipStream_t stream);

}  // namespace crisp
