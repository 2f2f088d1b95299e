// The attention kernel's work order: how the (query-block pair, head) work
// items of one sequence are laid out over the eight per-XCD queues.  Host and
// device share it: the host sizes the queues (work_plan) and the kernel
// decodes each claimed slot (work_item).
#pragma once

#include "crisp_kernels.h"

namespace crisp {

// Run length of one head's pairs on an XCD: a whole head when it has at most
// kWholeHeadPairs pairs, else kPairRun; never so long that an XCD is left
// without a chunk of its own (fewer KV heads than XCDs).  Measured at 1024
// and 4096 blocks: whole heads were 0.9% faster at 1024, runs of 256 0.2%
// faster than 512 or 1024 at 4096.
constexpr int kPairRun = 256;
constexpr int kWholeHeadPairs = 512;
// Pair-major order (below) while one KV head's K and V^T take at most this
// many bytes (16384 tokens at head_dim 128).  Measured against head-major:
// -7% at 8192 tokens, -3% at 16384, +4% at 32768, +13% at 131072.
constexpr long long kPairMajorKvBytes = 8ll << 20;
// Pair-major runs are this many pairs, and chunk c takes KV head
// (c + c / hkv) % hkv (below), so that each XCD walks the KV groups in turn
// instead of serving one group for the whole launch: with few items per
// work-group, the groups' unequal totals otherwise leave some XCDs idle at
// the end.  Measured against one run per head: -0.5% at 4096 tokens, -1.6%
// at 8192, -3.4% at 12288, -2.1% at 16384 (runs of 4: -0.8%, -2.0%, -3.1%,
// -1.3%).  Head-major order keeps each group on its XCD: the same rotation
// there, with runs of 64-256 pairs, was 0.5-1.4% slower at 65536 and
// 131072 tokens (L2 reuse within a group counts more there).
constexpr int kPairMajorRun = 8;

// Work items.  Pair p is query blocks Nb-1-2p and Nb-2-2p.  A chunk is `run`
// consecutive pairs of the G query heads of one KV head: chunk c covers KV
// head c % hkv (pair-major: (c % hkv + c / hkv) % hkv) and pairs
// run * (c / hkv) onward, and holds its G x run items
// head-major (one head's run of pairs, then the next head's), or for short
// sequences pair-major (the G heads' pair p, then their pair p + 1).  Item b belongs
// to XCD b % 8; its j = b / 8-th slot there is item j % (G run) of chunk
// (j / (G run)) * 8 + b % 8.  In head-major order each XCD keeps whole GQA
// groups and walks the pairs from the longest causal rows down in runs, and
// the work-groups of an XCD start one head's adjacent pairs close together
// in time: their lists
// are alike, they walk them in step, and all but the first find most K/V
// tiles in L2.  (Interleaving the heads instead, pair by pair, leaves almost
// no reuse: the long rows of diffuse heads start far apart in time.)  XCD x
// starts its chunks' heads at head x % G: vertical-slash heads, with short,
// scattered lists, miss L2 far more often than diffuse heads, and this keeps
// the XCDs from all running them at the same time.  (Runs inside a chunk are
// rotated, never reordered across chunks, so the walk from the longest rows
// down is kept.)  When a KV head's K and V fit in an XCD's L2
// whatever the order, pair-major is the better schedule: it hands out the
// longest items of all G heads first, so no head's long rows start late;
// its chunks are short and rotate over the KV groups (kPairMajorRun).
struct WorkPlan {
    int run;          // pairs per chunk
    int per_xcd;      // slots per XCD queue
    int pair_major;   // 1: pair-major order inside a chunk
};

__host__ __device__ inline WorkPlan work_plan(int n, int hq, int hkv)
{
    const int nb = (n + kB - 1) / kB, G = hq / hkv;
    const int npairs = (nb + 1) / 2;
    const bool pair_major = (long long)n * kD * 4 <= kPairMajorKvBytes;
    int run = npairs <= kWholeHeadPairs ? npairs : kPairRun;
    if (pair_major && run > kPairMajorRun) run = kPairMajorRun;
    if (run > npairs * hkv / 8) run = npairs * hkv / 8;
    if (run < 1) run = 1;
    const long long chunks = (long long)((npairs + run - 1) / run) * hkv;
    const long long items = ((chunks + 7) / 8) * 8 * G * run;
    return WorkPlan{run, (int)(items / 8), pair_major ? 1 : 0};
}

struct WorkItem {
    int pair;         // query blocks nb - 1 - 2 pair and nb - 2 - 2 pair
    int g;            // KV head
    int h;            // query head (of group g)
};

// Slot b of the queues (queue b % 8, position b / 8); false for the padding
// slots past the last pair.
__host__ __device__ inline bool work_item(int b, int nb, int hkv, int G, int run, bool pair_major,
                                          WorkItem* it)
{
    const int npairs = (nb + 1) >> 1;
    const int slot = b >> 3;
    const int per_chunk = G * run;
    const int chunk = (slot / per_chunk) * 8 + (b & 7);
    const int r = slot % per_chunk;
    const int pair = (chunk / hkv) * run + (pair_major ? r / G : r % run);
    if (pair >= npairs) return false;
    const int g = (chunk % hkv + (pair_major ? chunk / hkv : 0)) % hkv;
    it->pair = pair;
    it->g = g;
    it->h = g * G + ((pair_major ? r % G : r / run) + (b & 7)) % G;
    return true;
}

}  // namespace crisp
