/*
 * crisp.h -- C ABI of the MI355X (gfx950) CRISP sparse-prefill library.
 *
 * CRISP ("Cliff-awaRe Input-adaptive Sparse Prefilling with Structural-Mass-
 * Motivated Routing", arXiv 2609.01925) prefills one attention layer in three
 * steps per query head (Alg. 1): route the head with the structural proxy
 * C_struct (Alg. 2, Eq. 2), select a block index set -- the sink-aware noise
 * floor on vertical-slash heads (Alg. 3, Eq. 3-4) or gamma-cumsum over a
 * pooled map on pooled-estimation heads (Alg. 4) -- and run block-sparse
 * causal attention over that set (Eq. 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors: bf16, contiguous, batch 1.  q is [n_heads][seq_len][head_dim];
 *   k, v are [n_kv_heads][seq_len][head_dim]; query head h reads KV head
 *   h / (n_heads / n_kv_heads) (grouped-query attention).  out has q's shape.
 *   crisp_prefill_batch alone takes several sequences and strided layouts.
 * Device pointers: every array argument is device memory, 16-byte aligned
 *   (the workspace 256-byte aligned).  opts is a host pointer (may be NULL).
 * Sizes: head_dim == 128 and block_size == 128 (B in the paper); any
 *   seq_len >= 0; n_heads a multiple of n_kv_heads.  Blocks partition the
 *   sequence as in Section 4.3 of the paper: N_b = ceil(seq_len /
 *   block_size), the last block holding seq_len - (N_b - 1) * block_size
 *   tokens.  seq_len == 0 is an empty call: after the size and option checks
 *   it returns CRISP_OK without reading any pointer or launching anything.
 * Ownership: the caller allocates and owns all memory, including the
 *   workspace (size from crisp_workspace_size).  The library keeps no
 *   pointer after a call returns and never allocates device memory.
 * Streams: stream is a hipStream_t (NULL = the default stream).  Every call
 *   is asynchronous on it; results are valid once the stream has reached
 *   them.  Calls on different streams need distinct workspaces.  No call
 *   synchronises, allocates, copies through the host or records a memset,
 *   so a call (or a whole prefill) can be captured into a HIP graph and
 *   replayed; the workspace and the pointers are then fixed by the graph.
 * Errors: every call returns CRISP_OK (0) or a positive CRISP_ERR_* code.
 *   Arguments are validated on the host before anything is launched; on a
 *   validation error nothing is launched and no output is touched.
 *   CRISP_ERR_HIP reports a failed launch (hipGetLastError after a launch);
 *   outputs are then unspecified.  No call aborts or throws.
 */
#ifndef CRISP_H
#define CRISP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum crisp_status {
    CRISP_OK = 0,
    CRISP_ERR_INVALID_ARG = 1, /* NULL or misaligned pointer, bad option value   */
    CRISP_ERR_SHAPE = 2,       /* seq_len < 0, n_heads % n_kv_heads, heads <= 0   */
    CRISP_ERR_UNSUPPORTED = 3, /* head_dim / block_size / anchor windows != 128   */
    CRISP_ERR_WORKSPACE = 4,   /* workspace or CSR capacity too small             */
    CRISP_ERR_HIP = 5          /* a kernel launch failed                          */
};

/* Routers (crisp_opts.router). */
enum crisp_router {
    CRISP_ROUTER_CSTRUCT = 0,  /* structural proxy C_struct >= tau_proxy (Alg. 2, Eq. 2)  */
    CRISP_ROUTER_JSD = 1       /* FlexPrefill's D_JS >= tau_jsd (Alg. 5), the baseline     */
};

/* VS budget rules (crisp_opts.vs_rule); every rule clips to k_min. */
enum crisp_vs_rule {
    CRISP_VS_NOISE_MEAN = 0,   /* p_j > alpha * r / (N_b - 2) (Alg. 3, Eq. 3-4)           */
    CRISP_VS_NOISE_MEDIAN = 1, /* p_j > alpha * median(p_1 .. p_{N_b-2}) (Appendix H)      */
    CRISP_VS_GAMMA = 2         /* shortest prefix of sorted p with sum >= gamma_vs (Alg. 6) */
};

/*
 * Hyper-parameters (Section 5, "Setup"; Section 3.2; Appendices A and H).
 * NULL selects the defaults crisp_default_opts() writes:
 * {0.2, 0.95, 1024, 128, 128, CRISP_ROUTER_CSTRUCT, 0.1, CRISP_VS_NOISE_MEAN,
 * 0.95, 0}.
 *   tau_proxy     routing threshold: VS iff C_struct >= tau_proxy (Alg. 2)
 *   gamma         PE coverage target (Alg. 4), in (0, 1]
 *   k_min_tokens  minimum budget per VS direction, in tokens (a multiple of
 *                 block_size; clip(k, k_min, N_b) of Alg. 3)
 *   w_sink        anchor windows of C_struct (Eq. 2); must equal block_size,
 *   w_local       which makes them exactly the first and last key block
 *   router        enum crisp_router
 *   tau_jsd       threshold of CRISP_ROUTER_JSD (not given by the paper; 0.1)
 *   vs_rule       enum crisp_vs_rule
 *   gamma_vs      coverage target of CRISP_VS_GAMMA, in (0, 1]
 *   dense_below_tokens  context-length gate (Section 5.3, "Short contexts":
 *                 routing is a fixed cost that outweighs its savings on short
 *                 sequences): crisp_prefill and crisp_prefill_batch run dense
 *                 causal attention, skipping routing and selection, for a
 *                 sequence with seq_len < dense_below_tokens.  >= 0; 0 (the
 *                 default) never gates.
 * CRISP itself is router 0 with rule 0; router 1 with rule 2 is the
 * FlexPrefill baseline the paper compares against (Appendix A).
 */
typedef struct crisp_opts {
    float tau_proxy;
    float gamma;
    int k_min_tokens;
    int w_sink;
    int w_local;
    int router;
    float tau_jsd;
    int vs_rule;
    float gamma_vs;
    int dense_below_tokens;
} crisp_opts;

/* Writes the defaults listed above into *opts (host pointer, not NULL). */
void crisp_default_opts(crisp_opts *opts);

/* Static text for a status code. */
const char *crisp_status_string(int code);

/*
 * Worst-case sizes for one layer shape, so that no call needs a host sync.
 *   ws_bytes      workspace for crisp_prefill; it also suffices for every
 *                 other call of the same shape, and it never decreases as
 *                 seq_len grows (a workspace sized for the longest sequence
 *                 serves every shorter one with the same heads)
 *   csr_capacity  col_idx entries crisp_select may write:
 *                 n_heads * N_b * (N_b + 1) / 2
 * Host-only, pure.  Returns CRISP_ERR_SHAPE / _UNSUPPORTED like the others.
 */
int crisp_workspace_size(int seq_len, int n_heads, int n_kv_heads, int head_dim, int block_size,
                         size_t *ws_bytes, int64_t *csr_capacity);

/*
 * PatSearch (Alg. 2) for every query head.  The representative queries are
 * the last R = min(block_size, seq_len) rows; A^ = Softmax(Q^ K^T / sqrt(d))
 * with the causal mask.  Outputs (device):
 *   p_v, p_s   float [n_heads][N_b]  block-pooled column / diagonal means of
 *              A^ over its R rows (Alg. 3); each row sums to 1.
 *              Entry (i, k) lies on the diagonal at offset o = q_i - k from
 *              its query q_i; diagonal (slash) block j collects the offsets
 *              (N_b-1-j)*B .. (N_b-j)*B - 1, so block N_b-1 is the recency
 *              band and block 0 the farthest diagonals.
 *   c_struct   float [n_heads]  the routing statistic: the anchor mass of
 *              Eq. 2, the first and the last block (= p_v[0] + p_v[N_b-1];
 *              p_v[0] when N_b = 1), or D_JS (Alg. 5) under CRISP_ROUTER_JSD
 *   pattern    uint8 [n_heads]  1 = vertical-slash, 0 = pooled estimation
 * CRISP_ROUTER_JSD: D_JS = sqrt(KL(p_v||m)/2 + KL(abar||m)/2), m the mean of
 * the two, abar = Softmax over blocks of the mean representative query
 * against the per-block key means (natural logarithms).
 * A^ itself is never materialised.
 */
int crisp_route(const void *q, const void *k, int seq_len, int n_heads, int n_kv_heads,
                int head_dim, int block_size, const crisp_opts *opts, void *ws, size_t ws_bytes,
                uint8_t *pattern, float *c_struct, float *p_v, float *p_s, void *stream);

/*
 * Index selection (Alg. 3 for pattern 1, Alg. 4 for pattern 0) and block-list
 * expansion, reading crisp_route's outputs.
 *   sel_v, sel_s  int32 [n_heads][N_b]  ascending selected vertical / slash
 *                 blocks of VS heads (Eq. 3-4, clip to [k_min, N_b], top-k)
 *   sel_counts    int32 [n_heads][3]    (k_v, k_s, K*): list lengths of VS
 *                 heads, K* (pooled entries kept by gamma-cumsum) of PE heads
 *   row_ptr       int32 [n_heads][N_b+1] absolute offsets into col_idx; the
 *                 key blocks of (h, qb) are col_idx[row_ptr[h][qb] ..
 *                 row_ptr[h][qb+1]), ascending, unique, all <= qb, always
 *                 containing 0 and qb.  Head h's lists start at
 *                 h * N_b * (N_b + 1) / 2.
 *   col_idx       int32 [csr_capacity]
 * VS rows: {0, qb} u {v in S_v : v <= qb} u {qb - (N_b-1-j) : j in S_s, >= 0}.
 * PE rows: the kept (qb, kb) entries of the pooled map, plus {0, qb}.
 * alpha is the noise-floor multiplier of Eq. 4 (>= 0; 1.0 recommended);
 * opts->vs_rule picks the VS budget rule (alpha is unused by CRISP_VS_GAMMA).
 */
int crisp_select(const void *q, const void *k, const uint8_t *pattern, const float *p_v,
                 const float *p_s, int seq_len, int n_heads, int n_kv_heads, int head_dim,
                 int block_size, float alpha, const crisp_opts *opts, void *ws, size_t ws_bytes,
                 int32_t *sel_v, int32_t *sel_s, int32_t *sel_counts, int32_t *row_ptr,
                 int32_t *col_idx, int64_t csr_capacity, void *stream);

/*
 * Block-sparse causal attention on given lists, Eq. 1: for a query at
 * position t in block qb, softmax over the keys k <= t of the listed key
 * blocks of (h, qb), times V.  row_ptr / col_idx as written by crisp_select
 * (any absolute layout with unique lists; row_ptr must stay inside col_idx).
 * Listed blocks outside [0, qb] are ignored; a row with no valid block yields
 * zeros.  Accumulates in fp32, writes bf16 out (rows < seq_len only).
 * Uses the workspace for V re-laid out as transposed 64-key tiles (zero past
 * seq_len).
 */
int crisp_attend(const void *q, const void *k, const void *v, const int32_t *row_ptr,
                 const int32_t *col_idx, int seq_len, int n_heads, int n_kv_heads, int head_dim,
                 int block_size, void *ws, size_t ws_bytes, void *out, void *stream);

/* Dense causal attention with the same kernel (every block 0..qb listed). */
int crisp_attend_dense(const void *q, const void *k, const void *v, int seq_len, int n_heads,
                       int n_kv_heads, int head_dim, int block_size, void *ws, size_t ws_bytes,
                       void *out, void *stream);

/*
 * Alg. 1 end to end: crisp_route -> crisp_select -> crisp_attend, with
 * every intermediate kept in the workspace and no host synchronisation.
 * Below opts->dense_below_tokens it runs crisp_attend_dense instead.
 */
int crisp_prefill(const void *q, const void *k, const void *v, int seq_len, int n_heads,
                  int n_kv_heads, int head_dim, int block_size, float alpha,
                  const crisp_opts *opts, void *ws, size_t ws_bytes, void *out, void *stream);

/*
 * crisp_prefill without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The caller still passes q, k, v
 * and out (as for crisp_prefill); the workspace is a static device array of
 * CRISP_NOALLOC_SCRATCH_BYTES held by the library, one per device it runs
 * on, for the life of the process.  The call uses the array of the device
 * current on the calling thread (stream must belong to that device); its
 * address is looked up on the first call on each device, after which no
 * call allocates, frees or synchronises.
 * Limit: a layer whose crisp_workspace_size exceeds the array returns
 * CRISP_ERR_WORKSPACE before anything is launched.  The 64 MiB hold, e.g.,
 * 32 query / 8 KV heads up to 30848 tokens, or 4 / 1 heads up to 191488.
 * Every call on one device shares its array: the kernels clear what must
 * start at zero, so results do not depend on earlier calls, but calls that
 * overlap in time on one device (other streams, unordered threads) race.
 * CRISP_ERR_HIP if the array's address cannot be obtained.
 */
#define CRISP_NOALLOC_SCRATCH_BYTES (64u << 20)

int crisp_prefill_noalloc(const void *q, const void *k, const void *v, int seq_len, int n_heads,
                          int n_kv_heads, int head_dim, int block_size, float alpha,
                          const crisp_opts *opts, void *out, void *stream);

/* One sequence of a batch: device pointers to token 0 of head 0 of its q, k,
 * v and out, and its length (>= 0; 0 skips the sequence). */
typedef struct crisp_seq {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    int seq_len;
} crisp_seq;

/* Element strides of the four tensors: row (h, t) of q starts at
 * q + h * q_head + t * q_token, and likewise for k, v (KV heads) and out.
 * The head_dim values of a row stay contiguous.  Every stride is positive
 * and a multiple of 8 elements (16-byte aligned rows).  Examples, with H
 * query and H_kv KV heads, d = head_dim:
 *   [heads][tokens][d] per sequence:   q_head = seq_len * d, q_token = d
 *   [tokens][heads][d] (packed varlen
 *   or [batch][seq][heads][d]):         q_head = d, q_token = H * d
 *                                       (k, v: k_head = d, k_token = H_kv * d) */
typedef struct crisp_strides {
    int64_t q_head, q_token;
    int64_t k_head, k_token;
    int64_t v_head, v_token;
    int64_t out_head, out_token;
} crisp_strides;

/*
 * crisp_prefill over `batch` independent sequences of any lengths (variable-
 * length batches), each routed, selected and attended on its own as in
 * Alg. 1, on `stream`.
 *   seqs      host array [batch] (may be NULL when batch == 0)
 *   strides   host pointer; NULL means each sequence is contiguous
 *             [heads][seq_len][head_dim] as in crisp_prefill
 *   ws_bytes  at least crisp_workspace_size of the longest sequence: the
 *             sequences then run one after another, reusing the workspace
 *             (the stage events, when set, time the last sequence);
 *             at least crisp_workspace_size_batch of the batch: every
 *             sequence is routed and selected into a region of its own and
 *             the attention of the whole batch runs in one launch, one work
 *             queue over all sequences (the stage events then time the
 *             batch: routing of all, selection of all, V re-layout of all,
 *             the attention launch).
 * Either way each sequence's output is the same bits as crisp_prefill on it
 * alone.  All sequences are validated before the first launch; an error
 * leaves every output untouched.  Sequences with seq_len <
 * dense_below_tokens run dense attention.
 */
/*
 * Workspace for crisp_prefill_batch to attend a whole batch in one launch:
 * the routing / selection scratch of the longest sequence, plus per sequence
 * its intermediates and transposed V, plus a small table.  seq_lens: host
 * array [batch].  Host-only and pure; errors as crisp_workspace_size.
 */
int crisp_workspace_size_batch(const int *seq_lens, int batch, int n_heads, int n_kv_heads,
                               int head_dim, int block_size, size_t *ws_bytes);

int crisp_prefill_batch(const crisp_seq *seqs, int batch, const crisp_strides *strides,
                        int n_heads, int n_kv_heads, int head_dim, int block_size, float alpha,
                        const crisp_opts *opts, void *ws, size_t ws_bytes, void *stream);

/*
 * Stage timing for measurement: events is an array of `count` hipEvent_t
 * (cast to void*) owned by the caller, or NULL to stop.  While set (per
 * calling thread), each call records events[i] on its stream at the stage
 * boundaries it crosses: 0 = route start, 1 = select start, 2 = attend
 * start (before the V re-layout), 3 = attention kernel start, 4 = end.
 * crisp_route records 0 and 1, crisp_select 1 and 2, crisp_attend and
 * crisp_attend_dense 2, 3 and 4, crisp_prefill all five.  count must be 5.
 */
int crisp_set_stage_events(void *const *events, int count);

#ifdef __cplusplus
}
#endif

#endif /* CRISP_H */
