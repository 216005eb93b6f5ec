/*
 * spec_attn.h -- C ABI of libspecattn, the attention hot path of long-context
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * The operations, each a set of HIP kernels launched asynchronously on the
 * caller's stream:
 *
 *   spec_attn_draft_sparse  draft-phase attention over a sparse view of the KV
 *                           cache: attention sink + sliding window, or an
 *                           explicit budget list of positions.
 *   spec_attn_draft_ring    the window draft over a draft-KV ring buffer.
 *   spec_attn_verify_tree   verify-phase attention of N speculated tree nodes
 *                           over the full cache plus their own tree, with
 *                           padded ragged batches and remapped positions.
 *   spec_accept_greedy      greedy tree acceptance: an argmax per node, then
 *                           the longest accepted root path and the bonus token.
 *   spec_kv_commit          append the accepted path's K/V to the cache,
 *                           padding the batch to one uniform length.
 *   spec_kv_compact         drop a cache's padding slots (the valid slots
 *                           move to the front, in order).
 *   spec_block_means,       budget selection: block summaries of the keys,
 *   spec_select_blocks      then a budget list of sink, best-scoring blocks
 *                           and window for the draft's budget mode.
 *   spec_kv_gather,         partial verification: a contiguous partial cache
 *   spec_verify_mode        built from a budget list, and the full / partial
 *                           schedule.
 *
 * Conventions for every call
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps caller memory; buffers must stay alive
 *     until the stream work has completed.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Strides are in elements; the head dimension is always contiguous.
 *   - Every host-visible argument is checked before anything is launched; on
 *     an error nothing is launched and the call returns a negative status
 *     with a message available from spec_last_error() (thread-local).
 *   - Values that live only on the device (cache_len, budget indices,
 *     parents) are checked by the kernels.  A bad value sets a bit in the
 *     device error word kept in the workspace, and the affected outputs are
 *     written as NaN (attention) or -1 (token outputs).  spec_device_status()
 *     reports and clears that word.
 *   - Workspace: a caller-allocated device buffer of at least the size the
 *     matching spec_*_workspace_bytes() returns, zero-filled before its first
 *     use.  Every workspace has the same layout: a 256-byte header (the
 *     device error word), a 1 MiB counter region (arrival counters of the
 *     split merges and of acceptance), then the call's own scratch (split
 *     partials, scores).  Every call leaves the counters it used at zero
 *     and no call's scratch overlaps the counter region, so one workspace,
 *     zero-filled once, can be reused by any sequence of calls issued to the
 *     same stream, of any kind and shape, as long as it is as large as each
 *     call requires (the largest of their spec_*_workspace_bytes()).  Calls
 *     that overlap in time (different streams) need separate workspaces.
 *     Sizes depend only on the arguments, never on the device.
 *   - dtype SPEC_BF16 is the tuned path (bf16 inputs, fp32 accumulation, bf16
 *     outputs rounded to nearest-even); SPEC_F32 is a plain fp32 path.
 *   - head_dim must be 64 or 128.  Query head h reads KV head h / (Hq / Hkv).
 *   - Size limits of the bf16 path (SPEC_E_UNSUPPORTED beyond them): a
 *     draft budget of at most 524288 positions; a verify cache capacity plus
 *     N of at most 2^23 slots; at most 65536 query rows (tokens x query
 *     heads per KV head) per sequence and KV head.
 *
 * Sources (page title, then the passage):
 *   [WM] "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
 *        Context" (Pith review), "What carries the argument" and Eq. 1.
 *   [BD] "BudgetDraft: Acceptance-Aware Multi-View Training for Sparse-KV
 *        Speculative Decoding" (Pith review), abstract and Figure 2.
 *   [SM] "SpecMemo: Speculative Decoding is in Your Pocket" (Pith review),
 *        "What carries the argument" and Figure 9.
 *   [PV] "SpecPV: Improving Self-Speculative Decoding for Long-Context
 *        Generation via Partial Verification", section 3.2 "Partial
 *        Verification", section 3.3 "Rectified with Full Verification" and
 *        section 4.1 (its metrics and the setup of its experiments).
 */
#ifndef SPEC_ATTN_H
#define SPEC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 2

typedef int32_t spec_status;
enum {
  SPEC_OK = 0,
  SPEC_E_INVALID = -1,       /* bad argument: null pointer, shape, stride, alignment */
  SPEC_E_UNSUPPORTED = -2,   /* well-formed but outside what the library supports */
  SPEC_E_WORKSPACE = -3,     /* workspace missing or smaller than required */
  SPEC_E_HIP = -4,           /* the HIP runtime reported an error */
  SPEC_E_DEVICE_RANGE = -5   /* a kernel found an out-of-range device value */
};

/* Verification schedule (spec_verify_mode). */
enum { SPEC_VERIFY_FULL = 0, SPEC_VERIFY_PARTIAL = 1 };

/* Element types of q, K, V and out. */
enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

/* Bits of spec_dims.flags.
 * SPEC_FLAG_DETERMINISTIC: every split of an attention call sums a fixed
 * range of keys in a fixed order, so repeated calls with the same inputs,
 * shapes and workspace size give bitwise equal outputs.  Without it, long
 * single-sequence reads with few query rows (for instance a chain verify
 * over a million cached tokens) let wavefronts take chunks of keys from a
 * shared pool to balance the load across the chip; the sums are then the
 * same within rounding but their order, and so the last bit of an output,
 * can change from run to run.  Every other launch shape is deterministic
 * either way. */
enum { SPEC_FLAG_DETERMINISTIC = 1u };

/* Bits of the device error word (spec_device_status). */
enum {
  SPEC_DEV_CACHE_LEN = 1u,   /* cache_len[b] < 0, > capacity, < n_q_tokens (draft), or
                                > capacity - P (kv commit) */
  SPEC_DEV_INDEX = 2u,       /* a budget index outside [0, cache_len[b]) */
  SPEC_DEV_PARENT = 4u,      /* parents[i] not in [-1, i) */
  SPEC_DEV_DEPTH = 8u,       /* accepted path longer than max_depth */
  SPEC_DEV_COMMIT = 16u      /* kv commit: accept length outside [0, min(max_depth, N)]
                                or a path entry outside [0, N) */
};

typedef struct {
  int32_t batch;          /* B >= 0; with B = 0 a call launches nothing and
                             returns SPEC_OK (tensor pointers may be NULL) */
  int32_t n_q_heads;      /* Hq >= 1 */
  int32_t n_kv_heads;     /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t dtype;          /* SPEC_F32 or SPEC_BF16 */
  float softmax_scale;    /* finite, > 0; scores are softmax_scale * <q, k> */
  uint32_t flags;         /* SPEC_FLAG_* bits (0: the defaults); unknown bits are
                             SPEC_E_INVALID */
} spec_dims;

/* A K/V pair laid out as [B][Hkv][capacity][D] with arbitrary strides (in
 * elements) over the first three dimensions; D is contiguous.  K and V share
 * the strides.  bf16: pointers 16-byte aligned, strides multiples of 8;
 * fp32: pointers 16-byte aligned, strides multiples of 4. */
typedef struct {
  const void* k;
  const void* v;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;       /* >= D */
  int32_t capacity;       /* allocated slots per (b, h); cache_len[b] <= capacity */
} spec_kv;

/* The same layout for a K/V pair the library writes (spec_kv_commit). */
typedef struct {
  void* k;
  void* v;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;
  int32_t capacity;
} spec_kv_mut;

/*
 * Draft attention over a sparse view of the cache ([WM] "What carries the
 * argument"; [BD] abstract).
 *
 * q [B][Tq][Hq][D] contiguous; the Tq >= 1 queries are the last Tq positions
 * of each sequence, so query t sits at position e_t - 1 with
 * e_t = cache_len[b] - Tq + t + 1, and never sees a position >= e_t.
 *
 * Window mode (idx == NULL): query t attends to the union of the first
 * n_sink positions and the last `window` positions ending at itself, each
 * counted once: {j < min(n_sink, e_t)} U {max(0, e_t - window) <= j < e_t}.
 * n_sink >= 0, window >= 1.  RoPE is already applied to the cached keys.
 *
 * Budget mode (idx != NULL): query t attends to the listed positions
 * idx[b][h'][0..budget) that are < e_t, with h' = kv head (idx_stride_h > 0)
 * or 0 for every head (idx_stride_h == 0).  Duplicates count as often as
 * listed.  An entry of -1 is padding and selects nothing, so one list length
 * serves views of different sizes ([PV] section 3.3: a sequence shorter than
 * the budget uses its whole cache).  Any other value outside
 * [0, cache_len[b]) raises SPEC_DEV_INDEX and poisons that (b, kv head)'s
 * outputs with NaN.  A row that sees no
 * position gets out = 0 and lse = -inf.  idx is int32, 4-byte aligned.
 *
 * out [B][Tq][Hq][D] (dtype), lse [B][Tq][Hq] fp32 natural-log sum-exp of
 * the scaled scores (optional).  cache_len[b] < Tq raises SPEC_DEV_CACHE_LEN.
 */
spec_status spec_attn_draft_sparse(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                                   const spec_kv* cache, const int32_t* cache_len,
                                   int32_t n_sink, int32_t window,
                                   const int32_t* idx, int32_t budget,
                                   int64_t idx_stride_b, int64_t idx_stride_h,
                                   void* out, float* lse_or_null,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Window draft over a draft-KV ring buffer ([WM] "What carries the
 * argument": the draft KV working set is a constant window, so the draft KV
 * pool compacts into a ring; the referee's remarks on its appendix name the
 * slot mapping "ring base + logical position", wrapping, with a slack).
 *
 * The same attention as window mode of spec_attn_draft_sparse, but the
 * cache holds only the sink and a ring: position p < n_sink lives in slot
 * p, position p >= n_sink in slot n_sink + (p - n_sink) mod ring, and
 * cache_len[b] is the sequence's logical length (it may exceed the ring
 * cache's capacity).  The caller writes each new token's K/V at its slot,
 * overwriting the position `ring` earlier.  ring >= window + n_q_tokens - 1
 * (the chained queries reach back that far) and capacity >= n_sink + ring.
 * cache_len[b] < n_q_tokens raises SPEC_DEV_CACHE_LEN.  Workspace as
 * spec_draft_workspace_bytes(dims, n_q_tokens, n_sink + window + n_q_tokens
 * - 1).
 */
spec_status spec_attn_draft_ring(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                                 const spec_kv* ring_cache, const int32_t* cache_len,
                                 int32_t n_sink, int32_t window, int32_t ring, void* out,
                                 float* lse_or_null, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Tree-masked verify attention ([SM] "What carries the argument", Figure 9).
 *
 * q [B][N][Hq][D] contiguous, 1 <= N <= 64 speculated nodes.  parents int32,
 * [N] (parents_stride_b == 0, shared) or [B][N]: parents[i] = -1 for a child
 * of the anchor (the last committed token, already in the cache), otherwise
 * an earlier node (parents[i] < i); anything else raises SPEC_DEV_PARENT and
 * poisons that sequence's outputs.
 *
 * Node i of sequence b attends to every cache slot j < cache_len[b] whose
 * pad[b][j] is 0 (padding slots score -inf; pad == NULL means no padding),
 * then to the tree nodes on its root path, itself included.  Tree keys and
 * values come from `tree` ([B][Hkv][N][D] through its strides; it may alias
 * the cache slots just past cache_len).  pad is uint8 [B][pad_stride_b],
 * 4-byte aligned with pad_stride_b % 4 == 0 and >= capacity.
 *
 * Outputs: out [B][N][Hq][D] (dtype); lse [B][N][Hq] fp32 (optional);
 * pos_ids [B][N] int32 (optional) = number of non-padding slots in
 * [0, cache_len[b]) + depth(i), depth 0 for children of the anchor.
 */
spec_status spec_attn_verify_tree(const spec_dims* dims, const void* q, int32_t n_nodes,
                                  const spec_kv* cache, const int32_t* cache_len,
                                  const uint8_t* pad_or_null, int64_t pad_stride_b,
                                  const spec_kv* tree, const int32_t* parents,
                                  int64_t parents_stride_b,
                                  void* out, float* lse_or_null, int32_t* pos_ids_or_null,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the tree
 * verify of spec_attn_verify_tree, same arguments, same kernels and the
 * same results, but without a workspace argument.  Its scratch (the
 * workspace layout: error word, counters, split partials) is a static
 * device array of 64 MiB in the library, one copy per GPU, held from the
 * first call on that GPU until the process ends.  A shape whose workspace
 * (spec_verify_workspace_bytes) exceeds 64 MiB returns SPEC_E_UNSUPPORTED
 * before anything is launched.  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine, on the first call or later.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, or two threads) race and must not be issued.
 * The stream must belong to the current device.  Device range errors poison
 * the outputs as in spec_attn_verify_tree; the static error word is not
 * reported (spec_device_status needs a caller workspace).
 */
spec_status spec_attn_verify_tree_noalloc(const spec_dims* dims, const void* q, int32_t n_nodes,
                                          const spec_kv* cache, const int32_t* cache_len,
                                          const uint8_t* pad_or_null, int64_t pad_stride_b,
                                          const spec_kv* tree, const int32_t* parents,
                                          int64_t parents_stride_b, void* out,
                                          float* lse_or_null, int32_t* pos_ids_or_null,
                                          void* stream);

/*
 * Greedy tree acceptance ([BD] Figure 2; [WM] losslessness; [PV] 4.1).
 *
 * logits fp32 [B][N+1][V] contiguous, 16-byte aligned: row 0 is the
 * verifier's output at the anchor, row i+1 its output at node i.  The greedy
 * target of a row is its argmax (ties: smallest index; NaN counts as the
 * maximum, first NaN wins).  Node i is accepted iff its parent is accepted
 * (the anchor always is) and draft_tokens[b][i] equals the parent's target.
 * The result is the deepest accepted node (ties: smallest index):
 *   accept_len[b]  = its depth + 1, or 0 when no node is accepted;
 *   accept_path[b] = node ids root-first, -1 padded to max_depth;
 *   bonus[b]       = the target of the last accepted row (row 0 if none).
 * A path longer than max_depth raises SPEC_DEV_DEPTH (the first max_depth
 * entries are written).  1 <= N <= 64; parents as in spec_attn_verify_tree.
 * batch >= 0; with batch = 0 nothing is launched (pointers may be NULL).
 */
spec_status spec_accept_greedy(int32_t batch, int32_t n_nodes, int32_t vocab,
                               const float* logits, const int32_t* draft_tokens,
                               const int32_t* parents, int64_t parents_stride_b,
                               int32_t max_depth,
                               int32_t* accept_len, int32_t* accept_path, int32_t* bonus,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * KV commit of the accepted path ([SM] "What carries the argument", Figure 9;
 * [PV] section 3.3), the step after spec_accept_greedy.
 *
 * For every sequence b with a valid acceptance result (0 <= accept_len[b]
 * <= min(max_depth, N) and accept_path[b][j] in [0, N) for j < accept_len[b]),
 * the K and V rows of the accepted nodes accept_path[b][0..tau) are copied,
 * in path order, from `tree` ([B][Hkv][N][D]) into the cache slots
 * [cache_len[b], cache_len[b] + tau).  Slot cache_len[b] + tau is the bonus
 * token's: it is marked valid and no K/V is written there (the caller's next
 * forward pass computes it; that token is the next anchor).  The whole batch
 * appends the same P = 1 + max_b tau_b slots (invalid sequences count 0):
 * pad[b][cache_len[b] + j] = 0 for j <= tau, 1 for tau < j < P, and
 * cache_len[b] grows by P.  *n_appended_or_null receives P.
 *
 * A sequence with an invalid acceptance result raises SPEC_DEV_COMMIT,
 * commits nothing and appends P padding slots.  A sequence whose
 * cache_len[b] is outside [0, capacity - P] raises SPEC_DEV_CACHE_LEN and is
 * left untouched (no slot written, cache_len unchanged).
 *
 * The tree rows of a (sequence, KV head) may alias that pair's cache slots at
 * or after cache_len[b] (node n at slot cache_len[b] + n + c, c >= 0, as when
 * verify wrote the tree K/V into the cache): the copy never overwrites a row
 * it has still to read.  Apart from that, the cache, the tree, pad and the
 * integer arrays must not overlap.
 *
 * dtype SPEC_F32 or SPEC_BF16 (element size only: the commit copies bytes);
 * head_dim 64 or 128; cache and tree follow the spec_kv layout rules.
 * cache_len int32 [B] (read and written), pad uint8 [B][pad_stride_b] with
 * pad_stride_b >= capacity, accept_len int32 [B], accept_path int32
 * [B][max_depth] (as written by spec_accept_greedy), 1 <= N <= 64,
 * max_depth >= 1.  batch = 0 launches nothing (pointers may be NULL).
 * Workspace: spec_commit_workspace_bytes() bytes (the device error word).
 */
spec_status spec_kv_commit(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                           const spec_kv_mut* cache, int32_t* cache_len,
                           uint8_t* pad, int64_t pad_stride_b,
                           const spec_kv* tree, int32_t n_nodes,
                           const int32_t* accept_len, const int32_t* accept_path,
                           int32_t max_depth, int32_t* n_appended_or_null,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Compaction of a cache's padding slots ([SM] Figure 9: batched commits pad
 * every sequence to one length per step; [PV] section 3.3: tokens that were
 * not accepted leave the cache once verification is done).  The maintenance
 * step that removes the pads spec_kv_commit leaves behind.
 *
 * For every sequence b with 0 <= cache_len[b] <= capacity: the slots
 * j < cache_len[b] whose pad byte is 0 keep their order and their K and V
 * rows (every KV head) move to slots 0, 1, ..., n_b - 1; cache_len[b]
 * becomes n_b; pad[b][j] becomes 0 for every j below the old cache_len.  The
 * contents of the slots from n_b to the old cache_len are unspecified
 * afterwards; slots and pad bytes at or past the old cache_len are not
 * touched.  Attention over the compacted cache needs no mask, and the
 * position of every token (spec_attn_verify_tree's pos_ids) is unchanged.
 * A sequence with cache_len[b] outside [0, capacity] raises
 * SPEC_DEV_CACHE_LEN and is left untouched.
 *
 * In place.  The time grows with the slots after a sequence's first pad
 * (those rows move): pads near the end, as per-step commits leave them,
 * keep it short.  Finding the first pad reads the pad bytes below cache_len
 * once, in 64 slices per sequence.
 *
 * dtype SPEC_F32 or SPEC_BF16 (element size only: rows are copied);
 * head_dim 64 or 128; the cache follows the spec_kv layout rules; cache_len
 * int32 [B] (read and written); pad uint8 [B][pad_stride_b] (read and
 * written), 4-byte aligned with pad_stride_b % 4 == 0 and >= capacity.
 * batch = 0 launches nothing (pointers may be NULL).  Workspace:
 * spec_compact_workspace_bytes(batch) bytes (the device error word and 128
 * int32 per sequence).
 */
spec_status spec_kv_compact(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                            const spec_kv_mut* cache, int32_t* cache_len,
                            uint8_t* pad, int64_t pad_stride_b,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block summaries for budget selection ([PV] section 3.2: the partial cache
 * is chosen at the block level of the cache manager; section 4.1: mean
 * reduction for the retrieval).
 *
 * Block c holds the positions [c * block, (c + 1) * block).  For every
 * c in [first_block, first_block + n_blocks), means[b][h][c][0..D) (fp32,
 * contiguous [B][Hkv][max_blocks][D], 16-byte aligned) receives the mean of
 * the keys cache.k[b][h][j] over the positions j of the block below
 * cache_len[b] whose pad byte is 0 (pad == NULL: no padding), accumulated in
 * fp32; a block with no such position gets NaN.  Other blocks are not
 * touched, so a caller can keep a table and refresh only the blocks an
 * append changed.  cache.v is not read.  cache_len[b] outside
 * [0, capacity] raises SPEC_DEV_CACHE_LEN and that sequence's blocks get
 * NaN.  block >= 1; batch and Hkv at most 65535.
 * Workspace: at least spec_select_workspace_bytes(dims, 0) bytes (the device
 * error word).
 */
spec_status spec_block_means(const spec_dims* dims, const spec_kv* cache, const int32_t* cache_len,
                             const uint8_t* pad_or_null, int64_t pad_stride_b, int32_t block,
                             int32_t first_block, int32_t n_blocks, float* means,
                             int32_t max_blocks, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Budget list by block-mean scoring ([PV] sections 3.2 and 4.1; [BD]
 * abstract: a sparse KV view under a fixed budget).
 *
 * For each (sequence b, KV head h), with L = cache_len[b]:
 *   - the sink [0, min(n_sink, L)) and the window [max(n_sink, L - window), L)
 *     are always listed;
 *   - the candidate blocks are those meeting the middle [n_sink, L - window);
 *     block c scores (mean of the h's G query heads x n_q_tokens queries of
 *     q) . means[b][h][c] in fp32 (a block with a NaN mean has no score);
 *   - the n_select best scores are chosen, ties to the smaller block index
 *     (all blocks with a score if fewer have one), and each chosen block
 *     contributes its positions inside the middle;
 *   - idx[b][h][0..budget) receives the listed positions whose pad byte is 0,
 *     in increasing order, then -1 entries up to the budget: the list is the
 *     budget-mode input of spec_attn_draft_sparse (idx_stride_h = budget).
 * With shared != 0 there is one list per sequence, idx[b][0][0..budget): a
 * block's score is the mean of its Hkv heads' scores, as a partial cache
 * keeps whole cache-manager blocks (spec_kv_gather takes such lists).
 * scores_or_null[b][h or 0][0..max_blocks) receives the block scores, NaN
 * for blocks that are not candidates or have no score.  q is [B][Tq][Hq][D]
 * (dims->dtype), means as written by spec_block_means for every block below
 * capacity (max_blocks * block >= capacity; max_blocks <= 8192).
 * Requirements: budget >= n_sink + window + n_select * block, n_select <=
 * 2048.  cache_len[b] outside [0, capacity] raises SPEC_DEV_CACHE_LEN and
 * writes an all -1 list.  Workspace: spec_select_workspace_bytes(dims,
 * max_blocks) bytes (the error word and the block scores).
 */
spec_status spec_select_blocks(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                               const float* means, int32_t max_blocks, int32_t block,
                               const int32_t* cache_len, int32_t capacity,
                               const uint8_t* pad_or_null, int64_t pad_stride_b, int32_t n_sink,
                               int32_t window, int32_t n_select, int32_t shared, int32_t* idx,
                               int32_t budget, float* scores_or_null, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Partial KV cache for partial verification ([PV] section 3.2: a sink,
 * retrieved blocks, a local window and a buffer, contiguous in token order
 * and handled as one KV segment; section 3.3: a full verification refreshes
 * it).
 *
 * idx holds one budget list per sequence, idx[b * idx_stride_b + j] for j <
 * budget (e.g. spec_select_blocks with shared != 0).  Slot j of every KV head
 * of `partial` receives the K and V rows of position idx[b][j]; a -1 entry
 * gives a padding slot (zero K/V, partial_pad[b][j] = 1), a listed position
 * gives partial_pad[b][j] = 0, and partial_len[b] = budget.  Slots at or past
 * the budget are not touched: the buffer of later tokens goes there through
 * spec_kv_commit on the partial cache.  Partial verification is then
 * spec_attn_verify_tree over (partial, partial_len, partial_pad); the
 * pos_ids it returns count the partial cache's valid slots, so a caller that
 * needs the full sequence's positions takes them from its last full
 * verification plus the tokens committed since.
 *
 * A listed value outside [0, cache_len[b]) other than -1 raises
 * SPEC_DEV_INDEX and gives a padding slot; cache_len[b] outside
 * [0, capacity] raises SPEC_DEV_CACHE_LEN and pads every slot.  partial
 * follows the spec_kv layout rules with capacity >= budget; partial_pad is
 * uint8 [B][partial_pad_stride_b], stride >= partial capacity.  batch at
 * most 65535.  Workspace: spec_select_workspace_bytes(dims, 0) bytes.
 */
spec_status spec_kv_gather(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                           const spec_kv* cache, const int32_t* cache_len, const int32_t* idx,
                           int32_t budget, int64_t idx_stride_b, const spec_kv_mut* partial,
                           int32_t* partial_len, uint8_t* partial_pad,
                           int64_t partial_pad_stride_b, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Full or partial verification for the next step ([PV] section 3.3), a host
 * computation: SPEC_VERIFY_FULL while the sequence (seq_len tokens) is
 * shorter than the partial budget, or when the partially verified tokens
 * kept in the buffer plus the n_nodes new candidates exceed
 * buffer_capacity; SPEC_VERIFY_PARTIAL otherwise.  A full verification
 * refreshes the partial cache and empties the buffer.  Negative arguments,
 * budget < 1 or n_nodes < 1 return SPEC_E_INVALID.
 */
int32_t spec_verify_mode(int64_t seq_len, int32_t budget, int32_t buffered, int32_t n_nodes,
                         int32_t buffer_capacity);

/* Workspace sizes in bytes (0 on invalid arguments; see spec_last_error).
 * max_view_len for the draft: min(capacity, n_sink + window + n_q_tokens - 1)
 * in window mode, the budget in budget mode (a larger value is always safe).
 * capacity for verify: the cache capacity passed to the call. */
size_t spec_draft_workspace_bytes(const spec_dims* dims, int32_t n_q_tokens,
                                  int32_t max_view_len);
size_t spec_verify_workspace_bytes(const spec_dims* dims, int32_t n_nodes,
                                   int32_t capacity);
size_t spec_accept_workspace_bytes(int32_t batch, int32_t n_nodes, int32_t vocab);
size_t spec_commit_workspace_bytes(void);
size_t spec_compact_workspace_bytes(int32_t batch);
size_t spec_select_workspace_bytes(const spec_dims* dims, int32_t max_blocks);

/* Waits for `stream`, reads and clears the device error word of `workspace`.
 * Returns SPEC_OK, SPEC_E_DEVICE_RANGE (bits in *bits_or_null) or
 * SPEC_E_HIP. */
spec_status spec_device_status(void* workspace, void* stream, uint32_t* bits_or_null);

const char* spec_status_string(spec_status s);
const char* spec_last_error(void);
int32_t spec_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_ATTN_H */
