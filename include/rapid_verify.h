/*
 * rapid_verify -- the target model's speculative verification step for
 * long-context decoding, for AMD Instinct MI355X (gfx950).
 *
 * The step has two halves.
 *
 * 1. Attention of the verify queries (the last committed token plus the draft
 *    tokens, or the nodes of a draft tree) over the long history KV cache and
 *    over the draft block itself.  Following the hybrid tree attention of the
 *    LongSpec summary (gist.science, "LongSpec", section 2.3 "Fast Tree
 *    Attention"), it is computed in two parts and merged:
 *      spec_attn_prefix  -- unmasked attention over the history cache, split
 *                           along the sequence into partial results (O, LSE)
 *                           (spec_attn_prefix_ev also records timing events
 *                           on its kernel);
 *      spec_attn_block   -- attention among the draft rows under the causal
 *                           or tree mask;
 *      lse_merge         -- log-sum-exp merge of all partials;
 *      spec_attn_block_merge -- the last two in one launch (spec_attn_block_merge_ev
 *                           also records timing events on its kernel);
 *      spec_attn_verify  -- all three in one launch where the device holds
 *                           the history pass at once.
 *    The LongSpec drafter's own attention (same summary, sections 2.1-2.2)
 *    uses spec_attn_prefix at n = 1 with lse_merge and no block for its
 *    cross-attention over the target's cache, and
 *      spec_attn_window  -- sliding-window self-attention with anchor tokens
 *                           over the drafter's constant-size ring cache.
 *
 * 2. RAPID's acceptance over the vocabulary (RAPID blog post,
 *    leeon-k.github.io, sections 2.1, 2.3, 2.4; abeam.tech RAPID article,
 *    "Key idea 1"):
 *      rapid_accept      -- p = softmax(z/T), q = softmax(y/T),
 *                           p_hat = softmax(z/T + eta*(q - p)); draft t is
 *                           kept while r_t <= min(1, p_hat_t[x_t]/q_t[x_t]);
 *                           at the first rejection a token is drawn from
 *                           norm(max(p_hat - q, 0)) by inverse CDF with the
 *                           caller's uniform; if every draft is kept, a bonus
 *                           token is drawn from the last row's p;
 *      rapid_accept_ex   -- the same with section 2.4's tail-preserving rule
 *                           and/or its printed residual as options;
 *      rapid_tree_accept -- the same over a draft tree, with a rule among
 *                           sibling candidates taken from outside the pages.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are caller-owned DEVICE pointers (except
 *   parent_host, which is host memory), dense row-major in the stated
 *   shapes.  bf16 data are IEEE bfloat16 bit patterns.  Pointers to bf16 and
 *   fp32 tensors must be 16-byte aligned.
 * - The library allocates nothing, frees nothing, keeps no state between
 *   calls and never synchronises.  Work is enqueued asynchronously on
 *   `stream` (a hipStream_t; NULL is the null stream).  Calls on different
 *   streams may run concurrently if their outputs do not overlap.
 * - Every scalar and pointer argument is validated on the host before any
 *   HIP call.  On a failed check the call returns a nonzero rv_status and
 *   writes nothing.  A failed kernel launch returns RV_ERR_HIP (the HIP error
 *   is cleared).  No C++ exception crosses this interface.
 * - Device data are the caller's responsibility: spec_attn_prefix reads
 *   min(max(seq_lens[b], 0), L_max, num_splits * split_len) history tokens of
 *   sequence b (the partials hold num_splits splits, so a device length
 *   above the host's max_seq_len is cut at num_splits * split_len, never
 *   read past); a draft id outside [0, V) makes rapid_accept report
 *   n_accept = -1 for that sequence; non-finite logits give unspecified
 *   tokens but never an out-of-bounds access.
 * - Results are bit-deterministic: every reduction has a fixed order; the
 *   atomics (the acceptance passes' per-sequence arrival counters,
 *   spec_attn_verify's split masks) only decide which workgroup performs a
 *   step, not what it computes.
 * - Workspaces (rapid_accept, rapid_tree_accept, spec_attn_window) are
 *   caller-owned device scratch; they need no initial contents and hold
 *   nothing between calls.  spec_attn_verify's sync words are the exception:
 *   zero before the first call, zero after every call.
 *   A workspace counts as an output: calls that may run at the same time
 *   (different streams) each need their own; calls on one stream may share
 *   one.
 *
 * - Sizes beyond the launch grid's reach (B or Hq above 65535, a window or
 *   sink above 2^24) return RV_ERR_UNSUPPORTED.
 *
 * Notation: B batch, Hq query heads, Hkv kv heads (Hq % Hkv == 0, query head
 * h reads kv head h / (Hq/Hkv)), n block rows (gamma+1 for a chain, the node
 * count for a tree), d head dim, L_max cache capacity per sequence, S number
 * of history splits, gamma draft tokens, V vocabulary size.
 */
#ifndef RAPID_VERIFY_H
#define RAPID_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RV_OK = 0,
  RV_ERR_NULL = 1,        /* a required pointer is NULL                       */
  RV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent           */
  RV_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. d not 64 or 128) */
  RV_ERR_VALUE = 4,       /* a scalar is out of range (T <= 0, NaN eta, tree) */
  RV_ERR_WORKSPACE = 5,   /* workspace too small                              */
  RV_ERR_HIP = 6,         /* a HIP launch failed                              */
  RV_ERR_ALIGNMENT = 7    /* a tensor pointer is not 16-byte aligned          */
} rv_status;

/* Static, human-readable name of a status code (never NULL). */
const char* rv_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int rv_version(void);

/* Largest supported block size n, and largest (Hq/Hkv)*n rows per kv head. */
#define RV_MAX_BLOCK_ROWS 64
#define RV_MAX_GROUP_ROWS 256

/*
 * Choose the history split for spec_attn_prefix on this device class:
 * writes *split_len (tokens per split, a multiple of 128) and *num_splits
 * (S = ceil(max_seq_len / split_len), at least 1) so that the launch fills the
 * MI355X's 256 compute units, with splits of at least 512 tokens.  Pure host
 * arithmetic, no HIP call.
 */
rv_status rv_prefix_default_split(int64_t max_seq_len, int B, int Hq, int Hkv, int n,
                                  int d, int64_t* split_len, int* num_splits);

/*
 * The same choice from the batch's own lengths, for callers that know them
 * on the host (a serving loop does: it manages the cache).  seq_lens_host is
 * HOST int32 [B], each >= 0 (else RV_ERR_VALUE); num_cus is the device's
 * compute-unit count.  Writes the shortest split_len (a multiple of 128, at
 * least 512) for which the splits that hold keys, Hkv * sum_b
 * ceil(L_b / split_len), all fit on the compute units at once, and
 * S = ceil(max_b L_b / split_len); when even one split per sequence does not
 * fit, one split per sequence.  A ragged batch then keeps every compute unit
 * busy, where a split chosen from the longest sequence alone leaves the units
 * of the short sequences' empty splits idle.  Pure host arithmetic.
 */
rv_status rv_prefix_balanced_split(const int32_t* seq_lens_host, int B, int Hq, int Hkv, int n,
                                   int d, int num_cus, int64_t* split_len, int* num_splits);

/*
 * spec_attn_prefix -- unmasked attention of every block row over the history
 * cache, one normalised partial result per split (LongSpec summary, section
 * 2.3: the history part needs no mask; the partials are merged by
 * log-sum-exp).
 *
 *   q         bf16 [B, Hq, n, d]       block-row queries
 *   k_cache   bf16 [B, Hkv, L_max, d]  history keys
 *   v_cache   bf16 [B, Hkv, L_max, d]  history values
 *   seq_lens  int32 [B] (device)       history length of each sequence
 *   max_seq_len  host bound >= every seq_lens[b]; sizes the grid
 *   sm_scale  score scale, finite and > 0: s_j = sm_scale * <q, k_j>
 *   split_len tokens per split (a positive multiple of 128)
 *   num_splits S >= ceil(max_seq_len / split_len): capacity of the partials
 *   o_part    fp32 [B, Hq, n, S, d]  out: sum_j softmax_split(s)_j v_j
 *   lse_part  fp32 [B, Hq, n, S]     out: natural-log sum_j exp(s_j) over the
 *                                    split; -inf (and o_part = 0) for a split
 *                                    that holds no history token
 * Split s of sequence b covers tokens [s*split_len, min((s+1)*split_len,
 * L_b)), L_b = min(max(seq_lens[b], 0), L_max): the call attends over the
 * first min(L_b, S*split_len) tokens.  Supports d in {64, 128}, n <= 64,
 * (Hq/Hkv)*n <= 256.
 */
rv_status spec_attn_prefix(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq,
                           int Hkv, int n, int d, int64_t L_max, float sm_scale,
                           int64_t split_len, int num_splits, float* o_part, float* lse_part,
                           void* stream);

/*
 * spec_attn_prefix_ev -- spec_attn_prefix that also records two HIP events
 * on the history kernel's own dispatch, for callers that time it:
 * start_event and stop_event are hipEvent_t created by the caller (either may
 * be NULL) and take the kernel's start and end timestamps, so
 * hipEventElapsedTime(start, stop) is the kernel's duration, without the
 * marker packets a record before and after the call would add.  Everything
 * else as spec_attn_prefix.
 */
rv_status spec_attn_prefix_ev(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq,
                              int Hkv, int n, int d, int64_t L_max, float sm_scale,
                              int64_t split_len, int num_splits, float* o_part, float* lse_part,
                              void* stream, void* start_event, void* stop_event);

/*
 * spec_attn_block -- attention of the block rows over the block's own keys
 * under the speculative mask (LongSpec summary, section 2.3: only the few
 * speculative tokens need a mask).
 *
 *   q            bf16 [B, Hq, n, d]
 *   k_blk, v_blk bf16 [B, Hkv, n, d]   keys/values of the block rows
 *   parent_host  HOST int32 [n] or NULL.  NULL: causal chain, row i sees
 *                block rows j <= i.  Otherwise a tree shared by the batch:
 *                parent_host[0] == -1 and 0 <= parent_host[i] < i; row i sees
 *                itself and its ancestors.  Invalid trees -> RV_ERR_VALUE.
 *   sm_scale     score scale, finite and > 0
 *   o_blk        fp32 [B, Hq, n, d]   out: normalised over the visible rows
 *   lse_blk      fp32 [B, Hq, n]      out: natural-log sum exp of the scores
 * Supports d in {64, 128}, 1 <= n <= 64.
 */
rv_status spec_attn_block(const void* q, const void* k_blk, const void* v_blk,
                          const int32_t* parent_host, int B, int Hq, int Hkv, int n, int d,
                          float sm_scale, float* o_blk, float* lse_blk, void* stream);

/*
 * lse_merge -- log-sum-exp merge of the S history partials and the block
 * partial (LongSpec summary, section 2.3: the two parts' outputs are combined
 * with the log-sum-exp trick).  With M = max_k LSE_k and a_k = exp(LSE_k-M):
 *   out = sum_k a_k O_k / sum_k a_k,   lse_out = M + log sum_k a_k.
 * Partials with LSE = -inf have weight 0.
 *
 *   o_part, lse_part  fp32 [B, Hq, n, S, d], [B, Hq, n, S]
 *   o_blk, lse_blk    fp32 [B, Hq, n, d],    [B, Hq, n], or both NULL to
 *                     merge the history partials alone (e.g. a drafter's
 *                     cross-attention over the target's cache, LongSpec
 *                     summary section 2.1); one NULL without the other is
 *                     RV_ERR_NULL
 *   out               bf16 [B, Hq, n, d]  (round to nearest even)
 *   lse_out           fp32 [B, Hq, n] or NULL
 * A row with no visible key at all gets out = 0 and lse_out = -inf.
 */
rv_status lse_merge(const float* o_part, const float* lse_part, int S, const float* o_blk,
                    const float* lse_blk, int B, int Hq, int n, int d, void* out,
                    float* lse_out, void* stream);

/*
 * spec_attn_block_merge -- spec_attn_block and lse_merge in one pass (the
 * same LongSpec section 2.3 split: masked block part, log-sum-exp merge with
 * the history partials), for callers that need only the merged result: the
 * block partial is computed where it is merged and never stored.
 *
 *   q, k_blk, v_blk, parent_host, sm_scale  as spec_attn_block
 *   o_part, lse_part, S                     as lse_merge (from spec_attn_prefix)
 *   out        bf16 [B, Hq, n, d]  (round to nearest even)
 *   lse_out    fp32 [B, Hq, n] or NULL
 * Same results as the two calls up to fp32 rounding order.  Supports d in
 * {64, 128}, 1 <= n <= 64.
 */
rv_status spec_attn_block_merge(const void* q, const void* k_blk, const void* v_blk,
                                const int32_t* parent_host, const float* o_part,
                                const float* lse_part, int S, int B, int Hq, int Hkv, int n,
                                int d, float sm_scale, void* out, float* lse_out, void* stream);

/*
 * spec_attn_block_merge_ev -- spec_attn_block_merge that also records two
 * caller-created HIP events (either may be NULL) on its kernel's own
 * dispatch, as spec_attn_prefix_ev does for the history kernel.
 */
rv_status spec_attn_block_merge_ev(const void* q, const void* k_blk, const void* v_blk,
                                   const int32_t* parent_host, const float* o_part,
                                   const float* lse_part, int S, int B, int Hq, int Hkv, int n,
                                   int d, float sm_scale, void* out, float* lse_out,
                                   void* stream, void* start_event, void* stop_event);

/*
 * spec_attn_verify -- the whole verify attention (spec_attn_prefix, then
 * spec_attn_block_merge) in one call (LongSpec summary, section 2.3: an
 * unmasked pass over the history, a masked pass over the draft block, their
 * outputs combined by log-sum-exp).  On small grids it is one launch: each
 * workgroup of the history pass, once the other splits of its (sequence,
 * kv head) are done, merges a share of that group's rows, so the merge needs
 * no launch of its own.  Otherwise it is the two launches.
 *
 *   q, k_cache, v_cache, seq_lens, max_seq_len, L_max, sm_scale, split_len,
 *   num_splits, o_part, lse_part   as spec_attn_prefix (o_part and lse_part
 *                                  are still written, then read back)
 *   k_blk, v_blk, parent_host      as spec_attn_block
 *   out, lse_out                   as spec_attn_block_merge
 *   sync        device scratch of spec_attn_verify_sync_size(B, Hkv) bytes
 *               (sync_bytes smaller: RV_ERR_WORKSPACE), 16-byte aligned,
 *               ZERO-FILLED by the caller before its first use; every call
 *               leaves it zero again (the two-launch form does not touch
 *               it).  Unlike the other workspaces it must not be shared by
 *               calls that may run at the same time (different streams).
 *   help_after_us  microseconds a workgroup whose split is done waits for
 *               the rest before it computes a missing split itself (negative:
 *               200; 0 makes every waiting workgroup help at once; at most
 *               10^7, else RV_ERR_VALUE).  Results do not depend on it.
 *   start_event, stop_event  hipEvent_t created by the caller, or NULL:
 *               recorded on the first and last kernel's own dispatch.
 * The single launch is taken when rv_verify_single_launch(B, Hq, Hkv, n, d,
 * num_splits, number of compute units of the current device) is 1; otherwise
 * the call runs the two launches of spec_attn_prefix and
 * spec_attn_block_merge.  Either way out and lse_out equal those of the two
 * calls up to fp32 rounding order (the single launch sums each row's
 * partials in one ascending chain).
 */
size_t spec_attn_verify_sync_size(int B, int Hkv);

/*
 * 1 when spec_attn_verify runs as a single launch: the history pass takes the
 * per-wave kernel (M = (Hq/Hkv)*n <= 64 rows per kv head, and <= 48 at
 * d = 128), num_splits <= 64, ceil(M / num_splits) <= 4 (one merged row per
 * wave), and its B*Hkv*num_splits workgroups number at most 64 and at most
 * num_cus; else 0 (also for invalid sizes).  Small grids are where the one
 * launch pays: on larger ones the exchange between workgroups on different
 * XCDs costs more than the second launch.  Pure host arithmetic.
 */
int rv_verify_single_launch(int B, int Hq, int Hkv, int n, int d, int num_splits, int num_cus);

rv_status spec_attn_verify(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq, int Hkv,
                           int n, int d, int64_t L_max, float sm_scale, int64_t split_len,
                           int num_splits, const void* k_blk, const void* v_blk,
                           const int32_t* parent_host, float* o_part, float* lse_part,
                           void* sync, size_t sync_bytes, void* out, float* lse_out,
                           int help_after_us, void* stream, void* start_event,
                           void* stop_event);

/*
 * spec_attn_window -- the drafter's sliding-window self-attention with
 * attention-sink anchors over its constant-size ring cache (LongSpec
 * summary, section 2.1: the drafter's self-attention sees only the latest
 * `window` tokens, so its own cache does not grow with the context; section
 * 2.2: the first tokens are kept as anchors).
 *
 *   q        bf16 [B, Hq, n, d]   row i of sequence b is the token at
 *                                 position pos[b] + i
 *   k_ring, v_ring bf16 [B, Hkv, cap, d]  the drafter's cache: position p
 *                                 is in slot p if p < sink, else in slot
 *                                 sink + (p - sink) mod (cap - sink); the
 *                                 caller has written every position up to
 *                                 pos[b] + n - 1
 *   pos      device int32 [B]     clamped on the device to [0, 2^30]
 *   cap, sink, window             1 <= window, 0 <= sink,
 *                                 cap - sink >= window + n - 1 (so every
 *                                 visible position is still resident), else
 *                                 RV_ERR_SHAPE
 *   sm_scale finite and > 0
 *   out      bf16 [B, Hq, n, d]   (round to nearest even)
 *   lse_out  fp32 [B, Hq, n] or NULL  natural-log sum exp of the scores
 *   workspace device scratch of spec_attn_window_workspace_size bytes
 *            (16-byte aligned; no initial contents needed)
 * The row at position P sees positions p <= P with p < sink or
 * p > P - window (the window includes the row itself).  Query head h reads
 * kv head h / (Hq / Hkv).  Two launches on `stream`: per-segment partials,
 * then their log-sum-exp merge.  Supports d in {64, 128}, 1 <= n <= 64,
 * B * n <= 65535.
 */
size_t spec_attn_window_workspace_size(int B, int Hq, int n, int d, int sink, int window);
rv_status spec_attn_window(const void* q, const void* k_ring, const void* v_ring,
                           const int32_t* pos, int B, int Hq, int Hkv, int n, int d, int cap,
                           int sink, int window, float sm_scale, void* out, float* lse_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace rapid_accept needs for (B, gamma, V). */
size_t rapid_accept_workspace_size(int B, int gamma, int V);

/*
 * rapid_accept -- RAPID's acceptance for B sequences (RAPID blog post,
 * section 2.1 acceptance test and residual draw; section 2.3 acceptance
 * against the full-context target; section 2.4 retrieval-augmented target
 * p_hat used in place of p at inference).
 *
 *   z          fp32 [B, gamma+1, V]  target logits; row t scores the token
 *                                    after block row t
 *   y          fp32 [B, gamma, V]    draft logits of draft t
 *   draft      int32 [B, gamma]      draft token ids x_t
 *   r          fp32 [B, gamma]       acceptance uniforms in [0, 1)
 *   u          fp32 [B, gamma+1]     sampling uniforms in [0, 1); u[b,t] is
 *                                    used only for a draw at row t
 *   T          temperature > 0 for both p and q;  eta  finite
 *   n_accept   int32 [B]             out: number of leading accepted drafts
 *                                    (-1 if a draft id is out of range)
 *   out_tokens int32 [B, gamma+1]    out: x_0..x_{n-1}, then the drawn token,
 *                                    then -1
 *   ratio_out  fp32 [B, gamma] or NULL  out: min(1, p_hat_t[x_t]/q_t[x_t])
 *   p_hat_out  fp32 [B, gamma, V] or NULL  out: p_hat for every draft row
 *   workspace  device scratch of at least rapid_accept_workspace_size bytes
 * The draw at row t picks the smallest id k (ascending) whose cumulative
 * weight exceeds u_t * W, W the row's total weight; if rounding leaves no
 * such id, the largest id of positive weight.  Supports gamma in [1, 63],
 * V in [2, 2^22].
 */
rv_status rapid_accept(const float* z, const float* y, const int32_t* draft, const float* r,
                       const float* u, int B, int gamma, int V, float T, float eta,
                       int32_t* n_accept, int32_t* out_tokens, float* ratio_out,
                       float* p_hat_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Options of rapid_accept_ex: RAPID blog post, section 2.4 prints two more
 * inference rules.
 *   RV_ACCEPT_TAIL_PRESERVE    every entry of p_hat below 0.1 x max p_hat
 *                              takes the target's p, and the result is
 *                              renormalised (the page states no
 *                              renormalisation; without one p_hat is not a
 *                              distribution).  The adjusted p_hat is used in
 *                              the ratios, the residual and p_hat_out.
 *   RV_ACCEPT_PRINTED_RESIDUAL on rejection draw from the printed residual
 *                              norm(max(p - p_hat, p - q)) =
 *                              norm(p - min(p_hat, q)), clipped at zero
 *                              (its entries can be negative; the page gives
 *                              no clip).
 */
#define RV_ACCEPT_TAIL_PRESERVE 1u
#define RV_ACCEPT_PRINTED_RESIDUAL 2u

/*
 * rapid_accept_ex -- rapid_accept with options (flags = 0 is rapid_accept).
 * Same arguments and workspace; unknown flag bits -> RV_ERR_VALUE.
 */
rv_status rapid_accept_ex(const float* z, const float* y, const int32_t* draft, const float* r,
                          const float* u, int B, int gamma, int V, float T, float eta,
                          unsigned flags, int32_t* n_accept, int32_t* out_tokens,
                          float* ratio_out, float* p_hat_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of device workspace rapid_tree_accept needs for (B, n, V), for any
 * tree of n nodes. */
size_t rapid_tree_accept_workspace_size(int B, int n, int V);

/*
 * rapid_tree_accept -- acceptance over a draft tree for B sequences that share
 * one tree.  The pages verify trees only as attention (LongSpec summary,
 * section 1 challenge 3 and section 2.3); the rule among siblings is taken
 * from outside them (recursive rejection, with RAPID's p_hat as the target,
 * RAPID blog post section 2.4): at node v the children are tested in
 * ascending node id, child c with its uniform r[c] against a residual R that
 * starts at p_hat_v and becomes norm(max(R - q_v, 0)) after each rejection,
 * where q_v = softmax(y_v/T) and p_hat_v = softmax(z_v/T + eta (q_v - p_v));
 * the first child accepted continues the walk; if every child is rejected a
 * token is drawn from the last residual with u[v]; at a leaf a bonus token is
 * drawn from p_v = softmax(z_v/T) with u[v].  On a chain (parent[i] = i - 1)
 * this is rapid_accept.  Given the path, the token emitted at a node follows
 * p_hat of the node when its children were drawn independently from its q.
 *
 *   z, y         fp32 [B, n, V]  target and drafter logits after each node
 *                                (node 0 is the root, the last committed
 *                                token; leaves' y rows are not read)
 *   tokens       int32 [B, n]    draft token of each node (tokens[b][0] is
 *                                not read)
 *   parent_host  HOST int32 [n]  parent[0] == -1, 0 <= parent[i] < i (else
 *                                RV_ERR_VALUE); 1 <= n <= 64
 *   r, u         fp32 [B, n]     acceptance uniform of each node, sampling
 *                                uniform used if the walk stops at the node
 *   T > 0, eta finite
 *   n_accept     int32 [B]       out: nodes accepted on the path (-1 if a
 *                                token of a non-root node is outside [0, V))
 *   path         int32 [B, n]    out: the accepted node ids in order, then -1
 *   out_tokens   int32 [B, n]    out: their tokens, then the drawn token,
 *                                then -1
 *   ratio_out    fp32 [B, n] or NULL  out: the ratio min(1, R[x_c]/q[x_c]) of
 *                                every child tested on the path, NaN elsewhere
 *   workspace    device scratch of rapid_tree_accept_workspace_size bytes (no
 *                initial contents needed)
 * The draw is rapid_accept's inverse CDF (smallest id whose cumulative weight
 * exceeds u * W).  Launches 3 + (largest child count - 1) kernels on stream.
 * Supports V in [2, 2^22].
 */
rv_status rapid_tree_accept(const float* z, const float* y, const int32_t* tokens,
                            const int32_t* parent_host, const float* r, const float* u, int B,
                            int n, int V, float T, float eta, int32_t* n_accept, int32_t* path,
                            int32_t* out_tokens, float* ratio_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * rapid_accept_noalloc -- rapid_accept_ex with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Its workspace is
 * a static device array of RV_NOALLOC_SCRATCH_BYTES (4 MiB; one copy on each
 * device the library runs on, held until the process ends); the call itself
 * allocates and frees nothing.  Shapes whose workspace
 * (rapid_accept_workspace_size) exceeds it return RV_ERR_WORKSPACE before
 * any HIP call; the other arguments and their checks are those of
 * rapid_accept_ex.  The first call on a device looks up that device's copy
 * (hipGetSymbolAddress) and keeps the address; a failure there is
 * RV_ERR_HIP.  Every call on one device shares that device's array, so calls
 * that may overlap on one device (different streams) race and must not be
 * made; calls in one stream are safe, each one clearing what it needs.
 */
#define RV_NOALLOC_SCRATCH_BYTES (4u << 20)
rv_status rapid_accept_noalloc(const float* z, const float* y, const int32_t* draft,
                               const float* r, const float* u, int B, int gamma, int V,
                               float T, float eta, unsigned flags, int32_t* n_accept,
                               int32_t* out_tokens, float* ratio_out, float* p_hat_out,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RAPID_VERIFY_H */
