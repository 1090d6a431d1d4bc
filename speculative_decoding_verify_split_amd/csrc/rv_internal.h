// Internal declarations shared by the library's translation units.
// Host-only: argument validation and launch planning (no HIP types here, so
// the validation unit builds and runs without a GPU).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "rapid_verify.h"

namespace rv {

// --- attention --------------------------------------------------------------

constexpr int kKeysPerTile = 32;    // keys per wave iteration (two 16-key MFMA blocks)
constexpr int kWavesPerGroup = 4;   // waves per workgroup in the history kernel
constexpr int kMaxTilesPerWave = 4; // 16-row MFMA tiles a wave keeps in registers
constexpr int kSplitQuantum = kKeysPerTile * kWavesPerGroup;  // split_len granularity

// How the rows of one (sequence, kv-head) group are spread over workgroups:
// M = (Hq/Hkv)*n rows in MT = ceil(M/16) row tiles.  Up to kMaxTilesPerWave
// tiles every wave keeps all of them (MTW = MT) and streams its own share of
// the keys; wider groups go to the shared-stage kernel, where wave w keeps
// tiles w, w + 4, ... (MTW = ceil(MT/4) of them) and sees every key.
struct RowPlan {
  int M, MT, MTW;
  bool wide;
};
RowPlan row_plan(int Hq, int Hkv, int n);

rv_status check_prefix(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq, int Hkv,
                       int n, int d, int64_t L_max, float sm_scale, int64_t split_len,
                       int num_splits, const float* o_part, const float* lse_part);

// Tree / chain visibility as one 64-bit mask per block row: bit j of
// bits[i] is set iff row i sees block row j.
struct BlockMask {
  uint64_t bits[RV_MAX_BLOCK_ROWS];
};
rv_status check_block(const void* q, const void* k_blk, const void* v_blk,
                      const int32_t* parent_host, int B, int Hq, int Hkv, int n, int d,
                      float sm_scale, const float* o_blk, const float* lse_blk, BlockMask* mask);

rv_status check_block_merge(const void* q, const void* k_blk, const void* v_blk,
                            const int32_t* parent_host, const float* o_part,
                            const float* lse_part, int S, int B, int Hq, int Hkv, int n, int d,
                            float sm_scale, const void* out, BlockMask* mask);

// The block + merge launch of spec_attn_block_merge with a prebuilt mask;
// start_event and stop_event (hipEvent_t or NULL) are recorded on the
// kernel's own dispatch.
rv_status block_merge_launch(const void* q, const void* k_blk, const void* v_blk,
                             const BlockMask& mask, const float* o_part, const float* lse_part,
                             int S, int B, int Hq, int Hkv, int n, int d, float scale_log2,
                             void* out, float* lse_out, void* stream, void* start_event,
                             void* stop_event);

// --- single-launch verify pass (spec_attn_verify) -----------------------------

// The splits of one (sequence, kv head) are tracked in one 64-bit mask word.
constexpr int kVerifyMaxSplits = 64;
// The single launch pays where its grid is small: measured on MI355X at
// 32/8 heads, n = 11, it took 13.5 us against 17.6-26 us for the two
// launches at 16 workgroups (8/2 heads, 4K tokens), tied at 128, and lost at
// 256 (97 against 89 us at 128K tokens): the cross-XCD publish and poll cost
// grows with the grid, and a workgroup merging more than one row per wave
// serialises them (32 workgroups of 11 rows each: 34 against 22 us).
constexpr int kVerifySingleMaxGroups = 64;
// Default wait before a workgroup computes a missing split itself: 200 us of
// the 100 MHz constant clock (s_memrealtime).
constexpr int kVerifyHelpDefaultUs = 200;
constexpr int kVerifyHelpMaxUs = 10000000;
// Sync words: per (sequence, kv head) the split mask and the finished count.
inline size_t verify_sync_bytes(int B, int Hkv) { return (size_t)B * (size_t)Hkv * 16; }

rv_status check_verify(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq, int Hkv,
                       int n, int d, int64_t L_max, float sm_scale, int64_t split_len,
                       int num_splits, const void* k_blk, const void* v_blk,
                       const int32_t* parent_host, const float* o_part, const float* lse_part,
                       const void* sync, size_t sync_bytes, const void* out, int help_after_us,
                       BlockMask* mask);

// Largest first-row position spec_attn_window accepts (device values above
// it are clamped), so that positions of a block's rows stay in int range.
constexpr int kMaxWindowPos = 1 << 30;

// Largest window or sink spec_attn_window accepts (keeps key counts and
// segment counts far from int overflow; a drafter's window is ~10^3).
constexpr int kMaxWindowKeys = 1 << 24;

// spec_attn_window's key list is cut into 64-key segments; its workspace is
// the segments' partials, o [B*Hq*n][S][d] then lse [B*Hq*n][S] (fp32).
inline int window_segments(int sink, int window) {
  return (int)(((int64_t)sink + window + 63) / 64);
}
inline size_t window_o_words(size_t rows, size_t S, int d) {
  return (rows * S * (size_t)d + 63) & ~(size_t)63;
}
inline size_t window_workspace_words(size_t rows, size_t S, int d) {
  return window_o_words(rows, S, d) + ((rows * S + 63) & ~(size_t)63);
}

rv_status check_window(const void* q, const void* k_ring, const void* v_ring,
                       const int32_t* pos, int B, int Hq, int Hkv, int n, int d, int cap,
                       int sink, int window, float sm_scale, const void* out,
                       const void* workspace, size_t workspace_bytes);

rv_status check_merge(const float* o_part, const float* lse_part, int S, const float* o_blk,
                      const float* lse_blk, int B, int Hq, int n, int d, const void* out);

// --- vocabulary pass --------------------------------------------------------

constexpr int kVocabThreads = 256;
// Elements per thread, hence chunk lengths, of the passes over the
// vocabulary.  The statistics and p_hat passes run many rows at once and
// take long chunks (fewer partials for the next pass to combine); the
// decide/draw pass works on one row, so it takes short chunks to spread that
// row's exp work over more workgroups, and its last workgroup re-evaluates
// one whole chunk alone.
constexpr int kStatPer = 16;
constexpr int kPhatPer = 16;
constexpr int kDrawPer = 4;
constexpr int kStatChunk = kVocabThreads * kStatPer;  // 4096
constexpr int kPhatChunk = kVocabThreads * kPhatPer;  // 4096
constexpr int kDrawChunk = kVocabThreads * kDrawPer;  // 1024
// Words between two sequences' arrival counters: one 256-byte line each, so
// the atomics of different sequences never queue on one cache line.
constexpr int kArrivalStride = 64;
constexpr int kMaxVocab = 1 << 22;
constexpr int kMaxGamma = 63;  // one wave decides the first-reject cut

// Workspace layout of rapid_accept, in 4-byte words from the base.
struct AcceptLayout {
  int cs, cp, cd;      // chunk counts: ceil(V / kStatChunk), kPhatChunk, kDrawChunk
  size_t zstat;        // [B][gamma+1][cs][2]  (max, sum) of z/T in log2 units
  size_t ystat;        // [B][gamma][cs][2]
  size_t sstat;        // [B][gamma][cp][2]    of s = z/T + eta (q - p)
  size_t rowtab;       // [B][4][gamma+1]      base-2 LSE of z/T and y/T per row,
                       //                      then each draft token's z and y
  size_t tstat;        // [B][gamma][cp]       chunk sums of the tail-adjusted p_hat
  size_t wsum;         // [B][cd] uint64       residual and p_hat weight per chunk
                       //                      (one slot each, vocab_common.h)
  size_t arrivals;     // [B][kArrivalStride] uint32: chunks done with their draw weight
  size_t words;        // total
};
AcceptLayout accept_layout(int B, int gamma, int V);

constexpr unsigned kAcceptFlags = RV_ACCEPT_TAIL_PRESERVE | RV_ACCEPT_PRINTED_RESIDUAL;

// --- acceptance over a draft tree ---------------------------------------------

constexpr int kMaxTreeNodes = RV_MAX_BLOCK_ROWS;

// The tree as the kernels see it, built on the host from the caller's parent
// array and passed to them by value.  Internal nodes (those with children)
// are numbered by slot in node order.
struct TreePlan {
  int n;                         // nodes
  int ni;                        // internal nodes
  int npass;                     // residual passes: largest child count - 1
  int8_t parent[kMaxTreeNodes];
  int8_t rank[kMaxTreeNodes];    // position of node c among its siblings (by id)
  int8_t nchild[kMaxTreeNodes];
  int8_t slot[kMaxTreeNodes];    // internal slot of node v, -1 for a leaf
  int8_t inode[kMaxTreeNodes];   // node of internal slot a
  uint64_t kids[kMaxTreeNodes];  // children of node v, bit c for node c
};
// Builds the plan; RV_ERR_VALUE unless parent[0] == -1 and
// 0 <= parent[i] < i for every other node.
rv_status tree_plan(const int32_t* parent_host, int n, TreePlan* plan);

// Workspace layout of rapid_tree_accept, in 4-byte words (independent of the
// tree's shape: sized for any tree of n nodes).
struct TreeLayout {
  int cs, cp, cd;      // chunk counts as in AcceptLayout
  size_t zstat;        // [B][n][cs][2]  (max, sum) of z/T per node
  size_t ystat;        // [B][n][cs][2]  of y/T per internal slot
  size_t sstat;        // [B][n][cp][2]  of s per internal slot
  size_t rowtab;       // [B][2][n]      base-2 LSE of z/T per node, of y/T per slot
  size_t rstat;        // [B][n][n][cp]  chunk sums of residual pass j per slot
  size_t wsum;         // [B][cd] uint64 draw weights per chunk (slots)
  size_t arrivals;     // [B][kArrivalStride]
  size_t words;
};
TreeLayout tree_layout(int B, int n, int V);

rv_status check_tree_accept(const float* z, const float* y, const int32_t* tokens,
                            const int32_t* parent_host, const float* r, const float* u, int B,
                            int n, int V, float T, float eta, const int32_t* n_accept,
                            const int32_t* path, const int32_t* out_tokens,
                            const void* workspace, size_t workspace_bytes, TreePlan* plan);

// Every argument check of rapid_accept except those of the workspace.
rv_status check_accept_args(const float* z, const float* y, const int32_t* draft,
                            const float* r, const float* u, int B, int gamma, int V, float T,
                            float eta, unsigned flags, const int32_t* n_accept,
                            const int32_t* out_tokens);

// Largest workspace rapid_accept_noalloc's static scratch holds.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;

rv_status check_accept(const float* z, const float* y, const int32_t* draft, const float* r,
                       const float* u, int B, int gamma, int V, float T, float eta, unsigned flags,
                       const int32_t* n_accept, const int32_t* out_tokens, const void* workspace,
                       size_t workspace_bytes);

}  // namespace rv
