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
// M = (Hq/Hkv)*n rows, MT = ceil(M/16) row tiles, RG row groups of MTW tiles.
struct RowPlan {
  int M, MT, RG, MTW;
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

rv_status check_merge(const float* o_part, const float* lse_part, int S, const float* o_blk,
                      const float* lse_blk, int B, int Hq, int n, int d, const void* out);

// --- vocabulary pass --------------------------------------------------------

constexpr int kVocabThreads = 256;
constexpr int kVocabPerThread = 16;
constexpr int kVocabChunk = kVocabThreads * kVocabPerThread;  // elements per workgroup
constexpr int kMaxVocab = 1 << 22;
constexpr int kMaxGamma = 63;  // one wave decides the first-reject cut

// Workspace layout of rapid_accept, in 4-byte words from the base.
struct AcceptLayout {
  int chunks;          // C = ceil(V / kVocabChunk)
  size_t zstat;        // [B][gamma+1][C][2]  (max, sum) of z/T in log2 units
  size_t ystat;        // [B][gamma][C][2]
  size_t sstat;        // [B][gamma][C][2]    of s = z/T + eta (q - p)
  size_t rowtab;       // [B][2][gamma+1]     base-2 LSE of z/T and y/T per row
  size_t tstat;        // [B][gamma][C]       chunk sums of the tail-adjusted p_hat
  size_t wsum;         // [B][C][2]           residual and p_hat weight per chunk
  size_t arrivals;     // [B] uint32          chunks done with their draw weight
  size_t words;        // total
};
AcceptLayout accept_layout(int B, int gamma, int V);

constexpr unsigned kAcceptFlags = RV_ACCEPT_TAIL_PRESERVE | RV_ACCEPT_PRINTED_RESIDUAL;

rv_status check_accept(const float* z, const float* y, const int32_t* draft, const float* r,
                       const float* u, int B, int gamma, int V, float T, float eta, unsigned flags,
                       const int32_t* n_accept, const int32_t* out_tokens, const void* workspace,
                       size_t workspace_bytes);

}  // namespace rv
