// Host-side argument validation and launch planning for rapid_verify.
// This unit makes no HIP call, so every check can be exercised without a GPU.

#include <math.h>
#include <string.h>

#include "rv_internal.h"

namespace rv {

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(int a, int b) { return (int)(((int64_t)a + b - 1) / b); }

}  // namespace

// Callers validate (Hq/Hkv)*n <= RV_MAX_GROUP_ROWS first; larger groups are
// clamped here only so the arithmetic stays defined.
RowPlan row_plan(int Hq, int Hkv, int n) {
  RowPlan p;
  const int64_t M = (int64_t)(Hq / Hkv) * n;
  p.M = (int)(M < RV_MAX_GROUP_ROWS ? M : RV_MAX_GROUP_ROWS);
  p.MT = ceil_div(p.M, 16);
  p.wide = p.MT > kMaxTilesPerWave;
  p.MTW = p.wide ? ceil_div(p.MT, kWavesPerGroup) : p.MT;
  return p;
}

static rv_status check_heads(int B, int Hq, int Hkv, int n, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || n < 1) return RV_ERR_SHAPE;
  if (Hq % Hkv != 0) return RV_ERR_SHAPE;
  if (B > 65535 || Hq > 65535) return RV_ERR_UNSUPPORTED;  // grid dimensions
  if (n > RV_MAX_BLOCK_ROWS) return RV_ERR_UNSUPPORTED;
  if ((int64_t)(Hq / Hkv) * n > RV_MAX_GROUP_ROWS) return RV_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return RV_ERR_UNSUPPORTED;
  return RV_OK;
}

rv_status check_prefix(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq, int Hkv,
                       int n, int d, int64_t L_max, float sm_scale, int64_t split_len,
                       int num_splits, const float* o_part, const float* lse_part) {
  if (!q || !k_cache || !v_cache || !seq_lens || !o_part || !lse_part) return RV_ERR_NULL;
  rv_status st = check_heads(B, Hq, Hkv, n, d);
  if (st != RV_OK) return st;
  if (L_max < 0 || max_seq_len < 0 || max_seq_len > L_max) return RV_ERR_SHAPE;
  // buffer offsets inside one (sequence, kv-head) slab are 32-bit
  if (L_max > (int64_t)0x7fffffff / (2 * d)) return RV_ERR_UNSUPPORTED;
  if (split_len <= 0 || split_len % kSplitQuantum != 0) return RV_ERR_SHAPE;
  if (num_splits < 1 || num_splits > 65535) return RV_ERR_SHAPE;
  if ((max_seq_len + split_len - 1) / split_len > num_splits) return RV_ERR_SHAPE;
  if (!isfinite(sm_scale) || !(sm_scale > 0.0f)) return RV_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_part) ||
      !aligned16(lse_part))
    return RV_ERR_ALIGNMENT;
  if (Hkv > 65535) return RV_ERR_UNSUPPORTED;  // grid dimension
  return RV_OK;
}

static rv_status block_mask(const int32_t* parent_host, int n, BlockMask* mask) {
  BlockMask m;
  memset(&m, 0, sizeof(m));
  if (parent_host == nullptr) {
    for (int i = 0; i < n; ++i) m.bits[i] = (i == 63) ? ~0ull : ((1ull << (i + 1)) - 1ull);
  } else {
    if (parent_host[0] != -1) return RV_ERR_VALUE;
    m.bits[0] = 1ull;
    for (int i = 1; i < n; ++i) {
      int p = parent_host[i];
      if (p < 0 || p >= i) return RV_ERR_VALUE;
      // ancestors of i = ancestors of its parent (already final) plus i itself
      m.bits[i] = m.bits[p] | (1ull << i);
    }
  }
  if (mask) *mask = m;
  return RV_OK;
}

rv_status check_block(const void* q, const void* k_blk, const void* v_blk,
                      const int32_t* parent_host, int B, int Hq, int Hkv, int n, int d,
                      float sm_scale, const float* o_blk, const float* lse_blk, BlockMask* mask) {
  if (!q || !k_blk || !v_blk || !o_blk || !lse_blk) return RV_ERR_NULL;
  rv_status st = check_heads(B, Hq, Hkv, n, d);
  if (st != RV_OK) return st;
  if (!isfinite(sm_scale) || !(sm_scale > 0.0f)) return RV_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o_blk) ||
      !aligned16(lse_blk))
    return RV_ERR_ALIGNMENT;
  if ((int64_t)B * Hq > 65535) return RV_ERR_UNSUPPORTED;  // grid dimension y
  return block_mask(parent_host, n, mask);
}

rv_status check_block_merge(const void* q, const void* k_blk, const void* v_blk,
                            const int32_t* parent_host, const float* o_part,
                            const float* lse_part, int S, int B, int Hq, int Hkv, int n, int d,
                            float sm_scale, const void* out, BlockMask* mask) {
  if (!q || !k_blk || !v_blk || !o_part || !lse_part || !out) return RV_ERR_NULL;
  rv_status st = check_heads(B, Hq, Hkv, n, d);
  if (st != RV_OK) return st;
  if (S < 1) return RV_ERR_SHAPE;
  if (!isfinite(sm_scale) || !(sm_scale > 0.0f)) return RV_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o_part) ||
      !aligned16(lse_part) || !aligned16(out))
    return RV_ERR_ALIGNMENT;
  if ((int64_t)B * Hq * n > 0x7fffffff / 4) return RV_ERR_UNSUPPORTED;  // one row per workgroup
  return block_mask(parent_host, n, mask);
}

rv_status check_verify(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, int64_t max_seq_len, int B, int Hq, int Hkv,
                       int n, int d, int64_t L_max, float sm_scale, int64_t split_len,
                       int num_splits, const void* k_blk, const void* v_blk,
                       const int32_t* parent_host, const float* o_part, const float* lse_part,
                       const void* sync, size_t sync_bytes, const void* out, int help_after_us,
                       BlockMask* mask) {
  if (!sync) return RV_ERR_NULL;
  rv_status st = check_prefix(q, k_cache, v_cache, seq_lens, max_seq_len, B, Hq, Hkv, n, d, L_max,
                              sm_scale, split_len, num_splits, o_part, lse_part);
  if (st != RV_OK) return st;
  st = check_block_merge(q, k_blk, v_blk, parent_host, o_part, lse_part, num_splits, B, Hq, Hkv,
                         n, d, sm_scale, out, mask);
  if (st != RV_OK) return st;
  if (!aligned16(sync)) return RV_ERR_ALIGNMENT;
  if (sync_bytes < verify_sync_bytes(B, Hkv)) return RV_ERR_WORKSPACE;
  if (help_after_us > kVerifyHelpMaxUs) return RV_ERR_VALUE;
  return RV_OK;
}

rv_status check_window(const void* q, const void* k_ring, const void* v_ring,
                       const int32_t* pos, int B, int Hq, int Hkv, int n, int d, int cap,
                       int sink, int window, float sm_scale, const void* out,
                       const void* workspace, size_t workspace_bytes) {
  if (!q || !k_ring || !v_ring || !pos || !out || !workspace) return RV_ERR_NULL;
  rv_status st = check_heads(B, Hq, Hkv, n, d);
  if (st != RV_OK) return st;
  if (window < 1 || sink < 0 || cap < 1) return RV_ERR_SHAPE;
  if (window > kMaxWindowKeys || sink > kMaxWindowKeys) return RV_ERR_UNSUPPORTED;
  // every position a row of the block sees must still be in the ring
  if ((int64_t)cap - sink < (int64_t)window + n - 1) return RV_ERR_SHAPE;
  if (!isfinite(sm_scale) || !(sm_scale > 0.0f)) return RV_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_ring) || !aligned16(v_ring) || !aligned16(out))
    return RV_ERR_ALIGNMENT;
  if ((int64_t)B * Hq * n > 0x7fffffff / 4) return RV_ERR_UNSUPPORTED;  // one row per workgroup
  if ((int64_t)B * n > 65535 || Hkv > 65535) return RV_ERR_UNSUPPORTED;  // grid dimensions
  if (!aligned16(workspace)) return RV_ERR_ALIGNMENT;
  const size_t rows = (size_t)B * Hq * n;
  if (workspace_bytes < window_workspace_words(rows, window_segments(sink, window), d) * 4)
    return RV_ERR_WORKSPACE;
  return RV_OK;
}

rv_status check_merge(const float* o_part, const float* lse_part, int S, const float* o_blk,
                      const float* lse_blk, int B, int Hq, int n, int d, const void* out) {
  if (!o_part || !lse_part || !out) return RV_ERR_NULL;
  if ((o_blk == nullptr) != (lse_blk == nullptr)) return RV_ERR_NULL;  // both or neither
  if (B < 1 || Hq < 1 || n < 1 || S < 1) return RV_ERR_SHAPE;
  if (n > RV_MAX_BLOCK_ROWS || B > 65535 || Hq > 65535) return RV_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return RV_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * n > 0x7fffffff / 4) return RV_ERR_UNSUPPORTED;
  if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(out)) return RV_ERR_ALIGNMENT;
  if (o_blk && (!aligned16(o_blk) || !aligned16(lse_blk))) return RV_ERR_ALIGNMENT;
  return RV_OK;
}

static size_t round_words(size_t w) { return (w + 63) & ~(size_t)63; }  // 256-byte regions

AcceptLayout accept_layout(int B, int gamma, int V) {
  AcceptLayout L;
  L.cs = ceil_div(V, kStatChunk);
  L.cp = ceil_div(V, kPhatChunk);
  L.cd = ceil_div(V, kDrawChunk);
  const size_t Bz = (size_t)B, g = (size_t)gamma;
  size_t off = 0;
  L.zstat = off;
  off += round_words(Bz * (g + 1) * L.cs * 2);
  L.ystat = off;
  off += round_words(Bz * g * L.cs * 2);
  L.sstat = off;
  off += round_words(Bz * g * L.cp * 2);
  L.rowtab = off;
  off += round_words(Bz * 4 * (g + 1));
  L.tstat = off;
  off += round_words(Bz * g * L.cp);
  L.wsum = off;
  off += round_words(Bz * L.cd * 2);
  L.arrivals = off;
  off += round_words(Bz * kArrivalStride);
  L.words = off;
  return L;
}

rv_status check_accept_args(const float* z, const float* y, const int32_t* draft,
                            const float* r, const float* u, int B, int gamma, int V, float T,
                            float eta, unsigned flags, const int32_t* n_accept,
                            const int32_t* out_tokens) {
  if (!z || !y || !draft || !r || !u || !n_accept || !out_tokens) return RV_ERR_NULL;
  if (B < 1 || gamma < 1 || V < 2) return RV_ERR_SHAPE;
  if (gamma > kMaxGamma || V > kMaxVocab || B > 65535) return RV_ERR_UNSUPPORTED;
  if (!(T > 0.0f) || !isfinite(T) || !isfinite(eta)) return RV_ERR_VALUE;
  if (flags & ~kAcceptFlags) return RV_ERR_VALUE;
  if (!aligned16(z) || !aligned16(y)) return RV_ERR_ALIGNMENT;
  return RV_OK;
}

rv_status check_accept(const float* z, const float* y, const int32_t* draft, const float* r,
                       const float* u, int B, int gamma, int V, float T, float eta, unsigned flags,
                       const int32_t* n_accept, const int32_t* out_tokens, const void* workspace,
                       size_t workspace_bytes) {
  if (!workspace) return RV_ERR_NULL;
  const rv_status st =
      check_accept_args(z, y, draft, r, u, B, gamma, V, T, eta, flags, n_accept, out_tokens);
  if (st != RV_OK) return st;
  if (!aligned16(workspace)) return RV_ERR_ALIGNMENT;
  if (workspace_bytes < accept_layout(B, gamma, V).words * 4) return RV_ERR_WORKSPACE;
  return RV_OK;
}

rv_status tree_plan(const int32_t* parent, int n, TreePlan* P) {
  if (!parent) return RV_ERR_NULL;
  if (n < 1 || n > kMaxTreeNodes) return RV_ERR_SHAPE;
  if (parent[0] != -1) return RV_ERR_VALUE;
  for (int i = 1; i < n; ++i)
    if (parent[i] < 0 || parent[i] >= i) return RV_ERR_VALUE;
  *P = TreePlan{};
  P->n = n;
  for (int v = 0; v < n; ++v) {
    P->parent[v] = (int8_t)parent[v];
    P->slot[v] = -1;
    P->inode[v] = -1;
  }
  for (int c = 1; c < n; ++c) {
    const int v = parent[c];
    P->rank[c] = P->nchild[v]++;
    P->kids[v] |= 1ull << c;
  }
  int maxk = 0;
  for (int v = 0; v < n; ++v) {
    if (P->nchild[v] > 0) {
      P->slot[v] = (int8_t)P->ni;
      P->inode[P->ni++] = (int8_t)v;
    }
    if (P->nchild[v] > maxk) maxk = P->nchild[v];
  }
  P->npass = maxk > 0 ? maxk - 1 : 0;
  return RV_OK;
}

TreeLayout tree_layout(int B, int n, int V) {
  TreeLayout L;
  L.cs = ceil_div(V, kStatChunk);
  L.cp = ceil_div(V, kPhatChunk);
  L.cd = ceil_div(V, kDrawChunk);
  const size_t Bz = (size_t)B, N = (size_t)n;
  size_t off = 0;
  L.zstat = off;
  off += round_words(Bz * N * L.cs * 2);
  L.ystat = off;
  off += round_words(Bz * N * L.cs * 2);
  L.sstat = off;
  off += round_words(Bz * N * L.cp * 2);
  L.rowtab = off;
  off += round_words(Bz * 2 * N);
  L.rstat = off;
  off += round_words(Bz * N * N * L.cp);
  L.wsum = off;
  off += round_words(Bz * L.cd * 2);
  L.arrivals = off;
  off += round_words(Bz * kArrivalStride);
  L.words = off;
  return L;
}

rv_status check_tree_accept(const float* z, const float* y, const int32_t* tokens,
                            const int32_t* parent_host, const float* r, const float* u, int B,
                            int n, int V, float T, float eta, const int32_t* n_accept,
                            const int32_t* path, const int32_t* out_tokens,
                            const void* workspace, size_t workspace_bytes, TreePlan* plan) {
  if (!z || !y || !tokens || !parent_host || !r || !u || !n_accept || !path || !out_tokens ||
      !workspace)
    return RV_ERR_NULL;
  if (B < 1 || n < 1 || V < 2) return RV_ERR_SHAPE;
  if (n > kMaxTreeNodes || V > kMaxVocab || B > 65535) return RV_ERR_UNSUPPORTED;
  if (!(T > 0.0f) || !isfinite(T) || !isfinite(eta)) return RV_ERR_VALUE;
  const rv_status st = tree_plan(parent_host, n, plan);
  if (st != RV_OK) return st;
  if (!aligned16(z) || !aligned16(y) || !aligned16(workspace)) return RV_ERR_ALIGNMENT;
  if (workspace_bytes < tree_layout(B, n, V).words * 4) return RV_ERR_WORKSPACE;
  return RV_OK;
}

}  // namespace rv

extern "C" {

const char* rv_status_string(int status) {
  switch (status) {
    case RV_OK: return "RV_OK";
    case RV_ERR_NULL: return "RV_ERR_NULL: a required pointer is NULL";
    case RV_ERR_SHAPE: return "RV_ERR_SHAPE: a size is out of range or inconsistent";
    case RV_ERR_UNSUPPORTED: return "RV_ERR_UNSUPPORTED: shape not supported by this library";
    case RV_ERR_VALUE: return "RV_ERR_VALUE: a scalar or the tree is invalid";
    case RV_ERR_WORKSPACE: return "RV_ERR_WORKSPACE: workspace too small";
    case RV_ERR_HIP: return "RV_ERR_HIP: a HIP launch failed";
    case RV_ERR_ALIGNMENT: return "RV_ERR_ALIGNMENT: a tensor pointer is not 16-byte aligned";
    default: return "unknown rv_status";
  }
}

int rv_version(void) { return 100; }

rv_status rv_prefix_default_split(int64_t max_seq_len, int B, int Hq, int Hkv, int n, int d,
                                  int64_t* split_len, int* num_splits) {
  if (!split_len || !num_splits) return RV_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || n < 1 || Hq % Hkv != 0 || max_seq_len < 0)
    return RV_ERR_SHAPE;
  if (B > 65535 || max_seq_len > ((int64_t)1 << 40)) return RV_ERR_UNSUPPORTED;
  if (n > RV_MAX_BLOCK_ROWS || (int64_t)(Hq / Hkv) * n > RV_MAX_GROUP_ROWS)
    return RV_ERR_UNSUPPORTED;
  (void)d;
  const int64_t q = rv::kSplitQuantum;
  const int64_t groups = (int64_t)B * Hkv;
  const int64_t target_groups = 256;  // one 4-wave workgroup per compute unit
  // with at least one group per compute unit every group takes its whole
  // sequence as one split (and the product below could overflow)
  int64_t per = groups >= target_groups
                    ? max_seq_len
                    : (max_seq_len * groups + target_groups - 1) / target_groups;
  int64_t len = ((per + q - 1) / q) * q;
  const int64_t min_len = 4 * q;  // at least 4 tiles per wave
  if (len < min_len) len = min_len;
  int64_t S = (max_seq_len + len - 1) / len;
  if (S < 1) S = 1;
  if (S > 65535) return RV_ERR_UNSUPPORTED;
  *split_len = len;
  *num_splits = (int)S;
  return RV_OK;
}

rv_status rv_prefix_balanced_split(const int32_t* seq_lens_host, int B, int Hq, int Hkv, int n,
                                   int d, int num_cus, int64_t* split_len, int* num_splits) {
  if (!seq_lens_host || !split_len || !num_splits) return RV_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || n < 1 || Hq % Hkv != 0 || num_cus < 1) return RV_ERR_SHAPE;
  if (B > 65535) return RV_ERR_UNSUPPORTED;
  if (n > RV_MAX_BLOCK_ROWS || (int64_t)(Hq / Hkv) * n > RV_MAX_GROUP_ROWS)
    return RV_ERR_UNSUPPORTED;
  (void)d;
  int64_t max_len = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t L = seq_lens_host[b];
    if (L < 0) return RV_ERR_VALUE;
    if (L > max_len) max_len = L;
  }
  const int64_t q = rv::kSplitQuantum;
  const int64_t min_len = 4 * q;  // at least 4 tiles per wave
  // Workgroups that get keys with splits of m quanta: Hkv * sum_b ceil(L_b / (m q)).
  auto busy = [&](int64_t m) {
    int64_t c = 0;
    for (int b = 0; b < B; ++b) c += (seq_lens_host[b] + m * q - 1) / (m * q);
    return c * Hkv;
  };
  int64_t lo = min_len / q;
  int64_t hi = (max_len + q - 1) / q;  // one split per sequence
  if (hi < lo) hi = lo;
  if (busy(hi) <= num_cus) {
    // smallest split whose non-empty workgroups fit on the compute units at once
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (busy(mid) <= num_cus) hi = mid;
      else lo = mid + 1;
    }
  }
  const int64_t len = hi * q;
  int64_t S = (max_len + len - 1) / len;
  if (S < 1) S = 1;
  if (S > 65535) return RV_ERR_UNSUPPORTED;
  *split_len = len;
  *num_splits = (int)S;
  return RV_OK;
}

size_t spec_attn_verify_sync_size(int B, int Hkv) {
  if (B < 1 || Hkv < 1 || B > 65535 || Hkv > 65535) return 0;
  return rv::verify_sync_bytes(B, Hkv);
}

int rv_verify_single_launch(int B, int Hq, int Hkv, int n, int d, int num_splits, int num_cus) {
  if (B < 1 || Hq < 1 || Hkv < 1 || n < 1 || Hq % Hkv != 0 || num_cus < 1) return 0;
  if (n > RV_MAX_BLOCK_ROWS || (int64_t)(Hq / Hkv) * n > RV_MAX_GROUP_ROWS) return 0;
  if (d != 64 && d != 128) return 0;
  if (num_splits < 1 || num_splits > rv::kVerifyMaxSplits) return 0;
  const rv::RowPlan rp = rv::row_plan(Hq, Hkv, n);
  if (rp.wide) return 0;
  // d = 128 with 4 row tiles: the fused kernel would exceed 512 registers
  if (d == 128 && rp.MT == 4) return 0;
  // at most one merged row per wave, a small grid, and every workgroup of it
  // resident at once (one per compute unit)
  if ((rp.M + num_splits - 1) / num_splits > rv::kWavesPerGroup) return 0;
  const int64_t groups = (int64_t)B * Hkv * num_splits;
  return groups <= rv::kVerifySingleMaxGroups && groups <= num_cus ? 1 : 0;
}

}  // extern "C"
