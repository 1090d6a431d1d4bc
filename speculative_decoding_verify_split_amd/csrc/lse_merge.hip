// lse_merge: log-sum-exp merge of the history partials and the draft-block
// partial (LongSpec summary, gist.science, section 2.3 "Fast Tree Attention":
// the outputs of the two parts are combined with the log-sum-exp trick).
// With M = max_k LSE_k and a_k = exp(LSE_k - M):
//   O = sum_k a_k O_k / sum_k a_k,   LSE = M + log sum_k a_k.
// Without a block partial (o_blk = lse_blk = NULL) the history partials are
// merged alone, as for a drafter's cross-attention over the target cache.
//
// One workgroup of NWV waves per output row; the row's S partials are
// contiguous ([row][S][d]).  Wave w folds splits w, w + NWV, ... in
// ascending order (each split one 4*d-byte line read by all 64 lanes), the
// wave sums are added in wave order and the block partial last, so the
// result is bit-deterministic for a given S.  A wave's partials are loaded
// in batches of FB with every load of a batch in flight at once: the loads
// do not depend on the row's maximum, so a row costs ceil(S / (NWV FB))
// memory round trips.  The launch picks (FB, NWV) from S: (8, 4), (16, 4)
// and (32, 4) up to S = 32, 64 and 128, then (32, 8), so that a row takes
// one round trip up to S = 256 while short folds keep their registers low.
//
// spec_attn_block_merge does the same with the block partial computed in
// place: wave 0 of each row's workgroup also runs the row's masked block
// attention (block_row.h) while the history partials are in flight, which
// saves the block pass its own launch and its round trip through memory.

#include <hip/hip_ext.h>

#include "block_row.h"
#include "merge_fold.h"
#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

template <int D, int FB, int NWV>
__global__ __launch_bounds__(NWV * 64) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int S,
                                                    const float* __restrict__ o_blk,
                                                    const float* __restrict__ lse_blk,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  __shared__ float part[NWV][D];
  __shared__ float wpart[NWV];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x;
  const float* lp = lse_part + (size_t)row * S;
  const float* op = o_part + (size_t)row * S * D + lane * PER;
  // The first batch of this wave's partials is requested before the max is
  // known (empty splits hold zeros).
  PartialFold<D, NWV, FB> pf;
  pf.load(op, lp, S, wave, 0);
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s]);
  M = wave_max(M);
  const float lb = lse_blk != nullptr ? lse_blk[row] : -INFINITY;  // no block part: weight 0
  M = fmaxf(M, lb);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) pf.fold(op, lp, S, wave, M, acc, wsum);
#pragma unroll
  for (int e = 0; e < PER; ++e) part[wave][lane * PER + e] = acc[e];
  if (lane == 0) wpart[wave] = wsum;
  __syncthreads();
  if (wave != 0) return;
  float tot = wave_order_sum<NWV>(wpart, 1);
  float res[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = wave_order_sum<NWV>(&part[0][lane * PER + e], D);
  if (M != -INFINITY && lse_blk != nullptr) {
    const float a = exp2_hw((lb - M) * kLog2e);
    tot += a;
    const float* bp = o_blk + (size_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] = fmaf(a, bp[e], res[e]);
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  uint16_t* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = f32_to_bf16_bits(res[e] * inv);
  if (lse_out != nullptr && lane == 0)
    lse_out[row] = (M == -INFINITY) ? -INFINITY : M + log2_hw(tot) * kLn2;
}

// grid (B * Hq * n): the merge above with the block partial computed by
// wave 0 of the row's workgroup.  The history splits are folded against
// their own maximum Ms; the final combine rescales the history sums by
// exp(Ms - M) and the block partial by exp(LSE_blk - M), M the larger of the
// two, which is the same log-sum-exp merge.
template <int D, int FB, int NWV>
__global__ __launch_bounds__(NWV * 64) void block_merge_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, BlockMask mask, int Hq, int G, int n, float scale_log2,
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int S,
    uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  __shared__ float part[NWV][D];
  __shared__ float wpart[NWV];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x;  // (b * Hq + h) * n + i
  const int i = row % n;
  const int bh = row / n;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const float* lp = lse_part + (size_t)row * S;
  const float* op = o_part + (size_t)row * S * D + lane * PER;
  PartialFold<D, NWV, FB> pf;
  pf.load(op, lp, S, wave, 0);
  float ob[PER], lb2 = 0.f;
  if (wave == 0) {
    const size_t kv0 = ((size_t)b * (Hq / G) + h / G) * n * D;
    block_row_attention<D>(q + (size_t)row * D, kb + kv0, vb + kv0, mask.bits[i], n, scale_log2,
                           ob, lb2);
  }
  float Ms = -INFINITY;
  for (int s = lane; s < S; s += 64) Ms = fmaxf(Ms, lp[s]);
  Ms = wave_max(Ms);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (Ms != -INFINITY) pf.fold(op, lp, S, wave, Ms, acc, wsum);
#pragma unroll
  for (int e = 0; e < PER; ++e) part[wave][lane * PER + e] = acc[e];
  if (lane == 0) wpart[wave] = wsum;
  __syncthreads();
  if (wave != 0) return;
  const float lb = lb2 * kLn2;  // finite: a row always sees itself
  const float M = fmaxf(Ms, lb);
  const float fs = (Ms == -INFINITY) ? 0.f : exp2_hw((Ms - M) * kLog2e);
  const float fb = exp2_hw((lb - M) * kLog2e);
  const float tot = fmaf(fs, wave_order_sum<NWV>(wpart, 1), fb);
  const float inv = 1.0f / tot;  // tot >= fb = 1 or fs * wsum >= 1
  uint16_t* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane * PER + e;
    const float hs = wave_order_sum<NWV>(&part[0][c], D);
    dst[e] = f32_to_bf16_bits(fmaf(fs, hs, fb * ob[e]) * inv);
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = M + log2_hw(tot) * kLn2;
}

// Fold shape for S partials per row: partials per wave per batch of loads
// (FB) and waves per row (NWV); the index 0..3 selects one of the four.
int fold_shape(int S) { return S <= 32 ? 0 : (S <= 64 ? 1 : (S <= 128 ? 2 : 3)); }

// With events the launch records them on the kernel's own dispatch.
template <int D, int FB, int NWV>
void launch_block_merge(dim3 grid, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const BlockMask& mask, int Hq, int G, int n, float scale_log2,
                        const float* o_part, const float* lse_part, int S, uint16_t* out,
                        float* lse_out) {
  if (ev_start != nullptr || ev_stop != nullptr)
    hipExtLaunchKernelGGL((block_merge_kernel<D, FB, NWV>), grid, dim3(NWV * 64), 0, s, ev_start,
                          ev_stop, 0, q, k, v, mask, Hq, G, n, scale_log2, o_part, lse_part, S,
                          out, lse_out);
  else
    hipLaunchKernelGGL((block_merge_kernel<D, FB, NWV>), grid, dim3(NWV * 64), 0, s, q, k, v,
                       mask, Hq, G, n, scale_log2, o_part, lse_part, S, out, lse_out);
}

template <int D, int FB, int NWV>
void launch_merge(dim3 grid, hipStream_t s, const float* o_part, const float* lse_part, int S,
                  const float* o_blk, const float* lse_blk, uint16_t* out, float* lse_out) {
  hipLaunchKernelGGL((merge_kernel<D, FB, NWV>), grid, dim3(NWV * 64), 0, s, o_part, lse_part,
                     S, o_blk, lse_blk, out, lse_out);
}

}  // namespace
}  // namespace rv

namespace rv {

rv_status block_merge_launch(const void* q, const void* k_blk, const void* v_blk,
                             const BlockMask& mask, const float* o_part, const float* lse_part,
                             int S, int B, int Hq, int Hkv, int n, int d, float scale_log2,
                             void* out, float* lse_out, void* stream, void* start_event,
                             void* stop_event) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t ev0 = static_cast<hipEvent_t>(start_event);
  hipEvent_t ev = static_cast<hipEvent_t>(stop_event);
  dim3 grid((unsigned)(B * Hq * n));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_blk);
  const uint16_t* vv = static_cast<const uint16_t*>(v_blk);
  uint16_t* o16 = static_cast<uint16_t*>(out);
  const int G = Hq / Hkv;
  const int fs = fold_shape(S);
#define RV_BM_CASE(DD, F, FB, NWV)                                                           \
  if (d == DD && fs == F)                                                                    \
    launch_block_merge<DD, FB, NWV>(grid, s, ev0, ev, qq, kk, vv, mask, Hq, G, n, scale_log2, \
                                    o_part, lse_part, S, o16, lse_out);
  RV_BM_CASE(64, 0, 8, 4)
  else RV_BM_CASE(64, 1, 16, 4)
  else RV_BM_CASE(64, 2, 32, 4)
  else RV_BM_CASE(64, 3, 32, 8)
  else RV_BM_CASE(128, 0, 8, 4)
  else RV_BM_CASE(128, 1, 16, 4)
  else RV_BM_CASE(128, 2, 32, 4)
  else RV_BM_CASE(128, 3, 32, 8)
#undef RV_BM_CASE
  if (hipGetLastError() != hipSuccess) return RV_ERR_HIP;
  return RV_OK;
}

}  // namespace rv

extern "C" rv_status spec_attn_block_merge(const void* q, const void* k_blk, const void* v_blk,
                                           const int32_t* parent_host, const float* o_part,
                                           const float* lse_part, int S, int B, int Hq, int Hkv,
                                           int n, int d, float sm_scale, void* out,
                                           float* lse_out, void* stream) {
  rv::BlockMask mask;
  rv_status st = rv::check_block_merge(q, k_blk, v_blk, parent_host, o_part, lse_part, S, B, Hq,
                                       Hkv, n, d, sm_scale, out, &mask);
  if (st != RV_OK) return st;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  return rv::block_merge_launch(q, k_blk, v_blk, mask, o_part, lse_part, S, B, Hq, Hkv, n, d,
                                scale_log2, out, lse_out, stream, nullptr, nullptr);
}

extern "C" rv_status spec_attn_block_merge_ev(const void* q, const void* k_blk, const void* v_blk,
                                              const int32_t* parent_host, const float* o_part,
                                              const float* lse_part, int S, int B, int Hq,
                                              int Hkv, int n, int d, float sm_scale, void* out,
                                              float* lse_out, void* stream, void* start_event,
                                              void* stop_event) {
  rv::BlockMask mask;
  rv_status st = rv::check_block_merge(q, k_blk, v_blk, parent_host, o_part, lse_part, S, B, Hq,
                                       Hkv, n, d, sm_scale, out, &mask);
  if (st != RV_OK) return st;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  return rv::block_merge_launch(q, k_blk, v_blk, mask, o_part, lse_part, S, B, Hq, Hkv, n, d,
                                scale_log2, out, lse_out, stream, start_event, stop_event);
}

extern "C" rv_status lse_merge(const float* o_part, const float* lse_part, int S,
                               const float* o_blk, const float* lse_blk, int B, int Hq, int n,
                               int d, void* out, float* lse_out, void* stream) {
  rv_status st = rv::check_merge(o_part, lse_part, S, o_blk, lse_blk, B, Hq, n, d, out);
  if (st != RV_OK) return st;
  const int rows = B * Hq * n;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)rows);
  uint16_t* o16 = static_cast<uint16_t*>(out);
  const int fs = rv::fold_shape(S);
#define RV_M_CASE(DD, F, FB, NWV)                                                            \
  if (d == DD && fs == F)                                                                    \
    rv::launch_merge<DD, FB, NWV>(grid, s, o_part, lse_part, S, o_blk, lse_blk, o16, lse_out);
  RV_M_CASE(64, 0, 8, 4)
  else RV_M_CASE(64, 1, 16, 4)
  else RV_M_CASE(64, 2, 32, 4)
  else RV_M_CASE(64, 3, 32, 8)
  else RV_M_CASE(128, 0, 8, 4)
  else RV_M_CASE(128, 1, 16, 4)
  else RV_M_CASE(128, 2, 32, 4)
  else RV_M_CASE(128, 3, 32, 8)
#undef RV_M_CASE
  if (hipGetLastError() != hipSuccess) return RV_ERR_HIP;
  return RV_OK;
}
