// lse_merge: log-sum-exp merge of the history partials and the draft-block
// partial (LongSpec summary, gist.science, section 2.3 "Fast Tree Attention":
// the outputs of the two parts are combined with the log-sum-exp trick).
// With M = max_k LSE_k and a_k = exp(LSE_k - M):
//   O = sum_k a_k O_k / sum_k a_k,   LSE = M + log sum_k a_k.
// Without a block partial (o_blk = lse_blk = NULL) the history partials are
// merged alone, as for a drafter's cross-attention over the target cache.
//
// One 4-wave workgroup per output row; the row's S partials are contiguous
// ([row][S][d]).  Wave w folds splits w, w + 4, ... (each step one 4*d-byte
// line read by all 64 lanes, four steps in flight), the four wave sums are
// added in wave order and the block partial last, so the result is
// bit-deterministic.
//
// spec_attn_block_merge does the same with the block partial computed in
// place: wave 0 of each row's workgroup also runs the row's masked block
// attention (block_row.h) while the history partials are in flight, which
// saves the block pass its own launch and its round trip through memory.

#include "block_row.h"
#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int S,
                                                    const float* __restrict__ o_blk,
                                                    const float* __restrict__ lse_blk,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  constexpr int NWV = 4;
  __shared__ float part[NWV][D];
  __shared__ float wpart[NWV];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x;
  const float* lp = lse_part + (size_t)row * S;
  const float* op = o_part + (size_t)row * S * D + lane * PER;
  // The first batch of this wave's partials is requested before the max is
  // known (empty splits hold zeros), so the row costs one memory round trip.
  constexpr int FIRST = 8;
  float val0[FIRST][PER];
#pragma unroll
  for (int j = 0; j < FIRST; ++j) {
    const int s = wave + j * NWV;
#pragma unroll
    for (int e = 0; e < PER; ++e) val0[j][e] = (s < S) ? op[(size_t)s * D + e] : 0.f;
  }
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s]);
  M = wave_max(M);
  const float lb = lse_blk != nullptr ? lse_blk[row] : -INFINITY;  // no block part: weight 0
  M = fmaxf(M, lb);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    // wave w folds splits w, w + 4, w + 8, ... in ascending order
#pragma unroll
    for (int j = 0; j < FIRST; ++j) {
      const int s = wave + j * NWV;
      if (s < S) {
        const float a = exp2_hw((lp[s] - M) * kLog2e);
        wsum += a;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, val0[j][e], acc[e]);
      }
    }
    int s = wave + FIRST * NWV;
    for (; s + 3 * NWV < S; s += 4 * NWV) {
      float a[4], val[4][PER];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = exp2_hw((lp[s + j * NWV] - M) * kLog2e);
#pragma unroll
        for (int e = 0; e < PER; ++e) val[j][e] = op[(size_t)(s + j * NWV) * D + e];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wsum += a[j];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(a[j], val[j][e], acc[e]);
      }
    }
    for (; s < S; s += NWV) {
      const float a = exp2_hw((lp[s] - M) * kLog2e);
      wsum += a;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, op[(size_t)s * D + e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) part[wave][lane * PER + e] = acc[e];
  if (lane == 0) wpart[wave] = wsum;
  __syncthreads();
  if (wave != 0) return;
  float tot = ((wpart[0] + wpart[1]) + wpart[2]) + wpart[3];
  float res[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane * PER + e;
    res[e] = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
  }
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
template <int D>
__global__ __launch_bounds__(256) void block_merge_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, BlockMask mask, int Hq, int G, int n, float scale_log2,
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int S,
    uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  constexpr int NWV = 4;
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
  constexpr int FIRST = 8;
  float val0[FIRST][PER];
#pragma unroll
  for (int j = 0; j < FIRST; ++j) {
    const int s = wave + j * NWV;
#pragma unroll
    for (int e = 0; e < PER; ++e) val0[j][e] = (s < S) ? op[(size_t)s * D + e] : 0.f;
  }
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
  if (Ms != -INFINITY) {
#pragma unroll
    for (int j = 0; j < FIRST; ++j) {
      const int s = wave + j * NWV;
      if (s < S) {
        const float a = exp2_hw((lp[s] - Ms) * kLog2e);
        wsum += a;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, val0[j][e], acc[e]);
      }
    }
    int s = wave + FIRST * NWV;
    for (; s + 3 * NWV < S; s += 4 * NWV) {
      float a[4], val[4][PER];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = exp2_hw((lp[s + j * NWV] - Ms) * kLog2e);
#pragma unroll
        for (int e = 0; e < PER; ++e) val[j][e] = op[(size_t)(s + j * NWV) * D + e];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wsum += a[j];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(a[j], val[j][e], acc[e]);
      }
    }
    for (; s < S; s += NWV) {
      const float a = exp2_hw((lp[s] - Ms) * kLog2e);
      wsum += a;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, op[(size_t)s * D + e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) part[wave][lane * PER + e] = acc[e];
  if (lane == 0) wpart[wave] = wsum;
  __syncthreads();
  if (wave != 0) return;
  const float lb = lb2 * kLn2;  // finite: a row always sees itself
  const float M = fmaxf(Ms, lb);
  const float fs = (Ms == -INFINITY) ? 0.f : exp2_hw((Ms - M) * kLog2e);
  const float fb = exp2_hw((lb - M) * kLog2e);
  const float tot = fmaf(fs, ((wpart[0] + wpart[1]) + wpart[2]) + wpart[3], fb);
  const float inv = 1.0f / tot;  // tot >= fb = 1 or fs * wsum >= 1
  uint16_t* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane * PER + e;
    const float hs = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
    dst[e] = f32_to_bf16_bits(fmaf(fs, hs, fb * ob[e]) * inv);
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = M + log2_hw(tot) * kLn2;
}

}  // namespace
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)(B * Hq * n));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_blk);
  const uint16_t* vv = static_cast<const uint16_t*>(v_blk);
  uint16_t* o16 = static_cast<uint16_t*>(out);
  if (d == 64)
    hipLaunchKernelGGL((rv::block_merge_kernel<64>), grid, dim3(256), 0, s, qq, kk, vv, mask, Hq,
                       Hq / Hkv, n, scale_log2, o_part, lse_part, S, o16, lse_out);
  else
    hipLaunchKernelGGL((rv::block_merge_kernel<128>), grid, dim3(256), 0, s, qq, kk, vv, mask, Hq,
                       Hq / Hkv, n, scale_log2, o_part, lse_part, S, o16, lse_out);
  if (hipGetLastError() != hipSuccess) return RV_ERR_HIP;
  return RV_OK;
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
  if (d == 64)
    hipLaunchKernelGGL((rv::merge_kernel<64>), grid, dim3(256), 0, s, o_part, lse_part, S, o_blk,
                       lse_blk, o16, lse_out);
  else
    hipLaunchKernelGGL((rv::merge_kernel<128>), grid, dim3(256), 0, s, o_part, lse_part, S, o_blk,
                       lse_blk, o16, lse_out);
  if (hipGetLastError() != hipSuccess) return RV_ERR_HIP;
  return RV_OK;
}
