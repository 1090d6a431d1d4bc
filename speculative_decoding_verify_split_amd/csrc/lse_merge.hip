// lse_merge: log-sum-exp merge of the history partials and the draft-block
// partial (LongSpec summary, gist.science, section 2.3 "Fast Tree Attention":
// the outputs of the two parts are combined with the log-sum-exp trick).
// With M = max_k LSE_k and a_k = exp(LSE_k - M):
//   O = sum_k a_k O_k / sum_k a_k,   LSE = M + log sum_k a_k.
//
// One wave per output row; the row's S partials are contiguous
// ([row][S][d]), so each step reads one 4*d-byte line with all 64 lanes.
// Partials are combined in a fixed order (splits ascending, then the block),
// so the result is bit-deterministic.

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int S,
                                                    const float* __restrict__ o_blk,
                                                    const float* __restrict__ lse_blk, int rows,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* lp = lse_part + (size_t)row * S;
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s]);
  M = wave_max(M);
  const float lb = lse_blk[row];
  M = fmaxf(M, lb);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    const float* op = o_part + (size_t)row * S * D + lane * PER;
    int s = 0;
    for (; s + 4 <= S; s += 4) {
      float a[4], val[4][PER];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = exp2_hw((lp[s + j] - M) * kLog2e);
#pragma unroll
        for (int e = 0; e < PER; ++e) val[j][e] = op[(size_t)(s + j) * D + e];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wsum += a[j];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(a[j], val[j][e], acc[e]);
      }
    }
    for (; s < S; ++s) {
      const float a = exp2_hw((lp[s] - M) * kLog2e);
      wsum += a;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, op[(size_t)s * D + e], acc[e]);
    }
    const float a = exp2_hw((lb - M) * kLog2e);
    wsum += a;
    const float* bp = o_blk + (size_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, bp[e], acc[e]);
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  uint16_t* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = f32_to_bf16_bits(acc[e] * inv);
  if (lse_out != nullptr && lane == 0)
    lse_out[row] = (M == -INFINITY) ? -INFINITY : M + log2_hw(wsum) * kLn2;
}

}  // namespace
}  // namespace rv

extern "C" rv_status lse_merge(const float* o_part, const float* lse_part, int S,
                               const float* o_blk, const float* lse_blk, int B, int Hq, int n,
                               int d, void* out, float* lse_out, void* stream) {
  rv_status st = rv::check_merge(o_part, lse_part, S, o_blk, lse_blk, B, Hq, n, d, out);
  if (st != RV_OK) return st;
  const int rows = B * Hq * n;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)((rows + 3) / 4));
  uint16_t* o16 = static_cast<uint16_t*>(out);
  if (d == 64)
    hipLaunchKernelGGL((rv::merge_kernel<64>), grid, dim3(256), 0, s, o_part, lse_part, S, o_blk,
                       lse_blk, rows, o16, lse_out);
  else
    hipLaunchKernelGGL((rv::merge_kernel<128>), grid, dim3(256), 0, s, o_part, lse_part, S, o_blk,
                       lse_blk, rows, o16, lse_out);
  if (hipGetLastError() != hipSuccess) return RV_ERR_HIP;
  return RV_OK;
}
