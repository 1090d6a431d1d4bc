// lse_merge: log-sum-exp merge of the history partials and the draft-block
// partial (LongSpec summary, gist.science, section 2.3 "Fast Tree Attention":
// the outputs of the two parts are combined with the log-sum-exp trick).
// With M = max_k LSE_k and a_k = exp(LSE_k - M):
//   O = sum_k a_k O_k / sum_k a_k,   LSE = M + log sum_k a_k.
//
// One 4-wave workgroup per output row; the row's S partials are contiguous
// ([row][S][d]).  Wave w folds splits w, w + 4, ... (each step one 4*d-byte
// line read by all 64 lanes, four steps in flight), the four wave sums are
// added in wave order and the block partial last, so the result is
// bit-deterministic.

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
  const float lb = lse_blk[row];
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
  if (M != -INFINITY) {
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

}  // namespace
}  // namespace rv

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
