// spec_attn_block: attention of the verify rows over the draft block's own
// keys under the speculative mask (LongSpec summary, gist.science, section 2.3
// "Fast Tree Attention": only the few speculative tokens need a mask, and that
// part gets a small dedicated kernel).  A chain uses the causal mask (row i
// sees rows j <= i); a tree lets a node see itself and its ancestors.  One
// wave per output row (four rows per workgroup); the per-row routine is in
// block_row.h.

#include "block_row.h"
#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

// grid (ceil(n / 4), B * Hq): wave w of workgroup x handles block row 4x + w
// of query head h of sequence b (blockIdx.y = b * Hq + h).
template <int D>
__global__ __launch_bounds__(256) void block_kernel(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ kb,
                                                    const uint16_t* __restrict__ vb,
                                                    BlockMask mask, int Hq, int G, int n,
                                                    float scale_log2,
                                                    float* __restrict__ o_blk,
                                                    float* __restrict__ lse_blk) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  const int bh = blockIdx.y;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int Hkv = Hq / G;
  const size_t kv0 = ((size_t)b * Hkv + h / G) * n * D;
  const size_t row = (size_t)bh * n + i;  // layout of q, o_blk and lse_blk
  float o[PER], lse2;
  block_row_attention<D>(q + row * D, kb + kv0, vb + kv0, mask.bits[i], n, scale_log2, o, lse2);
  float* op = o_blk + row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[e] = o[e];
  if (lane == 0) lse_blk[row] = lse2 * kLn2;
}

}  // namespace
}  // namespace rv

extern "C" rv_status spec_attn_block(const void* q, const void* k_blk, const void* v_blk,
                                     const int32_t* parent_host, int B, int Hq, int Hkv, int n,
                                     int d, float sm_scale, float* o_blk, float* lse_blk,
                                     void* stream) {
  rv::BlockMask mask;
  rv_status st = rv::check_block(q, k_blk, v_blk, parent_host, B, Hq, Hkv, n, d, sm_scale, o_blk,
                                 lse_blk, &mask);
  if (st != RV_OK) return st;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)((n + 3) / 4), (unsigned)(B * Hq));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_blk);
  const uint16_t* vv = static_cast<const uint16_t*>(v_blk);
  if (d == 64)
    hipLaunchKernelGGL((rv::block_kernel<64>), grid, dim3(256), 0, s, qq, kk, vv, mask, Hq, Hq / Hkv,
                       n, scale_log2, o_blk, lse_blk);
  else
    hipLaunchKernelGGL((rv::block_kernel<128>), grid, dim3(256), 0, s, qq, kk, vv, mask, Hq, Hq / Hkv,
                       n, scale_log2, o_blk, lse_blk);
  if (hipGetLastError() != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}
