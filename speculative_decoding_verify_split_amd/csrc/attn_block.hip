// spec_attn_block: attention of the verify rows over the draft block's own
// keys under the speculative mask (LongSpec summary, gist.science, section 2.3
// "Fast Tree Attention": only the few speculative tokens need a mask, and that
// part is handled by a small dedicated kernel).  A chain uses the causal mask
// (row i sees rows j <= i); a tree lets a node see itself and its ancestors.
//
// The work is tiny (n <= 64 rows and keys per head), so it runs on the vector
// ALU in fp32: one workgroup per (query head, sequence), one lane per row, the
// head's block K/V staged once in LDS (bf16) and read by broadcast.

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

template <int D>
__global__ __launch_bounds__(64) void block_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ kb,
                                                   const uint16_t* __restrict__ vb,
                                                   BlockMask mask, int Hq, int Hkv, int n,
                                                   float scale_log2, float* __restrict__ o_blk,
                                                   float* __restrict__ lse_blk) {
  __shared__ uint16_t ks[RV_MAX_BLOCK_ROWS * D];
  __shared__ uint16_t vs[RV_MAX_BLOCK_ROWS * D];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int kvh = h / (Hq / Hkv);
  const size_t kv_off = ((size_t)b * Hkv + kvh) * n * D;
  for (int idx = threadIdx.x; idx < n * D; idx += 64) {
    ks[idx] = kb[kv_off + idx];
    vs[idx] = vb[kv_off + idx];
  }
  __syncthreads();
  const int i = threadIdx.x;
  if (i >= n) return;

  auto widen = [](uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); };
  const uint16_t* qp = q + (((size_t)b * Hq + h) * n + i) * D;
  float qr[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = widen(qp[c]);
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const uint64_t vis = mask.bits[i];
  for (int j = 0; j < n; ++j) {
    if (!((vis >> j) & 1ull)) continue;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) dot = fmaf(qr[c], widen(ks[j * D + c]), dot);
    const float x = dot * scale_log2;
    const float mn = fmaxf(m, x);
    const float a = exp2_hw(m - mn);
    const float p = exp2_hw(x - mn);
    l = l * a + p;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = fmaf(p, widen(vs[j * D + c]), o[c] * a);
    m = mn;
  }
  // A row always sees itself, so l > 0.
  float* op = o_blk + (((size_t)b * Hq + h) * n + i) * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < D; c += 4)
    *reinterpret_cast<f32x4*>(op + c) = f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
  lse_blk[((size_t)b * Hq + h) * n + i] = (m + log2_hw(l)) * kLn2;
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
  dim3 grid((unsigned)Hq, (unsigned)B);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_blk);
  const uint16_t* vv = static_cast<const uint16_t*>(v_blk);
  if (d == 64)
    hipLaunchKernelGGL((rv::block_kernel<64>), grid, dim3(64), 0, s, qq, kk, vv, mask, Hq, Hkv, n,
                       scale_log2, o_blk, lse_blk);
  else
    hipLaunchKernelGGL((rv::block_kernel<128>), grid, dim3(64), 0, s, qq, kk, vv, mask, Hq, Hkv,
                       n, scale_log2, o_blk, lse_blk);
  if (hipGetLastError() != hipSuccess) return RV_ERR_HIP;
  return RV_OK;
}
