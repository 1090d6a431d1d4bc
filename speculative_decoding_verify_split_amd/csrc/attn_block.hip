// spec_attn_block: attention of the verify rows over the draft block's own
// keys under the speculative mask (LongSpec summary, gist.science, section 2.3
// "Fast Tree Attention": only the few speculative tokens need a mask, and that
// part gets a small dedicated kernel).  A chain uses the causal mask (row i
// sees rows j <= i); a tree lets a node see itself and its ancestors.
//
// With at most 64 block keys per row there is no dense contraction worth a
// matrix-core tile, so this runs on the vector ALU in fp32: one wave per
// output row (four rows per workgroup).  Lane j scores block key j (if the
// row's mask bit j is set), the wave reduces max and sum, and then each lane
// owns d/64 output columns of P V.  Reductions use a fixed butterfly and the
// P V sum runs over keys in ascending order, so results are bit-deterministic.

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

__device__ __forceinline__ float bf16_lo(int w) { return __uint_as_float((uint32_t)w << 16); }
__device__ __forceinline__ float bf16_hi(int w) { return __uint_as_float((uint32_t)w & 0xffff0000u); }

template <int D>
__global__ __launch_bounds__(256) void block_kernel(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ kb,
                                                    const uint16_t* __restrict__ vb,
                                                    BlockMask mask, int Hq, int Hkv, int n,
                                                    float scale_log2, int rows,
                                                    float* __restrict__ o_blk,
                                                    float* __restrict__ lse_blk) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  // row = (b * Hq + h) * n + i, the layout of q, o_blk and lse_blk
  const int i = row % n;
  const int bh = row / n;
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  const size_t kv0 = ((size_t)b * Hkv + kvh) * n * D;

  float s = -INFINITY;
  if (lane < n && ((mask.bits[i] >> lane) & 1ull)) {
    const i32x4* kr = reinterpret_cast<const i32x4*>(kb + kv0 + (size_t)lane * D);
    const i32x4* qr = reinterpret_cast<const i32x4*>(q + (size_t)row * D);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const i32x4 kk = kr[c];
      const i32x4 qq = qr[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf16_lo(qq[e]), bf16_lo(kk[e]), acc);
        acc = fmaf(bf16_hi(qq[e]), bf16_hi(kk[e]), acc);
      }
    }
    s = acc * scale_log2;
  }
  const float m = wave_max(s);  // finite: a row always sees itself
  const float p = (s == -INFINITY) ? 0.f : exp2_hw(s - m);
  const float l = wave_sum(p);

  // P V: no data-dependent branch, so the loads of many keys are in flight
  // together (masked keys have p = 0).
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  const uint16_t* vcol = vb + kv0 + lane * PER;
  for (int j0 = 0; j0 < n; j0 += 8) {
    float pj[8], vv[8][PER];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;  // uniform across the wave
      pj[jj] = __shfl(p, j < n ? j : 0, 64);
#pragma unroll
      for (int e = 0; e < PER; ++e)
        vv[jj][e] = (j < n) ? __uint_as_float((uint32_t)vcol[(size_t)j * D + e] << 16) : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = fmaf(j0 + jj < n ? pj[jj] : 0.f, vv[jj][e], o[e]);
  }
  const float inv = 1.0f / l;
  float* op = o_blk + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[e] = o[e] * inv;
  if (lane == 0) lse_blk[row] = (m + log2_hw(l)) * kLn2;
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
  const int rows = B * Hq * n;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)((rows + 3) / 4));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_blk);
  const uint16_t* vv = static_cast<const uint16_t*>(v_blk);
  if (d == 64)
    hipLaunchKernelGGL((rv::block_kernel<64>), grid, dim3(256), 0, s, qq, kk, vv, mask, Hq, Hkv,
                       n, scale_log2, rows, o_blk, lse_blk);
  else
    hipLaunchKernelGGL((rv::block_kernel<128>), grid, dim3(256), 0, s, qq, kk, vv, mask, Hq, Hkv,
                       n, scale_log2, rows, o_blk, lse_blk);
  if (hipGetLastError() != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}
