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

  // V columns of this lane for the first 8 keys, requested up front.
  const uint16_t* vcol = vb + kv0 + lane * PER;
  typedef uint16_t u16xP __attribute__((ext_vector_type(PER)));
  u16xP vpre[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    vpre[j] = (j < n) ? *reinterpret_cast<const u16xP*>(vcol + (size_t)j * D) : u16xP{};

  float s = -INFINITY;
  if (lane < n && ((mask.bits[i] >> lane) & 1ull)) {
    const i32x4* kr = reinterpret_cast<const i32x4*>(kb + kv0 + (size_t)lane * D);
    const i32x4* qr = reinterpret_cast<const i32x4*>(q + row * D);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const i32x4 kk = kr[c];
      const i32x4 qq = qr[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(bf16_lo(qq[e]), bf16_lo(kk[e]), acc[e]);
        acc[e] = fmaf(bf16_hi(qq[e]), bf16_hi(kk[e]), acc[e]);
      }
    }
    s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * scale_log2;
  }
  const float m = wave_max(s);  // finite: a row always sees itself
  const float p = (s == -INFINITY) ? 0.f : exp2_hw(s - m);
  const float l = wave_sum(p);

  // P V over keys in ascending order (masked keys have p = 0).
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float pj = __shfl(p, j < n ? j : 0, 64);
#pragma unroll
    for (int e = 0; e < PER; ++e)
      o[e] = fmaf(j < n ? pj : 0.f, __uint_as_float((uint32_t)vpre[j][e] << 16), o[e]);
  }
  for (int j0 = 8; j0 < n; j0 += 8) {
    u16xP vv[8];
    float pj[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;  // uniform across the wave
      pj[jj] = __shfl(p, j < n ? j : 0, 64);
      vv[jj] = (j < n) ? *reinterpret_cast<const u16xP*>(vcol + (size_t)j * D) : u16xP{};
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int e = 0; e < PER; ++e)
        o[e] = fmaf(j0 + jj < n ? pj[jj] : 0.f, __uint_as_float((uint32_t)vv[jj][e] << 16), o[e]);
  }
  const float inv = 1.0f / l;
  float* op = o_blk + row * D + lane * PER;
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
