// Attention of one draft-block row over the block's own keys under the
// speculative mask (LongSpec summary, gist.science, section 2.3 "Fast Tree
// Attention": only the few speculative tokens need a mask).  Shared by the
// block kernel and the fused block + merge kernel.
//
// With at most 64 block keys per row there is no dense contraction worth a
// matrix-core tile, so one wave computes the row on the vector ALU in fp32:
// lane j scores block key j (if bit j of the row's mask is set), the wave
// reduces max and sum with a fixed butterfly, and then each lane owns d/64
// output columns of P V, summed over keys in ascending order.  Results are
// bit-deterministic.
#pragma once

#include "rv_device.h"

namespace rv {

__device__ __forceinline__ float bf16_lo(int w) { return __uint_as_float((uint32_t)w << 16); }
__device__ __forceinline__ float bf16_hi(int w) { return __uint_as_float((uint32_t)w & 0xffff0000u); }

// qrow: the row's query (D bf16); kh, vh: the kv head's block keys and
// values ([n][D] bf16); bits: the row's visibility mask (bit i set for the
// row itself); scale_log2 = sm_scale / ln 2.  Returns this lane's D/64
// normalised output columns (columns lane*D/64 ...) and the base-2 log-sum-
// exp of the scaled scores.  Called by all 64 lanes of a wave.
template <int D>
__device__ __forceinline__ void block_row_attention(const uint16_t* __restrict__ qrow,
                                                    const uint16_t* __restrict__ kh,
                                                    const uint16_t* __restrict__ vh,
                                                    uint64_t bits, int n, float scale_log2,
                                                    float (&o)[D / 64], float& lse2) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  // V columns of this lane for the first kPre keys (a chain of up to 15
  // drafts), requested up front with the K rows, so the row costs one round
  // trip.
  constexpr int kPre = 16;
  const uint16_t* vcol = vh + lane * PER;
  typedef uint16_t u16xP __attribute__((ext_vector_type(PER)));
  u16xP vpre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j)
    vpre[j] = (j < n) ? *reinterpret_cast<const u16xP*>(vcol + (size_t)j * D) : u16xP{};

  float s = -INFINITY;
  if (lane < n && ((bits >> lane) & 1ull)) {
    const i32x4* kr = reinterpret_cast<const i32x4*>(kh + (size_t)lane * D);
    const i32x4* qr = reinterpret_cast<const i32x4*>(qrow);
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
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const float pj = __shfl(p, j < n ? j : 0, 64);
#pragma unroll
    for (int e = 0; e < PER; ++e)
      o[e] = fmaf(j < n ? pj : 0.f, __uint_as_float((uint32_t)vpre[j][e] << 16), o[e]);
  }
  for (int j0 = kPre; j0 < n; j0 += 8) {
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
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] *= inv;
  lse2 = m + log2_hw(l);
}

}  // namespace rv
