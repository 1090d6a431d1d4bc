// The history-partial fold shared by the merges (lse_merge.hip) and the
// single-launch verify pass (attn_prefix.hip): a row's S partials are
// log-sum-exp merged (LongSpec summary, gist.science, section 2.3: the parts
// are combined with the log-sum-exp trick) by NWV waves, each folding its
// share of the splits in batches of FB loads in flight.
#pragma once

#include "rv_device.h"

namespace rv {

// A partial's load: plain, or (DEV) a device-scope load that misses any
// stale copy in this XCD's L2, for partials written earlier in the same
// launch by workgroups on other XCDs.
template <bool DEV>
__device__ __forceinline__ float partial_load(const float* p) {
  if constexpr (DEV) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// One wave's share of a row's history partials, s = wave, wave + NWV, ...,
// batch b holding the FB of them from s = wave + b FB NWV.  op points at
// this lane's PER columns of the row's first partial.
template <int D, int NWV, int FB, bool DEV = false>
struct PartialFold {
  static constexpr int PER = D / 64;
  float val[FB][PER];
  float lse[FB];

  // Issues every load of batch b; partials past S read as empty.
  __device__ __forceinline__ void load(const float* __restrict__ op,
                                       const float* __restrict__ lp, int S, int wave, int b) {
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      const int s = wave + (b * FB + j) * NWV;
      lse[j] = s < S ? partial_load<DEV>(lp + s) : -INFINITY;
#pragma unroll
      for (int e = 0; e < PER; ++e) val[j][e] = s < S ? partial_load<DEV>(op + (size_t)s * D + e) : 0.f;
    }
  }

  // acc += a_s O_s and wsum += a_s over batch b in ascending s, with
  // a_s = exp(LSE_s - M) (0 for an empty split, whose O_s is 0).
  __device__ __forceinline__ void add(int S, int wave, int b, float M, float (&acc)[PER],
                                      float& wsum) const {
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      const int s = wave + (b * FB + j) * NWV;
      if (s < S) {
        const float a = exp2_hw((lse[j] - M) * kLog2e);
        wsum += a;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(a, val[j][e], acc[e]);
      }
    }
  }

  // Every batch of this wave, the first already loaded.
  __device__ __forceinline__ void fold(const float* __restrict__ op,
                                       const float* __restrict__ lp, int S, int wave, float M,
                                       float (&acc)[PER], float& wsum) {
    add(S, wave, 0, M, acc, wsum);
    for (int b = 1; wave + b * FB * NWV < S; ++b) {
      load(op, lp, S, wave, b);
      add(S, wave, b, M, acc, wsum);
    }
  }
};

// Fixed-order (left to right) sum of the NWV wave values.
template <int NWV>
__device__ __forceinline__ float wave_order_sum(const float* v, int stride) {
  float t = v[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) t += v[w * stride];
  return t;
}

}  // namespace rv
