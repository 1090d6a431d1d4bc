// Device helpers of the vocabulary passes (rapid_accept and
// rapid_tree_accept): vector loads of row runs, workgroup reductions and
// scans with fixed orders, the log-sum-exp pair merge, the per-entry p, q and
// s of the retrieval-augmented target (RAPID blog post, leeon-k.github.io,
// section 2.4), and the inverse-CDF draw over published chunk weights.
#pragma once

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

constexpr int TPB = kVocabThreads;

// Chunk draw-weight slots.  Each chunk of the decide pass publishes its two
// weights as one 64-bit word with one device-scope atomic store; the pass's
// first kernel sets every slot to kSlotEmpty, a bit pattern no published pair
// takes, so the workgroup that draws can tell a slot whose store has not
// landed yet and read it again.  A published slot holds (first weight, second
// weight) in its (low, high) halves.
constexpr uint64_t kSlotEmpty = ~0ull;
constexpr uint64_t kSlotWaitTicks = 10000000;  // 100 ms of the 100 MHz clock

__device__ __forceinline__ uint64_t pack_slot(float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  // (only a NaN pair with every bit set can collide; publish it as another NaN)
  return v == kSlotEmpty ? 0x7FC000007FC00000ull : v;
}

// Publishes one chunk's weights, then counts its arrival; returns the count
// before this one.  The slot store is issued before the increment (the empty
// asm keeps the compiler from moving it), so once the count shows every other
// chunk arrived, every slot's store has been issued and will land.
__device__ __forceinline__ uint32_t publish_and_arrive(uint64_t* slot, float a, float b,
                                                       uint32_t* counter) {
  __hip_atomic_store(slot, pack_slot(a, b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::: "memory");
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// x[e] = row[start + e] for e < N (zero at or past V).
template <bool VEC, int N>
__device__ __forceinline__ void load_run(const float* __restrict__ row, int V, int start,
                                         float (&x)[N]) {
  static_assert(N % 4 == 0, "runs are whole float4s");
  if (VEC && start + N <= V) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row + start);
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      const f32x4 v = p[j];
      x[4 * j + 0] = v[0];
      x[4 * j + 1] = v[1];
      x[4 * j + 2] = v[2];
      x[4 * j + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] = (start + e < V) ? row[start + e] : 0.f;
  }
}

__device__ float block_max(float v) {
  __shared__ float sh[TPB / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return r;
}

__device__ float block_sum(float v) {
  __shared__ float sh[TPB / 64];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return r;
}

// Two workgroup sums with one pair of barriers.
__device__ float2 block_sum2(float a, float b) {
  __shared__ float sh[2][TPB / 64];
  a = wave_sum(a);
  b = wave_sum(b);
  if ((threadIdx.x & 63) == 0) {
    sh[0][threadIdx.x >> 6] = a;
    sh[1][threadIdx.x >> 6] = b;
  }
  __syncthreads();
  const float2 r = make_float2((sh[0][0] + sh[0][1]) + (sh[0][2] + sh[0][3]),
                               (sh[1][0] + sh[1][1]) + (sh[1][2] + sh[1][3]));
  __syncthreads();
  return r;
}

// Inclusive prefix sums of (v.x, v.y) over the workgroup in thread order:
// a scan inside each wave, then the wave totals added in wave order.  *total
// receives the workgroup sums, which equal the last thread's inclusive
// values exactly (the same additions in the same order).
__device__ float2 block_incl_scan2(float2 v, float2* total) {
  __shared__ float2 sh[TPB / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float2 in = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float a = __shfl_up(in.x, o, 64);
    const float b = __shfl_up(in.y, o, 64);
    if (lane >= o) {
      in.x += a;
      in.y += b;
    }
  }
  if (lane == 63) sh[wave] = in;
  __syncthreads();
  float2 run = make_float2(0.f, 0.f), off = run;
#pragma unroll
  for (int w = 0; w < TPB / 64; ++w) {
    if (w == wave) off = run;
    run.x += sh[w].x;
    run.y += sh[w].y;
  }
  __syncthreads();
  *total = run;
  return make_float2(off.x + in.x, off.y + in.y);
}

// Sets the cd draw-weight slots of one sequence to kSlotEmpty, spread over
// the workgroups of a grid's x dimension (the pass's first kernel).
__device__ __forceinline__ void clear_slots(uint64_t* __restrict__ slots, int cd) {
  for (int i = blockIdx.x * TPB + threadIdx.x; i < cd; i += gridDim.x * TPB)
    slots[i] = kSlotEmpty;
}

// Index of the first thread with `hit` and of the last thread with `pos`
// (-1 if none); every thread gets the same pair.
__device__ int2 block_first_last(bool hit, bool pos) {
  __shared__ int sf[TPB / 64], sl[TPB / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t h = __ballot(hit), p = __ballot(pos);
  if (lane == 0) {
    sf[wave] = h ? wave * 64 + (int)__ffsll((long long)h) - 1 : -1;
    sl[wave] = p ? wave * 64 + 63 - (int)__builtin_clzll(p) : -1;
  }
  __syncthreads();
  int f = -1, l = -1;
#pragma unroll
  for (int w = 0; w < TPB / 64; ++w) {
    if (f < 0) f = sf[w];
    if (sl[w] >= 0) l = sl[w];
  }
  __syncthreads();
  return make_int2(f, l);
}

// Merge two (max, sum-of-2^(x - max)) pairs.  Symmetric in its arguments, so
// both lanes of a butterfly step obtain bit-identical results.
__device__ __forceinline__ void lse_pair_merge(float& m, float& l, float mo, float lo) {
  const float mn = fmaxf(m, mo);
  const float a = (m == -INFINITY) ? 0.f : l * exp2_hw(m - mn);
  const float c = (mo == -INFINITY) ? 0.f : lo * exp2_hw(mo - mn);
  l = a + c;
  m = mn;
}

// Base-2 log-sum-exp of a row from its per-chunk (max, sum) pairs, reduced by
// a group of `width` lanes (16 or 64, aligned) in one pass: lane j of the
// group folds chunks j, j + width, ... in order, then the group merges with
// symmetric lane pairings (DPP quad permutes and mirrors, then the row-swap
// permutes).  Every lane of the group returns the same value.
template <int width>
__device__ __forceinline__ float group_combine(const float* __restrict__ st, int C, int j,
                                               float* max_out = nullptr) {
  static_assert(width == 16 || width == 64, "group width");
  float m = -INFINITY, l = 0.f;
  for (int c = j; c < C; c += width) lse_pair_merge(m, l, st[2 * c], st[2 * c + 1]);
  lse_pair_merge(m, l, dpp_f<kDppXor1>(m), dpp_f<kDppXor1>(l));
  lse_pair_merge(m, l, dpp_f<kDppXor2>(m), dpp_f<kDppXor2>(l));
  lse_pair_merge(m, l, dpp_f<kDppHalfMirror>(m), dpp_f<kDppHalfMirror>(l));
  lse_pair_merge(m, l, dpp_f<kDppMirror>(m), dpp_f<kDppMirror>(l));
  if constexpr (width == 64) {
    float2 a = swap16(m), c = swap16(l);
    m = a.x; l = c.x;
    lse_pair_merge(m, l, a.y, c.y);
    a = swap32(m);
    c = swap32(l);
    m = a.x; l = c.x;
    lse_pair_merge(m, l, a.y, c.y);
  }
  if (max_out) *max_out = m;
  return m + log2_hw(l);
}

// Sum of st[c], c < C, by a 16-lane group: lane j adds c = j, j + 16, ... in
// order, then the group adds by symmetric pairings; all 16 lanes agree.
__device__ __forceinline__ float group16_sum(const float* __restrict__ st, int C, int j) {
  float v = 0.f;
  for (int c = j; c < C; c += 16) v += st[c];
  return row16_sum(v);
}

// p, q and s/ln2 of one vocabulary entry.  x2 = z/T/ln2, lz = log2 sum 2^x2,
// likewise for y; s2 = (z/T + eta (q - p)) / ln2.
__device__ __forceinline__ void pq_s(float zv, float yv, float invT2, float eta2, float lz,
                                     float ly, float& p, float& q, float& s2) {
  const float x2 = zv * invT2;
  p = exp2_hw(x2 - lz);
  q = exp2_hw(yv * invT2 - ly);
  s2 = fmaf(eta2, q - p, x2);
}

// Inverse CDF of one row with the caller's uniform, run by one whole
// workgroup, over the cd chunks of TPB * PER elements whose weights (both
// kinds) the pass has published in slots ws[c].  Chunk level: a scan
// of the chunk weights (kind 1 only if the kind-0 weights have no mass at
// all, which exact arithmetic rules out at a rejected row) picks the first
// chunk of positive weight whose running total exceeds u * W; thread level:
// the same over the chunk's thread totals; element level: the same inside the
// thread.  Where rounding leaves no such unit, the last unit of positive
// weight is taken (and every lower level then takes its last positive unit,
// i.e. the largest id of positive weight).  wfun(z, y, kind) is the weight
// of one element from its target and drafter logits (yrow may be null: y is
// then 0); the chosen id goes to *out_slot.
template <bool VEC, int PER, typename WF>
__device__ void draw_from_chunks(const float* __restrict__ zrow, const float* __restrict__ yrow,
                                 float u_val, int V, int cd, const uint64_t* __restrict__ ws,
                                 int32_t* __restrict__ out_slot, WF wfun) {
  __shared__ float sh_base;
  // Every chunk's slot store has been issued (publish_and_arrive); read each
  // slot with device-scope atomic loads until its store has landed.  The
  // wait is also bounded in time (kSlotWaitTicks of the 100 MHz clock, far
  // beyond any store's latency), so that the pass ends even if a store were
  // ever lost; an empty slot then counts as no weight.
  auto chunk_w = [&](int i) {
    if (i >= cd) return make_float2(0.f, 0.f);
    uint64_t v = __hip_atomic_load(ws + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v == kSlotEmpty) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      do {
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(ws + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } while (v == kSlotEmpty && __builtin_amdgcn_s_memrealtime() - t0 < kSlotWaitTicks);
      if (v == kSlotEmpty) v = 0;
    }
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
  };
  // Totals of both kinds, block of TPB chunks by block.  The last block's
  // values stay in registers (with cd <= TPB the only block).
  float2 wv = make_float2(0.f, 0.f), incl = wv, tot = wv, carry = wv;
  for (int c0 = 0; c0 < cd; c0 += TPB) {
    carry.x += tot.x;
    carry.y += tot.y;
    wv = chunk_w(c0 + threadIdx.x);
    incl = block_incl_scan2(wv, &tot);
  }
  const float2 W2 = make_float2(carry.x + tot.x, carry.y + tot.y);
  const int kind = W2.x > 0.f ? 0 : 1;
  const float tau = u_val * (kind ? W2.y : W2.x);

  int pick = -1, last = -1;
  float tau_c = INFINITY;
  float run = 0.f;
  for (int c0 = 0; c0 < cd; c0 += TPB) {
    if (cd > TPB) {
      wv = chunk_w(c0 + threadIdx.x);
      incl = block_incl_scan2(wv, &tot);
    }
    const float wk = kind ? wv.y : wv.x;
    const float ik = run + (kind ? incl.y : incl.x);
    const int2 fl = block_first_last(wk > 0.f && ik > tau, wk > 0.f);
    if (fl.x >= 0) {
      if ((int)threadIdx.x == fl.x) sh_base = ik - wk;
      __syncthreads();
      pick = c0 + fl.x;
      tau_c = tau - sh_base;
      break;
    }
    if (fl.y >= 0) last = c0 + fl.y;
    run += kind ? tot.y : tot.x;
  }
  if (pick < 0) pick = last < 0 ? 0 : last;  // tau_c stays infinite

  const int start = pick * (TPB * PER) + threadIdx.x * PER;
  float zx[PER], yx[PER], w[PER];
  load_run<VEC>(zrow, V, start, zx);
  if (yrow != nullptr)
    load_run<VEC>(yrow, V, start, yx);
  else
#pragma unroll
    for (int e = 0; e < PER; ++e) yx[e] = 0.f;
  float tsum = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    w[e] = (start + e < V) ? wfun(zx[e], yx[e], kind) : 0.f;
    tsum += w[e];
  }
  float2 ttot;
  const float tincl = block_incl_scan2(make_float2(tsum, 0.f), &ttot).x;
  const int2 fl = block_first_last(tsum > 0.f && tincl > tau_c, tsum > 0.f);
  const int sel = fl.x >= 0 ? fl.x : (fl.y >= 0 ? fl.y : 0);
  if ((int)threadIdx.x != sel) return;
  const float tau_l = fl.x >= 0 ? tau_c - (tincl - tsum) : INFINITY;
  float acc = 0.f;
  int k = -1, klast = -1;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (w[e] > 0.f) {
      if (k < 0 && acc + w[e] > tau_l) k = e;
      klast = e;
    }
    acc += w[e];
  }
  if (k < 0) k = klast < 0 ? 0 : klast;
  int tok = start + k;
  if (tok >= V) tok = V - 1;
  *out_slot = tok;
}


}  // namespace
}  // namespace rv
