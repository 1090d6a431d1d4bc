// rapid_accept: RAPID's acceptance over the vocabulary (RAPID blog post,
// leeon-k.github.io: section 2.1, the acceptance test r <= min(1, p(x)/q(x))
// and the residual draw from norm(max(p - q, 0)); section 2.3, the test
// against the full-context target; section 2.4, the retrieval-augmented target
// p_hat = softmax(z/T + eta (q - p)) used in place of p at inference).
//
// Each row is a V-long fp32 stream (V ~ 1.3e5), so the pass is bandwidth-
// and latency-bound; every row is cut into 4096-element chunks, one
// 256-thread workgroup per chunk (16 contiguous elements per thread), and
// cross-chunk results go through a small workspace:
//   stats_kernel   (chunk, row, b): max and sum of 2^(x - max) of z/T (rows
//                  0..gamma) and y/T (rows 0..gamma-1), base-2 units
//   phat_kernel    (chunk, t, b):   the same for s = z/T + eta (q - p)
//   tail_kernel    (chunk, t, b):   only with RV_ACCEPT_TAIL_PRESERVE (blog
//                  section 2.4's tail rule): per chunk, the sum of the
//                  tail-adjusted row (p_hat where p_hat >= 0.1 max p_hat,
//                  p elsewhere), from which decide_kernel renormalises
//   decide_kernel  (chunk, b):      every chunk recomputes the gamma ratios
//                  min(1, p_hat_t[x_t]/q_t[x_t]) and the first-reject cut t*;
//                  chunk 0 writes n_accept, the accepted tokens and the
//                  ratios; every chunk writes its share of the draw weights
//                  (max(p_hat - q, 0) at t* < gamma, or with
//                  RV_ACCEPT_PRINTED_RESIDUAL section 2.4's printed
//                  max(p - min(p_hat, q), 0); p_gamma otherwise) and,
//                  on request, p_hat.  The last chunk to finish (one
//                  per-sequence arrival counter) then draws the token by
//                  inverse CDF with the caller's uniform: chunk -> wave ->
//                  lane -> element, each level taking the first unit whose
//                  running total exceeds the target.
// Every reduction has a fixed order and the counter only decides which
// workgroup runs the draw, so results are bit-exact run to run; no
// workgroup ever waits for another.

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

constexpr int TPB = kVocabThreads;
constexpr int PER = kVocabPerThread;
constexpr int CH = kVocabChunk;

template <bool VEC>
__device__ __forceinline__ void load_run(const float* __restrict__ row, int V, int start,
                                         float (&x)[PER]) {
  if (VEC && start + PER <= V) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row + start);
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const f32x4 v = p[j];
      x[4 * j + 0] = v[0];
      x[4 * j + 1] = v[1];
      x[4 * j + 2] = v[2];
      x[4 * j + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] = (start + e < V) ? row[start + e] : 0.f;
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

template <bool VEC>
__global__ __launch_bounds__(TPB) void stats_kernel(const float* __restrict__ z,
                                                    const float* __restrict__ y, int gamma, int V,
                                                    float invT2, int C, float* __restrict__ zstat,
                                                    float* __restrict__ ystat,
                                                    uint32_t* __restrict__ arrivals) {
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  // The decide kernel counts chunk arrivals per sequence; start from zero on
  // every call (the workspace is not assumed to be initialised).
  if (c == 0 && r == 0 && threadIdx.x == 0) arrivals[b] = 0u;
  const float* row;
  float* dst;
  if (r <= gamma) {
    row = z + ((size_t)b * (gamma + 1) + r) * V;
    dst = zstat + (((size_t)b * (gamma + 1) + r) * C + c) * 2;
  } else {
    const int t = r - gamma - 1;
    row = y + ((size_t)b * gamma + t) * V;
    dst = ystat + (((size_t)b * gamma + t) * C + c) * 2;
  }
  const int start = c * CH + threadIdx.x * PER;
  float x[PER];
  load_run<VEC>(row, V, start, x);
  float tm = -INFINITY;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    x[e] = (start + e < V) ? x[e] * invT2 : -INFINITY;
    tm = fmaxf(tm, x[e]);
  }
  const float cm = block_max(tm);
  float ts = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) ts += exp2_hw(x[e] - cm);
  const float cs = block_sum(ts);
  if (threadIdx.x == 0) {
    dst[0] = cm;
    dst[1] = cs;
  }
}

// grid (C, gamma + 1, B).  Rows t < gamma: chunk stats of s; chunk 0 also
// publishes the row's z and y log-sum-exps.  Row gamma: chunk 0 publishes
// the last target row's log-sum-exp (for the bonus draw).
template <bool VEC>
__global__ __launch_bounds__(TPB) void phat_kernel(const float* __restrict__ z,
                                                   const float* __restrict__ y, int gamma, int V,
                                                   float invT2, float eta2, int C,
                                                   const float* __restrict__ zstat,
                                                   const float* __restrict__ ystat,
                                                   float* __restrict__ sstat,
                                                   float* __restrict__ rowtab) {
  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  float* rt = rowtab + (size_t)b * 2 * (gamma + 1);
  if (t == gamma) {
    if (c == 0 && threadIdx.x < 64) {
      const float lz = group_combine<64>(zstat + ((size_t)b * (gamma + 1) + t) * C * 2, C, lane);
      if (lane == 0) rt[t] = lz;
    }
    return;
  }
  __shared__ float sh_l[2];
  if (threadIdx.x < 64) {
    const float lz = group_combine<64>(zstat + ((size_t)b * (gamma + 1) + t) * C * 2, C, lane);
    const float ly = group_combine<64>(ystat + ((size_t)b * gamma + t) * C * 2, C, lane);
    if (lane == 0) {
      sh_l[0] = lz;
      sh_l[1] = ly;
      if (c == 0) {
        rt[t] = lz;
        rt[(gamma + 1) + t] = ly;
      }
    }
  }
  const float* zrow = z + ((size_t)b * (gamma + 1) + t) * V;
  const float* yrow = y + ((size_t)b * gamma + t) * V;
  const int start = c * CH + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(zrow, V, start, zx);
  load_run<VEC>(yrow, V, start, yx);
  __syncthreads();
  const float lz = sh_l[0], ly = sh_l[1];
  float s2[PER];
  float tm = -INFINITY;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float p, q, s;
    pq_s(zx[e], yx[e], invT2, eta2, lz, ly, p, q, s);
    s2[e] = (start + e < V) ? s : -INFINITY;
    tm = fmaxf(tm, s2[e]);
  }
  const float cm = block_max(tm);
  float ts = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) ts += exp2_hw(s2[e] - cm);
  const float cs = block_sum(ts);
  if (threadIdx.x == 0) {
    float* dst = sstat + (((size_t)b * gamma + t) * C + c) * 2;
    dst[0] = cm;
    dst[1] = cs;
  }
}

// log2(0.1): the tail rule keeps p_hat_k when p_hat_k >= 0.1 max p_hat, i.e.
// when s_k >= max s + log2(0.1) in base-2 units.
constexpr float kLog2Tenth = -3.321928094887362f;

// Row constants of one sequence in LDS: base-2 LSEs of z/T, y/T and s, and
// for the tail rule each row's keep threshold on s and 1 / (sum of the
// adjusted p_hat).
struct RowLse {
  float lz[kMaxGamma + 1];
  float ly[kMaxGamma];
  float ls[kMaxGamma];
  float thr[kMaxGamma];
  float zinv[kMaxGamma];
  unsigned flags;
};

// The (possibly tail-adjusted) p_hat of one entry of draft row t.
__device__ __forceinline__ float p_hat_entry(float p, float s2, int t, const RowLse& rc) {
  const float ph = exp2_hw(s2 - rc.ls[t]);
  if (!(rc.flags & RV_ACCEPT_TAIL_PRESERVE)) return ph;
  return (s2 >= rc.thr[t] ? ph : p) * rc.zinv[t];
}

// Draw weight of one entry at row ts: the residual (kind 0) or p_hat itself
// (kind 1) for a rejected draft row, p_gamma for the bonus row.  The
// residual is max(p_hat - q, 0), or with RV_ACCEPT_PRINTED_RESIDUAL
// max(p - min(p_hat, q), 0).
__device__ __forceinline__ float draw_weight(float zv, float yv, int ts, int gamma, int kind,
                                             float invT2, float eta2, const RowLse& rc) {
  if (ts == gamma) return exp2_hw(zv * invT2 - rc.lz[gamma]);
  float p, q, s2;
  pq_s(zv, yv, invT2, eta2, rc.lz[ts], rc.ly[ts], p, q, s2);
  const float ph = p_hat_entry(p, s2, ts, rc);
  if (kind != 0) return ph;
  return (rc.flags & RV_ACCEPT_PRINTED_RESIDUAL) ? fmaxf(p - fminf(ph, q), 0.f)
                                                  : fmaxf(ph - q, 0.f);
}

// grid (C, gamma, B), RV_ACCEPT_TAIL_PRESERVE only: chunk sums of the
// unnormalised tail-adjusted p_hat (p_hat where s >= max s + log2 0.1, else
// p).  The row's LSE and max of s come from the same 16-lane combine the
// decide kernel uses, so both kernels classify every entry identically.
template <bool VEC>
__global__ __launch_bounds__(TPB) void tail_kernel(const float* __restrict__ z,
                                                   const float* __restrict__ y, int gamma, int V,
                                                   float invT2, float eta2, int C,
                                                   const float* __restrict__ sstat,
                                                   const float* __restrict__ rowtab,
                                                   float* __restrict__ tstat) {
  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  __shared__ float sh[4];
  const float* rt = rowtab + (size_t)b * 2 * (gamma + 1);
  if (threadIdx.x < 16) {
    float ms;
    const float ls = group_combine<16>(sstat + ((size_t)b * gamma + t) * C * 2, C,
                                       threadIdx.x, &ms);
    if (threadIdx.x == 0) {
      sh[0] = ls;
      sh[1] = ms + kLog2Tenth;
      sh[2] = rt[t];
      sh[3] = rt[(gamma + 1) + t];
    }
  }
  const int start = c * CH + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(z + ((size_t)b * (gamma + 1) + t) * V, V, start, zx);
  load_run<VEC>(y + ((size_t)b * gamma + t) * V, V, start, yx);
  __syncthreads();
  const float ls = sh[0], thr = sh[1], lz = sh[2], ly = sh[3];
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float p, q, s2;
    pq_s(zx[e], yx[e], invT2, eta2, lz, ly, p, q, s2);
    if (start + e < V) acc += (s2 >= thr) ? exp2_hw(s2 - ls) : p;
  }
  const float cs = block_sum(acc);
  if (threadIdx.x == 0) tstat[((size_t)b * gamma + t) * C + c] = cs;
}

// Inverse CDF of the draw row ts of sequence b with the caller's uniform:
// chunk -> wave -> lane -> element, each level taking the first unit of
// positive weight whose running total exceeds the target; if rounding leaves
// none, the last unit of positive weight (and every lower level then takes
// its last positive unit, i.e. the largest id of positive weight).  Run by
// one whole workgroup; wsh is LDS for the 2 C chunk weights.
template <bool VEC>
__device__ void draw_row(const float* __restrict__ z, const float* __restrict__ y,
                         const float* __restrict__ u, int b, int ts, int gamma, int V,
                         float invT2, float eta2, int C, const RowLse& rc,
                         const float* __restrict__ wsum, float* wsh,
                         int32_t* __restrict__ out_tokens) {
  __shared__ int sh_chunk, sh_kind;
  __shared__ float sh_tau;
  __shared__ float wtot[TPB / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // The chunk weights were published by the other workgroups before their
  // arrival was counted; read them past the caches.
  const float* ws = wsum + (size_t)b * C * 2;
  for (int i = threadIdx.x; i < 2 * C; i += TPB) wsh[i] = __builtin_nontemporal_load(ws + i);
  const float u_ts = u[(size_t)b * (gamma + 1) + ts];
  __syncthreads();

  if (wave == 0) {
    // Chunk level, one wave: an inclusive scan of the chunk weights in
    // blocks of 64 (fixed pattern), then the first chunk of positive weight
    // whose running total exceeds u * W.  kind 1 (p_hat itself) only if a
    // rejected row has no residual mass, which exact arithmetic rules out.
    int kind = 0;
    float W = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
      kind = pass;
      float carry = 0.f;
      for (int c0 = 0; c0 < C; c0 += 64) {
        const int c = c0 + lane;
        float incl = (c < C) ? wsh[2 * c + kind] : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const float v = __shfl_up(incl, o, 64);
          if (lane >= o) incl += v;
        }
        carry += __shfl(incl, 63, 64);
      }
      W = carry;
      if (W > 0.f) break;
    }
    const float tau = u_ts * W;
    float carry = 0.f;
    int pick = -1, last = -1;
    float pick_base = 0.f;
    for (int c0 = 0; c0 < C && pick < 0; c0 += 64) {
      const int c = c0 + lane;
      const float wc = (c < C) ? wsh[2 * c + kind] : 0.f;
      float incl = wc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const float excl = carry + (incl - wc);
      const uint64_t hit = __ballot(wc > 0.f && carry + incl > tau);
      const uint64_t pos = __ballot(wc > 0.f);
      if (hit) {
        const int lsel = (int)__ffsll((long long)hit) - 1;
        pick = c0 + lsel;
        pick_base = __shfl(excl, lsel, 64);
      } else if (pos) {
        last = c0 + 63 - (int)__builtin_clzll(pos);
      }
      carry += __shfl(incl, 63, 64);
    }
    float tau_c = tau - pick_base;
    if (pick < 0) {  // rounding: the last chunk with weight, its last positive id
      pick = last < 0 ? 0 : last;
      tau_c = INFINITY;
    }
    if (lane == 0) {
      sh_chunk = pick;
      sh_kind = kind;
      sh_tau = tau_c;
    }
  }
  __syncthreads();
  const int chunk = sh_chunk, kind = sh_kind;
  const float tau_c = sh_tau;
  const int start = chunk * CH + threadIdx.x * PER;
  float zx[PER], yx[PER], w[PER];
  load_run<VEC>(z + ((size_t)b * (gamma + 1) + ts) * V, V, start, zx);
  if (ts < gamma)
    load_run<VEC>(y + ((size_t)b * gamma + ts) * V, V, start, yx);
  else
#pragma unroll
    for (int e = 0; e < PER; ++e) yx[e] = 0.f;
  float tsum = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    w[e] = (start + e < V) ? draw_weight(zx[e], yx[e], ts, gamma, kind, invT2, eta2, rc) : 0.f;
    tsum += w[e];
  }
  // Inclusive scan of the thread totals inside each wave (fixed pattern).
  float incl = tsum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  // Wave level (same arithmetic in every thread).
  float tau = tau_c, base = 0.f;
  int wsel = -1, wlast = -1;
  float wlast_base = 0.f;
  for (int ww = 0; ww < TPB / 64; ++ww) {
    const float wt = wtot[ww];
    if (wt > 0.f) {
      if (base + wt > tau) {
        wsel = ww;
        break;
      }
      wlast = ww;
      wlast_base = base;
    }
    base += wt;
  }
  if (wsel < 0) {
    wsel = wlast < 0 ? 0 : wlast;
    base = wlast_base;
    tau = INFINITY;
  }
  if (wave != wsel) return;
  const float tau_w = tau - base;
  // Lane level.
  const uint64_t hit = __ballot(tsum > 0.f && incl > tau_w);
  int lsel;
  float tau_l;
  const float excl = incl - tsum;
  if (hit) {
    lsel = (int)__ffsll((long long)hit) - 1;
    tau_l = tau_w - __shfl(excl, lsel, 64);
  } else {
    const uint64_t pos = __ballot(tsum > 0.f);
    lsel = pos ? 63 - (int)__builtin_clzll(pos) : 0;
    tau_l = INFINITY;
  }
  if (lane != lsel) return;
  // Element level.
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
  out_tokens[(size_t)b * (gamma + 1) + ts] = tok;
}

// grid (C, B).  Every chunk recomputes the row LSEs of s (16 lanes per row,
// all rows at once), the ratios and the first-reject cut, then writes its
// share of the draw weights; chunk 0 writes the per-sequence outputs.
template <bool VEC>
__global__ __launch_bounds__(TPB) void decide_kernel(
    const float* __restrict__ z, const float* __restrict__ y, const int32_t* __restrict__ draft,
    const float* __restrict__ r, int gamma, int V, float invT2, float eta2, int C,
    const float* __restrict__ sstat, const float* __restrict__ tstat, unsigned flags,
    float* __restrict__ rowtab, float* __restrict__ wsum,
    uint32_t* __restrict__ arrivals, const float* __restrict__ u,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ out_tokens,
    float* __restrict__ ratio_out, float* __restrict__ p_hat_out) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ RowLse rc;
  __shared__ int sh_ts;
  float* rt = rowtab + (size_t)b * 2 * (gamma + 1);
  // Round trip 1: row table, s statistics, draft ids and acceptance uniforms.
  int x = 0;
  float rv = 0.f;
  if (wave == 0 && lane < gamma) {
    x = draft[(size_t)b * gamma + lane];
    rv = r[(size_t)b * gamma + lane];
  }
  for (int i = threadIdx.x; i <= gamma; i += TPB) {
    rc.lz[i] = rt[i];
    if (i < gamma) rc.ly[i] = rt[(gamma + 1) + i];
  }
  if (threadIdx.x == 0) rc.flags = flags;
  {
    const int grp = threadIdx.x >> 4, j = threadIdx.x & 15;
    for (int t = grp; t < gamma; t += TPB / 16) {
      float ms;
      const float ls = group_combine<16>(sstat + ((size_t)b * gamma + t) * C * 2, C, j, &ms);
      float zsum = 1.f;
      if (flags & RV_ACCEPT_TAIL_PRESERVE)
        zsum = group16_sum(tstat + ((size_t)b * gamma + t) * C, C, j);
      if (j == 0) {
        rc.ls[t] = ls;
        rc.thr[t] = ms + kLog2Tenth;
        rc.zinv[t] = 1.0f / zsum;
      }
    }
  }
  __syncthreads();

  if (wave == 0) {
    // Round trip 2: the draft tokens' target and draft logits.
    bool bad = false, acc = true;
    float ratio = 0.f;
    if (lane < gamma) {
      bad = (x < 0 || x >= V);
      if (!bad) {
        float p, q, s2;
        pq_s(z[((size_t)b * (gamma + 1) + lane) * V + x], y[((size_t)b * gamma + lane) * V + x],
             invT2, eta2, rc.lz[lane], rc.ly[lane], p, q, s2);
        const float ph = p_hat_entry(p, s2, lane, rc);
        ratio = fminf(1.0f, ph / q);
        acc = rv <= ratio;
      }
    }
  const uint64_t badm = __ballot(bad);
    const uint64_t rej = __ballot(lane < gamma && !acc);
    int ts = rej ? (int)__ffsll((long long)rej) - 1 : gamma;
    if (badm) ts = -1;
    if (lane == 0) sh_ts = ts;
    if (c == 0) {
      if (ratio_out != nullptr && lane < gamma)
        ratio_out[(size_t)b * gamma + lane] = bad ? __builtin_nanf("") : ratio;
      if (lane <= gamma) out_tokens[(size_t)b * (gamma + 1) + lane] = (lane < ts) ? x : -1;
      if (lane == 0) n_accept[b] = ts;
    }
  }
  __syncthreads();
  const int ts = sh_ts;
  const int start = c * CH + threadIdx.x * PER;

  if (p_hat_out != nullptr) {
    for (int t = 0; t < gamma; ++t) {
      float zx[PER], yx[PER];
      load_run<VEC>(z + ((size_t)b * (gamma + 1) + t) * V, V, start, zx);
      load_run<VEC>(y + ((size_t)b * gamma + t) * V, V, start, yx);
      float* dst = p_hat_out + ((size_t)b * gamma + t) * V;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        float p, q, s2;
        pq_s(zx[e], yx[e], invT2, eta2, rc.lz[t], rc.ly[t], p, q, s2);
        if (start + e < V) dst[start + e] = p_hat_entry(p, s2, t, rc);
      }
    }
  }
  if (ts < 0) return;  // uniform across the workgroup

  float zx[PER], yx[PER];
  load_run<VEC>(z + ((size_t)b * (gamma + 1) + ts) * V, V, start, zx);
  if (ts < gamma)
    load_run<VEC>(y + ((size_t)b * gamma + ts) * V, V, start, yx);
  else
#pragma unroll
    for (int e = 0; e < PER; ++e) yx[e] = 0.f;
  float w0 = 0.f, w1 = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (start + e < V) {
      w0 += draw_weight(zx[e], yx[e], ts, gamma, 0, invT2, eta2, rc);
      w1 += draw_weight(zx[e], yx[e], ts, gamma, 1, invT2, eta2, rc);
    }
  }
  const float W0 = block_sum(w0);
  const float W1 = block_sum(w1);
  // Publish this chunk's draw weights, then count its arrival.  The
  // workgroup that arrives last draws the token: which workgroup that is
  // does not change what is drawn, and nothing ever waits for another
  // workgroup.
  __shared__ uint32_t sh_arrived;
  if (threadIdx.x == 0) {
    wsum[((size_t)b * C + c) * 2 + 0] = W0;
    wsum[((size_t)b * C + c) * 2 + 1] = W1;
    __threadfence();
    sh_arrived = atomicAdd(arrivals + b, 1u);
  }
  __syncthreads();
  if (sh_arrived != (uint32_t)(C - 1)) return;  // uniform
  __threadfence();
  extern __shared__ float wsh[];  // [C][2]
  draw_row<VEC>(z, y, u, b, ts, gamma, V, invT2, eta2, C, rc, wsum, wsh, out_tokens);
}

template <bool VEC>
hipError_t launch_accept(const float* z, const float* y, const int32_t* draft, const float* r,
                         const float* u, int B, int gamma, int V, float invT2, float eta2,
                         unsigned flags, const AcceptLayout& L, float* ws, int32_t* n_accept,
                         int32_t* out_tokens, float* ratio_out, float* p_hat_out,
                         hipStream_t s) {
  const int C = L.chunks;
  float* zstat = ws + L.zstat;
  float* ystat = ws + L.ystat;
  float* sstat = ws + L.sstat;
  float* rowtab = ws + L.rowtab;
  float* tstat = ws + L.tstat;
  float* wsm = ws + L.wsum;
  uint32_t* arrivals = reinterpret_cast<uint32_t*>(ws + L.arrivals);
  hipLaunchKernelGGL((stats_kernel<VEC>), dim3(C, 2 * gamma + 1, B), dim3(TPB), 0, s, z, y, gamma,
                     V, invT2, C, zstat, ystat, arrivals);
  hipLaunchKernelGGL((phat_kernel<VEC>), dim3(C, gamma + 1, B), dim3(TPB), 0, s, z, y, gamma, V,
                     invT2, eta2, C, zstat, ystat, sstat, rowtab);
  if (flags & RV_ACCEPT_TAIL_PRESERVE)
    hipLaunchKernelGGL((tail_kernel<VEC>), dim3(C, gamma, B), dim3(TPB), 0, s, z, y, gamma, V,
                       invT2, eta2, C, sstat, rowtab, tstat);
  hipLaunchKernelGGL((decide_kernel<VEC>), dim3(C, B), dim3(TPB), (size_t)C * 2 * sizeof(float),
                     s, z, y, draft, r, gamma, V, invT2, eta2, C, sstat, tstat, flags, rowtab,
                     wsm, arrivals, u, n_accept, out_tokens, ratio_out, p_hat_out);
  return hipGetLastError();
}

}  // namespace
}  // namespace rv

extern "C" size_t rapid_accept_workspace_size(int B, int gamma, int V) {
  if (B < 1 || gamma < 1 || V < 2 || gamma > rv::kMaxGamma || V > rv::kMaxVocab) return 0;
  return rv::accept_layout(B, gamma, V).words * 4;
}

extern "C" rv_status rapid_accept_ex(const float* z, const float* y, const int32_t* draft,
                                     const float* r, const float* u, int B, int gamma, int V,
                                     float T, float eta, unsigned flags, int32_t* n_accept,
                                     int32_t* out_tokens, float* ratio_out, float* p_hat_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  rv_status st = rv::check_accept(z, y, draft, r, u, B, gamma, V, T, eta, flags, n_accept,
                                  out_tokens, workspace, workspace_bytes);
  if (st != RV_OK) return st;
  const rv::AcceptLayout L = rv::accept_layout(B, gamma, V);
  const double log2e = 1.4426950408889634;
  const float invT2 = (float)(log2e / (double)T);
  const float eta2 = (float)((double)eta * log2e);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  hipError_t e;
  if (V % 4 == 0)
    e = rv::launch_accept<true>(z, y, draft, r, u, B, gamma, V, invT2, eta2, flags, L, ws,
                                n_accept, out_tokens, ratio_out, p_hat_out, s);
  else
    e = rv::launch_accept<false>(z, y, draft, r, u, B, gamma, V, invT2, eta2, flags, L, ws,
                                 n_accept, out_tokens, ratio_out, p_hat_out, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}

extern "C" rv_status rapid_accept(const float* z, const float* y, const int32_t* draft,
                                  const float* r, const float* u, int B, int gamma, int V,
                                  float T, float eta, int32_t* n_accept, int32_t* out_tokens,
                                  float* ratio_out, float* p_hat_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return rapid_accept_ex(z, y, draft, r, u, B, gamma, V, T, eta, 0u, n_accept, out_tokens,
                         ratio_out, p_hat_out, workspace, workspace_bytes, stream);
}
