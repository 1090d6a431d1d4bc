// rapid_accept: RAPID's acceptance over the vocabulary (RAPID blog post,
// leeon-k.github.io: section 2.1, the acceptance test r <= min(1, p(x)/q(x))
// and the residual draw from norm(max(p - q, 0)); section 2.3, the test
// against the full-context target; section 2.4, the retrieval-augmented target
// p_hat = softmax(z/T + eta (q - p)) used in place of p at inference).
//
// Each row is a V-long fp32 stream (V ~ 1.3e5): little data, so the pass is
// bound by latency, i.e. by how many workgroups share each dependent step.
// Rows are cut into chunks, one 256-thread workgroup per chunk, and
// cross-chunk results go through a small workspace:
//   stats_kernel   (chunk, row, b), 4096-element chunks: max and sum of
//                  2^(x - max) of z/T (rows 0..gamma) and y/T (rows
//                  0..gamma-1), base-2 units
//   phat_kernel    (chunk, t, b), 4096-element chunks: the same for
//                  s = z/T + eta (q - p); the chunk holding draft token x_t
//                  also publishes z_t[x_t] and y_t[x_t]
//   tail_kernel    (chunk, t, b), 4096-element chunks, only with
//                  RV_ACCEPT_TAIL_PRESERVE (blog section 2.4's tail rule):
//                  chunk sums of the tail-adjusted row (p_hat where
//                  p_hat >= 0.1 max p_hat, p elsewhere), from which
//                  decide_kernel renormalises
//   decide_kernel  (chunk, b), 1024-element chunks: every chunk recomputes
//                  the gamma ratios min(1, p_hat_t[x_t]/q_t[x_t]) and the
//                  first-reject cut t*; chunk 0 writes n_accept, the accepted
//                  tokens and the ratios; every chunk writes its share of the
//                  draw weights (max(p_hat - q, 0) at t* < gamma, or with
//                  RV_ACCEPT_PRINTED_RESIDUAL section 2.4's printed
//                  max(p - min(p_hat, q), 0); p_gamma otherwise) and, on
//                  request, p_hat.  The last chunk to finish (one per-sequence
//                  arrival counter) then draws the token by inverse CDF with
//                  the caller's uniform: chunk -> thread -> element, each
//                  level taking the first unit of positive weight whose
//                  running total exceeds the target.
// Every reduction and scan has a fixed order and the counter only decides
// which workgroup runs the draw, so results are bit-exact run to run; no
// workgroup waits for another to run (the drawing one waits at most for slot
// stores already issued).

#include <mutex>

#include "vocab_common.h"

namespace rv {
namespace {

// Row-table offsets, per sequence, in words: [4][gamma+1].
__device__ __forceinline__ int rt_lz(int, int t) { return t; }
__device__ __forceinline__ int rt_ly(int gamma, int t) { return (gamma + 1) + t; }
__device__ __forceinline__ int rt_zx(int gamma, int t) { return 2 * (gamma + 1) + t; }
__device__ __forceinline__ int rt_yx(int gamma, int t) { return 3 * (gamma + 1) + t; }

template <bool VEC>
__global__ __launch_bounds__(TPB) void stats_kernel(const float* __restrict__ z,
                                                    const float* __restrict__ y, int gamma, int V,
                                                    float invT2, int cs, float* __restrict__ zstat,
                                                    float* __restrict__ ystat,
                                                    uint32_t* __restrict__ arrivals,
                                                    uint64_t* __restrict__ slots, int cd) {
  constexpr int PER = kStatPer;
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  // The decide kernel counts chunk arrivals per sequence and publishes its
  // chunk weights in slots; start from zero and empty slots on every call
  // (the workspace is not assumed to be initialised).
  if (c == 0 && r == 0 && threadIdx.x == 0) arrivals[(size_t)b * kArrivalStride] = 0u;
  if (r == 0) clear_slots(slots + (size_t)b * cd, cd);
  const float* row;
  float* dst;
  if (r <= gamma) {
    row = z + ((size_t)b * (gamma + 1) + r) * V;
    dst = zstat + (((size_t)b * (gamma + 1) + r) * cs + c) * 2;
  } else {
    const int t = r - gamma - 1;
    row = y + ((size_t)b * gamma + t) * V;
    dst = ystat + (((size_t)b * gamma + t) * cs + c) * 2;
  }
  const int start = c * kStatChunk + threadIdx.x * PER;
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
  const float cs_sum = block_sum(ts);
  if (threadIdx.x == 0) {
    dst[0] = cm;
    dst[1] = cs_sum;
  }
}

// grid (cp, gamma + 1, B).  Rows t < gamma: chunk stats of s; chunk 0 also
// publishes the row's z and y log-sum-exps, and the chunk holding the draft
// token x_t publishes z_t[x_t] and y_t[x_t] (no chunk does if x_t is out of
// range; the decide kernel rejects such a draft before reading them).
// Row gamma: chunk 0 publishes the last target row's log-sum-exp (for the
// bonus draw).
template <bool VEC>
__global__ __launch_bounds__(TPB) void phat_kernel(const float* __restrict__ z,
                                                   const float* __restrict__ y,
                                                   const int32_t* __restrict__ draft, int gamma,
                                                   int V, float invT2, float eta2, int cs, int cp,
                                                   const float* __restrict__ zstat,
                                                   const float* __restrict__ ystat,
                                                   float* __restrict__ sstat,
                                                   float* __restrict__ rowtab) {
  constexpr int PER = kPhatPer;
  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  float* rt = rowtab + (size_t)b * 4 * (gamma + 1);
  if (t == gamma) {
    if (c == 0 && threadIdx.x < 64) {
      const float lz =
          group_combine<64>(zstat + ((size_t)b * (gamma + 1) + t) * cs * 2, cs, lane);
      if (lane == 0) rt[rt_lz(gamma, t)] = lz;
    }
    return;
  }
  // Issue the chunk loads first: they do not depend on the row statistics.
  const int start = c * kPhatChunk + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(z + ((size_t)b * (gamma + 1) + t) * V, V, start, zx);
  load_run<VEC>(y + ((size_t)b * gamma + t) * V, V, start, yx);
  const int x = draft[(size_t)b * gamma + t];
  __shared__ float sh_l[2];
  if (threadIdx.x < 64) {
    const float lz =
        group_combine<64>(zstat + ((size_t)b * (gamma + 1) + t) * cs * 2, cs, lane);
    const float ly = group_combine<64>(ystat + ((size_t)b * gamma + t) * cs * 2, cs, lane);
    if (lane == 0) {
      sh_l[0] = lz;
      sh_l[1] = ly;
      if (c == 0) {
        rt[rt_lz(gamma, t)] = lz;
        rt[rt_ly(gamma, t)] = ly;
      }
    }
  }
  const int off = x - start;
  if (off >= 0 && off < PER) {
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (e == off) {
        rt[rt_zx(gamma, t)] = zx[e];
        rt[rt_yx(gamma, t)] = yx[e];
      }
  }
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
  const float csum = block_sum(ts);
  if (threadIdx.x == 0) {
    float* dst = sstat + (((size_t)b * gamma + t) * cp + c) * 2;
    dst[0] = cm;
    dst[1] = csum;
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

// grid (cp, gamma, B), RV_ACCEPT_TAIL_PRESERVE only: chunk sums of the
// unnormalised tail-adjusted p_hat (p_hat where s >= max s + log2 0.1, else
// p).  The row's LSE and max of s come from the same 16-lane combine the
// decide kernel uses, so both kernels classify every entry identically.
template <bool VEC>
__global__ __launch_bounds__(TPB) void tail_kernel(const float* __restrict__ z,
                                                   const float* __restrict__ y, int gamma, int V,
                                                   float invT2, float eta2, int cp,
                                                   const float* __restrict__ sstat,
                                                   const float* __restrict__ rowtab,
                                                   float* __restrict__ tstat) {
  constexpr int PER = kPhatPer;
  const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  __shared__ float sh[4];
  const int start = c * kPhatChunk + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(z + ((size_t)b * (gamma + 1) + t) * V, V, start, zx);
  load_run<VEC>(y + ((size_t)b * gamma + t) * V, V, start, yx);
  const float* rt = rowtab + (size_t)b * 4 * (gamma + 1);
  if (threadIdx.x < 16) {
    float ms;
    const float ls = group_combine<16>(sstat + ((size_t)b * gamma + t) * cp * 2, cp,
                                       threadIdx.x, &ms);
    if (threadIdx.x == 0) {
      sh[0] = ls;
      sh[1] = ms + kLog2Tenth;
      sh[2] = rt[rt_lz(gamma, t)];
      sh[3] = rt[rt_ly(gamma, t)];
    }
  }
  __syncthreads();
  const float ls = sh[0], thr = sh[1], lz = sh[2], ly = sh[3];
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float p, q, s2;
    pq_s(zx[e], yx[e], invT2, eta2, lz, ly, p, q, s2);
    if (start + e < V) acc += (s2 >= thr) ? exp2_hw(s2 - ls) : p;
  }
  const float csum = block_sum(acc);
  if (threadIdx.x == 0) tstat[((size_t)b * gamma + t) * cp + c] = csum;
}

// grid (cd, B).  Every chunk recomputes the row LSEs of s (16 lanes per row,
// all rows at once), the ratios and the first-reject cut, then writes its
// share of the draw weights; chunk 0 writes the per-sequence outputs.
template <bool VEC>
__global__ __launch_bounds__(TPB) void decide_kernel(
    const float* __restrict__ z, const float* __restrict__ y, const int32_t* __restrict__ draft,
    const float* __restrict__ r, int gamma, int V, float invT2, float eta2, int cp, int cd,
    const float* __restrict__ sstat, const float* __restrict__ tstat, unsigned flags,
    const float* __restrict__ rowtab, uint64_t* __restrict__ wsum,
    uint32_t* __restrict__ arrivals, const float* __restrict__ u,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ out_tokens,
    float* __restrict__ ratio_out, float* __restrict__ p_hat_out) {
  constexpr int PER = kDrawPer;
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ RowLse rc;
  __shared__ int sh_ts;
  const float* rt = rowtab + (size_t)b * 4 * (gamma + 1);
  // One round trip: draft ids, acceptance uniforms, the draft tokens' logits,
  // the row table and the s statistics are all independent loads.
  int x = 0;
  float rv = 0.f, zxv = 0.f, yxv = 0.f;
  if (wave == 0 && lane < gamma) {
    x = draft[(size_t)b * gamma + lane];
    rv = r[(size_t)b * gamma + lane];
    zxv = rt[rt_zx(gamma, lane)];
    yxv = rt[rt_yx(gamma, lane)];
  }
  for (int i = threadIdx.x; i <= gamma; i += TPB) {
    rc.lz[i] = rt[rt_lz(gamma, i)];
    if (i < gamma) rc.ly[i] = rt[rt_ly(gamma, i)];
  }
  if (threadIdx.x == 0) rc.flags = flags;
  {
    const int grp = threadIdx.x >> 4, j = threadIdx.x & 15;
    for (int t = grp; t < gamma; t += TPB / 16) {
      float ms;
      const float ls = group_combine<16>(sstat + ((size_t)b * gamma + t) * cp * 2, cp, j, &ms);
      float zsum = 1.f;
      if (flags & RV_ACCEPT_TAIL_PRESERVE)
        zsum = group16_sum(tstat + ((size_t)b * gamma + t) * cp, cp, j);
      if (j == 0) {
        rc.ls[t] = ls;
        rc.thr[t] = ms + kLog2Tenth;
        rc.zinv[t] = 1.0f / zsum;
      }
    }
  }
  __syncthreads();

  if (wave == 0) {
    bool bad = false, acc = true;
    float ratio = 0.f;
    if (lane < gamma) {
      bad = (x < 0 || x >= V);
      if (!bad) {
        float p, q, s2;
        pq_s(zxv, yxv, invT2, eta2, rc.lz[lane], rc.ly[lane], p, q, s2);
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
      // Slot ts belongs to the drawing workgroup alone (no two workgroups
      // write one word: their L2s may write back in either order).
      if (lane <= gamma && lane != ts)
        out_tokens[(size_t)b * (gamma + 1) + lane] = (lane < ts) ? x : -1;
      if (lane == 0) n_accept[b] = ts;
    }
  }
  __syncthreads();
  const int ts = sh_ts;
  const int start = c * kDrawChunk + threadIdx.x * PER;

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
  const float2 W = block_sum2(w0, w1);
  // Publish this chunk's draw weights and count its arrival.  The workgroup
  // that arrives last draws the token: which workgroup that is does not
  // change what is drawn, and it waits only for stores already issued.
  __shared__ uint32_t sh_arrived;
  if (threadIdx.x == 0)
    sh_arrived = publish_and_arrive(wsum + (size_t)b * cd + c, W.x, W.y,
                                    arrivals + (size_t)b * kArrivalStride);
  __syncthreads();
  if (sh_arrived != (uint32_t)(cd - 1)) return;  // uniform
  draw_from_chunks<VEC, kDrawPer>(
      z + ((size_t)b * (gamma + 1) + ts) * V,
      ts < gamma ? y + ((size_t)b * gamma + ts) * V : nullptr, u[(size_t)b * (gamma + 1) + ts], V,
      cd, wsum + (size_t)b * cd, out_tokens + (size_t)b * (gamma + 1) + ts,
      [&](float zv, float yv, int kind) {
        return draw_weight(zv, yv, ts, gamma, kind, invT2, eta2, rc);
      });
}

template <bool VEC>
hipError_t launch_accept(const float* z, const float* y, const int32_t* draft, const float* r,
                         const float* u, int B, int gamma, int V, float invT2, float eta2,
                         unsigned flags, const AcceptLayout& L, float* ws, int32_t* n_accept,
                         int32_t* out_tokens, float* ratio_out, float* p_hat_out,
                         hipStream_t s) {
  float* zstat = ws + L.zstat;
  float* ystat = ws + L.ystat;
  float* sstat = ws + L.sstat;
  float* rowtab = ws + L.rowtab;
  float* tstat = ws + L.tstat;
  uint64_t* wsm = reinterpret_cast<uint64_t*>(ws + L.wsum);
  uint32_t* arrivals = reinterpret_cast<uint32_t*>(ws + L.arrivals);
  hipLaunchKernelGGL((stats_kernel<VEC>), dim3(L.cs, 2 * gamma + 1, B), dim3(TPB), 0, s, z, y,
                     gamma, V, invT2, L.cs, zstat, ystat, arrivals, wsm, L.cd);
  hipLaunchKernelGGL((phat_kernel<VEC>), dim3(L.cp, gamma + 1, B), dim3(TPB), 0, s, z, y, draft,
                     gamma, V, invT2, eta2, L.cs, L.cp, zstat, ystat, sstat, rowtab);
  if (flags & RV_ACCEPT_TAIL_PRESERVE)
    hipLaunchKernelGGL((tail_kernel<VEC>), dim3(L.cp, gamma, B), dim3(TPB), 0, s, z, y, gamma, V,
                       invT2, eta2, L.cp, sstat, rowtab, tstat);
  hipLaunchKernelGGL((decide_kernel<VEC>), dim3(L.cd, B), dim3(TPB), 0, s, z, y, draft, r, gamma,
                     V, invT2, eta2, L.cp, L.cd, sstat, tstat, flags, rowtab, wsm, arrivals, u,
                     n_accept, out_tokens, ratio_out, p_hat_out);
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

// ---------------------------------------------------------------------------
// rapid_accept_noalloc: the same pass with its workspace in a static device
// array, for callers that cannot allocate.  The array has one copy per device
// (held until the process ends).  On the host its name stands for no device
// address, so it is never passed to a kernel: each device's address comes
// from hipGetSymbolAddress, taken once with that device current and kept.
// The pass clears what must start at zero (its arrival counters) itself.

static_assert(RV_NOALLOC_SCRATCH_BYTES == rv::kNoAllocScratchBytes, "scratch size");
static __device__ __align__(256) unsigned char scratch[rv::kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];

rv_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return RV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return RV_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RV_OK;
}
}  // namespace

extern "C" rv_status rapid_accept_noalloc(const float* z, const float* y, const int32_t* draft,
                                          const float* r, const float* u, int B, int gamma,
                                          int V, float T, float eta, unsigned flags,
                                          int32_t* n_accept, int32_t* out_tokens,
                                          float* ratio_out, float* p_hat_out, void* stream) {
  rv_status st = rv::check_accept_args(z, y, draft, r, u, B, gamma, V, T, eta, flags, n_accept,
                                       out_tokens);
  if (st != RV_OK) return st;
  if (rv::accept_layout(B, gamma, V).words * 4 > rv::kNoAllocScratchBytes)
    return RV_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != RV_OK) return st;
  return rapid_accept_ex(z, y, draft, r, u, B, gamma, V, T, eta, flags, n_accept, out_tokens,
                         ratio_out, p_hat_out, ws, rv::kNoAllocScratchBytes, stream);
}
