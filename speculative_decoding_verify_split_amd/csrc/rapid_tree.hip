// rapid_tree_accept: RAPID's acceptance over a draft tree.
//
// The pages verify draft trees only as attention (LongSpec summary,
// gist.science, section 1 "Problem", challenge 3; section 2.3 "Fast Tree
// Attention"); the rule among sibling candidates is taken from outside them:
// recursive rejection.  At node v the children are tested in ascending node
// id against a residual R that starts at p_hat_v (RAPID blog post,
// leeon-k.github.io, section 2.4) and becomes norm(max(R - q_v, 0)) after each
// rejection; the first child accepted continues the walk; if none is, the
// token is drawn from the last residual; a leaf draws a bonus from p_v.
//
// The residual after j rejections has a closed form: max(p_hat - C_j q, 0)
// with mass M_j, where C_0 = 0, M_0 = 1 and C_{j+1} = C_j + M_j.  The M_j of
// a node do not depend on the uniforms, so every child's ratio can be formed
// before the walk: child c of rank j under v is tested against
// R_j = max(p_hat_v - C_j q_v, 0) / M_j.  The passes:
//   tree_stats_kernel   (chunk, row, b): chunk (max, sum) of z/T for every node
//                       and of y/T for every internal node
//   tree_phat_kernel    (chunk, slot, b): the same for s = z/T + eta (q - p) of
//                       each internal node; an extra workgroup per sequence
//                       forms every node's log-sum-exp of z/T
//   tree_resid_kernel   pass j = 1 .. (largest child count - 1), (chunk, slot,
//                       b): chunk sums of max(p_hat - C_j q, 0) for internal
//                       nodes with more than j children
//   tree_decide_kernel  (chunk, b): every workgroup forms all children's
//                       ratios, walks the tree (a few bit operations), then
//                       writes its chunk's draw weights of the stop node; the
//                       last to arrive draws the token (draw_from_chunks) and
//                       workgroup 0 writes the path and the other outputs.
// Every reduction has a fixed order; results are bit-exact run to run.

#include "vocab_common.h"

namespace rv {
namespace {

// grid (cs, n + ni, B): rows < n are z rows of nodes, the rest y rows of
// internal slots.  Also clears the sequence's arrival counter and empties its
// draw-weight slots.
template <bool VEC>
__global__ __launch_bounds__(TPB) void tree_stats_kernel(const float* __restrict__ z,
                                                         const float* __restrict__ y, TreePlan tp,
                                                         int V, float invT2, int cs,
                                                         float* __restrict__ zstat,
                                                         float* __restrict__ ystat,
                                                         uint32_t* __restrict__ arrivals,
                                                         uint64_t* __restrict__ slots, int cd) {
  constexpr int PER = kStatPer;
  const int c = blockIdx.x, rr = blockIdx.y, b = blockIdx.z;
  const int n = tp.n;
  if (c == 0 && rr == 0 && threadIdx.x == 0) arrivals[(size_t)b * kArrivalStride] = 0u;
  if (rr == 0) clear_slots(slots + (size_t)b * cd, cd);
  const float* row;
  float* dst;
  if (rr < n) {
    row = z + ((size_t)b * n + rr) * V;
    dst = zstat + (((size_t)b * n + rr) * cs + c) * 2;
  } else {
    const int a = rr - n;
    row = y + ((size_t)b * n + tp.inode[a]) * V;
    dst = ystat + (((size_t)b * n + a) * cs + c) * 2;
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
  const float csum = block_sum(ts);
  if (threadIdx.x == 0) {
    dst[0] = cm;
    dst[1] = csum;
  }
}

// Row table offsets per sequence, in words: lz of node v at v, ly of internal
// slot a at n + a.
__device__ __forceinline__ float* tree_rt(float* rowtab, int b, int n) {
  return rowtab + (size_t)b * 2 * n;
}

// grid (cp, ni + 1, B).  Slot a < ni: chunk (max, sum) of s for internal node
// inode[a]; chunk 0 publishes the slot's y log-sum-exp.  Slot ni, chunk 0:
// the z log-sum-exp of every node (others return at once).
template <bool VEC>
__global__ __launch_bounds__(TPB) void tree_phat_kernel(const float* __restrict__ z,
                                                        const float* __restrict__ y, TreePlan tp,
                                                        int V, float invT2, float eta2, int cs,
                                                        int cp, const float* __restrict__ zstat,
                                                        const float* __restrict__ ystat,
                                                        float* __restrict__ sstat,
                                                        float* __restrict__ rowtab) {
  constexpr int PER = kPhatPer;
  const int c = blockIdx.x, a = blockIdx.y, b = blockIdx.z;
  const int n = tp.n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* rt = tree_rt(rowtab, b, n);
  if (a == tp.ni) {
    if (c != 0) return;
    for (int v = wave; v < n; v += TPB / 64) {
      const float lz = group_combine<64>(zstat + ((size_t)b * n + v) * cs * 2, cs, lane);
      if (lane == 0) rt[v] = lz;
    }
    return;
  }
  const int v = tp.inode[a];
  const int start = c * kPhatChunk + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(z + ((size_t)b * n + v) * V, V, start, zx);
  load_run<VEC>(y + ((size_t)b * n + v) * V, V, start, yx);
  __shared__ float sh_l[2];
  if (threadIdx.x < 64) {
    const float lz = group_combine<64>(zstat + ((size_t)b * n + v) * cs * 2, cs, lane);
    const float ly = group_combine<64>(ystat + ((size_t)b * n + a) * cs * 2, cs, lane);
    if (lane == 0) {
      sh_l[0] = lz;
      sh_l[1] = ly;
      if (c == 0) rt[n + a] = ly;
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
    float* dst = sstat + (((size_t)b * n + a) * cp + c) * 2;
    dst[0] = cm;
    dst[1] = csum;
  }
}

// The constants of internal slot a needed by the residual: base-2 LSE of s
// (ls) and C_j = 1 + M_1 + ... + M_{j-1} (C_0 = 0), formed by a 16-lane
// group from the published chunk statistics, in a fixed order.
__device__ __forceinline__ float resid_c(const float* __restrict__ rstat, int b, int n, int a,
                                         int cp, int j, int lane16) {
  if (j == 0) return 0.f;
  float C = 1.0f;
  for (int i = 1; i < j; ++i)
    C += group16_sum(rstat + (((size_t)b * n + a) * n + (i - 1)) * cp, cp, lane16);
  return C;
}

// Pass j (1 <= j <= npass), grid (cp, ni, B): chunk sums of
// max(p_hat - C_j q, 0) for internal nodes with more than j children.
template <bool VEC>
__global__ __launch_bounds__(TPB) void tree_resid_kernel(const float* __restrict__ z,
                                                         const float* __restrict__ y, TreePlan tp,
                                                         int j, int V, float invT2, float eta2,
                                                         int cp, const float* __restrict__ sstat,
                                                         const float* __restrict__ rowtab,
                                                         float* __restrict__ rstat) {
  constexpr int PER = kPhatPer;
  const int c = blockIdx.x, a = blockIdx.y, b = blockIdx.z;
  const int n = tp.n;
  const int v = tp.inode[a];
  if (tp.nchild[v] <= j) return;  // uniform
  const int start = c * kPhatChunk + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(z + ((size_t)b * n + v) * V, V, start, zx);
  load_run<VEC>(y + ((size_t)b * n + v) * V, V, start, yx);
  __shared__ float sh[4];
  if (threadIdx.x < 16) {
    const float ls = group_combine<16>(sstat + ((size_t)b * n + a) * cp * 2, cp, threadIdx.x);
    const float C = resid_c(rstat, b, n, a, cp, j, threadIdx.x);
    if (threadIdx.x == 0) {
      const float* rt = tree_rt(const_cast<float*>(rowtab), b, n);
      sh[0] = ls;
      sh[1] = C;
      sh[2] = rt[v];
      sh[3] = rt[n + a];
    }
  }
  __syncthreads();
  const float ls = sh[0], C = sh[1], lz = sh[2], ly = sh[3];
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float p, q, s;
    pq_s(zx[e], yx[e], invT2, eta2, lz, ly, p, q, s);
    if (start + e < V) acc += fmaxf(exp2_hw(s - ls) - C * q, 0.f);
  }
  const float csum = block_sum(acc);
  if (threadIdx.x == 0) rstat[(((size_t)b * n + a) * n + (j - 1)) * cp + c] = csum;
}

// Per-sequence constants of the decide pass, in LDS.
struct TreeConsts {
  float lz[kMaxTreeNodes];   // by node
  float ly[kMaxTreeNodes];   // by slot
  float ls[kMaxTreeNodes];   // by slot
  float ratio[kMaxTreeNodes];
  int32_t tok[kMaxTreeNodes];
  int32_t path[kMaxTreeNodes];
  uint64_t tested;
  int m, vstop, kstop;       // path length, stop node, residual index at it (-1: bonus)
  float Cstop;               // C_k of the stop node's residual
  int bad;
};

// grid (cd, B).
template <bool VEC>
__global__ __launch_bounds__(TPB) void tree_decide_kernel(
    const float* __restrict__ z, const float* __restrict__ y, const int32_t* __restrict__ tokens,
    const float* __restrict__ r, const float* __restrict__ u, TreePlan tp, int V, float invT2,
    float eta2, int cp, int cd, const float* __restrict__ sstat,
    const float* __restrict__ rowtab, const float* __restrict__ rstat, uint64_t* __restrict__ wsum,
    uint32_t* __restrict__ arrivals, int32_t* __restrict__ n_accept, int32_t* __restrict__ path,
    int32_t* __restrict__ out_tokens, float* __restrict__ ratio_out) {
  constexpr int PER = kDrawPer;
  const int c = blockIdx.x, b = blockIdx.y;
  const int n = tp.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ TreeConsts tc;
  __shared__ float sh_M[kMaxTreeNodes][kMaxTreeNodes];  // [slot][j]: mass of residual j

  // Loads of the first round trip: tokens and acceptance uniforms (wave 0,
  // lane = node), the row table, the slots' s statistics and residual sums.
  int x = 0;
  float rv = 0.f;
  if (wave == 0 && lane < n) {
    x = tokens[(size_t)b * n + lane];
    rv = r[(size_t)b * n + lane];
    tc.tok[lane] = x;
  }
  {
    const float* rt = tree_rt(const_cast<float*>(rowtab), b, n);
    for (int i = threadIdx.x; i < n; i += TPB) tc.lz[i] = rt[i];
    for (int i = threadIdx.x; i < tp.ni; i += TPB) tc.ly[i] = rt[n + i];
  }
  {
    const int grp = threadIdx.x >> 4, j16 = threadIdx.x & 15;
    for (int a = grp; a < tp.ni; a += TPB / 16) {
      const float ls = group_combine<16>(sstat + ((size_t)b * n + a) * cp * 2, cp, j16);
      if (j16 == 0) tc.ls[a] = ls;
      const int k = tp.nchild[tp.inode[a]];
      for (int i = 1; i < k; ++i) {
        const float M = group16_sum(rstat + (((size_t)b * n + a) * n + (i - 1)) * cp, cp, j16);
        if (j16 == 0) sh_M[a][i] = M;
      }
    }
  }
  __syncthreads();

  // Every child's ratio against the residual it would be tested with (second
  // round trip: the logits at the child's token), then the walk.
  if (wave == 0) {
    bool bad = false, acc = false;
    float ratio = 0.f;
    if (lane >= 1 && lane < n) {
      bad = x < 0 || x >= V;
      if (!bad) {
        const int v = tp.parent[lane], a = tp.slot[v], j = tp.rank[lane];
        const float zxv = z[((size_t)b * n + v) * V + x];
        const float yxv = y[((size_t)b * n + v) * V + x];
        float p, q, s;
        pq_s(zxv, yxv, invT2, eta2, tc.lz[v], tc.ly[a], p, q, s);
        const float ph = exp2_hw(s - tc.ls[a]);
        float C = 0.f, M = 1.f;
        if (j > 0) {
          C = 1.f;
          for (int i = 1; i < j; ++i) C += sh_M[a][i];
          M = sh_M[a][j];
        }
        const float w = j > 0 ? fmaxf(ph - C * q, 0.f) : ph;
        ratio = fminf(1.0f, w / (M * q));
        acc = rv <= ratio;
      }
      tc.ratio[lane] = bad ? __builtin_nanf("") : ratio;
    }
    const uint64_t badm = __ballot(bad);
    const uint64_t accm = __ballot(acc);
    if (lane == 0) {
      tc.bad = badm != 0;
      int v = 0, m = 0, kstop = -1;
      uint64_t tested = 0;
      float Cstop = 0.f;
      if (!badm) {
        for (;;) {
          const uint64_t kids = tp.kids[v];
          if (kids == 0) break;  // leaf: bonus draw
          const uint64_t hit = accm & kids;
          if (hit == 0) {
            // every child rejected: draw from residual k = child count
            tested |= kids;
            kstop = tp.nchild[v];
            const int a = tp.slot[v];
            Cstop = 1.f;
            for (int i = 1; i < kstop; ++i) Cstop += sh_M[a][i];
            break;
          }
          const int ch = __ffsll((long long)hit) - 1;
          tested |= kids & ((2ull << ch) - 1ull);
          tc.path[m++] = ch;
          v = ch;
        }
      }
      tc.m = m;
      tc.vstop = v;
      tc.kstop = kstop;
      tc.Cstop = Cstop;
      tc.tested = tested;
    }
  }
  __syncthreads();

  if (c == 0 && wave == 0) {
    const bool badseq = tc.bad != 0;
    const int m = tc.m;
    if (lane < n) {
      const bool on = !badseq && lane < m;
      path[(size_t)b * n + lane] = on ? tc.path[lane] : -1;
      // slot m belongs to the drawing workgroup
      if (badseq || lane != m) out_tokens[(size_t)b * n + lane] = on ? tc.tok[tc.path[lane]] : -1;
      if (ratio_out != nullptr)
        ratio_out[(size_t)b * n + lane] =
            (!badseq && ((tc.tested >> lane) & 1ull)) ? tc.ratio[lane] : __builtin_nanf("");
    }
    if (lane == 0) n_accept[b] = badseq ? -1 : m;
  }
  if (tc.bad) return;  // uniform

  // This chunk's draw weights of the stop node: the residual
  // max(p_hat - C q, 0) after kstop rejections (kind 0), or p_hat itself if
  // that has no mass (kind 1); at a leaf, p (both kinds).
  const int v = tc.vstop, kstop = tc.kstop;
  const int a = tp.slot[v];
  const bool bonus = kstop < 0;
  const float lz = tc.lz[v], ly = bonus ? 0.f : tc.ly[a], ls = bonus ? 0.f : tc.ls[a];
  const float C = tc.Cstop;
  auto wfun = [&](float zv, float yv, int kind) {
    if (bonus) return exp2_hw(zv * invT2 - lz);
    float p, q, s;
    pq_s(zv, yv, invT2, eta2, lz, ly, p, q, s);
    const float ph = exp2_hw(s - ls);
    return kind ? ph : fmaxf(ph - C * q, 0.f);
  };
  const float* zrow = z + ((size_t)b * n + v) * V;
  const float* yrow = bonus ? nullptr : y + ((size_t)b * n + v) * V;
  const int start = c * kDrawChunk + threadIdx.x * PER;
  float zx[PER], yx[PER];
  load_run<VEC>(zrow, V, start, zx);
  if (yrow != nullptr)
    load_run<VEC>(yrow, V, start, yx);
  else
#pragma unroll
    for (int e = 0; e < PER; ++e) yx[e] = 0.f;
  float w0 = 0.f, w1 = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (start + e < V) {
      w0 += wfun(zx[e], yx[e], 0);
      w1 += wfun(zx[e], yx[e], 1);
    }
  }
  const float2 W = block_sum2(w0, w1);
  // Publish and count the arrival; the last workgroup to arrive draws (as in
  // decide_kernel of rapid_accept).
  __shared__ uint32_t sh_arrived;
  if (threadIdx.x == 0)
    sh_arrived = publish_and_arrive(wsum + (size_t)b * cd + c, W.x, W.y,
                                    arrivals + (size_t)b * kArrivalStride);
  __syncthreads();
  if (sh_arrived != (uint32_t)(cd - 1)) return;  // uniform
  draw_from_chunks<VEC, PER>(zrow, yrow, u[(size_t)b * n + v], V, cd, wsum + (size_t)b * cd,
                             out_tokens + (size_t)b * n + tc.m, wfun);
}

template <bool VEC>
hipError_t launch_tree(const float* z, const float* y, const int32_t* tokens, const float* r,
                       const float* u, int B, const TreePlan& tp, int V, float invT2, float eta2,
                       const TreeLayout& L, float* ws, int32_t* n_accept, int32_t* path,
                       int32_t* out_tokens, float* ratio_out, hipStream_t s) {
  float* zstat = ws + L.zstat;
  float* ystat = ws + L.ystat;
  float* sstat = ws + L.sstat;
  float* rowtab = ws + L.rowtab;
  float* rstat = ws + L.rstat;
  uint64_t* wsm = reinterpret_cast<uint64_t*>(ws + L.wsum);
  uint32_t* arrivals = reinterpret_cast<uint32_t*>(ws + L.arrivals);
  hipLaunchKernelGGL((tree_stats_kernel<VEC>), dim3(L.cs, tp.n + tp.ni, B), dim3(TPB), 0, s, z,
                     y, tp, V, invT2, L.cs, zstat, ystat, arrivals, wsm, L.cd);
  hipLaunchKernelGGL((tree_phat_kernel<VEC>), dim3(L.cp, tp.ni + 1, B), dim3(TPB), 0, s, z, y, tp,
                     V, invT2, eta2, L.cs, L.cp, zstat, ystat, sstat, rowtab);
  for (int j = 1; j <= tp.npass; ++j)
    hipLaunchKernelGGL((tree_resid_kernel<VEC>), dim3(L.cp, tp.ni, B), dim3(TPB), 0, s, z, y, tp,
                       j, V, invT2, eta2, L.cp, sstat, rowtab, rstat);
  hipLaunchKernelGGL((tree_decide_kernel<VEC>), dim3(L.cd, B), dim3(TPB), 0, s, z, y, tokens, r,
                     u, tp, V, invT2, eta2, L.cp, L.cd, sstat, rowtab, rstat, wsm, arrivals,
                     n_accept, path, out_tokens, ratio_out);
  return hipGetLastError();
}

}  // namespace
}  // namespace rv

extern "C" size_t rapid_tree_accept_workspace_size(int B, int n, int V) {
  if (B < 1 || n < 1 || V < 2 || n > rv::kMaxTreeNodes || V > rv::kMaxVocab) return 0;
  return rv::tree_layout(B, n, V).words * 4;
}

extern "C" rv_status rapid_tree_accept(const float* z, const float* y, const int32_t* tokens,
                                       const int32_t* parent_host, const float* r,
                                       const float* u, int B, int n, int V, float T, float eta,
                                       int32_t* n_accept, int32_t* path, int32_t* out_tokens,
                                       float* ratio_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  rv::TreePlan tp;
  rv_status st = rv::check_tree_accept(z, y, tokens, parent_host, r, u, B, n, V, T, eta,
                                       n_accept, path, out_tokens, workspace, workspace_bytes,
                                       &tp);
  if (st != RV_OK) return st;
  const rv::TreeLayout L = rv::tree_layout(B, n, V);
  const double log2e = 1.4426950408889634;
  const float invT2 = (float)(log2e / (double)T);
  const float eta2 = (float)((double)eta * log2e);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  const hipError_t e =
      V % 4 == 0 ? rv::launch_tree<true>(z, y, tokens, r, u, B, tp, V, invT2, eta2, L, ws,
                                         n_accept, path, out_tokens, ratio_out, s)
                 : rv::launch_tree<false>(z, y, tokens, r, u, B, tp, V, invT2, eta2, L, ws,
                                          n_accept, path, out_tokens, ratio_out, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}
