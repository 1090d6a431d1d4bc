// spec_attn_window: the drafter's sliding-window self-attention with
// attention-sink anchors over its constant-size ring cache (LongSpec summary,
// gist.science, section 2.1: self-attention limited to the latest 512
// tokens, so the drafter's own cache does not grow with the context;
// section 2.2: the first four tokens are kept as anchors).
//
// Row i of sequence b is the token at position P = pos[b] + i.  It sees the
// sink positions below min(sink, P + 1) and the window positions
// max(sink, P - window + 1) .. P, read from ring slots: position p lives in
// slot p below the sink and in slot sink + (p - sink) mod (cap - sink)
// otherwise.  The window part of the key list is consecutive positions, so
// its slots are consecutive modulo the ring and each row needs one modulo.
//
// At most sink + window keys per row (516 for the drafter) and G*n rows per
// kv head: no contraction worth a matrix-core tile, so this runs on the
// vector ALU in fp32.  One workgroup per row; its key list is cut into
// 64-key chunks dealt to the four waves in turn.  In a chunk, lane j scores
// key j (its K row against the query held in registers) while the lane's
// d/64 output columns of all 64 V rows are requested at the same time (the
// slots are known before any score); online softmax per wave, then a
// log-sum-exp merge of the four waves through LDS in wave order, so the
// result is bit-deterministic.

#include <type_traits>

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

constexpr int WNW = 8;  // waves per workgroup

__device__ __forceinline__ float bf16_at(uint32_t w, int e) {
  return __uint_as_float(e == 0 ? (w << 16) : (w & 0xffff0000u));
}

template <int D>
__global__ __launch_bounds__(WNW * 64) void window_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vr, const int32_t* __restrict__ pos, int Hq, int G, int n,
    int cap, int sink, int window, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse_out) {
  constexpr int PER = D / 64;  // output columns per lane
  constexpr int KQ = D / 8;    // 16-byte pieces per row
  const int row = blockIdx.x;  // (b * Hq + h) * n + i
  const int i = row % n;
  const int bh = row / n;
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  int P0 = pos[b];
  P0 = P0 < 0 ? 0 : (P0 > kMaxWindowPos ? kMaxWindowPos : P0);
  const int P = P0 + i;
  const int ns = min(sink, P + 1);                   // sink keys
  const int lo = max(sink, P - window + 1);          // first window position
  const int K = ns + max(0, P - lo + 1);             // keys of this row (>= 1)
  const int R = cap - sink;                          // circular slots
  const int base = (lo >= sink) ? (lo - sink) % R : 0;
  auto slot_of = [&](int idx) {
    if (idx < ns) return idx;
    int u = base + (idx - ns);  // < 2R: idx - ns < window <= R
    if (u >= R) u -= R;
    return sink + u;
  };
  const size_t kv0 = ((size_t)b * (Hq / G) + h / G) * (size_t)cap * D;
  const uint16_t* kh = kr + kv0;
  const uint16_t* vh = vr + kv0 + lane * PER;

  i32x4 qv[KQ];
  {
    const i32x4* qp = reinterpret_cast<const i32x4*>(q + (size_t)row * D);
#pragma unroll
    for (int c = 0; c < KQ; ++c) qv[c] = qp[c];
  }
  typedef typename std::conditional<PER == 2, uint32_t, uint16_t>::type vcol_t;

  float m = -INFINITY, l = 0.f, o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  const int nchunks = (K + 63) / 64;
  for (int c = wave; c < nchunks; c += WNW) {
    const int c0 = c * 64;
    const int idx = c0 + lane;
    const bool valid = idx < K;
    i32x4 kk[KQ];
    if (valid) {
      const i32x4* kp = reinterpret_cast<const i32x4*>(kh + (size_t)slot_of(idx) * D);
#pragma unroll
      for (int cc = 0; cc < KQ; ++cc) kk[cc] = kp[cc];
    }
    vcol_t vv[64];
#pragma unroll
    for (int j = 0; j < 64; ++j)
      vv[j] = (c0 + j < K) ? *reinterpret_cast<const vcol_t*>(vh + (size_t)slot_of(c0 + j) * D)
                           : vcol_t(0);
    float s = -INFINITY;
    if (valid) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < KQ; ++cc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = (uint32_t)qv[cc][e], bb = (uint32_t)kk[cc][e];
          acc[e] = fmaf(bf16_at(a, 0), bf16_at(bb, 0), acc[e]);
          acc[e] = fmaf(bf16_at(a, 1), bf16_at(bb, 1), acc[e]);
        }
      }
      s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * scale_log2;
    }
    const float mn = fmaxf(m, wave_max(s));  // finite: key c0 is valid
    const float alpha = (m == -INFINITY) ? 0.f : exp2_hw(m - mn);
    const float p = valid ? exp2_hw(s - mn) : 0.f;
    l = fmaf(l, alpha, wave_sum(p));
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j));
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float v = PER == 2 ? bf16_at((uint32_t)vv[j], e) : bf16_at((uint32_t)vv[j], 0);
        o[e] = fmaf(pj, v, o[e]);
      }
    }
    m = mn;
  }

  __shared__ float sm[WNW], sl[WNW];
  __shared__ float so[WNW][D];
  if (lane == 0) {
    sm[wave] = m;
    sl[wave] = l;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) so[wave][lane * PER + e] = o[e];
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < WNW; ++w) M = fmaxf(M, sm[w]);
  float a[WNW], L = 0.f;
#pragma unroll
  for (int w = 0; w < WNW; ++w) {
    a[w] = (sm[w] == -INFINITY) ? 0.f : exp2_hw(sm[w] - M);
    L = fmaf(a[w], sl[w], L);
  }
  const float inv = 1.0f / L;  // L >= 1: the wave holding the maximum contributes 2^0
  uint16_t* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int col = lane * PER + e;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < WNW; ++w) acc = fmaf(a[w], so[w][col], acc);
    dst[e] = f32_to_bf16_bits(acc * inv);
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = (M + log2_hw(L)) * kLn2;
}

}  // namespace
}  // namespace rv

extern "C" rv_status spec_attn_window(const void* q, const void* k_ring, const void* v_ring,
                                      const int32_t* pos, int B, int Hq, int Hkv, int n, int d,
                                      int cap, int sink, int window, float sm_scale, void* out,
                                      float* lse_out, void* stream) {
  rv_status st = rv::check_window(q, k_ring, v_ring, pos, B, Hq, Hkv, n, d, cap, sink, window,
                                  sm_scale, out);
  if (st != RV_OK) return st;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)(B * Hq * n));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_ring);
  const uint16_t* vv = static_cast<const uint16_t*>(v_ring);
  uint16_t* o16 = static_cast<uint16_t*>(out);
  if (d == 64)
    hipLaunchKernelGGL((rv::window_kernel<64>), grid, dim3(rv::WNW * 64), 0, s, qq, kk, vv, pos,
                       Hq, Hq / Hkv, n, cap, sink, window, scale_log2, o16, lse_out);
  else
    hipLaunchKernelGGL((rv::window_kernel<128>), grid, dim3(rv::WNW * 64), 0, s, qq, kk, vv, pos,
                       Hq, Hq / Hkv, n, cap, sink, window, scale_log2, o16, lse_out);
  if (hipGetLastError() != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}
