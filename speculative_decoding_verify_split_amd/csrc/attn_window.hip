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
// Split-K over the key list, then the log-sum-exp merge: one workgroup per
// (sequence, kv head, row, 64-key segment of the row's list) stages the
// segment's K and V once in LDS with coalesced loads, and its waves score
// the G query heads of that kv head against it (vector ALU in fp32: with 64
// keys and G rows there is no contraction worth a matrix-core tile), each
// writing a normalised partial (O, LSE) per (row, segment); lse_merge
// without a block part then merges the segments.  Fixed orders throughout,
// so results are bit-deterministic.

#include <type_traits>

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

constexpr int WSEG = 64;  // keys per segment

__device__ __forceinline__ float bf16_at(uint32_t w, int e) {
  return __uint_as_float(e == 0 ? (w << 16) : (w & 0xffff0000u));
}

// grid (S, Hkv, B * n).  o_part [B, Hq, n, S, d], lse_part [B, Hq, n, S].
template <int D>
__global__ __launch_bounds__(256) void window_part_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vr, const int32_t* __restrict__ pos, int Hq, int G, int n,
    int cap, int sink, int window, float scale_log2, int S, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  constexpr int PER = D / 64;  // output columns per lane
  constexpr int KQ = D / 8;    // 16-byte pieces per row
  constexpr int KROW = D * 2 + 16;  // padded K row in LDS: lane j reading row j hits distinct banks
  constexpr int VROWB = D * 2;
  __shared__ __attribute__((aligned(16))) unsigned char kt[WSEG * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char vt[WSEG * VROWB];
  const int s = blockIdx.x, kvh = blockIdx.y;
  const int b = blockIdx.z / n, i = blockIdx.z - (blockIdx.z / n) * n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Hkv = Hq / G;

  int P0 = pos[b];
  P0 = P0 < 0 ? 0 : (P0 > kMaxWindowPos ? kMaxWindowPos : P0);
  const int P = P0 + i;
  const int ns = min(sink, P + 1);           // sink keys
  const int lo = max(sink, P - window + 1);  // first window position
  const int K = ns + max(0, P - lo + 1);     // keys of this row (>= 1)
  const int R = cap - sink;                  // circular slots
  const int base = (lo >= sink) ? (lo - sink) % R : 0;
  // Slot of key idx of the row's list; indices past the list are clamped to
  // its last key (a written slot), so every load is in bounds and finite.
  auto slot_of = [&](int idx) {
    idx = min(idx, K - 1);
    int u = base + (idx - ns);  // < 2R: idx - ns < window <= R
    u -= (u >= R) ? R : 0;
    return (idx < ns) ? idx : sink + u;
  };
  const int c0 = s * WSEG;
  const int nk = min(WSEG, K - c0);  // keys of this segment (<= 0: empty)

  if (nk > 0) {
    const size_t kv0 = ((size_t)b * Hkv + kvh) * (size_t)cap * D;
    for (int pc = threadIdx.x; pc < WSEG * KQ; pc += 256) {
      const int r = pc / KQ, col = pc - r * KQ;
      const size_t off = kv0 + (size_t)slot_of(c0 + r) * D + col * 8;
      const i32x4 kx = *reinterpret_cast<const i32x4*>(kr + off);
      const i32x4 vx = *reinterpret_cast<const i32x4*>(vr + off);
      *reinterpret_cast<i32x4*>(kt + r * KROW + col * 16) = kx;
      *reinterpret_cast<i32x4*>(vt + r * VROWB + col * 16) = vx;
    }
  }
  __syncthreads();

  for (int g = wave; g < G; g += 4) {
    const int h = kvh * G + g;
    const size_t row = ((size_t)b * Hq + h) * n + i;
    float* op = o_part + (row * S + s) * D + lane * PER;
    if (nk <= 0) {  // uniform: an empty segment
#pragma unroll
      for (int e = 0; e < PER; ++e) op[e] = 0.f;
      if (lane == 0) lse_part[row * S + s] = -INFINITY;
      continue;
    }
    const i32x4* qp = reinterpret_cast<const i32x4*>(q + row * D);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < KQ; ++cc) {
      const i32x4 qq = qp[cc];
      const i32x4 kk = *reinterpret_cast<const i32x4*>(kt + lane * KROW + cc * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(bf16_at((uint32_t)qq[e], 0), bf16_at((uint32_t)kk[e], 0), acc[e]);
        acc[e] = fmaf(bf16_at((uint32_t)qq[e], 1), bf16_at((uint32_t)kk[e], 1), acc[e]);
      }
    }
    const float sc = lane < nk ? ((acc[0] + acc[1]) + (acc[2] + acc[3])) * scale_log2 : -INFINITY;
    const float m = wave_max(sc);  // finite: key c0 is in the list
    const float p = lane < nk ? exp2_hw(sc - m) : 0.f;
    const float l = wave_sum(p);
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
    for (int j = 0; j < WSEG; ++j) {
      const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j));
      if (PER == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(vt + j * VROWB + lane * 4);
        o[0] = fmaf(pj, bf16_at(w, 0), o[0]);
        o[PER - 1] = fmaf(pj, bf16_at(w, 1), o[PER - 1]);
      } else {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(vt + j * VROWB + lane * 2);
        o[0] = fmaf(pj, bf16_at(w, 0), o[0]);
      }
    }
    const float inv = 1.0f / l;  // l >= 1: the maximum contributes 2^0
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = o[e] * inv;
    if (lane == 0) lse_part[row * S + s] = (m + log2_hw(l)) * kLn2;
  }
}

}  // namespace
}  // namespace rv

extern "C" size_t spec_attn_window_workspace_size(int B, int Hq, int n, int d, int sink,
                                                  int window) {
  if (B < 1 || Hq < 1 || n < 1 || (d != 64 && d != 128) || sink < 0 || window < 1 ||
      sink > rv::kMaxWindowKeys || window > rv::kMaxWindowKeys)
    return 0;
  const size_t S = rv::window_segments(sink, window);
  const size_t rows = (size_t)B * Hq * n;
  return rv::window_workspace_words(rows, S, d) * 4;
}

extern "C" rv_status spec_attn_window(const void* q, const void* k_ring, const void* v_ring,
                                      const int32_t* pos, int B, int Hq, int Hkv, int n, int d,
                                      int cap, int sink, int window, float sm_scale, void* out,
                                      float* lse_out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  rv_status st = rv::check_window(q, k_ring, v_ring, pos, B, Hq, Hkv, n, d, cap, sink, window,
                                  sm_scale, out, workspace, workspace_bytes);
  if (st != RV_OK) return st;
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int S = rv::window_segments(sink, window);
  const size_t rows = (size_t)B * Hq * n;
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = o_part + rv::window_o_words(rows, S, d);
  dim3 grid((unsigned)S, (unsigned)Hkv, (unsigned)(B * n));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_ring);
  const uint16_t* vv = static_cast<const uint16_t*>(v_ring);
  if (d == 64)
    hipLaunchKernelGGL((rv::window_part_kernel<64>), grid, dim3(256), 0, s, qq, kk, vv, pos, Hq,
                       Hq / Hkv, n, cap, sink, window, scale_log2, S, o_part, lse_part);
  else
    hipLaunchKernelGGL((rv::window_part_kernel<128>), grid, dim3(256), 0, s, qq, kk, vv, pos, Hq,
                       Hq / Hkv, n, cap, sink, window, scale_log2, S, o_part, lse_part);
  if (hipGetLastError() != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  // the segments' partials merge exactly like history splits, with no block
  return lse_merge(o_part, lse_part, S, nullptr, nullptr, B, Hq, n, d, out, lse_out, stream);
}
