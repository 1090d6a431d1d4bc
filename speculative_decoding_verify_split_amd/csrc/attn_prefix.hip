// spec_attn_prefix: unmasked attention of the verify rows over the history KV
// cache, split along the sequence (LongSpec summary, gist.science, section 2.3
// "Fast Tree Attention": the history key/value pairs need no mask, so they go
// to a plain fast attention pass whose result is later merged by log-sum-exp).
//
// Work decomposition (gfx950, 64-wide waves):
//   grid  = (split s, kv-head x row-group, sequence b); 4 waves per workgroup.
//   A workgroup owns one split of one (b, kv-head): the G = Hq/Hkv query heads
//   of that kv-head share every K/V byte, so their G*n rows are stacked into
//   16-row MFMA tiles (up to 4 tiles per wave; larger groups use several row
//   groups).  Wave w streams the split's 32-key tiles w, w+4, w+8, ...
//   Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_16x16x32_bf16: the K tile is the A operand and is loaded
//   straight from HBM into registers (each lane reads 4 x 16 B of one key row;
//   one instruction covers 16 keys x 64 contiguous bytes).  In the transposed
//   layout a lane holds 8 scores of one query row, which is exactly the B
//   operand layout of the P V product, so P needs no shuffle.  V must be
//   transposed for its operand: each wave stages its 32 x d V tile in a
//   private LDS slice (row pitch 2d + 8 bytes: conflict-free gathers) and
//   gathers 8 keys of one column per lane.  Online softmax runs in fp32 in
//   base-2 units; the next tile's K/V loads are in flight while the current
//   tile is computed.  The four waves' (max, sum, O) states are merged through
//   LDS and one normalised partial (O, LSE) per row is written.
//   Loads use buffer resources bounded by the split's length, so keys past
//   the split or the sequence read as zero and are masked to -inf.

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

constexpr int KT = kKeysPerTile;
constexpr int NW = kWavesPerGroup;

template <int D>
struct PrefixGeom {
  static constexpr int KS = D / 32;             // MFMA k-steps over the head dim
  static constexpr int NB = D / 16;             // 16-column blocks of the output
  static constexpr int VCH = KT * D / 8 / 64;   // 16-byte V chunks per lane per tile
  static constexpr int VROW = 2 * D + 8;        // bytes per key row of a V tile in LDS
  static constexpr int VTILE = KT * VROW;       // bytes per wave V tile
  static constexpr int OROW = D + 4;            // floats per row of the merge buffer
};

template <int D, int MT>
__global__ __launch_bounds__(NW * 64, 1) void prefix_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ seq_lens, int Hq, int Hkv,
    int n, int64_t L_max, float scale_log2, int64_t split_len, int S, int RG,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  using Gm = PrefixGeom<D>;
  constexpr int KS = Gm::KS, NB = Gm::NB, VCH = Gm::VCH, VROW = Gm::VROW, OROW = Gm::OROW;
  constexpr int VBYTES = NW * Gm::VTILE;
  constexpr int OBYTES = MT * 16 * OROW * 4;
  constexpr int SMEM = VBYTES > OBYTES ? VBYTES : OBYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ float m_lds[MT * 16];
  __shared__ float l_lds[MT * 16];

  const int s = blockIdx.x;
  const int kvh = blockIdx.y / RG;
  const int rg = blockIdx.y - kvh * RG;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int G = Hq / Hkv;
  const int M = G * n;
  const int row0 = rg * MT * 16;
  const int rows_here = min(MT * 16, M - row0);

  int64_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > L_max ? L_max : L);
  const int64_t kbeg = (int64_t)s * split_len;
  int64_t kend = kbeg + split_len;
  if (kend > L) kend = L;
  const int nkeys = kend > kbeg ? (int)(kend - kbeg) : 0;
  const int ntiles = (nkeys + KT - 1) / KT;

  // Query fragments, B operand of S^T = K Q^T: lane (row lr, group lg) holds
  // d = 32*ks + 8*lg .. +7 of its row.
  bf16x8 qf[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = row0 + mt * 16 + lr;
    if (row < M) {
      const int gq = row / n;
      const int i = row - gq * n;
      const int h = kvh * G + gq;
      const uint16_t* qp = q + (((int64_t)b * Hq + h) * n + i) * D + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[mt][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[mt][ks] = bf16x8{};
    }
  }

  const size_t slab = ((size_t)b * Hkv + kvh) * (size_t)L_max * D + (size_t)kbeg * D;
  const uint32_t nbytes = (uint32_t)nkeys * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + slab, nbytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + slab, nbytes);

  f32x4 oacc[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[MT], l_run[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    m_run[mt] = -INFINITY;
    l_run[mt] = 0.f;
  }

  unsigned char* vt = smem + wave * Gm::VTILE;
  i32x4 kreg[2][KS], vreg[VCH];

  auto load_tile = [&](int tt, i32x4(&kr)[2][KS], i32x4(&vr)[VCH]) {
    const uint32_t base = (uint32_t)tt * KT * D * 2;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kr[kb][ks] = buffer_load16(krs, base + (uint32_t)(((kb * 16 + lr) * D + ks * 32 + lg * 8) * 2));
#pragma unroll
    for (int i = 0; i < VCH; ++i) vr[i] = buffer_load16(vrs, base + (uint32_t)((i * 64 + lane) * 16));
  };

  int t = wave;
  if (t < ntiles) load_tile(t, kreg, vreg);
  for (; t < ntiles; t += NW) {
    i32x4 knext[2][KS], vnext[VCH];
    load_tile(t + NW, knext, vnext);  // past the split: reads zeros, never used

    // Stage the V tile: chunk c = 64 i + lane is key c / (D/8), columns
    // 8 (c % (D/8)) .. +7.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = i * 64 + lane;
      const int key = c / (D / 8);
      const int dch = c - key * (D / 8);
      i32x2* dst = reinterpret_cast<i32x2*>(vt + key * VROW + dch * 16);
      dst[0] = i32x2{vreg[i][0], vreg[i][1]};
      dst[1] = i32x2{vreg[i][2], vreg[i][3]};
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // S^T for the tile: key block kb (16 keys) x row tile mt.
    f32x4 sacc[2][MT];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kreg[kb][ks]), qf[mt][ks], acc, 0, 0, 0);
        sacc[kb][mt] = acc;
      }

    // Online softmax.  Lane (lr, lg) holds row lr's scores for keys
    // 16 kb + 4 lg + v; the 4 lanes lr + 16 g share a row.
    const int key0 = t * KT + lg * 4;
    bf16x8 pf[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int kk = key0 + kb * 16 + v;
          x[kb * 4 + v] = kk < nkeys ? sacc[kb][mt][v] * scale_log2 : -INFINITY;
        }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[mt], mx);
      const float alpha = exp2_hw(m_run[mt] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_hw(x[e] - m_new);
        ps += p;
        pf[mt][e] = (__bf16)p;
      }
      l_run[mt] = l_run[mt] * alpha + ps;
      m_run[mt] = m_new;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb][mt] *= alpha;
    }

    // O^T += V^T P^T: A operand lane (column d = 16 nb + lr, group lg) holds
    // V[key][d] for keys 4 lg + e (e < 4) and 16 + 4 lg + (e - 4) (e >= 4),
    // the same key order as pf.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bf16x8 va;
      const unsigned char* col = vt + (nb * 16 + lr) * 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = (e < 4) ? (lg * 4 + e) : (16 + lg * 4 + e - 4);
        va[e] = *reinterpret_cast<const __bf16*>(col + key * VROW);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        oacc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[mt], oacc[nb][mt], 0, 0, 0);
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kreg[kb][ks] = knext[kb][ks];
#pragma unroll
    for (int i = 0; i < VCH; ++i) vreg[i] = vnext[i];
  }

  // Row sums: each lane holds a quarter of its row's keys.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    l_run[mt] += __shfl_xor(l_run[mt], 16, 64);
    l_run[mt] += __shfl_xor(l_run[mt], 32, 64);
  }

  // Merge the four waves' states through LDS, one wave at a time.
  __syncthreads();  // V tiles are dead; the buffer becomes the merge buffer
  float* obuf = reinterpret_cast<float*>(smem);
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 16 + lr;
        const float mo = (w == 0) ? -INFINITY : m_lds[row];
        const float lo = (w == 0) ? 0.f : l_lds[row];
        const float mn = fmaxf(mo, m_run[mt]);
        const float a = (mo == -INFINITY) ? 0.f : exp2_hw(mo - mn);
        const float c = (m_run[mt] == -INFINITY) ? 0.f : exp2_hw(m_run[mt] - mn);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4* op = reinterpret_cast<f32x4*>(obuf + row * OROW + nb * 16 + lg * 4);
          const f32x4 prev = (w == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : *op;
          *op = a * prev + c * oacc[nb][mt];
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (lg == 0) {
          m_lds[row] = mn;
          l_lds[row] = a * lo + c * l_run[mt];
        }
      }
    }
    __syncthreads();
  }

  // Normalised partial output and its natural-log LSE.
  for (int idx = threadIdx.x; idx < rows_here * (D / 4); idx += NW * 64) {
    const int row = idx / (D / 4);
    const int c4 = idx - row * (D / 4);
    const float l = l_lds[row];
    const f32x4 o = *reinterpret_cast<const f32x4*>(obuf + row * OROW + c4 * 4);
    const f32x4 res = l > 0.f ? o / l : f32x4{0.f, 0.f, 0.f, 0.f};
    const int grow = row0 + row;
    const int gq = grow / n;
    const int i = grow - gq * n;
    const int h = kvh * G + gq;
    float* dst = o_part + ((((int64_t)b * Hq + h) * n + i) * S + s) * D + c4 * 4;
    *reinterpret_cast<f32x4*>(dst) = res;
  }
  for (int row = threadIdx.x; row < rows_here; row += NW * 64) {
    const float l = l_lds[row];
    const float lse = l > 0.f ? (m_lds[row] + log2_hw(l)) * kLn2 : -INFINITY;
    const int grow = row0 + row;
    const int gq = grow / n;
    const int i = grow - gq * n;
    const int h = kvh * G + gq;
    lse_part[(((int64_t)b * Hq + h) * n + i) * S + s] = lse;
  }
}

template <int D, int MT>
hipError_t launch_prefix(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                         int B, int Hq, int Hkv, int n, int64_t L_max, float scale_log2,
                         int64_t split_len, int S, int RG, float* o_part, float* lse_part,
                         hipStream_t stream) {
  dim3 grid((unsigned)S, (unsigned)(Hkv * RG), (unsigned)B);
  hipLaunchKernelGGL((prefix_kernel<D, MT>), grid, dim3(NW * 64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), seq_lens, Hq, Hkv, n, L_max, scale_log2,
                     split_len, S, RG, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace
}  // namespace rv

extern "C" rv_status spec_attn_prefix(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* seq_lens, int64_t max_seq_len, int B,
                                      int Hq, int Hkv, int n, int d, int64_t L_max,
                                      float sm_scale, int64_t split_len, int num_splits,
                                      float* o_part, float* lse_part, void* stream) {
  rv_status st = rv::check_prefix(q, k_cache, v_cache, seq_lens, max_seq_len, B, Hq, Hkv, n, d,
                                  L_max, sm_scale, split_len, num_splits, o_part, lse_part);
  if (st != RV_OK) return st;
  const rv::RowPlan rp = rv::row_plan(Hq, Hkv, n);
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
#define RV_PREFIX_CASE(DD, MM)                                                                  \
  if (d == DD && rp.MTW == MM)                                                                  \
    e = rv::launch_prefix<DD, MM>(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max,          \
                                  scale_log2, split_len, num_splits, rp.RG, o_part, lse_part, s);
  RV_PREFIX_CASE(64, 1)
  else RV_PREFIX_CASE(64, 2) else RV_PREFIX_CASE(64, 3) else RV_PREFIX_CASE(64, 4)
  else RV_PREFIX_CASE(128, 1) else RV_PREFIX_CASE(128, 2) else RV_PREFIX_CASE(128, 3)
  else RV_PREFIX_CASE(128, 4) else return RV_ERR_UNSUPPORTED;
#undef RV_PREFIX_CASE
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}
