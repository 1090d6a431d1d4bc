// spec_attn_prefix: unmasked attention of the verify rows over the history KV
// cache, split along the sequence (LongSpec summary, gist.science, section 2.3
// "Fast Tree Attention": the history key/value pairs need no mask, so they go
// to a plain fast attention pass whose result is later merged by log-sum-exp).
//
// Work decomposition (gfx950, 64-wide waves):
//   grid  = (split s, kv-head x row-group, sequence b); 4 waves per workgroup.
//   A workgroup owns one split of one (b, kv-head).  The G = Hq/Hkv query
//   heads of that kv-head share every K/V byte, so their G*n rows are stacked
//   into 16-row MFMA tiles (up to 4 per wave; larger groups use several row
//   groups).  Wave w streams the split's 32-key tiles w, w+4, w+8, ...
//
// Per tile:
//   * K and V arrive by non-temporal 16-byte buffer loads (read once; range-
//     checked, so keys past the split read as zero), one tile ahead of use.
//   * Scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_16x16x32_bf16 with K straight from registers as the A
//     operand (one load instruction covers 16 keys x 64 contiguous bytes).
//     In that layout a lane holds 8 scores of one query row: exactly the B
//     operand of the P V product, so P needs no shuffle.
//   * Online softmax in fp32, base-2 units, with a lazily raised running
//     max (raised only when a tile exceeds it by more than 8), so the fp32
//     accumulators are rescaled only on rare tiles; row max/sum across the
//     four lanes of a row use the gfx950 row-swap permutes.
//   * V is staged per wave in LDS in its natural [key][d] layout (row pitch
//     2d + 32 bytes) and read back transposed for the A operand of
//     O^T += V^T P^T with ds_read_b64_tr_b16, two reads per 16 columns.
// The four waves park their (max, sum, O) states in per-wave LDS slots; one
// thread per row turns the four (max, sum) pairs into the row's LSE and wave
// weights, and then all threads form and write one normalised partial
// (O, LSE) per row, with non-temporal stores (the merge reads it once, as a
// rule from another XCD).

#include <hip/hip_ext.h>

#include "rv_device.h"
#include "rv_internal.h"

namespace rv {
namespace {

constexpr int KT = kKeysPerTile;
constexpr int NW = kWavesPerGroup;
// Slack, in base-2 units, before the running max of a row is raised.
constexpr float kRescaleSlack = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Max over the four lanes lr + 16 g (g = 0..3) that share a row, with the
// gfx950 row-swap permutes (no LDS traffic).  Symmetric, so all four lanes
// get the same value.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
struct PrefixGeom {
  static constexpr int KS = D / 32;             // MFMA k-steps over the head dim
  static constexpr int NB = D / 16;             // 16-column blocks of the output
  static constexpr int VCH = KT * D / 8 / 64;   // 16-byte V chunks per lane per tile
  static constexpr int VROW = 2 * D + 32;       // bytes per key row of a V tile in LDS
  static constexpr int VTILE = KT * VROW;       // bytes per wave V tile
  static constexpr int OROW = D + 4;            // floats per row of the merge buffer
};

// One 32-key tile in registers: K as MFMA A fragments, V as 16-byte chunks.
template <int D>
struct TileRegs {
  i32x4 k[2][PrefixGeom<D>::KS];
  i32x4 v[PrefixGeom<D>::VCH];
};

// History pass over split s of the cache (no mask).
template <int D, int MT>
__global__ __launch_bounds__(NW * 64, 1) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ seq_lens, int Hq, int Hkv,
    int n, int64_t L_max, float scale_log2, int64_t split_len, int S, int RG,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  using Gm = PrefixGeom<D>;
  constexpr int KS = Gm::KS, NB = Gm::NB, VCH = Gm::VCH, VROW = Gm::VROW, OROW = Gm::OROW;
  constexpr int VBYTES = NW * Gm::VTILE;
  constexpr int OBYTES = NW * MT * 16 * OROW * 4;  // one merge slot per wave
  // The widest shape keeps its query fragments in LDS to stay within 512
  // registers per lane; the others keep them in registers.
  constexpr bool kQLds = (D == 128 && MT == 4);
  constexpr int QLDS_BYTES = kQLds ? MT * KS * 64 * 16 : 16;
  // Merge slots get LDS of their own where it fits next to the V tiles, so a
  // wave parks its state as soon as its own stream ends; otherwise they
  // reuse the V tiles' LDS after a barrier.
  constexpr bool kOwnSlots = VBYTES + OBYTES + QLDS_BYTES <= 150 * 1024;
  constexpr int SMEM = kOwnSlots ? VBYTES + OBYTES : (VBYTES > OBYTES ? VBYTES : OBYTES);
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ __attribute__((aligned(16))) bf16x8 q_lds[QLDS_BYTES / 16];
  __shared__ float m_lds[NW][MT * 16];
  __shared__ float l_lds[NW][MT * 16];

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
  bf16x8 qf[kQLds ? 1 : MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = row0 + mt * 16 + lr;
    bf16x8 frag[KS];
    if (row < M) {
      const int gq = row / n;
      const int i = row - gq * n;
      const int h = kvh * G + gq;
      const uint16_t* qp = q + (((int64_t)b * Hq + h) * n + i) * D + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) frag[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) frag[ks] = bf16x8{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kQLds) {
        if (wave == 0) q_lds[(mt * KS + ks) * 64 + lane] = frag[ks];
      } else {
        qf[kQLds ? 0 : mt][ks] = frag[ks];
      }
    }
  }
  if constexpr (kQLds) __syncthreads();
  auto qfrag = [&](int mt, int ks) -> bf16x8 {
    if constexpr (kQLds) return q_lds[(mt * KS + ks) * 64 + lane];
    else return qf[kQLds ? 0 : mt][ks];
  };

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

  // Loads past the split read zeros (buffer range check) and are never used.
  auto load_tile = [&](int tt, TileRegs<D>& r) {
    const uint32_t base = (uint32_t)tt * KT * D * 2;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        r.k[kb][ks] = buffer_load16_stream(
            krs, base + (uint32_t)(((kb * 16 + lr) * D + ks * 32 + lg * 8) * 2));
#pragma unroll
    for (int i = 0; i < VCH; ++i)
      r.v[i] = buffer_load16_stream(vrs, base + (uint32_t)((i * 64 + lane) * 16));
  };

  // Per-lane byte offsets into the wave's V tile for the transposed operand
  // reads: in 16-lane group lg, source lane sl = 4 e + q points at
  // V[key 16 h + 4 lg + e][16 nb + 4 q]; ds_read_b64_tr_b16 then hands lane
  // (lr, lg) the four values V[16 h + 4 lg + e][16 nb + lr], e = 0..3.
  const int sl = lane & 15;
  const int vtr_off = (4 * lg + (sl >> 2)) * VROW + (sl & 3) * 8;

  auto compute_tile = [&](const TileRegs<D>& r, int t) {
    // Stage the V tile in its natural [key][d] layout: chunk c = 64 i + lane
    // is key c / (D/8), columns 8 (c % (D/8)) .. +7.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = i * 64 + lane;
      const int key = c / (D / 8);
      const int dch = c - key * (D / 8);
      *reinterpret_cast<i32x4*>(vt + key * VROW + dch * 16) = r.v[i];
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
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[kb][ks]),
                                                        qfrag(mt, ks), acc, 0, 0, 0);
        sacc[kb][mt] = acc;
      }

    // Keys past the split are masked only in a split's partial last tile.
    if ((t + 1) * KT > nkeys) {
      const int key0 = t * KT + lg * 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (key0 + kb * 16 + v >= nkeys) sacc[kb][mt][v] = -INFINITY;
          }
    }

    // Online softmax with a lazily updated running max: row lr's scores for
    // keys 16 kb + 4 lg + v live in lanes lr + 16 g.  The running max m_run
    // (base-2 units) is raised only when a tile's max exceeds it by more
    // than kRescaleSlack, so p = 2^(x - m_run) <= 2^kRescaleSlack and the
    // accumulators are rescaled only on those rare tiles.
    bf16x8 pf[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][mt][0], sacc[0][mt][1]),
                             fmaxf(sacc[0][mt][2], sacc[0][mt][3])),
                       fmaxf(fmaxf(sacc[1][mt][0], sacc[1][mt][1]),
                             fmaxf(sacc[1][mt][2], sacc[1][mt][3])));
      mx = row_max4(mx);
      const float m_tile = mx * scale_log2;
      const bool raise = m_tile > m_run[mt] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float m_new = raise ? m_tile : m_run[mt];
        const float alpha = exp2_hw(m_run[mt] - m_new);
        l_run[mt] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][mt] *= alpha;
        m_run[mt] = m_new;
      }
      // (every tile holds a valid key, so m_run is finite from here on;
      // the guard keeps an empty state well defined)
      const float neg_m = (m_run[mt] == -INFINITY) ? 0.f : -m_run[mt];
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = exp2_hw(fmaf(sacc[kb][mt][v], scale_log2, neg_m));
          ps += p;
          pf[mt][kb * 4 + v] = (__bf16)p;
        }
      l_run[mt] += ps;
    }

    // O^T += V^T P^T: A operand lane (column d = 16 nb + lr, group lg) holds
    // V[key][d] for keys 4 lg + e (e < 4) and 16 + 4 lg + (e - 4) (e >= 4),
    // the same key order as pf; two transposed LDS reads per operand.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const unsigned char* base = vt + vtr_off + nb * 32;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(base + 16 * VROW));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        oacc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[mt], oacc[nb][mt], 0, 0, 0);
    }
  };

  // Two register buffers: while tile t is computed, tile t + NW of this wave
  // is in flight.  (Measured on MI355X at the 8B shape: a third buffer, which
  // costs registers and 3x unrolled code, is ~1.5 us slower per launch.)
  TileRegs<D> ra, rb;
  int t = wave;
  if (t < ntiles) {
    load_tile(t, ra);
    for (;;) {
      load_tile(t + NW, rb);
      compute_tile(ra, t);
      t += NW;
      if (t >= ntiles) break;
      load_tile(t + NW, ra);
      compute_tile(rb, t);
      t += NW;
      if (t >= ntiles) break;
    }
  }

  // Row sums: each lane holds a quarter of its row's keys.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) l_run[mt] = row_sum4(l_run[mt]);

  // Each wave parks its state (running max, row sum, unnormalised O) in its
  // own LDS slot.  After a barrier one thread per row turns the four
  // (max, sum) pairs into the row's LSE and per-wave weights
  // 2^(m_w - M) / l; after a second barrier every thread forms its share of
  // the normalised partial with all of its LDS reads in one unrolled batch.
  if constexpr (!kOwnSlots) __syncthreads();  // V tiles dead: their LDS becomes the slots
  float* obuf = reinterpret_cast<float*>(smem + (kOwnSlots ? VBYTES : 0));
  {
    float* slot = obuf + wave * (MT * 16 * OROW);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = mt * 16 + lr;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<f32x4*>(slot + row * OROW + nb * 16 + lg * 4) = oacc[nb][mt];
      if (lg == 0) {
        m_lds[wave][row] = m_run[mt];
        l_lds[wave][row] = l_run[mt];
      }
    }
  }
  __syncthreads();

  auto out_row = [&](int row) {  // (b, h, i) index of local row `row`
    const int grow = row0 + row;
    const int gq = grow / n;
    const int i = grow - gq * n;
    return ((int64_t)b * Hq + kvh * G + gq) * n + i;
  };
  if ((int)threadIdx.x < rows_here) {
    const int row = threadIdx.x;
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = m_lds[w][row];
      M = fmaxf(M, mw[w]);
    }
    float a[NW], l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      a[w] = (mw[w] == -INFINITY) ? 0.f : exp2_hw(mw[w] - M);
      l += a[w] * l_lds[w][row];
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) m_lds[w][row] = a[w] * inv;  // this row's weights
    lse_part[out_row(row) * S + s] = l > 0.f ? (M + log2_hw(l)) * kLn2 : -INFINITY;
  }
  __syncthreads();

  constexpr int ITEMS = MT * 16 * (D / 4);  // f32x4 items of the partial
  constexpr int PER_T = (ITEMS + NW * 64 - 1) / (NW * 64);
#pragma unroll
  for (int j = 0; j < PER_T; ++j) {
    const int idx = threadIdx.x + j * NW * 64;
    const int row = idx / (D / 4);
    const int c4 = idx - row * (D / 4);
    if (row < rows_here) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w)
        o += m_lds[w][row] * *reinterpret_cast<const f32x4*>(obuf + (w * MT * 16 + row) * OROW +
                                                             c4 * 4);
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(o_part + (out_row(row) * S + s) * D +
                                                          c4 * 4));
    }
  }
}

// With start/stop events the launch records them on the kernel's own
// dispatch (hipExtLaunchKernel), so their elapsed time is the kernel's.
template <int D, int MT>
hipError_t launch_attn(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                       int B, int Hq, int Hkv, int n, int64_t L_max, float scale_log2,
                       int64_t split_len, int S, int RG, float* o_part, float* lse_part,
                       hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  dim3 grid((unsigned)S, (unsigned)(Hkv * RG), (unsigned)B);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (ev_start != nullptr || ev_stop != nullptr)
    hipExtLaunchKernelGGL((attn_kernel<D, MT>), grid, dim3(NW * 64), 0, stream, ev_start,
                          ev_stop, 0, qq, kk, vv, seq_lens, Hq, Hkv, n, L_max, scale_log2,
                          split_len, S, RG, o_part, lse_part);
  else
    hipLaunchKernelGGL((attn_kernel<D, MT>), grid, dim3(NW * 64), 0, stream, qq, kk, vv,
                       seq_lens, Hq, Hkv, n, L_max, scale_log2, split_len, S, RG, o_part,
                       lse_part);
  return hipGetLastError();
}

rv_status dispatch_attn(int d, int MTW, const void* q, const void* k, const void* v,
                        const int32_t* seq_lens, int B, int Hq, int Hkv, int n, int64_t L_max,
                        float scale_log2, int64_t split_len, int S, int RG, float* o_part,
                        float* lse_part, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  hipError_t e;
#define RV_ATTN_CASE(DD, MM)                                                                 \
  if (d == DD && MTW == MM)                                                                  \
    e = launch_attn<DD, MM>(q, k, v, seq_lens, B, Hq, Hkv, n, L_max, scale_log2, split_len,  \
                            S, RG, o_part, lse_part, s, e0, e1);
  RV_ATTN_CASE(64, 1)
  else RV_ATTN_CASE(64, 2) else RV_ATTN_CASE(64, 3) else RV_ATTN_CASE(64, 4)
  else RV_ATTN_CASE(128, 1) else RV_ATTN_CASE(128, 2) else RV_ATTN_CASE(128, 3)
  else RV_ATTN_CASE(128, 4) else return RV_ERR_UNSUPPORTED;
#undef RV_ATTN_CASE
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
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
  return rv::dispatch_attn(d, rp.MTW, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max,
                           scale_log2, split_len, num_splits, rp.RG, o_part, lse_part,
                           static_cast<hipStream_t>(stream), nullptr, nullptr);
}

extern "C" rv_status spec_attn_prefix_ev(const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* seq_lens,
                                         int64_t max_seq_len, int B, int Hq, int Hkv, int n,
                                         int d, int64_t L_max, float sm_scale, int64_t split_len,
                                         int num_splits, float* o_part, float* lse_part,
                                         void* stream, void* start_event, void* stop_event) {
  rv_status st = rv::check_prefix(q, k_cache, v_cache, seq_lens, max_seq_len, B, Hq, Hkv, n, d,
                                  L_max, sm_scale, split_len, num_splits, o_part, lse_part);
  if (st != RV_OK) return st;
  const rv::RowPlan rp = rv::row_plan(Hq, Hkv, n);
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  return rv::dispatch_attn(d, rp.MTW, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max,
                           scale_log2, split_len, num_splits, rp.RG, o_part, lse_part,
                           static_cast<hipStream_t>(stream),
                           static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event));
}
