// spec_attn_prefix: unmasked attention of the verify rows over the history KV
// cache, split along the sequence (LongSpec summary, gist.science, section 2.3
// "Fast Tree Attention": the history key/value pairs need no mask, so they go
// to a plain fast attention pass whose result is later merged by log-sum-exp).
//
// Work decomposition (gfx950, 64-wide waves):
//   grid  = S x Hkv x B workgroups, one per (split s, kv-head, sequence b)
//   slot; for one sequence workgroup (s, kv-head) is its grid position, for
//   a batch the slots that hold keys are numbered so that they spread evenly
//   over the XCDs (split_item).  A workgroup owns one split of one
//   (b, kv-head).  The G = Hq/Hkv query heads of that kv-head share every
//   K/V byte, so their G*n rows are stacked into 16-row MFMA tiles, and one
//   workgroup takes all of them, so every byte of the split is read once.
//   Up to 4 row tiles (64 rows): attn_kernel below, 4 waves, wave w streams
//   the split's 32-key tiles w, w+4, w+8, ... through its own registers.
//   More rows: attn_wide_kernel further down, which stages K/V in LDS for
//   all waves (its own notes describe it).
//
// attn_kernel, per tile:
//   * K and V arrive by non-temporal 16-byte buffer loads (read once; range-
//     checked, so keys past the split read as zero), one tile ahead of use.
//   * Scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_16x16x32_bf16 with K straight from registers as the A
//     operand (one load instruction covers 16 keys x 64 contiguous bytes).
//     In that layout a lane holds 8 scores of one query row: exactly the B
//     operand of the P V product, so P needs no shuffle.
//   * Online softmax in fp32, base-2 units, with a lazily raised running
//     max (raised only when a tile exceeds it by more than 8), so the fp32
//     accumulators are rescaled only on rare tiles; each lane tests its own
//     8 scores first, and only on those tiles is the row max taken across
//     the four lanes of a row (gfx950 row-swap permutes, as the row sum).
//   * V is staged per wave in LDS in its natural [key][d] layout (row pitch
//     2d + 32 bytes) and read back transposed for the A operand of
//     O^T += V^T P^T with ds_read_b64_tr_b16, two reads per 16 columns.
// The four waves park their (max, sum, O) states in per-wave LDS slots; one
// thread per row turns the four (max, sum) pairs into the row's LSE and wave
// weights, and then all threads form and write one normalised partial
// (O, LSE) per row, with non-temporal stores (the merge reads it once, as a
// rule from another XCD).

#include <hip/hip_ext.h>

#include <utility>

#include "block_row.h"
#include "merge_fold.h"
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

// Which (sequence b, kv head, split s) this workgroup takes.  The triples
// whose split holds keys are numbered in (b, kv head, s) order and item w
// goes to the workgroup of linear index w.  The hardware hands workgroups to
// the 8 XCDs round-robin by linear index, so the busy workgroups spread
// evenly over the XCDs and their compute units whatever the batch's lengths
// (with the plain (s, kv head, b) grid a ragged batch can put more busy
// workgroups on one XCD than it has units).  Workgroups past the last item
// take the empty slots, in the same order, and write their empty partials.
// Slot s of sequence b always covers keys [s * split_len, (s+1) * split_len).
struct SplitItem {
  int b, kvh, s;
};

__device__ __forceinline__ int64_t wave_incl_scan64(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ SplitItem split_item(const int32_t* __restrict__ seq_lens, int B, int Hkv, int S,
                                int64_t L_max, int64_t split_len) {
  // One sequence: the plain grid position (its busy splits are the first of
  // every kv head's row of S, so they already spread over the XCDs), with
  // no length load in front of the workgroup's first request.
  if (B == 1) return SplitItem{0, (int)blockIdx.y, (int)blockIdx.x};
  const int lane = threadIdx.x & 63;
  const int64_t w =
      blockIdx.x + (int64_t)S * (blockIdx.y + (int64_t)Hkv * (int64_t)blockIdx.z);
  // splits of sequence b that hold keys (at most S)
  auto busy = [&](int b) -> int {
    int64_t L = seq_lens[b];
    L = L < 0 ? 0 : (L > L_max ? L_max : L);
    const int64_t p = (L + split_len - 1) / split_len;
    return (int)(p < S ? p : S);
  };
  // number of busy triples (the first 64 sequences' counts stay in a
  // register for the search below: one load round trip for B <= 64)
  const int p_first = lane < B ? busy(lane) : 0;
  int64_t N = __shfl(wave_incl_scan64(p_first), 63, 64);
  for (int b0 = 64; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int64_t c = b < B ? (int64_t)busy(b) : 0;
    N += __shfl(wave_incl_scan64(c), 63, 64);
  }
  N *= Hkv;
  // item w among the busy triples, or w - N among the empty slots: find the
  // sequence whose running count passes the target, then (kv head, s) in it
  const bool empty = w >= N;
  const int64_t target = empty ? w - N : w;
  int64_t base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int p = b0 == 0 ? p_first : (b < B ? busy(b) : 0);
    const int per = b < B ? (empty ? S - p : p) : 0;  // slots per kv head
    const int64_t c = (int64_t)per * Hkv;
    const int64_t incl = base + wave_incl_scan64(c);
    const uint64_t hit = __ballot(b < B && incl > target);
    if (hit != 0) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      const int64_t excl = __shfl(incl - c, l, 64);
      const int pl = __shfl(p, l, 64);
      const int perl = __shfl(per, l, 64);
      const int64_t r = target - excl;  // < perl * Hkv
      const int kvh = (int)(r / perl);
      const int j = (int)(r - (int64_t)kvh * perl);
      // (uniform across the wave: keep it in scalar registers)
      SplitItem it;
      it.b = __builtin_amdgcn_readfirstlane(b0 + l);
      it.kvh = __builtin_amdgcn_readfirstlane(kvh);
      it.s = __builtin_amdgcn_readfirstlane(empty ? pl + j : j);
      return it;
    }
    base = __shfl(incl, 63, 64);
  }
  // unreachable for a grid of S * Hkv * B workgroups (every slot is either
  // busy or empty); keep a defined answer
  SplitItem it{B - 1, Hkv - 1, S - 1};
  return it;
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

// What the single-launch verify pass (attn_kernel<D, MT, true>) needs beyond
// the history pass: the draft block, the merged outputs and one pair of
// sync words per (sequence, kv head).
template <bool FUSE>
struct TailArgs {};
template <>
struct TailArgs<true> {
  const uint16_t* k_blk;     // [B][Hkv][n][D] bf16
  const uint16_t* v_blk;     // [B][Hkv][n][D] bf16
  uint16_t* out;             // [B][Hq][n][D] bf16
  float* lse_out;            // [B][Hq][n] or null
  uint64_t* sync;            // [B][Hkv][2]: mask of published splits, finished count
  uint32_t help_ticks;       // wait (100 MHz ticks) before computing a missing split
  BlockMask mask;            // visibility bits of the block rows
};

// The fused tail: after its own split, a workgroup (b, kv head, s) waits for
// the other splits of its (b, kv head) and then merges local rows
// s, s + S, s + 2S, ... < M (LongSpec summary, section 2.3: the history part
// and the masked block part are combined by log-sum-exp), so the merge needs
// no launch of its own.  It is taken for small grids only (the host rule in
// rv_verify_single_launch: at most 64 workgroups, at most one merged row per
// wave), where it saves the second launch; on the full 8B-shaped layer the
// cross-XCD publish and poll below cost more than a kernel boundary.
//   * Publish: the split's partials are written with device-scope stores,
//     which leave no dirty lines in the XCD's L2 (plain stores made the
//     release below write back ~20 us of L2 at 256 workgroups); every wave
//     waits for its stores to complete, the workgroup meets at a barrier,
//     and one thread sets the split's bit in the group's mask word with an
//     agent-scope release.
//   * Block part: then wave w computes the block attention of its first row
//     (local row s + w S; block_row.h) while the other splits finish.
//     (Before the split's first tiles, its time lands on every split;
//     issuing its loads during the split's epilogue gained nothing.)
//   * Wait: one thread polls the mask word, then takes an agent-scope
//     acquire before the workgroup reads the partials.  The launch is used
//     only when every workgroup of the grid fits on the device at once, but
//     other work may hold compute units; so a workgroup that has waited
//     help_ticks computes the first missing split after its own itself and
//     publishes it.  A split computed twice is written twice with the same
//     bits, and every wait ends: each help sets a bit, so after at most S
//     helps the mask is full.
//   * Merge: wave w merges rows s + w S, s + (w + 4) S, ...: the row's S
//     partials (device-scope loads) in ascending split order against their
//     maximum, then the block part, as in spec_attn_block_merge (one wave per
//     row here, so the sums run in a different order: equal up to fp32
//     rounding).
//   * The finished count: each workgroup adds one once it needs the mask no
//     more (after its own bits are set); the last of the S clears both
//     words, so they are zero again for the next call (the caller zero-fills
//     them once).

// Wait until every vector-memory access this wave issued has completed
// (stores acknowledged at their scope); also a compiler barrier.
__device__ __forceinline__ void wait_vm_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, typename RunSplit>
__device__ __forceinline__ void verify_tail(RunSplit& run_split, const TailArgs<true>& vt,
                                            const uint16_t* __restrict__ q, int Hq, int Hkv,
                                            int n, float scale_log2, int S,
                                            const float* __restrict__ o_part,
                                            const float* __restrict__ lse_part, int b, int kvh,
                                            int s0, int M) {
  constexpr int PER = D / 64;
  __shared__ int sh_next;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = Hq / Hkv;
  uint64_t* const mword = vt.sync + 2 * ((size_t)b * Hkv + kvh);
  uint64_t* const fword = mword + 1;
  const uint64_t full = S >= 64 ? ~0ull : ((1ull << S) - 1ull);
  const size_t kv0 = ((size_t)b * Hkv + kvh) * (size_t)n * D;
  auto grow_of = [&](int r) -> int64_t {  // (b, h, i) index of local row r
    const int gq = r / n;
    const int i = r - gq * n;
    return ((int64_t)b * Hq + kvh * G + gq) * n + i;
  };
  auto block_part = [&](int r, float (&ob)[PER], float& lb2) {
    block_row_attention<D>(q + grow_of(r) * D, vt.k_blk + kv0, vt.v_blk + kv0,
                           vt.mask.bits[r % n], n, scale_log2, ob, lb2);
  };
  // (after this thread's own mask updates have completed)
  auto finish = [&]() {
    wait_vm_stores();
    const uint64_t old =
        __hip_atomic_fetch_add(fword, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint64_t)(S - 1)) {
      __hip_atomic_store(mword, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(fword, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // Every wave's device-scope partial stores complete, then split sp is
  // marked done with a release: a workgroup that sees the bit and then
  // acquires (wait() below) sees the partials.
  auto publish = [&](int sp) {
    wait_vm_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_or(mword, 1ull << sp, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  };
  // -1 once every split of the group is published (and this workgroup is
  // counted out), else the split to compute on another's behalf.
  auto wait = [&]() -> int {
    if (threadIdx.x == 0) {
      int next = -1;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        const uint64_t m = __hip_atomic_load(mword, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((m & full) == full) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 >= vt.help_ticks) {
          for (int t = 1; t <= S; ++t) {  // first missing split after this one
            const int u = (s0 + t) % S;
            if (!((m >> u) & 1ull)) {
              next = u;
              break;
            }
          }
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      // (pairs with the releases of the splits seen published; the barrier
      // below passes the ordering on to the other waves)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (next < 0) finish();
      sh_next = next;
    }
    __syncthreads();
    return sh_next;
  };

  float ob[PER], lb2 = 0.f;
  const int r_first = s0 + wave * S;  // this wave's first row
  run_split(s0);
  publish(s0);
  if (s0 >= M) {  // no row to merge here
    if (threadIdx.x == 0) finish();
    return;
  }
  if (r_first < M) block_part(r_first, ob, lb2);
  // (a split to help with: the barrier in wait() ended every LDS read of the
  // last one, so run_split may reuse the LDS)
  for (int u = wait(); u >= 0; u = wait()) {
    run_split(u);
    publish(u);
  }

  for (int j = wave;; j += NW) {
    const int r = s0 + j * S;
    if (r >= M) break;
    if (j != wave) block_part(r, ob, lb2);
    const int64_t grow = grow_of(r);
    const float* lp = lse_part + grow * S;
    const float* op = o_part + grow * S * D + lane * PER;
    PartialFold<D, 1, 32, true> pf;
    pf.load(op, lp, S, 0, 0);
    float Ms = -INFINITY;
    for (int t = lane; t < S; t += 64) Ms = fmaxf(Ms, partial_load<true>(lp + t));
    Ms = wave_max(Ms);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    if (Ms != -INFINITY) pf.fold(op, lp, S, 0, Ms, acc, wsum);
    const float lb = lb2 * kLn2;  // finite: a row always sees itself
    const float Mx = fmaxf(Ms, lb);
    const float fs = (Ms == -INFINITY) ? 0.f : exp2_hw((Ms - Mx) * kLog2e);
    const float fb = exp2_hw((lb - Mx) * kLog2e);
    const float tot = fmaf(fs, wsum, fb);
    const float inv = 1.0f / tot;  // tot >= fb = 1 or fs * wsum >= 1
    uint16_t* dst = vt.out + grow * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = f32_to_bf16_bits(fmaf(fs, acc[e], fb * ob[e]) * inv);
    if (vt.lse_out != nullptr && lane == 0) vt.lse_out[grow] = Mx + log2_hw(tot) * kLn2;
  }
}

// History pass over split s of the cache (no mask).  With FUSE the same
// launch also computes the draft-block part and merges the result (see the
// notes at the fused tail below).
template <int D, int MT, bool FUSE>
__global__ __launch_bounds__(NW * 64, 1) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ seq_lens, int Hq, int Hkv,
    int n, int64_t L_max, float scale_log2, int64_t split_len, int S,
    float* __restrict__ o_part, float* __restrict__ lse_part, const TailArgs<FUSE> vt) {
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

  const SplitItem item = split_item(seq_lens, (int)gridDim.z, Hkv, S, L_max, split_len);
  const int kvh = item.kvh;
  const int b = item.b;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int G = Hq / Hkv;
  const int M = G * n;

  int64_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > L_max ? L_max : L);

  // The partial (O, LSE) of split s for every row of the group.
  auto run_split = [&](const int s) {
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
    const int row = mt * 16 + lr;
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
      // The lane's own 8 scores decide whether any row of the tile may
      // raise (the row max exceeds the threshold exactly when one of its
      // lanes' maxima does); only then is the row max formed.
      const float lmx = fmaxf(fmaxf(fmaxf(sacc[0][mt][0], sacc[0][mt][1]),
                                    fmaxf(sacc[0][mt][2], sacc[0][mt][3])),
                              fmaxf(fmaxf(sacc[1][mt][0], sacc[1][mt][1]),
                                    fmaxf(sacc[1][mt][2], sacc[1][mt][3])));
      if (__builtin_amdgcn_ballot_w64(lmx * scale_log2 > m_run[mt] + kRescaleSlack)) {
        const float m_tile = row_max4(lmx) * scale_log2;
        const bool raise = m_tile > m_run[mt] + kRescaleSlack;
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
    const int gq = row / n;
    const int i = row - gq * n;
    return ((int64_t)b * Hq + kvh * G + gq) * n + i;
  };
  if ((int)threadIdx.x < M) {
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
    const float lse_s = l > 0.f ? (M + log2_hw(l)) * kLn2 : -INFINITY;
    if constexpr (FUSE)  // device-scope store: read by other XCDs in this launch
      __hip_atomic_store(lse_part + out_row(row) * S + s, lse_s, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      lse_part[out_row(row) * S + s] = lse_s;
  }
  __syncthreads();

  constexpr int ITEMS = MT * 16 * (D / 4);  // f32x4 items of the partial
  constexpr int PER_T = (ITEMS + NW * 64 - 1) / (NW * 64);
#pragma unroll
  for (int j = 0; j < PER_T; ++j) {
    const int idx = threadIdx.x + j * NW * 64;
    const int row = idx / (D / 4);
    const int c4 = idx - row * (D / 4);
    if (row < M) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w)
        o += m_lds[w][row] * *reinterpret_cast<const f32x4*>(obuf + (w * MT * 16 + row) * OROW +
                                                             c4 * 4);
      float* const dst = o_part + (out_row(row) * S + s) * D + c4 * 4;
      if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_store(dst + e, o[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(dst));
      }
    }
  }
  };

  if constexpr (!FUSE) {
    run_split(item.s);
  } else {
    verify_tail<D>(run_split, vt, q, Hq, Hkv, n, scale_log2, S, o_part, lse_part, b, kvh, item.s,
                   M);
  }
}

// History pass for wide groups (more than 64 rows per kv head: 64/8 heads
// with 11 verify rows, a 32-node tree over 4 heads per kv head).  One
// workgroup takes every row of the group, so each K/V byte of the split
// leaves HBM once, and each wave runs every key against its own row tiles
// mt = wave, wave + 4, ... (MTW of them; a tile past the group's rows holds
// zero queries and is never written).  A wave holds complete rows, so it
// normalises and writes its own partials.
//
// K/V move HBM -> LDS with gfx950's 16-byte buffer loads into LDS (no
// register staging), in 64-key stages through a ring of kBufs LDS buffers:
// while stage st is computed, stages st + 1 .. st + kBufs - 1 are in flight.
// Each 1 KB load instruction lands in one contiguous 1 KB LDS block (lane L
// at 16 L) and reads whole 128-byte lines: 8 keys x 128 bytes (half a key
// row at d = 128), lane L taking row L / 8.  Within a row the eight 16-byte
// chunks are stored permuted, chunk c at slot c ^ f(row), so that the MFMA
// operand reads spread over all LDS banks:
//   * K (A operand, ds_read_b128 of 16 keys x 16 bytes): f = r ^ (g & 1)
//     for row r of 8-row group g;
//   * V (ds_read_b64_tr_b16 of 4 keys x 32 bytes per 16 lanes):
//     f = 2 ((r1 ^ r2) << 1 | (r0 ^ r2)) over the bits r2 r1 r0 of r.
// (Loads of 16 keys x 64 bytes, one operand per instruction, leave half of
// every line to another wave's instruction and stream ~15% slower.)
// Every load reads a key inside the split (keys past its end are clamped to
// its last key, whose scores are then masked), so no padding is ever read.
// The pipeline's waits are explicit: a wave waits for its own loads of
// stage st (vmcnt counts them in issue order), then a barrier makes the
// whole stage visible and frees stage st - 1's buffer for reuse.
// s_waitcnt encoding (gfx9 family) for vmcnt(0), expcnt and lgkmcnt at
// their maxima (no wait on them).
constexpr int kWaitVmcnt0 = 0x0F70;

template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Chunk permutation of the V rows (see the layout note above).
__device__ __forceinline__ int swz_v(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1;
  return 2 * (((r1 ^ r2) << 1) | (r0 ^ r2));
}

template <int D, int NWV>
struct WideGeom {
  static constexpr int KS = D / 32, NB = D / 16;
  static constexpr int SK = 64;                  // keys per stage
  static constexpr int HALVES = D / 64;          // 128-byte lines per key row
  static constexpr int KBLK = (SK / 8) * HALVES; // 1 KB K blocks per stage (8 keys x 128 B)
  static constexpr int VBLK = KBLK;              // and V blocks
  static constexpr int NI = KBLK + VBLK;         // 1 KB loads per stage
  static constexpr int PW = NI / NWV;            // of which each wave issues
  static constexpr int KPW = KBLK / NWV;         // the first KPW of a wave's loads are K
  static constexpr int STAGE = NI * 1024;
  static constexpr int kBufs = (128 * 1024) / STAGE;
  static_assert(KBLK % NWV == 0 && VBLK % NWV == 0, "loads must split evenly over the waves");
  static_assert(kBufs >= 2 && (kBufs - 2) * PW <= 63, "vmcnt range");
};

typedef __attribute__((address_space(3))) const unsigned char lds_cu8;

// ds_read_b64_tr_b16 issued from inline asm.  The compiler treats the
// builtin as a possible reader of every pending LDS-DMA write and waits for
// all of them (vmcnt(0)) in front of it, which would drain the load
// pipeline every tile; here the pipeline's explicit waits already order it.
// The result is valid only after lds_wait().
template <int OFF>
__device__ __forceinline__ s16x4 ds_read_tr16_asm(uint32_t lds_addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "n"(OFF));
  return r;
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector-memory loads are outstanding,
// then meet the workgroup at a barrier.  LDS reads of earlier stages are
// complete too (lgkmcnt), so the buffer they used may be refilled.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int PW, int K>
__device__ __forceinline__ void wait_stage(int ahead) {
  if constexpr (K == 0) {
    wait_vm_barrier<0>();
  } else {
    if (ahead >= K) wait_vm_barrier<K * PW>();
    else wait_stage<PW, K - 1>(ahead);
  }
}

// KP key phases: 4 * KP waves; wave w computes the tiles tt of each stage
// with tt % KP == w / 4 (its phase) for a contiguous run of the group's row
// tiles (at most MTW).  With KP = 2 two waves share every SIMD (waves w and
// w + 4), so one wave's MFMA and LDS latencies hide behind the other's
// softmax, and the two phases of a row tile merge at the end.  The runs are
// sized so that the two waves of a SIMD together hold as even a share of
// the 2 MT (row tile, phase) units as possible: phase 0 gives the extra
// tiles to its first waves, phase 1 to its last.
template <int D, int MTW, int KP>
__global__ __launch_bounds__(NW * KP * 64, 1) void attn_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ seq_lens, int Hq, int Hkv,
    int n, int64_t L_max, float scale_log2, int64_t split_len, int S,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  constexpr int NWV = NW * KP;
  using W = WideGeom<D, NWV>;
  constexpr int KS = W::KS, NB = W::NB, SK = W::SK, PW = W::PW, KPW = W::KPW;
  constexpr int STAGE = W::STAGE, NBUF = W::kBufs;
  constexpr int TPS = SK / KT;  // 32-key tiles per stage
  static_assert(TPS % KP == 0, "each phase takes whole tiles of a stage");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NBUF * STAGE];

  const SplitItem item = split_item(seq_lens, (int)gridDim.z, Hkv, S, L_max, split_len);
  const int s = item.s;
  const int kvh = item.kvh;
  const int b = item.b;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rgw = wave % NW;    // row-tile owner
  const int phase = wave / NW;  // key phase
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int G = Hq / Hkv;
  const int M = G * n;
  const int MT = (M + 15) / 16;
  const int tbase = MT / NW, textra = MT - (MT / NW) * NW;
  const int tcnt = phase == 0 ? tbase + (rgw < textra) : tbase + (rgw >= NW - textra);
  const int tfirst = phase == 0 ? rgw * tbase + min(rgw, textra)
                                : rgw * tbase + max(0, rgw - (NW - textra));

  int64_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > L_max ? L_max : L);
  const int64_t kbeg = (int64_t)s * split_len;
  int64_t kend = kbeg + split_len;
  if (kend > L) kend = L;
  const int nkeys = kend > kbeg ? (int)(kend - kbeg) : 0;
  const int nst = (nkeys + SK - 1) / SK;

  // Query fragments (B operand of S^T = K Q^T) of this wave's row tiles.
  bf16x8 qf[MTW][KS];
#pragma unroll
  for (int j = 0; j < MTW; ++j) {
    const int row = (tfirst + j) * 16 + lr;
    if (j < tcnt && row < M) {
      const int gq = row / n;
      const int i = row - gq * n;
      const uint16_t* qp = q + (((int64_t)b * Hq + kvh * G + gq) * n + i) * D + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[j][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[j][ks] = bf16x8{};
    }
  }

  const size_t slab = ((size_t)b * Hkv + kvh) * (size_t)L_max * D + (size_t)kbeg * D;
  const uint32_t nbytes = (uint32_t)nkeys * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + slab, nbytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + slab, nbytes);

  // This wave issues loads i = wave + NWV j (j < PW) of every stage; loads
  // below KBLK are K blocks, the rest V blocks.  Per lane: the key within
  // the stage and the byte offset within the key's row.
  constexpr int HALVES = W::HALVES;
  const int r8 = lane >> 3;  // row of the lane within its load's 8 keys
  int key_l[PW], col_b[PW];
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int i = wave + NWV * j;
    const int blk = j < KPW ? i : i - W::KBLK;
    const int g = blk / HALVES, h = blk - (blk / HALVES) * HALVES;
    const int f = j < KPW ? (r8 ^ (g & 1)) : swz_v(r8);
    key_l[j] = 8 * g + r8;
    col_b[j] = 128 * h + 16 * ((lane & 7) ^ f);
  }
  // Per-lane LDS offsets of the operand reads within a tile's blocks.
  // K, k-step ks: row lr of the 16-key block, chunk 4 (ks & 1) + lg.
  const int kx = lg ^ (lr & 7) ^ (lr >> 3);
  const uint32_t krow = (uint32_t)((lr >> 3) * HALVES * 1024 + (lr & 7) * 128);
  const uint32_t kofs[2] = {krow + 16u * (uint32_t)kx, krow + 16u * (uint32_t)(kx ^ 4)};
  // V, 16-column group nb: source lane 4 e + c4 of 16-lane group lg reads
  // key 4 lg + e of the 16-key block, columns 16 nb + 4 c4 .. + 3, i.e.
  // chunk 2 (nb % 4) + c4 / 2 of line nb / 4, byte 8 (c4 & 1).
  const int vr = 4 * (lg & 1) + ((lane & 15) >> 2);
  const int vy = ((lane & 3) >> 1) | swz_v(vr);
  const uint32_t vrow = (uint32_t)((lg >> 1) * HALVES * 1024 + vr * 128 + 8 * (lane & 1));
  uint32_t vofs[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) vofs[m] = vrow + 16u * (uint32_t)((2 * m) ^ vy);
  auto issue_stage = [&](int st) {
    unsigned char* buf = smem + (st % NBUF) * STAGE;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int i = wave + NWV * j;
      const int key = min(st * SK + key_l[j], nkeys - 1);
      const uint32_t off = (uint32_t)key * (D * 2) + (uint32_t)col_b[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          j < KPW ? krs : vrs, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16,
          off, 0, 0, 2);
    }
  };

  f32x4 oacc[NB][MTW];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < MTW; ++j) oacc[nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Running max (base 2), its negation as the exponent offset (0 while the
  // row has seen no key), and the row sum as a 16-column MFMA accumulator
  // of P against a ones operand: every lane then holds its row's full sum,
  // taken over the same bf16-rounded p that multiply V.
  float m_run[MTW], neg_m[MTW], thr[MTW];  // thr = m_run + kRescaleSlack
  f32x4 lacc[MTW];
#pragma unroll
  for (int j = 0; j < MTW; ++j) {
    m_run[j] = -INFINITY;
    neg_m[j] = 0.f;
    thr[j] = -INFINITY;
    lacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // One 32-key tile t; kt: the stage's K blocks of its two 16-key blocks,
  // vt: their V blocks.  Score layout, online softmax and P V product as
  // in the per-wave streaming kernel above.
  auto compute_tile = [&](const unsigned char* kt, const unsigned char* vt, int t) {
    bf16x8 kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[kb][ks] = *reinterpret_cast<const bf16x8*>(
            kt + kofs[ks & 1] + (2 * kb * HALVES + (ks >> 1)) * 1024);
    f32x4 sacc[2][MTW];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (j == 0 || j < tcnt) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][ks], qf[j][ks], acc, 0, 0, 0);
        }
        sacc[kb][j] = acc;
      }
    // V operands next (after the K reads the score MFMAs wait for): their
    // LDS latency hides behind the scores and the softmax.
    s16x4 vlo[NB], vhi[NB];
    const uint32_t vbase = (uint32_t)(uintptr_t)(lds_cu8*)vt;
    uint32_t vaddr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) vaddr[m] = vbase + vofs[m];
    static_for<NB>([&](auto nb) {
      vlo[nb] = ds_read_tr16_asm<(nb / 4) * 1024>(vaddr[nb % 4]);
      vhi[nb] = ds_read_tr16_asm<(2 * HALVES + nb / 4) * 1024>(vaddr[nb % 4]);
    });

    if ((t + 1) * KT > nkeys) {
      const int key0 = t * KT + lg * 4;
#pragma unroll
      for (int j = 0; j < MTW; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (key0 + kb * 16 + v >= nkeys) sacc[kb][j][v] = -INFINITY;
          }
    }

    // Row tile by row tile: softmax, then its P V and row-sum MFMAs, which
    // run on the matrix core while the next tile's softmax is on the VALU.
    bf16x8 va[NB];
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      if (j > 0 && j >= tcnt) break;
      bf16x8 pf;
      // (the lanes' own maxima decide whether the row max is needed, as in
      // the per-wave kernel above)
      const float lmx = fmaxf(
          fmaxf(fmaxf(fmaxf(sacc[0][j][0], sacc[0][j][1]), sacc[0][j][2]),
                fmaxf(fmaxf(sacc[0][j][3], sacc[1][j][0]), sacc[1][j][1])),
          fmaxf(sacc[1][j][2], sacc[1][j][3]));
      if (__builtin_amdgcn_ballot_w64(lmx * scale_log2 > thr[j])) {
        // (a tile always holds a valid key, so m_tile and m_new are finite)
        const float m_tile = row_max4(lmx) * scale_log2;
        const bool raise = m_tile > thr[j];
        const float m_new = raise ? m_tile : m_run[j];
        const float alpha = exp2_hw(m_run[j] - m_new);
        lacc[j] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][j] *= alpha;
        m_run[j] = m_new;
        neg_m[j] = -m_new;
        thr[j] = m_new + kRescaleSlack;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          pf[kb * 4 + v] = (__bf16)exp2_hw(fmaf(sacc[kb][j][v], scale_log2, neg_m[j]));
      if (j == 0) {
        lds_wait();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          va[nb] = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(vlo[nb], vhi[nb], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[nb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[nb], pf, oacc[nb][j], 0, 0, 0);
      lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc[j], 0, 0, 0);
    }
  };

  // The query loads complete before the first stage is issued, so the
  // compiler's wait for them does not also wait for the stages.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // nst is the same for every wave of the workgroup, so every thread
  // reaches every barrier.
  for (int st = 0; st < nst && st < NBUF - 1; ++st) issue_stage(st);
  for (int st = 0; st < nst; ++st) {
    // stages issued after st and still possibly in flight
    const int ahead = min(NBUF - 2, nst - 1 - st);
    wait_stage<PW, NBUF - 2>(ahead);
    if (st + NBUF - 1 < nst) issue_stage(st + NBUF - 1);  // into stage st - 1's buffer
    const unsigned char* buf = smem + (st % NBUF) * STAGE;
#pragma unroll
    for (int u = 0; u < TPS / KP; ++u) {
      const int tt = u * KP + phase;
      const int t = st * TPS + tt;
      if (t * KT >= nkeys) break;
      compute_tile(buf + tt * 4 * HALVES * 1024, buf + (W::KBLK + tt * 4 * HALVES) * 1024, t);
    }
  }

  float l_row[MTW];
#pragma unroll
  for (int j = 0; j < MTW; ++j) l_row[j] = lacc[j][0];

  if constexpr (KP == 2) {
    // Phase 1 parks (max, sum, O) of its row tiles in LDS slots indexed by
    // row tile (the stage ring is idle once every wave has passed the
    // barrier); the phase-0 owner of each tile folds them into its own
    // state, lane by lane: both hold the same (row, column) positions.
    constexpr int OROW = D + 4;  // floats per parked row (bank spread)
    float* obuf = reinterpret_cast<float*>(smem);
    float* mbuf = obuf + NW * MTW * 16 * OROW;
    float* lbuf = mbuf + NW * MTW * 16;
    static_assert((NW * MTW * 16 * (OROW + 2)) * 4 <= NBUF * STAGE, "merge slots fit the ring");
    __syncthreads();
    if (phase == 1) {
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        if (j >= tcnt) break;
        const int slot = (tfirst + j) * 16 + lr;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          *reinterpret_cast<f32x4*>(obuf + slot * OROW + nb * 16 + lg * 4) = oacc[nb][j];
        if (lg == 0) {
          mbuf[slot] = m_run[j];
          lbuf[slot] = l_row[j];
        }
      }
    }
    __syncthreads();
    if (phase == 1) return;
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      if (j >= tcnt) break;
      const int slot = (tfirst + j) * 16 + lr;
      const float m1 = mbuf[slot], l1 = lbuf[slot];
      const float mm = fmaxf(m_run[j], m1);
      const float a0 = m_run[j] == -INFINITY ? 0.f : exp2_hw(m_run[j] - mm);
      const float a1 = m1 == -INFINITY ? 0.f : exp2_hw(m1 - mm);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[nb][j] = a0 * oacc[nb][j] +
                      a1 * *reinterpret_cast<const f32x4*>(obuf + slot * OROW + nb * 16 + lg * 4);
      l_row[j] = a0 * l_row[j] + a1 * l1;
      m_run[j] = mm;
    }
  }

#pragma unroll
  for (int j = 0; j < MTW; ++j) {
    const float l = l_row[j];
    const int row = (tfirst + j) * 16 + lr;
    if (j < tcnt && row < M) {
      const int gq = row / n;
      const int i = row - gq * n;
      const int64_t orow = ((int64_t)b * Hq + kvh * G + gq) * n + i;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float* op = o_part + (orow * S + s) * D + lg * 4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        __builtin_nontemporal_store(oacc[nb][j] * inv, reinterpret_cast<f32x4*>(op + nb * 16));
      if (lg == 0) lse_part[orow * S + s] = l > 0.f ? (m_run[j] + log2_hw(l)) * kLn2 : -INFINITY;
    }
  }
}

// With start/stop events the launch records them on the kernel's own
// dispatch (hipExtLaunchKernel), so their elapsed time is the kernel's.
// (extra: the narrow kernel's tail arguments; none for the wide kernel)
template <typename Kernel, typename... Extra>
hipError_t launch_attn(Kernel kernel, int waves, const void* q, const void* k, const void* v,
                       const int32_t* seq_lens, int B, int Hq, int Hkv, int n, int64_t L_max,
                       float scale_log2, int64_t split_len, int S, float* o_part,
                       float* lse_part, hipStream_t stream, hipEvent_t ev_start,
                       hipEvent_t ev_stop, const Extra&... extra) {
  dim3 grid((unsigned)S, (unsigned)Hkv, (unsigned)B);
  const dim3 block((unsigned)(waves * 64));
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (ev_start != nullptr || ev_stop != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev_start, ev_stop, 0, qq, kk,
                          vv, seq_lens, Hq, Hkv, n, L_max, scale_log2, split_len, S, o_part,
                          lse_part, extra...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, qq, kk, vv, seq_lens, Hq, Hkv,
                       n, L_max, scale_log2, split_len, S, o_part, lse_part, extra...);
  return hipGetLastError();
}

rv_status dispatch_attn(int d, const RowPlan& rp, const void* q, const void* k, const void* v,
                        const int32_t* seq_lens, int B, int Hq, int Hkv, int n, int64_t L_max,
                        float scale_log2, int64_t split_len, int S, float* o_part,
                        float* lse_part, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  hipError_t e;
#define RV_ATTN_CASE(DD, MM, KERNEL, WAVES)                                                     \
  if (d == DD && rp.MTW == MM)                                                                 \
    e = launch_attn(KERNEL, WAVES, q, k, v, seq_lens, B, Hq, Hkv, n, L_max, scale_log2,       \
                    split_len, S, o_part, lse_part, s, e0, e1);
#define RV_NARROW_CASE(DD, MM)                                                                 \
  if (d == DD && rp.MTW == MM)                                                                 \
    e = launch_attn((attn_kernel<DD, MM, false>), NW, q, k, v, seq_lens, B, Hq, Hkv, n, L_max, \
                    scale_log2, split_len, S, o_part, lse_part, s, e0, e1, none);
  // Up to 4 row tiles: the per-wave streaming kernel.  5..8 tiles: the
  // shared-stage kernel with two key phases (8 waves, 2 tiles each); wider
  // groups: one phase (4 waves, 3 or 4 tiles each).
  const TailArgs<false> none{};
  if (!rp.wide) {
    RV_NARROW_CASE(64, 1)
    else RV_NARROW_CASE(64, 2)
    else RV_NARROW_CASE(64, 3)
    else RV_NARROW_CASE(64, 4)
    else RV_NARROW_CASE(128, 1)
    else RV_NARROW_CASE(128, 2)
    else RV_NARROW_CASE(128, 3)
    else RV_NARROW_CASE(128, 4)
    else return RV_ERR_UNSUPPORTED;
  } else {
    RV_ATTN_CASE(64, 2, (attn_wide_kernel<64, 2, 2>), 2 * NW)
    else RV_ATTN_CASE(64, 3, (attn_wide_kernel<64, 3, 1>), NW)
    else RV_ATTN_CASE(64, 4, (attn_wide_kernel<64, 4, 1>), NW)
    else RV_ATTN_CASE(128, 2, (attn_wide_kernel<128, 2, 2>), 2 * NW)
    else RV_ATTN_CASE(128, 3, (attn_wide_kernel<128, 3, 1>), NW)
    else RV_ATTN_CASE(128, 4, (attn_wide_kernel<128, 4, 1>), NW)
    else return RV_ERR_UNSUPPORTED;
  }
#undef RV_ATTN_CASE
#undef RV_NARROW_CASE
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  return RV_OK;
}

rv_status dispatch_verify(int d, const RowPlan& rp, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, int B, int Hq, int Hkv, int n, int64_t L_max,
                          float scale_log2, int64_t split_len, int S, float* o_part,
                          float* lse_part, const TailArgs<true>& tail, hipStream_t s,
                          hipEvent_t e0, hipEvent_t e1) {
  hipError_t e;
#define RV_VERIFY_CASE(DD, MM)                                                                 \
  if (d == DD && rp.MTW == MM)                                                                 \
    e = launch_attn((attn_kernel<DD, MM, true>), NW, q, k, v, seq_lens, B, Hq, Hkv, n, L_max,  \
                    scale_log2, split_len, S, o_part, lse_part, s, e0, e1, tail);
  if (rp.wide) return RV_ERR_UNSUPPORTED;
  RV_VERIFY_CASE(64, 1)
  else RV_VERIFY_CASE(64, 2)
  else RV_VERIFY_CASE(64, 3)
  else RV_VERIFY_CASE(64, 4)
  else RV_VERIFY_CASE(128, 1)
  else RV_VERIFY_CASE(128, 2)
  else RV_VERIFY_CASE(128, 3)
  else return RV_ERR_UNSUPPORTED;  // (d = 128 with 4 row tiles: two launches)
#undef RV_VERIFY_CASE
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
  return rv::dispatch_attn(d, rp, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max,
                           scale_log2, split_len, num_splits, o_part, lse_part,
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
  return rv::dispatch_attn(d, rp, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max,
                           scale_log2, split_len, num_splits, o_part, lse_part,
                           static_cast<hipStream_t>(stream),
                           static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event));
}

extern "C" rv_status spec_attn_verify(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* seq_lens, int64_t max_seq_len, int B,
                                      int Hq, int Hkv, int n, int d, int64_t L_max,
                                      float sm_scale, int64_t split_len, int num_splits,
                                      const void* k_blk, const void* v_blk,
                                      const int32_t* parent_host, float* o_part, float* lse_part,
                                      void* sync, size_t sync_bytes, void* out, float* lse_out,
                                      int help_after_us, void* stream, void* start_event,
                                      void* stop_event) {
  rv::BlockMask mask;
  rv_status st = rv::check_verify(q, k_cache, v_cache, seq_lens, max_seq_len, B, Hq, Hkv, n, d,
                                  L_max, sm_scale, split_len, num_splits, k_blk, v_blk,
                                  parent_host, o_part, lse_part, sync, sync_bytes, out,
                                  help_after_us, &mask);
  if (st != RV_OK) return st;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return RV_ERR_HIP;
  }
  const rv::RowPlan rp = rv::row_plan(Hq, Hkv, n);
  const float scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event);
  hipEvent_t e1 = static_cast<hipEvent_t>(stop_event);
  if (rv_verify_single_launch(B, Hq, Hkv, n, d, num_splits, cus)) {
    rv::TailArgs<true> tail;
    tail.k_blk = static_cast<const uint16_t*>(k_blk);
    tail.v_blk = static_cast<const uint16_t*>(v_blk);
    tail.out = static_cast<uint16_t*>(out);
    tail.lse_out = lse_out;
    tail.sync = static_cast<uint64_t*>(sync);
    const int us = help_after_us < 0 ? rv::kVerifyHelpDefaultUs : help_after_us;
    tail.help_ticks = (uint32_t)us * 100u;  // 100 MHz constant clock
    tail.mask = mask;
    return rv::dispatch_verify(d, rp, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max,
                               scale_log2, split_len, num_splits, o_part, lse_part, tail, s, e0,
                               e1);
  }
  st = rv::dispatch_attn(d, rp, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, n, L_max, scale_log2,
                         split_len, num_splits, o_part, lse_part, s, e0, nullptr);
  if (st != RV_OK) return st;
  return rv::block_merge_launch(q, k_blk, v_blk, mask, o_part, lse_part, num_splits, B, Hq, Hkv, n,
                                d, scale_log2, out, lse_out, stream, nullptr, stop_event);
}
