// Host-side driver for the sanitizer test: calls every argument validator
// and layout helper of the library's HIP-free unit with edge and extreme
// sizes.  Built with AddressSanitizer and UndefinedBehaviorSanitizer (host
// code only, no device code involved), so any overflow, out-of-range shift
// or out-of-bounds read in the host arithmetic aborts the run.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "rv_internal.h"

using namespace rv;

static void* const P = reinterpret_cast<void*>(0x10000);  // aligned, never dereferenced
static long calls = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "unexpected result: %s\n", what);
    exit(2);
  }
}

int main() {
  const int ints[] = {INT_MIN, -1, 0, 1, 2, 3, 4, 7, 8, 63, 64, 65, 128, 255, 256, 65535, 65536,
                      1 << 22, (1 << 22) + 1, INT_MAX};
  const int64_t longs[] = {INT64_MIN, -1, 0, 1, 127, 128, 4096, 131072, 1 << 20,
                           (int64_t)1 << 31, (int64_t)1 << 40, (int64_t)1 << 41, INT64_MAX};
  const float scales[] = {0.f, -1.f, 1.f, NAN, INFINITY, 1e-30f, 3e38f};
  const float* F = static_cast<const float*>(P);
  const int32_t* I = static_cast<const int32_t*>(P);

  // spec_attn_prefix and the default split
  for (int64_t L : longs)
    for (int64_t msl : longs)
      for (int64_t split : longs)
        for (int d : {0, 64, 96, 128})
          for (int S : {0, 1, 32, 65535, 65536, INT_MAX}) {
            check_prefix(P, P, P, I, msl, 1, 32, 8, 11, d, L, 1.f, split, S, F, F);
            ++calls;
          }
  for (int B : ints)
    for (int Hq : ints)
      for (int Hkv : {1, 2, 8, 0, -1, INT_MAX})
        for (int n : ints) {
          check_prefix(P, P, P, I, 4096, B, Hq, Hkv, n, 128, 4096, 1.f, 1024, 4, F, F);
          int64_t sl = 0;
          int ns = 0;
          for (int64_t msl : longs) {
            rv_status st = rv_prefix_default_split(msl, B, Hq, Hkv, n, 128, &sl, &ns);
            if (st == RV_OK) expect(sl > 0 && sl % kSplitQuantum == 0 && ns >= 1 &&
                                        (msl + sl - 1) / sl <= ns, "default split covers");
            ++calls;
          }
        }
  // the balanced split, from host lengths
  {
    const int32_t lens_a[] = {48330, 92427, 125481, 53507, 127380, 42193, 70031, 103537};
    const int32_t lens_b[] = {INT32_MAX, 0, 1, INT32_MAX, 128};
    const int32_t lens_c[] = {0, 0, 0};
    const int32_t lens_d[] = {5, -1, 7};
    struct { const int32_t* p; int B; } sets[] = {{lens_a, 8}, {lens_b, 5}, {lens_c, 3},
                                                  {lens_d, 3}, {nullptr, 2}};
    for (auto set : sets)
      for (int Hkv : {1, 4, 8, 0, INT_MAX})
        for (int cus : {0, 1, 256, INT_MAX}) {
          int64_t sl = 0;
          int ns = 0;
          const rv_status st =
              rv_prefix_balanced_split(set.p, set.B, Hkv > INT_MAX / 4 ? Hkv : 4 * Hkv, Hkv, 11,
                                       128, cus, &sl, &ns);
          if (st == RV_OK) {
            int64_t mx = 0;
            for (int b = 0; b < set.B; ++b) mx = set.p[b] > mx ? set.p[b] : mx;
            expect(sl > 0 && sl % kSplitQuantum == 0 && ns >= 1 && (mx + sl - 1) / sl <= ns,
                   "balanced split covers");
          }
          ++calls;
        }
  }
  for (float sc : scales) {
    check_prefix(P, P, P, I, 4096, 1, 8, 2, 5, 64, 4096, sc, 1024, 4, F, F);
    ++calls;
  }

  // block masks: valid and invalid trees of every size up to the limit
  int32_t par[80];
  for (int n = 0; n <= 70; ++n) {
    for (int kind = 0; kind < 4; ++kind) {
      par[0] = kind == 3 ? 0 : -1;
      for (int i = 1; i < n && i < 80; ++i)
        par[i] = kind == 0 ? i - 1 : kind == 1 ? 0 : kind == 2 ? i : (i + 1) % (i + 1);
      BlockMask m;
      rv_status a = check_block(P, P, P, n ? par : nullptr, 1, 8, 2, n, 128, 1.f, F, F, &m);
      rv_status b = check_block(P, P, P, n ? par : nullptr, 1, 8, 2, n, 128, 1.f, F, F, &m);
      expect(a == b, "deterministic");
      if (kind == 2 && n > 1) expect(a != RV_OK, "parent[i] = i is rejected");
      check_block_merge(P, P, P, n ? par : nullptr, F, F, 32, 1, 8, 2, n, 128, 1.f, P, &m);
      calls += 3;
    }
  }
  for (int B : ints)
    for (int Hq : {1, 8, 64, 65535, INT_MAX})
      for (int n : {1, 11, 64}) {
        check_block(P, P, P, nullptr, B, Hq, 1, n, 64, 1.f, F, F, nullptr);
        check_block_merge(P, P, P, nullptr, F, F, 32, B, Hq, 1, n, 64, 1.f, P, nullptr);
        for (int S : ints) check_merge(F, F, S, F, F, B, Hq, n, 128, P);
        calls += 2 + sizeof(ints) / sizeof(ints[0]);
      }
  check_merge(F, F, 4, nullptr, nullptr, 1, 8, 5, 64, P);
  expect(check_merge(F, F, 4, F, nullptr, 1, 8, 5, 64, P) == RV_ERR_NULL, "half a block partial");

  // window attention and its workspace arithmetic
  for (int cap : ints)
    for (int sink : ints)
      for (int window : ints)
        for (int n : {1, 5, 64}) {
          rv_status st = check_window(P, P, P, I, 1, 8, 2, n, 128, cap, sink, window, 1.f, P, P,
                                      (size_t)1 << 40);
          if (st == RV_OK) {
            const int S = window_segments(sink, window);
            expect(S >= 1 && (int64_t)S * 64 >= (int64_t)sink + window, "segments cover keys");
            expect(window_workspace_words((size_t)8 * n, S, 128) * 4 < ((size_t)1 << 40),
                   "workspace fits");
          }
          ++calls;
        }

  // vocabulary pass: layouts at every extreme the validator admits
  for (int B : ints)
    for (int g : ints)
      for (int V : ints) {
        rv_status st = check_accept(F, F, I, F, F, B, g, V, 1.f, 0.5f, 0u, I, I, P, (size_t)-1);
        if (st == RV_OK) {
          AcceptLayout L = accept_layout(B, g, V);
          expect(L.cs >= 1 && L.cp >= 1 && L.cd >= 1, "chunks");
          expect((size_t)L.cd * kDrawChunk >= (size_t)V && (size_t)L.cs * kStatChunk >= (size_t)V,
                 "chunks cover the vocabulary");
          expect(L.zstat < L.ystat && L.ystat < L.sstat && L.sstat < L.rowtab &&
                     L.rowtab < L.tstat && L.tstat < L.wsum && L.wsum < L.arrivals &&
                     L.arrivals < L.words,
                 "regions in order");
        }
        ++calls;
      }
  for (unsigned flags : {0u, 1u, 2u, 3u, 4u, 0x80000000u})
    for (float T : scales) {
      check_accept(F, F, I, F, F, 1, 4, 32000, T, 0.5f, flags, I, I, P, (size_t)1 << 30);
      check_accept(F, F, I, F, F, 1, 4, 32000, 1.f, T, flags, I, I, P, (size_t)1 << 30);
      calls += 2;
    }

  for (int c = -5; c < 20; ++c) expect(rv_status_string(c) != nullptr, "status string");
  printf("host validators: %ld calls, no sanitizer report\n", calls);
  return 0;
}
