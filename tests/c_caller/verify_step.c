/*
 * One verify step driven from plain C99 through the library's C ABI: the
 * history pass over the cache (LongSpec summary, section 2.3: unmasked,
 * split along the sequence), the causal draft block fused with the
 * log-sum-exp merge, and RAPID's acceptance over the vocabulary (RAPID blog,
 * sections 2.1 and 2.4).  Device memory comes from hipMalloc, the calls run
 * on the null stream, and no C++ or Python is involved.  The GPU test that
 * loads this file's shared object compares its outputs with the Python
 * binding's and with the fp64 oracle.
 *
 * Host buffers in, host buffers out (layouts as in rapid_verify.h):
 *   q [B,Hq,n,d], k_cache/v_cache [B,Hkv,L_max,d], k_blk/v_blk [B,Hkv,n,d]
 *   as bf16 bit patterns; seq_lens [B]; z [B,gamma+1,V], y [B,gamma,V];
 *   draft, r [B,gamma]; u [B,gamma+1].  Outputs: out [B,Hq,n,d] bf16 bits,
 *   lse_out [B,Hq,n], n_accept [B], out_tokens [B,gamma+1], ratio [B,gamma],
 *   and the split the balanced planner chose.
 * Returns 0, a positive rv_status of the first failing library call, or
 * -1 (allocation or copy failure) / -2 (device query failure).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rapid_verify.h"

#define N_DEV 19

int rv_c_verify_step(int B, int Hq, int Hkv, int n, int d, int64_t L_max, int gamma, int V,
                     float sm_scale, float T, float eta, const uint16_t* q,
                     const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* seq_lens,
                     const uint16_t* k_blk, const uint16_t* v_blk, const float* z,
                     const float* y, const int32_t* draft, const float* r, const float* u,
                     uint16_t* out, float* lse_out, int32_t* n_accept, int32_t* out_tokens,
                     float* ratio, int64_t* split_len_out, int32_t* num_splits_out) {
  int num_cus = 0;
  if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess)
    return -2;
  int64_t split_len = 0;
  int S = 0;
  int st = rv_prefix_balanced_split(seq_lens, B, Hq, Hkv, n, d, num_cus, &split_len, &S);
  if (st != RV_OK) return st;
  *split_len_out = split_len;
  *num_splits_out = S;
  int64_t max_len = 0;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] > max_len) max_len = seq_lens[b];

  const size_t nq = (size_t)B * Hq * n * d, nkv = (size_t)B * Hkv * L_max * d;
  const size_t nblk = (size_t)B * Hkv * n * d, rows = (size_t)B * Hq * n;
  const size_t nz = (size_t)B * (gamma + 1) * V, ny = (size_t)B * gamma * V;
  const size_t ws_bytes = rapid_accept_workspace_size(B, gamma, V);
  /* device buffers: sizes, then the host source (NULL for outputs) */
  const size_t bytes[N_DEV] = {
      nq * 2, nkv * 2, nkv * 2, (size_t)B * 4, nblk * 2, nblk * 2,
      rows * (size_t)S * d * 4, rows * (size_t)S * 4, nq * 2, rows * 4,
      nz * 4, ny * 4, (size_t)B * gamma * 4, (size_t)B * gamma * 4, (size_t)B * (gamma + 1) * 4,
      (size_t)B * 4, (size_t)B * (gamma + 1) * 4, (size_t)B * gamma * 4, ws_bytes};
  const void* src[N_DEV] = {q, k_cache, v_cache, seq_lens, k_blk, v_blk, NULL, NULL, NULL, NULL,
                            z, y, draft, r, u, NULL, NULL, NULL, NULL};
  void* dev[N_DEV];
  memset(dev, 0, sizeof(dev));
  int rc = 0;
  for (int i = 0; i < N_DEV && rc == 0; ++i) {
    if (hipMalloc(&dev[i], bytes[i]) != hipSuccess) rc = -1;
    else if (src[i] != NULL && hipMemcpy(dev[i], src[i], bytes[i], hipMemcpyHostToDevice) != hipSuccess)
      rc = -1;
  }
  if (rc == 0)
    rc = spec_attn_prefix(dev[0], dev[1], dev[2], (const int32_t*)dev[3], max_len, B, Hq, Hkv,
                          n, d, L_max, sm_scale, split_len, S, (float*)dev[6], (float*)dev[7],
                          NULL);
  if (rc == 0)
    rc = spec_attn_block_merge(dev[0], dev[4], dev[5], NULL, (const float*)dev[6],
                               (const float*)dev[7], S, B, Hq, Hkv, n, d, sm_scale, dev[8],
                               (float*)dev[9], NULL);
  if (rc == 0)
    rc = rapid_accept((const float*)dev[10], (const float*)dev[11], (const int32_t*)dev[12],
                      (const float*)dev[13], (const float*)dev[14], B, gamma, V, T, eta,
                      (int32_t*)dev[15], (int32_t*)dev[16], (float*)dev[17], NULL, dev[18],
                      ws_bytes, NULL);
  if (rc == 0 && hipDeviceSynchronize() != hipSuccess) rc = -1;
  if (rc == 0) {
    void* dst[5] = {out, lse_out, n_accept, out_tokens, ratio};
    const int from[5] = {8, 9, 15, 16, 17};
    for (int i = 0; i < 5 && rc == 0; ++i)
      if (hipMemcpy(dst[i], dev[from[i]], bytes[from[i]], hipMemcpyDeviceToHost) != hipSuccess)
        rc = -1;
  }
  for (int i = 0; i < N_DEV; ++i)
    if (dev[i] != NULL) (void)hipFree(dev[i]);
  return rc;
}
