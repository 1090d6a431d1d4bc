"""GPU-vs-oracle comparison rules (test infrastructure only).

* Attention output: per output row (b, h, i), max_c |O - O_ref| / max_c |O_ref|
  must be <= 2e-2 (bf16 inputs, fp32 accumulation, bf16 output).  Entries are
  about 1/sqrt(keys) in size and cross zero, so an element-wise relative
  error would be meaningless.
* p_hat: <= 1e-5 absolute, element-wise.
* Accept decisions and token ids: bit-exact, except at positions flagged
  because the uniform lies within `tol` of the decision boundary:
    - accept step t is flagged iff |r_t - ratio_ref_t| <= tol; if the GPU and
      the oracle decide differently there, the two continuations diverge and
      the sequence is counted, not compared further;
    - the draw is flagged iff u*W lies within tol*W of either edge of the
      oracle's chosen interval [C_{k-1}, C_k); the GPU token must then still
      satisfy w_k > 0 and C_{k-1} - tol*W <= u*W <= C_k + tol*W.
"""

import numpy as np

ATTN_ROW_TOL = 2e-2
P_HAT_TOL = 1e-5
BOUNDARY_TOL = 1e-4


def attn_row_errors(o_gpu, o_ref):
    """Per-row relative error, shape o_ref.shape[:-1]."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    num = np.max(np.abs(o_gpu - o_ref), axis=-1)
    den = np.max(np.abs(o_ref), axis=-1)
    return num / np.maximum(den, 1e-30)


def compare_accept(ref, n_gpu, tok_gpu, r, u, tol=BOUNDARY_TOL):
    """Compare rapid_accept outputs with the oracle's.

    Returns a dict: errors (list of strings; empty means pass), diverged
    (sequences whose continuation split at a flagged accept step),
    flagged_accept, flagged_draw (counts at `tol`)."""
    errors = []
    diverged = 0
    flagged_accept = 0
    flagged_draw = 0
    B, g1 = np.asarray(tok_gpu).shape
    gamma = g1 - 1
    for b in range(B):
        n_ref = int(ref["n_accept"][b])
        n_g = int(n_gpu[b])
        ratio = ref["ratio"][b]
        for t in range(min(n_ref + 1, gamma)):
            if abs(float(r[b, t]) - ratio[t]) <= tol:
                flagged_accept += 1
        if n_g != n_ref:
            t0 = min(n_g, n_ref)
            if t0 < gamma and abs(float(r[b, t0]) - ratio[t0]) <= tol:
                diverged += 1
                continue
            errors.append("b=%d: n_accept %d != oracle %d (r=%r ratio=%r)"
                          % (b, n_g, n_ref, float(r[b, t0]) if t0 < gamma else None,
                             float(ratio[t0]) if t0 < gamma else None))
            continue
        toks = [int(x) for x in tok_gpu[b]]
        ref_toks = [int(x) for x in ref["out_tokens"][b]]
        if toks[:n_ref] != ref_toks[:n_ref]:
            errors.append("b=%d: accepted tokens differ" % b)
        if any(x != -1 for x in toks[n_ref + 1:]):
            errors.append("b=%d: tokens past the draw are not -1" % b)
        dr = ref["draw"][b]
        C, W, tgt, k = dr["C"], dr["W"], dr["target"], dr["k"]
        lo = C[k - 1] if k > 0 else 0.0
        hi = C[k]
        flagged = min(abs(tgt - lo), abs(tgt - hi)) <= tol * W
        kg = toks[n_ref]
        if flagged:
            flagged_draw += 1
            ok = 0 <= kg < len(C) and dr["w"][kg] > 0
            if ok:
                lo_g = C[kg - 1] if kg > 0 else 0.0
                ok = (lo_g - tol * W <= tgt <= C[kg] + tol * W)
            if not ok:
                errors.append("b=%d: flagged draw token %d outside the widened interval" % (b, kg))
        elif kg != k:
            errors.append("b=%d: drawn token %d != oracle %d (u*W=%r, [%r, %r))"
                          % (b, kg, k, tgt, lo, hi))
    return {"errors": errors, "diverged": diverged, "flagged_accept": flagged_accept,
            "flagged_draw": flagged_draw}
