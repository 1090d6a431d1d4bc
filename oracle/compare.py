"""GPU-vs-oracle comparison rules (test infrastructure only).

* Attention output: per output row (b, h, i), max_c |O - O_ref| / max_c |O_ref|
  must be <= 2e-2 (bf16 inputs, fp32 accumulation, bf16 output).  Entries are
  about 1/sqrt(keys) in size and cross zero, so an element-wise relative
  error would be meaningless.
* p_hat: <= 1e-5 absolute, element-wise.
* Accept decisions and token ids (the procedure of the RAPID blog post,
  section 2.1, with p_hat for p as in section 2.4): bit-exact, except at
  positions flagged because the uniform lies within `tol` of the decision
  boundary:
    - a GPU n_accept outside [0, gamma] is always an error;
    - accept step t is flagged iff |r_t - ratio_ref_t| <= tol; every decision
      the GPU took (accept below its n_accept, reject at it) must match the
      oracle's r_t <= ratio_ref_t unless flagged.  If the two n_accept differ
      (only possible through a flagged step) the draws are at different rows:
      the sequence is counted as diverged, and only its accepted prefix, its
      -1 tail and the range of its drawn id are checked;
    - the draw is flagged iff u*W lies within tol*W of either edge of the
      oracle's chosen interval [C_{k-1}, C_k); the GPU token must then still
      satisfy w_k > 0 and C_{k-1} - tol*W <= u*W <= C_k + tol*W.

Pinned by tests/test_oracle_compare.py on hand-built outputs.
"""

import numpy as np

ATTN_ROW_TOL = 2e-2
P_HAT_TOL = 1e-5
BOUNDARY_TOL = 1e-4
# Log-sum-exp of attention rows.  Where the row sum adds the same bf16-rounded
# probabilities that multiply V (matrix-core row sums), each term carries a
# relative rounding error of at most 2^-8 (bf16 has 8 significant bits), so
# the sum does too and |dLSE| <= -ln(1 - 2^-8) = 3.9e-3.  With fp32 sums the
# error is a few fp32 ulps of the scores; 1e-4 leaves room for the hardware
# exp2/log2 approximations.
LSE_TOL_BF16_SUMS = 4e-3
LSE_TOL_FP32 = 1e-4
# Block partial computed in fp32 on the vector ALU: absolute bound on its
# outputs (entries are O(1)).
BLOCK_FP32_TOL = 1e-4


def attn_row_errors(o_gpu, o_ref):
    """Per-row relative error, shape o_ref.shape[:-1]."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    num = np.max(np.abs(o_gpu - o_ref), axis=-1)
    den = np.max(np.abs(o_ref), axis=-1)
    return num / np.maximum(den, 1e-30)


def compare_accept(ref, n_gpu, tok_gpu, r, u, tol=BOUNDARY_TOL, draft=None):
    """Compare rapid_accept outputs with the oracle's.

    draft  [B, gamma] draft ids (optional): the GPU's accepted tokens are
           checked against them; without it, against the oracle's accepted
           prefix where the two agree.

    Per sequence b, with the GPU's n = n_gpu[b]:
    * n outside [0, gamma] is an error (checked before any indexing);
    * the GPU's decisions (accept rows t < n, reject row n when n < gamma)
      must equal the oracle's r_t <= ratio_t wherever |r_t - ratio_t| > tol;
    * tokens: the accepted drafts, then one id in [0, V), then -1;
    * if n differs from the oracle's (possible only through flagged
      decisions), the draws are at different rows: the sequence is counted
      as diverged and its draw is range-checked only;
    * otherwise the drawn id must equal the oracle's, or, at a flagged draw,
      lie in the widened interval with positive weight.

    Returns a dict: errors (list of strings; empty means pass), diverged,
    flagged_accept and flagged_draw (counts at `tol`)."""
    errors = []
    diverged = 0
    flagged_accept = 0
    flagged_draw = 0
    exact_draws = 0
    tok_gpu = np.asarray(tok_gpu)
    B, g1 = tok_gpu.shape
    gamma = g1 - 1
    V = np.asarray(ref["p_hat"]).shape[-1]
    for b in range(B):
        n_ref = int(ref["n_accept"][b])
        n_g = int(n_gpu[b])
        ratio = ref["ratio"][b]
        near = [abs(float(r[b, t]) - float(ratio[t])) <= tol for t in range(gamma)]
        flagged_accept += sum(near[:min(n_ref + 1, gamma)])
        if not 0 <= n_g <= gamma:
            errors.append("b=%d: n_accept %d outside [0, %d] (oracle %d)"
                          % (b, n_g, gamma, n_ref))
            continue
        bad = [t for t in range(min(n_g + 1, gamma))
               if (t < n_g) != (float(r[b, t]) <= float(ratio[t])) and not near[t]]
        if bad:
            t = bad[0]
            errors.append("b=%d: n_accept %d (oracle %d) %s row %d unflagged (r=%r ratio=%r)"
                          % (b, n_g, n_ref, "accepts" if t < n_g else "rejects", t,
                             float(r[b, t]), float(ratio[t])))
            continue
        toks = [int(x) for x in tok_gpu[b]]
        if draft is not None:
            want = [int(x) for x in np.asarray(draft)[b, :n_g]]
        else:
            want = [int(x) for x in ref["out_tokens"][b, :min(n_g, n_ref)]]
        if toks[:len(want)] != want:
            errors.append("b=%d: accepted tokens %s != drafts %s" % (b, toks[:len(want)], want))
        if any(x != -1 for x in toks[n_g + 1:]):
            errors.append("b=%d: tokens past the draw are not -1: %s" % (b, toks[n_g + 1:]))
        kg = toks[n_g]
        if not 0 <= kg < V:
            errors.append("b=%d: drawn token %d outside [0, %d)" % (b, kg, V))
            continue
        if n_g != n_ref:
            diverged += 1
            continue
        dr = ref["draw"][b]
        C, W, tgt, k = dr["C"], dr["W"], dr["target"], dr["k"]
        lo = C[k - 1] if k > 0 else 0.0
        hi = C[k]
        flagged = min(abs(tgt - lo), abs(tgt - hi)) <= tol * W
        if flagged:
            flagged_draw += 1
            ok = dr["w"][kg] > 0
            if ok:
                lo_g = C[kg - 1] if kg > 0 else 0.0
                ok = (lo_g - tol * W <= tgt <= C[kg] + tol * W)
            if not ok:
                errors.append("b=%d: flagged draw token %d outside the widened interval" % (b, kg))
        elif kg != k:
            errors.append("b=%d: drawn token %d != oracle %d (u*W=%r, [%r, %r))"
                          % (b, kg, k, tgt, lo, hi))
        else:
            exact_draws += 1
    return {"errors": errors, "diverged": diverged, "flagged_accept": flagged_accept,
            "flagged_draw": flagged_draw, "exact_draws": exact_draws}


def flag_counts(ref, r, tol):
    """Flagged positions of an oracle result at boundary distance `tol`,
    without any GPU output: accept steps the oracle evaluated with
    |r_t - ratio_t| <= tol, and draws whose target u*W lies within tol*W of
    an edge of the chosen interval.  Returns (flagged_accept, flagged_draw,
    draws)."""
    fa = fd = 0
    B, gamma = np.asarray(ref["ratio"]).shape
    for b in range(B):
        n_ref = int(ref["n_accept"][b])
        fa += sum(abs(float(r[b, t]) - float(ref["ratio"][b, t])) <= tol
                  for t in range(min(n_ref + 1, gamma)))
        dr = ref["draw"][b]
        C, W, tgt, k = dr["C"], dr["W"], dr["target"], dr["k"]
        lo = C[k - 1] if k > 0 else 0.0
        fd += min(abs(tgt - lo), abs(tgt - C[k])) <= tol * W
    return fa, fd, B
