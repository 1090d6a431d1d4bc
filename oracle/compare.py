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


def _draw_check(dr, kg, tol):
    """(flagged, error message or None) for a GPU draw kg against the oracle's
    draw record, by the rules above."""
    C, W, tgt, k = dr["C"], dr["W"], dr["target"], dr["k"]
    lo = C[k - 1] if k > 0 else 0.0
    hi = C[k]
    flagged = min(abs(tgt - lo), abs(tgt - hi)) <= tol * W
    if flagged:
        ok = dr["w"][kg] > 0
        if ok:
            lo_g = C[kg - 1] if kg > 0 else 0.0
            ok = lo_g - tol * W <= tgt <= C[kg] + tol * W
        return True, None if ok else "flagged draw token %d outside the widened interval" % kg
    if kg != k:
        return False, "drawn token %d != oracle %d (u*W=%r, [%r, %r))" % (kg, k, tgt, lo, hi)
    return False, None


def compare_tree_accept(ref, parent, tokens, n_gpu, path_gpu, tok_gpu, r, tol=BOUNDARY_TOL):
    """Compare rapid_tree_accept outputs with the tree oracle's.

    Per sequence b, with the GPU's path of n = n_gpu[b] nodes:
    * n outside [0, number of nodes - 1] is an error;
    * the path must run down the tree from the root (each node a child of the
      one before), be padded with -1, and carry the nodes' draft tokens, then
      one id in [0, V), then -1;
    * every decision the path implies (at each node on it, the children
      before the accepted one rejected, the accepted one accepted; at the
      stop node every child rejected) must equal the oracle's
      r_c <= ratio_c wherever the oracle tested c and |r_c - ratio_c| > tol;
    * if the path differs from the oracle's (possible only through flagged
      decisions) the sequence is counted as diverged and its draw is
      range-checked only; otherwise the draw is checked as for a chain.
    Returns a dict like compare_accept's."""
    from .tree import tree_children
    ch = tree_children(parent)
    tok_gpu = np.asarray(tok_gpu)
    path_gpu = np.asarray(path_gpu)
    B, nn = tok_gpu.shape
    errors = []
    diverged = flagged_accept = flagged_draw = exact_draws = 0
    for b in range(B):
        ratio = ref["ratio"][b]
        tested = ~np.isnan(ratio)
        flagged_accept += int(np.sum(np.abs(np.asarray(r[b], dtype=np.float64)[tested]
                                            - ratio[tested]) <= tol))
        m = int(n_gpu[b])
        if not 0 <= m <= nn - 1:
            errors.append("b=%d: n_accept %d outside [0, %d]" % (b, m, nn - 1))
            continue
        gp = [int(x) for x in path_gpu[b, :m]]
        prev, ok = 0, True
        for c in gp:
            if not (0 < c < nn and c in ch[prev]):
                ok = False
                break
            prev = c
        if not ok:
            errors.append("b=%d: path %s does not run down the tree" % (b, gp))
            continue
        if any(int(x) != -1 for x in path_gpu[b, m:]):
            errors.append("b=%d: path entries past n_accept are not -1" % b)
        toks = [int(x) for x in tok_gpu[b]]
        want = [int(tokens[b, c]) for c in gp]
        if toks[:m] != want:
            errors.append("b=%d: accepted tokens %s != the path's %s" % (b, toks[:m], want))
        if any(x != -1 for x in toks[m + 1:]):
            errors.append("b=%d: tokens past the draw are not -1" % b)
        kg = toks[m]
        V = len(ref["draw"][b]["C"])
        if not 0 <= kg < V:
            errors.append("b=%d: drawn token %d outside [0, %d)" % (b, kg, V))
            continue
        bad = None
        v = 0
        for i in range(m + 1):
            acc = gp[i] if i < m else None
            for c in ch[v]:
                if acc is not None and c > acc:
                    break
                if not tested[c]:
                    continue  # past a flagged divergence: the oracle never tested c
                decided = c == acc
                if decided != (float(r[b, c]) <= ratio[c]) and abs(float(r[b, c]) - ratio[c]) > tol:
                    bad = "b=%d: node %d %s unflagged (r=%r ratio=%r)" % (
                        b, c, "accepted" if decided else "rejected", float(r[b, c]), ratio[c])
                    break
            if bad or acc is None:
                break
            v = acc
        if bad:
            errors.append(bad)
            continue
        ref_path = [int(x) for x in ref["path"][b, :int(ref["n_accept"][b])]]
        if gp != ref_path:
            diverged += 1
            continue
        flagged, msg = _draw_check(ref["draw"][b], kg, tol)
        flagged_draw += flagged
        if msg:
            errors.append("b=%d: %s" % (b, msg))
        elif not flagged:
            exact_draws += 1
    return {"errors": errors, "diverged": diverged, "flagged_accept": flagged_accept,
            "flagged_draw": flagged_draw, "exact_draws": exact_draws}
