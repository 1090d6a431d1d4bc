"""fp64 oracle for RAPID's acceptance step (test infrastructure only).

Sources (RAPID blog post, leeon-k.github.io; RAPID article, abeam.tech):

* Speculative decoding background (blog section 2.1): a draft token x ~ q is
  kept iff a uniform r satisfies r <= min(1, p(x)/q(x)); on rejection a new
  token is drawn from the normalised positive part of (p - q).  All gamma
  candidates are checked in one target pass and generation continues from
  the first rejection (blog section 2.1; abeam article, inference flow
  step 3).
* RAPID's acceptance (blog section 2.3): the same test, with p the target
  distribution on the full context and q the RAG drafter's distribution.
* Retrieval-augmented target (blog section 2.4, the p_hat display; abeam
  article, "Key idea 1"): p = softmax(z/T) and
  p_hat = softmax(z/T + eta * (q - p)); at inference p_hat takes the place of
  p in the acceptance test.

Readings where the pages are silent or disagree (each restated where used):
* q = softmax(y/T) with the target's temperature T (the pages define T only
  for the target).
* The residual on rejection is norm(max(p_hat - q, 0)), i.e. the background
  rule with p replaced by p_hat.  (Blog section 2.4 also prints a different
  residual and a tail-preserving rule; both are options, off by default.)
* When all gamma drafts are accepted, a bonus token is drawn from the target
  distribution of the last row, p_gamma = softmax(z_gamma/T), with u_gamma.
* The acceptance inequality is inclusive (r <= ratio), with r in [0, 1).
* Inverse CDF: ascending token id, C_k = sum_{j<=k} w_j, pick the smallest k
  with C_k > u*W (W = total weight), so a zero-weight id is never picked; if
  rounding leaves no such k, pick the largest k with w_k > 0.
* A rejected row with W == 0 cannot happen in exact arithmetic (W == 0 forces
  p_hat == q, hence ratio 1); if it did, the token is drawn from p_hat.

Two further rules printed in blog section 2.4, off by default:
* tail preservation: every entry of p_hat below 0.1 times its largest entry
  is replaced by the target's p; the page states no renormalisation, but
  without one p_hat is no distribution, so the result is renormalised.
* the printed residual norm(max(p - p_hat, p - q)) = norm(p - min(p_hat, q)):
  its entries can be negative and the page gives no clip, so it is clipped
  at zero.  The page's claim that the output then follows p holds exactly
  when p >= min(p_hat, q) everywhere (no clipping needed).
"""

import numpy as np


def softmax_ref(x):
    """softmax(x)_v = exp(x_v - m) / sum_u exp(x_u - m), m = max_u x_u."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def target_probs(z_row, T):
    """p = softmax(z/T): the target's tempered distribution (blog section 2.4)."""
    return softmax_ref(np.asarray(z_row, dtype=np.float64) / T)


def draft_probs(y_row, T):
    """q = softmax(y/T): the drafter's distribution, tempered with the target's T."""
    return softmax_ref(np.asarray(y_row, dtype=np.float64) / T)


def retrieval_augmented_target(z_row, y_row, T, eta):
    """Return (p, q, p_hat) with p_hat = softmax(z/T + eta*(q - p))
    (blog section 2.4, the p_hat display)."""
    z = np.asarray(z_row, dtype=np.float64)
    p = target_probs(z, T)
    q = draft_probs(y_row, T)
    s = z / T + eta * (q - p)
    return p, q, softmax_ref(s)


def tail_preserve_ref(p, p_hat, frac=0.1, force=None):
    """Blog section 2.4's tail rule: p_hat_k := p_k where
    p_hat_k < frac * max_j p_hat_j, then renormalise.

    force: optional {entry id: keep} fixing the side of the threshold those
    entries fall on.  The rule itself never needs it; a check of an
    implementation in another precision uses it for entries that lie within
    that precision's error of the threshold, where either side is correct.
    """
    p = np.asarray(p, dtype=np.float64)
    p_hat = np.asarray(p_hat, dtype=np.float64)
    keep = p_hat >= frac * np.max(p_hat)
    if force:
        for k, v in force.items():
            keep[int(k)] = bool(v)
    adj = np.where(keep, p_hat, p)
    return adj / np.sum(adj)


def inverse_cdf_ref(w, u):
    """Inverse-CDF draw from the unnormalised weights w with uniform u.

    Returns (k, C, W): the chosen id, the cumulative sums C (ascending id)
    and the total W = C[-1].  k is the smallest id with C_k > u*W; when no
    such id exists because of rounding, the largest id with w_k > 0.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    W = C[-1]
    above = C > u * W
    if above.any():
        k = int(np.argmax(above))
    else:
        k = int(np.nonzero(w > 0)[0][-1])
    return k, C, W


def rapid_accept_ref(z, y, draft, r, u, T, eta, tail_preserve=False, residual="p_hat",
                     tail_force=None):
    """One verify step of RAPID's acceptance, per sequence, step by step.

    tail_preserve  apply the tail rule to p_hat (and use it everywhere p_hat
                   is used: ratios, residual, p_hat output)
    residual       "p_hat": max(p_hat - q, 0) (the background rule with p
                   replaced by p_hat); "printed": max(p - min(p_hat, q), 0)
    tail_force     optional {(b, t): {entry id: keep}}: the tail rule's
                   classification of those entries, fixed (tail_preserve_ref)

    z     [B, gamma+1, V] target logits (row t scores the token after row t)
    y     [B, gamma, V]   draft logits; draft[b, t] was drawn from softmax(y[b,t]/T)
    draft [B, gamma]      draft token ids
    r     [B, gamma]      acceptance uniforms in [0, 1)
    u     [B, gamma+1]    sampling uniforms in [0, 1); u[b, t] is used only
                          for a draw at row t
    Returns a dict:
      n_accept   int64 [B]            number of leading accepted drafts
      out_tokens int64 [B, gamma+1]   accepted drafts, then the drawn token,
                                      then -1
      ratio      f64 [B, gamma]       min(1, p_hat_t[x_t]/q_t[x_t]) for every t
      p_hat      f64 [B, gamma, V]
      draw       list of dicts, one per sequence: row, kind ('residual',
                 'bonus' or 'p_hat'), weights' cumulative sums C, total W,
                 target u*W and the chosen id k (for boundary flagging)
    """
    z = np.asarray(z)
    y = np.asarray(y)
    B, g1, V = z.shape
    gamma = g1 - 1
    if y.shape != (B, gamma, V):
        raise ValueError("y must be [B, gamma, V]")
    if not (T > 0):
        raise ValueError("T must be positive")
    if residual not in ("p_hat", "printed"):
        raise ValueError("residual must be 'p_hat' or 'printed'")
    n_accept = np.zeros(B, dtype=np.int64)
    out_tokens = np.full((B, gamma + 1), -1, dtype=np.int64)
    ratio = np.zeros((B, gamma))
    p_hat_all = np.zeros((B, gamma, V))
    draws = []
    for b in range(B):
        q_rows, p_rows = [], []
        for t in range(gamma):
            x = int(draft[b, t])
            if not (0 <= x < V):
                raise ValueError("draft token id out of range")
            p, q, p_hat = retrieval_augmented_target(z[b, t], y[b, t], T, eta)
            if tail_preserve:
                force = tail_force.get((b, t)) if tail_force else None
                p_hat = tail_preserve_ref(p, p_hat, force=force)
            p_hat_all[b, t] = p_hat
            q_rows.append(q)
            p_rows.append(p)
            ratio[b, t] = min(1.0, p_hat[x] / q[x])
        # First-reject cut: keep drafts while r_t <= ratio_t.
        t_star = gamma
        for t in range(gamma):
            if float(r[b, t]) <= ratio[b, t]:
                continue
            t_star = t
            break
        n_accept[b] = t_star
        out_tokens[b, :t_star] = draft[b, :t_star]
        ub = float(u[b, t_star])
        if t_star < gamma:
            if residual == "p_hat":
                w = np.maximum(p_hat_all[b, t_star] - q_rows[t_star], 0.0)
            else:
                w = np.maximum(p_rows[t_star] - np.minimum(p_hat_all[b, t_star], q_rows[t_star]),
                               0.0)
            kind = "residual"
            if not np.any(w > 0):
                w = p_hat_all[b, t_star]
                kind = "p_hat"
        else:
            w = target_probs(z[b, gamma], T)
            kind = "bonus"
        k, C, W = inverse_cdf_ref(w, ub)
        out_tokens[b, t_star] = k
        draws.append({"row": t_star, "kind": kind, "C": C, "W": W,
                      "target": ub * W, "k": k, "w": w})
    return {"n_accept": n_accept, "out_tokens": out_tokens, "ratio": ratio,
            "p_hat": p_hat_all, "draw": draws}
