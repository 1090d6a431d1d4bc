"""fp64 oracle for acceptance over a draft tree (test infrastructure only).

The pages verify draft trees only as attention (LongSpec summary,
gist.science, section 1 "Problem", challenge 3, and section 2.3 "Fast Tree
Attention": every node attends to its ancestors).  They give no rule for
accepting among sibling candidates, so this module adopts one from outside
them: the per-node recursive rejection used for multi-candidate speculative
sampling, with RAPID's p_hat in the place of the target distribution (RAPID
blog post, leeon-k.github.io, section 2.1 for the single-candidate test and
residual, section 2.4 for p_hat at inference).  With one child per node it is
exactly rapid_accept_ref's chain rule.

Tree and inputs, per sequence:
* node 0 is the root (the last committed token); parent[i] < i for i >= 1;
  node i >= 1 carries the draft token tokens[i];
* z[i] are the target's logits after node i, y[i] the drafter's logits
  after node i (the children of i were drafted from q_i = softmax(y_i/T));
* r[i] is the acceptance uniform used when node i is tested, u[i] the
  sampling uniform used when the walk stops at node i.

The walk, starting at v = 0:
* if v has no children, draw a bonus token from p_v = softmax(z_v/T) with
  u_v (the chain's bonus reading), and stop;
* otherwise R = p_hat_v; for each child c of v in ascending node id: if
  r_c <= min(1, R[x_c] / q_v[x_c]), accept c (emit x_c, v = c, continue the
  walk); else R = norm(max(R - q_v, 0));
* if every child is rejected, draw from R with u_v by inverse CDF and stop.

Given the path, when the children of v are independent draws from q_v, the
token emitted at v (an accepted child's token or the final draw) follows
p_hat_v; this is what the pins in tests/test_oracle_tree.py check by exact
enumeration and by Monte-Carlo.

A rejection whose residual max(R - q, 0) has no mass cannot happen in exact
arithmetic (it would need R <= q everywhere, hence R = q and a ratio of 1);
if rounding produced it, R would be kept unchanged.
"""

import numpy as np

from .rapid import inverse_cdf_ref, retrieval_augmented_target, target_probs


def tree_children(parent):
    """children[v]: the children of node v in ascending node id."""
    parent = [int(p) for p in parent]
    n = len(parent)
    if n == 0 or parent[0] != -1:
        raise ValueError("node 0 is the root and must have parent -1")
    for i in range(1, n):
        if not 0 <= parent[i] < i:
            raise ValueError("parent[%d]=%d is not an earlier node" % (i, parent[i]))
    ch = [[] for _ in range(n)]
    for i in range(1, n):
        ch[parent[i]].append(i)
    return ch


def residual_sequence(p_hat, q, k):
    """R_0 = p_hat and R_j = norm(max(R_{j-1} - q, 0)) for j = 1..k: the
    distribution tested against child j+1 (R_j for j < k) and the final draw
    distribution after k rejections (R_k)."""
    R = [np.asarray(p_hat, dtype=np.float64)]
    q = np.asarray(q, dtype=np.float64)
    for _ in range(k):
        w = np.maximum(R[-1] - q, 0.0)
        W = np.sum(w)
        R.append(w / W if W > 0 else R[-1])
    return R


def rapid_tree_accept_ref(z, y, parent, tokens, r, u, T, eta):
    """The walk above for B sequences sharing one tree.

    z, y    [B, n, V]  logits after each node (target, drafter)
    parent  [n]        parent array, parent[0] = -1
    tokens  [B, n]     draft token of each node (tokens[:, 0] unused)
    r, u    [B, n]     acceptance and sampling uniforms in [0, 1)
    Returns a dict:
      n_accept   int64 [B]      accepted nodes on the path
      path       int64 [B, n]   accepted node ids in order, then -1
      out_tokens int64 [B, n]   their tokens, then the drawn token, then -1
      ratio      f64 [B, n]     min(1, R[x_c]/q[x_c]) of every child c tested
                                (nan for nodes not tested)
      draw       list of dicts per sequence: node, kind ('residual' or
                 'bonus'), rejected (children rejected at the node),
                 cumulative sums C, total W, target u*W, chosen id k, weights w
    """
    z = np.asarray(z)
    y = np.asarray(y)
    B, n, V = z.shape
    if y.shape != (B, n, V):
        raise ValueError("y must be [B, n, V]")
    ch = tree_children(parent)
    n_accept = np.zeros(B, dtype=np.int64)
    path = np.full((B, n), -1, dtype=np.int64)
    out_tokens = np.full((B, n), -1, dtype=np.int64)
    ratio = np.full((B, n), np.nan)
    draws = []
    for b in range(B):
        v = 0
        m = 0
        while True:
            if not ch[v]:
                w = target_probs(z[b, v], T)
                kind, rejected = "bonus", 0
                break
            _, q, p_hat = retrieval_augmented_target(z[b, v], y[b, v], T, eta)
            R = p_hat
            accepted = None
            rejected = 0
            for c in ch[v]:
                x = int(tokens[b, c])
                if not 0 <= x < V:
                    raise ValueError("draft token id out of range")
                ratio[b, c] = min(1.0, R[x] / q[x])
                if float(r[b, c]) <= ratio[b, c]:
                    accepted = c
                    break
                w_next = np.maximum(R - q, 0.0)
                W_next = np.sum(w_next)
                R = w_next / W_next if W_next > 0 else R
                rejected += 1
            if accepted is None:
                w, kind = R, "residual"
                break
            path[b, m] = accepted
            out_tokens[b, m] = int(tokens[b, accepted])
            m += 1
            v = accepted
        k, C, W = inverse_cdf_ref(w, float(u[b, v]))
        out_tokens[b, m] = k
        n_accept[b] = m
        draws.append({"node": v, "kind": kind, "rejected": rejected, "C": C, "W": W,
                      "target": float(u[b, v]) * W, "k": k, "w": w})
    return {"n_accept": n_accept, "path": path, "out_tokens": out_tokens, "ratio": ratio,
            "draw": draws}
