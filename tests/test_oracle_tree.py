"""Pins for the draft-tree acceptance oracle (CPU only).

The rule is not on the pages (they verify trees only as attention), so it is
pinned by what the mathematics fixes for it:
* on a chain (one child per node) it is the chain procedure of RAPID blog
  section 2.1 with p_hat for p (section 2.4), i.e. rapid_accept_ref, itself
  pinned elsewhere;
* given the path, the token emitted at a node follows p_hat of that node when
  the node's children are independent draws from its q: checked exactly on
  V = 5 with 2 and 3 siblings, using the walk's own ratios and draw weights
  in each branch, and by a seeded Monte-Carlo chi-square on a two-level tree
  (the law at the root and, given the accepted child, at that child);
* the residual after j rejections has the closed form
  max(p_hat - C_j q, 0) / sum, C_1 = 1, C_{j+1} = C_j + sum_v max(p_hat - C_j q, 0),
  derived from the recursion; the library's kernels compute that form.
"""

import itertools

import numpy as np
import pytest
from scipy import stats

from oracle import (draft_probs, rapid_accept_ref, rapid_tree_accept_ref,
                    retrieval_augmented_target, residual_sequence, target_probs,
                    tree_children)

REJECT = np.nextafter(1.0, 0.0)  # rejects every ratio below 1


def _logits(rng, n, V, zs=2.0, noise=1.0):
    z = rng.standard_normal((1, n, V)) * zs
    y = z + rng.standard_normal((1, n, V)) * noise
    return z, y


def test_children_and_validation():
    assert tree_children([-1, 0, 0, 1, 2, 2]) == [[1, 2], [3], [4, 5], [], [], []]
    with pytest.raises(ValueError):
        tree_children([0, 0])
    with pytest.raises(ValueError):
        tree_children([-1, 1])
    rng = np.random.default_rng(1)
    z, y = _logits(rng, 3, 4)
    with pytest.raises(ValueError):
        rapid_tree_accept_ref(z, y, [-1, 0, 0], np.array([[0, 4, 1]]), np.zeros((1, 3)),
                              np.zeros((1, 3)), 1.0, 0.5)


@pytest.mark.parametrize("T,eta", [(1.0, 0.5), (0.7, 1.0), (1.3, 0.0), (1.0, 2.0)])
def test_chain_reduces_to_the_chain_rule(T, eta):
    rng = np.random.default_rng(int(10 * T + eta * 7))
    B, g, V = 6, 5, 50
    z = rng.standard_normal((B, g + 1, V)) * 3
    y = rng.standard_normal((B, g, V)) + z[:, :g]
    draft = rng.integers(0, V, (B, g))
    r = rng.random((B, g))
    r[0] = 0.0  # one sequence accepts every draft (bonus draw)
    u = rng.random((B, g + 1))
    ref = rapid_accept_ref(z, y, draft, r, u, T, eta)
    # the chain as a tree: node t+1 is draft t, child of node t
    parent = [-1] + list(range(g))
    yt = np.concatenate([y, rng.standard_normal((B, 1, V))], axis=1)  # leaf row unused
    tok = np.concatenate([np.zeros((B, 1), int), draft], axis=1)
    rt = np.concatenate([np.full((B, 1), 0.5), r], axis=1)
    tr = rapid_tree_accept_ref(z, yt, parent, tok, rt, u, T, eta)
    np.testing.assert_array_equal(tr["n_accept"], ref["n_accept"])
    np.testing.assert_array_equal(tr["out_tokens"][:, :g + 1], ref["out_tokens"])
    for b in range(B):
        n = int(ref["n_accept"][b])
        np.testing.assert_array_equal(tr["path"][b, :n], np.arange(1, n + 1))
        tested = min(n + 1, g)
        np.testing.assert_allclose(tr["ratio"][b, 1:tested + 1], ref["ratio"][b, :tested],
                                   rtol=0, atol=0)
        assert np.all(np.isnan(tr["ratio"][b, tested + 1:]))
    assert ref["n_accept"][0] == g and tr["draw"][0]["kind"] == "bonus"


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("T,eta", [(1.0, 0.5), (0.7, 2.0), (1.0, 0.0)])
def test_emitted_token_law_exact_enumeration(k, T, eta):
    """Root with k leaf children whose tokens are i.i.d. from q_root: the law
    of the token emitted at the root, assembled from the walk's own ratios and
    final draw weights over every token combination, equals p_hat_root."""
    V = 5
    rng = np.random.default_rng(100 * k + int(10 * T) + int(eta))
    z, y = _logits(rng, k + 1, V)
    parent = [-1] + [0] * k
    _, q, p_hat = retrieval_augmented_target(z[0, 0], y[0, 0], T, eta)
    law = np.zeros(V)
    for xs in itertools.product(range(V), repeat=k):
        prob = np.prod([q[x] for x in xs])
        tok = np.array([[0] + list(xs)])
        stay = 1.0  # probability that every earlier child was rejected
        for j in range(k):
            # children before j rejected, child j (node j+1) accepted
            r = np.full((1, k + 1), REJECT)
            r[0, j + 1] = 0.0
            out = rapid_tree_accept_ref(z, y, parent, tok, r, np.full((1, k + 1), 0.5), T, eta)
            a = out["ratio"][0, j + 1]
            assert out["path"][0, 0] == j + 1 and out["out_tokens"][0, 0] == xs[j]
            law[xs[j]] += prob * stay * a
            stay *= 1.0 - a
            if stay == 0.0:
                break
        if stay > 0.0:
            r = np.full((1, k + 1), REJECT)
            out = rapid_tree_accept_ref(z, y, parent, tok, r, np.full((1, k + 1), 0.5), T, eta)
            d = out["draw"][0]
            assert d["node"] == 0 and d["kind"] == "residual" and d["rejected"] == k
            law += prob * stay * d["w"] / d["W"]
    np.testing.assert_allclose(law, p_hat, rtol=0, atol=1e-15)


def test_residual_closed_form():
    """R_j = max(p_hat - C_j q, 0) / sum, with C_1 = 1 and
    C_{j+1} = C_j + sum max(p_hat - C_j q, 0)."""
    rng = np.random.default_rng(7)
    for V in (5, 50, 2000):
        for _ in range(5):
            z = rng.standard_normal(V) * 2
            y = z + rng.standard_normal(V)
            _, q, p_hat = retrieval_augmented_target(z, y, 1.0, 0.7)
            R = residual_sequence(p_hat, q, 6)
            C = 1.0
            for j in range(1, 7):
                U = np.maximum(p_hat - C * q, 0.0)
                M = np.sum(U)
                if M <= 0:
                    break
                np.testing.assert_allclose(R[j], U / M, rtol=1e-12, atol=1e-15)
                C += M


def test_q_equal_to_p_hat_accepts_the_first_child():
    V = 30
    rng = np.random.default_rng(3)
    z = rng.standard_normal((1, 4, V)) * 2
    y = z.copy()  # q = p, and with eta = 0 p_hat = p = q
    tok = np.array([[0, 5, 6, 7]])
    out = rapid_tree_accept_ref(z, y, [-1, 0, 0, 0], tok, np.full((1, 4), REJECT),
                                np.full((1, 4), 0.3), 1.0, 0.0)
    assert out["n_accept"][0] == 1 and out["path"][0, 0] == 1
    assert out["ratio"][0, 1] == 1.0 and np.all(np.isnan(out["ratio"][0, 2:]))


def test_rejected_siblings_shrink_the_residual_towards_p_hat_minus_q():
    """After a rejection the residual is zero wherever the previous one was
    at most q, and every later sibling is tested against it."""
    V = 40
    rng = np.random.default_rng(4)
    z, y = _logits(rng, 4, V, noise=2.0)
    _, q, p_hat = retrieval_augmented_target(z[0, 0], y[0, 0], 1.0, 0.5)
    R = residual_sequence(p_hat, q, 3)
    # each sibling's token has ratio below 1 against its residual
    tok = np.array([[0] + [int(np.argmax(q - R[j])) for j in range(3)]])
    out = rapid_tree_accept_ref(z, y, [-1, 0, 0, 0], tok, np.full((1, 4), REJECT),
                                np.full((1, 4), 0.3), 1.0, 0.5)
    assert out["n_accept"][0] == 0
    for j in range(3):
        x = tok[0, j + 1]
        assert out["ratio"][0, j + 1] == min(1.0, R[j][x] / q[x])
    np.testing.assert_allclose(out["draw"][0]["w"], R[3], rtol=0, atol=0)
    assert np.all(R[1][p_hat <= q] == 0)


def test_law_monte_carlo_two_levels():
    """Root with 3 children, child 1 with 2 children: over 60000 seeded walks
    with fresh i.i.d. draft tokens, the token emitted at the root follows
    p_hat_root, and given that child 1 was accepted, the next emitted token
    follows p_hat of node 1 (chi-square, p > 1e-3 at the fixed seed)."""
    V, N = 6, 60000
    rng = np.random.default_rng(11)
    parent = [-1, 0, 0, 0, 1, 1]
    n = len(parent)
    z, y = _logits(rng, n, V)
    T, eta = 1.0, 0.8
    q0 = draft_probs(y[0, 0], T)
    q1 = draft_probs(y[0, 1], T)
    _, _, ph0 = retrieval_augmented_target(z[0, 0], y[0, 0], T, eta)
    _, _, ph1 = retrieval_augmented_target(z[0, 1], y[0, 1], T, eta)
    c0 = np.zeros(V)
    c1 = np.zeros(V)
    tok = np.zeros((1, n), int)
    for _ in range(N):
        tok[0, 1:4] = rng.choice(V, 3, p=q0)
        tok[0, 4:6] = rng.choice(V, 2, p=q1)
        out = rapid_tree_accept_ref(z, y, parent, tok, rng.random((1, n)), rng.random((1, n)),
                                    T, eta)
        c0[out["out_tokens"][0, 0]] += 1
        if out["n_accept"][0] >= 1 and out["path"][0, 0] == 1:
            c1[out["out_tokens"][0, 1]] += 1
    for counts, law in ((c0, ph0), (c1, ph1)):
        assert counts.sum() > 1000
        p = stats.chisquare(counts, counts.sum() * law).pvalue
        assert p > 1e-3, (counts, law, p)


def test_leaf_draws_the_bonus_from_p():
    V = 20
    rng = np.random.default_rng(5)
    z, y = _logits(rng, 3, V)
    tok = np.array([[0, 4, 9]])
    # accept node 1 then node 2 (a leaf): bonus from p_2 with u_2
    out = rapid_tree_accept_ref(z, y, [-1, 0, 1], tok, np.zeros((1, 3)),
                                np.array([[0.1, 0.2, 0.77]]), 1.0, 0.5)
    d = out["draw"][0]
    assert out["n_accept"][0] == 2 and d["node"] == 2 and d["kind"] == "bonus"
    np.testing.assert_allclose(d["w"], target_probs(z[0, 2], 1.0), rtol=0, atol=0)
    C = np.cumsum(target_probs(z[0, 2], 1.0))
    assert out["out_tokens"][0, 2] == int(np.searchsorted(C, 0.77 * C[-1], side="right"))
