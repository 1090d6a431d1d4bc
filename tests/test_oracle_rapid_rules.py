"""Pins for the two optional rules of RAPID blog section 2.4 (CPU only):
the tail-preserving adjustment of p_hat and the printed residual
norm(max(p - p_hat, p - q)), clipped at zero."""

import json
import os

import numpy as np
import pytest
from scipy import special

from oracle import rapid_accept_ref, retrieval_augmented_target, tail_preserve_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rapid_tail_rule_examples.json")


def test_tail_rule_hand_examples():
    fx = json.load(open(GOLDEN))
    for c in fx["cases"]:
        got = tail_preserve_ref(np.array(c["p"]), np.array(c["p_hat"]))
        np.testing.assert_allclose(got, c["expected"], rtol=0, atol=1e-15, err_msg=c["name"])


def test_tail_rule_is_identity_when_p_hat_is_p_or_has_no_tail():
    rng = np.random.default_rng(0)
    z = rng.standard_normal(500) * 3
    y = z + rng.standard_normal(500)
    p, _, ph = retrieval_augmented_target(z, y, 1.0, 0.0)  # eta = 0: p_hat == p
    np.testing.assert_allclose(tail_preserve_ref(p, ph), p, rtol=1e-14)
    flat = np.full(8, 1 / 8)
    np.testing.assert_array_equal(tail_preserve_ref(special.softmax(rng.random(8)), flat), flat)


def test_tail_rule_keeps_head_ratios_and_sums_to_one():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.standard_normal(64) * 3
        y = z + rng.standard_normal(64)
        p, _, ph = retrieval_augmented_target(z, y, 0.8, 1.5)
        adj = tail_preserve_ref(p, ph)
        assert abs(adj.sum() - 1) < 1e-14
        head = ph >= 0.1 * ph.max()
        # head entries keep their mutual ratios; tail entries are p up to one scale
        np.testing.assert_allclose(adj[head] / adj[head].sum(), ph[head] / ph[head].sum(),
                                   rtol=1e-12)
        if (~head).any():
            s = adj[~head] / p[~head]
            np.testing.assert_allclose(s, s[0], rtol=1e-12)


def test_tail_rule_forced_sides():
    """The classification override: forcing each entry to the side the rule
    puts it on changes nothing; moving one tail entry k into the head gives
    p_hat_k (not p_k) for it, every other entry keeps its value relative to
    the rest, and the row still sums to one (hand-checkable on 4 entries)."""
    p = np.array([0.4, 0.3, 0.2, 0.1])
    ph = np.array([0.70, 0.20, 0.06, 0.04])   # threshold 0.07: entries 2, 3 in the tail
    base = tail_preserve_ref(p, ph)
    np.testing.assert_array_equal(tail_preserve_ref(p, ph, force={0: True, 2: False}), base)
    # by hand: kept (0.70, 0.20), tail from p (0.2, 0.1), sum 1.2
    np.testing.assert_allclose(base, np.array([0.70, 0.20, 0.2, 0.1]) / 1.2, rtol=0, atol=1e-15)
    moved = tail_preserve_ref(p, ph, force={2: True})
    np.testing.assert_allclose(moved, np.array([0.70, 0.20, 0.06, 0.1]) / 1.06, rtol=0,
                               atol=1e-15)
    dropped = tail_preserve_ref(p, ph, force={1: False})
    np.testing.assert_allclose(dropped, np.array([0.70, 0.3, 0.2, 0.1]) / 1.3, rtol=0, atol=1e-15)


def test_tail_force_reaches_the_acceptance_step():
    """rapid_accept_ref's tail_force is the same override, per (sequence,
    row): an empty one leaves every output bit-identical, and forcing the
    drafted token's entry changes that row's ratio exactly as the forced
    rule says."""
    g = np.random.default_rng(7)
    V, gamma = 30, 3
    z = g.standard_normal((1, gamma + 1, V)) * 3
    y = z[:, :gamma] + g.standard_normal((1, gamma, V))
    draft = g.integers(0, V, size=(1, gamma))
    r = np.zeros((1, gamma))
    u = g.random((1, gamma + 1))
    a = rapid_accept_ref(z, y, draft, r, u, 1.0, 1.0, tail_preserve=True)
    b = rapid_accept_ref(z, y, draft, r, u, 1.0, 1.0, tail_preserve=True, tail_force={})
    for k in ("n_accept", "out_tokens", "ratio", "p_hat"):
        np.testing.assert_array_equal(a[k], b[k])
    x = int(draft[0, 1])
    p, q, ph = retrieval_augmented_target(z[0, 1], y[0, 1], 1.0, 1.0)
    side = bool(ph[x] >= 0.1 * ph.max())
    c = rapid_accept_ref(z, y, draft, r, u, 1.0, 1.0, tail_preserve=True,
                         tail_force={(0, 1): {x: not side}})
    want = tail_preserve_ref(p, ph, force={x: not side})
    assert c["ratio"][0, 1] == min(1.0, want[x] / q[x])
    np.testing.assert_array_equal(c["ratio"][0, [0, 2]], a["ratio"][0, [0, 2]])


def test_printed_residual_is_the_background_rule_when_eta_is_zero():
    """With eta = 0, p_hat = p and max(p - min(p, q), 0) = max(p - q, 0):
    the printed rule reduces to the background residual of section 2.1."""
    rng = np.random.default_rng(2)
    V, gamma = 40, 4
    for s in range(40):
        g = np.random.default_rng(100 + s)
        z = g.standard_normal((2, gamma + 1, V)) * 3
        y = z[:, :gamma] + g.standard_normal((2, gamma, V))
        draft = g.integers(0, V, size=(2, gamma))
        r, u = g.random((2, gamma)), g.random((2, gamma + 1))
        a = rapid_accept_ref(z, y, draft, r, u, 1.0, 0.0, residual="p_hat")
        b = rapid_accept_ref(z, y, draft, r, u, 1.0, 0.0, residual="printed")
        np.testing.assert_array_equal(a["out_tokens"], b["out_tokens"])


def _stratified_law(z, y, T, eta, M, **kw):
    V = z.shape[-1]
    qd = special.softmax(y / T)
    grid = (np.arange(M) + 0.5) / M
    zz = np.stack([z, z])[None]
    law = np.zeros(V)
    for x in range(V):
        acc = sum(int(rapid_accept_ref(zz, y[None, None], np.array([[x]]), np.array([[r]]),
                                       np.array([[0.5, 0.5]]), T, eta, **kw)["n_accept"][0] == 1)
                  for r in grid) / M
        res = np.zeros(V)
        for uu in grid:
            out = rapid_accept_ref(zz, y[None, None], np.array([[x]]), np.array([[1 - 1e-12]]),
                                   np.array([[uu, 0.5]]), T, eta, **kw)
            if out["n_accept"][0] == 0:
                res[out["out_tokens"][0, 0]] += 1
        if res.sum():
            res /= M
        law += qd[x] * acc * np.eye(V)[x] + qd[x] * (1 - acc) * res
    return law


@pytest.mark.parametrize("tail,residual", [(True, "p_hat"), (False, "printed"), (True, "printed")])
def test_output_law_under_each_rule(tail, residual):
    """Integrated over the uniforms, the procedure's output law is
    min(q, a) + (1 - sum min(q, a)) w / sum w, with a the (adjusted) p_hat and
    w the residual weights of the rule; with the p_hat residual it is a."""
    rng = np.random.default_rng(3)
    V, T, eta = 5, 1.0, 1.5
    z = rng.standard_normal(V) * 2
    y = z + rng.standard_normal(V) * 1.5
    p, q, ph = retrieval_augmented_target(z, y, T, eta)
    a = tail_preserve_ref(p, ph) if tail else ph
    w = np.maximum(a - q, 0) if residual == "p_hat" else np.maximum(p - np.minimum(a, q), 0)
    mins = np.minimum(q, a)
    law_expect = mins + (1 - mins.sum()) * w / w.sum()
    law = _stratified_law(z, y, T, eta, 600, tail_preserve=tail, residual=residual)
    np.testing.assert_allclose(law, law_expect, atol=5e-3)
    if residual == "p_hat":
        np.testing.assert_allclose(law, a, atol=5e-3)
    else:
        # the page claims the output follows p; with eta > 0 the clip makes it
        # differ unless p >= min(p_hat, q) everywhere
        clipped = (p - np.minimum(a, q)) < 0
        if not clipped.any():
            np.testing.assert_allclose(law, p, atol=5e-3)


def test_printed_rule_law_is_p_when_nothing_is_clipped():
    """eta = 0: p_hat = p, p >= min(p, q) holds everywhere, and the output
    law is exactly the target p (the guarantee the page states)."""
    rng = np.random.default_rng(4)
    V, T = 5, 0.8
    z = rng.standard_normal(V) * 2
    y = z + rng.standard_normal(V) * 1.5
    p = special.softmax(z / T)
    law = _stratified_law(z, y, T, 0.0, 600, residual="printed")
    np.testing.assert_allclose(law, p, atol=5e-3)
