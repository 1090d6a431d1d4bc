"""Pins for the RAPID acceptance oracle (CPU only).

What fixes each part, from outside the oracle:
* softmax: scipy's routine and hand values;
* p_hat: the hand-derived two/three-token examples in
  tests/golden/rapid_hand_examples.json, the eta = 0 fixed point, and the
  gradient-step derivation of the RAPID blog post (section 2.4,
  Proposition 1) evaluated with a finite-difference gradient;
* the inverse CDF: brute force and numpy.searchsorted;
* the accept / resample procedure: its output law must be p_hat (the
  speculative-sampling guarantee of blog section 2.1 with p replaced by
  p_hat), checked by a stratified exact integration over the uniforms and by
  a seeded Monte-Carlo chi-square test; the first-reject cut by the
  accepted-length law and by constructed uniforms.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

from oracle import (draft_probs, inverse_cdf_ref, rapid_accept_ref, retrieval_augmented_target,
                    softmax_ref, target_probs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rapid_hand_examples.json")


# ------------------------------------------------------------- softmax (P1)

def test_softmax_matches_scipy_and_hand_values():
    rng = np.random.default_rng(0)
    for scale in (0.1, 3.0, 40.0):
        x = rng.standard_normal(1000) * scale
        np.testing.assert_allclose(softmax_ref(x), special.softmax(x), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(softmax_ref([0.0, math.log(2), math.log(3)]), [1 / 6, 1 / 3, 1 / 2],
                               rtol=1e-15)
    p = softmax_ref([1000.0, 1000.0 - math.log(3)])  # no overflow
    np.testing.assert_allclose(p, [0.75, 0.25], rtol=1e-12)  # 1000 - ln 3 is itself rounded


def test_temperature_divides_logits():
    for T in (0.7, 1.0, 2.5):
        z = np.array([0.0, T * math.log(2.0)])
        np.testing.assert_allclose(target_probs(z, T), [1 / 3, 2 / 3], rtol=1e-15)
        np.testing.assert_allclose(draft_probs(z, T), [1 / 3, 2 / 3], rtol=1e-15)


# ------------------------------------------------------------ p_hat (P2-P4)

def test_p_hat_hand_examples():
    fx = json.load(open(GOLDEN))
    for c in fx["cases"]:
        p, q, ph = retrieval_augmented_target(np.array(c["z"]), np.array(c["y"]), c["T"], c["eta"])
        np.testing.assert_allclose(p, c["p"], rtol=0, atol=1e-15, err_msg=c["name"])
        if "q" in c:
            np.testing.assert_allclose(q, c["q"], rtol=0, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(ph, c["p_hat"], rtol=0, atol=1e-15, err_msg=c["name"])


@pytest.mark.parametrize("T", [0.7, 1.0, 1.9])
def test_eta_zero_is_the_target_exactly(T):
    rng = np.random.default_rng(1)
    z = rng.standard_normal(4000) * 3
    y = z + rng.standard_normal(4000)
    p, _, ph = retrieval_augmented_target(z, y, T, 0.0)
    np.testing.assert_array_equal(ph, p)


def _kd_loss(z, q, T):
    """T^2 * KL(q || softmax(z/T)) with scipy's log-sum-exp."""
    logp = z / T - special.logsumexp(z / T)
    return T * T * float(np.sum(q * (np.log(q) - logp)))


@pytest.mark.parametrize("T,eta", [(1.0, 0.5), (0.7, 1.0), (2.0, 2.0)])
def test_p_hat_equals_one_distillation_step(T, eta):
    """Proposition 1 (blog section 2.4): dL/dz = T (p - q) for
    L = T^2 KL(q||p); the distilled logits z - eta*dL/dz, tempered by T, give
    p_hat.  The gradient is taken here by central differences."""
    rng = np.random.default_rng(2)
    V = 12
    z = rng.standard_normal(V) * 2
    q = special.softmax(rng.standard_normal(V))
    h = 1e-6
    grad = np.zeros(V)
    for i in range(V):
        e = np.zeros(V)
        e[i] = h
        grad[i] = (_kd_loss(z + e, q, T) - _kd_loss(z - e, q, T)) / (2 * h)
    p = special.softmax(z / T)
    np.testing.assert_allclose(grad, T * (p - q), rtol=0, atol=1e-8)
    z_hat = z - eta * grad
    # feed the oracle draft logits whose tempered softmax is q
    _, q_or, ph = retrieval_augmented_target(z, T * np.log(q), T, eta)
    np.testing.assert_allclose(q_or, q, rtol=1e-13)
    np.testing.assert_allclose(ph, special.softmax(z_hat / T), rtol=0, atol=1e-8)


# -------------------------------------------------------- inverse CDF (P7)

def test_inverse_cdf_bruteforce_and_searchsorted():
    rng = np.random.default_rng(3)
    for trial in range(200):
        V = int(rng.integers(1, 9))
        w = rng.random(V)
        w[rng.random(V) < 0.4] = 0.0
        if not (w > 0).any():
            w[int(rng.integers(0, V))] = 0.3
        for u in list(rng.random(5)) + [0.0]:
            k, C, W = inverse_cdf_ref(w, u)
            # brute force: walk the ids in order
            acc, kb = 0.0, None
            for j in range(V):
                acc += w[j]
                if acc > u * W:
                    kb = j
                    break
            assert k == kb
            assert k == min(int(np.searchsorted(C, u * W, side="right")), V - 1)
            assert w[k] > 0


def test_inverse_cdf_never_returns_zero_weight_ids():
    w = np.array([0.0, 0.2, 0.0, 0.0, 0.5, 0.0])
    seen = set()
    for u in np.linspace(0, 1, 1001, endpoint=False):
        k, _, _ = inverse_cdf_ref(w, u)
        seen.add(k)
    assert seen == {1, 4}
    # rounding fallback: target at the very top picks the last positive id
    k, _, _ = inverse_cdf_ref(w, 1.0)
    assert k == 4


# --------------------------------------------------- hand accept examples

def test_accept_hand_examples():
    fx = json.load(open(GOLDEN))
    for a in fx["accept_cases"]:
        c = fx["cases"][a["case"]]
        V = len(c["z"])
        z_last = a.get("z_last", [0.0] * V)
        z = np.array([[c["z"], z_last]], dtype=np.float64)
        y = np.array([[c["y"]]], dtype=np.float64)
        u = np.array([[a.get("u", 0.5), a.get("u_bonus", 0.5)]])
        out = rapid_accept_ref(z, y, np.array([[a["draft"]]]), np.array([[a["r"]]]), u,
                               c["T"], c["eta"])
        assert abs(out["ratio"][0, 0] - min(1.0, a["ratio"])) < 1e-15, a["name"]
        assert out["n_accept"][0] == a["n_accept"], a["name"]
        assert out["out_tokens"][0].tolist() == a["tokens"], a["name"]


# ------------------------------------------------- sampling law (P5, P6)

def _law_by_stratification(z, y, T, eta, M=4000):
    """Output law of one verify step (gamma = 1) integrated over the
    uniforms: r and u each run over M midpoints of [0, 1); the draft runs
    over every id weighted by the drafter's probability (scipy softmax)."""
    V = z.shape[-1]
    qd = special.softmax(np.asarray(y, np.float64) / T)
    grid = (np.arange(M) + 0.5) / M
    law = np.zeros(V)
    zz = np.stack([z, z])[None]  # bonus row unused when a draft is rejected
    for x in range(V):
        acc = 0
        for r in grid:
            out = rapid_accept_ref(zz, y[None, None], np.array([[x]]), np.array([[r]]),
                                   np.array([[0.5, 0.5]]), T, eta)
            acc += int(out["n_accept"][0] == 1)
        f_acc = acc / M
        res = np.zeros(V)
        for uu in grid:
            out = rapid_accept_ref(zz, y[None, None], np.array([[x]]), np.array([[1.0 - 1e-12]]),
                                   np.array([[uu, 0.5]]), T, eta)
            if out["n_accept"][0] == 0:
                res[out["out_tokens"][0, 0]] += 1
        res = res / M if res.sum() > 0 else res
        law[x] += qd[x] * f_acc
        law += qd[x] * (1 - f_acc) * res
    return law


@pytest.mark.parametrize("T,eta,kind", [(1.0, 0.5, "random"), (0.7, 2.0, "random"),
                                        (1.0, 0.0, "random"), (1.0, 1.0, "disjoint")])
def test_output_law_is_p_hat_stratified(T, eta, kind):
    rng = np.random.default_rng(4)
    V = 5
    if kind == "random":
        z = rng.standard_normal(V) * 2
        y = z + rng.standard_normal(V) * 1.5
    else:  # target favours id 0, drafter favours id 4: almost every draft is rejected
        z = np.array([6.0, 0.0, 0.0, 0.0, -2.0])
        y = np.array([-3.0, 0.0, 0.0, 0.0, 7.0])
    _, _, ph = retrieval_augmented_target(z, y, T, eta)
    law = _law_by_stratification(z, y, T, eta, M=1000)
    # each stratified fraction is within 1/M of its exact value
    np.testing.assert_allclose(law, ph, rtol=0, atol=3e-3)


def test_q_equal_p_hat_never_rejects():
    rng = np.random.default_rng(5)
    V, gamma = 50, 4
    z = rng.standard_normal((1, gamma + 1, V)) * 3
    y = z[:, :gamma].copy()  # q == p and eta == 0 -> p_hat == q
    for s in range(30):
        g = np.random.default_rng(100 + s)
        draft = g.integers(0, V, size=(1, gamma))
        r = g.random((1, gamma)) * (1 - 1e-9)
        out = rapid_accept_ref(z, y, draft, r, g.random((1, gamma + 1)), 1.0, 0.0)
        assert out["n_accept"][0] == gamma
        np.testing.assert_allclose(out["ratio"], 1.0, rtol=1e-12)


def test_monte_carlo_chi_square_against_p_hat():
    """Seeded end-to-end sampler: draft from q, then r, then u."""
    rng = np.random.default_rng(6)
    V, T, eta = 5, 0.7, 2.0
    z = rng.standard_normal(V) * 2
    y = z + rng.standard_normal(V)
    _, q, ph = retrieval_augmented_target(z, y, T, eta)
    N = 40000
    g = np.random.default_rng(7)
    xs = g.choice(V, size=N, p=special.softmax(y / T))
    rs = g.random(N)
    us = g.random(N)
    counts = np.zeros(V)
    zz = np.stack([z, z])[None]
    for x, r, uu in zip(xs, rs, us):
        out = rapid_accept_ref(zz, y[None, None], np.array([[x]]), np.array([[r]]),
                               np.array([[uu, 0.5]]), T, eta)
        counts[out["out_tokens"][0, 0]] += 1
    chi2, pval = stats.chisquare(counts, N * ph)
    assert pval > 1e-3, (counts, N * ph, pval)


def test_first_reject_cut_and_token_layout():
    rng = np.random.default_rng(8)
    V, gamma = 40, 5
    z = rng.standard_normal((1, gamma + 1, V)) * 3
    y = z[:, :gamma] + rng.standard_normal((1, gamma, V))
    out0 = rapid_accept_ref(z, y, np.zeros((1, gamma), int), np.zeros((1, gamma)),
                            np.full((1, gamma + 1), 0.5), 1.0, 0.5)
    ratio = out0["ratio"][0]
    draft = rng.integers(0, V, size=(1, gamma))
    out0 = rapid_accept_ref(z, y, draft, np.zeros((1, gamma)), np.full((1, gamma + 1), 0.5), 1.0, 0.5)
    ratio = out0["ratio"][0]
    # r = 0 accepts everything (ratio > 0): bonus drawn from the last target row
    assert out0["n_accept"][0] == gamma
    assert out0["out_tokens"][0, :gamma].tolist() == draft[0].tolist()
    assert out0["draw"][0]["kind"] == "bonus"
    # reject exactly at position 2: r above ratio there, below it before
    for cut in range(gamma):
        if ratio[cut] >= 1.0:
            continue
        r = np.zeros((1, gamma))
        r[0, cut] = min(1 - 1e-9, ratio[cut] + (1 - ratio[cut]) / 2)
        r[0, cut + 1:] = 0.999  # must not matter
        out = rapid_accept_ref(z, y, draft, r, np.full((1, gamma + 1), 0.37), 1.0, 0.5)
        assert out["n_accept"][0] == cut
        toks = out["out_tokens"][0].tolist()
        assert toks[:cut] == draft[0, :cut].tolist()
        assert toks[cut] >= 0 and all(t == -1 for t in toks[cut + 1:])
        assert out["draw"][0]["row"] == cut and out["draw"][0]["kind"] == "residual"
        # only u[cut] is used
        u2 = np.full((1, gamma + 1), 0.9)
        u2[0, cut] = 0.37
        assert rapid_accept_ref(z, y, draft, r, u2, 1.0, 0.5)["out_tokens"][0].tolist() == toks
    # boundary: r equal to the ratio is accepted (inclusive test)
    r = np.zeros((1, gamma))
    r[0, 0] = ratio[0]
    assert rapid_accept_ref(z, y, draft, r, np.full((1, gamma + 1), 0.5), 1.0, 0.5)["n_accept"][0] >= 1


def test_bonus_token_law_is_last_target_row():
    rng = np.random.default_rng(9)
    V, T = 6, 0.7
    z = rng.standard_normal((1, 2, V)) * 2
    y = z[:, :1].copy()
    counts = np.zeros(V)
    M = 3000
    for uu in (np.arange(M) + 0.5) / M:
        out = rapid_accept_ref(z, y, np.array([[0]]), np.array([[0.0]]), np.array([[0.5, uu]]), T, 0.0)
        counts[out["out_tokens"][0, 1]] += 1
    np.testing.assert_allclose(counts / M, special.softmax(z[0, 1] / T), atol=2.0 / M)


def test_accepted_length_law():
    """Rows are independent here, so P(accept row t | rows < t accepted) is
    alpha_t = sum_v min(q_t, p_hat_t) and E[n_accept] = sum_k prod_{t<k} alpha_t."""
    rng = np.random.default_rng(10)
    V, gamma, T, eta = 8, 4, 1.0, 0.5
    z = rng.standard_normal((1, gamma + 1, V)) * 2
    y = z[:, :gamma] + rng.standard_normal((1, gamma, V)) * 1.2
    alphas = []
    qs = []
    for t in range(gamma):
        _, q, ph = retrieval_augmented_target(z[0, t], y[0, t], T, eta)
        alphas.append(np.minimum(q, ph).sum())
        qs.append(special.softmax(y[0, t] / T))
    expect = sum(np.prod(alphas[:k]) for k in range(1, gamma + 1))
    N = 6000
    g = np.random.default_rng(11)
    tot, tot2 = 0.0, 0.0
    for _ in range(N):
        draft = np.array([[g.choice(V, p=qs[t]) for t in range(gamma)]])
        n = rapid_accept_ref(z, y, draft, g.random((1, gamma)), g.random((1, gamma + 1)), T, eta)["n_accept"][0]
        tot += n
        tot2 += n * n
    mean = tot / N
    sd = math.sqrt(max(tot2 / N - mean ** 2, 1e-12) / N)
    assert abs(mean - expect) < 4 * sd, (mean, expect, sd)
