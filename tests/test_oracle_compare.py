"""Pins for the GPU-vs-oracle comparison rules (CPU only).

Every token and n_accept verdict of the GPU tests goes through
oracle.compare.compare_accept, so it is checked here on outputs built by
hand around an oracle result: the rules it must apply are those of the
acceptance procedure (RAPID blog post, section 2.1 "Background: speculative
decoding": the first rejection cuts the chain and one token is drawn there;
section 2.4: p_hat in place of p), with the boundary flagging at 1e-4.
"""

import numpy as np

from oracle import rapid_accept_ref
from oracle.compare import BOUNDARY_TOL, attn_row_errors, compare_accept, flag_counts

TOL = BOUNDARY_TOL


def _case(r=None, u=None):
    """One sequence, gamma = 3, V = 6, hand-picked logits whose residual at
    every row has both positive and zero entries."""
    z = np.array([[[2.0, 0.5, -1.0, 1.0, 0.0, -0.5],
                   [0.3, 1.5, 0.2, -0.7, 1.1, 0.0],
                   [1.2, -0.3, 0.8, 0.8, -1.5, 0.4],
                   [0.0, 0.9, -0.2, 1.7, 0.3, -1.0]]])
    y = np.array([[[1.0, 1.5, -1.0, 0.2, 0.0, -0.5],
                   [0.9, 0.4, 0.2, -0.1, 1.6, -0.8],
                   [0.2, 0.1, 1.8, 0.3, -1.0, 0.4]]])
    draft = np.array([[1, 4, 2]])
    T, eta = 1.0, 0.5
    r0 = np.array([[0.5, 0.5, 0.5]]) if r is None else np.array([r], dtype=np.float64)
    u0 = np.array([[0.37, 0.37, 0.37, 0.37]]) if u is None else np.array([u], dtype=np.float64)
    ref = rapid_accept_ref(z, y, draft, r0, u0, T, eta)
    return z, y, draft, r0, u0, T, eta, ref


def _ratios():
    return _case()[-1]["ratio"][0]


def _reject_at(t_star, flag_t=None):
    """Uniforms that accept rows < t_star and reject row t_star, each at
    least 0.05 from its ratio unless it is flag_t, which sits at ratio +
    tol/2 (a flagged rejection)."""
    ratio = _ratios()
    r = []
    for t in range(3):
        if t == flag_t:
            r.append(ratio[t] + 0.5 * TOL)
        elif t < t_star:
            r.append(max(0.0, ratio[t] - 0.05))
        else:
            r.append(min(0.999, ratio[t] + 0.05))
    return r


def test_case_has_rejections_and_zero_weights():
    ratio = _ratios()
    assert np.all(ratio < 0.9) and np.all(ratio > 0.1)
    ref = _case(r=_reject_at(1))[-1]
    assert ref["n_accept"][0] == 1
    w = ref["draw"][0]["w"]
    assert np.any(w == 0) and np.any(w > 0)


def test_identical_outputs_pass():
    for t_star in range(4):
        z, y, draft, r, u, T, eta, ref = _case(r=_reject_at(t_star))
        assert ref["n_accept"][0] == t_star
        res = compare_accept(ref, ref["n_accept"], ref["out_tokens"], r, u, draft=draft)
        assert res["errors"] == [] and res["diverged"] == 0
        assert res["flagged_accept"] == 0 and res["flagged_draw"] == 0


def test_wrong_unflagged_n_accept_is_an_error():
    z, y, draft, r, u, T, eta, ref = _case(r=_reject_at(1))
    for n_bad in (0, 2, 3):
        tok = np.full((1, 4), -1)
        tok[0, :n_bad] = draft[0, :n_bad]
        tok[0, n_bad] = 0
        res = compare_accept(ref, [n_bad], tok, r, u, draft=draft)
        assert res["errors"] and res["diverged"] == 0, n_bad


def test_n_accept_outside_range_is_an_error_whatever_the_flags():
    # The last draft's uniform sits on its ratio: a negative index must not
    # read that flag and call the sequence "diverged".
    ratio = _ratios()
    r = [ratio[0] + 0.05, ratio[1] - 0.05, ratio[2]]
    z, y, draft, r, u, T, eta, ref = _case(r=r)
    for n_bad in (-1, -2, 4, 7):
        tok = np.full((1, 4), -1)
        res = compare_accept(ref, [n_bad], tok, r, u, draft=draft)
        assert res["errors"], n_bad
        assert res["diverged"] == 0


def test_wrong_unflagged_token_is_an_error():
    z, y, draft, r, u, T, eta, ref = _case(r=_reject_at(2))
    tok = ref["out_tokens"].copy()
    k = tok[0, 2]
    w = ref["draw"][0]["w"]
    other = [j for j in range(6) if j != k and w[j] > 0][0]
    tok[0, 2] = other
    res = compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)
    assert res["errors"] and res["flagged_draw"] == 0
    tok[0, 2] = 6  # out of the vocabulary
    assert compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)["errors"]


def test_wrong_accepted_prefix_is_an_error():
    z, y, draft, r, u, T, eta, ref = _case(r=_reject_at(2))
    tok = ref["out_tokens"].copy()
    tok[0, 1] = (tok[0, 1] + 1) % 6
    assert compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)["errors"]
    assert compare_accept(ref, ref["n_accept"], tok, r, u)["errors"]


def test_tokens_past_the_draw_must_be_minus_one():
    z, y, draft, r, u, T, eta, ref = _case(r=_reject_at(1))
    for j in (2, 3):
        tok = ref["out_tokens"].copy()
        tok[0, j] = 0
        assert compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)["errors"], j


def _edge_uniform(row, k_edge, r):
    """A uniform whose target u*W lies tol/2 below C[k_edge] at draw row
    `row` (the oracle then picks the first positive id at or below k_edge
    whose interval holds the target)."""
    ref = _case(r=r)[-1]
    d = ref["draw"][0]
    assert d["row"] == row
    C, W = d["C"], d["W"]
    u = (C[k_edge] - 0.5 * TOL * W) / W
    uu = [0.37] * 4
    uu[row] = u
    return uu


def test_flagged_draw_inside_the_widened_interval_passes():
    r = _reject_at(1)
    ref0 = _case(r=r)[-1]
    w = ref0["draw"][0]["w"]
    pos = [j for j in range(6) if w[j] > 0]
    k = pos[0]
    nxt = pos[1]  # next id of positive weight
    u = _edge_uniform(1, k, r)
    z, y, draft, r, u, T, eta, ref = _case(r=r, u=u)
    assert ref["out_tokens"][0, 1] == k
    tok = ref["out_tokens"].copy()
    res = compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)
    assert res["errors"] == [] and res["flagged_draw"] == 1
    tok[0, 1] = nxt  # across the edge, within tol*W of it
    res = compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)
    assert res["errors"] == [] and res["flagged_draw"] == 1


def test_flagged_draw_outside_the_interval_or_on_zero_weight_fails():
    r = _reject_at(1)
    ref0 = _case(r=r)[-1]
    w = ref0["draw"][0]["w"]
    pos = [j for j in range(6) if w[j] > 0]
    zero = [j for j in range(6) if w[j] == 0]
    k = pos[0]
    u = _edge_uniform(1, k, r)
    z, y, draft, r, u, T, eta, ref = _case(r=r, u=u)
    tok = ref["out_tokens"].copy()
    tok[0, 1] = pos[-1]  # far from the target
    if pos[-1] != pos[1]:
        res = compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)
        assert res["errors"] and res["flagged_draw"] == 1
    for j in zero:  # zero-weight ids are never a valid draw, widened or not
        tok[0, 1] = j
        res = compare_accept(ref, ref["n_accept"], tok, r, u, draft=draft)
        assert res["errors"], j


def test_disagreement_at_a_flagged_accept_counts_as_diverged():
    # Oracle: accept row 0, reject row 1 (r_1 = ratio_1 + tol/2, flagged);
    # row 2's uniform is well below its ratio.  A GPU that accepted row 1
    # and row 2 and drew the bonus is consistent with the flag.
    ratio = _ratios()
    r = [ratio[0] - 0.05, ratio[1] + 0.5 * TOL, ratio[2] - 0.05]
    z, y, draft, r, u, T, eta, ref = _case(r=r)
    assert ref["n_accept"][0] == 1
    tok = np.array([[draft[0, 0], draft[0, 1], draft[0, 2], 3]])
    res = compare_accept(ref, [3], tok, r, u, draft=draft)
    assert res["errors"] == [] and res["diverged"] == 1 and res["flagged_accept"] == 1
    # The GPU's continuation past the flag must still agree with the
    # oracle's unflagged decisions: rejecting row 2 there is an error.
    tok = np.array([[draft[0, 0], draft[0, 1], 0, -1]])
    res = compare_accept(ref, [2], tok, r, u, draft=draft)
    assert res["errors"] and res["diverged"] == 0
    # ... and its accepted prefix and tail are checked too.
    tok = np.array([[draft[0, 0], (draft[0, 1] + 1) % 6, draft[0, 2], 3]])
    assert compare_accept(ref, [3], tok, r, u, draft=draft)["errors"]
    tok = np.array([[draft[0, 0], draft[0, 1], 5, 3]])  # n=2: slot 3 must be -1
    assert compare_accept(ref, [2], tok, r, u, draft=draft)["errors"]


def test_disagreement_at_an_unflagged_accept_is_an_error():
    ratio = _ratios()
    r = [ratio[0] - 0.05, ratio[1] + 0.05, ratio[2] - 0.05]
    z, y, draft, r, u, T, eta, ref = _case(r=r)
    tok = np.array([[draft[0, 0], draft[0, 1], draft[0, 2], 3]])
    res = compare_accept(ref, [3], tok, r, u, draft=draft)
    assert res["errors"] and res["diverged"] == 0


def test_batch_counts_are_per_sequence():
    ratio = _ratios()
    cases = [_case(r=_reject_at(1)), _case(r=[ratio[0] + 0.5 * TOL, 0.5, 0.5])]
    z = np.concatenate([c[0] for c in cases])
    y = np.concatenate([c[1] for c in cases])
    draft = np.concatenate([c[2] for c in cases])
    r = np.concatenate([c[3] for c in cases])
    u = np.concatenate([c[4] for c in cases])
    ref = rapid_accept_ref(z, y, draft, r, u, 1.0, 0.5)
    res = compare_accept(ref, ref["n_accept"], ref["out_tokens"], r, u, draft=draft)
    assert res["errors"] == [] and res["flagged_accept"] == 1
    n = ref["n_accept"].copy()
    n[0] = -1
    res = compare_accept(ref, n, ref["out_tokens"], r, u, draft=draft)
    assert len(res["errors"]) == 1 and res["errors"][0].startswith("b=0")


def test_attn_row_errors_hand_values():
    o_ref = np.array([[1.0, -2.0, 0.5], [0.1, 0.0, -0.1]])
    o_gpu = np.array([[1.01, -2.0, 0.5], [0.1, 0.02, -0.1]])
    e = attn_row_errors(o_gpu, o_ref)
    assert e.shape == (2,)
    np.testing.assert_allclose(e, [0.01 / 2.0, 0.02 / 0.1], rtol=1e-12)
    # the error is per row: a bad row does not hide behind a good one
    assert e[0] < 2e-2 < e[1]
    np.testing.assert_array_equal(attn_row_errors(o_ref, o_ref), [0.0, 0.0])


def test_flag_counts_and_exact_draws():
    ratio = _ratios()
    r = [ratio[0] - 0.05, ratio[1] + 0.5 * TOL, 0.5]
    z, y, draft, r, u, T, eta, ref = _case(r=r)
    # rows 0 and 1 evaluated; row 1 flagged at 1e-4, not at 1e-6
    assert flag_counts(ref, r, TOL)[0] == 1
    assert flag_counts(ref, r, 1e-6)[0] == 0
    res = compare_accept(ref, ref["n_accept"], ref["out_tokens"], r, u, draft=draft)
    assert res["exact_draws"] == 1 - flag_counts(ref, r, TOL)[1]
    # a draw placed tol/2 below an edge is flagged at 1e-4 only
    rr = _reject_at(1)
    k = [j for j in range(6) if _case(r=rr)[-1]["draw"][0]["w"][j] > 0][0]
    uu = _edge_uniform(1, k, rr)
    z, y, draft, r, u, T, eta, ref = _case(r=rr, u=uu)
    assert flag_counts(ref, r, TOL)[1:] == (1, 1)
    assert flag_counts(ref, r, 1e-6)[1:] == (0, 1)
    res = compare_accept(ref, ref["n_accept"], ref["out_tokens"], r, u, draft=draft)
    assert res["exact_draws"] == 0 and res["flagged_draw"] == 1


# ------------------------------------------------------ tree comparison rule

from oracle import rapid_tree_accept_ref  # noqa: E402
from oracle.compare import compare_tree_accept  # noqa: E402

_TREE = [-1, 0, 0, 1, 1]


def _tree_case(r, u=None):
    rng = np.random.default_rng(21)
    z = rng.standard_normal((1, 5, 6)) * 2
    y = z + rng.standard_normal((1, 5, 6))
    from oracle import retrieval_augmented_target
    _, q1, ph1 = retrieval_augmented_target(z[0, 1], y[0, 1], 1.0, 0.5)
    # node 3's token is where p_hat_1 falls shortest of q_1: its ratio is below 1
    tok = np.array([[0, 1, 4, int(np.argmax(q1 - ph1)), 5]])
    r = np.array([r], dtype=np.float64)
    u = np.full((1, 5), 0.37) if u is None else np.array([u], dtype=np.float64)
    ref = rapid_tree_accept_ref(z, y, _TREE, tok, r, u, 1.0, 0.5)
    return tok, r, u, ref


def _tree_out(ref):
    return ref["n_accept"].copy(), ref["path"].copy(), ref["out_tokens"].copy()


def test_tree_compare_identical_and_broken_outputs():
    # accept node 1, reject node 3, accept node 4 (a leaf: bonus)
    r0 = _tree_case([0.5] * 5)[-1]["ratio"][0]
    base = [0.5, 0.0, 0.5, 0.999999, 0.0]
    tok, r, u, ref = _tree_case(base)
    assert list(ref["path"][0, :2]) == [1, 4], ref["path"]
    n, p, t = _tree_out(ref)
    res = compare_tree_accept(ref, _TREE, tok, n, p, t, r)
    assert res["errors"] == [] and res["exact_draws"] == 1 and res["diverged"] == 0
    for bad_n in (-1, 5, 9):
        assert compare_tree_accept(ref, _TREE, tok, [bad_n], p, t, r)["errors"]
    p2 = p.copy()
    p2[0, 1] = 3  # node 3 was rejected (r ~ 1): an unflagged wrong decision
    t2 = t.copy()
    t2[0, 1] = tok[0, 3]
    assert compare_tree_accept(ref, _TREE, tok, n, p2, t2, r)["errors"]
    p3 = p.copy()
    p3[0, 1] = 2  # node 2 is not a child of node 1
    assert compare_tree_accept(ref, _TREE, tok, n, p3, t, r)["errors"]
    t3 = t.copy()
    t3[0, 0] = 3  # not node 1's token
    assert compare_tree_accept(ref, _TREE, tok, n, p, t3, r)["errors"]
    t4 = t.copy()
    t4[0, 3] = 0  # past the draw
    assert compare_tree_accept(ref, _TREE, tok, n, p, t4, r)["errors"]
    t5 = t.copy()
    w = ref["draw"][0]["w"]
    t5[0, 2] = [j for j in range(6) if j != t[0, 2] and w[j] > 0][0]
    assert compare_tree_accept(ref, _TREE, tok, n, p, t5, r)["errors"]
    p6 = p.copy()
    p6[0, 3] = 1  # path padding not -1
    assert compare_tree_accept(ref, _TREE, tok, n, p6, t, r)["errors"]
    del r0


def test_tree_compare_flagged_divergence():
    r0 = _tree_case([0.5] * 5)[-1]["ratio"][0]
    # node 1's uniform sits just above its ratio: the oracle rejects node 1;
    # a GPU that accepted it took a flagged decision and diverges
    base = [0.5, r0[1] + 0.5 * BOUNDARY_TOL, 0.999999, 0.0, 0.0]
    tok, r, u, ref = _tree_case(base)
    assert ref["path"][0, 0] != 1
    n = np.array([1])
    p = np.full((1, 5), -1)
    p[0, 0] = 1
    t = np.full((1, 5), -1)
    t[0, 0] = tok[0, 1]
    t[0, 1] = 0
    res = compare_tree_accept(ref, _TREE, tok, n, p, t, r)
    assert res["errors"] == [] and res["diverged"] == 1 and res["flagged_accept"] >= 1
