"""GPU Monte-Carlo: the output law of rapid_accept / rapid_accept_ex.

With gamma = 1 the first emitted token is the draft x ~ q if it is accepted
and a residual draw otherwise, so over the uniforms its law is
    min(q, a) + (1 - sum min(q, a)) * w / sum w,
a the (possibly tail-adjusted) p_hat and w the rule's residual weights (the
oracle tests pin this closed form against the step-by-step procedure).  With
the p_hat residual it is a itself; RAPID blog section 2.4 states that the
printed residual makes the output follow the target p, which holds when no
weight is clipped.  Each rule runs on 262,140 independent sequences sharing
one pair of logit rows; the empirical law is tested against the closed form
(chi-square) and its total-variation distances to p and to p_hat are
reported.
"""

import numpy as np
import pytest
import torch
from scipy import stats

from oracle import retrieval_augmented_target, tail_preserve_ref
from speculative_decoding_verify_split_amd import rapid_verify as rv

pytestmark = pytest.mark.gpu

B = 65535
CALLS = 4


def _inputs(seed, V, T):
    g = np.random.default_rng(seed)
    z = g.standard_normal(V) * 2.0
    y = z + g.standard_normal(V) * 1.5
    return z.astype(np.float32), y.astype(np.float32)


def _law(z, y, T, eta, tail, printed):
    p, q, ph = retrieval_augmented_target(z.astype(np.float64), y.astype(np.float64), T, eta)
    a = tail_preserve_ref(p, ph) if tail else ph
    w = np.maximum(p - np.minimum(a, q), 0) if printed else np.maximum(a - q, 0)
    mins = np.minimum(q, a)
    return p, q, a, mins + (1 - mins.sum()) * w / w.sum()


@pytest.mark.parametrize("flags", [0, rv.RV_ACCEPT_TAIL_PRESERVE, rv.RV_ACCEPT_PRINTED_RESIDUAL,
                                   rv.RV_ACCEPT_TAIL_PRESERVE | rv.RV_ACCEPT_PRINTED_RESIDUAL])
def test_first_token_law(flags):
    V, T, eta = 48, 1.0, 1.5
    tail = bool(flags & rv.RV_ACCEPT_TAIL_PRESERVE)
    printed = bool(flags & rv.RV_ACCEPT_PRINTED_RESIDUAL)
    z1, y1 = _inputs(7, V, T)
    p, q, a, law = _law(z1, y1, T, eta, tail, printed)
    dev = "cuda"
    z = torch.from_numpy(np.broadcast_to(np.stack([z1, z1]), (B, 2, V)).copy()).to(dev)
    y = torch.from_numpy(np.broadcast_to(y1, (B, 1, V)).copy()).to(dev)
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, 2, dtype=torch.int32, device=dev)
    ws = torch.empty(rv.rapid_accept_workspace_size(B, 1, V), dtype=torch.uint8, device=dev)
    g = np.random.default_rng(1000 + flags)
    cq = np.cumsum(q)
    counts = np.zeros(V, np.int64)
    accepted = 0
    for _ in range(CALLS):
        # drafts x ~ q by inverse CDF of host uniforms; acceptance and sampling
        # uniforms in [0, 1)
        x = np.minimum(np.searchsorted(cq, g.random(B) * cq[-1], side="right"), V - 1)
        draft = torch.from_numpy(x.astype(np.int32).reshape(B, 1)).to(dev)
        r = torch.from_numpy(g.random((B, 1), dtype=np.float32)).to(dev)
        u = torch.from_numpy(g.random((B, 2), dtype=np.float32)).to(dev)
        if flags:
            rv.rapid_accept_ex(z, y, draft, r, u, T, eta, flags, n_acc, tok, ws)
        else:
            rv.rapid_accept(z, y, draft, r, u, T, eta, n_acc, tok, ws)
        torch.cuda.synchronize()
        first = tok[:, 0].cpu().numpy()
        na = n_acc.cpu().numpy()
        assert set(np.unique(na)) <= {0, 1}
        assert np.all((first >= 0) & (first < V))
        counts += np.bincount(first, minlength=V)
        accepted += int(na.sum())
    N = counts.sum()
    emp = counts / N
    pos = law > 0
    assert counts[~pos].sum() == 0, "a token of zero probability was emitted"
    chi2 = float(np.sum((counts[pos] - N * law[pos]) ** 2 / (N * law[pos])))
    pval = float(stats.chi2.sf(chi2, pos.sum() - 1))
    tv = lambda u_, v_: 0.5 * float(np.abs(u_ - v_).sum())
    acc_expect = float(np.minimum(q, a).sum())
    print("[gpu-case] law flags=%d N=%d chi2=%.1f (dof %d) p=%.3g  TV(emp,law)=%.4f "
          "TV(emp,p)=%.4f TV(emp,p_hat)=%.4f  accept rate %.4f (expect %.4f)"
          % (flags, N, chi2, pos.sum() - 1, pval, tv(emp, law), tv(emp, p), tv(emp, a),
             accepted / N, acc_expect), flush=True)
    assert pval > 1e-4
    assert tv(emp, law) < 0.01
    assert abs(accepted / N - acc_expect) < 5 * np.sqrt(acc_expect * (1 - acc_expect) / N)
    if not printed:
        assert tv(emp, a) < 0.01  # the p_hat residual reproduces p_hat itself
