"""GPU parity of rapid_tree_accept (acceptance over a draft tree) against the
fp64 tree oracle, through the C ABI.  Tolerances and boundary flagging as for
the chain (oracle/compare.py): ratios of the tested children to 1e-5, paths
and tokens bit-exact outside flagged positions."""

import sys

import numpy as np
import pytest
import torch

from oracle import rapid_tree_accept_ref
from oracle.compare import compare_tree_accept
from workloads import config_tree_vocab, config_vocab, make_tree_vocab, tree_parents
from speculative_decoding_verify_split_amd import rapid_verify as rv
from speculative_decoding_verify_split_amd.step import VerifyStep, to_device

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def _run_tree(vi):
    B, n, V = vi.z.shape
    dev = {k: to_device(getattr(vi, k)) for k in ("z", "y", "tokens", "r", "u")}
    n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    path = torch.empty((B, n), dtype=torch.int32, device="cuda")
    tok = torch.empty((B, n), dtype=torch.int32, device="cuda")
    ratio = torch.empty((B, n), dtype=torch.float32, device="cuda")
    ws = torch.empty((rv.rapid_tree_accept_workspace_size(B, n, V),), dtype=torch.uint8,
                     device="cuda")
    rv.rapid_tree_accept(dev["z"], dev["y"], dev["tokens"], list(vi.parent), dev["r"], dev["u"],
                         vi.T, vi.eta, n_acc, path, tok, ws, ratio)
    torch.cuda.synchronize()
    return (n_acc.cpu().numpy(), path.cpu().numpy(), tok.cpu().numpy(), ratio.cpu().numpy())


def _check_tree(vi, tag):
    n_g, path_g, tok_g, ratio_g = _run_tree(vi)
    ref = rapid_tree_accept_ref(vi.z, vi.y, vi.parent, vi.tokens, vi.r, vi.u, vi.T, vi.eta)
    res = compare_tree_accept(ref, vi.parent, vi.tokens, n_g, path_g, tok_g, vi.r)
    # ratios of children both sides tested (the same set where paths agree)
    both = ~np.isnan(ref["ratio"]) & ~np.isnan(ratio_g)
    dr = float(np.max(np.abs(ratio_g[both] - ref["ratio"][both]))) if both.any() else 0.0
    same = [np.array_equal(path_g[b], ref["path"][b]) for b in range(len(n_g))]
    for b in range(len(n_g)):
        if same[b]:
            assert np.array_equal(np.isnan(ratio_g[b]), np.isnan(ref["ratio"][b])), b
    announce("  %s: n_accept gpu=%s ref=%s |dratio|=%.2e flagged(acc=%d, draw=%d) diverged=%d "
             "exact draws=%d" % (tag, n_g.tolist()[:8], ref["n_accept"].tolist()[:8], dr,
                                 res["flagged_accept"], res["flagged_draw"], res["diverged"],
                                 res["exact_draws"]))
    assert not res["errors"], res["errors"]
    assert dr <= 1e-5
    return ref, res


TREE_CASES = [
    # name, seed, B, n, depth, V, z_sigma, noise, T, eta
    ("root-only", 71, 2, 1, 0, 1000, 3.0, 1.0, 1.0, 0.5),
    ("n2-V2", 72, 4, 2, 1, 2, 1.0, 1.0, 1.0, 0.5),
    ("n5-V5", 73, 6, 5, 2, 5, 2.0, 1.0, 1.0, 1.0),
    ("n17-V5001-odd", 74, 3, 17, 4, 5001, 3.0, 1.0, 0.8, 1.5),
    ("n32-V32000", 75, 4, 32, 6, 32000, 3.0, 1.0, 1.0, 0.5),
    ("n64-V4096", 76, 2, 64, 8, 4096, 3.0, 0.5, 1.2, 0.0),
]


@pytest.mark.parametrize("case", TREE_CASES, ids=[c[0] for c in TREE_CASES])
def test_tree_random(case):
    name, seed, B, n, depth, V, zs, noise, T, eta = case
    parent = tree_parents(np.random.SeedSequence(seed), n, depth) if n > 1 else np.array([-1])
    vi = make_tree_vocab(seed, B, parent, V, zs, noise, T, eta)
    announce("rapid_tree_accept %s parent=%s" % (name, parent.tolist()))
    _check_tree(vi, name)


def _random_tree_cases(seed=4444, count=12):
    """Seeded random draft trees within the library's limits: 1-64 nodes,
    depth up to 12, V from 2 to 50257 (odd sizes take the scalar loads),
    B up to 4, three temperatures and three eta."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(count):
        n = int(rng.integers(1, 65))
        depth = int(rng.integers(1, min(n, 12) + 1)) if n > 1 else 0
        V = int(rng.choice([2, 3, 7, 1000, 4099, 32000, 50257]))
        B = int(rng.integers(1, 5))
        T = float(rng.choice([0.7, 1.0, 1.3]))
        eta = float(rng.choice([0.0, 0.5, 1.5]))
        cases.append((k, 5000 + k, B, n, depth, V, T, eta))
    return cases


RANDOM_TREES = _random_tree_cases()


@pytest.mark.parametrize("case", RANDOM_TREES, ids=["rt%d" % c[0] for c in RANDOM_TREES])
def test_tree_random_shapes(case):
    k, seed, B, n, depth, V, T, eta = case
    parent = tree_parents(np.random.SeedSequence(seed), n, depth) if n > 1 else np.array([-1])
    vi = make_tree_vocab(seed, B, parent, V, 3.0, 1.0, T, eta)
    announce("rapid_tree_accept random rt%d: n=%d depth=%d V=%d B=%d T=%g eta=%g"
             % (k, n, depth, V, B, T, eta))
    _check_tree(vi, "rt%d" % k)


def test_tree_star_forced_rejections():
    """A root with 12 children and uniforms near 1: children of ratio below 1
    are rejected in turn (11 residual passes); a sequence whose 12 children
    all are draws from the last residual.  Then uniforms of 0 accept the first
    child."""
    n = 13
    parent = np.array([-1] + [0] * 12, np.int32)
    vi = make_tree_vocab(77, 5, parent, 20000, 3.0, 1.0, 1.0, 0.5)
    vi.r[:] = np.float32(1.0 - 2 ** -24)
    announce("rapid_tree_accept star of 12, forced rejections")
    ref, _ = _check_tree(vi, "star reject")
    assert any(d["node"] == 0 and d["rejected"] == 12 for d in ref["draw"])
    vi.r[:] = 0.0
    ref, _ = _check_tree(vi, "star accept")
    assert np.all(ref["path"][:, 0] == 1)


def test_tree_star_of_63_children():
    """The widest tree: a root with 63 children (62 residual passes, 65
    launches), uniforms near 1 so that rejections pile up, at V = 4096."""
    n = 64
    parent = np.array([-1] + [0] * 63, np.int32)
    vi = make_tree_vocab(79, 3, parent, 4096, 3.0, 1.0, 1.0, 0.5)
    vi.r[:] = np.float32(1.0 - 2 ** -24)
    announce("rapid_tree_accept star of 63, forced rejections")
    _check_tree(vi, "star63 reject")
    vi.r[0, :] = 0.5
    _check_tree(vi, "star63 mixed")


def test_tree_workload_tree_full_vocab():
    """The 32-node tree of the 1M-token tree workload at V = 128256, eight
    sequences."""
    vi = config_tree_vocab("tree1m", B_override=8)
    announce("rapid_tree_accept tree1m tree, B=8, V=%d" % vi.z.shape[2])
    _check_tree(vi, "tree1m")


def test_tree_on_a_chain_equals_the_chain_pass():
    """On a chain the tree pass and rapid_accept take the same steps with the
    same chunking, so their outputs are bit-identical (8B vocabulary)."""
    vc = config_vocab("llama8b", eta=0.5, B_override=4)
    B, g1, V = vc.z.shape
    g = g1 - 1
    st = VerifyStep(None, vc, want_ratio=True)
    st.accept()
    torch.cuda.synchronize()
    from workloads import TreeVocabInputs
    vt = TreeVocabInputs(
        z=vc.z, y=np.concatenate([vc.y, np.zeros((B, 1, V), np.float32)], axis=1),
        parent=np.array([-1] + list(range(g)), np.int32),
        tokens=np.concatenate([np.zeros((B, 1), np.int32), vc.draft], axis=1),
        r=np.concatenate([np.full((B, 1), 0.5, np.float32), vc.r], axis=1), u=vc.u, T=vc.T,
        eta=vc.eta)
    announce("rapid_tree_accept on a chain vs rapid_accept, V=%d" % V)
    n_g, path_g, tok_g, ratio_g = _run_tree(vt)
    assert np.array_equal(n_g, st.n_accept.cpu().numpy())
    assert np.array_equal(tok_g[:, :g1], st.out_tokens.cpu().numpy())
    rc = st.ratio.cpu().numpy()
    for b in range(B):
        k = min(int(n_g[b]) + 1, g)
        assert np.array_equal(ratio_g[b, 1:k + 1].view(np.int32), rc[b, :k].view(np.int32))


def test_tree_bad_token_sentinel():
    parent = tree_parents(np.random.SeedSequence(78), 9, 3)
    vi = make_tree_vocab(78, 3, parent, 3000, 3.0, 1.0, 1.0, 0.5)
    vi.tokens[1, 4] = 3000
    vi.tokens[2, 8] = -2
    announce("rapid_tree_accept bad tokens")
    n_g, path_g, tok_g, ratio_g = _run_tree(vi)
    assert n_g[1] == -1 and n_g[2] == -1
    for b in (1, 2):
        assert np.all(path_g[b] == -1) and np.all(tok_g[b] == -1) and np.all(np.isnan(ratio_g[b]))
    ref = rapid_tree_accept_ref(vi.z[:1], vi.y[:1], vi.parent, vi.tokens[:1], vi.r[:1],
                                vi.u[:1], vi.T, vi.eta)
    res = compare_tree_accept(ref, vi.parent, vi.tokens[:1], n_g[:1], path_g[:1], tok_g[:1],
                              vi.r[:1])
    assert not res["errors"], res["errors"]


def test_tree_nan_with_every_bit_set_and_a_filled_workspace():
    """The empty-slot pattern of the draw weights (every bit set) as the
    leaves' target rows: with every first child accepted the walk ends at a
    leaf and draws its bonus token from those NaNs, which must still give an
    id in [0, V); the workspace starts filled with 0xFF bytes."""
    parent = np.array([-1, 0, 0, 1, 1, 2], np.int32)
    V = 3000
    vi = make_tree_vocab(71, 2, parent, V, 3.0, 1.0, 1.0, 0.5)
    vi.r[:] = 0.0
    vi.z.view(np.uint32)[:, 3:] = 0xFFFFFFFF   # the leaves 3, 4, 5
    B, n, _ = vi.z.shape
    dev = {k: to_device(getattr(vi, k)) for k in ("z", "y", "tokens", "r", "u")}
    n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    path = torch.empty((B, n), dtype=torch.int32, device="cuda")
    tok = torch.empty((B, n), dtype=torch.int32, device="cuda")
    ws = torch.full((rv.rapid_tree_accept_workspace_size(B, n, V),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    announce("rapid_tree_accept all-ones NaN leaves, 0xFF-filled workspace")
    rv.rapid_tree_accept(dev["z"], dev["y"], dev["tokens"], list(parent), dev["r"], dev["u"],
                         vi.T, vi.eta, n_acc, path, tok, ws)
    torch.cuda.synchronize()
    n_g, path_g, tok_g = n_acc.cpu().numpy(), path.cpu().numpy(), tok.cpu().numpy()
    for b in range(B):
        assert n_g[b] == 2 and list(path_g[b, :2]) == [1, 3], (n_g[b], path_g[b])
        assert np.all(path_g[b, 2:] == -1)
        assert list(tok_g[b, :2]) == [vi.tokens[b, 1], vi.tokens[b, 3]]
        assert 0 <= tok_g[b, 2] < V, tok_g[b]
        assert np.all(tok_g[b, 3:] == -1)
