"""GPU parity of the LongSpec drafter's attention (through the C ABI):

* spec_attn_window, the sliding-window self-attention with sink anchors over
  the drafter's ring cache, against ``oracle.window_attn_ref`` on every
  output element, including wrapped rings and never-written slots holding
  NaN (which must never be read);
* the drafter's cross-attention over the target's cache, i.e.
  spec_attn_prefix at n = 1 and a history-only lse_merge, against the
  plain attention definition;
* both at the full 8B-shaped drafter workload (128K-token target cache).
"""

import sys

import numpy as np
import pytest
import torch

from oracle import attn_keys_ref, bf16_bits_to_f64, window_attn_ref
from oracle.compare import ATTN_ROW_TOL, attn_row_errors
from workloads import config_drafter, make_attention, make_window
from speculative_decoding_verify_split_amd.step import VerifyStep, WindowStep

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


WINDOW_CASES = [
    # name, seed, B, Hq, Hkv, d, n, pos, cap, sink, window
    ("drafter-shape-wrapped", 61, 1, 8, 2, 128, 1, [131072], 516, 4, 512),
    ("early-positions-nan-pad", 62, 3, 4, 2, 128, 1, [0, 3, 200], 516, 4, 512),
    ("block-n5-wrap", 63, 2, 8, 2, 128, 5, [1000, 517], 520, 4, 512),
    ("no-sink-d64", 64, 2, 4, 1, 64, 3, [77, 5000], 66, 0, 64),
    ("small-window-many-rows", 65, 1, 16, 4, 128, 16, [300], 40, 2, 23),
    ("window-1", 66, 1, 4, 2, 64, 2, [9], 6, 4, 1),
    ("keys-not-multiple-of-64", 67, 2, 4, 2, 128, 1, [130, 70], 134, 4, 130),
    # query heads per kv head other than 4: the waves loop over the G rows
    ("g7-two-rows-per-wave", 70, 1, 28, 4, 128, 1, [100000], 516, 4, 512),
    ("g1-mha-d64", 71, 2, 4, 4, 64, 2, [600, 50], 517, 4, 512),
    ("g8-block-n3", 72, 1, 16, 2, 128, 3, [9999], 518, 4, 512),
]


def _random_window_cases(seed=79, count=16):
    """Window shapes drawn at random: windows of 1 to 700 keys, 0 to 8
    anchors, rings from the tightest capacity to 40 slots more, query
    positions before and after the ring wraps."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(count):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4, 7, 8]))
        n = int(rng.integers(1, 17))
        sink = int(rng.choice([0, 1, 4, 8]))
        window = int(rng.integers(1, 701))
        cap = sink + window + n - 1 + int(rng.integers(0, 41))
        B = int(rng.integers(1, 4))
        pos = [int(rng.integers(0, 3 * cap)) for _ in range(B)]
        cases.append(("r%02d-d%d-g%d-n%d-s%d-w%d-c%d" % (k, d, G, n, sink, window, cap),
                      seed * 1000 + k, B, G * Hkv, Hkv, d, n, pos, cap, sink, window))
    return cases


@pytest.mark.parametrize("case", WINDOW_CASES + _random_window_cases(),
                         ids=[c[0] for c in WINDOW_CASES + _random_window_cases()])
def test_window_small(case):
    name, seed, B, Hq, Hkv, d, n, pos, cap, sink, window = case
    wi = make_window(seed, B, Hq, Hkv, d, n, pos=pos, cap=cap, sink=sink, window=window)
    announce("spec_attn_window %s B=%d Hq=%d Hkv=%d d=%d n=%d pos=%s cap=%d sink=%d window=%d"
             % (name, B, Hq, Hkv, d, n, list(wi.pos), cap, sink, window))
    st = WindowStep(wi)
    st.run()
    torch.cuda.synchronize()
    out = st.out.float().cpu().numpy()
    lse = st.lse_out.cpu().numpy()
    O_ref, L_ref = window_attn_ref(wi.q, wi.k_ring, wi.v_ring, wi.pos, cap, sink, window,
                                   wi.sm_scale)
    err = attn_row_errors(out, O_ref)
    dl = np.abs(lse - L_ref).max()
    announce("  max row rel err %.3e, max |dLSE| %.3e" % (err.max(), dl))
    assert np.isfinite(out).all()
    assert err.max() <= ATTN_ROW_TOL
    assert dl <= 1e-3


def test_window_sm_scale_and_determinism():
    wi = make_window(68, 1, 8, 2, 128, 2, pos=[700], cap=517, sink=4, window=512)
    wi.sm_scale = 0.61
    announce("spec_attn_window sm_scale 0.61, repeated")
    st = WindowStep(wi)
    outs = []
    for _ in range(2):
        st.run()
        torch.cuda.synchronize()
        outs.append((st.out.view(torch.int16).cpu().clone(), st.lse_out.cpu().clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    O_ref, L_ref = window_attn_ref(wi.q, wi.k_ring, wi.v_ring, wi.pos, 517, 4, 512, 0.61)
    assert attn_row_errors(st.out.float().cpu().numpy(), O_ref).max() <= ATTN_ROW_TOL
    assert np.abs(st.lse_out.cpu().numpy() - L_ref).max() <= 1e-3


def test_cross_attention_n1_small():
    """spec_attn_prefix at n = 1 and the history-only merge, ragged lengths
    (one empty history: that row sees no key, out = 0, lse = -inf)."""
    ai = make_attention(69, 3, 8, 2, 128, 1, [5000, 0, 777], pad_bits=0x7FC0)
    announce("cross-attention n=1 small")
    st = VerifyStep(ai, None, split=(1024, 5))
    st.attention(block=False)
    torch.cuda.synchronize()
    out = st.out.float().cpu().numpy()
    lse = st.lse_out.cpu().numpy()
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    for b in (0, 2):
        L = int(ai.seq_lens[b])
        for h in range(8):
            o, l = attn_keys_ref(bf16_bits_to_f64(ai.q[b, h]), bf16_bits_to_f64(ai.k_cache[b, h // 4, :L]),
                                 bf16_bits_to_f64(ai.v_cache[b, h // 4, :L]), np.ones((1, L), bool), 1.0)
            assert attn_row_errors(out[b, h], o).max() <= ATTN_ROW_TOL
            assert np.abs(lse[b, h] - l).max() <= 1e-2


@pytest.mark.timeout(600)
def test_drafter8b_workload():
    announce("generating drafter8b inputs")
    cross, win = config_drafter("drafter8b")
    announce("drafter8b cross-attention (n=1 over 131072 tokens) + window")
    st = VerifyStep(cross, None)  # default split: the benchmark's launch configuration
    st.attention(block=False)
    ws = WindowStep(win)
    ws.run()
    torch.cuda.synchronize()
    out = st.out.float().cpu().numpy()
    lse = st.lse_out.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    L = int(cross.seq_lens[0])
    for h in (0, 13, 31):
        o, l = attn_keys_ref(bf16_bits_to_f64(cross.q[0, h]),
                             bf16_bits_to_f64(cross.k_cache[0, h // 4, :L]),
                             bf16_bits_to_f64(cross.v_cache[0, h // 4, :L]), np.ones((1, L), bool),
                             1.0)
        err = attn_row_errors(out[0, h], o).max()
        announce("  cross h=%d row rel err %.3e |dLSE| %.3e" % (h, err, abs(lse[0, h, 0] - l[0])))
        assert err <= ATTN_ROW_TOL
        assert np.abs(lse[0, h] - l).max() <= 1e-2
    O_ref, L_ref = window_attn_ref(win.q, win.k_ring, win.v_ring, win.pos, win.cap, win.sink,
                                   win.window)
    wout = ws.out.float().cpu().numpy()
    err = attn_row_errors(wout, O_ref).max()
    announce("  window all heads row rel err %.3e" % err)
    assert err <= ATTN_ROW_TOL
    assert np.abs(ws.lse_out.cpu().numpy() - L_ref).max() <= 1e-3
