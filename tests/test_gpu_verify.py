"""GPU parity of spec_attn_verify (history pass, draft block and log-sum-exp
merge in one launch; LongSpec summary, section 2.3) against the fp64 oracle
and against the separate calls, through the C ABI.

The single launch's merge sums each row's partials in one ascending chain,
so its bf16 output may differ from the separate calls' by one bf16 step; the
oracle bounds are those of every attention path (row error 2e-2, LSE 1e-4
for groups of at most 64 rows).  Helping (a workgroup computing a split on a
late one's behalf) writes the same bits, so it must not change the output at
all, and every call must leave the sync words zero."""

import sys

import numpy as np
import pytest
import torch

from oracle import attn_ref
from oracle.compare import ATTN_ROW_TOL, LSE_TOL_FP32, attn_row_errors
from workloads import config_attention, make_attention, tree_parents
from speculative_decoding_verify_split_amd import rapid_verify as rv
from speculative_decoding_verify_split_amd.step import VerifyStep

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def _outputs(st):
    torch.cuda.synchronize()
    return st.out.float().cpu().numpy(), st.lse_out.cpu().numpy()


def _bits(a):
    return a.view(np.uint32)


def _check_oracle(ai, out, lse, tag):
    O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens,
                            ai.parent, ai.sm_scale)
    err = attn_row_errors(out, O_ref).max()
    dl = np.abs(lse - L_ref).max()
    announce("  %s: max row rel err %.3e, max |dLSE| %.3e" % (tag, err, dl))
    assert err <= ATTN_ROW_TOL
    assert dl <= LSE_TOL_FP32


VERIFY_CASES = [
    # name, seed, B, Hq, Hkv, d, n, lengths, parent, split
    ("b3-ragged-empty", 51, 3, 4, 2, 128, 11, [3000, 0, 1500], None, (512, 6)),
    ("tree16-64rows-d64", 52, 1, 8, 2, 64, 16, [2000], "tree", (128, 16)),
    ("star16-d64-64groups", 53, 2, 8, 2, 64, 16, [700, 1200], "star", (128, 16)),
    ("n1-drafter-like", 54, 1, 32, 8, 128, 1, [5000], None, (640, 8)),
    ("s64-one-kv-head", 55, 1, 4, 1, 128, 11, [8192], None, (128, 64)),
    ("s1", 56, 2, 4, 2, 128, 2, [100, 128], None, (128, 1)),
    ("4-rows-per-group", 57, 1, 16, 4, 128, 4, [1024], None, (256, 4)),
    ("all-empty-history", 58, 2, 4, 2, 64, 2, [0, 0], None, (128, 1)),
]


def _case(c):
    name, seed, B, Hq, Hkv, d, n, lens, parent, split = c
    if parent == "tree":
        parent = tree_parents(np.random.SeedSequence(seed), n, 5)
    elif parent == "star":
        parent = np.array([-1] + [0] * (n - 1), np.int32)
    L_max = max(max(lens), 128)  # (an empty cache still has a buffer)
    return make_attention(seed, B, Hq, Hkv, d, n, lens, L_max=L_max, parent=parent,
                          pad_bits=0x7FC0), split


@pytest.mark.parametrize("case", VERIFY_CASES, ids=[c[0] for c in VERIFY_CASES])
def test_verify_single_launch(case):
    ai, split = _case(case)
    B, Hq, n, d = ai.q.shape
    Hkv = ai.k_cache.shape[1]
    assert rv.rv_verify_single_launch(B, Hq, Hkv, n, d, split[1]), "case takes two launches"
    announce("spec_attn_verify %s shape=%s lens=%s split=%s" % (case[0], ai.shape,
                                                                list(ai.seq_lens), split))
    st = VerifyStep(ai, None, split=split)
    st.attention(fused=True)
    out_f, lse_f = _outputs(st)
    res = {}
    for help_us in (-1, 0, 3):
        st.out.zero_()
        st.lse_out.zero_()
        st.attention(single=True, help_after_us=help_us)
        res[help_us] = _outputs(st)
        assert not st.sync.any()
    out, lse = res[-1]
    _check_oracle(ai, out, lse, "one launch")
    for h in (0, 3):
        assert np.array_equal(_bits(res[h][0]), _bits(out)), h
        assert np.array_equal(_bits(res[h][1]), _bits(lse)), h
    assert attn_row_errors(out, out_f).max() <= 1e-2  # one bf16 step
    assert np.abs(lse - lse_f).max() <= 1e-5


def test_verify_repeated_calls_share_the_sync_words():
    """Calls of different shapes on one stream share one zeroed sync buffer
    (sized for the largest); each call's output equals its own first run."""
    cases = [_case(c) for c in VERIFY_CASES[:3]]
    big = max(rv.spec_attn_verify_sync_size(ai.q.shape[0], ai.k_cache.shape[1])
              for ai, _ in cases)
    sync = torch.zeros((big,), dtype=torch.uint8, device="cuda")
    steps = []
    for ai, split in cases:
        st = VerifyStep(ai, None, split=split)
        st.sync = sync
        steps.append(st)
    first = []
    for st in steps:
        st.attention(single=True)
        first.append(_outputs(st))
    announce("spec_attn_verify: 3 shapes x 4 rounds on one sync buffer")
    for rnd in range(4):
        for st, (o0, l0) in zip(steps, first):
            st.out.zero_()
            st.attention(single=True, help_after_us=0 if rnd == 2 else -1)
            o, l = _outputs(st)
            assert np.array_equal(_bits(o), _bits(o0)) and np.array_equal(_bits(l), _bits(l0))
            assert not sync.any()


def test_verify_without_lse_out():
    ai, split = _case(VERIFY_CASES[0])
    st = VerifyStep(ai, None, split=split)
    st.attention(single=True)
    out_ref, _ = _outputs(st)
    st.out.zero_()
    rv.spec_attn_verify(st.q, st.k_cache, st.v_cache, st.seq_lens, st.max_seq_len, st.split_len,
                        st.num_splits, st.k_blk, st.v_blk, st.parent, st.o_part, st.lse_part,
                        st.sync, st.out, None, st.sm_scale)
    out, _ = _outputs(st)
    assert np.array_equal(_bits(out), _bits(out_ref))


def test_verify_tiny_workload_help_path():
    """The tiny workload (8/2 heads, d = 64, 4096 tokens: 16 workgroups, one
    launch) with every waiting workgroup helping at once: the same bits as
    the default wait, and every row within the oracle bounds."""
    ai = config_attention("tiny")
    B, Hq, n, d = ai.q.shape
    st = VerifyStep(ai, None)
    assert rv.rv_verify_single_launch(B, Hq, st.Hkv, n, d, st.num_splits)
    announce("spec_attn_verify tiny split=%d x %d, help 0 vs default"
             % (st.split_len, st.num_splits))
    st.attention(single=True)
    out, lse = _outputs(st)
    for _ in range(3):
        st.out.zero_()
        st.attention(single=True, help_after_us=0)
        out0, lse0 = _outputs(st)
        assert not st.sync.any()
        assert np.array_equal(_bits(out0), _bits(out)) and np.array_equal(_bits(lse0), _bits(lse))
    _check_oracle(ai, out, lse, "tiny, one launch")


def test_verify_8b_shape_takes_two_launches():
    """At the 8B shape (256 workgroups) spec_attn_verify runs the history
    pass and the fused block + merge as two launches: the same bits as those
    two calls."""
    ai = config_attention("llama8b")
    B, Hq, n, d = ai.q.shape
    st = VerifyStep(ai, None)
    assert not rv.rv_verify_single_launch(B, Hq, st.Hkv, n, d, st.num_splits)
    announce("spec_attn_verify llama8b: two launches")
    st.attention(fused=True)
    out_f, lse_f = _outputs(st)
    st.out.zero_()
    st.lse_out.zero_()
    st.attention(single=True)
    out, lse = _outputs(st)
    assert np.array_equal(_bits(out), _bits(out_f)) and np.array_equal(_bits(lse), _bits(lse_f))
    assert not st.sync.any()


@pytest.mark.parametrize("L", [4096, 40960], ids=["one-launch", "two-launches"])
def test_verify_events_bracket_the_attention(L):
    """spec_attn_verify's start and stop events ride on its own dispatches:
    positive elapsed time, and the output equals the call without events."""
    import ctypes
    ai = make_attention(63, 1, 8, 2, 64, 5, [L])
    st = VerifyStep(ai, None)
    announce("spec_attn_verify events, %d tokens, split %d x %d"
             % (L, st.split_len, st.num_splits))
    st.attention(single=True)
    ref = _outputs(st)
    hip = ctypes.CDLL("libamdhip64.so")
    evs = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in evs:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        st.out.zero_()
        st.attention(single=True, events=(evs[0], evs[1]))
        got = _outputs(st)
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
        announce("  %.2f us" % (ms.value * 1e3))
        assert ms.value > 0
    finally:
        for e in evs:
            hip.hipEventDestroy(e)
    assert np.array_equal(_bits(got[0]), _bits(ref[0]))
    assert np.array_equal(_bits(got[1]), _bits(ref[1]))
    assert not st.sync.any()


def _random_single_launch_cases(seed=90, count=16):
    """Seeded random shapes that take the single launch: d in {64, 128},
    up to 64 rows per kv head (48 at d = 128), at most 64 workgroups, at most
    4 rows per workgroup; ragged and empty lengths; chain, tree or star."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 5))
        G = int(rng.integers(1, 9))
        n = int(rng.integers(1, 33))
        M = G * n
        if M > (48 if d == 128 else 64):
            continue
        B = int(rng.integers(1, 4))
        S = int(rng.integers(-(-M // 4), 17))  # at least ceil(M / 4) splits
        if B * Hkv * S > 64 or S > 64:
            continue
        split_len = 128 * int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, S * split_len + 1, size=B)]
        parent = str(rng.choice(["chain", "tree", "star"])) if n > 1 else "chain"
        cases.append((len(cases), B, G * Hkv, Hkv, d, n, lens, parent, (split_len, S)))
    return cases


RANDOM_SINGLE = _random_single_launch_cases()


@pytest.mark.parametrize("case", RANDOM_SINGLE, ids=["r%d" % c[0] for c in RANDOM_SINGLE])
def test_verify_single_launch_random_shapes(case):
    idx, B, Hq, Hkv, d, n, lens, kind, split = case
    parent = None
    if kind == "tree":
        parent = tree_parents(np.random.SeedSequence(1000 + idx), n, min(5, n - 1))
    elif kind == "star":
        parent = np.array([-1] + [0] * (n - 1), np.int32)
    L_max = max(max(lens), 1)
    ai = make_attention(1000 + idx, B, Hq, Hkv, d, n, lens, L_max=L_max, parent=parent,
                        pad_bits=0x7FC0)
    assert rv.rv_verify_single_launch(B, Hq, Hkv, n, d, split[1])
    announce("spec_attn_verify random r%d: B=%d Hq=%d Hkv=%d d=%d n=%d %s lens=%s split=%s"
             % (idx, B, Hq, Hkv, d, n, kind, lens, split))
    st = VerifyStep(ai, None, split=split)
    st.attention(single=True)
    out, lse = _outputs(st)
    _check_oracle(ai, out, lse, "r%d" % idx)
    st.out.zero_()
    st.attention(single=True, help_after_us=0)
    out0, lse0 = _outputs(st)
    assert np.array_equal(_bits(out0), _bits(out)) and np.array_equal(_bits(lse0), _bits(lse))
    assert not st.sync.any()
