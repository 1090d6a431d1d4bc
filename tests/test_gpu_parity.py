"""GPU parity: librapid_verify.so (through its C ABI) against the fp64 oracle.

Small cases compare every output element; the five workloads at full size run
in the launch configuration the benchmark times and are compared on every
query head (attention) and in full (vocabulary pass), plus properties that
hold at any size; many-sequence sweeps at the workloads' vocabulary sizes
compare hundreds of draws.  Tolerances and boundary flagging follow
oracle/compare.py.
"""

import itertools
import sys

import numpy as np
import pytest
import torch

from oracle import (attn_keys_ref, attn_ref, bf16_bits_to_f64, block_visibility, lse_merge_ref,
                    rapid_accept_ref, retrieval_augmented_target)
from oracle.compare import (ATTN_ROW_TOL, BLOCK_FP32_TOL, BOUNDARY_TOL, LSE_TOL_BF16_SUMS,
                            LSE_TOL_FP32, P_HAT_TOL, attn_row_errors, compare_accept,
                            flag_counts)
from workloads import (CONFIGS, config_attention, config_vocab, make_attention, make_vocab,
                       tree_parents)
from speculative_decoding_verify_split_amd.rapid_verify import (RV_ACCEPT_PRINTED_RESIDUAL,
                                                                RV_ACCEPT_TAIL_PRESERVE)
from speculative_decoding_verify_split_amd import rapid_verify as rv
from speculative_decoding_verify_split_amd.step import VerifyStep

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def _tree(seed, n, depth):
    return tree_parents(np.random.SeedSequence(seed), n, depth)


def _lse_tol(Hq, Hkv, n):
    """Bound on |dLSE| of a history pass: groups of more than 64 rows per kv
    head go to the shared-stage kernel, whose row sums add the bf16-rounded
    probabilities on the matrix cores; narrower groups sum them in fp32."""
    return LSE_TOL_BF16_SUMS if (Hq // Hkv) * n > 64 else LSE_TOL_FP32


def _attn_outputs(st):
    torch.cuda.synchronize()
    return st.out.float().cpu().numpy(), st.lse_out.cpu().numpy()


# ------------------------------------------------------- attention, small

ATTN_CASES = [
    # name, seed, B, Hq, Hkv, d, n, lengths, L_max, parent, split
    ("d128-g4-n11-ragged", 21, 2, 8, 2, 128, 11, [3000, 1777], 3072, None, (512, 6)),
    ("d128-g8-n11-wide", 22, 1, 16, 2, 128, 11, [2500], None, None, None),
    ("d128-g7-n11-b3-empty", 23, 3, 28, 4, 128, 11, [1500, 0, 2049], None, None, (256, 9)),
    ("d128-g4-tree32", 24, 1, 8, 2, 128, 32, [2000], None, "tree", None),
    ("d128-g8-tree32-256rows", 25, 1, 16, 2, 128, 32, [700], None, "tree", (128, 6)),
    ("d64-g1-n1", 26, 2, 4, 4, 64, 1, [33, 31], None, None, (128, 1)),
    ("d64-g2-n16", 27, 1, 4, 2, 64, 16, [4097], None, None, None),
    ("d64-g4-n16-star", 28, 1, 8, 2, 64, 16, [1000], None, "star", None),
    ("d128-n64-chain", 29, 1, 2, 2, 128, 64, [300], None, None, None),
    ("empty-history", 30, 2, 4, 2, 128, 5, [0, 0], 128, None, (128, 1)),
    ("short-lengths", 31, 5, 4, 2, 128, 3, [1, 31, 32, 33, 129], None, None, (128, 2)),
    ("d64-g3-n5-many-splits", 32, 1, 6, 2, 64, 5, [5000], None, None, (128, 40)),
    # more than 64 rows per kv head: the shared-stage kernel, 2, 3 and 4 row
    # tiles per wave, stages cut by the split end and by the history end
    ("d64-g8-n16-wide", 33, 2, 16, 2, 64, 16, [3000, 130], None, None, (256, 12)),
    ("d64-g12-tree16-wide3", 34, 1, 12, 1, 64, 16, [999], None, "tree", None),
    ("d128-g5-tree32-wide3", 35, 1, 10, 2, 128, 32, [1234], None, "tree", (256, 5)),
    ("d64-g16-n16-wide4", 36, 1, 16, 1, 64, 16, [777], None, "star", (384, 3)),
    ("wide-short-lengths", 37, 5, 16, 2, 128, 11, [1, 127, 128, 129, 0], None, None, (128, 2)),
    # 300 partials per row: the merges fold them in three batches per wave
    ("d128-g2-n3-300-splits", 38, 1, 4, 2, 128, 3, [38300], None, None, (128, 300)),
]


def _make_case(c):
    name, seed, B, Hq, Hkv, d, n, lens, L_max, parent, split = c
    if parent == "tree":
        parent = _tree(seed, n, 6)
    elif parent == "star":
        parent = np.array([-1] + [0] * (n - 1), np.int32)
    ai = make_attention(seed, B, Hq, Hkv, d, n, lens, L_max=L_max, parent=parent,
                        pad_bits=0x7FC0)  # NaN past each history: must never be read
    return ai, split


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_small(case):
    ai, split = _make_case(case)
    announce("attention %s shape=%s lens=%s split=%s" % (case[0], ai.shape, list(ai.seq_lens), split))
    st = VerifyStep(ai, None, split=split)
    O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens,
                            ai.parent, ai.sm_scale)
    B, Hq, n, d = ai.q.shape
    single = rv.rv_verify_single_launch(B, Hq, ai.k_cache.shape[1], n, d, st.num_splits)
    res = {}
    # block+merge, block_merge, then spec_attn_verify with the default wait
    # and with help_after_us = 0 (every waiting workgroup computes missing
    # splits itself at once: the help path)
    for mode in ("split", "fused", "verify", "verify-help0"):
        st.out.zero_()
        st.lse_out.zero_()
        if mode.startswith("verify"):
            st.attention(single=True, help_after_us=0 if mode == "verify-help0" else -1)
        else:
            st.attention(fused=mode == "fused")
        out, lse = _attn_outputs(st)
        err = attn_row_errors(out, O_ref)
        dl = np.abs(lse - L_ref).max()
        announce("  %s%s: max row rel err %.3e, max |dLSE| %.3e"
                 % (mode, " (one launch)" if mode.startswith("verify") and single else "",
                    err.max(), dl))
        assert err.max() <= ATTN_ROW_TOL
        assert dl <= _lse_tol(ai.q.shape[1], ai.k_cache.shape[1], ai.q.shape[2])
        res[mode] = (out, lse)
    assert not st.sync.any()  # spec_attn_verify leaves its sync words zero
    # the fused calls differ from the two calls only in fp32 rounding order,
    # so their bf16 outputs differ by at most one bf16 step (2^-7 of an
    # entry's binade): 7.8e-3 of the row's largest entry
    for mode in ("fused", "verify"):
        assert attn_row_errors(res[mode][0], res["split"][0]).max() <= 1e-2
        assert np.abs(res[mode][1] - res["split"][1]).max() <= 1e-4
    # a split computed on another's behalf has the same bits, so the help
    # path changes nothing; without the single launch the call is the fused
    # call's two launches
    same = (("verify", "verify-help0"),) + ((("verify", "fused"),) if not single else ())
    for a, b in same:
        assert np.array_equal(res[a][0].view(np.uint32), res[b][0].view(np.uint32)), (a, b)
        assert np.array_equal(res[a][1].view(np.uint32), res[b][1].view(np.uint32)), (a, b)


# Batches of more than 64 sequences take the multi-chunk path of the history
# kernels' workgroup-to-slot numbering; lengths include empty sequences.
_B70_LENS = [int(x) for x in np.random.default_rng(41).integers(0, 700, 70)]
_B70_LENS[5] = _B70_LENS[67] = 0
PARTIAL_CASES = [
    ATTN_CASES[0],
    ("b70-narrow-d64", 42, 70, 4, 2, 64, 3, _B70_LENS, None, None, (128, 6)),
    ("b70-wide-d64", 43, 70, 16, 2, 64, 11, _B70_LENS, None, None, (256, 3)),
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=[c[0] for c in PARTIAL_CASES])
def test_prefix_and_block_partials_match_split_oracle(case):
    """The history splits and the masked block part separately, against the
    oracle evaluated on exactly those key sets."""
    ai, split = _make_case(case)
    announce("partials %s B=%d" % (case[0], ai.q.shape[0]))
    st = VerifyStep(ai, None, split=split)
    st.attention()
    torch.cuda.synchronize()
    o_part = st.o_part.cpu().numpy()
    lse_part = st.lse_part.cpu().numpy()
    o_blk = st.o_blk.cpu().numpy()
    lse_blk = st.lse_blk.cpu().numpy()
    B, Hq, n, d = ai.q.shape
    Hkv = ai.k_cache.shape[1]
    G = Hq // Hkv
    split_len, S = split
    vis = block_visibility(n, ai.parent)
    for b in range(B):
        L = int(ai.seq_lens[b])
        for h in range(Hq):
            g = h // G
            q = bf16_bits_to_f64(ai.q[b, h])
            for s in range(S):
                lo, hi = s * split_len, min((s + 1) * split_len, L)
                if hi <= lo:
                    assert np.all(np.isneginf(lse_part[b, h, :, s]))
                    assert np.all(o_part[b, h, :, s] == 0)
                    continue
                o, l = attn_keys_ref(q, bf16_bits_to_f64(ai.k_cache[b, g, lo:hi]),
                                     bf16_bits_to_f64(ai.v_cache[b, g, lo:hi]),
                                     np.ones((n, hi - lo), bool), 1.0)
                assert attn_row_errors(o_part[b, h, :, s], o).max() <= ATTN_ROW_TOL
                assert np.abs(lse_part[b, h, :, s] - l).max() <= _lse_tol(Hq, Hkv, n)
            o, l = attn_keys_ref(q, bf16_bits_to_f64(ai.k_blk[b, g]), bf16_bits_to_f64(ai.v_blk[b, g]),
                                 vis, 1.0)
            # the block part is fp32 on the vector ALU (bf16 inputs widened
            # exactly), so it is held to an fp32 bound
            assert np.abs(o_blk[b, h] - o).max() <= BLOCK_FP32_TOL
            assert np.abs(lse_blk[b, h] - l).max() <= BLOCK_FP32_TOL


# ------------------------------------------------ seeded random shapes

def _random_attention_cases(seed=77, count=24):
    """Shapes drawn at random within the library's limits: both kernels
    (up to and above 64 rows per kv head), both head dims, ragged and empty
    histories, split lengths from 128 to 1408 keys, spare splits past every
    history, causal chains and random trees."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(count):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16]))
        n = int(rng.integers(1, min(64, 256 // G) + 1))
        B = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, 2600, B)]
        if rng.random() < 0.3:
            lens[int(rng.integers(0, B))] = 0
        L_max = max(max(lens), 1) + int(rng.integers(0, 200))
        parent = None
        if n > 2 and rng.random() < 0.4:
            parent = tree_parents(np.random.SeedSequence(seed * 1000 + k), n,
                                  int(rng.integers(1, min(6, n - 1) + 1)))
        split_len = 128 * int(rng.integers(1, 12))
        S = max(1, -(-max(lens) // split_len)) + int(rng.integers(0, 3))
        name = "r%02d-d%d-b%d-g%d-n%d%s" % (k, d, B, G, n, "-tree" if parent is not None else "")
        cases.append((name, seed * 1000 + k, B, G * Hkv, Hkv, d, n, lens, L_max, parent,
                      (split_len, S)))
    return cases


RANDOM_ATTN_CASES = _random_attention_cases()


@pytest.mark.parametrize("case", RANDOM_ATTN_CASES, ids=[c[0] for c in RANDOM_ATTN_CASES])
def test_attention_random_shapes(case):
    name, seed, B, Hq, Hkv, d, n, lens, L_max, parent, split = case
    ai = make_attention(seed, B, Hq, Hkv, d, n, lens, L_max=L_max, parent=parent,
                        pad_bits=0x7FC0)
    announce("random attention %s lens=%s split=%s" % (name, lens, split))
    st = VerifyStep(ai, None, split=split)
    O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens,
                            ai.parent, ai.sm_scale)
    for fused in (False, True):
        st.attention(fused=fused)
        out, lse = _attn_outputs(st)
        err = attn_row_errors(out, O_ref).max()
        dl = np.abs(lse - L_ref).max()
        announce("  %s: max row rel err %.3e, max |dLSE| %.3e"
                 % ("block_merge" if fused else "block+merge", err, dl))
        assert err <= ATTN_ROW_TOL and dl <= _lse_tol(Hq, Hkv, n)


def _random_vocab_cases(seed=78, count=16):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(count):
        kw = dict(seed=seed * 1000 + k, B=int(rng.integers(1, 7)), gamma=int(rng.integers(1, 13)),
                  V=int(rng.choice([2, 3, 5]) if rng.random() < 0.15 else rng.integers(6, 60000)),
                  z_sigma=float(rng.uniform(0.5, 4.0)), noise=float(rng.uniform(0.2, 2.0)),
                  T=float(rng.uniform(0.5, 1.5)), eta=float(rng.choice([0.0, rng.uniform(0.1, 2.5)])))
        cases.append(("r%02d-b%d-g%d-V%d" % (k, kw["B"], kw["gamma"], kw["V"]), kw))
    return cases


RANDOM_VOCAB_CASES = _random_vocab_cases()


@pytest.mark.parametrize("case", RANDOM_VOCAB_CASES, ids=[c[0] for c in RANDOM_VOCAB_CASES])
def test_accept_random_shapes(case):
    name, kw = case
    vi = make_vocab(**kw)
    announce("random rapid_accept %s T=%.2f eta=%.2f" % (name, kw["T"], kw["eta"]))
    _check_accept(vi, _run_accept(vi), name)


@pytest.mark.parametrize("flags", [RV_ACCEPT_TAIL_PRESERVE, RV_ACCEPT_PRINTED_RESIDUAL,
                                   RV_ACCEPT_TAIL_PRESERVE | RV_ACCEPT_PRINTED_RESIDUAL])
@pytest.mark.parametrize("case", RANDOM_VOCAB_CASES[:8], ids=[c[0] for c in RANDOM_VOCAB_CASES[:8]])
def test_accept_rules_random_shapes(case, flags):
    name, kw = case
    vi = make_vocab(**kw)
    announce("random rapid_accept_ex %s flags=%d" % (name, flags))
    _check_accept(vi, _run_accept(vi, flags=flags), "%s flags=%d" % (name, flags), flags)


# Split counts around the merges' fold batches (8, 16 or 32 partials per
# wave, 4 waves) and several batches per wave.
MERGE_S = [1, 7, 32, 33, 64, 65, 128, 129, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", MERGE_S)
def test_merges_fold_any_number_of_partials(S, d):
    """lse_merge (with and without a block partial) and spec_attn_block_merge
    on random fp32 partials, a quarter of the splits empty and one row with
    every split empty, against the oracle's log-sum-exp merge."""
    from speculative_decoding_verify_split_amd import rapid_verify as rv
    from speculative_decoding_verify_split_amd.step import bf16_to_device
    announce("merge fold S=%d d=%d" % (S, d))
    rng = np.random.default_rng(5000 + 7 * S + d)
    B, Hq, Hkv, n = 2, 4, 2, 5
    o = rng.standard_normal((B, Hq, n, S, d)).astype(np.float32)
    lse = (3.0 * rng.standard_normal((B, Hq, n, S))).astype(np.float32)
    empty = rng.random((B, Hq, n, S)) < 0.25
    empty[0, 0, 0, :] = True
    lse[empty] = -np.inf
    o[empty] = 0.0
    o_blk = rng.standard_normal((B, Hq, n, d)).astype(np.float32)
    lse_blk = (3.0 * rng.standard_normal((B, Hq, n))).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o_t, lse_t, ob_t, lb_t = dev(o), dev(lse), dev(o_blk), dev(lse_blk)
    out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    hist = [(o[:, :, :, s].astype(np.float64), lse[:, :, :, s].astype(np.float64))
            for s in range(S)]

    def check(O_ref, L_ref, what):
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        got_l = lse_out.cpu().numpy()
        err = attn_row_errors(got, O_ref).max()
        both_inf = np.isneginf(got_l) & np.isneginf(L_ref)
        with np.errstate(invalid="ignore"):  # -inf - -inf where both rows are empty
            diff = np.abs(got_l - L_ref)
        dl = np.where(both_inf, 0.0, diff).max()
        announce("  %s: max row rel err %.3e, max |dLSE| %.3e" % (what, err, dl))
        assert err <= 1e-2 and dl <= 1e-4

    rv.lse_merge(o_t, lse_t, ob_t, lb_t, out, lse_out)
    check(*lse_merge_ref(hist + [(o_blk.astype(np.float64), lse_blk.astype(np.float64))]),
          "lse_merge")
    rv.lse_merge(o_t, lse_t, None, None, out, lse_out)
    O_ref, L_ref = lse_merge_ref(hist)
    assert np.isneginf(L_ref[0, 0, 0]) and np.all(O_ref[0, 0, 0] == 0)
    check(O_ref, L_ref, "lse_merge, history only")

    # the fused call computes the causal block part itself
    ai = make_attention(6000 + S + d, B, Hq, Hkv, d, n, [0] * B, L_max=128)
    rv.spec_attn_block_merge(bf16_to_device(ai.q), bf16_to_device(ai.k_blk),
                             bf16_to_device(ai.v_blk), None, o_t, lse_t, out, lse_out, 1.0)
    vis = block_visibility(n, None)
    O_b = np.zeros((B, Hq, n, d))
    L_b = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            O_b[b, h], L_b[b, h] = attn_keys_ref(bf16_bits_to_f64(ai.q[b, h]),
                                                 bf16_bits_to_f64(ai.k_blk[b, g]),
                                                 bf16_bits_to_f64(ai.v_blk[b, g]), vis, 1.0)
    check(*lse_merge_ref(hist + [(O_b, L_b)]), "spec_attn_block_merge")


def test_prefix_ev_matches_prefix_and_records_the_kernel():
    """spec_attn_prefix_ev writes the same partials as spec_attn_prefix and
    its events bracket the kernel (positive elapsed time)."""
    import ctypes
    from speculative_decoding_verify_split_amd import rapid_verify as rv
    ai, split = _make_case(ATTN_CASES[0])
    announce("spec_attn_prefix_ev")
    st = VerifyStep(ai, None, split=split)
    st.attention()
    torch.cuda.synchronize()
    ref = (st.o_part.clone(), st.lse_part.clone())
    st.o_part.zero_()
    st.lse_part.zero_()
    hip = ctypes.CDLL("libamdhip64.so")
    evs = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in evs:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        rv.spec_attn_prefix_ev(st.q, st.k_cache, st.v_cache, st.seq_lens, st.max_seq_len,
                               st.split_len, st.num_splits, st.o_part, st.lse_part, evs[0],
                               evs[1], st.sm_scale)
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
        announce("  kernel %.2f us" % (ms.value * 1e3))
        assert ms.value > 0
    finally:
        for e in evs:
            hip.hipEventDestroy(e)
    assert torch.equal(st.o_part, ref[0]) and torch.equal(st.lse_part, ref[1])


def test_block_merge_ev_matches_block_merge_and_records_the_kernel():
    """spec_attn_block_merge_ev writes the same output as
    spec_attn_block_merge and its events bracket the kernel."""
    import ctypes
    from speculative_decoding_verify_split_amd import rapid_verify as rv
    ai, split = _make_case(ATTN_CASES[0])
    announce("spec_attn_block_merge_ev")
    st = VerifyStep(ai, None, split=split)
    st.attention(fused=True)
    torch.cuda.synchronize()
    ref = (st.out.clone(), st.lse_out.clone())
    st.out.zero_()
    st.lse_out.zero_()
    hip = ctypes.CDLL("libamdhip64.so")
    evs = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in evs:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        rv.spec_attn_block_merge_ev(st.q, st.k_blk, st.v_blk, st.parent, st.o_part, st.lse_part,
                                    st.out, evs[0], evs[1], st.lse_out, st.sm_scale)
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
        announce("  kernel %.2f us" % (ms.value * 1e3))
        assert ms.value > 0
    finally:
        for e in evs:
            hip.hipEventDestroy(e)
    assert torch.equal(st.out.view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(st.lse_out, ref[1])


def test_seq_lens_are_clamped_on_the_device():
    ai = make_attention(33, 3, 4, 2, 128, 4, [640, 640, 640], L_max=640)
    announce("seq_lens clamp")
    st = VerifyStep(ai, None, split=(256, 3))
    st.seq_lens.copy_(torch.tensor([640 + 77, -5, 300], dtype=torch.int32))
    st.attention()
    out, lse = _attn_outputs(st)
    eff = np.array([640, 0, 300])
    O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, eff)
    assert attn_row_errors(out, O_ref).max() <= ATTN_ROW_TOL
    assert np.abs(lse - L_ref).max() <= _lse_tol(4, 2, 4)


@pytest.mark.parametrize("G", [2, 8])
def test_seq_lens_beyond_the_splits_are_cut_at_their_capacity(G):
    """A device length in (S*split_len, L_max] attends over the first
    S*split_len tokens only (the partials hold S splits); both kernels."""
    ai = make_attention(35, 2, 2 * G, 2, 128, 11, [500, 200], L_max=1000)
    announce("seq_lens past the splits, G=%d" % G)
    st = VerifyStep(ai, None, split=(256, 2))
    st.seq_lens.copy_(torch.tensor([900, 513], dtype=torch.int32))
    for fused in (False, True):
        st.attention(fused=fused)
        out, lse = _attn_outputs(st)
        O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk,
                                np.array([512, 512]))
        assert attn_row_errors(out, O_ref).max() <= ATTN_ROW_TOL
        assert np.abs(lse - L_ref).max() <= _lse_tol(2 * G, 2, 11)


def test_sm_scale_is_applied():
    ai = make_attention(34, 1, 4, 2, 64, 5, [900])
    announce("sm_scale 0.37")
    ai.sm_scale = 0.37
    st = VerifyStep(ai, None)
    st.attention()
    out, lse = _attn_outputs(st)
    O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens,
                            sm_scale=0.37)
    assert attn_row_errors(out, O_ref).max() <= ATTN_ROW_TOL
    assert np.abs(lse - L_ref).max() <= _lse_tol(4, 2, 5)


# ------------------------------------------------------ vocabulary, small

def _run_accept(vi, p_hat=True, flags=0):
    st = VerifyStep(None, vi, want_ratio=True, want_p_hat=p_hat, flags=flags)
    st.accept()
    torch.cuda.synchronize()
    return st


TAIL_AMBIGUITY = 1e-5   # relative distance to the tail threshold fp32 may misplace
TAIL_MAX_AMBIGUOUS = 6  # entries whose sides are enumerated (2^6 oracle runs)


def _tail_ambiguous(vi):
    """The p_hat entries within TAIL_AMBIGUITY (relative) of the tail
    threshold 0.1 max p_hat, per (sequence, row), in oracle arithmetic:
    fp32 and fp64 may place them on different sides, and either is the
    rule applied correctly."""
    amb = {}
    for b in range(vi.z.shape[0]):
        for t in range(vi.y.shape[1]):
            _, _, ph = retrieval_augmented_target(vi.z[b, t], vi.y[b, t], vi.T, vi.eta)
            thr = 0.1 * ph.max()
            ks = np.nonzero(np.abs(ph - thr) <= TAIL_AMBIGUITY * thr)[0]
            if len(ks):
                amb[(b, t)] = [int(k) for k in ks]
    return amb


def _tail_forcings(vi):
    """Every assignment of sides to the ambiguous entries, as tail_force
    dicts for rapid_accept_ref (one empty dict when there is none)."""
    slots = [(bt, k) for bt, ks in _tail_ambiguous(vi).items() for k in ks]
    if len(slots) > TAIL_MAX_AMBIGUOUS:
        return None
    out = []
    for sides in itertools.product((False, True), repeat=len(slots)):
        f = {}
        for (bt, k), side in zip(slots, sides):
            f.setdefault(bt, {})[k] = side
        out.append(f)
    return out


def _check_accept(vi, st, tag, flags=0):
    """The GPU's acceptance outputs against the oracle.  Under the tail rule,
    p_hat entries within TAIL_AMBIGUITY of the threshold may fall on either
    side: the check passes if the outputs match the oracle under one of the
    assignments of sides to those entries (skipped only when more than
    TAIL_MAX_AMBIGUOUS entries are that close)."""
    tail = bool(flags & RV_ACCEPT_TAIL_PRESERVE)
    forcings = _tail_forcings(vi) if tail else [{}]
    if forcings is None:
        pytest.skip("%s: more than %d p_hat entries lie within %g of the tail threshold"
                    % (tag, TAIL_MAX_AMBIGUOUS, TAIL_AMBIGUITY))
    n_g = st.n_accept.cpu().numpy()
    tok = st.out_tokens.cpu().numpy()
    ratio = st.ratio.cpu().numpy()
    ph_g = st.p_hat.cpu().numpy() if st.p_hat is not None else None
    tried = []
    for force in forcings:
        ref = rapid_accept_ref(vi.z, vi.y, vi.draft, vi.r, vi.u, vi.T, vi.eta,
                               tail_preserve=tail,
                               residual="printed" if flags & RV_ACCEPT_PRINTED_RESIDUAL
                               else "p_hat", tail_force=force)
        res = compare_accept(ref, n_g, tok, vi.r, vi.u, draft=vi.draft)
        dr = np.abs(ratio - ref["ratio"]).max()
        dp = np.abs(ph_g - ref["p_hat"]).max() if ph_g is not None else None
        ok = not res["errors"] and dr <= 1e-5 and (dp is None or dp <= P_HAT_TOL)
        tried.append((ok, ref, res, dr, dp, force))
        if ok:
            break
    ok, ref, res, dr, dp, force = next((x for x in tried if x[0]), tried[0])
    announce("  %s: n_accept gpu=%s ref=%s |dratio|=%.2e |dp_hat|=%s flagged(acc=%d, draw=%d) "
             "diverged=%d%s" % (tag, n_g.tolist(), ref["n_accept"].tolist(), dr,
                                "%.2e" % dp if dp is not None else "-", res["flagged_accept"],
                                res["flagged_draw"], res["diverged"],
                                (" (tail sides of %d near-threshold entries: %s, %d of %d "
                                 "assignments tried)" % (sum(len(v) for v in force.values()),
                                                         force, len(tried), len(forcings)))
                                if force else ""))
    assert not res["errors"], res["errors"]
    assert dr <= 1e-5
    if dp is not None:
        assert dp <= P_HAT_TOL
    return ref, res


VOCAB_CASES = [
    ("V9001-g3-b3-scalar-path", dict(seed=41, B=3, gamma=3, V=9001, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)),
    ("V2-g1-b4", dict(seed=42, B=4, gamma=1, V=2, z_sigma=1.0, noise=1.0, T=1.0, eta=0.5)),
    ("V5000-g63", dict(seed=43, B=1, gamma=63, V=5000, z_sigma=3.0, noise=0.3, T=1.0, eta=0.5)),
    ("V20000-T0.7-eta2-b2", dict(seed=44, B=2, gamma=10, V=20000, z_sigma=3.0, noise=1.0, T=0.7, eta=2.0)),
    ("V12000-eta0", dict(seed=45, B=2, gamma=5, V=12000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.0)),
    ("V8192-g7-b5", dict(seed=46, B=5, gamma=7, V=8192, z_sigma=2.0, noise=0.5, T=1.3, eta=1.0)),
]


@pytest.mark.parametrize("case", VOCAB_CASES, ids=[c[0] for c in VOCAB_CASES])
def test_accept_small(case):
    name, kw = case
    vi = make_vocab(**kw)
    announce("rapid_accept %s" % name)
    st = _run_accept(vi)
    _check_accept(vi, st, name)


@pytest.mark.timeout(300)
def test_accept_max_vocab():
    """V = 2^22, the largest vocabulary: 1024 statistics chunks and 4096
    decide/draw chunks, so the draw's chunk scan runs over 16 blocks."""
    vi = make_vocab(48, B=2, gamma=2, V=1 << 22, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    announce("rapid_accept V=2^22 B=2 gamma=2")
    st = _run_accept(vi, p_hat=False)
    _check_accept(vi, st, "V=2^22")
    vi.r = np.zeros_like(vi.r)  # every draft kept: the bonus draw over 2^22 ids
    st = _run_accept(vi, p_hat=False)
    _check_accept(vi, st, "V=2^22 all-accept")


def test_accept_batch64():
    vi = make_vocab(49, B=64, gamma=4, V=32000, z_sigma=3.0, noise=1.0, T=0.9, eta=1.0)
    announce("rapid_accept B=64 gamma=4 V=32000")
    _check_accept(vi, _run_accept(vi), "B=64")


def test_draw_slot_survives_repeated_calls():
    """The drawn token's slot is written by the drawing workgroup alone: 100
    back-to-back calls at the 8B vocabulary (126 decide workgroups spread
    over the XCDs) all reproduce the first call's outputs."""
    vi = config_vocab("llama8b", eta=0.5, B_override=4)
    announce("rapid_accept x100, B=4, V=128256")
    st = VerifyStep(None, vi, want_ratio=True)
    st.accept()
    torch.cuda.synchronize()
    ref = (st.n_accept.clone(), st.out_tokens.clone())
    assert (ref[0] >= 0).all()
    for i in range(100):
        st.out_tokens.fill_(-7)
        st.accept()
    torch.cuda.synchronize()
    assert torch.equal(st.n_accept, ref[0]) and torch.equal(st.out_tokens, ref[1])
    for i in range(20):  # and with each call checked on its own
        st.out_tokens.fill_(-7)
        st.accept()
        torch.cuda.synchronize()
        assert torch.equal(st.out_tokens, ref[1]), "call %d" % i


def test_accept_tiny_config():
    vi = config_vocab("tiny")
    announce("rapid_accept tiny config")
    _check_accept(vi, _run_accept(vi), "tiny")


def test_accept_forced_cuts():
    """r = 0 accepts every draft (bonus draw); r close to 1 rejects early;
    r just outside the flag zone on either side of each ratio."""
    base = make_vocab(47, B=4, gamma=6, V=30000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    ref = rapid_accept_ref(base.z, base.y, base.draft, base.r, base.u, base.T, base.eta)
    ratio = ref["ratio"]
    variants = {
        "all-accept": np.zeros_like(base.r),
        "near-one": np.full_like(base.r, np.float32(1.0 - 2 ** -24)),
        "just-below": np.clip(ratio - 3e-4, 0.0, 1.0 - 2 ** -24).astype(np.float32),
        "just-above": np.clip(ratio + 3e-4, 0.0, 1.0 - 2 ** -24).astype(np.float32),
    }
    for tag, r in variants.items():
        vi = make_vocab(47, B=4, gamma=6, V=30000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
        vi.r = r
        announce("rapid_accept forced %s" % tag)
        refv, _ = _check_accept(vi, _run_accept(vi, p_hat=False), tag)
        if tag == "all-accept":
            assert np.all(refv["n_accept"] == 6)


def test_accept_bad_draft_id_sentinel():
    vi = make_vocab(48, B=3, gamma=4, V=5000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    vi.draft[1, 2] = 5000
    vi.draft[2, 0] = -7
    announce("rapid_accept bad draft ids")
    st = _run_accept(vi, p_hat=False)
    n_g = st.n_accept.cpu().numpy()
    tok = st.out_tokens.cpu().numpy()
    assert n_g[1] == -1 and n_g[2] == -1
    assert np.all(tok[1] == -1) and np.all(tok[2] == -1)
    good = make_vocab(48, B=3, gamma=4, V=5000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    ref = rapid_accept_ref(good.z[:1], good.y[:1], good.draft[:1], good.r[:1], good.u[:1], 1.0, 0.5)
    res = compare_accept(ref, n_g[:1], tok[:1], good.r[:1], good.u[:1], draft=good.draft[:1])
    assert not res["errors"]


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_accept_nonfinite_logits_stay_in_range(flags):
    """Non-finite logits give unspecified tokens, never an out-of-range one:
    every drawn id lies in [0, V), accepted prefixes are the drafts, the
    rest is -1.  (Every address in the pass comes from loop indices and the
    validated draft ids; no float value indexes memory.)"""
    V, g = 5000, 4
    vi = make_vocab(49, B=5, gamma=g, V=V, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    vi.z[0] = np.nan                        # all-NaN target
    vi.z[1, :, ::97] = np.inf               # +inf target entries
    vi.y[1, :, ::89] = -np.inf              # -inf draft entries
    vi.y[2] = np.nan                        # all-NaN draft
    vi.z[3, :, 17] = np.inf                 # one +inf per target row
    vi.y[3, :, 17] = np.inf
    vi.z[4] = -np.inf                       # all -inf target
    announce("rapid_accept non-finite logits, flags %d" % flags)
    st = _run_accept(vi, p_hat=False, flags=flags)
    n_g = st.n_accept.cpu().numpy()
    tok = st.out_tokens.cpu().numpy()
    for b in range(5):
        n = int(n_g[b])
        assert 0 <= n <= g, (b, n)
        assert np.array_equal(tok[b, :n], vi.draft[b, :n])
        assert 0 <= tok[b, n] < V, (b, tok[b])
        assert np.all(tok[b, n + 1:] == -1)


def test_accept_nan_with_every_bit_set_and_a_filled_workspace():
    """A chunk's two draw weights travel as one 64-bit slot whose all-ones
    pattern means "not yet written".  A bonus row of NaNs with every bit set
    makes both weights that pattern; the pass publishes it as another NaN,
    so the draw still ends with an id in [0, V).  The workspace starts
    filled with 0xFF bytes (stale slots and counters), which the pass clears
    itself."""
    V, g = 5000, 4
    vi = make_vocab(50, B=3, gamma=g, V=V, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    vi.r[:] = 0.0                             # every draft accepted: the bonus row is drawn
    zb = vi.z.view(np.uint32)
    zb[0, g] = 0xFFFFFFFF                     # whole bonus row
    zb[1, g, ::3] = 0xFFFFFFFF                # every third entry
    announce("rapid_accept all-ones NaN bonus rows, 0xFF-filled workspace")
    st = VerifyStep(None, vi, want_ratio=True)
    for _ in range(2):
        st.workspace.fill_(0xFF)
        st.out_tokens.fill_(-7)
        st.accept()
        torch.cuda.synchronize()
        n_g = st.n_accept.cpu().numpy()
        tok = st.out_tokens.cpu().numpy()
        assert list(n_g) == [g, g, g]
        for b in range(3):
            assert np.array_equal(tok[b, :g], vi.draft[b, :g])
            assert 0 <= tok[b, g] < V, (b, tok[b])
    ref = rapid_accept_ref(vi.z[2:], vi.y[2:], vi.draft[2:], vi.r[2:], vi.u[2:], 1.0, 0.5)
    res = compare_accept(ref, n_g[2:], tok[2:], vi.r[2:], vi.u[2:], draft=vi.draft[2:])
    assert not res["errors"]


def test_step_is_bit_deterministic():
    ai = config_attention("tiny")
    vi = config_vocab("tiny")
    announce("determinism tiny")
    outs = []
    for _ in range(2):
        st = VerifyStep(ai, vi, want_p_hat=True)
        st.run()
        torch.cuda.synchronize()
        res = [t.cpu().clone() for t in (st.out.view(torch.int16), st.lse_out, st.o_part,
                                         st.n_accept, st.out_tokens, st.ratio, st.p_hat)]
        st.attention(fused=True)
        torch.cuda.synchronize()
        res += [st.out.view(torch.int16).cpu().clone(), st.lse_out.cpu().clone()]
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------- the five workloads, full size

def _config_attention_check(name):
    announce("generating %s attention inputs" % name)
    ai = config_attention(name)
    B, Hq, n, d = ai.q.shape
    Hkv = ai.k_cache.shape[1]
    announce("attention %s shape=%s" % (name, ai.shape))
    st = VerifyStep(ai, None)  # default split: the benchmark's launch configuration
    st.attention()
    out, lse = _attn_outputs(st)
    lse_part = st.lse_part.cpu().numpy()
    lse_blk = st.lse_blk.cpu().numpy()
    st.attention(fused=True)  # the fused block + merge
    out_f, lse_f = _attn_outputs(st)
    # the whole attention through spec_attn_verify (the benchmark's step),
    # one launch where rv_verify_single_launch says so
    single = rv.rv_verify_single_launch(B, Hq, Hkv, n, d, st.num_splits)
    st.attention(single=True)
    out_s, lse_s = _attn_outputs(st)
    assert not st.sync.any()  # the sync words are left zero
    # properties at any size
    for o, l in ((out, lse), (out_f, lse_f), (out_s, lse_s)):
        assert np.isfinite(o).all() and np.isfinite(l).all()
        assert np.all(l >= np.maximum(lse_part.max(axis=-1), lse_blk) - 1e-4)
    for o, l in ((out_f, lse_f), (out_s, lse_s)):
        assert attn_row_errors(o, out).max() <= 1e-2  # one bf16 step, as above
        assert np.abs(l - lse).max() <= 1e-4
    if not single:  # the same two launches as the fused call
        assert np.array_equal(out_s.view(np.uint16), out_f.view(np.uint16))
        assert np.array_equal(lse_s, lse_f)
    # every (sequence, query head, row) against the oracle, one kv head at a
    # time (the oracle's scores for a kv head are G*n rows by the history)
    tol = _lse_tol(Hq, Hkv, n)
    worst = {False: (0.0, 0.0), True: (0.0, 0.0), "single": (0.0, 0.0)}
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            heads = list(range(g * G, (g + 1) * G))
            O_ref, L_ref = attn_ref(ai.q[b:b + 1, g * G:(g + 1) * G], ai.k_cache[b:b + 1, g:g + 1],
                                    ai.v_cache[b:b + 1, g:g + 1], ai.k_blk[b:b + 1, g:g + 1],
                                    ai.v_blk[b:b + 1, g:g + 1], ai.seq_lens[b:b + 1], ai.parent,
                                    ai.sm_scale)
            for fused, o, l in ((False, out, lse), (True, out_f, lse_f),
                                ("single", out_s, lse_s)):
                err = attn_row_errors(o[b, heads], O_ref[0]).max()
                dl = np.abs(l[b, heads] - L_ref[0]).max()
                worst[fused] = (max(worst[fused][0], err), max(worst[fused][1], dl))
                assert err <= ATTN_ROW_TOL, (b, g, fused, err)
                assert dl <= tol, (b, g, fused, dl)
        announce("  b=%d: %d query heads x %d rows checked" % (b, Hq, n))
    names = {False: "block+merge", True: "block_merge",
             "single": "verify (%s)" % ("one launch" if single else "two launches")}
    for fused in (False, True, "single"):
        announce("  %s: max row rel err %.3e, max |dLSE| %.3e over all %d rows"
                 % (names[fused], worst[fused][0], worst[fused][1], B * Hq * n))


# (llama8b_tp8: one GPU's share under 8-way head parallelism; its default
# 512-key splits give 256 partials per row, the eight-wave merge fold)
@pytest.mark.parametrize("name", ["tiny", "llama8b", "llama70b", "qwen7b_ragged", "llama8b_tp8"])
@pytest.mark.timeout(600)
def test_config_attention(name):
    _config_attention_check(name)


@pytest.mark.timeout(1100)
def test_config_attention_tree1m():
    _config_attention_check("tree1m")


RULE_FLAGS = [RV_ACCEPT_TAIL_PRESERVE, RV_ACCEPT_PRINTED_RESIDUAL,
              RV_ACCEPT_TAIL_PRESERVE | RV_ACCEPT_PRINTED_RESIDUAL]


@pytest.mark.parametrize("flags", RULE_FLAGS)
@pytest.mark.parametrize("case", VOCAB_CASES[:4] + [("V8192-g7-b5", VOCAB_CASES[5][1])],
                         ids=[c[0] for c in VOCAB_CASES[:4]] + ["V8192-g7-b5"])
def test_accept_rules_small(case, flags):
    """RAPID blog section 2.4's tail rule and printed residual (flags)."""
    name, kw = case
    vi = make_vocab(**kw)
    announce("rapid_accept_ex %s flags=%d" % (name, flags))
    _check_accept(vi, _run_accept(vi, flags=flags), "%s flags=%d" % (name, flags), flags)


def test_accept_rules_forced_rejections():
    """Every sequence rejects its first draft, so every draw uses the rule's
    residual."""
    for flags in RULE_FLAGS:
        vi = make_vocab(49, B=6, gamma=3, V=20000, z_sigma=3.0, noise=1.0, T=1.0, eta=1.0)
        vi.r[:] = np.float32(1.0 - 2 ** -24)
        announce("rapid_accept_ex forced rejections flags=%d" % flags)
        ref, _ = _check_accept(vi, _run_accept(vi, flags=flags), "reject flags=%d" % flags, flags)
        assert np.all(ref["n_accept"] <= 1)


@pytest.mark.parametrize("flags", RULE_FLAGS)
@pytest.mark.timeout(600)
def test_config_vocab_rules(flags):
    vi = config_vocab("llama8b", eta=2.0)
    announce("rapid_accept_ex llama8b eta=2 flags=%d" % flags)
    _check_accept(vi, _run_accept(vi, flags=flags), "llama8b flags=%d" % flags, flags)


@pytest.mark.parametrize("name,eta", [("llama8b", 0.0), ("llama8b", 0.5), ("llama8b", 2.0),
                                      ("llama70b", None), ("qwen7b_ragged", None),
                                      ("tree1m", None)])
@pytest.mark.timeout(600)
def test_config_vocab(name, eta):
    vi = config_vocab(name, eta=eta)
    announce("rapid_accept %s eta=%s B=%d gamma=%d V=%d" % (name, vi.eta, *vi.y.shape))
    _check_accept(vi, _run_accept(vi), "%s eta=%s" % (name, vi.eta))


# Many sequences at the workloads' vocabulary sizes: every setting's draws
# compared one by one (bit-exact outside flagged positions).  About 40% of
# the draws at V ~ 1.3e5 fall within 1e-4 of an interval edge (the residual
# mass spreads over ~10^3 ids), so 384 sequences leave well over 150
# unflagged draws per setting.
SWEEP = [("llama8b", 0.0), ("llama8b", 0.5), ("llama8b", 2.0), ("llama70b", 1.0),
         ("qwen7b_ragged", 0.5)]


@pytest.mark.parametrize("name,eta", SWEEP, ids=["%s-eta%g" % c for c in SWEEP])
@pytest.mark.timeout(900)
def test_config_vocab_many_sequences(name, eta):
    B = 384
    vi = config_vocab(name, eta=eta, B_override=B)
    announce("rapid_accept sweep %s eta=%g T=%g B=%d gamma=%d V=%d"
             % (name, eta, vi.T, B, vi.y.shape[1], vi.y.shape[2]))
    st = _run_accept(vi, p_hat=False)
    ref, res = _check_accept(vi, st, "%s eta=%g sweep" % (name, eta))
    fa6, fd6, _ = flag_counts(ref, vi.r, 1e-6)
    fa4, fd4, _ = flag_counts(ref, vi.r, BOUNDARY_TOL)
    alpha = float(np.mean([np.sum(np.minimum(ref["p_hat"][b, t], _q_row(vi, b, t)))
                           for b in range(4) for t in range(vi.y.shape[1])]))
    announce("  exact draws %d of %d; flagged accepts %d (1e-4) / %d (1e-6); flagged draws "
             "%d (1e-4) / %d (1e-6); diverged %d; mean n_accept %.3f; alpha (4 seqs) %.3f"
             % (res["exact_draws"], B, fa4, fa6, fd4, fd6, res["diverged"],
                float(np.mean(ref["n_accept"])), alpha))
    assert res["exact_draws"] >= 150
    assert res["diverged"] <= 3


def _q_row(vi, b, t):
    from oracle import draft_probs
    return draft_probs(vi.y[b, t], vi.T)


# Chunking edges of the vocabulary pass: a vocabulary of exactly one decide
# chunk, an odd one (scalar loads), gamma = 16 and 20, and V = 300000, whose
# draw scans more than one block of 256 decide chunks.
ACCEPT_EDGE_CASES = [
    ("V100000-g16-b2", dict(seed=51, B=2, gamma=16, V=100000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)),
    ("V5001-g20-b3", dict(seed=52, B=3, gamma=20, V=5001, z_sigma=3.0, noise=1.0, T=0.8, eta=1.5)),
    ("V300000-g4-b2", dict(seed=53, B=2, gamma=4, V=300000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)),
    ("V1024-g10-b3", dict(seed=54, B=3, gamma=10, V=1024, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)),
]


@pytest.mark.parametrize("flags", [0, RV_ACCEPT_TAIL_PRESERVE | RV_ACCEPT_PRINTED_RESIDUAL])
@pytest.mark.parametrize("case", ACCEPT_EDGE_CASES, ids=[c[0] for c in ACCEPT_EDGE_CASES])
def test_accept_chunking_edges(case, flags):
    name, kw = case
    vi = make_vocab(**kw)
    announce("rapid_accept %s flags=%d" % (name, flags))
    _check_accept(vi, _run_accept(vi, flags=flags), "%s flags=%d" % (name, flags), flags)
