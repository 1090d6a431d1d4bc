"""Pins for the attention oracle (CPU only).

Each test fixes the oracle to something other than itself: a library
conversion, a brute-force double loop, a closed form, or the split/merge
identity of the LongSpec summary (gist.science, section 2.3 "Fast Tree
Attention": the unmasked history part and the masked speculative part are
merged by log-sum-exp and must give the unsplit result).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attn_keys_ref, attn_ref, bf16_bits_to_f64, block_visibility, lse_merge_ref
from workloads import f32_to_bf16_bits, make_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- bf16 decode

def test_bf16_decode_matches_torch_and_hand_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    exp_field = (bits >> 7) & 0xFF
    bits = bits[exp_field != 0xFF]  # drop NaN/Inf patterns
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(bf16_bits_to_f64(bits), ref)
    hand = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x3F00: 0.5, 0x4049: 3.140625,
            0x7F80: math.inf, 0x0001: 2.0 ** -133}
    for b, v in hand.items():
        assert bf16_bits_to_f64(np.array([b], dtype=np.uint16))[0] == v


def test_generator_rounding_is_nearest_even():
    # ties: 1 + 2^-8 is exactly half way between bf16 1.0 and 1 + 2^-7 -> even (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    got = bf16_bits_to_f64(_bits(x))
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5])
    t = torch.from_numpy(np.random.default_rng(1).standard_normal(5000).astype(np.float32))
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(_bits(t.numpy()), ref)


# ------------------------------------------------------- brute force (P10)

def _brute(q, k, v, kb, vb, lens, parent, scale):
    """Independent double loop in pure Python floats."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    f = lambda a: float(bf16_bits_to_f64(np.array([a], dtype=np.uint16))[0])
    O = np.zeros((B, Hq, n, d))
    LSE = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(n):
                qi = [f(q[b, h, i, c]) for c in range(d)]
                keys, vals = [], []
                for j in range(int(lens[b])):
                    keys.append([f(k[b, g, j, c]) for c in range(d)])
                    vals.append([f(v[b, g, j, c]) for c in range(d)])
                for j in range(n):
                    if parent is None:
                        ok = j <= i
                    else:
                        a, ok = i, False
                        while a != -1:
                            if a == j:
                                ok = True
                            a = int(parent[a])
                    if ok:
                        keys.append([f(kb[b, g, j, c]) for c in range(d)])
                        vals.append([f(vb[b, g, j, c]) for c in range(d)])
                s = [scale * sum(qi[c] * kk[c] for c in range(d)) for kk in keys]
                m = max(s)
                tot = sum(math.exp(x - m) for x in s)
                lse = m + math.log(tot)
                LSE[b, h, i] = lse
                for c in range(d):
                    O[b, h, i, c] = sum(math.exp(s[j] - lse) * vals[j][c] for j in range(len(s)))
    return O, LSE


@pytest.mark.parametrize("parent", [None, np.array([-1, 0, 0, 1], np.int32)])
def test_attn_matches_bruteforce(parent):
    ai = make_attention(7, B=2, Hq=4, Hkv=2, d=8, n=4, L=[5, 0], L_max=6, parent=parent)
    # scale the queries up so the softmax is far from uniform
    scale = 3.0
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, parent, scale)
    Ob, Lb = _brute(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, parent, scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


def test_pairs_selection_matches_full():
    ai = make_attention(8, B=2, Hq=6, Hkv=3, d=16, n=3, L=[40, 17], L_max=48)
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens)
    pairs = [(1, 5), (0, 0), (1, 2)]
    Os, Ls = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, pairs=pairs)
    for i, (b, h) in enumerate(pairs):
        np.testing.assert_array_equal(Os[i], O[b, h])
        np.testing.assert_array_equal(Ls[i], L[b, h])


# ----------------------------------------------------- closed forms (P8)

def test_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    O, L = attn_keys_ref(q, k, v, np.ones((3, 1), bool), 0.7)
    np.testing.assert_allclose(O, np.repeat(v, 3, axis=0), atol=1e-15)
    np.testing.assert_allclose(L, 0.7 * (q @ k[0]), atol=1e-14)


def test_zero_query_gives_mean_of_visible_values_and_log_count():
    ai = make_attention(3, B=1, Hq=2, Hkv=1, d=8, n=5, L=9)
    ai.q[:] = 0
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens)
    vpre = bf16_bits_to_f64(ai.v_cache[0, 0, :9])
    vblk = bf16_bits_to_f64(ai.v_blk[0, 0])
    for i in range(5):
        vis = np.concatenate([vpre, vblk[: i + 1]])
        np.testing.assert_allclose(O[0, 0, i], vis.mean(axis=0), atol=1e-14)
        assert abs(L[0, 1, i] - math.log(9 + i + 1)) < 1e-14


def test_empty_history_single_row_is_block_value():
    ai = make_attention(4, B=1, Hq=1, Hkv=1, d=16, n=1, L=0, L_max=4)
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, sm_scale=1.3)
    np.testing.assert_allclose(O[0, 0, 0], bf16_bits_to_f64(ai.v_blk[0, 0, 0]), atol=1e-15)
    qk = bf16_bits_to_f64(ai.q[0, 0, 0]) @ bf16_bits_to_f64(ai.k_blk[0, 0, 0])
    assert abs(L[0, 0, 0] - 1.3 * qk) < 1e-14


def test_chain_parent_equals_causal_mask():
    n = 9
    chain = np.arange(-1, n - 1, dtype=np.int32)
    np.testing.assert_array_equal(block_visibility(n, chain), block_visibility(n, None))
    np.testing.assert_array_equal(block_visibility(n, None), np.tril(np.ones((n, n), bool)))
    ai = make_attention(5, B=1, Hq=2, Hkv=1, d=8, n=n, L=13)
    a = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, None)
    b = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, chain)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_star_tree_sees_root_and_self_only():
    n = 6
    star = np.array([-1] + [0] * (n - 1), np.int32)
    vis = block_visibility(n, star)
    for i in range(n):
        expect = {0, i}
        assert set(np.nonzero(vis[i])[0].tolist()) == expect
    ai = make_attention(6, B=1, Hq=1, Hkv=1, d=8, n=n, L=4)
    ai.q[:] = 0
    O, _ = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, star)
    vpre = bf16_bits_to_f64(ai.v_cache[0, 0, :4])
    vblk = bf16_bits_to_f64(ai.v_blk[0, 0])
    for i in range(1, n):
        vis_v = np.concatenate([vpre, vblk[[0, i]]])
        np.testing.assert_allclose(O[0, 0, i], vis_v.mean(axis=0), atol=1e-14)


def test_tree_validation_rejects_bad_parents():
    with pytest.raises(ValueError):
        block_visibility(3, np.array([0, 0, 1]))
    with pytest.raises(ValueError):
        block_visibility(3, np.array([-1, 2, 0]))
    with pytest.raises(ValueError):
        block_visibility(3, np.array([-1, 0]))


def test_gqa_head_map_is_contiguous_groups():
    # kv head g holds the constant value g+1 everywhere: every query head h
    # must return h // G + 1 whatever it attends to.
    ai = make_attention(9, B=1, Hq=8, Hkv=4, d=8, n=3, L=10)
    for g in range(4):
        ai.v_cache[0, g] = _bits(g + 1.0)
        ai.v_blk[0, g] = _bits(g + 1.0)
    O, _ = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens)
    for h in range(8):
        np.testing.assert_allclose(O[0, h], h // 2 + 1.0, atol=1e-14)


def test_history_beyond_seq_len_is_never_read():
    nan_bits = 0x7FC0
    ai = make_attention(10, B=3, Hq=2, Hkv=1, d=8, n=3, L=[5, 0, 7], L_max=9, pad_bits=nan_bits)
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    # same result as a cache trimmed to each sequence's length
    for b, Lb in enumerate([5, 0, 7]):
        o1, l1 = attn_ref(ai.q[b:b + 1], ai.k_cache[b:b + 1, :, :Lb], ai.v_cache[b:b + 1, :, :Lb],
                          ai.k_blk[b:b + 1], ai.v_blk[b:b + 1], np.array([Lb]))
        np.testing.assert_array_equal(o1[0], O[b])
        np.testing.assert_array_equal(l1[0], L[b])


def test_scale_is_applied_to_scores():
    ai = make_attention(11, B=1, Hq=2, Hkv=1, d=8, n=2, L=6)
    q2 = _bits(bf16_bits_to_f64(ai.q).astype(np.float32) * 2)  # exact (power of two)
    a = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, sm_scale=2.0)
    b = attn_ref(q2, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, sm_scale=1.0)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_large_scores_do_not_overflow():
    q = np.array([[1.0, 0.0]])
    k = np.array([[1000.0, 0.0], [999.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    O, L = attn_keys_ref(q, k, v, np.ones((1, 2), bool), 1.0)
    e = math.exp(-1.0)
    np.testing.assert_allclose(O[0], [1 / (1 + e), e / (1 + e)], atol=1e-15)
    assert abs(L[0] - (1000.0 + math.log1p(e))) < 1e-12


# ----------------------------------------------- split + LSE merge (P9)

def test_lse_merge_closed_form_two_parts():
    o1, o2 = np.array([1.0, 2.0]), np.array([-3.0, 0.5])
    a, b = 0.3, -1.7
    O, L = lse_merge_ref([(o1, np.array(a)), (o2, np.array(b))])
    assert abs(L - np.logaddexp(a, b)) < 1e-15
    wa = 1.0 / (1.0 + math.exp(b - a))
    np.testing.assert_allclose(O, wa * o1 + (1 - wa) * o2, atol=1e-15)


def test_lse_merge_ignores_empty_parts():
    o1 = np.array([[1.0, 2.0]])
    O, L = lse_merge_ref([(o1, np.array([0.25])), (np.zeros((1, 2)), np.array([-np.inf]))])
    np.testing.assert_array_equal(O, o1)
    np.testing.assert_array_equal(L, [0.25])
    O, L = lse_merge_ref([(np.zeros((1, 2)), np.array([-np.inf]))] * 2)
    np.testing.assert_array_equal(O, 0.0)
    assert np.isneginf(L).all()


@pytest.mark.parametrize("seed", range(6))
def test_split_and_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    R, K, d = 7, 60, 16
    q = rng.standard_normal((R, d))
    k = rng.standard_normal((K, d))
    v = rng.standard_normal((K, d))
    vis = rng.random((R, K)) < 0.8
    vis[:, 0] = True
    O, L = attn_keys_ref(q, k, v, vis, 0.9)
    nparts = 1 + seed
    cuts = np.sort(rng.choice(np.arange(1, K), size=nparts - 1, replace=False)) if nparts > 1 else []
    bounds = [0, *cuts, K]
    parts = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        parts.append(attn_keys_ref(q, k[lo:hi], v[lo:hi], vis[:, lo:hi], 0.9))
    parts.append(attn_keys_ref(q, k[:0], v[:0], vis[:, :0], 0.9))  # an empty split
    Om, Lm = lse_merge_ref(parts)
    np.testing.assert_allclose(Om, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lm, L, rtol=0, atol=1e-12)


def test_hybrid_split_prefix_plus_masked_block_equals_definition():
    """History part (no mask) + draft-block part (tree mask) merged by LSE."""
    parent = np.array([-1, 0, 0, 1, 3, 2], np.int32)
    ai = make_attention(12, B=1, Hq=4, Hkv=2, d=16, n=6, L=50, parent=parent)
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, parent, 1.0)
    vis = block_visibility(6, parent)
    for h in range(4):
        g = h // 2
        q = bf16_bits_to_f64(ai.q[0, h])
        kp, vp = bf16_bits_to_f64(ai.k_cache[0, g, :50]), bf16_bits_to_f64(ai.v_cache[0, g, :50])
        kb, vb = bf16_bits_to_f64(ai.k_blk[0, g]), bf16_bits_to_f64(ai.v_blk[0, g])
        parts = [attn_keys_ref(q, kp[lo:lo + 16], vp[lo:lo + 16], np.ones((6, min(16, 50 - lo)), bool), 1.0)
                 for lo in range(0, 50, 16)]
        parts.append(attn_keys_ref(q, kb, vb, vis, 1.0))
        Om, Lm = lse_merge_ref(parts)
        np.testing.assert_allclose(Om, O[0, h], atol=1e-12)
        np.testing.assert_allclose(Lm, L[0, h], atol=1e-12)
