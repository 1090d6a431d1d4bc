"""fp64 oracle for the verify attention (test infrastructure only).

The verify queries are the rows of the draft block: for a chain, row 0 is the
last committed token and rows 1..gamma are the draft tokens; for a tree, the
rows are the tree's nodes.  Every row attends to

* the whole history KV cache of its sequence, with no mask (LongSpec summary,
  gist.science, section 2.3 "Fast Tree Attention": the history key/value
  pairs need no mask), and
* the draft block's own keys under the causal mask (chain) or the tree mask
  (a node sees its ancestors and itself), which is the small masked part of
  the same section.

Softmax attention over that visible key set is written out as its plain
definition:  s_j = sm_scale * <q, k_j>,  LSE = log sum_j exp(s_j),
O = sum_j exp(s_j - LSE) v_j  (natural log).  The unmasked-prefix / masked-
block split with a log-sum-exp merge, which the same section describes,
reaches this result exactly up to rounding order; ``lse_merge_ref`` is that
merge, kept here so tests can pin the split identity against the definition.

Readings where the page is silent:
* query head h reads kv head h // G with G = H_q / H_kv (contiguous groups);
* the draft block's keys/values are separate tensors, not appended to the
  cache; the prefix length of sequence b is seq_lens[b] (0 allowed);
* a row that sees no key (impossible here, since a row always sees itself)
  or an empty split has LSE = -inf and O = 0.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Widen bf16 values, given as raw uint16 bit patterns, to float64.

    A bf16 value is the upper 16 bits of an IEEE binary32 value, so shifting
    the pattern left by 16 gives that binary32 exactly; binary32 -> binary64
    is exact.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def block_visibility(n, parent=None):
    """Visibility of the draft block's keys: vis[i, j] is True iff row i sees
    block key j.

    parent is None  -> chain / causal mask: j <= i.
    parent given    -> tree mask: j is i or an ancestor of i, where
                       parent[0] == -1 and 0 <= parent[i] < i for i >= 1.
    """
    vis = np.zeros((n, n), dtype=bool)
    if parent is None:
        for i in range(n):
            vis[i, : i + 1] = True
        return vis
    parent = [int(p) for p in parent]
    if len(parent) != n:
        raise ValueError("parent array must have one entry per block row")
    if n > 0 and parent[0] != -1:
        raise ValueError("node 0 is the root and must have parent -1")
    for i in range(1, n):
        if not (0 <= parent[i] < i):
            raise ValueError("parent[%d]=%d is not an earlier node" % (i, parent[i]))
    for i in range(n):
        j = i
        while j != -1:
            vis[i, j] = True
            j = parent[j]
    return vis


def attn_keys_ref(q_rows, keys, values, visible, sm_scale):
    """Softmax attention of R query rows over K keys, restricted by a
    visibility mask.

    q_rows [R, d], keys [K, d], values [K, d] (float64), visible [R, K] bool.
    Returns O [R, d] and LSE [R] (natural log).  A row with no visible key
    gets LSE = -inf and O = 0.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    R = q_rows.shape[0]
    d = values.shape[1] if values.ndim == 2 else q_rows.shape[1]
    out = np.zeros((R, d), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    if keys.shape[0] == 0 or R == 0:
        return out, lse
    scores = sm_scale * (q_rows @ keys.T)
    scores = np.where(visible, scores, -np.inf)
    m = scores.max(axis=1)
    has = np.isfinite(m)
    if not has.any():
        return out, lse
    m_safe = np.where(has, m, 0.0)
    e = np.exp(scores - m_safe[:, None])  # exp(-inf) = 0 for hidden keys
    total = e.sum(axis=1)
    lse = np.where(has, m_safe + np.log(np.where(has, total, 1.0)), -np.inf)
    w = np.where(has[:, None], e / np.where(has, total, 1.0)[:, None], 0.0)
    out = w @ values
    return out, lse


def _group_ref(q_bits, k_bits, v_bits, kb_bits, vb_bits, L, vis_blk, sm_scale):
    """All query heads of one (sequence, kv-head) group.

    q_bits [G, n, d]; k_bits/v_bits [>=L, d] (prefix); kb_bits/vb_bits [n, d].
    Returns O [G, n, d], LSE [G, n].
    """
    G, n, d = q_bits.shape
    keys = np.concatenate([bf16_bits_to_f64(k_bits[:L]), bf16_bits_to_f64(kb_bits)], axis=0)
    vals = np.concatenate([bf16_bits_to_f64(v_bits[:L]), bf16_bits_to_f64(vb_bits)], axis=0)
    visible = np.concatenate([np.ones((n, L), dtype=bool), vis_blk], axis=1)
    visible = np.tile(visible, (G, 1))
    q = bf16_bits_to_f64(q_bits).reshape(G * n, d)
    o, lse = attn_keys_ref(q, keys, vals, visible, sm_scale)
    return o.reshape(G, n, d), lse.reshape(G, n)


def attn_ref(q, k_cache, v_cache, k_blk, v_blk, seq_lens, parent=None, sm_scale=1.0,
             pairs=None):
    """Verify attention over the history cache plus the masked draft block.

    q        uint16 (bf16 bits) [B, Hq, n, d]
    k_cache  uint16 [B, Hkv, L_max, d];  v_cache likewise
    k_blk    uint16 [B, Hkv, n, d];      v_blk likewise
    seq_lens int [B], 0 <= seq_lens[b] <= L_max: history length of sequence b
    parent   None (causal chain) or int [n] parent array (tree)
    pairs    None -> every (b, h); else a list of (b, h) query heads to compute

    Returns (O, LSE): float64 [B, Hq, n, d] and [B, Hq, n] when pairs is None,
    else [len(pairs), n, d] and [len(pairs), n] in the order given.
    """
    B, Hq, n, d = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    vis_blk = block_visibility(n, parent)
    if pairs is None:
        O = np.zeros((B, Hq, n, d))
        LSE = np.zeros((B, Hq, n))
        for b in range(B):
            L = int(seq_lens[b])
            for g in range(Hkv):
                o, lse = _group_ref(q[b, g * G:(g + 1) * G], k_cache[b, g], v_cache[b, g],
                                    k_blk[b, g], v_blk[b, g], L, vis_blk, sm_scale)
                O[b, g * G:(g + 1) * G] = o
                LSE[b, g * G:(g + 1) * G] = lse
        return O, LSE
    O = np.zeros((len(pairs), n, d))
    LSE = np.zeros((len(pairs), n))
    for idx, (b, h) in enumerate(pairs):
        g = h // G
        L = int(seq_lens[b])
        o, lse = _group_ref(q[b, h:h + 1], k_cache[b, g], v_cache[b, g],
                            k_blk[b, g], v_blk[b, g], L, vis_blk, sm_scale)
        O[idx] = o[0]
        LSE[idx] = lse[0]
    return O, LSE


def lse_merge_ref(parts):
    """Merge partial softmax-attention results by log-sum-exp.

    parts: sequence of (O_k [..., d], LSE_k [...]) where O_k is normalised
    over its own key subset and LSE_k = log sum exp of its scores (-inf for
    an empty subset).  With M = max_k LSE_k and a_k = exp(LSE_k - M):
        O = sum_k a_k O_k / sum_k a_k,   LSE = M + log sum_k a_k.
    If every part is empty the result is O = 0, LSE = -inf.
    """
    Os = [np.asarray(o, dtype=np.float64) for o, _ in parts]
    Ls = [np.asarray(l, dtype=np.float64) for _, l in parts]
    M = np.max(np.stack(Ls), axis=0)
    has = np.isfinite(M)
    M_safe = np.where(has, M, 0.0)
    a = [np.where(np.isfinite(l), np.exp(l - M_safe), 0.0) for l in Ls]
    denom = np.sum(np.stack(a), axis=0)
    num = np.sum(np.stack([ak[..., None] * o for ak, o in zip(a, Os)]), axis=0)
    O = np.where(has[..., None], num / np.where(has, denom, 1.0)[..., None], 0.0)
    LSE = np.where(has, M_safe + np.log(np.where(has, denom, 1.0)), -np.inf)
    return O, LSE
