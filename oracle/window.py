"""fp64 oracle for the drafter's sliding-window self-attention (test
infrastructure only).

Source: LongSpec summary (gist.science), section 2.1 "Memory-efficient
architecture": the drafter's self-attention layers attend only to a sliding
window of the most recent 512 tokens, so its own KV cache has constant size
(its cross-attention instead reads the target's cache, which is
``attention.attn_keys_ref`` over the history).  Section 2.2 keeps the first
4 tokens of a sequence as attention-sink anchors.

Readings where the page is silent (each restated where used):
* the window includes the query's own position: the row at position P sees
  positions P - window + 1 .. P; the first ``sink`` positions of the sequence
  are visible to every later row as well;
* the constant-size cache is a ring of ``cap`` slots: position p lives in
  slot p for p < sink and in slot sink + (p - sink) mod (cap - sink)
  otherwise, the caller having written every position up to the last query
  row's; cap - sink >= window + n - 1 keeps every visible position resident
  for a block of n consecutive query rows at positions pos, pos + 1, ...;
* query head h reads kv head h // G, G = H_q / H_kv, as in the verify
  attention.
"""

import numpy as np

from .attention import attn_keys_ref, bf16_bits_to_f64


def window_positions(P, sink, window):
    """Positions the row at position P sees, ascending: the sink positions
    below min(sink, P + 1), then max(sink, P - window + 1) .. P."""
    lo = max(sink, P - window + 1)
    return list(range(min(sink, P + 1))) + list(range(lo, P + 1))


def ring_slot(p, cap, sink):
    """Slot of position p in the drafter's ring cache."""
    return p if p < sink else sink + (p - sink) % (cap - sink)


def window_attn_ref(q, k_ring, v_ring, pos, cap, sink, window, sm_scale=1.0):
    """Sliding-window (+ sink) attention of n consecutive query rows.

    q       uint16 bf16 bits [B, Hq, n, d]; row i of sequence b is the token
            at position pos[b] + i
    k_ring, v_ring  uint16 bf16 bits [B, Hkv, cap, d]
    pos     int [B], position of each sequence's first query row
    Returns O [B, Hq, n, d] and LSE [B, Hq, n] (natural log), float64.
    """
    B, Hq, n, d = q.shape
    Hkv = k_ring.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, Hq, n, d))
    LSE = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i in range(n):
                P = int(pos[b]) + i
                slots = [ring_slot(p, cap, sink) for p in window_positions(P, sink, window)]
                keys = bf16_bits_to_f64(k_ring[b, kv, slots])
                vals = bf16_bits_to_f64(v_ring[b, kv, slots])
                qr = bf16_bits_to_f64(q[b, h, i])[None]
                o, l = attn_keys_ref(qr, keys, vals, np.ones((1, len(slots)), bool), sm_scale)
                O[b, h, i] = o[0]
                LSE[b, h, i] = l[0]
    return O, LSE
