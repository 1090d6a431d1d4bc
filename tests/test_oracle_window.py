"""Pins for the sliding-window (+ sink) attention oracle (CPU only).

The oracle's slot formula is checked against a ring filled position by
position; its visibility rule against a brute-force set; its attention
against a pure-Python softmax over the simulated ring and against closed
forms (window 1 is the token itself; a window covering everything with no
sink is causal attention)."""

import math

import numpy as np
import pytest

from oracle import attn_keys_ref, bf16_bits_to_f64, ring_slot, window_attn_ref, window_positions
from workloads import make_window


def _simulate_ring(last, cap, sink):
    """Write positions 0..last into a ring one by one: the first `sink`
    positions take slots 0..sink-1 for good, later ones take the next slot of
    the circular part [sink, cap), wrapping.  Returns (slot of each position,
    resident position of each slot or -1)."""
    slot_of, resident = [], [-1] * cap
    nxt = sink
    for p in range(last + 1):
        if p < sink:
            s = p
        else:
            s = nxt
            nxt = nxt + 1 if nxt + 1 < cap else sink
        slot_of.append(s)
        resident[s] = p
    return slot_of, resident


@pytest.mark.parametrize("cap,sink", [(9, 0), (9, 4), (16, 4), (516, 4), (5, 4)])
def test_slot_formula_matches_a_ring_filled_in_order(cap, sink):
    slot_of, _ = _simulate_ring(3000, cap, sink)
    assert [ring_slot(p, cap, sink) for p in range(3001)] == slot_of


def test_window_positions_bruteforce():
    rng = np.random.default_rng(0)
    for _ in range(500):
        P = int(rng.integers(0, 300))
        sink = int(rng.integers(0, 6))
        window = int(rng.integers(1, 80))
        brute = [p for p in range(P + 1) if p < sink or P - p < window]
        assert window_positions(P, sink, window) == brute


@pytest.mark.parametrize("n", [1, 3, 8])
def test_capacity_rule_keeps_every_visible_position_resident(n):
    """cap - sink = window + n - 1 suffices for n consecutive rows and is
    tight: one slot fewer loses a visible position."""
    sink, window = 4, 12
    for cap, ok in ((sink + window + n - 1, True), (sink + window + n - 2, False)):
        lost = False
        for P0 in range(0, 80):
            _, resident = _simulate_ring(P0 + n - 1, cap, sink)
            for i in range(n):
                for p in window_positions(P0 + i, sink, window):
                    if resident[ring_slot(p, cap, sink)] != p:
                        lost = True
        assert lost != ok


def _python_window_attention(qv, kring, vring, P, last, cap, sink, window, scale):
    """Pure-Python softmax over the slots whose resident position (from the
    simulated ring) is visible to the row at position P."""
    _, resident = _simulate_ring(last, cap, sink)
    vis = [s for s in range(cap)
           if resident[s] >= 0 and resident[s] <= P
           and (resident[s] < sink or P - resident[s] < window)]
    scores = [scale * sum(a * b for a, b in zip(qv, kring[s])) for s in vis]
    m = max(scores)
    w = [math.exp(x - m) for x in scores]
    tot = sum(w)
    out = [sum(wi * vring[s][c] for wi, s in zip(w, vis)) / tot for c in range(len(qv))]
    return out, m + math.log(tot)


@pytest.mark.parametrize("pos,n,cap,sink,window", [(0, 1, 8, 4, 4), (3, 2, 9, 4, 4),
                                                    (57, 3, 14, 4, 8), (200, 4, 13, 0, 10),
                                                    (41, 1, 6, 2, 4)])
def test_against_python_softmax_on_a_simulated_ring(pos, n, cap, sink, window):
    wi = make_window(11 + pos, B=2, Hq=4, Hkv=2, d=8, n=n, pos=[pos, pos + 5], cap=cap,
                     sink=sink, window=window)
    O, L = window_attn_ref(wi.q, wi.k_ring, wi.v_ring, wi.pos, cap, sink, window, 0.7)
    for b in range(2):
        for h in range(4):
            kr = bf16_bits_to_f64(wi.k_ring[b, h // 2]).tolist()
            vr = bf16_bits_to_f64(wi.v_ring[b, h // 2]).tolist()
            last = int(wi.pos[b]) + n - 1
            for i in range(n):
                qv = bf16_bits_to_f64(wi.q[b, h, i]).tolist()
                o, l = _python_window_attention(qv, kr, vr, int(wi.pos[b]) + i, last, cap, sink,
                                                window, 0.7)
                np.testing.assert_allclose(O[b, h, i], o, rtol=1e-12, atol=1e-12)
                assert abs(L[b, h, i] - l) < 1e-12


def test_window_of_one_is_the_token_itself():
    wi = make_window(5, B=1, Hq=2, Hkv=1, d=16, n=3, pos=[100], cap=4, sink=0, window=1)
    O, L = window_attn_ref(wi.q, wi.k_ring, wi.v_ring, wi.pos, 4, 0, 1, 1.3)
    for i in range(3):
        s = ring_slot(100 + i, 4, 0)
        np.testing.assert_array_equal(O[0, :, i], np.stack([bf16_bits_to_f64(wi.v_ring[0, 0, s])] * 2))
        for h in range(2):
            expect = 1.3 * float(bf16_bits_to_f64(wi.q[0, h, i]) @ bf16_bits_to_f64(wi.k_ring[0, 0, s]))
            assert abs(L[0, h, i] - expect) < 1e-12


def test_unbounded_window_without_sink_is_causal_attention():
    """No wrap, window past the start, no sink: causal attention over the
    cache in position order (attn_keys_ref with a lower-triangular mask)."""
    n, pos = 5, 20
    wi = make_window(6, B=1, Hq=4, Hkv=2, d=16, n=n, pos=[pos], cap=64, sink=0, window=1000)
    O, L = window_attn_ref(wi.q, wi.k_ring, wi.v_ring, wi.pos, 64, 0, 1000, 1.0)
    last = pos + n - 1
    vis = np.arange(last + 1)[None, :] <= (pos + np.arange(n))[:, None]
    for h in range(4):
        o, l = attn_keys_ref(bf16_bits_to_f64(wi.q[0, h]), bf16_bits_to_f64(wi.k_ring[0, h // 2, :last + 1]),
                             bf16_bits_to_f64(wi.v_ring[0, h // 2, :last + 1]), vis, 1.0)
        np.testing.assert_allclose(O[0, h], o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L[0, h], l, rtol=1e-12, atol=1e-13)


def test_sink_matters_only_past_the_window():
    kw = dict(B=1, Hq=2, Hkv=1, d=16, n=1, cap=40, window=16)
    for pos, same in ((10, True), (15, True), (30, False)):
        a = make_window(7, pos=[pos], sink=4, **kw)
        O4, _ = window_attn_ref(a.q, a.k_ring, a.v_ring, a.pos, 40, 4, 16)
        O0, _ = window_attn_ref(a.q, a.k_ring, a.v_ring, a.pos, 40, 0, 16)
        if pos < 36:  # below the wrap of either ring layout, slots hold the same positions
            assert np.allclose(O4, O0) == same
