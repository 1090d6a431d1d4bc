"""Seeded synthetic inputs for the verify step.

This module is shared by the oracle-side tests and the GPU path; it holds
none of the verify step's arithmetic.  It only draws random tensors with the
shapes and distributions of the workloads and rounds them to the storage
types (bf16 as raw uint16 bit patterns, fp32, int32).

Recipe (every tensor has its own child stream of ``SeedSequence(seed)``;
large tensors are further split into fixed 2**22-element chunks, each with
its own grandchild stream, so the bytes do not depend on thread count):

* K/V cache, block K/V: N(0, 1) in fp32, rounded to bf16 (nearest-even).
* Q: N(0, 1) / sqrt(d) in fp32, rounded to bf16; the attention scale is
  therefore 1.0 (the 1/sqrt(d) is folded into Q).
* history lengths: fixed, or uniform integers in [lo, hi] (ragged batch).
* tree: node 0 is the root; nodes 1..D form the chain parent[t] = t-1; every
  later node picks its parent uniformly among earlier nodes of depth <= D-1,
  so no node is deeper than D and node D stays a leaf.
* target logits z ~ N(0, z_sigma^2); draft logits y = z + N(0, noise^2),
  fp32.
* draft tokens: drawn from the drafter's tempered distribution with the
  Gumbel-max trick, x = argmax_v (y_v / T + g_v), g_v ~ Gumbel(0, 1), in
  float64; this samples the categorical law of y/T without forming it.
* uniforms r, u: (uint32 >> 8) * 2**-24, exact fp32 values in [0, 1).
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

CHUNK = 1 << 22

# The five workloads.  L is the history length (or (lo, hi) for a ragged
# batch); gamma is the number of draft tokens in the chain; a tree workload
# has n_nodes block rows and runs acceptance on its chain of depth tree_depth.
CONFIGS = {
    "tiny": dict(desc="tiny chain verify: 8/2 heads, d=64, 4096-token cache, gamma=4",
                 B=1, Hq=8, Hkv=2, d=64, L=4096, gamma=4, V=32000,
                 z_sigma=3.0, noise=1.0, T=1.0, etas=(0.5,), seed=100),
    "llama8b": dict(desc="LLaMA-3.1-8B-shaped verify layer: 32/8 heads, d=128, "
                         "128K cache, gamma=10, vocab 128256",
                    B=1, Hq=32, Hkv=8, d=128, L=131072, gamma=10, V=128256,
                    z_sigma=3.0, noise=1.0, T=1.0, etas=(0.0, 0.5, 2.0), seed=200),
    "llama70b": dict(desc="LLaMA-3.1-70B-shaped verify layer: 64/8 heads, d=128, "
                          "120K cache, gamma=10, T=0.7",
                     B=1, Hq=64, Hkv=8, d=128, L=122880, gamma=10, V=128256,
                     z_sigma=3.0, noise=1.0, T=0.7, etas=(1.0,), seed=300),
    "qwen7b_ragged": dict(desc="Qwen2.5-7B-shaped ragged batch: 28/4 heads, d=128, "
                               "8 sequences with 32K..128K caches, gamma=10",
                          B=8, Hq=28, Hkv=4, d=128, L=(32768, 131072), gamma=10,
                          V=152064, z_sigma=3.0, noise=0.5, T=1.0, etas=(0.5,), seed=400),
    # One GPU's share of the 8B-shaped layer under 8-way head parallelism
    # (one kv head and its 4 query heads per GPU); the acceptance pass stays
    # whole, as every rank needs the same decision.
    "llama8b_tp8": dict(desc="one GPU's share of the LLaMA-3.1-8B-shaped layer under 8-way "
                             "head parallelism: 4/1 heads, d=128, 128K cache, gamma=10, "
                             "vocab 128256",
                        B=1, Hq=4, Hkv=1, d=128, L=131072, gamma=10, V=128256,
                        z_sigma=3.0, noise=1.0, T=1.0, etas=(0.5,), seed=210),
    "tree1m": dict(desc="tree verify at 1M tokens: 32/8 heads, d=128, 32-node tree "
                        "of depth <= 6, chain 0..6",
                   B=1, Hq=32, Hkv=8, d=128, L=1048576, gamma=6, V=128256,
                   n_nodes=32, tree_depth=6, z_sigma=3.0, noise=1.0, T=1.0,
                   etas=(0.5,), seed=500),
}

# LongSpec drafter workloads: the drafter's decode step, one query row per
# head cross-attending over the target's cache, and its sliding-window
# self-attention with sink anchors over its own ring cache of sink + window
# slots, for the token at position L.
DRAFTER_CONFIGS = {
    "drafter8b": dict(desc="LongSpec drafter decode step at the LLaMA-3.1-8B shape: one query "
                           "row per head over the target's 128K cache (32/8 heads, d=128) + "
                           "512-token sliding window with 4 anchors",
                      B=1, Hq=32, Hkv=8, d=128, L=131072, window=512, sink=4, seed=600),
}

# child-stream slots of SeedSequence(seed).spawn(...)
_S_LENS, _S_Q, _S_K, _S_V, _S_KB, _S_VB, _S_TREE, _S_Z, _S_Y, _S_G, _S_R, _S_U = range(12)
_N_SLOTS = 12


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite normals, so NaN handling is not needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).copy()
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    b += np.uint32(0x7FFF)
    b += t
    b >>= np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to fp32 (exact).  Used to build device tensors."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_normal_bf16(out_flat, seed_seq, scale, threads):
    """Fill out_flat (uint16, contiguous) with bf16(N(0,1) * scale), chunked."""
    n = out_flat.size
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = seed_seq.spawn(nchunks)
    sc = np.float32(scale)

    def work(ci):
        lo = ci * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[ci]))
        buf = np.empty(hi - lo, dtype=np.float32)
        g.standard_normal(out=buf, dtype=np.float32)
        if scale != 1.0:
            buf *= sc
        b = buf.view(np.uint32)
        t = b >> np.uint32(16)
        t &= np.uint32(1)
        b += np.uint32(0x7FFF)
        b += t
        b >>= np.uint32(16)
        out_flat[lo:hi] = b
        return None

    if nchunks == 1 or threads == 1:
        for ci in range(nchunks):
            work(ci)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(nchunks)))


def tree_parents(seed_seq, n_nodes, depth):
    """Random draft tree: chain 0..depth, other nodes hang off nodes of depth <= depth-1."""
    g = np.random.Generator(np.random.PCG64(seed_seq))
    parent = np.full(n_nodes, -1, dtype=np.int32)
    dep = np.zeros(n_nodes, dtype=np.int64)
    for t in range(1, min(depth, n_nodes - 1) + 1):
        parent[t] = t - 1
        dep[t] = t
    for t in range(depth + 1, n_nodes):
        cand = [j for j in range(t) if dep[j] <= depth - 1]
        j = cand[int(g.integers(0, len(cand)))]
        parent[t] = j
        dep[t] = dep[j] + 1
    return parent


@dataclass
class AttnInputs:
    q: np.ndarray          # uint16 bf16 bits [B, Hq, n, d]
    k_cache: np.ndarray    # uint16 [B, Hkv, L_max, d]
    v_cache: np.ndarray    # uint16 [B, Hkv, L_max, d]
    k_blk: np.ndarray      # uint16 [B, Hkv, n, d]
    v_blk: np.ndarray      # uint16 [B, Hkv, n, d]
    seq_lens: np.ndarray   # int32 [B]
    parent: Optional[np.ndarray]  # int32 [n] or None (causal chain)
    sm_scale: float = 1.0

    @property
    def shape(self):
        B, Hq, n, d = self.q.shape
        return dict(B=B, Hq=Hq, Hkv=self.k_cache.shape[1], n=n, d=d,
                    L_max=self.k_cache.shape[2])


@dataclass
class VocabInputs:
    z: np.ndarray       # fp32 [B, gamma+1, V]
    y: np.ndarray       # fp32 [B, gamma, V]
    draft: np.ndarray   # int32 [B, gamma]
    r: np.ndarray       # fp32 [B, gamma]
    u: np.ndarray       # fp32 [B, gamma+1]
    T: float
    eta: float


def make_attention(seed, B, Hq, Hkv, d, n, L, L_max=None, parent=None,
                   pad_bits=0, threads=None):
    """Attention inputs.  L is an int (every sequence), a list of per-sequence
    lengths, or a (lo, hi) tuple drawn uniformly per sequence."""
    threads = threads or _threads()
    ss = np.random.SeedSequence(seed).spawn(_N_SLOTS)
    if isinstance(L, tuple):
        g = np.random.Generator(np.random.PCG64(ss[_S_LENS]))
        seq_lens = g.integers(L[0], L[1] + 1, size=B).astype(np.int32)
    elif isinstance(L, (list, np.ndarray)):
        seq_lens = np.asarray(L, dtype=np.int32)
        assert seq_lens.shape == (B,)
    else:
        seq_lens = np.full(B, int(L), dtype=np.int32)
    if L_max is None:
        L_max = int(seq_lens.max()) if B > 0 else 0
    assert int(seq_lens.max(initial=0)) <= L_max
    q = np.empty((B, Hq, n, d), dtype=np.uint16)
    _fill_normal_bf16(q.reshape(-1), ss[_S_Q], 1.0 / math.sqrt(d), threads)
    kb = np.empty((B, Hkv, n, d), dtype=np.uint16)
    vb = np.empty((B, Hkv, n, d), dtype=np.uint16)
    _fill_normal_bf16(kb.reshape(-1), ss[_S_KB], 1.0, threads)
    _fill_normal_bf16(vb.reshape(-1), ss[_S_VB], 1.0, threads)
    k = np.empty((B, Hkv, L_max, d), dtype=np.uint16)
    v = np.empty((B, Hkv, L_max, d), dtype=np.uint16)
    kseq = ss[_S_K].spawn(B * Hkv)
    vseq = ss[_S_V].spawn(B * Hkv)
    for b in range(B):
        Lb = int(seq_lens[b])
        for h in range(Hkv):
            _fill_normal_bf16(k[b, h, :Lb].reshape(-1), kseq[b * Hkv + h], 1.0, threads)
            _fill_normal_bf16(v[b, h, :Lb].reshape(-1), vseq[b * Hkv + h], 1.0, threads)
            if Lb < L_max:
                k[b, h, Lb:] = pad_bits
                v[b, h, Lb:] = pad_bits
    return AttnInputs(q=q, k_cache=k, v_cache=v, k_blk=kb, v_blk=vb,
                      seq_lens=seq_lens, parent=parent, sm_scale=1.0)


@dataclass
class WindowInputs:
    q: np.ndarray       # uint16 bf16 bits [B, Hq, n, d]; row i is position pos[b] + i
    k_ring: np.ndarray  # uint16 [B, Hkv, cap, d]
    v_ring: np.ndarray  # uint16 [B, Hkv, cap, d]
    pos: np.ndarray     # int32 [B]
    cap: int
    sink: int
    window: int
    sm_scale: float = 1.0


def make_window(seed, B, Hq, Hkv, d, n, pos, cap, sink, window, pad_bits=0x7FC0, threads=None):
    """Drafter self-attention inputs: queries of n consecutive positions and a
    ring cache of cap slots.  Positions below cap occupy slots 0..cap-1 in
    order, so while the last query position is below cap - 1 the slots past
    it have never been written and hold pad_bits (a NaN by default: any read
    of them shows in the result); once the ring has wrapped every slot holds
    data."""
    threads = threads or _threads()
    ss = np.random.SeedSequence(seed).spawn(_N_SLOTS)
    pos = np.broadcast_to(np.asarray(pos, dtype=np.int32), (B,)).copy()
    q = np.empty((B, Hq, n, d), dtype=np.uint16)
    _fill_normal_bf16(q.reshape(-1), ss[_S_Q], 1.0 / math.sqrt(d), threads)
    k = np.empty((B, Hkv, cap, d), dtype=np.uint16)
    v = np.empty((B, Hkv, cap, d), dtype=np.uint16)
    _fill_normal_bf16(k.reshape(-1), ss[_S_K], 1.0, threads)
    _fill_normal_bf16(v.reshape(-1), ss[_S_V], 1.0, threads)
    for b in range(B):
        written = min(cap, int(pos[b]) + n)
        k[b, :, written:] = pad_bits
        v[b, :, written:] = pad_bits
    return WindowInputs(q=q, k_ring=k, v_ring=v, pos=pos, cap=int(cap), sink=int(sink),
                        window=int(window))


def _uniform_f32(seed_seq, shape):
    g = np.random.Generator(np.random.PCG64(seed_seq))
    bits = g.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)
    return ((bits >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24))


def make_vocab(seed, B, gamma, V, z_sigma, noise, T, eta):
    """Vocabulary-pass inputs for B sequences and gamma drafts."""
    ss = np.random.SeedSequence(seed).spawn(_N_SLOTS)
    gz = np.random.Generator(np.random.PCG64(ss[_S_Z]))
    gy = np.random.Generator(np.random.PCG64(ss[_S_Y]))
    gg = np.random.Generator(np.random.PCG64(ss[_S_G]))
    z = gz.standard_normal((B, gamma + 1, V), dtype=np.float32)
    z *= np.float32(z_sigma)
    y = gy.standard_normal((B, gamma, V), dtype=np.float32)
    y *= np.float32(noise)
    y += z[:, :gamma, :]
    draft = np.empty((B, gamma), dtype=np.int32)
    for b in range(B):
        for t in range(gamma):
            gum = gg.gumbel(size=V)
            draft[b, t] = int(np.argmax(y[b, t].astype(np.float64) / T + gum))
    r = _uniform_f32(ss[_S_R], (B, gamma))
    u = _uniform_f32(ss[_S_U], (B, gamma + 1))
    return VocabInputs(z=z, y=y, draft=draft, r=r, u=u, T=float(T), eta=float(eta))


@dataclass
class TreeVocabInputs:
    z: np.ndarray          # fp32 [B, n, V] target logits after each node
    y: np.ndarray          # fp32 [B, n, V] drafter logits after each node
    parent: np.ndarray     # int32 [n]
    tokens: np.ndarray     # int32 [B, n] draft token of each node (0 at the root)
    r: np.ndarray          # fp32 [B, n] acceptance uniforms
    u: np.ndarray          # fp32 [B, n] sampling uniforms
    T: float
    eta: float


def make_tree_vocab(seed, B, parent, V, z_sigma, noise, T, eta):
    """Inputs of an acceptance over a draft tree: per node, z ~ N(0, z_sigma^2)
    and y = z + N(0, noise^2); the token of node c is drawn from the drafter
    distribution of its parent, softmax(y_parent / T), by the Gumbel-max
    trick, so siblings are independent draws."""
    parent = np.asarray(parent, dtype=np.int32)
    n = len(parent)
    ss = np.random.SeedSequence(seed).spawn(_N_SLOTS)
    gz = np.random.Generator(np.random.PCG64(ss[_S_Z]))
    gy = np.random.Generator(np.random.PCG64(ss[_S_Y]))
    gg = np.random.Generator(np.random.PCG64(ss[_S_G]))
    z = gz.standard_normal((B, n, V), dtype=np.float32)
    z *= np.float32(z_sigma)
    y = gy.standard_normal((B, n, V), dtype=np.float32)
    y *= np.float32(noise)
    y += z
    tokens = np.zeros((B, n), dtype=np.int32)
    for b in range(B):
        for c in range(1, n):
            gum = gg.gumbel(size=V)
            tokens[b, c] = int(np.argmax(y[b, parent[c]].astype(np.float64) / T + gum))
    r = _uniform_f32(ss[_S_R], (B, n))
    u = _uniform_f32(ss[_S_U], (B, n))
    return TreeVocabInputs(z=z, y=y, parent=parent, tokens=tokens, r=r, u=u, T=float(T),
                           eta=float(eta))


def config_tree_vocab(name, B_override=None, V_override=None, eta=None):
    """Tree acceptance inputs on a tree workload's own tree (the tree1m
    workload's 32-node tree and vocabulary)."""
    c = CONFIGS[name]
    ss = np.random.SeedSequence(c["seed"]).spawn(_N_SLOTS)
    parent = tree_parents(ss[_S_TREE], c["n_nodes"], c["tree_depth"])
    return make_tree_vocab(c["seed"] + 1, B_override or c["B"], parent, V_override or c["V"],
                           c["z_sigma"], c["noise"], c["T"],
                           c["etas"][0] if eta is None else eta)


def config_attention(name, L_override=None, B_override=None, pad_bits=0, threads=None):
    """Attention inputs of a named workload (optionally with a shorter history)."""
    c = CONFIGS[name]
    B = B_override or c["B"]
    L = c["L"] if L_override is None else L_override
    if "n_nodes" in c:
        ss = np.random.SeedSequence(c["seed"]).spawn(_N_SLOTS)
        parent = tree_parents(ss[_S_TREE], c["n_nodes"], c["tree_depth"])
        n = c["n_nodes"]
    else:
        parent = None
        n = c["gamma"] + 1
    return make_attention(c["seed"], B, c["Hq"], c["Hkv"], c["d"], n, L,
                          parent=parent, pad_bits=pad_bits, threads=threads)


def config_vocab(name, eta=None, B_override=None, V_override=None):
    """Vocabulary-pass inputs of a named workload."""
    c = CONFIGS[name]
    eta = c["etas"][0] if eta is None else eta
    B = B_override or c["B"]
    V = V_override or c["V"]
    return make_vocab(c["seed"], B, c["gamma"], V, c["z_sigma"], c["noise"], c["T"], eta)


def config_drafter(name, threads=None):
    """(cross-attention inputs with n = 1, window inputs) of a drafter workload.
    The cross-attention inputs' block tensors are unused (no draft block)."""
    c = DRAFTER_CONFIGS[name]
    cross = make_attention(c["seed"], c["B"], c["Hq"], c["Hkv"], c["d"], 1, c["L"],
                           threads=threads)
    win = make_window(c["seed"] + 1, c["B"], c["Hq"], c["Hkv"], c["d"], 1, pos=c["L"],
                      cap=c["sink"] + c["window"], sink=c["sink"], window=c["window"],
                      threads=threads)
    return cross, win


# Whole-model verify step: every attention layer of the 8B-shaped model at
# 128K tokens (32 layers, 17.2 GB of bf16 K/V), then one acceptance pass.
MODEL_CONFIGS = {
    "llama8b_model": dict(desc="LLaMA-3.1-8B-shaped model verify step: 32 attention layers "
                               "(32/8 heads, d=128, 128K cache, gamma=10) + one acceptance "
                               "pass over vocab 128256",
                          layers=32, layer_config="llama8b", seed=700),
}


def make_layer_device(seed, layer, B, Hq, Hkv, d, n, L, device="cuda"):
    """One layer's attention inputs generated on the device (the host cannot
    hold a 32-layer cache quickly): a torch generator seeded with
    (seed, layer) draws N(0, 1) fp32 per tensor in a fixed order, rounded to
    bf16 (nearest-even); Q is scaled by 1/sqrt(d) before rounding, so the
    attention scale is 1.  Returns (q, k_cache, v_cache, k_blk, v_blk) as
    torch bf16 tensors."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(layer))

    def draw(shape, scale=1.0):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x *= scale
        return x.to(torch.bfloat16)

    q = draw((B, Hq, n, d), 1.0 / math.sqrt(d))
    kb = draw((B, Hkv, n, d))
    vb = draw((B, Hkv, n, d))
    k = draw((B, Hkv, L, d))
    v = draw((B, Hkv, L, d))
    return q, k, v, kb, vb
