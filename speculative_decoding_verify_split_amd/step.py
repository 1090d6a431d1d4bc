"""One verify step on the GPU: device buffers plus the four library calls.

Plumbing only: torch allocates device memory and supplies the stream; every
arithmetic step runs inside librapid_verify.so.
"""

import numpy as np

from . import rapid_verify as rv


def bf16_to_device(bits, device="cuda"):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor on the GPU."""
    import torch
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def to_device(arr, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


class VerifyStep:
    """Device-resident inputs and outputs of one verify step.

    attn: a workloads.AttnInputs-like object (numpy uint16 bf16 bits), or
          None for the vocabulary pass only;
    vocab: a workloads.VocabInputs-like object, or None for attention only.
    split: (split_len, num_splits), or None to plan it from the batch's host
           lengths (rv_prefix_balanced_split; for one sequence this is the
           same as rv_prefix_default_split).
    """

    def __init__(self, attn, vocab=None, split=None, want_ratio=True, want_p_hat=False,
                 device="cuda", flags=0):
        import torch
        self.device = device
        self.attn = attn
        f32 = torch.float32
        if attn is not None:
            B, Hq, n, d = attn.q.shape
            Hkv, L_max = attn.k_cache.shape[1], attn.k_cache.shape[2]
            self.B, self.Hq, self.Hkv, self.n, self.d, self.L_max = B, Hq, Hkv, n, d, L_max
            self.max_seq_len = int(np.max(attn.seq_lens)) if B else 0
            self.parent = None if attn.parent is None else [int(x) for x in attn.parent]
            self.sm_scale = float(attn.sm_scale)
            self.q = bf16_to_device(attn.q, device)
            self.k_cache = bf16_to_device(attn.k_cache, device)
            self.v_cache = bf16_to_device(attn.v_cache, device)
            self.k_blk = bf16_to_device(attn.k_blk, device)
            self.v_blk = bf16_to_device(attn.v_blk, device)
            self.seq_lens = to_device(attn.seq_lens.astype(np.int32), device)
            if split is None:
                split = rv.rv_prefix_balanced_split(attn.seq_lens, Hq, Hkv, n, d)
            self.split_len, self.num_splits = int(split[0]), int(split[1])
            S = self.num_splits
            self.o_part = torch.empty((B, Hq, n, S, d), dtype=f32, device=device)
            self.lse_part = torch.empty((B, Hq, n, S), dtype=f32, device=device)
            self.o_blk = torch.empty((B, Hq, n, d), dtype=f32, device=device)
            self.lse_blk = torch.empty((B, Hq, n), dtype=f32, device=device)
            self.out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device=device)
            self.lse_out = torch.empty((B, Hq, n), dtype=f32, device=device)
            # spec_attn_verify's sync words: zero once, left zero by every call
            self.sync = torch.zeros((rv.spec_attn_verify_sync_size(B, Hkv),), dtype=torch.uint8,
                                    device=device)
        self.vocab = vocab
        self.flags = int(flags)
        if vocab is not None:
            Bv, g1, V = vocab.z.shape
            self.gamma, self.V = g1 - 1, V
            self.T, self.eta = float(vocab.T), float(vocab.eta)
            self.z = to_device(vocab.z, device)
            self.y = to_device(vocab.y, device)
            self.draft = to_device(vocab.draft.astype(np.int32), device)
            self.r = to_device(vocab.r, device)
            self.u = to_device(vocab.u, device)
            self.n_accept = torch.empty((Bv,), dtype=torch.int32, device=device)
            self.out_tokens = torch.empty((Bv, g1), dtype=torch.int32, device=device)
            ws = rv.rapid_accept_workspace_size(Bv, self.gamma, V)
            self.workspace = torch.empty((ws,), dtype=torch.uint8, device=device)
            self.ratio = torch.empty((Bv, self.gamma), dtype=f32, device=device) if want_ratio else None
            self.p_hat = (torch.empty((Bv, self.gamma, V), dtype=f32, device=device)
                          if want_p_hat else None)

    def attention(self, k_cache=None, v_cache=None, stream=None, fused=False, block=True,
                  single=False, help_after_us=-1, events=(None, None)):
        """The attention calls; k_cache/v_cache override the resident cache
        (same shape), e.g. to rotate copies when timing.  fused: the block
        pass and the merge as one spec_attn_block_merge call (o_blk and
        lse_blk are then left untouched).  single: the whole attention as one
        spec_attn_verify call (events: its start/stop hipEvent_t handles).
        block=False: no draft block, the history partials are merged alone
        (a drafter's cross-attention)."""
        kc = self.k_cache if k_cache is None else k_cache
        vc = self.v_cache if v_cache is None else v_cache
        if single:
            rv.spec_attn_verify(self.q, kc, vc, self.seq_lens, self.max_seq_len, self.split_len,
                                self.num_splits, self.k_blk, self.v_blk, self.parent, self.o_part,
                                self.lse_part, self.sync, self.out, self.lse_out, self.sm_scale,
                                help_after_us, stream, events[0], events[1])
            return
        rv.spec_attn_prefix(self.q, kc, vc, self.seq_lens, self.max_seq_len, self.split_len,
                            self.num_splits, self.o_part, self.lse_part, self.sm_scale, stream)
        if not block:
            rv.lse_merge(self.o_part, self.lse_part, None, None, self.out, self.lse_out, stream)
            return
        if fused:
            rv.spec_attn_block_merge(self.q, self.k_blk, self.v_blk, self.parent, self.o_part,
                                     self.lse_part, self.out, self.lse_out, self.sm_scale, stream)
            return
        rv.spec_attn_block(self.q, self.k_blk, self.v_blk, self.parent, self.o_blk, self.lse_blk,
                           self.sm_scale, stream)
        rv.lse_merge(self.o_part, self.lse_part, self.o_blk, self.lse_blk, self.out, self.lse_out,
                     stream)

    def accept(self, z=None, y=None, stream=None):
        z = self.z if z is None else z
        y = self.y if y is None else y
        if self.flags:
            rv.rapid_accept_ex(z, y, self.draft, self.r, self.u, self.T, self.eta, self.flags,
                               self.n_accept, self.out_tokens, self.workspace, self.ratio,
                               self.p_hat, stream)
        else:
            rv.rapid_accept(z, y, self.draft, self.r, self.u, self.T, self.eta, self.n_accept,
                            self.out_tokens, self.workspace, self.ratio, self.p_hat, stream)

    def run(self, stream=None, fused=False, single=False):
        if self.attn is not None:
            self.attention(stream=stream, fused=fused, single=single)
        if self.vocab is not None:
            self.accept(stream=stream)


class WindowStep:
    """Device copies of a workloads.WindowInputs-like object and the output
    buffers of spec_attn_window."""

    def __init__(self, win, device="cuda"):
        import torch
        self.win = win
        B, Hq, n, d = win.q.shape
        self.q = bf16_to_device(win.q, device)
        self.k_ring = bf16_to_device(win.k_ring, device)
        self.v_ring = bf16_to_device(win.v_ring, device)
        self.pos = to_device(np.asarray(win.pos, dtype=np.int32), device)
        self.sink, self.window, self.sm_scale = int(win.sink), int(win.window), float(win.sm_scale)
        self.out = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device=device)
        self.lse_out = torch.empty((B, Hq, n), dtype=torch.float32, device=device)
        ws = rv.spec_attn_window_workspace_size(B, Hq, n, d, self.sink, self.window)
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=device)

    def run(self, stream=None):
        rv.spec_attn_window(self.q, self.k_ring, self.v_ring, self.pos, self.sink, self.window,
                            self.out, self.workspace, self.lse_out, self.sm_scale, stream)


class ModelStep:
    """Every attention layer of a model's verify step, then one acceptance
    pass.  layer_inputs: one (q, k_cache, v_cache, k_blk, v_blk) tuple of
    device bf16 tensors per layer, shaped as spec_attn_prefix and
    spec_attn_block take them, every layer's cache holding L history tokens
    per sequence.  The split partials are reused from layer to layer (stream
    order keeps each merge ahead of the next layer's history pass); each
    layer keeps its own output."""

    def __init__(self, layer_inputs, L, vocab=None, device="cuda"):
        import torch
        self.layer_inputs = list(layer_inputs)
        B, Hq, n, d = self.layer_inputs[0][0].shape
        Hkv = self.layer_inputs[0][1].shape[1]
        layers = len(self.layer_inputs)
        self.B, self.Hq, self.Hkv, self.d, self.n, self.L = B, Hq, Hkv, d, n, int(L)
        self.seq_lens = torch.full((B,), self.L, dtype=torch.int32, device=device)
        self.split_len, self.num_splits = rv.rv_prefix_default_split(self.L, B, Hq, Hkv, n, d)
        S = self.num_splits
        f32 = torch.float32
        self.o_part = torch.empty((B, Hq, n, S, d), dtype=f32, device=device)
        self.lse_part = torch.empty((B, Hq, n, S), dtype=f32, device=device)
        self.out = torch.empty((layers, B, Hq, n, d), dtype=torch.bfloat16, device=device)
        self.lse_out = torch.empty((layers, B, Hq, n), dtype=f32, device=device)
        self.vocab = VerifyStep(None, vocab, want_ratio=False, device=device) if vocab else None

    def attention(self, stream=None):
        for l, (q, k, v, kb, vb) in enumerate(self.layer_inputs):
            rv.spec_attn_prefix(q, k, v, self.seq_lens, self.L, self.split_len, self.num_splits,
                                self.o_part, self.lse_part, 1.0, stream)
            rv.spec_attn_block_merge(q, kb, vb, None, self.o_part, self.lse_part, self.out[l],
                                     self.lse_out[l], 1.0, stream)

    def run(self, stream=None):
        self.attention(stream)
        if self.vocab is not None:
            self.vocab.accept(stream=stream)
