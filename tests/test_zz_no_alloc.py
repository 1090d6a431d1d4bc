"""rapid_accept_noalloc (static per-device scratch) against rapid_accept_ex
(caller's workspace) through the C ABI: the same kernels on the same inputs,
so every output must be bit-identical, on two calls in a row, the second
with a smaller input."""

import sys

import numpy as np
import pytest
import torch

from workloads import config_vocab, make_vocab
from speculative_decoding_verify_split_amd import rapid_verify as rv
from speculative_decoding_verify_split_amd.step import VerifyStep

pytestmark = pytest.mark.gpu


def _announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def _both(vi, flags):
    st = VerifyStep(None, vi, want_ratio=True, want_p_hat=True, flags=flags)
    st.accept()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (st.n_accept, st.out_tokens, st.ratio, st.p_hat)]
    for t in (st.n_accept, st.out_tokens, st.ratio, st.p_hat):
        t.fill_(-3)
    rv.rapid_accept_noalloc(st.z, st.y, st.draft, st.r, st.u, st.T, st.eta, flags, st.n_accept,
                            st.out_tokens, st.ratio, st.p_hat)
    torch.cuda.synchronize()
    got = (st.n_accept, st.out_tokens, st.ratio, st.p_hat)
    for name, a, b in zip(("n_accept", "out_tokens", "ratio", "p_hat"), ref, got):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    return ref


@pytest.mark.parametrize("flags", [0, rv.RV_ACCEPT_TAIL_PRESERVE | rv.RV_ACCEPT_PRINTED_RESIDUAL])
def test_noalloc_matches_workspace_call_twice(flags):
    _announce("rapid_accept_noalloc B=2 V=128256 gamma=10, then B=1 V=32000 gamma=4, flags=%d"
              % flags)
    big = config_vocab("llama8b", eta=0.5, B_override=2)
    small = make_vocab(61, B=1, gamma=4, V=32000, z_sigma=3.0, noise=1.0, T=1.0, eta=0.5)
    r1 = _both(big, flags)
    r2 = _both(small, flags)
    assert (r1[0] >= 0).all() and (r2[0] >= 0).all()


def test_noalloc_rejects_shapes_beyond_its_scratch():
    assert rv.rapid_accept_workspace_size(64, 63, 1 << 22) > (4 << 20)
    P = 256  # aligned placeholder; the size check comes before any pointer use
    st = rv.load_library().rapid_accept_noalloc(P, P, P, P, P, 64, 63, 1 << 22, 1.0, 0.5, 0, P, P,
                                                None, None, None)
    assert st == 5, rv.rv_status_string(st)  # RV_ERR_WORKSPACE
