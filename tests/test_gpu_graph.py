"""A verify step captured in a HIP graph replays to the eager result.

The library launches only kernels on the caller's stream (no memsets, no
allocation, no synchronisation), so a whole step can be captured.  Each
replay is checked bit for bit against an eager run, with eager work and
synchronisations between replays.
"""

import sys

import pytest
import torch

from speculative_decoding_verify_split_amd.step import VerifyStep
from workloads import config_vocab, make_attention

pytestmark = pytest.mark.gpu


def _outputs(st):
    return [t.clone() for t in (st.out.view(torch.int16), st.lse_out, st.o_part, st.lse_part,
                                 st.o_blk, st.lse_blk, st.n_accept, st.out_tokens, st.ratio)]


def test_graph_replay_matches_eager():
    print("[gpu-case] graph replay, tiny shapes", flush=True)
    sys.stdout.flush()
    ai = make_attention(61, 2, 8, 2, 64, 5, [3000, 1234])
    vi = config_vocab("tiny", B_override=2)
    st = VerifyStep(ai, vi)
    st.run()
    torch.cuda.synchronize()
    ref = _outputs(st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()

    for rep in range(4):
        # disturb every output, then replay and compare
        for t in (st.out, st.lse_out, st.o_part, st.lse_part, st.o_blk, st.lse_blk, st.ratio):
            t.fill_(float("nan"))
        st.n_accept.fill_(-7)
        st.out_tokens.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(st)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), "replay %d differs" % rep
        st.run()  # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(ref, _outputs(st)):
            assert torch.equal(a, b)


@pytest.mark.parametrize("single", [True, False], ids=["one-launch", "two-launches"])
def test_graph_replay_of_spec_attn_verify(single):
    """spec_attn_verify captured in a graph: the single launch (whose sync
    words each call leaves zero) and the two launches replay to the eager
    result, with eager calls between the replays."""
    from speculative_decoding_verify_split_amd import rapid_verify as rv
    # 8/2 heads, d = 64, n = 5 at 4096 tokens: 16 workgroups (one launch);
    # at 40960 tokens the default split gives too many for one launch
    L = 4096 if single else 40960
    ai = make_attention(62, 1, 8, 2, 64, 5, [L])
    st = VerifyStep(ai, None)
    assert rv.rv_verify_single_launch(1, 8, 2, 5, 64, st.num_splits) == single
    print("[gpu-case] graph replay of spec_attn_verify, %s" % ("one launch" if single else
                                                             "two launches"), flush=True)
    st.attention(single=True)
    torch.cuda.synchronize()
    ref = (st.out.view(torch.int16).clone(), st.lse_out.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.attention(single=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.attention(single=True)
    torch.cuda.synchronize()
    for rep in range(4):
        st.out.fill_(float("nan"))
        st.lse_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.int16), ref[0]), "replay %d differs" % rep
        assert torch.equal(st.lse_out, ref[1]), "replay %d differs" % rep
        assert not st.sync.any()
        st.attention(single=True)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.int16), ref[0])
