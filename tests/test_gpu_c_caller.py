"""The verify step driven from plain C through the C ABI
(tests/c_caller/verify_step.c: buffers from hipMalloc, the null stream, no
torch, the split from rv_prefix_balanced_split).  Its outputs equal the
Python binding's bit for bit on the same inputs and split, and meet the
oracle's bounds (attention: LongSpec summary, section 2.3; acceptance: RAPID
blog, sections 2.1 and 2.4)."""

import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from oracle import attn_ref, rapid_accept_ref
from oracle.compare import ATTN_ROW_TOL, LSE_TOL_FP32, attn_row_errors, compare_accept
from workloads import make_attention, make_vocab
from speculative_decoding_verify_split_amd.step import VerifyStep

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "c_caller", "libverify_step_c.so")

CASES = [
    # name, seed, B, Hq, Hkv, d, n, lengths, gamma, V
    ("tiny-shape", 301, 1, 8, 2, 64, 5, [4096], 4, 32000),
    ("ragged-b3-d128", 302, 3, 16, 4, 128, 11, [3000, 0, 9000], 10, 20001),
]


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def _c_step():
    if not os.path.exists(LIB):
        raise RuntimeError(LIB + " is missing: build it with __graft_entry__.build()")
    fn = ctypes.CDLL(LIB).rv_c_verify_step
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn.argtypes = [I, I, I, I, I, ctypes.c_int64, I, I, F, F, F] + [P] * 18
    fn.restype = I
    return fn


def _ptr(a):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_verify_step_from_c(case):
    name, seed, B, Hq, Hkv, d, n, lens, gamma, V = case
    fn = _c_step()
    ai = make_attention(seed, B, Hq, Hkv, d, n, lens)
    vi = make_vocab(seed, B, gamma, V, 3.0, 1.0, 1.0, 0.5)
    L_max = ai.k_cache.shape[2]
    out = np.zeros((B, Hq, n, d), np.uint16)
    lse = np.zeros((B, Hq, n), np.float32)
    n_acc = np.zeros((B,), np.int32)
    toks = np.zeros((B, gamma + 1), np.int32)
    ratio = np.zeros((B, gamma), np.float32)
    split_len = np.zeros((1,), np.int64)
    S = np.zeros((1,), np.int32)
    ins = [np.ascontiguousarray(a) for a in (ai.q, ai.k_cache, ai.v_cache,
                                             ai.seq_lens.astype(np.int32), ai.k_blk, ai.v_blk,
                                             vi.z, vi.y, vi.draft, vi.r, vi.u)]
    announce("C caller %s: B=%d Hq=%d Hkv=%d d=%d n=%d lens=%s gamma=%d V=%d"
             % (name, B, Hq, Hkv, d, n, lens, gamma, V))
    rc = fn(B, Hq, Hkv, n, d, L_max, gamma, V, ai.sm_scale, vi.T, vi.eta,
            *[_ptr(a) for a in ins],
            *[_ptr(a) for a in (out, lse, n_acc, toks, ratio, split_len, S)])
    assert rc == 0, rc
    split = (int(split_len[0]), int(S[0]))
    announce("  split %s, n_accept %s" % (split, n_acc.tolist()))

    # the Python binding on the same inputs and split
    st = VerifyStep(ai, vi, split=split)
    st.attention(fused=True)
    st.accept()
    torch.cuda.synchronize()
    assert np.array_equal(out, st.out.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(lse.view(np.uint32), st.lse_out.cpu().numpy().view(np.uint32))
    assert np.array_equal(n_acc, st.n_accept.cpu().numpy())
    assert np.array_equal(toks, st.out_tokens.cpu().numpy())
    assert np.array_equal(ratio.view(np.uint32), st.ratio.cpu().numpy().view(np.uint32))

    # and the oracle
    O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens,
                            ai.parent, ai.sm_scale)
    out_f = (out.astype(np.uint32) << 16).view(np.float32)
    assert attn_row_errors(out_f, O_ref).max() <= ATTN_ROW_TOL
    assert np.abs(lse - L_ref).max() <= LSE_TOL_FP32
    ref = rapid_accept_ref(vi.z, vi.y, vi.draft, vi.r, vi.u, vi.T, vi.eta)
    res = compare_accept(ref, n_acc, toks, vi.r, vi.u, draft=vi.draft)
    assert not res["errors"], res["errors"]
    valid = ~np.isnan(ref["ratio"])
    assert np.abs(ratio[valid] - ref["ratio"][valid]).max() <= 1e-5
