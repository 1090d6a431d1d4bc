"""bench.py's host-side logic on the CPU: the one-GPU contract, the counter
records' source digest, and the oracle check it runs on its own step (fed
here with hand-built "GPU" outputs, no device involved)."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import attn_ref, rapid_accept_ref  # noqa: E402
from workloads import make_attention, make_vocab  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_digest_ignores_comments_and_whitespace(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int f(int a) { // add one\n  return a + 1; /* done */ }\n")
    d0 = bench.kernel_source_digest(str(src))
    src.write_text("int f(int a) {\n\n  return a + 1;   }  // other words\n")
    assert bench.kernel_source_digest(str(src)) == d0
    src.write_text("int f(int a) { return a + 2; }\n")
    assert bench.kernel_source_digest(str(src)) != d0


def test_counter_records_are_tied_to_the_kernel_source():
    rec = bench._counter_record("llama8b")
    if rec is None:  # taken on other kernel source: the bench reports traffic as null
        assert bench._traffic_per_launch("llama8b") is None
        return
    assert rec["kernel_code_sha256"] == bench.kernel_source_digest()
    assert rec["hbm_bytes_per_launch"] == pytest.approx(
        rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"])
    assert bench._traffic_per_launch("llama8b") == rec["hbm_bytes_per_launch"]
    assert bench._counter_record("no_such_workload") is None


def _small_step():
    ai = make_attention(7, 1, 4, 2, 64, 3, [300])
    vi = make_vocab(8, 2, 3, 50, 2.0, 1.0, 1.0, 0.5)
    O, L = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens, ai.parent,
                    ai.sm_scale)
    ref = rapid_accept_ref(vi.z, vi.y, vi.draft, vi.r, vi.u, vi.T, vi.eta)
    gpu = {"out": O.astype(np.float32), "lse": L.astype(np.float32),
           "n_accept": ref["n_accept"].copy(), "out_tokens": ref["out_tokens"].copy(),
           "ratio": ref["ratio"].astype(np.float32), "p_hat": ref["p_hat"].astype(np.float32)}
    return O, L, ref, vi, gpu


def test_oracle_check_of_a_matching_step():
    O, L, ref, vi, gpu = _small_step()
    chk = bench._check_against_oracle(O, L, ref, vi, gpu)
    assert chk["tokens_errors"] == [] and chk["diverged"] == 0
    assert chk["attn_max_row_rel_err"] < 1e-6 and chk["p_hat_max_abs_err"] < 1e-6
    assert chk["n_accept"]["gpu"] == chk["n_accept"]["oracle"]
    # alpha_t = sum_v min(q_t, p_hat_t), a probability; expected length in [0, gamma]
    g = vi.draft.shape[1]
    assert len(chk["alpha_per_row"]) == g
    assert all(0.0 <= a <= 1.0 for a in chk["alpha_per_row"])
    assert 0.0 <= chk["expected_accepted_length"] <= g
    json.dumps(chk)  # goes into the bench's JSON line


def test_oracle_check_reports_a_wrong_token():
    O, L, ref, vi, gpu = _small_step()
    b = 0
    m = int(ref["n_accept"][b])
    tok = gpu["out_tokens"]
    tok[b, m] = (tok[b, m] + 1) % vi.z.shape[2]  # the drawn token, changed
    chk = bench._check_against_oracle(O, L, ref, vi, gpu)
    assert chk["flagged_1e-4"]["draw"] == 0  # this seed's draws are not near an edge
    assert chk["tokens_errors"] and "b=0" in chk["tokens_errors"][0]
