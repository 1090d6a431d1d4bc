#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

One step is the whole hot path on one batch of synthetic inputs: the verify
attention -- history pass over the KV cache, masked draft block and
log-sum-exp merge -- as one spec_attn_verify call (at the default workload
its two launches, spec_attn_prefix's history kernel then the fused block +
merge; a single launch on small grids), and rapid_accept (RAPID's
vocabulary pass), back to back on one stream.  --attention block_merge makes
the spec_attn_prefix and spec_attn_block_merge calls separately,
--attention unfused spec_attn_prefix, spec_attn_block and lse_merge.
Default workload: the LLaMA-3.1-8B-shaped verify layer (32 query / 8 kv
heads, d=128, 131072-token bf16 KV cache, gamma=10, vocab 128256, T=1,
eta=0.5), inputs resident in HBM.  Three copies of the KV cache and of the
logits rotate from step to step so that no step reads what the previous one
left in the 256 MB last-level cache.

Prints one JSON line: steps/s (value: K steps timed with nothing else on the
stream); per-kernel device times from HIP events recorded during a second,
untimed pass over the same K steps, the attention's pair riding on its own
dispatches (the KV-stream over that span is reported beside the main one);
the history kernel's and the block + merge kernel's own durations from a
third untimed pass in which each kernel's events ride on its own dispatch
(KV-stream = K+V bytes over their sum; the history kernel is the
roofline's kernel when the attention takes two launches); and the fp64 CPU
oracle timed on the host as a reported baseline, which also checks one step
of the library's outputs on the same inputs and reports their acceptance
statistics.  A plain 2 GiB device copy is measured before the warm-up
(context for the peak); its buffers stay in torch's cache, because a device
free slows the streaming kernels by ~7% for about 30 ms per GiB freed.  For
the same reason the HIP graphs reported beside the eager rate are captured
without torch.cuda.graph(), which empties that cache first.
"""

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "verify steps/s + KV-stream HBM GB/s, 8B-shaped layer, 128K ctx, gamma=10"
# HBM bytes per launch of the attention's dominant kernel (the single-launch
# spec_attn_verify, else the history pass of spec_attn_prefix), from rocprofv3
# FETCH_SIZE/WRITE_SIZE passes on this workload (one file per kernel and
# workload).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "%s_%s_traffic.json")
PREFIX_SRC = os.path.join(ROOT, "speculative_decoding_verify_split_amd", "csrc", "attn_prefix.hip")


class _HipEvents:
    """Raw HIP events (the runtime torch already loaded), for
    spec_attn_prefix_ev: recorded on the kernel's own dispatch."""

    def __init__(self, count):
        import ctypes
        self._c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def record(self, idx, stream):
        if self.hip.hipEventRecord(self.ev[idx], self._c.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self._c.c_float()
        if self.hip.hipEventElapsedTime(self._c.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def kernel_source_digest(path=PREFIX_SRC):
    """sha256 of the history kernels' source with comments and whitespace
    removed: a counter record stays valid across comment edits and is
    dropped by any change to the code itself."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


def _src_sha():
    return kernel_source_digest()


def _counter_record(workload, kernel="spec_attn_prefix"):
    """The committed counter summary of this workload's kernel, or None if
    it is missing or was taken on other kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE % (kernel, workload)))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_code_sha256") != _src_sha():
        return None
    return rec


def _traffic_per_launch(workload, kernel="spec_attn_prefix"):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE passes, scaled by a
    plain copy), or None."""
    rec = _counter_record(workload, kernel)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def _host_info():
    """The host the oracle ran on: CPU model, visible cores, affinity, BLAS threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")}
                for i in threadpool_info()]
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)), "blas": blas}


def _cpu_baseline(ai, vi, budget_s, gpu=None):
    """Time the fp64 oracle on the host: full unsplit attention over every
    head plus the step-by-step acceptance, repeated within the budget.  With
    gpu (the library's outputs for the same inputs) the oracle's last result
    is also compared with them, and the acceptance statistics of the inputs
    are reported (check)."""
    from oracle import attn_ref, rapid_accept_ref
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: count the affinity mask
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    reps, t0 = 0, time.perf_counter()
    while True:
        O_ref, L_ref = attn_ref(ai.q, ai.k_cache, ai.v_cache, ai.k_blk, ai.v_blk, ai.seq_lens,
                                ai.parent, ai.sm_scale)
        ref = rapid_accept_ref(vi.z, vi.y, vi.draft, vi.r, vi.u, vi.T, vi.eta)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 20:
            break
    out = {"value": reps / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
           "sample": "%d full verify step(s) of the same workload (all %d query heads over "
                     "%d history tokens + vocabulary pass), %.1f s" %
                     (reps, ai.q.shape[1], int(ai.seq_lens.max()), el),
           "host": _host_info()}
    if gpu is not None:
        out["check"] = _check_against_oracle(O_ref, L_ref, ref, vi, gpu)
    return out


def _check_against_oracle(O_ref, L_ref, ref, vi, gpu):
    """The benchmark step's own outputs against the oracle's on the same
    inputs (rules of oracle/compare.py), and the acceptance statistics of
    those inputs: alpha_t = sum_v min(q_t(v), p_hat_t(v)) per draft row and
    the expected accepted length sum_k prod_{t<k} alpha_t (RAPID blog
    section 2.1's test with p_hat, on independent rows)."""
    import numpy as np
    from oracle import draft_probs
    from oracle.compare import attn_row_errors, compare_accept, flag_counts
    res = compare_accept(ref, gpu["n_accept"], gpu["out_tokens"], vi.r, vi.u, draft=vi.draft)
    B, g = vi.draft.shape
    alpha = np.array([[np.sum(np.minimum(draft_probs(vi.y[b, t], vi.T), ref["p_hat"][b, t]))
                       for t in range(g)] for b in range(B)])
    exp_len = np.mean([sum(np.prod(alpha[b, :k]) for k in range(1, g + 1)) for b in range(B)])
    fa6, fd6, _ = flag_counts(ref, vi.r, 1e-6)
    return {
        "attn_max_row_rel_err": float(attn_row_errors(gpu["out"], O_ref).max()),
        "attn_max_abs_dlse": float(np.abs(gpu["lse"] - L_ref).max()),
        "p_hat_max_abs_err": float(np.abs(gpu["p_hat"] - ref["p_hat"]).max()),
        "ratio_max_abs_err": float(np.abs(gpu["ratio"] - ref["ratio"]).max()),
        "n_accept": {"gpu": [int(x) for x in gpu["n_accept"]],
                     "oracle": [int(x) for x in ref["n_accept"]]},
        "tokens_errors": res["errors"],
        "exact_draws": res["exact_draws"], "diverged": res["diverged"],
        "flagged_1e-4": {"accept": res["flagged_accept"], "draw": res["flagged_draw"]},
        "flagged_1e-6": {"accept": int(fa6), "draw": int(fd6)},
        "alpha_per_row": [float(a) for a in alpha.mean(axis=0)],
        "expected_accepted_length": float(exp_len),
        "note": "one step on the benchmark's resident inputs (first rotated copy), outputs "
                "read back after the timed region",
    }


def _tree_accept_time(workload, K, warmup):
    """rapid_tree_accept on the workload's own draft tree (all nodes, B = 1,
    the workload's vocabulary): K calls timed with events after the warm-up;
    the inputs and outputs of one call are kept (_io) for the oracle leg."""
    import numpy as np
    import torch
    from speculative_decoding_verify_split_amd import rapid_verify as rv
    from speculative_decoding_verify_split_amd.step import to_device
    from workloads import config_tree_vocab
    vt = config_tree_vocab(workload, B_override=1)
    B, n, V = vt.z.shape
    d = {k: to_device(getattr(vt, k)) for k in ("z", "y", "tokens", "r", "u")}
    n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    path = torch.empty((B, n), dtype=torch.int32, device="cuda")
    tok = torch.empty((B, n), dtype=torch.int32, device="cuda")
    ws = torch.empty((rv.rapid_tree_accept_workspace_size(B, n, V),), dtype=torch.uint8,
                     device="cuda")
    par = [int(p) for p in vt.parent]

    def call():
        rv.rapid_tree_accept(d["z"], d["y"], d["tokens"], par, d["r"], d["u"], vt.T, vt.eta,
                             n_acc, path, tok, ws)

    for _ in range(max(1, warmup)):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        call()
    e1.record()
    torch.cuda.synchronize()
    kids = np.bincount(np.asarray(vt.parent[1:]), minlength=n)
    return {"us_per_call": e0.elapsed_time(e1) * 1e3 / K, "calls": K, "nodes": n, "vocab": V,
            "launches": 3 + max(0, int(kids.max()) - 1),
            "note": "rapid_tree_accept over the workload's whole draft tree (the step above "
                    "accepts along its chain 0..depth)",
            "_io": (vt, (n_acc.cpu().numpy(), path.cpu().numpy(), tok.cpu().numpy()))}


def _tree_check(vt, outs):
    """The timed tree acceptance's outputs against the tree oracle."""
    from oracle import rapid_tree_accept_ref
    from oracle.compare import compare_tree_accept
    n_g, path_g, tok_g = outs
    ref = rapid_tree_accept_ref(vt.z, vt.y, vt.parent, vt.tokens, vt.r, vt.u, vt.T, vt.eta)
    res = compare_tree_accept(ref, vt.parent, vt.tokens, n_g, path_g, tok_g, vt.r)
    return {"errors": res["errors"], "n_accept": {"gpu": [int(x) for x in n_g],
                                                  "oracle": [int(x) for x in ref["n_accept"]]},
            "exact_draws": res["exact_draws"], "flagged_draw": res["flagged_draw"]}


def _copy_context(n_bytes=1 << 31, min_ms=0.0, reps=5):
    """A plain 2 GiB device-to-device copy_ on the same box, as context for
    the 8 TB/s peak: (read + write bytes) / time, over at least `reps`
    copies and at least min_ms of device time."""
    import torch
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    total_ms, done = 0.0, 0
    while done < reps or total_ms < min_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        total_ms += e0.elapsed_time(e1)
        done += reps
    s = total_ms / 1e3 / done
    # The buffers go back to torch's cache, not to the driver: on this part
    # a device free (hipFree, as torch's empty_cache makes) leaves the
    # streaming kernels ~7% slower for about 30 ms per GiB freed, so nothing
    # is freed to the driver before the timed steps.
    del src, dst
    return {"bytes_copied": n_bytes, "copies": done, "GBps_read_plus_write": 2 * n_bytes / s / 1e9}


def _capture_graph(fn):
    """fn's kernels captured into one HIP graph.  torch.cuda.graph() would
    first hand torch's cached device memory back to the driver
    (empty_cache); a device free leaves the streaming kernels slower for a
    while (about 30 ms per GiB freed), so the capture is begun directly, on
    a side stream of its own."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g.capture_begin()
        try:
            fn()
        finally:
            g.capture_end()
    torch.cuda.synchronize()
    return g


def _calibrate_copy(n_bytes, reps):
    """A plain device copy of known size, for scaling HBM counters."""
    import torch
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n_bytes, "reps": reps}))


def _timed_loop(step, K, warmup, n_events=3):
    import torch
    for i in range(warmup):
        step(i)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, evs[i])
    torch.cuda.synchronize()
    return evs, time.perf_counter() - t0


def run_drafter(args):
    """The LongSpec drafter's decode-step attention: cross-attention of one
    query row per head over the target's cache (spec_attn_prefix at n = 1,
    history-only lse_merge) and the sliding-window self-attention over the
    drafter's ring cache (spec_attn_window)."""
    import numpy as np
    import torch
    from oracle import attn_keys_ref, bf16_bits_to_f64, window_attn_ref
    from speculative_decoding_verify_split_amd import rapid_verify as rv
    from speculative_decoding_verify_split_amd.step import VerifyStep, WindowStep
    from workloads import DRAFTER_CONFIGS, config_drafter

    cfg = DRAFTER_CONFIGS[args.workload]
    cross, win = config_drafter(args.workload)
    st = VerifyStep(cross, None)
    ws = WindowStep(win)
    R = max(1, args.rotate)
    kvs = [(st.k_cache, st.v_cache)] + [(st.k_cache.clone(), st.v_cache.clone())
                                        for _ in range(R - 1)]

    K = args.steps
    hev = _HipEvents(4 * K)  # history kernel's own dispatch, then after merge and window
    sid = torch.cuda.current_stream().cuda_stream

    def step(i, timed=False):
        kc, vc = kvs[i % R]
        if timed:
            rv.spec_attn_prefix_ev(st.q, kc, vc, st.seq_lens, st.max_seq_len, st.split_len,
                                   st.num_splits, st.o_part, st.lse_part, hev.ev[4 * i],
                                   hev.ev[4 * i + 1], st.sm_scale)
        else:
            rv.spec_attn_prefix(st.q, kc, vc, st.seq_lens, st.max_seq_len, st.split_len,
                                st.num_splits, st.o_part, st.lse_part, st.sm_scale)
        rv.lse_merge(st.o_part, st.lse_part, None, None, st.out, st.lse_out)
        if timed:
            hev.record(4 * i + 2, sid)
        ws.run()
        if timed:
            hev.record(4 * i + 3, sid)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The same K steps again, untimed, with events at the kernel boundaries
    # for the per-kernel breakdown (event records are stream commands of
    # their own, so they stay out of the timed steps above).
    for i in range(K):
        step(i, timed=True)
    torch.cuda.synchronize()
    prefix_ms = [hev.elapsed_ms(4 * i, 4 * i + 1) for i in range(K)]
    merge_ms = [hev.elapsed_ms(4 * i + 1, 4 * i + 2) for i in range(K)]
    win_ms = [hev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(K)]
    step_ms = [hev.elapsed_ms(4 * i, 4 * i + 3) for i in range(K)]
    hev.close()
    L = int(np.max(cross.seq_lens))
    kv_bytes = int(2 * st.Hkv * st.d * 2 * int(np.sum(cross.seq_lens)))
    prefix_s = float(np.mean(prefix_ms)) / 1e3
    achieved = kv_bytes / prefix_s / 1e9
    line = {
        "metric": "drafter decode steps/s + KV-stream HBM GB/s, 8B-shaped, 128K ctx, n=1",
        "value": K / elapsed, "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / K, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "dtype_detail": "cross-attention: bf16 K/V/Q on MFMA, fp32 accumulation and softmax; "
                        "window: bf16 inputs, fp32 vector ALU",
        "data": "synthetic (seeded; K/V/Q ~ N(0,1) bf16)",
        "config": {"workload": cfg["desc"], "batch": st.B, "q_heads": st.Hq, "kv_heads": st.Hkv,
                   "head_dim": st.d, "kv_tokens": L, "query_rows": 1,
                   "window": ws.window, "sink": ws.sink, "split_len": st.split_len,
                   "num_splits": st.num_splits, "rotated_copies": R,
                   "parallelism": "single GPU"},
        "kernels_us": {"spec_attn_prefix": prefix_s * 1e6,
                       "lse_merge": float(np.mean(merge_ms)) * 1e3,
                       "spec_attn_window": float(np.mean(win_ms)) * 1e3,
                       "device_step": float(np.mean(step_ms)) * 1e3},
        "device_step_us": {"median": float(np.median(step_ms)) * 1e3,
                           "p10": float(np.percentile(step_ms, 10)) * 1e3,
                           "p90": float(np.percentile(step_ms, 90)) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "spec_attn_prefix (cross-attention, n=1)",
                     "algorithmic_bytes_per_launch": kv_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        reps, t0 = 0, time.perf_counter()
        G = st.Hq // st.Hkv
        while True:
            for h in range(st.Hq):
                attn_keys_ref(bf16_bits_to_f64(cross.q[0, h]),
                              bf16_bits_to_f64(cross.k_cache[0, h // G, :L]),
                              bf16_bits_to_f64(cross.v_cache[0, h // G, :L]),
                              np.ones((1, L), bool), 1.0)
            window_attn_ref(win.q, win.k_ring, win.v_ring, win.pos, win.cap, win.sink, win.window)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_budget or reps >= 20:
                break
        line["cpu_baseline"] = {"value": reps / el, "unit": "steps/s", "cores": threads,
                                "kind": "oracle",
                                "sample": "%d full drafter step(s) (all %d heads over %d tokens + "
                                          "window), %.1f s" % (reps, st.Hq, L, el)}
    print(json.dumps(line), flush=True)


def run_model(args):
    """Whole-model verify step: every attention layer (history pass + fused
    block/merge) back to back, then one acceptance pass, replayed from a HIP
    graph.  value is the replay rate; the eager rate is reported beside it."""
    import numpy as np
    import torch
    from speculative_decoding_verify_split_amd.step import ModelStep
    from workloads import CONFIGS, MODEL_CONFIGS, config_vocab, make_layer_device

    mc = MODEL_CONFIGS[args.workload]
    c = CONFIGS[mc["layer_config"]]
    eta = c["etas"][min(1, len(c["etas"]) - 1)] if args.eta is None else args.eta
    vi = config_vocab(mc["layer_config"], eta=eta)
    layers = [make_layer_device(mc["seed"], l, c["B"], c["Hq"], c["Hkv"], c["d"], c["gamma"] + 1,
                                c["L"]) for l in range(mc["layers"])]
    ms = ModelStep(layers, c["L"], vocab=vi)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        ms.attention()
        if ev is not None:
            ev[1].record()
        ms.vocab.accept()
        if ev is not None:
            ev[2].record()

    K = args.steps
    evs, elapsed = _timed_loop(step, K, args.warmup)
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    acc_ms = [e[1].elapsed_time(e[2]) for e in evs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ms.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = _capture_graph(ms.run)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    g_el = time.perf_counter() - g0
    kv_bytes = mc["layers"] * 2 * c["Hkv"] * c["d"] * 2 * c["L"] * c["B"]
    attn_s = float(np.mean(attn_ms)) / 1e3
    achieved = kv_bytes / attn_s / 1e9
    line = {
        "metric": "model verify steps/s (32 attention layers + acceptance), 8B-shaped, "
                  "128K ctx, gamma=10",
        "value": K / g_el, "unit": "steps/s", "value_mode": "HIP graph replay",
        "eager_steps_per_s": K / elapsed, "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": g_el * 1e3 / K, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "dtype_detail": "attention: bf16 K/V/Q on MFMA with fp32 accumulation and softmax; "
                        "vocabulary pass: fp32",
        "data": "synthetic (seeded on the device; K/V/Q ~ N(0,1) bf16, logits ~ N(0,9))",
        "config": {"workload": mc["desc"], "layers": mc["layers"], "batch": c["B"],
                   "q_heads": c["Hq"], "kv_heads": c["Hkv"], "head_dim": c["d"],
                   "kv_tokens": c["L"], "block_rows": c["gamma"] + 1, "gamma": c["gamma"],
                   "vocab": c["V"], "eta": eta, "kv_bytes_per_step": kv_bytes,
                   "parallelism": "single GPU"},
        "kernels_us": {"all_layers_attention": attn_s * 1e6,
                       "rapid_accept": float(np.mean(acc_ms)) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "all layers' spec_attn_prefix + spec_attn_block_merge (eager)",
                     "algorithmic_bytes_per_launch": kv_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The device comes out of the idle setup (input generation, copies) at
    # reduced clocks; ~100 steps (about 10 ms at the 8B shape) bring it to
    # the steady state a serving loop runs in.
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before the K timed ones (default 200)")
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--eta", type=float, default=None)
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of host time for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay measurement reported beside the eager one")
    ap.add_argument("--attention", choices=("verify", "block_merge", "unfused"),
                    default="verify",
                    help="verify: one spec_attn_verify call (default); block_merge: "
                         "spec_attn_prefix + spec_attn_block_merge; unfused: spec_attn_prefix + "
                         "spec_attn_block + lse_merge")
    ap.add_argument("--settle-ms", type=float, default=0.0,
                    help="device time of the copy-bandwidth measurement before the warm-up")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: rapid_verify runs on one GPU; there is no multi-GPU path to "
              "measure (how the step would shard is described, not built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        _calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return

    from workloads import DRAFTER_CONFIGS, MODEL_CONFIGS
    if args.workload in DRAFTER_CONFIGS:
        return run_drafter(args)
    if args.workload in MODEL_CONFIGS:
        return run_model(args)

    from speculative_decoding_verify_split_amd import rapid_verify as rv
    from speculative_decoding_verify_split_amd.step import VerifyStep
    from workloads import CONFIGS, config_attention, config_vocab

    cfg = CONFIGS[args.workload]
    eta = cfg["etas"][min(1, len(cfg["etas"]) - 1)] if args.eta is None else args.eta
    ai = config_attention(args.workload)
    vi = config_vocab(args.workload, eta=eta)
    st = VerifyStep(ai, vi, want_ratio=False, want_p_hat=False)
    R = max(1, args.rotate)
    kvs = [(st.k_cache, st.v_cache)] + [(st.k_cache.clone(), st.v_cache.clone())
                                        for _ in range(R - 1)]
    logits = [(st.z, st.y)] + [(st.z.clone(), st.y.clone()) for _ in range(R - 1)]

    # A plain device copy, measured before the warm-up (context for the 8 TB/s
    # peak; it also takes the device out of the idle clocks of the setup).
    copy_ctx = _copy_context(min_ms=args.settle_ms)

    K = args.steps
    mode = args.attention
    single = mode == "verify" and rv.rv_verify_single_launch(st.B, st.Hq, st.Hkv, st.n, st.d,
                                                             st.num_splits)
    # four raw HIP events per timed step: the attention's start and end on
    # its own dispatches (spec_attn_verify's events; with the separate calls,
    # the history kernel's, spec_attn_prefix_ev), then after the block + merge
    # and after the acceptance pass
    hev = _HipEvents(4 * K)
    sid = torch.cuda.current_stream().cuda_stream

    def step(i, timed=False, ev=None, calls=None):
        kc, vc = kvs[i % R]
        z, y = logits[i % R]
        ev = ev or hev
        evs = (ev.ev[4 * i], ev.ev[4 * i + 1]) if timed else (None, None)
        if (calls or mode) == "verify":
            st.attention(kc, vc, single=True, events=evs)
        else:
            rv.spec_attn_prefix_ev(st.q, kc, vc, st.seq_lens, st.max_seq_len, st.split_len,
                                   st.num_splits, st.o_part, st.lse_part, evs[0], evs[1],
                                   st.sm_scale)
            if (calls or mode) == "unfused":
                rv.spec_attn_block(st.q, st.k_blk, st.v_blk, st.parent, st.o_blk, st.lse_blk,
                                   st.sm_scale)
                rv.lse_merge(st.o_part, st.lse_part, st.o_blk, st.lse_blk, st.out, st.lse_out)
            else:
                rv.spec_attn_block_merge(st.q, st.k_blk, st.v_blk, st.parent, st.o_part,
                                         st.lse_part, st.out, st.lse_out, st.sm_scale)
        if timed:
            ev.record(4 * i + 2, sid)
        rv.rapid_accept(z, y, st.draft, st.r, st.u, st.T, st.eta, st.n_accept, st.out_tokens,
                        st.workspace)
        if timed:
            ev.record(4 * i + 3, sid)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The same K steps again, untimed, with events at the kernel boundaries
    # for the per-kernel breakdown (event records are stream commands of
    # their own, so they stay out of the timed steps above).
    for i in range(K):
        step(i, timed=True)
    torch.cuda.synchronize()
    # When the attention takes two launches, each kernel's own duration (the
    # history kernel is the roofline's kernel) comes from one more untimed
    # pass with the two calls made separately, each with its events on its
    # own dispatch.
    hist_ev = None
    if mode != "unfused" and not single:
        hist_ev = _HipEvents(4 * K)
        for i in range(K):
            kc, vc = kvs[i % R]
            z, y = logits[i % R]
            rv.spec_attn_prefix_ev(st.q, kc, vc, st.seq_lens, st.max_seq_len, st.split_len,
                                   st.num_splits, st.o_part, st.lse_part, hist_ev.ev[4 * i],
                                   hist_ev.ev[4 * i + 1], st.sm_scale)
            rv.spec_attn_block_merge_ev(st.q, st.k_blk, st.v_blk, st.parent, st.o_part,
                                        st.lse_part, st.out, hist_ev.ev[4 * i + 2],
                                        hist_ev.ev[4 * i + 3], st.lse_out, st.sm_scale)
            rv.rapid_accept(z, y, st.draft, st.r, st.u, st.T, st.eta, st.n_accept,
                            st.out_tokens, st.workspace)
        torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        # The same steps captured once per rotated copy and replayed: the
        # library only enqueues kernels on the caller's stream.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(R):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = [_capture_graph(lambda i=i: step(i)) for i in range(R)]
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for i in range(K):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        g_el = time.perf_counter() - g0
        graph = {"steps_per_s": K / g_el, "ms_per_step": g_el * 1e3 / K,
                 "note": "same K steps replayed from HIP graphs (one per rotated copy), "
                         "after the timed eager region"}
        # The R rotated steps captured back to back in one graph: the graph
        # launch is paid once per R steps, as in a serving loop that captures
        # several steps (or a whole model) at once.
        def all_steps():
            for i in range(R):
                step(i)
        gm = _capture_graph(all_steps)
        reps = max(1, K // R)
        for _ in range(max(1, args.warmup // R)):
            gm.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(reps):
            gm.replay()
        torch.cuda.synchronize()
        gm_el = time.perf_counter() - g0
        graph["multi_step"] = {"steps_per_s": reps * R / gm_el,
                               "ms_per_step": gm_el * 1e3 / (reps * R),
                               "steps_per_graph": R, "replays": reps}

    # One more step on the resident inputs (first rotated copy), with the
    # ratios and p_hat requested, whose outputs the oracle leg checks.
    ratio_t = torch.empty((st.B, st.gamma), dtype=torch.float32, device="cuda")
    p_hat_t = torch.empty((st.B, st.gamma, st.V), dtype=torch.float32, device="cuda")
    st.out.zero_()
    st.lse_out.zero_()
    if mode == "verify":
        st.attention(single=True)
    else:
        st.attention(fused=mode == "block_merge")
    rv.rapid_accept(st.z, st.y, st.draft, st.r, st.u, st.T, st.eta, st.n_accept, st.out_tokens,
                    st.workspace, ratio_t, p_hat_t)
    torch.cuda.synchronize()
    gpu_out = {"out": st.out.float().cpu().numpy(), "lse": st.lse_out.cpu().numpy(),
               "n_accept": st.n_accept.cpu().numpy(), "out_tokens": st.out_tokens.cpu().numpy(),
               "ratio": ratio_t.cpu().numpy(), "p_hat": p_hat_t.cpu().numpy()}
    del ratio_t, p_hat_t

    tree = None
    if "n_nodes" in cfg:
        tree = _tree_accept_time(args.workload, K, args.warmup)

    # verify: the attention's span on its own dispatches (one launch, or the
    # history kernel's start to the merge kernel's end); otherwise the
    # attention up to the marker after the merge.  prefix_ms: the roofline
    # kernel's own duration (the single launch, or the history kernel).
    span_ms = [hev.elapsed_ms(4 * i, 4 * i + 1) for i in range(K)]
    if mode == "verify":
        attn_ms = span_ms
    else:
        attn_ms = [hev.elapsed_ms(4 * i, 4 * i + 2) for i in range(K)]
    if hist_ev is not None:
        prefix_ms = [hist_ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(K)]
        merge_ms = [hist_ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(K)]
    else:
        prefix_ms = span_ms
        merge_ms = None
    # The KV stream over the attention's kernel time (their own durations,
    # without the gap between them), and over its span
    acc_ms = [hev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(K)]
    step_dev_ms = [hev.elapsed_ms(4 * i, 4 * i + 3) for i in range(K)]
    hev.close()
    if hist_ev is not None:
        hist_ev.close()
    B, Hkv, d = st.B, st.Hkv, st.d
    kv_bytes = int(2 * Hkv * d * 2 * int(np.sum(ai.seq_lens)))  # K and V, bf16
    prefix_s = float(np.mean(prefix_ms)) / 1e3
    attn_s = float(np.mean(attn_ms)) / 1e3
    merge_s = float(np.mean(merge_ms)) / 1e3 if merge_ms is not None else None
    # kernel time of the attention: one launch, or the two kernels' own
    # durations (the three calls of the unfused mode: their span)
    kern_s = attn_s if single or mode == "unfused" else prefix_s + merge_s
    achieved = kv_bytes / prefix_s / 1e9
    logits_bytes = int(B * (2 * st.gamma + 1) * st.V * 4)
    acc_s = float(np.mean(acc_ms)) / 1e3
    n_acc = st.n_accept.cpu().numpy()
    roof_kernel = "spec_attn_verify" if single else "spec_attn_prefix"

    line = {
        "metric": METRIC,
        "value": K / elapsed,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "attention: bf16 K/V/Q on MFMA with fp32 accumulation and softmax; "
                        "vocabulary pass: fp32",
        "data": "synthetic (seeded; K/V/Q ~ N(0,1) bf16, logits ~ N(0,9))",
        "config": {"workload": cfg["desc"], "batch": B, "q_heads": st.Hq, "kv_heads": Hkv,
                   "head_dim": d, "kv_tokens": int(np.max(ai.seq_lens)), "block_rows": st.n,
                   "gamma": st.gamma, "vocab": st.V, "T": st.T, "eta": st.eta,
                   "split_len": st.split_len, "num_splits": st.num_splits,
                   "rotated_copies": R,
                   "attention": {"verify": "spec_attn_verify (%s)" % (
                       "one launch" if single else "two launches"),
                                 "block_merge": "spec_attn_prefix + spec_attn_block_merge",
                                 "unfused": "spec_attn_prefix + spec_attn_block + lse_merge"}[mode],
                   "parallelism": "single GPU"},
        "kv_stream_GBps": kv_bytes / kern_s / 1e9,
        "kv_stream_frac_of_peak": kv_bytes / kern_s / 1e9 / HBM_PEAK_GBPS,
        "kv_stream_definition": (
            "K+V bytes over the attention's kernel time: the history kernel's and the block + "
            "merge kernel's own durations, each between HIP events on its own dispatch "
            "(separate untimed pass), without the gap between them" if kern_s != attn_s else
            "K+V bytes over the attention's span between HIP events on its dispatches"),
        "kv_stream_span_GBps": kv_bytes / attn_s / 1e9,
        "kv_stream_span_frac_of_peak": kv_bytes / attn_s / 1e9 / HBM_PEAK_GBPS,
        # one read of z [B, gamma+1, V] and y [B, gamma, V] (fp32) over the
        # acceptance pass's event time (a latency-bound pass at B = 1)
        "logits_bytes": logits_bytes,
        "logits_stream_GBps": logits_bytes / acc_s / 1e9,
        "logits_stream_frac_of_peak": logits_bytes / acc_s / 1e9 / HBM_PEAK_GBPS,
        "kernels_us": dict(
            ({"spec_attn_verify": attn_s * 1e6} if mode == "verify" else
             {"spec_attn_prefix": float(np.mean(span_ms)) * 1e3,
              ("spec_attn_block+lse_merge" if mode == "unfused" else
               "spec_attn_block_merge (to a marker)"):
                  (attn_s * 1e3 - float(np.mean(span_ms))) * 1e3}),
            **({"spec_attn_prefix (separate pass)": prefix_s * 1e6,
                "spec_attn_block_merge (separate pass)": merge_s * 1e6}
               if merge_ms is not None else {}),
            rapid_accept=float(np.mean(acc_ms)) * 1e3,
            device_step=float(np.mean(step_dev_ms)) * 1e3),
        "device_step_us": {"median": float(np.median(step_dev_ms)) * 1e3,
                           "p10": float(np.percentile(step_dev_ms, 10)) * 1e3,
                           "p90": float(np.percentile(step_dev_ms, 90)) * 1e3},
        ("spec_attn_verify_us" if mode == "verify" else "spec_attn_prefix_us"): {
            "median": float(np.median(span_ms)) * 1e3,
            "p10": float(np.percentile(span_ms, 10)) * 1e3,
            "p90": float(np.percentile(span_ms, 90)) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": _traffic_per_launch(args.workload, roof_kernel),
                     "kernel": ("spec_attn_verify (history pass, block and merge in one "
                                "launch)" if single else "spec_attn_prefix (history pass)"),
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "mfma_busy_frac": (_counter_record(args.workload, roof_kernel) or {}).get(
                         "mfma_busy_frac")},
        "mean_n_accept": float(np.mean(n_acc)),
        "graph_replay": graph,
        "copy_context": copy_ctx,
        "tree_accept": tree,
        "cpu_baseline": None,
    }
    del kvs, logits
    torch.cuda.empty_cache()
    tree_io = tree.pop("_io") if tree is not None else None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(ai, vi, args.cpu_budget, gpu=gpu_out)
        if tree is not None:
            tree["check"] = _tree_check(*tree_io)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
