"""Python binding of librapid_verify.so (argument marshalling only).

Each function has the name of the C entry point it wraps.  Tensors are torch
tensors on the GPU (torch is used for device memory and streams only); the
wrappers check dtype, device, contiguity and shapes, pass raw pointers and the
current HIP stream, and raise RuntimeError on a nonzero status.  Every step of
the computation runs in the library's HIP kernels; there is no fallback path.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librapid_verify.so")

_lib = None

# rapid_accept_ex options (RAPID blog section 2.4's two further rules)
RV_ACCEPT_TAIL_PRESERVE = 1
RV_ACCEPT_PRINTED_RESIDUAL = 2


class RapidVerifyError(RuntimeError):
    pass


def load_library():
    """Load librapid_verify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RapidVerifyError(
            "librapid_verify.so not found at %s: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.rv_status_string.argtypes = [i32]
    lib.rv_status_string.restype = ctypes.c_char_p
    lib.rv_version.argtypes = []
    lib.rv_version.restype = i32
    lib.rv_prefix_default_split.argtypes = [i64, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.rv_prefix_default_split.restype = i32
    lib.rv_prefix_balanced_split.argtypes = [vp, i32, i32, i32, i32, i32, i32,
                                             ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.rv_prefix_balanced_split.restype = i32
    lib.spec_attn_prefix.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i64, f32, i64,
                                     i32, vp, vp, vp]
    lib.spec_attn_prefix.restype = i32
    lib.spec_attn_prefix_ev.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i64, f32,
                                        i64, i32, vp, vp, vp, vp, vp]
    lib.spec_attn_prefix_ev.restype = i32
    lib.spec_attn_block.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.spec_attn_block.restype = i32
    lib.lse_merge.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.lse_merge.restype = i32
    lib.spec_attn_block_merge.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          f32, vp, vp, vp]
    lib.spec_attn_block_merge.restype = i32
    lib.spec_attn_block_merge_ev.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                             i32, f32, vp, vp, vp, vp, vp]
    lib.spec_attn_block_merge_ev.restype = i32
    lib.spec_attn_verify_sync_size.argtypes = [i32, i32]
    lib.spec_attn_verify_sync_size.restype = sz
    lib.rv_verify_single_launch.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.rv_verify_single_launch.restype = i32
    lib.spec_attn_verify.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i64, f32, i64,
                                     i32, vp, vp, vp, vp, vp, vp, sz, vp, vp, i32, vp, vp, vp]
    lib.spec_attn_verify.restype = i32
    lib.spec_attn_window_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.spec_attn_window_workspace_size.restype = sz
    lib.spec_attn_window.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                     vp, vp, vp, sz, vp]
    lib.spec_attn_window.restype = i32
    lib.rapid_accept_workspace_size.argtypes = [i32, i32, i32]
    lib.rapid_accept_workspace_size.restype = sz
    lib.rapid_accept.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp, vp, vp,
                                 sz, vp]
    lib.rapid_accept.restype = i32
    lib.rapid_accept_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, ctypes.c_uint,
                                    vp, vp, vp, vp, vp, sz, vp]
    lib.rapid_accept_ex.restype = i32
    lib.rapid_tree_accept_workspace_size.argtypes = [i32, i32, i32]
    lib.rapid_tree_accept_workspace_size.restype = sz
    lib.rapid_tree_accept.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp,
                                      vp, vp, sz, vp]
    lib.rapid_tree_accept.restype = i32
    lib.rapid_accept_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, f32,
                                         ctypes.c_uint, vp, vp, vp, vp, vp]
    lib.rapid_accept_noalloc.restype = i32
    _lib = lib
    return lib


def rv_status_string(status):
    return load_library().rv_status_string(int(status)).decode()


def rv_version():
    return load_library().rv_version()


def _check(status, what):
    if status != 0:
        raise RapidVerifyError("%s: %s" % (what, rv_status_string(status)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def rv_prefix_default_split(max_seq_len, B, Hq, Hkv, n, d):
    """Split choice for spec_attn_prefix -> (split_len, num_splits)."""
    sl = ctypes.c_int64()
    ns = ctypes.c_int()
    _check(load_library().rv_prefix_default_split(int(max_seq_len), B, Hq, Hkv, n, d,
                                                  ctypes.byref(sl), ctypes.byref(ns)),
           "rv_prefix_default_split")
    return sl.value, ns.value


def rv_prefix_balanced_split(seq_lens, Hq, Hkv, n, d, num_cus=None):
    """Split choice from the batch's host lengths (any int sequence or array)
    -> (split_len, num_splits).  num_cus defaults to the current device's
    compute-unit count."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int64))
    if lens.ndim != 1 or lens.size < 1:
        raise ValueError("seq_lens must be a non-empty 1-D sequence")
    if (lens < 0).any() or (lens > 0x7FFFFFFF).any():
        raise ValueError("seq_lens must lie in [0, 2^31)")
    lens = lens.astype(np.int32)
    if num_cus is None:
        import torch
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    sl = ctypes.c_int64()
    ns = ctypes.c_int()
    _check(load_library().rv_prefix_balanced_split(
        lens.ctypes.data_as(ctypes.c_void_p), int(lens.size), Hq, Hkv, n, d, int(num_cus),
        ctypes.byref(sl), ctypes.byref(ns)), "rv_prefix_balanced_split")
    return sl.value, ns.value


def spec_attn_prefix(q, k_cache, v_cache, seq_lens, max_seq_len, split_len, num_splits, o_part,
                     lse_part, sm_scale=1.0, stream=None):
    """History pass.  q bf16 [B,Hq,n,d]; k_cache/v_cache bf16 [B,Hkv,L_max,d];
    seq_lens int32 [B]; o_part fp32 [B,Hq,n,S,d]; lse_part fp32 [B,Hq,n,S]."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_cache, "k_cache", torch.bfloat16)
    Hkv, L_max = k_cache.shape[1], k_cache.shape[2]
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, L_max, d))
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, L_max, d))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(o_part, "o_part", torch.float32, (B, Hq, n, num_splits, d))
    _need(lse_part, "lse_part", torch.float32, (B, Hq, n, num_splits))
    _check(load_library().spec_attn_prefix(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), int(max_seq_len), B, Hq, Hkv, n, d,
        L_max, float(sm_scale), int(split_len), int(num_splits), _ptr(o_part), _ptr(lse_part),
        _stream(stream)), "spec_attn_prefix")


def spec_attn_prefix_ev(q, k_cache, v_cache, seq_lens, max_seq_len, split_len, num_splits,
                        o_part, lse_part, start_event, stop_event, sm_scale=1.0, stream=None):
    """spec_attn_prefix recording two caller-created hipEvent_t handles (ints
    or ctypes pointers; None allowed) on the history kernel's own dispatch."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_cache, "k_cache", torch.bfloat16)
    Hkv, L_max = k_cache.shape[1], k_cache.shape[2]
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, L_max, d))
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, L_max, d))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(o_part, "o_part", torch.float32, (B, Hq, n, num_splits, d))
    _need(lse_part, "lse_part", torch.float32, (B, Hq, n, num_splits))
    _check(load_library().spec_attn_prefix_ev(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), int(max_seq_len), B, Hq, Hkv, n, d,
        L_max, float(sm_scale), int(split_len), int(num_splits), _ptr(o_part), _ptr(lse_part),
        _stream(stream), ctypes.c_void_p(start_event) if isinstance(start_event, int) else start_event,
        ctypes.c_void_p(stop_event) if isinstance(stop_event, int) else stop_event),
        "spec_attn_prefix_ev")


def spec_attn_block(q, k_blk, v_blk, parent, o_blk, lse_blk, sm_scale=1.0, stream=None):
    """Draft-block pass.  parent: None (causal chain) or host int sequence [n]."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_blk, "k_blk", torch.bfloat16)
    Hkv = k_blk.shape[1]
    _need(k_blk, "k_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(v_blk, "v_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(o_blk, "o_blk", torch.float32, (B, Hq, n, d))
    _need(lse_blk, "lse_blk", torch.float32, (B, Hq, n))
    par = None
    if parent is not None:
        vals = [int(x) for x in parent]
        if len(vals) != n:
            raise ValueError("parent must have n entries")
        par = (ctypes.c_int32 * n)(*vals)
    _check(load_library().spec_attn_block(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), ctypes.cast(par, ctypes.c_void_p) if par else None,
        B, Hq, Hkv, n, d, float(sm_scale), _ptr(o_blk), _ptr(lse_blk), _stream(stream)),
        "spec_attn_block")


def lse_merge(o_part, lse_part, o_blk, lse_blk, out, lse_out=None, stream=None):
    """Merge.  out bf16 [B,Hq,n,d]; lse_out fp32 [B,Hq,n] or None; o_blk and
    lse_blk both None to merge the history partials alone."""
    import torch
    _need(o_part, "o_part", torch.float32)
    B, Hq, n, S, d = o_part.shape
    _need(lse_part, "lse_part", torch.float32, (B, Hq, n, S))
    if (o_blk is None) != (lse_blk is None):
        raise ValueError("o_blk and lse_blk must both be given or both be None")
    if o_blk is not None:
        _need(o_blk, "o_blk", torch.float32, (B, Hq, n, d))
        _need(lse_blk, "lse_blk", torch.float32, (B, Hq, n))
    _need(out, "out", torch.bfloat16, (B, Hq, n, d))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (B, Hq, n))
    _check(load_library().lse_merge(
        _ptr(o_part), _ptr(lse_part), S, _ptr(o_blk), _ptr(lse_blk), B, Hq, n, d, _ptr(out),
        _ptr(lse_out), _stream(stream)), "lse_merge")


def spec_attn_block_merge(q, k_blk, v_blk, parent, o_part, lse_part, out, lse_out=None,
                          sm_scale=1.0, stream=None):
    """Block pass and merge in one launch.  Shapes as spec_attn_block and
    lse_merge; out bf16 [B,Hq,n,d]; lse_out fp32 [B,Hq,n] or None."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_blk, "k_blk", torch.bfloat16)
    Hkv = k_blk.shape[1]
    _need(k_blk, "k_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(v_blk, "v_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(o_part, "o_part", torch.float32)
    S = o_part.shape[3]
    _need(o_part, "o_part", torch.float32, (B, Hq, n, S, d))
    _need(lse_part, "lse_part", torch.float32, (B, Hq, n, S))
    _need(out, "out", torch.bfloat16, (B, Hq, n, d))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (B, Hq, n))
    par = None
    if parent is not None:
        vals = [int(x) for x in parent]
        if len(vals) != n:
            raise ValueError("parent must have n entries")
        par = (ctypes.c_int32 * n)(*vals)
    _check(load_library().spec_attn_block_merge(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), ctypes.cast(par, ctypes.c_void_p) if par else None,
        _ptr(o_part), _ptr(lse_part), S, B, Hq, Hkv, n, d, float(sm_scale), _ptr(out),
        _ptr(lse_out), _stream(stream)), "spec_attn_block_merge")


def spec_attn_verify_sync_size(B, Hkv):
    """Bytes of spec_attn_verify's sync words (0 for invalid sizes)."""
    return int(load_library().spec_attn_verify_sync_size(B, Hkv))


def rv_verify_single_launch(B, Hq, Hkv, n, d, num_splits, num_cus=None):
    """True when spec_attn_verify takes the single launch; num_cus defaults
    to the current device's compute-unit count."""
    if num_cus is None:
        import torch
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    return bool(load_library().rv_verify_single_launch(B, Hq, Hkv, n, d, int(num_splits),
                                                       int(num_cus)))


def _event(ev):
    return ctypes.c_void_p(ev) if isinstance(ev, int) else ev


def spec_attn_verify(q, k_cache, v_cache, seq_lens, max_seq_len, split_len, num_splits, k_blk,
                     v_blk, parent, o_part, lse_part, sync, out, lse_out=None, sm_scale=1.0,
                     help_after_us=-1, stream=None, start_event=None, stop_event=None):
    """History pass, block pass and merge, in one launch where the device
    holds the history pass at once.  Shapes as spec_attn_prefix and
    spec_attn_block_merge; sync: a uint8 GPU tensor of at least
    spec_attn_verify_sync_size(B, Hkv) bytes, zero-filled before its first
    use (every call leaves it zero)."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_cache, "k_cache", torch.bfloat16)
    Hkv, L_max = k_cache.shape[1], k_cache.shape[2]
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, L_max, d))
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, L_max, d))
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(k_blk, "k_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(v_blk, "v_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(o_part, "o_part", torch.float32, (B, Hq, n, num_splits, d))
    _need(lse_part, "lse_part", torch.float32, (B, Hq, n, num_splits))
    _need(sync, "sync", torch.uint8)
    _need(out, "out", torch.bfloat16, (B, Hq, n, d))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (B, Hq, n))
    par = None
    if parent is not None:
        vals = [int(x) for x in parent]
        if len(vals) != n:
            raise ValueError("parent must have n entries")
        par = (ctypes.c_int32 * n)(*vals)
    _check(load_library().spec_attn_verify(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), int(max_seq_len), B, Hq, Hkv, n, d,
        L_max, float(sm_scale), int(split_len), int(num_splits), _ptr(k_blk), _ptr(v_blk),
        ctypes.cast(par, ctypes.c_void_p) if par else None, _ptr(o_part), _ptr(lse_part),
        _ptr(sync), sync.numel(), _ptr(out), _ptr(lse_out), int(help_after_us), _stream(stream),
        _event(start_event), _event(stop_event)), "spec_attn_verify")


def spec_attn_block_merge_ev(q, k_blk, v_blk, parent, o_part, lse_part, out, start_event,
                             stop_event, lse_out=None, sm_scale=1.0, stream=None):
    """spec_attn_block_merge recording two caller-created hipEvent_t handles
    (ints or ctypes pointers; None allowed) on its kernel's own dispatch."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_blk, "k_blk", torch.bfloat16)
    Hkv = k_blk.shape[1]
    _need(k_blk, "k_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(v_blk, "v_blk", torch.bfloat16, (B, Hkv, n, d))
    _need(o_part, "o_part", torch.float32)
    S = o_part.shape[3]
    _need(o_part, "o_part", torch.float32, (B, Hq, n, S, d))
    _need(lse_part, "lse_part", torch.float32, (B, Hq, n, S))
    _need(out, "out", torch.bfloat16, (B, Hq, n, d))
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (B, Hq, n))
    par = None
    if parent is not None:
        vals = [int(x) for x in parent]
        if len(vals) != n:
            raise ValueError("parent must have n entries")
        par = (ctypes.c_int32 * n)(*vals)
    _check(load_library().spec_attn_block_merge_ev(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), ctypes.cast(par, ctypes.c_void_p) if par else None,
        _ptr(o_part), _ptr(lse_part), S, B, Hq, Hkv, n, d, float(sm_scale), _ptr(out),
        _ptr(lse_out), _stream(stream), _event(start_event), _event(stop_event)),
        "spec_attn_block_merge_ev")


def spec_attn_window_workspace_size(B, Hq, n, d, sink, window):
    return int(load_library().spec_attn_window_workspace_size(B, Hq, n, d, sink, window))


def spec_attn_window(q, k_ring, v_ring, pos, sink, window, out, workspace, lse_out=None,
                     sm_scale=1.0, stream=None):
    """Drafter self-attention.  q bf16 [B,Hq,n,d]; k_ring/v_ring bf16
    [B,Hkv,cap,d]; pos int32 [B]; out bf16 [B,Hq,n,d]; lse_out fp32 [B,Hq,n];
    workspace uint8 of spec_attn_window_workspace_size bytes."""
    import torch
    _need(q, "q", torch.bfloat16)
    B, Hq, n, d = q.shape
    _need(k_ring, "k_ring", torch.bfloat16)
    Hkv, cap = k_ring.shape[1], k_ring.shape[2]
    _need(k_ring, "k_ring", torch.bfloat16, (B, Hkv, cap, d))
    _need(v_ring, "v_ring", torch.bfloat16, (B, Hkv, cap, d))
    _need(pos, "pos", torch.int32, (B,))
    _need(out, "out", torch.bfloat16, (B, Hq, n, d))
    _need(workspace, "workspace", torch.uint8)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, (B, Hq, n))
    _check(load_library().spec_attn_window(
        _ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(pos), B, Hq, Hkv, n, d, cap, int(sink),
        int(window), float(sm_scale), _ptr(out), _ptr(lse_out), _ptr(workspace),
        workspace.numel(), _stream(stream)), "spec_attn_window")


def rapid_accept_workspace_size(B, gamma, V):
    return int(load_library().rapid_accept_workspace_size(B, gamma, V))


def _accept_args(z, y, draft, r, u, n_accept, out_tokens, workspace, ratio_out, p_hat_out,
                 need_workspace=True):
    import torch
    _need(z, "z", torch.float32)
    B, g1, V = z.shape
    g = g1 - 1
    _need(y, "y", torch.float32, (B, g, V))
    _need(draft, "draft", torch.int32, (B, g))
    _need(r, "r", torch.float32, (B, g))
    _need(u, "u", torch.float32, (B, g + 1))
    _need(n_accept, "n_accept", torch.int32, (B,))
    _need(out_tokens, "out_tokens", torch.int32, (B, g + 1))
    if need_workspace:
        _need(workspace, "workspace", torch.uint8)
    if ratio_out is not None:
        _need(ratio_out, "ratio_out", torch.float32, (B, g))
    if p_hat_out is not None:
        _need(p_hat_out, "p_hat_out", torch.float32, (B, g, V))
    return B, g, V


def rapid_accept(z, y, draft, r, u, T, eta, n_accept, out_tokens, workspace, ratio_out=None,
                 p_hat_out=None, stream=None):
    """Vocabulary pass.  z fp32 [B,g+1,V]; y fp32 [B,g,V]; draft int32 [B,g];
    r fp32 [B,g]; u fp32 [B,g+1]; n_accept int32 [B]; out_tokens int32 [B,g+1];
    workspace uint8 tensor of rapid_accept_workspace_size bytes."""
    B, g, V = _accept_args(z, y, draft, r, u, n_accept, out_tokens, workspace, ratio_out,
                           p_hat_out)
    _check(load_library().rapid_accept(
        _ptr(z), _ptr(y), _ptr(draft), _ptr(r), _ptr(u), B, g, V, float(T), float(eta),
        _ptr(n_accept), _ptr(out_tokens), _ptr(ratio_out), _ptr(p_hat_out), _ptr(workspace),
        workspace.numel(), _stream(stream)), "rapid_accept")


def rapid_accept_ex(z, y, draft, r, u, T, eta, flags, n_accept, out_tokens, workspace,
                    ratio_out=None, p_hat_out=None, stream=None):
    """rapid_accept with options: RV_ACCEPT_TAIL_PRESERVE and/or
    RV_ACCEPT_PRINTED_RESIDUAL."""
    B, g, V = _accept_args(z, y, draft, r, u, n_accept, out_tokens, workspace, ratio_out,
                           p_hat_out)
    _check(load_library().rapid_accept_ex(
        _ptr(z), _ptr(y), _ptr(draft), _ptr(r), _ptr(u), B, g, V, float(T), float(eta),
        int(flags), _ptr(n_accept), _ptr(out_tokens), _ptr(ratio_out), _ptr(p_hat_out),
        _ptr(workspace), workspace.numel(), _stream(stream)), "rapid_accept_ex")


def rapid_accept_noalloc(z, y, draft, r, u, T, eta, flags, n_accept, out_tokens, ratio_out=None,
                         p_hat_out=None, stream=None):
    """rapid_accept_ex with the library's static per-device scratch as its
    workspace (no allocation by the call); calls that may overlap on one
    device must not be made."""
    B, g, V = _accept_args(z, y, draft, r, u, n_accept, out_tokens, None, ratio_out, p_hat_out,
                           need_workspace=False)
    _check(load_library().rapid_accept_noalloc(
        _ptr(z), _ptr(y), _ptr(draft), _ptr(r), _ptr(u), B, g, V, float(T), float(eta),
        int(flags), _ptr(n_accept), _ptr(out_tokens), _ptr(ratio_out), _ptr(p_hat_out),
        _stream(stream)), "rapid_accept_noalloc")


def rapid_tree_accept_workspace_size(B, n, V):
    return load_library().rapid_tree_accept_workspace_size(int(B), int(n), int(V))


def rapid_tree_accept(z, y, tokens, parent, r, u, T, eta, n_accept, path, out_tokens, workspace,
                      ratio_out=None, stream=None):
    """Acceptance over a draft tree.  z, y fp32 [B,n,V]; tokens int32 [B,n];
    parent: host sequence of n ints (parent[0] = -1); r, u fp32 [B,n];
    n_accept int32 [B]; path, out_tokens int32 [B,n]; ratio_out fp32 [B,n] or
    None; workspace uint8 of rapid_tree_accept_workspace_size bytes."""
    import torch
    _need(z, "z", torch.float32)
    B, n, V = z.shape
    _need(y, "y", torch.float32, (B, n, V))
    _need(tokens, "tokens", torch.int32, (B, n))
    _need(r, "r", torch.float32, (B, n))
    _need(u, "u", torch.float32, (B, n))
    _need(n_accept, "n_accept", torch.int32, (B,))
    _need(path, "path", torch.int32, (B, n))
    _need(out_tokens, "out_tokens", torch.int32, (B, n))
    _need(workspace, "workspace", torch.uint8)
    if ratio_out is not None:
        _need(ratio_out, "ratio_out", torch.float32, (B, n))
    if len(parent) != n:
        raise ValueError("parent must have n = %d entries" % n)
    par = (ctypes.c_int32 * n)(*[int(p) for p in parent])
    _check(load_library().rapid_tree_accept(
        _ptr(z), _ptr(y), _ptr(tokens), par, _ptr(r), _ptr(u), B, n, V, float(T), float(eta),
        _ptr(n_accept), _ptr(path), _ptr(out_tokens), _ptr(ratio_out), _ptr(workspace),
        workspace.numel(), _stream(stream)), "rapid_tree_accept")
