"""Thin ctypes binding of libhils.so (argument marshalling only).

The functions carry the C names: ``hils_forward``, ``hils_decode``,
``hils_backward``, ``hils_workspace_size``.  Tensors must be contiguous
torch tensors on a ROCm device (bf16 or fp32); outputs and the workspace are
allocated with torch when not given, and every kernel runs on torch's current
stream.  Nothing here computes any part of the method; a missing library is an
error, never a fallback.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhils.so")

HILS_OK, HILS_ERR_INVALID_ARG, HILS_ERR_UNSUPPORTED, HILS_ERR_WORKSPACE, HILS_ERR_HIP = range(5)
HILS_F32, HILS_BF16 = 0, 1
HILS_OP_FORWARD, HILS_OP_DECODE, HILS_OP_BACKWARD = 0, 1, 2

EXPORTS = ("hils_workspace_size", "hils_forward", "hils_decode", "hils_decode_noalloc",
           "hils_decode_noalloc_scratch_bytes", "hils_backward",
           "hils_landmarks", "hils_landmarks_backward", "hils_profile_kernel", "hils_profile_count", "hils_status_string", "hils_last_error")

KERNEL_IDS = {"generic_select": 1, "generic_attend": 2, "generic_bwd_rows": 3,
              "generic_bwd_chunks": 4, "decode_score": 5, "decode_merge": 6, "decode_attend": 7,
              "prefill_select": 8, "prefill_attend": 9, "prefill_bwd_rows": 10,
              "prefill_bwd_chunks": 11, "landmarks": 12, "landmarks_bwd": 13}


class HilsParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_q", ctypes.c_int32), ("seq_kv", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_landmarks", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("local_chunks", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class HilsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status


_STATUS = {0: "HILS_OK", 1: "HILS_ERR_INVALID_ARG", 2: "HILS_ERR_UNSUPPORTED",
           3: "HILS_ERR_WORKSPACE", 4: "HILS_ERR_HIP"}
_lib = None


def load_library(path=None):
    """Load libhils.so (built in-tree by chunk_wise_sparse_landmark_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libhils.so is not built (%s); run __graft_entry__.build()" % p)
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    P = ctypes.POINTER(HilsParams)
    lib.hils_workspace_size.argtypes = [P, i32]
    lib.hils_workspace_size.restype = sz
    lib.hils_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hils_forward.restype = ctypes.c_int
    lib.hils_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hils_decode.restype = ctypes.c_int
    lib.hils_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hils_decode_noalloc.restype = ctypes.c_int
    lib.hils_decode_noalloc_scratch_bytes.argtypes = []
    lib.hils_decode_noalloc_scratch_bytes.restype = sz
    lib.hils_backward.argtypes = [P] + [vp] * 16 + [vp, sz, vp]
    lib.hils_backward.restype = ctypes.c_int
    lib.hils_landmarks.argtypes = [P, vp, vp, vp, vp, vp]
    lib.hils_landmarks.restype = ctypes.c_int
    lib.hils_landmarks_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.hils_landmarks_backward.restype = ctypes.c_int
    lib.hils_status_string.argtypes = [ctypes.c_int]
    lib.hils_status_string.restype = ctypes.c_char_p
    lib.hils_profile_kernel.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32]
    lib.hils_profile_kernel.restype = ctypes.c_int
    lib.hils_profile_count.argtypes = []
    lib.hils_profile_count.restype = i32
    lib.hils_last_error.argtypes = []
    lib.hils_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _local(keep_own_chunk, local_chunks):
    """Width of the local window in chunk slots: local_chunks if given, else 1 for
    keep_own_chunk (the own chunk only) and 0 without it."""
    return (1 if keep_own_chunk else 0) if local_chunks is None else int(local_chunks)


def make_params(*, batch, heads_q, heads_kv, head_dim, seq_q, seq_kv, chunk_size, top_k,
                num_landmarks, causal=True, keep_own_chunk=True, scale=0.0, dtype=HILS_BF16,
                local_chunks=None):
    return HilsParams(batch, heads_q, heads_kv, head_dim, seq_q, seq_kv, chunk_size, top_k,
                      num_landmarks, int(bool(causal)), _local(keep_own_chunk, local_chunks),
                      float(scale or 0.0), dtype)


def _check(status):
    if status != HILS_OK:
        msg = load_library().hils_last_error().decode()
        raise HilsError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return HILS_BF16
    if t.dtype == torch.float32:
        return HILS_F32
    raise TypeError("HiLS tensors must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(name, t, dtype, shape, device):
    """A tensor argument the library reads or writes through a raw pointer: it must
    have exactly the dtype, shape and device the call implies and be contiguous
    (the kernels index it as a dense row-major array).  None passes."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _params_from(q, k, lmk, chunk_size, top_k, causal, keep_own_chunk, scale, local_chunks=None):
    if q.dim() != 4 or k.dim() != 4 or lmk.dim() != 4:
        raise ValueError("q, k and lmk must be 4-d [batch, heads, length, head_dim]")
    B, Hq, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    _dtype_code(q)
    _require("q", q, q.dtype, q.shape, q.device)
    _require("k", k, q.dtype, (B, Hkv, Lkv, d), q.device)
    _require("lmk", lmk, q.dtype, (B, Hkv, lmk.shape[2], d), q.device)
    return make_params(batch=B, heads_q=Hq, heads_kv=Hkv, head_dim=d, seq_q=Lq, seq_kv=Lkv,
                       chunk_size=chunk_size, top_k=top_k, num_landmarks=lmk.shape[2],
                       causal=causal, keep_own_chunk=keep_own_chunk, scale=scale,
                       dtype=_dtype_code(q), local_chunks=local_chunks)


def hils_workspace_size(params, op):
    return int(load_library().hils_workspace_size(ctypes.byref(params), op))


def _workspace(params, op, device, ws):
    need = hils_workspace_size(params, op)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if ws is not None:
        _require("ws", ws, torch.uint8, (ws.numel(),), device)
    return ws, need if ws is None else ws.numel()


def _check_qret(q, q_ret):
    _require("q_ret", q_ret, q.dtype, q.shape, q.device)


def _fwd(entry, op, q, k, v, lmk, lmk_bias, chunk_size, top_k, causal, keep_own_chunk, scale,
         out, sel_idx, lse, ws, stream, local_chunks, q_ret):
    p = _params_from(q, k, lmk, chunk_size, top_k, causal, keep_own_chunk, scale, local_chunks)
    _check_qret(q, q_ret)
    B, Hq, Lq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _require("v", v, q.dtype, k.shape, dev)
    _require("lmk_bias", lmk_bias, torch.float32, lmk.shape[:3], dev)
    _require("out", out, q.dtype, q.shape, dev)
    _require("sel_idx", sel_idx, torch.int32, (B, Hkv, Lq, top_k), dev)
    _require("lse", lse, torch.float32, (B, Hq, Lq), dev)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, Hkv, Lq, top_k), dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev)
    ws, nbytes = _workspace(p, op, dev, ws)
    lib = load_library()
    st = getattr(lib, entry)(ctypes.byref(p), _ptr(q), _ptr(q_ret), _ptr(k), _ptr(v), _ptr(lmk),
                             _ptr(lmk_bias), _ptr(out), _ptr(sel_idx), _ptr(lse), _ptr(ws),
                             nbytes, _stream(stream))
    _check(st)
    return out, sel_idx, lse


def hils_forward(q, k, v, lmk, lmk_bias=None, *, chunk_size, top_k, causal=True,
                 keep_own_chunk=True, scale=0.0, out=None, sel_idx=None, lse=None, ws=None,
                 stream=None, local_chunks=None, q_ret=None):
    """HiLS forward: returns (out [B,Hq,Lq,d], sel_idx int32 [B,Hkv,Lq,K], lse fp32 [B,Hq,Lq]).

    ``local_chunks`` (default: 1 with keep_own_chunk, else 0) is the width of the
    chunk-aligned local window in chunk slots; ``q_ret`` (shape of q) is an
    optional separate retrieval query for the chunk scores."""
    return _fwd("hils_forward", HILS_OP_FORWARD, q, k, v, lmk, lmk_bias, chunk_size, top_k,
                causal, keep_own_chunk, scale, out, sel_idx, lse, ws, stream, local_chunks, q_ret)


def hils_decode(q, k, v, lmk, lmk_bias=None, *, chunk_size, top_k, keep_own_chunk=True,
                scale=0.0, out=None, sel_idx=None, lse=None, ws=None, stream=None,
                local_chunks=None, q_ret=None):
    """Single-token decode over the cache k, v (q: [B,Hq,1,d], position seq_kv-1)."""
    return _fwd("hils_decode", HILS_OP_DECODE, q, k, v, lmk, lmk_bias, chunk_size, top_k,
                True, keep_own_chunk, scale, out, sel_idx, lse, ws, stream, local_chunks, q_ret)


def hils_decode_noalloc(q, k, v, lmk, lmk_bias=None, *, chunk_size, top_k, keep_own_chunk=True,
                        scale=0.0, out=None, sel_idx=None, lse=None, stream=None,
                        local_chunks=None, q_ret=None):
    """hils_decode on the library's own fixed scratch array (no workspace); outputs
    are allocated here only when not given."""
    p = _params_from(q, k, lmk, chunk_size, top_k, True, keep_own_chunk, scale, local_chunks)
    _check_qret(q, q_ret)
    B, Hq, Lq, d = q.shape
    dev = q.device
    _require("v", v, q.dtype, k.shape, dev)
    _require("lmk_bias", lmk_bias, torch.float32, lmk.shape[:3], dev)
    _require("out", out, q.dtype, q.shape, dev)
    _require("sel_idx", sel_idx, torch.int32, (B, k.shape[1], Lq, top_k), dev)
    _require("lse", lse, torch.float32, (B, Hq, Lq), dev)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, k.shape[1], Lq, top_k), dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev)
    _check(load_library().hils_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(q_ret), _ptr(k),
                                              _ptr(v), _ptr(lmk), _ptr(lmk_bias), _ptr(out),
                                              _ptr(sel_idx), _ptr(lse), _stream(stream)))
    return out, sel_idx, lse


def hils_backward(q, k, v, lmk, lmk_bias, out, dout, sel_idx, lse, *, chunk_size, top_k,
                  causal=True, keep_own_chunk=True, scale=0.0, need_dbias=None, ws=None,
                  stream=None, local_chunks=None, q_ret=None):
    """Gradients (dq, dk, dv, dlmk, dbias-or-None) of <dout, out> with the selection fixed;
    with ``q_ret`` a sixth tensor dq_ret follows and dq is the token-attention part."""
    p = _params_from(q, k, lmk, chunk_size, top_k, causal, keep_own_chunk, scale, local_chunks)
    _check_qret(q, q_ret)
    B, Hq, Lq, d = q.shape
    dev = q.device
    _require("v", v, q.dtype, k.shape, dev)
    _require("lmk_bias", lmk_bias, torch.float32, lmk.shape[:3], dev)
    _require("out", out, q.dtype, q.shape, dev)
    _require("dout", dout, q.dtype, q.shape, dev)
    _require("sel_idx", sel_idx, torch.int32, (B, k.shape[1], Lq, top_k), dev)
    _require("lse", lse, torch.float32, (B, Hq, Lq), dev)
    dq, dk, dv, dlmk = (torch.empty(t.shape, dtype=t.dtype, device=dev) for t in (q, k, k, lmk))
    dqr = torch.empty(q.shape, dtype=q.dtype, device=dev) if q_ret is not None else None
    if need_dbias is None:
        need_dbias = lmk_bias is not None
    dbias = torch.empty(lmk.shape[:3], dtype=torch.float32, device=q.device) if need_dbias else None
    ws, nbytes = _workspace(p, HILS_OP_BACKWARD, q.device, ws)
    lib = load_library()
    st = lib.hils_backward(ctypes.byref(p), _ptr(q), _ptr(q_ret), _ptr(k), _ptr(v), _ptr(lmk),
                           _ptr(lmk_bias), _ptr(out), _ptr(dout), _ptr(sel_idx), _ptr(lse),
                           _ptr(dq), _ptr(dqr), _ptr(dk), _ptr(dv), _ptr(dlmk), _ptr(dbias),
                           _ptr(ws), nbytes, _stream(stream))
    _check(st)
    if q_ret is not None:
        return dq, dk, dv, dlmk, dbias, dqr
    return dq, dk, dv, dlmk, dbias


def _landmark_params(lq, k, chunk_size, scale):
    if lq.dim() != 4 or k.dim() != 4:
        raise ValueError("lq and k must be 4-d [batch, kv heads, length, head_dim]")
    if lq.dtype != k.dtype:
        raise TypeError("lq and k must share a dtype")
    B, Hkv, Lkv, d = k.shape
    _dtype_code(k)
    _require("k", k, k.dtype, k.shape, k.device)
    _require("lq", lq, k.dtype, (B, Hkv, lq.shape[2], d), k.device)
    return make_params(batch=B, heads_q=Hkv, heads_kv=Hkv, head_dim=d, seq_q=0, seq_kv=Lkv,
                       chunk_size=chunk_size, top_k=1, num_landmarks=lq.shape[2], scale=scale,
                       dtype=_dtype_code(k))


def hils_landmarks(lq, k, *, chunk_size, scale=0.0, need_bias=True, stream=None):
    """Landmark keys [B,Hkv,NCcap,d] and entropy biases (fp32 [B,Hkv,NCcap], or None)
    from landmark queries lq [B,Hkv,NCcap,d] and keys k [B,Hkv,Lkv,d]."""
    p = _landmark_params(lq, k, chunk_size, scale)
    lmk = torch.empty(lq.shape, dtype=lq.dtype, device=lq.device)
    bias = torch.empty(lq.shape[:3], dtype=torch.float32, device=lq.device) if need_bias else None
    _check(load_library().hils_landmarks(ctypes.byref(p), _ptr(lq), _ptr(k), _ptr(lmk), _ptr(bias),
                                         _stream(stream)))
    return lmk, bias


def hils_landmarks_backward(lq, k, dlmk, dbias=None, *, chunk_size, scale=0.0, stream=None):
    """Gradients (dlq, dk) of the landmark formation; dk is its own contribution."""
    p = _landmark_params(lq, k, chunk_size, scale)
    _require("dlmk", dlmk, lq.dtype, lq.shape, lq.device)
    _require("dbias", dbias, torch.float32, lq.shape[:3], lq.device)
    dlq = torch.empty(lq.shape, dtype=lq.dtype, device=lq.device)
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device)
    _check(load_library().hils_landmarks_backward(ctypes.byref(p), _ptr(lq), _ptr(k), _ptr(dlmk),
                                                  _ptr(dbias), _ptr(dlq), _ptr(dk),
                                                  _stream(stream)))
    return dlq, dk


def hils_profile_kernel(kernel, starts, stops):
    """Arm per-launch event recording for a kernel family (names in KERNEL_IDS).

    ``starts``/``stops``: equal-length lists of raw hipEvent_t handles (ints)."""
    lib = load_library()
    n = len(starts)
    arr = ctypes.c_void_p * max(n, 1)
    a, b = arr(*starts), arr(*stops)
    kid = KERNEL_IDS[kernel] if isinstance(kernel, str) else int(kernel)
    _check(lib.hils_profile_kernel(kid, a, b, n))
    return (a, b)   # keep the arrays alive while armed


def hils_profile_count():
    return int(load_library().hils_profile_count())


def default_scale(d):
    return 1.0 / math.sqrt(d)
