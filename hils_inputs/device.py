"""Device copies of the synthetic inputs (torch tensors on a ROCm device).

Small tensors are generated on the host and copied; large K/V caches are
filled directly on the device by ``libhils_inputs.so`` with the same counter
generator, so the host can regenerate any slice (LazyNormalBF16).
"""
import ctypes
import os

import numpy as np
import torch

from .configs import LazyNormalBF16, make_host_inputs
from .gen import IH_INV_SD, f32_to_bf16_bits, TENSOR_IDS

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhils_inputs.so")
_lib = None


def _fill_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError("libhils_inputs.so is not built; run __graft_entry__.build()")
        _lib = ctypes.CDLL(_LIB)
        _lib.hils_inputs_fill_normal.argtypes = [
            ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
            ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        _lib.hils_inputs_fill_normal.restype = ctypes.c_int
        _lib.hils_inputs_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                          ctypes.c_void_p]
        _lib.hils_inputs_copy.restype = ctypes.c_int
        _lib.hils_inputs_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
        _lib.hils_inputs_read.restype = ctypes.c_int
        _lib.hils_inputs_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib.hils_inputs_mfma_loop.restype = ctypes.c_int
    return _lib


def to_device(x, dtype, device):
    """Host float32 array (representable in dtype) -> contiguous device tensor."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def fill_normal(t, seed, tid_name, offset=0, scale=1.0):
    """Fill a contiguous bf16/fp32 device tensor with generated N(0, scale^2) values."""
    assert t.is_contiguous()
    as_bf16 = t.dtype == torch.bfloat16
    st = torch.cuda.current_stream().cuda_stream
    rc = _fill_lib().hils_inputs_fill_normal(
        ctypes.c_void_p(t.data_ptr()), t.numel(), seed, TENSOR_IDS[tid_name], offset,
        float(IH_INV_SD), float(scale), int(as_bf16), ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError("device fill failed")
    return t


def device_copy(dst, src):
    """dst[:] = src[:] for contiguous device tensors of equal byte size (plain copy kernel)."""
    assert dst.is_contiguous() and src.is_contiguous()
    nb = src.numel() * src.element_size()
    assert nb == dst.numel() * dst.element_size()
    st = torch.cuda.current_stream().cuda_stream
    if _fill_lib().hils_inputs_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                    nb, ctypes.c_void_p(st)) != 0:
        raise RuntimeError("device copy failed")
    return dst


def make_device_inputs(cfg, device="cuda", host=None):
    """Returns (host dict, device dict).  Lazy host K/V are filled on the device."""
    host = make_host_inputs(cfg) if host is None else host
    dt = cfg["dtype"]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dev = {}
    for name in ("q", "q_ret", "lmk", "dout"):
        if host.get(name) is not None:
            dev[name] = to_device(host[name], dt, device)
    dev["bias"] = None if host.get("bias") is None else torch.from_numpy(
        np.ascontiguousarray(host["bias"], dtype=np.float32)).to(device)
    for name in ("k", "v"):
        x = host[name]
        if isinstance(x, LazyNormalBF16):
            t = torch.empty(x.shape, dtype=tdt, device=device)
            fill_normal(t, cfg["seed"], name)
            dev[name] = t
        else:
            dev[name] = to_device(x, dt, device)
    return host, dev


def make_decode_inputs_on_device(cfg, device="cuda", kv_from=None):
    """Decode workload with every large tensor generated on the device.

    q (small) and the needle rows are computed on the host; the landmark table,
    K and V are filled in place by the counter generator.  Same values as
    make_host_inputs(cfg) for the same seed.  ``kv_from``: another set whose K
    and V tensors are reused instead of generating new ones."""
    from .configs import _draw, _store, _needle_landmarks
    assert cfg["lmk"] in ("iid", "needle") and cfg["dtype"] == "bf16"
    B, Hq, Hkv, d, Lkv, S = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["Lkv"], cfg["S"]
    NC = Lkv // S
    q = _store(cfg, _draw(cfg, "q", (B, Hq, cfg["Lq"], d)))
    dev = {"q": to_device(q, "bf16", device), "bias": None}
    lmk = torch.empty((B, Hkv, NC, d), dtype=torch.bfloat16, device=device)
    fill_normal(lmk, cfg["seed"], "lmk")
    if cfg["lmk"] == "needle":
        rows = np.zeros((B, Hkv, max(NC, 1), d), dtype=np.float32)
        rows, pos = _needle_landmarks(cfg, q, rows)
        for b in range(B):
            for g in range(Hkv):
                if NC > 0 and (Lkv - 1) // S > 0:
                    c = int(pos[b, g])
                    lmk[b, g, c] = to_device(rows[b, g, c], "bf16", device)
    dev["lmk"] = lmk
    for name in ("k", "v"):
        if kv_from is not None:
            dev[name] = kv_from[name]
            continue
        t = torch.empty((B, Hkv, Lkv, d), dtype=torch.bfloat16, device=device)
        fill_normal(t, cfg["seed"], name)
        dev[name] = t
    return dev


def device_read(src, nbytes, sink, nwg):
    """Streaming read of the first `nbytes` of contiguous device tensor `src` by
    `nwg` workgroups (one word per thread into `sink`, nwg * 256 int32)."""
    assert src.is_contiguous() and sink.is_contiguous()
    assert nbytes <= src.numel() * src.element_size() and sink.numel() * sink.element_size() >= nwg * 1024
    st = torch.cuda.current_stream().cuda_stream
    if _fill_lib().hils_inputs_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                                    ctypes.c_void_p(sink.data_ptr()), nwg, ctypes.c_void_p(st)) != 0:
        raise RuntimeError("device read failed")


def device_mfma_loop(iters, sink):
    """256 workgroups x 8 waves of eight independent 16x16x32 bf16 MFMA chains,
    `iters` rounds each (one word per thread into `sink`, 256 * 512 floats)."""
    assert sink.is_contiguous() and sink.numel() * sink.element_size() >= 256 * 512 * 4
    st = torch.cuda.current_stream().cuda_stream
    if _fill_lib().hils_inputs_mfma_loop(int(iters), ctypes.c_void_p(sink.data_ptr()),
                                         ctypes.c_void_p(st)) != 0:
        raise RuntimeError("device MFMA loop failed")
