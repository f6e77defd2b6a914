"""The allocation-free decode entry point (hils_decode_noalloc) against hils_decode:
the same kernels on the library's fixed scratch array instead of a workspace, so
selections, outputs and LSEs must agree bit for bit.  Two calls in a row, the
second smaller, since every call on a GPU shares that array."""
import ctypes

import numpy as np
import pytest
import torch

from hils_inputs.configs import config
from hils_inputs.device import make_device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hl():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import chunk_wise_sparse_landmark_amd as m
    m.load_library()
    return m


def _both(hl, cfg):
    _, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], keep_own_chunk=True, local_chunks=cfg.get("win"))
    o1, i1, l1 = hl.hils_decode(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"], **kw)
    torch.cuda.synchronize()
    H = hl.hils
    p = H._params_from(dev["q"], dev["k"], dev["lmk"], cfg["S"], cfg["K"], True, True, 0.0,
                       cfg.get("win"))
    o2 = torch.full_like(o1, float("nan"))
    i2 = torch.full_like(i1, -7)
    l2 = torch.full_like(l1, float("nan"))
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    lib = H.load_library()
    st = lib.hils_decode_noalloc(ctypes.byref(p), vp(dev["q"]), None, vp(dev["k"]), vp(dev["v"]),
                                 vp(dev["lmk"]), vp(dev["bias"]), vp(o2), vp(i2), vp(l2),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == H.HILS_OK, lib.hils_last_error()
    np.testing.assert_array_equal(i2.cpu().numpy(), i1.cpu().numpy())
    assert torch.equal(o2.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l2, l1)


@pytest.mark.parametrize("first,second", [
    # G = 4 (MFMA attention), a local window, 2 then 1 score splits
    (dict(B=4, Lkv=70000, K=32, win=2, seed=71), dict(B=2, Lkv=20000, K=16, win=1, seed=72)),
    # G = 2 (general attention), many score splits then few
    (dict(B=2, Hq=8, Hkv=4, Lkv=300000, K=64, win=3, seed=73),
     dict(B=1, Hq=8, Hkv=4, Lkv=5000, K=8, win=1, seed=74)),
    # 16 x 8 pairs: one scoring workgroup per pair writes the selection (no
    # merge launch), then a split call
    (dict(Lkv=70000, K=32, win=1, seed=75), dict(B=2, Lkv=20000, K=16, win=2, seed=76)),
])
def test_noalloc_decode_matches_decode(hl, first, second):
    _both(hl, config("decode_128k", **first))
    _both(hl, config("decode_128k", **second))


def test_noalloc_decode_rejects_sizes_past_its_scratch(hl):
    H = hl.hils
    lib = H.load_library()
    cap = int(lib.hils_decode_noalloc_scratch_bytes())
    p = H.make_params(batch=64, heads_q=32, heads_kv=8, head_dim=128, seq_q=1, seq_kv=1 << 20,
                      chunk_size=64, top_k=64, num_landmarks=1 << 14, local_chunks=8)
    assert H.hils_workspace_size(p, H.HILS_OP_DECODE) > cap
    fake = ctypes.c_void_p(1 << 20)
    st = lib.hils_decode_noalloc(ctypes.byref(p), fake, None, fake, fake, fake, None, fake, fake,
                                 None, None)
    assert st == H.HILS_ERR_UNSUPPORTED
    assert b"scratch" in lib.hils_last_error()
