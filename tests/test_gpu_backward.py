"""GPU parity of the backward entry point against the oracle's analytic gradient
(itself pinned by finite differences and dense-attention gradients on the CPU)."""
import numpy as np
import pytest
import torch

from hils_inputs.configs import config
from hils_inputs.device import make_device_inputs
from oracle.hils_oracle import ref_backward
from tests.parity import assert_close, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hl():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import chunk_wise_sparse_landmark_amd as m
    m.load_library()
    return m


def _grad_case(hl, cfg, queries=None):
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=bool(cfg["causal"]),
              keep_own_chunk=bool(cfg["keep_own"]))
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"], **kw)
    dq, dk, dv, dl, db = hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"],
                                          out, dev["dout"], idx, lse, need_dbias=True, **kw)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().astype(np.int64)
    ref = ref_backward(host["q"], host["k"], host["v"], host["lmk"], host.get("bias"),
                       host["dout"], forced_idx=gi, **kw)
    tol = 1e-5 if cfg["dtype"] == "f32" else 2e-2
    for name, got, want in zip(("dq", "dk", "dv", "dlmk", "dbias"),
                               (dq, dk, dv, dl, db), ref):
        assert_close(name, to_np(got), want, "norm", tol)


def test_tiny_f32_backward(hl):
    _grad_case(hl, config("tiny_f32", dout=True))


@pytest.mark.parametrize("over", [
    dict(B=1, Hq=4, Hkv=2, d=128, Lq=320, Lkv=320, S=64, K=3, dtype="bf16", lmk="chunk_mean"),
    dict(B=2, Hq=6, Hkv=2, d=64, Lq=150, Lkv=150, S=16, K=4, dtype="bf16", lmk="iid", bias=0.5),
    dict(B=1, Hq=2, Hkv=1, d=32, Lq=70, Lkv=70, S=8, K=3, dtype="f32", lmk="iid", keep_own=0),
    dict(B=1, Hq=2, Hkv=2, d=64, Lq=45, Lkv=131, S=16, K=2, dtype="f32", lmk="iid", causal=0),
])
def test_backward_shapes(hl, over):
    cfg = dict(config("tiny_f32"), seed=31, dout=True)
    cfg.update(over)
    _grad_case(hl, cfg)
