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
              keep_own_chunk=bool(cfg["keep_own"]), local_chunks=cfg.get("win"))
    qr = dev.get("q_ret")
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"],
                                    q_ret=qr, **kw)
    grads = hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"],
                             out, dev["dout"], idx, lse, need_dbias=True, q_ret=qr, **kw)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().astype(np.int64)
    ref = ref_backward(host["q"], host["k"], host["v"], host["lmk"], host.get("bias"),
                       host["dout"], forced_idx=gi, q_ret=host.get("q_ret"), **kw)
    tol = 1e-5 if cfg["dtype"] == "f32" else 2e-2
    assert len(grads) == len(ref)
    for name, got, want in zip(("dq", "dk", "dv", "dlmk", "dbias", "dq_ret"), grads, ref):
        assert_close(name, to_np(got), want, "norm", tol)


def test_tiny_f32_backward(hl):
    _grad_case(hl, config("tiny_f32", dout=True))


@pytest.mark.parametrize("over", [
    dict(B=1, Hq=4, Hkv=2, d=128, Lq=320, Lkv=320, S=64, K=3, dtype="bf16", lmk="chunk_mean"),
    dict(B=2, Hq=6, Hkv=2, d=64, Lq=150, Lkv=150, S=16, K=4, dtype="bf16", lmk="iid", bias=0.5),
    dict(B=1, Hq=2, Hkv=1, d=32, Lq=70, Lkv=70, S=8, K=3, dtype="f32", lmk="iid", keep_own=0),
    dict(B=1, Hq=2, Hkv=2, d=64, Lq=45, Lkv=131, S=16, K=2, dtype="f32", lmk="iid", causal=0),
    # MFMA backward path (bf16, d = 128, S = 64, G = 4, causal, L % 64 == 0, K <= 32)
    dict(B=1, Hq=8, Hkv=2, d=128, Lq=1024, Lkv=1024, S=64, K=8, dtype="bf16", lmk="chunk_mean",
         bias=0.3),
    dict(B=2, Hq=4, Hkv=1, d=128, Lq=512, Lkv=512, S=64, K=4, dtype="bf16", lmk="iid",
         keep_own=0),
    dict(B=1, Hq=4, Hkv=1, d=128, Lq=1536, Lkv=1536, S=64, K=32, dtype="bf16", lmk="chunk_mean"),
    # chunk-aligned local window of `win` chunk slots
    dict(B=1, Hq=4, Hkv=2, d=64, Lq=150, Lkv=150, S=16, K=3, dtype="f32", lmk="iid", win=4,
         bias=0.5),
    dict(B=1, Hq=2, Hkv=2, d=64, Lq=45, Lkv=131, S=16, K=2, dtype="f32", lmk="iid", causal=0,
         win=3),
    dict(B=1, Hq=8, Hkv=2, d=128, Lq=512, Lkv=512, S=64, K=4, dtype="bf16", lmk="chunk_mean",
         win=4),
    dict(B=2, Hq=4, Hkv=1, d=128, Lq=1024, Lkv=1024, S=64, K=16, dtype="bf16", lmk="iid",
         win=8, bias=0.3),
    dict(B=1, Hq=4, Hkv=1, d=128, Lq=768, Lkv=768, S=64, K=8, dtype="bf16", lmk="chunk_mean",
         win=2),
    dict(B=1, Hq=4, Hkv=1, d=128, Lq=512, Lkv=512, S=64, K=4, dtype="bf16", lmk="iid", win=12),
    dict(B=1, Hq=4, Hkv=1, d=128, Lq=512, Lkv=512, S=64, K=4, dtype="bf16", lmk="iid", win=0),
    # separate retrieval query: generic (fp32, bf16) and MFMA paths
    dict(B=1, Hq=4, Hkv=2, d=64, Lq=150, Lkv=150, S=16, K=3, dtype="f32", lmk="iid", qret=8,
         bias=0.4, win=2),
    dict(B=1, Hq=4, Hkv=2, d=64, Lq=40, Lkv=200, S=16, K=3, dtype="bf16", lmk="iid", qret=8),
    dict(B=1, Hq=8, Hkv=2, d=128, Lq=1024, Lkv=1024, S=64, K=8, dtype="bf16", lmk="chunk_mean",
         qret=8, bias=0.3),
    dict(B=1, Hq=4, Hkv=1, d=128, Lq=768, Lkv=768, S=64, K=4, dtype="bf16", lmk="iid", qret=8,
         win=3),
])
def test_backward_shapes(hl, over):
    cfg = dict(config("tiny_f32"), seed=31, dout=True)
    cfg.update(over)
    _grad_case(hl, cfg)


@pytest.mark.parametrize("name", ["train_8k", "train_8k_qcal"])
def test_train_8k_sampled(hl, name):
    """Full training shape through the product path (and with a separate retrieval
    query).  dq (and dq_ret) are checked on sampled query rows; dk, dv of the last
    two chunks and dlmk, dbias of the second-to-last one are complete once every
    query of the last two windows is included (no earlier query can reach those
    chunks)."""
    cfg = config(name)
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=True)
    qr = dev.get("q_ret")
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, q_ret=qr, **kw)
    grads = hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out, dev["dout"], idx,
                             lse, need_dbias=True, q_ret=qr, **kw)
    dq, dk, dv, dl, db = grads[:5]
    torch.cuda.synchronize()
    L, S = cfg["Lq"], cfg["S"]
    rng = np.random.default_rng(3)
    qs = np.array(sorted(set(rng.choice(L - 2 * S, 24, replace=False).tolist())
                         | set(range(L - 2 * S, L))))
    gi = idx.cpu().numpy().astype(np.int64)[:, :, qs]
    ref = ref_backward(host["q"], host["k"], host["v"], host["lmk"], None, host["dout"],
                       forced_idx=gi, queries=qs, q_ret=host.get("q_ret"), **kw)
    rdq, rdk, rdv, rdl, rdb = ref[:5]
    assert_close("dq rows", to_np(dq)[:, :, qs], rdq[:, :, qs], "norm", 2e-2)
    if qr is not None:
        assert_close("dq_ret rows", to_np(grads[5])[:, :, qs], ref[5][:, :, qs], "norm", 2e-2)
    tail = slice(L - 2 * S, L)
    assert_close("dk tail", to_np(dk)[:, :, tail], rdk[:, :, tail], "norm", 2e-2)
    assert_close("dv tail", to_np(dv)[:, :, tail], rdv[:, :, tail], "norm", 2e-2)
    c = L // S - 2
    assert_close("dlmk", to_np(dl)[:, :, c], rdl[:, :, c], "norm", 2e-2)
    assert_close("dbias", to_np(db)[:, :, c], rdb[:, :, c], "norm", 2e-2)
    # rows past the complete chunks and chunks no query reaches get zero
    assert np.all(to_np(dl)[:, :, L // S - 1] == 0)


def test_train_8k_swa512_sampled(hl):
    """Training shape with a 512-token local window: dq on sampled rows; dk, dv of
    the last two chunks, which only the queries of the last two windows reach
    (through their local windows); dlmk, dbias of chunk NC - 9, which only the
    last window can retrieve (candidates precede the 8-slot window)."""
    cfg = config("train_8k_swa512")
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, local_chunks=8)
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, **kw)
    dq, dk, dv, dl, db = hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out,
                                          dev["dout"], idx, lse, need_dbias=True, **kw)
    torch.cuda.synchronize()
    L, S = cfg["Lq"], cfg["S"]
    NC = L // S
    rng = np.random.default_rng(4)
    tail = set(range((NC - 2) * S, L))
    qs = np.array(sorted(set(rng.choice((NC - 2) * S, 24, replace=False).tolist()) | tail))
    gi = idx.cpu().numpy().astype(np.int64)[:, :, qs]
    rdq, rdk, rdv, rdl, rdb = ref_backward(host["q"], host["k"], host["v"], host["lmk"], None,
                                           host["dout"], forced_idx=gi, queries=qs, **kw)
    assert_close("dq rows", to_np(dq)[:, :, qs], rdq[:, :, qs], "norm", 2e-2)
    kt = slice(L - 2 * S, L)
    assert_close("dk tail", to_np(dk)[:, :, kt], rdk[:, :, kt], "norm", 2e-2)
    assert_close("dv tail", to_np(dv)[:, :, kt], rdv[:, :, kt], "norm", 2e-2)
    c = NC - 9
    assert_close("dlmk", to_np(dl)[:, :, c], rdl[:, :, c], "norm", 2e-2)
    assert_close("dbias", to_np(db)[:, :, c], rdb[:, :, c], "norm", 2e-2)

