"""GPU parity of landmark formation and its backward against the oracle (pinned
on the CPU by the exact-at-expansion-point identity, the uniform and one-hot
limits, scipy's entropy and finite differences).

Bars: landmark keys fp32 1e-5 relative / bf16 2e-2 absolute (bf16 storage of an
average of keys of magnitude < 4); bias (fp32 output from the same inputs, S-term
fp32 sums of terms below ~30) 1e-4 absolute; gradients norm-relative 1e-5 (fp32)
/ 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

from hils_inputs.configs import config, make_landmark_inputs
from hils_inputs.device import to_device
from oracle.hils_oracle import landmark_formation, landmark_formation_backward
from tests.parity import assert_close, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hl():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import chunk_wise_sparse_landmark_amd as m
    m.load_library()
    return m


def _case(hl, cfg, lq_scale=1.0, ncap=None, with_dbias=True):
    host = make_landmark_inputs(cfg, lq_scale=lq_scale, num_landmarks=ncap, grads=True)
    dt = cfg["dtype"]
    lq, k, dlmk = (to_device(host[n], dt, "cuda") for n in ("lq", "k", "dlmk"))
    dbias = torch.from_numpy(host["dbias"]).cuda() if with_dbias else None
    S = cfg["S"]
    lmk, bias = hl.hils_landmarks(lq, k, chunk_size=S)
    dlq, dk = hl.hils_landmarks_backward(lq, k, dlmk, dbias, chunk_size=S)
    torch.cuda.synchronize()
    rl, rb = landmark_formation(host["lq"], host["k"], chunk_size=S)
    rdq, rdk = landmark_formation_backward(host["lq"], host["k"], host["dlmk"],
                                           host["dbias"] if with_dbias else None, chunk_size=S)
    kind, tol = ("rel", 1e-5) if dt == "f32" else ("abs", 2e-2)
    assert_close("lmk", to_np(lmk), rl, kind, tol)
    assert_close("bias", to_np(bias), rb, "abs", 1e-4)
    gtol = 1e-5 if dt == "f32" else 2e-2
    assert_close("dlq", to_np(dlq), rdq, "norm", gtol)
    assert_close("dk", to_np(dk), rdk, "norm", gtol)
    NC = cfg["Lkv"] // S
    # rows past the complete chunks and keys of a partial tail chunk: exactly 0
    assert np.all(to_np(lmk)[:, :, NC:] == 0) and np.all(to_np(bias)[:, :, NC:] == 0)
    assert np.all(to_np(dlq)[:, :, NC:] == 0)
    assert np.all(to_np(dk)[:, :, NC * S:] == 0)
    return to_np(lmk), to_np(bias)


def test_tiny_f32(hl):
    _case(hl, config("tiny_f32"))


def test_train_8k_full(hl):
    """Every chunk of the training shape (B=2, Hkv=4, 8192 keys, S=64, d=128, bf16)."""
    _case(hl, config("train_8k"))


@pytest.mark.parametrize("over,lq_scale,ncap", [
    (dict(Lkv=520, dtype="f32"), 1.0, 11),             # ragged tail, spare landmark rows
    (dict(Lkv=200, S=16, d=32, dtype="bf16"), 1.0, 14),
    (dict(Lkv=1024, S=256, d=64, dtype="f32"), 1.0, None),   # S * d at the 16384 bound
    (dict(Lkv=256, S=64, d=256, dtype="bf16"), 1.0, 5),      # d at its 256 bound
    (dict(Lkv=640, S=64, d=128, dtype="bf16"), 8.0, None),   # sharp in-chunk distributions
    (dict(B=2, Hkv=3, Lkv=700, S=64, d=128, dtype="bf16"), 1.0, 13),  # wave path, ragged
    (dict(Lkv=50, S=64, d=128, dtype="bf16"), 2.0, 3),       # wave path, no complete chunk
    (dict(Lkv=333, S=48, d=96, dtype="f32"), 3.0, 9),
    (dict(Lkv=40, S=64, d=64, dtype="f32"), 1.0, 2),         # no complete chunk
])
def test_shapes(hl, over, lq_scale, ncap):
    cfg = dict(config("tiny_f32"), seed=17)
    cfg.update(over)
    _case(hl, cfg, lq_scale=lq_scale, ncap=ncap)


def test_no_dbias_and_multi_head(hl):
    cfg = dict(config("tiny_f32"), B=2, Hkv=3, Lkv=300, S=32, d=64, dtype="bf16", seed=5)
    _case(hl, cfg, with_dbias=False, ncap=12)


def test_chunk_of_one_key(hl):
    """S = 1: p = 1, the landmark is the key itself and the bias is 0."""
    cfg = dict(config("tiny_f32"), Lkv=37, S=1, d=64, dtype="f32", seed=9)
    lmk, bias = _case(hl, cfg)
    host = make_landmark_inputs(cfg)
    assert np.array_equal(lmk, host["k"])
    assert np.all(bias == 0)


def test_empty_is_a_no_op(hl):
    lq = torch.empty((0, 2, 4, 64), device="cuda")
    k = torch.empty((0, 2, 256, 64), device="cuda")
    lmk, bias = hl.hils_landmarks(lq, k, chunk_size=64)
    assert lmk.shape == lq.shape and bias.shape == (0, 2, 4)
