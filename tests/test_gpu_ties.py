"""GPU checks of the deterministic tie rule of the group top-K: on an exact score
tie the lower chunk id wins [HSADR §4 "Architecture": the heads of a GQA group
share one retrieved set, which must not depend on the order of evaluation].

The inputs plant exact ties (hils_inputs.configs.plant_ties): either every
landmark row equal (every candidate ties, so the lowest ids win) or a four-way
tie exactly at the K-th score, with its members spread over different lanes,
candidate blocks and (decode) score splits.  The selected ids are compared with
the oracle's BIT FOR BIT -- no tolerance band -- and the outputs on that
selection as in the other parity tests.
"""
import numpy as np
import pytest
import torch

from hils_inputs.configs import config, make_host_inputs, plant_ties
from hils_inputs.device import make_device_inputs
from oracle.hils_oracle import ref_forward
from tests.parity import check_forward, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hl():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import chunk_wise_sparse_landmark_amd as m
    m.load_library()
    return m


def _run(hl, cfg, dev, entry):
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], keep_own_chunk=bool(cfg["keep_own"]),
              local_chunks=cfg.get("win"))
    if entry == "forward":
        out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"],
                                        causal=bool(cfg["causal"]), **kw)
    else:
        out, idx, lse = hl.hils_decode(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"], **kw)
    torch.cuda.synchronize()
    return to_np(out), idx.cpu().numpy(), lse.cpu().numpy()


def _ncand(cfg, i):
    win = cfg.get("win")
    win = (1 if cfg["keep_own"] else 0) if win is None else int(win)
    NC = cfg["Lkv"] // cfg["S"]
    if not cfg["causal"]:
        return NC
    own = (cfg["Lkv"] - cfg["Lq"] + i) // cfg["S"]
    return max(0, min(own - max(win - 1, 0), NC))


def _exact(host, cfg, idx, qs, planted, mode):
    """Selections of the queries ``qs`` equal the oracle's bit for bit."""
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=bool(cfg["causal"]),
              keep_own_chunk=bool(cfg["keep_own"]), local_chunks=cfg.get("win"))
    K = cfg["K"]
    kth_ties = 0
    for b in range(cfg["B"]):
        for g in range(cfg["Hkv"]):
            _, ri, _ = ref_forward(host["q"], host["k"], host["v"], host["lmk"], host["bias"],
                                   queries=qs, batches=[b], heads_kv=[g], **kw)
            got = idx[b, g][qs]
            np.testing.assert_array_equal(got, ri[b, g], err_msg="b=%d g=%d" % (b, g))
            for n, i in enumerate(qs):
                nc = _ncand(cfg, int(i))
                if mode == "all_equal":
                    want = np.full(K, -1)
                    want[:min(K, nc)] = np.arange(min(K, nc))
                    np.testing.assert_array_equal(got[n], want)
                else:
                    strong, tie = planted[(b, g)]
                    vis_s = [c for c in strong if c < nc]
                    vis_t = [c for c in tie if c < nc]
                    if len(vis_s) == K - 1 and len(vis_t) >= 2:
                        # the tie sits exactly at the K-th position: its lowest id wins
                        kth_ties += 1
                        assert sorted(vis_s + [vis_t[0]]) == sorted(int(c) for c in got[n]), (b, g, i)
    return kth_ties


def _queries(cfg, n_rand, seed):
    L = cfg["Lq"]
    if L <= 400:
        return np.arange(L)
    rng = np.random.default_rng(seed)
    return np.array(sorted(set(range(0, 70)) | set(range(L - 40, L))
                           | set(rng.choice(L, n_rand, replace=False).tolist())))


def _case(**kw):
    base = dict(B=1, Hq=4, Hkv=1, d=128, Lq=4096, Lkv=4096, S=64, K=16, causal=1, keep_own=1,
                dtype="bf16", lmk="iid", seed=41)
    base.update(kw)
    return base


# MFMA prefill path (G = 4): 64, 128, 256 and 512 chunks give 1, 2, 4 and 8
# candidate blocks per lane in the select kernel's search
PREFILL = {
    "r1_all_equal": (_case(Lq=4096, Lkv=4096), "all_equal"),
    "r1_kth": (_case(Lq=4096, Lkv=4096, seed=42), "kth"),
    "r2_all_equal_k32": (_case(Lq=8192, Lkv=8192, K=32), "all_equal"),
    "r2_kth": (_case(Lq=8192, Lkv=8192, seed=43), "kth"),
    "r2_kth_k32_win3": (_case(Lq=8192, Lkv=8192, K=32, win=3, seed=44), "kth"),
    "r4_all_equal": (_case(Lq=16384, Lkv=16384), "all_equal"),
    "r4_kth": (_case(Lq=16384, Lkv=16384, seed=45), "kth"),
    "r8_all_equal": (_case(Lq=32768, Lkv=32768), "all_equal"),
    "r8_kth_k32": (_case(Lq=32768, Lkv=32768, K=32, seed=46), "kth"),
    # shape-generic select kernel: G = 2, a ragged length, fp32
    "generic_g2_all_equal": (_case(Hq=4, Hkv=2, d=64, Lq=1000, Lkv=1000, S=16, K=8), "all_equal"),
    "generic_g2_kth": (_case(Hq=4, Hkv=2, d=64, Lq=1000, Lkv=1000, S=16, K=8, seed=47), "kth"),
    "generic_f32_kth": (_case(Hq=2, Hkv=2, d=64, Lq=400, Lkv=400, S=16, K=5, dtype="f32",
                              seed=48), "kth"),
}


@pytest.mark.parametrize("name", sorted(PREFILL))
def test_prefill_ties(hl, name):
    cfg, mode = PREFILL[name]
    print("tie case", name, flush=True)
    host = make_host_inputs(cfg)
    planted = plant_ties(host, cfg, mode)
    host, dev = make_device_inputs(cfg, host=host)
    out, idx, lse = _run(hl, cfg, dev, "forward")
    qs = _queries(cfg, 60, 7)
    n = _exact(host, cfg, idx, qs, planted, mode)
    if mode == "kth":
        assert n > 0, "no sampled query had the tie at its K-th position"
    assert check_forward(host, cfg, out, idx, lse, queries=qs) == 0


# decode: 8 score splits (single-wave merge), 128 splits (16-wave merge), and
# one eight-wave scoring workgroup per (b, kv head) that writes the selection
# itself (16 x 8 pairs, at most 2048 candidates); the tied chunks sit in
# different splits or waves
DECODE = {
    "fused_all_equal": (config("decode_128k", lmk="iid", seed=57), "all_equal"),
    "fused_kth": (config("decode_128k", Lkv=70000, lmk="iid", seed=58), "kth"),
    "split8_all_equal": (config("decode_128k", B=2, Hkv=2, Hq=8, lmk="iid", seed=51), "all_equal"),
    "split8_kth": (config("decode_128k", B=2, Hkv=2, Hq=8, lmk="iid", seed=52), "kth"),
    "split128_all_equal_k64": (config("decode_4m", Hkv=2, Hq=8, Lkv=1 << 21, lmk="iid", seed=53),
                               "all_equal"),
    "split128_kth_k64": (config("decode_4m", Hkv=2, Hq=8, Lkv=1 << 21, lmk="iid", seed=54), "kth"),
    "g2_split_kth": (config("decode_128k", B=1, Hkv=2, Hq=4, Lkv=1 << 19, lmk="iid", seed=55),
                     "kth"),
}


@pytest.mark.parametrize("name", sorted(DECODE))
def test_decode_ties(hl, name):
    cfg, mode = DECODE[name]
    print("tie case", name, flush=True)
    host = make_host_inputs(cfg)
    planted = plant_ties(host, cfg, mode)
    host, dev = make_device_inputs(cfg, host=host)
    out, idx, lse = _run(hl, cfg, dev, "decode")
    n = _exact(host, cfg, idx, np.arange(1), planted, mode)
    if mode == "kth":
        assert n == cfg["B"] * cfg["Hkv"]
    assert check_forward(host, cfg, out, idx, lse) == 0
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("G,win,B,Hkv", [(4, 1, 2, 2), (4, 8, 2, 2), (2, 3, 2, 2), (4, 1, 16, 8)])
def test_decode_values_one_give_output_one(hl, G, win, B, Hkv):
    """V = 1 gives O = 1 through the split decode path (and, at 16 x 8 pairs, the
    single-workgroup selection): the fusion weights of the selected chunks and
    the window sum to one (bf16 P and O rounding only)."""
    cfg = config("decode_128k", B=B, Hkv=Hkv, Hq=Hkv * G, Lkv=70000, K=32, win=win, seed=56)
    host, dev = make_device_inputs(cfg)
    dev["v"] = torch.ones_like(dev["v"])
    out, idx, lse = _run(hl, cfg, dev, "decode")
    assert np.abs(out - 1.0).max() <= 2.0 ** -9 + 2.0 ** -8 + 1e-6
