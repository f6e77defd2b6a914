"""GPU parity of the backward entry point against the oracle's analytic gradient
(itself pinned by finite differences and dense-attention gradients on the CPU)."""
import numpy as np
import pytest
import torch

from hils_inputs.configs import config
from hils_inputs.device import make_device_inputs
from oracle.hils_oracle import ref_backward, ref_forward
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


@pytest.mark.parametrize("name", ["train_8k", "train_8k_qcal", "train_32k"])
def test_train_sampled(hl, name):
    """Full training shapes through the product path (8K tokens, also with a
    separate retrieval query, and 32K tokens = 512 chunks).  dq (and dq_ret) are
    checked on sampled query rows; dk, dv of the last two chunks and dlmk, dbias
    of the second-to-last one are complete once every query of the last two
    windows is included (no earlier query can reach those chunks)."""
    cfg = config(name)
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=True)
    qr = dev.get("q_ret")
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, q_ret=qr, **kw)

    def bwd():
        return hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out, dev["dout"],
                                idx, lse, need_dbias=True, q_ret=qr, **kw)

    from bench import HipEvents, launched
    assert launched(hl, HipEvents(), "prefill_bwd_rows", bwd), "the MFMA backward path ran"
    grads = bwd()
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


def test_train_8k_full_group(hl):
    """One (batch, KV head) group of train_8k over all 8192 of its queries, so
    that every chunk's dk, dv, dlmk and dbias is complete -- including the early
    chunks that thousands of queries retrieve, which the backward splits into
    several work items and sums in its reduce pass.  The oracle runs on the host
    cores (a process pool over query blocks)."""
    from oracle.pool import default_workers, group_backward, make_pool
    cfg = config("train_8k")
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=True)
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, **kw)
    dq, dk, dv, dl, db = hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out,
                                          dev["dout"], idx, lse, need_dbias=True, **kw)
    torch.cuda.synchronize()
    b, g, G, L, S = 1, 2, cfg["Hq"] // cfg["Hkv"], cfg["Lq"], cfg["S"]
    gi = idx.cpu().numpy().astype(np.int64)[b, g]
    nitems = np.bincount(gi[gi >= 0].ravel(), minlength=L // S)
    assert nitems[0] > 8 * 64, "the early chunks are retrieved by many query tiles"
    workers = default_workers()
    with make_pool(workers) as pool:
        rdq, rdk, rdv, rdl, rdb = group_backward(pool, host, b, g, np.arange(L), gi, 4 * workers,
                                                 **kw)
    hs = slice(g * G, (g + 1) * G)
    assert_close("dq group", to_np(dq)[b, hs], rdq, "norm", 2e-2)
    assert_close("dk group", to_np(dk)[b, g], rdk, "norm", 2e-2)
    assert_close("dv group", to_np(dv)[b, g], rdv, "norm", 2e-2)
    assert_close("dlmk group", to_np(dl)[b, g], rdl, "norm", 2e-2)
    assert_close("dbias group", to_np(db)[b, g], rdb, "norm", 2e-2)
    # chunk by chunk for the most-retrieved ones (norm-relative per chunk)
    for c in np.argsort(-nitems)[:6]:
        rows = slice(c * S, (c + 1) * S)
        assert_close("dk chunk %d" % c, to_np(dk)[b, g, rows], rdk[rows], "norm", 2e-2)
        assert_close("dv chunk %d" % c, to_np(dv)[b, g, rows], rdv[rows], "norm", 2e-2)
        assert_close("dlmk chunk %d" % c, to_np(dl)[b, g, c], rdl[c], "norm", 2e-2)


@pytest.mark.parametrize("over", [dict(bias=0.3), dict(qret=8, win=8)])
def test_backward_past_256_chunks_full_group(hl, over):
    """The MFMA backward past 256 chunks (20480 tokens = 320 chunks, where it takes
    K <= 16 and lists two query windows per thread): one (batch, kv head) group
    over all its queries, so every gradient is complete, with a per-chunk bias,
    and with a separate retrieval query next to a 512-token local window (the
    landmark gradients then come from the q_ret pass)."""
    from bench import HipEvents, launched
    from oracle.pool import default_workers, group_backward, make_pool
    cfg = dict(config("train_8k"), B=1, Hq=4, Hkv=1, Lq=20480, Lkv=20480, seed=41)
    cfg.update(over)
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=True,
              local_chunks=cfg.get("win"))
    qr = dev.get("q_ret")
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"], q_ret=qr,
                                    **kw)

    def bwd():
        return hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], dev["bias"], out,
                                dev["dout"], idx, lse, need_dbias=True, q_ret=qr, **kw)

    assert launched(hl, HipEvents(), "prefill_bwd_rows", bwd), "the MFMA backward path ran"
    grads = bwd()
    torch.cuda.synchronize()
    L = cfg["Lq"]
    gi = idx.cpu().numpy().astype(np.int64)[0, 0]
    workers = default_workers()
    with make_pool(workers) as pool:
        ref = group_backward(pool, host, 0, 0, np.arange(L), gi, 4 * workers, **kw)
    names = ("dq", "dk", "dv", "dlmk", "dbias", "dq_ret")
    for n, (name, got, want) in enumerate(zip(names, grads, ref)):
        g = to_np(got)[0] if n in (0, 5) else to_np(got)[0, 0]
        assert_close(name + " group", g, want, "norm", 2e-2)


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



def _layout_ncand(cfg, i):
    win = cfg.get("win")
    win = (1 if cfg["keep_own"] else 0) if win is None else int(win)
    NC = cfg["Lkv"] // cfg["S"]
    if not cfg["causal"]:
        return NC
    own = (cfg["Lkv"] - cfg["Lq"] + i) // cfg["S"]
    return max(0, min(own - max(win - 1, 0), NC))


@pytest.mark.parametrize("over", [
    # MFMA backward path (G = 4) and the generic kernels (G = 2, fp32)
    dict(B=1, Hq=8, Hkv=2, d=128, Lq=1024, Lkv=1024, S=64, K=8, dtype="bf16", lmk="chunk_mean"),
    dict(B=1, Hq=4, Hkv=2, d=64, Lq=200, Lkv=200, S=16, K=4, dtype="f32", lmk="iid", win=2),
])
def test_backward_ignores_unusable_ids(hl, over):
    """A caller's selection with ids the query may not use -- its own or a later
    chunk (in bounds, not candidates), ids past the last chunk, negative ids and
    repeats within a row -- is read safely: those entries are skipped, so the
    gradients equal the oracle's for the selection without them."""
    cfg = dict(config("tiny_f32"), seed=61, dout=True)
    cfg.update(over)
    host, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True,
              keep_own_chunk=bool(cfg["keep_own"]), local_chunks=cfg.get("win"))
    out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, **kw)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy().copy()
    L, S, K = cfg["Lq"], cfg["S"], cfg["K"]
    NC = L // S
    rng = np.random.default_rng(9)
    bad = [lambda i: i // S, lambda i: min(NC - 1, i // S + 1), lambda i: NC + 3,
           lambda i: 10 ** 6, lambda i: -5, lambda i: 2 ** 31 - 1]
    for b in range(cfg["B"]):
        for g in range(cfg["Hkv"]):
            for i in range(L):
                row = sel[b, g, i]
                for _ in range(2):
                    s = int(rng.integers(K))
                    if rng.random() < 0.3 and row[0] >= 0:
                        row[s] = row[0] if s else row[-1]          # a repeat within the row
                    else:
                        row[s] = bad[int(rng.integers(len(bad)))](i)
    # what the backward must use: the candidates of each row, first occurrence only
    want = np.full_like(sel, -1)
    for b in range(cfg["B"]):
        for g in range(cfg["Hkv"]):
            for i in range(L):
                nc = _layout_ncand(cfg, i)
                seen, keep = set(), []
                for c in sel[b, g, i]:
                    c = int(c)
                    if 0 <= c < nc and c not in seen:
                        seen.add(c)
                        keep.append(c)
                want[b, g, i, :len(keep)] = keep
    # the forward outputs that go with that selection (the backward reads O and its
    # LSE), from the oracle, rounded as the library stores them
    from hils_inputs.device import to_device
    ro, _, rl = ref_forward(host["q"], host["k"], host["v"], host["lmk"], None,
                            forced_idx=want.astype(np.int64), **kw)
    out = to_device(ro.astype(np.float32), cfg["dtype"], dev["q"].device)
    lse = torch.from_numpy(rl.astype(np.float32)).to(dev["q"].device)
    gsel = torch.from_numpy(sel.astype(np.int32)).to(dev["q"].device)
    grads = hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out, dev["dout"],
                             gsel, lse, need_dbias=True, **kw)
    torch.cuda.synchronize()
    ref = ref_backward(host["q"], host["k"], host["v"], host["lmk"], None, host["dout"],
                       forced_idx=want.astype(np.int64), **kw)
    tol = 1e-5 if cfg["dtype"] == "f32" else 2e-2
    for name, got, w in zip(("dq", "dk", "dv", "dlmk", "dbias"), grads, ref):
        assert_close(name, to_np(got), w, "norm", tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_without_queries_zero_fills(hl, dtype):
    """seq_q = 0 (non-causal, a non-empty cache): the key-side gradients the call
    overwrites are all zero, not left as they were."""
    import ctypes
    H = hl.hils
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, Hq, Hkv, d, Lkv, S, NCc = 2, 4, 2, 64, 200, 16, 13
    p = H.make_params(batch=B, heads_q=Hq, heads_kv=Hkv, head_dim=d, seq_q=0, seq_kv=Lkv,
                      chunk_size=S, top_k=3, num_landmarks=NCc, causal=False,
                      dtype=H.HILS_BF16 if dtype == "bf16" else H.HILS_F32)
    dk = torch.full((B, Hkv, Lkv, d), float("nan"), dtype=tdt, device="cuda")
    dv = torch.full_like(dk, float("nan"))
    dl = torch.full((B, Hkv, NCc, d), float("nan"), dtype=tdt, device="cuda")
    db = torch.full((B, Hkv, NCc), float("nan"), dtype=torch.float32, device="cuda")
    lib = H.load_library()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.hils_backward(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                           None, None, None, vp(dk), vp(dv), vp(dl), vp(db), None, 0,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == H.HILS_OK, lib.hils_last_error()
    for t in (dk, dv, dl, db):
        assert bool((t == 0).all())
