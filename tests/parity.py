"""Comparison of the HIP library with the CPU oracle (helpers for the GPU tests).

Bars (from the workload definition):
* selected chunk ids are exact, except that a chunk in the symmetric difference
  of the two sets may differ when its oracle group score lies within 1e-3 of the
  K-th largest one; for such queries the outputs are compared against the oracle
  run with the GPU's selection forced;
* outputs: fp32 within 1e-5 relative (max |diff| / max |ref| over the tensor);
  bf16 within 2e-2 absolute;
* lse (not bounded by the definition): fp32 1e-5 relative; bf16 inputs with fp32
  arithmetic 1e-3 absolute (128-term fp32 dots on bf16 values, ~1e-6 relative,
  well inside);
* gradients: norm-relative 1e-5 (fp32) / 2e-2 (bf16).
"""
import math

import numpy as np
import torch

from oracle.hils_oracle import ref_forward, hils_query

SEL_BAND = 1e-3


def tol_out(dtype):
    return ("rel", 1e-5) if dtype == "f32" else ("abs", 2e-2)


def assert_close(name, got, ref, kind, tol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "%s: non-finite pattern differs" % name
    assert np.array_equal(got[~fin], ref[~fin]), "%s: infinities differ" % name
    if not fin.any():
        return 0.0
    d = np.abs(got[fin] - ref[fin])
    if kind == "rel":
        err = d.max() / max(np.abs(ref[fin]).max(), 1e-30)
    elif kind == "norm":
        err = np.linalg.norm(got[fin] - ref[fin]) / max(np.linalg.norm(ref[fin]), 1e-30)
    else:
        err = d.max()
    assert err <= tol, "%s: %s error %.3g > %.3g" % (name, kind, err, tol)
    return err


def to_np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def check_selection(host, cfg, gpu_idx, b, g, qi, ref_idx_row):
    """Compare one query's selection; returns True when the sets are equal.

    Raises if they differ outside the tolerance band."""
    got = sorted(int(c) for c in gpu_idx if c >= 0)
    want = sorted(int(c) for c in ref_idx_row if c >= 0)
    if got == want:
        return True
    assert len(got) == len(want), ("selection size differs", b, g, qi, got, want)
    G = cfg["Hq"] // cfg["Hkv"]
    d = cfg["d"]
    scale = 1.0 / math.sqrt(d)
    lmk = host["lmk"][b, g].astype(np.float64)
    bias = None if host.get("bias") is None else host["bias"][b, g].astype(np.float64)
    qrg = None if host.get("q_ret") is None else host["q_ret"][b, g * G:(g + 1) * G, qi].astype(np.float64)
    r = hils_query(host["q"][b, g * G:(g + 1) * G, qi].astype(np.float64), host["k"][b, g],
                   host["v"][b, g], lmk, bias, qi, Lq=cfg["Lq"], Lkv=cfg["Lkv"], S=cfg["S"],
                   K=cfg["K"], causal=bool(cfg["causal"]), keep_own=bool(cfg["keep_own"]),
                   local_chunks=cfg.get("win"), scale=scale, qrg=qrg)
    gb = dict(zip(r["cand"].tolist(), r["gbar"].tolist()))
    kth = sorted(gb[c] for c in want)[0]
    for c in set(got) ^ set(want):
        assert c in gb, ("selected a non-candidate", b, g, qi, c)
        assert abs(gb[c] - kth) <= SEL_BAND, ("selection differs outside the band", b, g, qi, c,
                                              gb[c], kth)
    return False


def check_forward(host, cfg, out, idx, lse, queries=None, batches=None, heads_kv=None):
    """out/idx/lse: GPU results (numpy) over ALL queries.  Compares the sampled ones."""
    B, Hq, Hkv, Lq = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Lq"]
    G = Hq // Hkv
    qs = np.arange(Lq) if queries is None else np.asarray(sorted(queries))
    bs = list(range(B)) if batches is None else list(batches)
    gs = list(range(Hkv)) if heads_kv is None else list(heads_kv)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=bool(cfg["causal"]),
              keep_own_chunk=bool(cfg["keep_own"]), local_chunks=cfg.get("win"))
    kind, tol = tol_out(cfg["dtype"])
    lkind, ltol = ("rel", 1e-5) if cfg["dtype"] == "f32" else ("abs", 1e-3)
    swaps = 0
    for b in bs:
        for g in gs:
            ro, ri, rl = ref_forward(host["q"], host["k"], host["v"], host["lmk"], host.get("bias"),
                                     queries=qs, batches=[b], heads_kv=[g],
                                     q_ret=host.get("q_ret"), **kw)
            forced = np.array(idx[b, g][qs])[None, None]       # GPU selection for these queries
            need_forced = False
            for n, i in enumerate(qs):
                same = check_selection(host, cfg, idx[b, g, i], b, g, int(i), ri[b, g, n])
                if not same:
                    need_forced = True
                    swaps += 1
            if need_forced:
                fidx = np.full((cfg["B"], Hkv, len(qs), cfg["K"]), -1, dtype=np.int64)
                fidx[b, g] = forced[0, 0]
                ro, _, rl = ref_forward(host["q"], host["k"], host["v"], host["lmk"],
                                        host.get("bias"), queries=qs, batches=[b], heads_kv=[g],
                                        forced_idx=fidx, q_ret=host.get("q_ret"), **kw)
            hs = slice(g * G, (g + 1) * G)
            assert_close("out[b=%d,g=%d]" % (b, g), out[b, hs][:, qs], ro[b, hs], kind, tol)
            assert_close("lse[b=%d,g=%d]" % (b, g), lse[b, hs][:, qs], rl[b, hs], lkind, ltol)
    return swaps
