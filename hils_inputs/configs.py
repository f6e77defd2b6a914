"""The synthetic HiLS workloads and their seeded input recipes.

Every workload is defined by a small dict of sizes plus a landmark recipe:

* ``iid``        landmark keys drawn N(0, 1) independently of the keys;
* ``chunk_mean`` landmark of chunk c = mean of that chunk's S keys (in fp64)
                 + N(0, 0.1^2) noise, rounded once to the storage type;
* ``needle``     landmark keys N(0, 1), plus one planted chunk per (b, kv head)
                 whose landmark points along the group's mean query with
                 cosine 0.9 and norm sqrt(d).

Queries are N(0, 1) and independent across positions, or, with ``qcorr`` = rho,
a first-order autoregressive sequence along the positions of each head
(q_0 = e_0, q_i = rho q_{i-1} + sqrt(1 - rho^2) e_i, e ~ N(0, 1) from the same
draws), which keeps each q_i ~ N(0, 1) but makes adjacent queries similar, so
that they retrieve mostly the same chunks.

With ``qret`` = r a separate retrieval query is drawn as a rank-r adaptation of
each head's query, q_ret = q + A (B^T q) with A, B [d, r] per head (entries
N(0, 1/r) / 2 and N(0, 1/d)), the form of a low-rank query calibration.

No part of the attention method is computed here.
"""
import math
import numpy as np

from .gen import (TENSOR_IDS, normal_f32, f32_to_bf16_bits, bf16_bits_to_f32,
                  uniform_u64)

CONFIGS = {
    # small case the oracle finishes in seconds; fp32 end to end
    "tiny_f32": dict(B=1, Hq=2, Hkv=2, d=64, Lq=512, Lkv=512, S=64, K=2,
                     causal=1, keep_own=1, dtype="f32", lmk="iid", seed=0),
    # causal prefill, GQA 32/8
    "prefill_8k": dict(B=1, Hq=32, Hkv=8, d=128, Lq=8192, Lkv=8192, S=64, K=16,
                       causal=1, keep_own=1, dtype="bf16", lmk="chunk_mean", seed=1),
    # batch-16 single-token decode over a 128K cache
    "decode_128k": dict(B=16, Hq=32, Hkv=8, d=128, Lq=1, Lkv=131072, S=64, K=32,
                        causal=1, keep_own=1, dtype="bf16", lmk="needle", seed=2),
    # batch-1 decode over a 4M-token cache (16 GiB of K/V)
    "decode_4m": dict(B=1, Hq=32, Hkv=8, d=128, Lq=1, Lkv=4194304, S=64, K=64,
                      causal=1, keep_own=1, dtype="bf16", lmk="needle", seed=3),
    # training step (forward + backward), landmarks are a leaf tensor
    "train_8k": dict(B=2, Hq=16, Hkv=4, d=128, Lq=8192, Lkv=8192, S=64, K=16,
                     causal=1, keep_own=1, dtype="bf16", lmk="chunk_mean", seed=4,
                     dout=True),
    # longer prefill with the same generator as prefill_8k
    "prefill_32k": dict(B=1, Hq=32, Hkv=8, d=128, Lq=32768, Lkv=32768, S=64, K=16,
                        causal=1, keep_own=1, dtype="bf16", lmk="chunk_mean", seed=5),
}
# the same workloads with a 512-token chunk-aligned local window (8 chunk slots:
# the own chunk and the 7 before it) next to the top-K retrieval
for _name in ("prefill_8k", "decode_128k", "train_8k"):
    CONFIGS[_name + "_swa512"] = dict(CONFIGS[_name], win=8)
# prefill_8k with correlated adjacent queries (rho = 0.98: adjacent queries share
# about 88% of their selected chunks on this generator)
CONFIGS["prefill_8k_corr"] = dict(CONFIGS["prefill_8k"], qcorr=0.98)
# the training step with a separate rank-8 retrieval query
CONFIGS["train_8k_qcal"] = dict(CONFIGS["train_8k"], qret=8)
# the training step at 32K tokens (512 chunks), batch 1
CONFIGS["train_32k"] = dict(CONFIGS["train_8k"], B=1, Lq=32768, Lkv=32768, seed=6)


def config(name, **overrides):
    cfg = dict(CONFIGS[name], name=name)
    cfg.update(overrides)
    if "Lq" not in overrides and cfg["Lq"] != 1 and "Lkv" in overrides:
        cfg["Lq"] = cfg["Lkv"]
    return cfg


def _draw(cfg, tid_name, shape, scale=1.0, offset=0):
    n = int(np.prod(shape))
    x = normal_f32(cfg["seed"], TENSOR_IDS[tid_name],
                   np.arange(offset, offset + n, dtype=np.uint64), scale)
    return x.reshape(shape)


def _store(cfg, x):
    """Round to the storage dtype; returns float32 values exactly representable in it."""
    if cfg["dtype"] == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x.astype(np.float32)))
    return np.asarray(x, dtype=np.float32)


class LazyNormalBF16:
    """Read-only view of a generated tensor that is never materialised on the host.

    ``arr[b, h]`` returns a lazy sub-view; ``arr[b, h, t0:t1, :]`` (or
    ``sub[t0:t1]``) regenerates exactly those elements from the counter
    generator (same bits as the device fill kernel) and returns float32 values.
    """

    def __init__(self, seed, tid_name, shape, as_bf16=True, _tid=None, _offset=0,
                 _strides=None):
        self.seed = seed
        self.tid = TENSOR_IDS[tid_name] if _tid is None else _tid
        self.tid_name = tid_name
        self.shape = tuple(int(s) for s in shape)
        self.ndim = len(self.shape)
        self.as_bf16 = as_bf16
        self.offset = int(_offset)
        if _strides is None:
            st, acc = [], 1
            for s in reversed(self.shape):
                st.append(acc)
                acc *= s
            _strides = tuple(reversed(st))
        self.strides = tuple(_strides)

    def __getitem__(self, key):
        if not isinstance(key, tuple):
            key = (key,)
        if len(key) < self.ndim and all(isinstance(k, (int, np.integer)) for k in key):
            off = self.offset
            for k, n, s in zip(key, self.shape, self.strides):
                k = int(k)
                if k < 0:
                    k += n
                if not 0 <= k < n:
                    raise IndexError("index out of range")
                off += k * s
            nk = len(key)
            return LazyNormalBF16(self.seed, self.tid_name, self.shape[nk:], self.as_bf16,
                                  _tid=self.tid, _offset=off, _strides=self.strides[nk:])
        key = key + (slice(None),) * (self.ndim - len(key))
        axes, keep = [], []
        for k, n in zip(key, self.shape):
            if isinstance(k, slice):
                axes.append(np.arange(n)[k])
                keep.append(True)
            else:
                k = int(k)
                if k < 0:
                    k += n
                if not 0 <= k < n:
                    raise IndexError("index out of range")
                axes.append(np.array([k]))
                keep.append(False)
        grids = np.ix_(*axes)
        flat = np.full([len(a) for a in axes], self.offset, dtype=np.uint64)
        for g, s in zip(grids, self.strides):
            flat = flat + g.astype(np.uint64) * np.uint64(s)
        x = normal_f32(self.seed, self.tid, flat)
        if self.as_bf16:
            x = bf16_bits_to_f32(f32_to_bf16_bits(x))
        out_shape = [len(a) for a, kp in zip(axes, keep) if kp]
        return x.reshape(out_shape)


def _needle_landmarks(cfg, q, lmk):
    """Plant one needle chunk per (b, kv head): landmark = sqrt(d)(0.9 qbar/|qbar| + 0.4359 u)."""
    B, Hq, Hkv, d, S, Lkv = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["S"], cfg["Lkv"]
    G = Hq // Hkv
    n_cand = (Lkv - 1) // S          # chunks strictly before the newest token's chunk
    pos = np.zeros((B, Hkv), dtype=np.int64)
    if n_cand <= 0:
        return lmk, pos
    draws = uniform_u64(cfg["seed"], TENSOR_IDS["needle_pos"],
                        np.arange(B * Hkv, dtype=np.uint64))
    for b in range(B):
        for g in range(Hkv):
            c = int(draws[b * Hkv + g] % np.uint64(n_cand))
            qbar = q[b, g * G:(g + 1) * G, -1, :].astype(np.float64).mean(axis=0)
            qn = qbar / np.linalg.norm(qbar)
            u = normal_f32(cfg["seed"], TENSOR_IDS["needle_u"],
                           np.arange((b * Hkv + g) * d, (b * Hkv + g + 1) * d,
                                     dtype=np.uint64)).astype(np.float64)
            u = u - (u @ qn) * qn
            u = u / np.linalg.norm(u)
            vec = math.sqrt(d) * (0.9 * qn + math.sqrt(1.0 - 0.81) * u)
            lmk[b, g, c, :] = _store(cfg, vec.astype(np.float32))
            pos[b, g] = c
    return lmk, pos


def make_host_inputs(cfg, lazy_kv=None):
    """Host float32 arrays (values exactly representable in cfg['dtype']).

    Returns dict with q, k, v, lmk, bias (None), dout (or None), needle_pos.
    With ``lazy_kv`` (default: when the cache exceeds 2^28 elements) k and v are
    LazyNormalBF16 views instead of arrays; they require an ``iid``-keyed recipe.
    """
    B, Hq, Hkv, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    Lq, Lkv, S = cfg["Lq"], cfg["Lkv"], cfg["S"]
    NC = Lkv // S
    kv_shape = (B, Hkv, Lkv, d)
    if lazy_kv is None:
        lazy_kv = int(np.prod(kv_shape)) > (1 << 28)
    out = {"cfg": dict(cfg)}
    qraw = _draw(cfg, "q", (B, Hq, Lq, d))
    if cfg.get("qcorr"):
        rho = float(cfg["qcorr"])
        a = np.float32(math.sqrt(1.0 - rho * rho))
        for i in range(1, Lq):
            qraw[:, :, i] = np.float32(rho) * qraw[:, :, i - 1] + a * qraw[:, :, i]
    out["q"] = _store(cfg, qraw)
    if lazy_kv:
        if cfg["lmk"] == "chunk_mean":
            raise ValueError("chunk_mean landmarks need materialised keys")
        as_bf16 = cfg["dtype"] == "bf16"
        out["k"] = LazyNormalBF16(cfg["seed"], "k", kv_shape, as_bf16)
        out["v"] = LazyNormalBF16(cfg["seed"], "v", kv_shape, as_bf16)
    else:
        # kscale: keys of a larger norm (logits far below the norm bound of a row)
        out["k"] = _store(cfg, _draw(cfg, "k", kv_shape, scale=float(cfg.get("kscale", 1.0))))
        out["v"] = _store(cfg, _draw(cfg, "v", kv_shape))
    recipe = cfg["lmk"]
    if recipe == "chunk_mean":
        km = out["k"][:, :, :NC * S, :].astype(np.float64).reshape(B, Hkv, NC, S, d).mean(axis=3)
        noise = _draw(cfg, "lmk_noise", (B, Hkv, NC, d), scale=0.1).astype(np.float64)
        out["lmk"] = _store(cfg, (km + noise).astype(np.float32))
        out["needle_pos"] = None
    else:
        lmk = _store(cfg, _draw(cfg, "lmk", (B, Hkv, NC, d)))
        if recipe == "needle":
            lmk, pos = _needle_landmarks(cfg, out["q"], lmk)
            out["needle_pos"] = pos
        else:
            out["needle_pos"] = None
        out["lmk"] = lmk
    out["q_ret"] = None
    if cfg.get("qret"):
        r = int(cfg["qret"])
        A = _draw(cfg, "qret_a", (Hq, d, r), scale=0.5 / math.sqrt(r)).astype(np.float64)
        Bm = _draw(cfg, "qret_b", (Hq, d, r), scale=1.0 / math.sqrt(d)).astype(np.float64)
        q64 = out["q"].astype(np.float64)
        low = np.einsum("hdr,bhld->bhlr", Bm, q64)
        out["q_ret"] = _store(cfg, (q64 + np.einsum("hdr,bhlr->bhld", A, low)).astype(np.float32))
    out["bias"] = None
    if cfg.get("bias"):
        out["bias"] = _draw(cfg, "bias", (B, Hkv, NC), scale=float(cfg["bias"]))
    out["dout"] = _store(cfg, _draw(cfg, "dout", (B, Hq, Lq, d))) if cfg.get("dout") else None
    return out


def plant_ties(host, cfg, mode):
    """Exact score ties for the tie-break tests (modifies host["lmk"] and host["bias"]).

    * ``all_equal``: every landmark row of a (b, kv head) is that group's row 0 and
      the bias is 0, so every candidate of a query has the same score (bit for bit,
      on any side that scores the rows alike) and the lowest ids must win.
    * ``kth``: per (b, kv head), K - 1 "strong" chunks get bias 100 + K - r (r = 1
      .. K - 1: distinct, far above every other score), a "tie" set of four chunks
      shares one landmark row (the first member's) and gets bias 50, and every
      other chunk bias 0.  A query that sees all of them has a four-way exact tie
      at its K-th score, which the lowest tied id must win.  Positions are drawn
      from the counter generator among the candidates of the last query.

    Returns {(b, g): (strong ids, tie ids)} for ``kth``, {} otherwise.
    """
    B, Hkv, S, K = cfg["B"], cfg["Hkv"], cfg["S"], cfg["K"]
    lmk = np.array(host["lmk"], dtype=np.float32, copy=True)
    NC = lmk.shape[2]
    bias = np.zeros((B, Hkv, NC), dtype=np.float32)
    planted = {}
    if mode == "all_equal":
        lmk[:] = lmk[:, :, :1, :]
    elif mode == "kth":
        win = cfg.get("win")
        win = (1 if cfg.get("keep_own", 1) else 0) if win is None else int(win)
        t_last = cfg["Lkv"] - 1 if cfg["causal"] else cfg["Lkv"]
        ncand = min(NC, max(0, t_last // S - max(win - 1, 0))) if cfg["causal"] else NC
        need = K - 1 + 4
        assert ncand >= need, "too few candidates to plant the ties"
        for b in range(B):
            for g in range(Hkv):
                draws = uniform_u64(cfg["seed"], TENSOR_IDS["ties"],
                                    np.arange((b * Hkv + g) * 4 * need,
                                              (b * Hkv + g + 1) * 4 * need, dtype=np.uint64))
                chosen = []
                for u in draws:
                    c = int(u % np.uint64(ncand))
                    if c not in chosen:
                        chosen.append(c)
                    if len(chosen) == need:
                        break
                assert len(chosen) == need
                strong, tie = chosen[:K - 1], sorted(chosen[K - 1:])
                for r, c in enumerate(strong):
                    bias[b, g, c] = 100.0 + (K - 1 - r)
                for c in tie:
                    lmk[b, g, c] = lmk[b, g, tie[0]]
                    bias[b, g, c] = 50.0
                planted[(b, g)] = (sorted(strong), tie)
    else:
        raise ValueError(mode)
    host["lmk"] = lmk
    host["bias"] = bias if mode == "kth" else None
    return planted


def make_landmark_inputs(cfg, lq_scale=1.0, num_landmarks=None, grads=False):
    """Inputs of landmark formation: landmark queries lq [B, Hkv, NCcap, d] drawn
    N(0, lq_scale^2) (a query-like vector per chunk; a larger scale gives sharper
    in-chunk distributions), the keys k of the workload (the same draw as the
    attention inputs), and with ``grads`` the incoming gradients dlmk (N(0, 1))
    and dbias (N(0, 1), fp32).  NCcap defaults to the number of complete chunks."""
    B, Hkv, d, Lkv, S = cfg["B"], cfg["Hkv"], cfg["d"], cfg["Lkv"], cfg["S"]
    ncap = Lkv // S if num_landmarks is None else int(num_landmarks)
    out = {"k": _store(cfg, _draw(cfg, "k", (B, Hkv, Lkv, d))),
           "lq": _store(cfg, _draw(cfg, "lq", (B, Hkv, ncap, d), scale=lq_scale))}
    if grads:
        out["dlmk"] = _store(cfg, _draw(cfg, "dlmk", (B, Hkv, ncap, d)))
        out["dbias"] = _draw(cfg, "dbias", (B, Hkv, ncap))
    return out


def make_inputs(name_or_cfg, **overrides):
    cfg = config(name_or_cfg, **overrides) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    return make_host_inputs(cfg)
