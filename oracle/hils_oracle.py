"""HiLS attention: plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library.

Source. "Hierarchical Sparse Attention Done Right: Toward Infinite Context
Modeling" (arXiv 2607.02980v1), source-linked summary page, cited below as
[HSADR <section>]. The page prints no equations, so each step restates the
prose it follows:

* keys are split into uniform chunks of S tokens; the local window is aligned
  to chunk boundaries and never overlaps retrieved chunks [HSADR §2 Preliminary];
* each query is scored against one learned summary key (landmark) per chunk;
  the score stands in for the chunk's LogSumExp mass and is affine: a
  query-summary relevance plus a per-chunk (entropy) bias [HSADR §3 Methodology,
  "Method overview", "Linear surrogate for chunk mass"];
* every query is routed over all chunk summaries and keeps the top-K chunks
  [HSADR §3, "Sparse training"];
* query heads of one GQA group share one retrieved chunk set [HSADR §4
  Practical Design Choices, "Architecture" (GQA)];
* the query attends to each retrieved chunk with its own softmax and the chunk
  outputs are fused by a softmax over the retrieval scores (hierarchical
  softmax) [HSADR Abstract; §3, "Hierarchical softmax"];
* gradients of the LM loss reach the retrieval scores through the fusion
  weights; unselected chunks get none [HSADR §3; §9 Discussion & Conclusion].

Readings where the page is silent (each is listed with its reason in the
design notes of the repository):

* score s_{h,i,c} = scale * <q_{h,i}, lmk_c> + bias_c, with the token-logit
  scale (default 1/sqrt(d)); bias is optional (absent = 0);
* GQA group score = mean over the group's heads of s_{h,i,c}; selection takes
  the top min(K, |C_i|) candidates by (group score rounded to fp32, descending;
  chunk index ascending) -- the fp32 rounding is the precision the kernels
  decide in; ``idx`` lists the chosen chunks in ascending order, padded with -1;
* causal mode: query i sits at key position t_i = Lkv - Lq + i; its own chunk
  o_i = floor(t_i / S) is never a candidate (its landmark would summarise
  future tokens); candidates are chunks c < o_i. Non-causal mode: all complete
  chunks are candidates and the trailing partial chunk (if any) is "own";
* chunk-aligned local window of w chunk slots (w = local_chunks; keep_own_chunk
  is w = 1): the own slot (the query's own chunk, its visible tokens only; in
  non-causal mode the trailing partial chunk) and the w - 1 complete chunks
  before it.  Each window chunk is attended exactly and enters the fusion as
  its own member with score = its exact LogSumExp [HSADR §2 Preliminary: the
  window is chunk-aligned and never overlaps retrieved chunks; §5 and §6: the
  measured models keep top-K retrieval plus a 512-token window].  Candidates
  are the complete chunks before the window; fusion weights are per head;
* an empty fusion set gives O = 0 and LSE = -inf;
* separate retrieval query (query calibration): when a retrieval query q_ret is
  given, the chunk scores -- and so the selection and the fusion weights --
  use q_ret in place of q, while the token logits inside each chunk keep q;
  the score gradients then reach q_ret (and the landmarks through q_ret), not q
  [HSADR §4 "Architecture": a low-rank query adaptation calibrates the
  chunk-level surrogate scores; the adaptation itself is model-side];
* landmark formation (the step before scoring): the chunk's landmark query lq_c
  induces p = softmax_j(scale <lq_c, k_j>) over its S keys; the landmark key is
  sum_j p_j k_j and the bias the entropy -sum_j p_j log p_j.  This is the
  first-order Taylor expansion of the chunk's LogSumExp at lq_c, so the score
  equals the exact chunk mass for q = lq_c [HSADR §3 "Linear surrogate for
  chunk mass"; the entropy limits log S / 0 are the page's].

Parity pins (what ties this oracle to something other than itself) live in
tests/test_oracle_pins.py: dense attention (S = 1, all chunks), exact chunk mass
= restricted softmax, top-1, weights summing to one, a hand-derived worked
example, decode = last prefill row, ties, invariances, central finite
differences for every gradient, and for the local window: dense attention when
it covers every key, restricted softmax under exact-mass scores, and a
token-level second formulation.
"""
import math
import numpy as np


# ----------------------------------------------------------------------------
# positions and candidate sets  [HSADR §2 Preliminary; §3 "Sparse training"]
# ----------------------------------------------------------------------------
def query_layout(i, Lq, Lkv, S, causal, local_chunks=1):
    """Return (candidate chunk ids, local-window members) for query i.

    The own slot o holds the query (causal: floor(t_i / S)); in non-causal mode it
    is the trailing partial chunk, slot NC.  The local window is the slots
    o - w + 1 .. o (w = local_chunks, clipped at 0): the own slot's visible tokens
    and the complete chunks before it.  Candidates are the complete chunks before
    the window, so window and retrieval never overlap.  Members are
    (slot, (a, b)) token ranges, own slot first; empty ranges are dropped.
    """
    NC = Lkv // S
    w = int(local_chunks)
    if causal:
        t = Lkv - Lq + i
        own = t // S
        own_rng = (own * S, t + 1)
    else:
        own = NC
        own_rng = (NC * S, Lkv)
    first_local = own - max(w - 1, 0)
    cand = np.arange(0, max(0, min(first_local, NC)))
    window = []
    for j in range(w):
        c = own - j
        if c < 0:
            break
        a, b = own_rng if j == 0 else (c * S, c * S + S)
        if b > a:
            window.append((c, (a, b)))
    return cand, window


def select_chunks(gbar, cand, K):
    """Top-min(K, |cand|) by (fp32(gbar) desc, chunk id asc); returned ascending."""
    if len(cand) == 0:
        return np.zeros(0, dtype=np.int64)
    g32 = np.asarray(gbar, dtype=np.float64).astype(np.float32).astype(np.float64)
    order = np.lexsort((cand, -g32))          # primary key: -score, then chunk id
    return np.sort(cand[order[:min(K, len(cand))]])


def _logsumexp(x):
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return -math.inf
    m = np.max(x)
    if not np.isfinite(m):
        return m
    return m + math.log(np.sum(np.exp(x - m)))


def _chunk_attention(q, k_blk, v_blk, scale):
    """Independent softmax attention of one query over one chunk's tokens.

    Returns (lse_c, o_c, p) with l_j = scale*<q,k_j>, lse_c = log sum exp l_j,
    p_j = exp(l_j - lse_c), o_c = sum_j p_j v_j.  [HSADR §3 "Hierarchical softmax"]
    """
    logits = scale * (k_blk @ q)
    lse = _logsumexp(logits)
    p = np.exp(logits - lse)
    return lse, p @ v_blk, p


# ----------------------------------------------------------------------------
# one query of one KV group: forward and (optionally) backward
# ----------------------------------------------------------------------------
def hils_query(qg, k, v, lmk, bias, i, *, Lq, Lkv, S, K, causal, keep_own, scale,
               forced=None, dout=None, local_chunks=None, qrg=None):
    """Forward (and backward if ``dout``) of query i for the G heads of one KV group.

    qg: [G, d] query rows of the group; k, v: [Lkv, d] (indexable) this group's
    cache; lmk: [NCcap, d]; bias: [NCcap] or None; forced: chunk ids to use
    instead of the selection (ascending), or None; local_chunks: width w of the
    local window in chunk slots (default: 1 if keep_own else 0); qrg: [G, d]
    retrieval queries of the group (default: qg) -- chunk scores use them.
    Returns a dict with idx, out [G, d], lse [G], scores, and for backward dq
    [G, d] and the lists of contributions to dk, dv (per token range), dlmk and
    dbias (per chunk).
    """
    G, d = qg.shape
    qr = qg if qrg is None else qrg
    w_loc = (1 if keep_own else 0) if local_chunks is None else int(local_chunks)
    cand, window = query_layout(i, Lq, Lkv, S, causal, w_loc)

    # retrieval scores of every candidate, per head  [HSADR §3 "Linear surrogate"]
    if len(cand):
        s_all = scale * (qr @ lmk[cand].T)                  # [G, |C|]
        if bias is not None:
            s_all = s_all + bias[cand][None, :]
        gbar = s_all.mean(axis=0)                           # group score [HSADR §4 GQA]
    else:
        s_all = np.zeros((G, 0))
        gbar = np.zeros(0)

    # top-K routing  [HSADR §3 "Sparse training"]
    sel = select_chunks(gbar, cand, K) if forced is None else np.asarray(forced, dtype=np.int64)
    idx = -np.ones(K, dtype=np.int64)
    idx[:len(sel)] = sel
    pos_in_cand = {int(c): n for n, c in enumerate(cand)}

    # members of the fusion set: (kind, chunk id, token range)
    members = [("ret", int(c), (int(c) * S, int(c) * S + S)) for c in sel]
    members += [("loc", int(c), rng) for c, rng in window]

    out = np.zeros((G, d))
    lse = np.full(G, -math.inf)
    res = {"idx": idx, "out": out, "lse": lse, "gbar": gbar, "cand": cand}
    if dout is not None:
        res.update(dq=np.zeros((G, d)), dqr=np.zeros((G, d)), dkv=[], dlmk=[], dbias=[])
    if not members:
        return res

    for h in range(G):
        q = qg[h]
        parts = []
        for kind, c, (a, b) in members:
            kb = np.asarray(k[a:b], dtype=np.float64)
            vb = np.asarray(v[a:b], dtype=np.float64)
            lse_c, o_c, p = _chunk_attention(q, kb, vb, scale)
            if kind == "ret":
                if c in pos_in_cand:
                    s_c = s_all[h, pos_in_cand[c]]
                else:                                       # forced chunk outside C_i
                    s_c = scale * float(qr[h] @ lmk[c]) + (0.0 if bias is None else float(bias[c]))
            else:
                s_c = lse_c                                  # exact mass of a window chunk
            parts.append((kind, c, a, b, kb, vb, p, o_c, s_c))
        # fusion by a softmax over the retrieval scores  [HSADR §3 "Hierarchical softmax"]
        s_vec = np.array([pt[8] for pt in parts])
        LSE = _logsumexp(s_vec)
        w = np.exp(s_vec - LSE)
        O = np.zeros(d)
        for wc, pt in zip(w, parts):
            O = O + wc * pt[7]
        out[h] = O
        lse[h] = LSE

        if dout is None:
            continue
        # backward with the selection held fixed  [HSADR §3; §9]
        g = np.asarray(dout[h], dtype=np.float64)
        D = float(g @ O)
        dq = np.zeros(d)
        dqr = np.zeros(d)                                    # through the chunk scores
        for wc, (kind, c, a, b, kb, vb, p, o_c, s_c) in zip(w, parts):
            u = vb @ g                                       # <dO, v_j>
            Dc = float(p @ u)                                # <dO, o_c>
            if kind == "ret":
                dl = wc * p * (u - Dc)                       # through the intra-chunk softmax
                ds = wc * (Dc - D)                           # through the fusion softmax
                dqr = dqr + scale * ds * np.asarray(lmk[c], dtype=np.float64)
                res["dlmk"].append((c, scale * ds * qr[h]))
                res["dbias"].append((c, ds))
            else:
                dl = wc * p * (u - D)                        # s_c = lse_c adds ds_c * p
            dq = dq + scale * (dl @ kb)
            res["dkv"].append((a, b, scale * np.outer(dl, q), np.outer(wc * p, g)))
        if qrg is None:
            res["dq"][h] = dq + dqr
        else:
            res["dq"][h] = dq
            res["dqr"][h] = dqr
    return res


# ----------------------------------------------------------------------------
# whole-tensor entry points (the same names as the library, prefixed ref_)
# ----------------------------------------------------------------------------
def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def ref_forward(q, k, v, lmk, bias=None, *, chunk_size, top_k, causal=True,
                keep_own_chunk=True, scale=None, queries=None, heads_kv=None,
                batches=None, forced_idx=None, local_chunks=None, q_ret=None):
    """HiLS forward. q [B,Hq,Lq,d]; k, v [B,Hkv,Lkv,d]; lmk [B,Hkv,NCcap,d]; bias [B,Hkv,NCcap].

    Returns out [B,Hq,nq,d], idx [B,Hkv,nq,K] (int64, -1 padded), lse [B,Hq,nq]
    for the query positions ``queries`` (default: all).  ``forced_idx``
    ([B,Hkv,nq,K], -1 padded) replaces the selection.  k and v may be lazy
    indexable objects; only the rows of the used chunks are read.
    ``local_chunks`` (default 1 if keep_own_chunk else 0) is the width of the
    chunk-aligned local window in chunk slots.  ``q_ret`` [B,Hq,Lq,d] (optional)
    is the retrieval query the chunk scores use.
    """
    B, Hq, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    S, K = int(chunk_size), int(top_k)
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    qs = np.arange(Lq) if queries is None else np.asarray(queries)
    bs = range(B) if batches is None else batches
    gs = range(Hkv) if heads_kv is None else heads_kv
    out = np.zeros((B, Hq, len(qs), d))
    lse = np.full((B, Hq, len(qs)), -math.inf)
    idx = -np.ones((B, Hkv, len(qs), K), dtype=np.int64)
    for b in bs:
        for g in gs:
            kg, vg = k[b, g], v[b, g]
            lg = _f64(lmk[b, g])
            bg = None if bias is None else _f64(bias[b, g])
            for n, i in enumerate(qs):
                forced = None
                if forced_idx is not None:
                    f = np.asarray(forced_idx[b, g, n])
                    forced = f[f >= 0]
                qrg = None if q_ret is None else _f64(q_ret[b, g * G:(g + 1) * G, i])
                r = hils_query(_f64(q[b, g * G:(g + 1) * G, i]), kg, vg, lg, bg, int(i),
                               Lq=Lq, Lkv=Lkv, S=S, K=K, causal=bool(causal),
                               keep_own=bool(keep_own_chunk), scale=sc, forced=forced,
                               local_chunks=local_chunks, qrg=qrg)
                idx[b, g, n] = r["idx"]
                out[b, g * G:(g + 1) * G, n] = r["out"]
                lse[b, g * G:(g + 1) * G, n] = r["lse"]
    return out, idx, lse


def ref_decode(q, k, v, lmk, bias=None, **kw):
    """Single-token decode: q [B,Hq,1,d] sits at position Lkv-1 (its K/V already cached)."""
    assert q.shape[2] == 1
    kw = dict(kw)
    kw["causal"] = True
    return ref_forward(q, k, v, lmk, bias, **kw)


def ref_backward(q, k, v, lmk, bias, dout, *, chunk_size, top_k, causal=True,
                 keep_own_chunk=True, scale=None, forced_idx=None, queries=None,
                 local_chunks=None, q_ret=None):
    """Gradients of sum(<dout, out>) for every input, selection held fixed.

    Returns dq [B,Hq,Lq,d] (rows outside ``queries`` are zero), dk, dv
    [B,Hkv,Lkv,d], dlmk [B,Hkv,NCcap,d], dbias [B,Hkv,NCcap] -- the last four
    summed over the contributions of the queries in ``queries`` (default all).
    With ``q_ret`` a sixth array dq_ret [B,Hq,Lq,d] follows (the score
    gradients), and dq holds the token-attention part only.
    """
    B, Hq, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    S, K = int(chunk_size), int(top_k)
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    qs = np.arange(Lq) if queries is None else np.asarray(queries)
    dq = np.zeros((B, Hq, Lq, d))
    dqr = np.zeros((B, Hq, Lq, d))
    dk = np.zeros((B, Hkv, Lkv, d))
    dv = np.zeros((B, Hkv, Lkv, d))
    dlmk = np.zeros(lmk.shape)
    dbias = np.zeros(lmk.shape[:3])
    for b in range(B):
        for g in range(Hkv):
            kg, vg = k[b, g], v[b, g]
            lg = _f64(lmk[b, g])
            bg = None if bias is None else _f64(bias[b, g])
            for n, i in enumerate(qs):
                forced = None
                if forced_idx is not None:
                    f = np.asarray(forced_idx[b, g, n])
                    forced = f[f >= 0]
                qrg = None if q_ret is None else _f64(q_ret[b, g * G:(g + 1) * G, i])
                r = hils_query(_f64(q[b, g * G:(g + 1) * G, i]), kg, vg, lg, bg, int(i),
                               Lq=Lq, Lkv=Lkv, S=S, K=K, causal=bool(causal),
                               keep_own=bool(keep_own_chunk), scale=sc, forced=forced,
                               dout=_f64(dout[b, g * G:(g + 1) * G, i]),
                               local_chunks=local_chunks, qrg=qrg)
                dq[b, g * G:(g + 1) * G, i] = r["dq"]
                dqr[b, g * G:(g + 1) * G, i] = r["dqr"]
                for a, e, dkp, dvp in r["dkv"]:
                    dk[b, g, a:e] += dkp
                    dv[b, g, a:e] += dvp
                for c, val in r["dlmk"]:
                    dlmk[b, g, c] += val
                for c, val in r["dbias"]:
                    dbias[b, g, c] += val
    if q_ret is not None:
        return dq, dk, dv, dlmk, dbias, dqr
    return dq, dk, dv, dlmk, dbias


# ----------------------------------------------------------------------------
# landmark formation  [HSADR §3 "Linear surrogate for chunk mass": the learned
# landmark query induces a distribution over the chunk's keys; the weighted key
# sum is the summary and an entropy term is the bias]
# ----------------------------------------------------------------------------
def _chunk_distribution(lq_c, k_blk, sc):
    l = sc * (k_blk @ lq_c)
    return np.exp(l - _logsumexp(l))


def landmark_formation(lq, k, *, chunk_size, scale=None):
    """Landmark key and entropy bias of every complete chunk.

    lq: [B, Hkv, NCcap, d] landmark queries (rows c < NC are used); k: [B, Hkv,
    Lkv, d].  For chunk c: p = softmax_j(scale * <lq_c, k_j>) over its S keys,
    lmk_c = sum_j p_j k_j and bias_c = -sum_j p_j log p_j.  Rows c >= NC are 0.
    """
    B, Hkv, Lkv, d = k.shape
    S = int(chunk_size)
    NC = Lkv // S
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    lmk = np.zeros(lq.shape)
    bias = np.zeros(lq.shape[:3])
    for b in range(B):
        for g in range(Hkv):
            for c in range(NC):
                kb = _f64(k[b, g, c * S:(c + 1) * S])
                p = _chunk_distribution(_f64(lq[b, g, c]), kb, sc)
                lmk[b, g, c] = p @ kb
                nz = p > 0
                bias[b, g, c] = -float(np.sum(p[nz] * np.log(p[nz])))
    return lmk, bias


def landmark_formation_backward(lq, k, dlmk, dbias, *, chunk_size, scale=None):
    """Gradients of sum(<dlmk, lmk>) + sum(dbias * bias) for lq and k.

    With l_j = scale <lq, k_j>, p = softmax(l): dp_j = <dlmk, k_j> - dbias (log p_j
    + 1); dl_j = p_j (dp_j - sum_i p_i dp_i); dlq = scale sum_j dl_j k_j and
    dk_j = scale dl_j lq + p_j dlmk.  Keys of an incomplete tail chunk get 0.
    """
    B, Hkv, Lkv, d = k.shape
    S = int(chunk_size)
    NC = Lkv // S
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    dlq = np.zeros(lq.shape)
    dk = np.zeros(k.shape)
    for b in range(B):
        for g in range(Hkv):
            for c in range(NC):
                kb = _f64(k[b, g, c * S:(c + 1) * S])
                q = _f64(lq[b, g, c])
                p = _chunk_distribution(q, kb, sc)
                dm = _f64(dlmk[b, g, c])
                db = 0.0 if dbias is None else float(dbias[b, g, c])
                logp = np.log(np.maximum(p, 1e-300))
                dp = kb @ dm - db * (logp + 1.0)
                dl = p * (dp - float(p @ dp))
                dlq[b, g, c] = sc * (dl @ kb)
                dk[b, g, c * S:(c + 1) * S] = sc * np.outer(dl, q) + np.outer(p, dm)
    return dlq, dk
