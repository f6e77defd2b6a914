"""Pins for the CPU oracle: every check compares it with something other than itself.

* dense attention from torch (S = 1, every chunk selected, landmarks = keys);
* exact chunk mass as the retrieval score reduces to softmax restricted to the
  selected tokens, with the selection equal to naive block-sparse attention's
  top-K by exact mass (Hierarchical Sparse Attention Done Right, §2 Preliminary);
* top-1 equals attention over the single best chunk;
* weights sum to one (V = 1 gives O = 1);
* a hand-derived worked example (tests/golden/hand_worked_example.json);
* a second, token-weight-matrix formulation built from library softmaxes;
* decode equals the last row of causal prefill; ties go to the lowest index;
  permutation inside a chunk and a constant bias shift change nothing; GQA with
  identical heads equals one head;
* central finite differences for every gradient, the dense-attention gradients
  from torch autograd, and the zero-sum of the fusion-score gradients;
* chunk-aligned local window (local_chunks = w): a window covering every key is
  dense attention (and dense gradients); with exact-mass scores it is the
  softmax restricted to the retrieved and window tokens; a token-level second
  formulation (window tokens weighted by their own logits); no overlap of
  window and retrieval; decode = last prefill row; finite differences;
* separate retrieval query q_ret: zero q_ret makes the chunk scores the biases
  (selection and fusion weights from scipy), exact-mass scores through q_ret
  give the restricted softmax of q, q_ret = q splits the base gradient of q in
  two, and finite differences for every gradient including dq_ret;
* landmark formation: the surrogate score equals the exact chunk LogSumExp (and
  its gradient) at the landmark query, uniform and one-hot limits (bias log S and
  0), the entropy against scipy, and finite differences of its backward.
"""
import heapq
import json
import math
import os
import re

import numpy as np
import pytest
import scipy.special
import torch

import scipy.stats

from oracle.hils_oracle import (ref_forward, ref_decode, ref_backward, landmark_formation,
                                landmark_formation_backward)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_example.json")


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    s = re.sub(r"ln\(([^)]*)\)", r"log(\1)", x)
    s = re.sub(r"ln(\d+)", r"log(\1)", s)
    return float(eval(s, {"__builtins__": {}}, {"log": math.log}))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _dense_torch(q, k, v, scale, mask):
    """Textbook softmax attention in fp64 (torch), with a boolean mask [Lq, Lkv]."""
    G = q.shape[1] // k.shape[1]
    qt = torch.tensor(q, dtype=torch.float64)
    kt = torch.tensor(np.repeat(k, G, axis=1), dtype=torch.float64)
    vt = torch.tensor(np.repeat(v, G, axis=1), dtype=torch.float64)
    m = torch.tensor(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    logits = scale * qt @ kt.transpose(-1, -2)
    lse = torch.logsumexp(logits.masked_fill(~m, -math.inf), dim=-1)
    return o.numpy(), lse.numpy()


# --------------------------------------------------------------------------- golden
def test_hand_worked_example():
    gold = json.load(open(GOLDEN))
    com = gold["common"]
    S, Lkv = com["S"], com["Lkv"]
    k = np.array([_ev(x) for x in com["k"]]).reshape(1, 1, Lkv, 1)
    v = np.array(com["v"], dtype=np.float64).reshape(1, 1, Lkv, 1)
    lmk = np.array([_ev(x) for x in com["lmk"]]).reshape(1, 1, -1, 1)
    for case in gold["cases"]:
        q = np.array(case["q"], dtype=np.float64)[None, :, None, :]   # [1, Hq, 1, 1]
        bias = None if case["bias"] is None else np.array([_ev(x) for x in case["bias"]]).reshape(1, 1, -1)
        kw = dict(chunk_size=S, top_k=case["K"], causal=bool(case["causal"]),
                  keep_own_chunk=bool(case["keep_own"]), scale=com["scale"])
        out, idx, lse = ref_forward(q, k, v, lmk, bias, **kw)
        assert idx[0, 0, 0].tolist() == case["idx"][0], case["name"]
        np.testing.assert_allclose(out[0, :, 0, 0], [o[0] for o in case["out"]], rtol=0, atol=1e-12,
                                   err_msg=case["name"])
        np.testing.assert_allclose(lse[0, :, 0], [_ev(x) for x in case["lse"]], rtol=0, atol=1e-12,
                                   err_msg=case["name"])
        if case.get("dout") is not None:
            dout = np.array(case["dout"], dtype=np.float64)[None, :, None, :]
            dq, dk, dv, dlmk, dbias = ref_backward(q, k, v, lmk, bias, dout, **kw)
            np.testing.assert_allclose(dq[0, :, 0, 0], [_ev(x[0]) for x in case["dq"]], atol=1e-12)
            np.testing.assert_allclose(dk[0, 0, :, 0], case["dk"], atol=1e-12)
            np.testing.assert_allclose(dv[0, 0, :, 0], case["dv"], atol=1e-12)
            np.testing.assert_allclose(dlmk[0, 0, :, 0], case["dlmk"], atol=1e-12)
            np.testing.assert_allclose(dbias[0, 0, :], case["dbias"], atol=1e-12)


# --------------------------------------------------------------------------- dense
@pytest.mark.parametrize("causal,Lq", [(False, 24), (True, 24), (True, 7)])
def test_dense_reduction(causal, Lq):
    """S = 1, K >= Lkv, landmarks = keys, no bias  =>  textbook dense attention."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, d, Lkv = 2, 4, 2, 8, 24
    q, k, v = _rand(rng, B, Hq, Lq, d), _rand(rng, B, Hkv, Lkv, d), _rand(rng, B, Hkv, Lkv, d)
    out, idx, lse = ref_forward(q, k, v, k.copy(), None, chunk_size=1, top_k=Lkv, causal=causal,
                                keep_own_chunk=True)
    if causal:
        mask = np.arange(Lkv)[None, :] <= (Lkv - Lq + np.arange(Lq))[:, None]
    else:
        mask = np.ones((Lq, Lkv), dtype=bool)
    ro, rl = _dense_torch(q, k, v, 1 / math.sqrt(d), mask)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_dense_reduction_gradients():
    """Under the dense reduction, gradients equal torch autograd of dense attention.

    With S = 1 a token's key enters twice (token logit and landmark score); the
    dense key gradient is the sum of the two: dk_dense = dk + dlmk.
    """
    rng = np.random.default_rng(2)
    B, Hq, Hkv, d, L = 1, 4, 2, 8, 20
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    dout = _rand(rng, B, Hq, L, d)
    dq, dk, dv, dlmk, dbias = ref_backward(q, k, v, k.copy(), None, dout, chunk_size=1, top_k=L,
                                           causal=True, keep_own_chunk=True)
    G = Hq // Hkv
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), is_causal=True)
    (o * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk + dlmk, kt.grad.numpy(), atol=1e-11)


# --------------------------------------------------------------------------- exact mass
def test_exact_mass_is_restricted_softmax():
    """Scores = exact chunk LogSumExp  =>  naive BSA: top-K by exact mass, softmax over kept tokens."""
    rng = np.random.default_rng(3)
    B, H, d, S, NC, K = 2, 3, 8, 4, 9, 3
    Lkv = NC * S + 2                                   # own (partial) chunk of 3 visible tokens
    q, k, v = _rand(rng, B, H, 1, d), _rand(rng, B, H, Lkv, d), _rand(rng, B, H, Lkv, d)
    lmk = _rand(rng, B, H, NC, d)
    scale = 1 / math.sqrt(d)
    logits = scale * np.einsum("bhd,bhtd->bht", q[:, :, 0], k)
    mass = scipy.special.logsumexp(logits[:, :, :NC * S].reshape(B, H, NC, S), axis=-1)
    bias = mass - scale * np.einsum("bhd,bhcd->bhc", q[:, :, 0], lmk)
    out, idx, lse = ref_decode(q, k, v, lmk, bias, chunk_size=S, top_k=K, keep_own_chunk=True)
    own = (Lkv - 1) // S
    for b in range(B):
        for h in range(H):
            best = sorted(np.argsort(-mass[b, h, :own], kind="stable")[:K].tolist())
            assert idx[b, h, 0].tolist() == best
            mask = np.zeros((1, Lkv), dtype=bool)
            for c in best:
                mask[0, c * S:(c + 1) * S] = True
            mask[0, own * S:Lkv] = True
            ro, rl = _dense_torch(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                  scale, mask)
            np.testing.assert_allclose(out[b, h, 0], ro[0, 0, 0], atol=1e-12)
            np.testing.assert_allclose(lse[b, h, 0], rl[0, 0, 0], atol=1e-12)


# --------------------------------------------------------------------------- top-1, sums
def test_top1_is_single_chunk_attention():
    rng = np.random.default_rng(4)
    B, H, d, S, NC = 2, 2, 16, 8, 6
    q, k, v = _rand(rng, B, H, 5, d), _rand(rng, B, H, NC * S, d), _rand(rng, B, H, NC * S, d)
    lmk = 3 * _rand(rng, B, H, NC, d)
    out, idx, lse = ref_forward(q, k, v, lmk, None, chunk_size=S, top_k=1, causal=False,
                                keep_own_chunk=False)
    scale = 1 / math.sqrt(d)
    st = scale * torch.tensor(q) @ torch.tensor(lmk).transpose(-1, -2)        # [B,H,Lq,NC]
    best = torch.argmax(st, dim=-1).numpy()
    for b in range(B):
        for h in range(H):
            for i in range(5):
                c = best[b, h, i]
                assert idx[b, h, i, 0] == c
                mask = np.zeros((1, NC * S), dtype=bool)
                mask[0, c * S:(c + 1) * S] = True
                ro, _ = _dense_torch(q[b:b + 1, h:h + 1, i:i + 1], k[b:b + 1, h:h + 1],
                                     v[b:b + 1, h:h + 1], scale, mask)
                np.testing.assert_allclose(out[b, h, i], ro[0, 0, 0], atol=1e-12)
                np.testing.assert_allclose(lse[b, h, i], st[b, h, i, c].item(), atol=1e-12)


def test_weights_sum_to_one():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, d, S, L = 1, 4, 2, 8, 4, 40
    q, k = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d)
    v = np.ones((B, Hkv, L, d))
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    out, idx, lse = ref_forward(q, k, v, lmk, bias, chunk_size=S, top_k=3, causal=True,
                                keep_own_chunk=True)
    np.testing.assert_allclose(out, 1.0, atol=1e-13)


def test_token_weight_formulation():
    """Second formulation: one weight per token from library softmaxes; O = a V, sum a = 1."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, d, S, L, K = 1, 4, 2, 8, 4, 37, 3
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    NC = L // S
    lmk, bias = _rand(rng, B, Hkv, NC, d), 0.3 * _rand(rng, B, Hkv, NC)
    out, idx, lse = ref_forward(q, k, v, lmk, bias, chunk_size=S, top_k=K, causal=True,
                                keep_own_chunk=True)
    scale = 1 / math.sqrt(d)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        logits = scale * q[0, h] @ k[0, g].T                          # [L, L] dense logits
        lscore = scale * q[0, h] @ lmk[0, g].T + bias[0, g][None, :]  # [L, NC]
        for i in range(L):
            sel = [c for c in idx[0, g, i] if c >= 0]
            own = i // S
            members = [(lscore[i, c], np.arange(c * S, c * S + S)) for c in sel]
            members.append((scipy.special.logsumexp(logits[i, own * S:i + 1]),
                            np.arange(own * S, i + 1)))
            wts = scipy.special.softmax([m[0] for m in members])
            a = np.zeros(L)
            for wc, (_, toks) in zip(wts, members):
                a[toks] += wc * scipy.special.softmax(logits[i, toks])
            assert abs(a.sum() - 1) < 1e-12
            np.testing.assert_allclose(out[0, h, i], a @ v[0, g], atol=1e-12)
            np.testing.assert_allclose(lse[0, h, i], scipy.special.logsumexp([m[0] for m in members]),
                                       atol=1e-12)


# --------------------------------------------------------------------------- selection
def test_selection_matches_heap_topk():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d, S, L, K = 2, 6, 2, 16, 4, 64, 5
    q = _rand(rng, B, Hq, L, d)
    k, v = _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    _, idx, _ = ref_forward(q, k, v, lmk, bias, chunk_size=S, top_k=K, causal=True,
                            keep_own_chunk=True)
    G = Hq // Hkv
    scale = 1 / math.sqrt(d)
    sc = scale * torch.tensor(q) @ torch.tensor(np.repeat(lmk, G, axis=1)).transpose(-1, -2)
    sc = sc + torch.tensor(np.repeat(bias, G, axis=1))[:, :, None, :]
    gs = sc.reshape(B, Hkv, G, L, -1).mean(dim=2).numpy().astype(np.float32)
    for b in range(B):
        for g in range(Hkv):
            for i in range(L):
                cands = range(i // S)
                best = heapq.nlargest(K, cands, key=lambda c: (gs[b, g, i, c], -c))
                want = sorted(best) + [-1] * (K - len(best))
                assert idx[b, g, i].tolist() == want


def test_ties_take_lowest_index():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, d, S, L, K = 1, 4, 2, 8, 4, 48, 3
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk = np.repeat(_rand(rng, B, Hkv, 1, d), L // S, axis=2)
    _, idx, _ = ref_forward(q, k, v, lmk, None, chunk_size=S, top_k=K, causal=True,
                            keep_own_chunk=True)
    for i in range(L):
        n = min(K, i // S)
        assert idx[0, :, i, :n].tolist() == [list(range(n))] * Hkv
        assert (idx[0, :, i, n:] == -1).all()


# --------------------------------------------------------------------------- invariances
def test_decode_is_last_prefill_row():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, S, L, K = 2, 4, 2, 8, 4, 45, 4
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    kw = dict(chunk_size=S, top_k=K, keep_own_chunk=True)
    o1, i1, l1 = ref_forward(q, k, v, lmk, bias, causal=True, **kw)
    o2, i2, l2 = ref_decode(q[:, :, -1:], k, v, lmk, bias, **kw)
    np.testing.assert_array_equal(i1[:, :, -1:], i2)
    np.testing.assert_allclose(o1[:, :, -1:], o2, atol=1e-13)
    np.testing.assert_allclose(l1[:, :, -1:], l2, atol=1e-13)


def test_permutation_inside_chunk():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, d, S, NC, K = 1, 2, 1, 8, 8, 6, 2
    L = NC * S
    q, k, v = _rand(rng, B, Hq, 7, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk = _rand(rng, B, Hkv, NC, d)
    kw = dict(chunk_size=S, top_k=K, causal=False, keep_own_chunk=True)
    o1, i1, l1 = ref_forward(q, k, v, lmk, None, **kw)
    perm = np.concatenate([c * S + rng.permutation(S) for c in range(NC)])
    o2, i2, l2 = ref_forward(q, k[:, :, perm], v[:, :, perm], lmk, None, **kw)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_bias_shift_invariance():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, S, NC, K = 1, 4, 2, 8, 4, 10, 3
    L = NC * S
    q, k, v = _rand(rng, B, Hq, 9, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk, bias = _rand(rng, B, Hkv, NC, d), _rand(rng, B, Hkv, NC)
    kw = dict(chunk_size=S, top_k=K, causal=False, keep_own_chunk=False)
    o1, i1, l1 = ref_forward(q, k, v, lmk, bias, **kw)
    o2, i2, l2 = ref_forward(q, k, v, lmk, bias + 0.75, **kw)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, 0.75, atol=1e-12)


def test_gqa_identical_heads_equals_single_head():
    rng = np.random.default_rng(12)
    d, S, L, K = 8, 4, 32, 3
    q1 = _rand(rng, 1, 1, L, d)
    k, v = _rand(rng, 1, 1, L, d), _rand(rng, 1, 1, L, d)
    lmk = _rand(rng, 1, 1, L // S, d)
    kw = dict(chunk_size=S, top_k=K, causal=True, keep_own_chunk=True)
    o1, i1, l1 = ref_forward(q1, k, v, lmk, None, **kw)
    o3, i3, l3 = ref_forward(np.repeat(q1, 3, axis=1), k, v, lmk, None, **kw)
    np.testing.assert_array_equal(i1, i3)
    for h in range(3):
        np.testing.assert_allclose(o3[:, h], o1[:, 0], atol=1e-13)
        np.testing.assert_allclose(l3[:, h], l1[:, 0], atol=1e-13)


def test_empty_fusion_set():
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 1, 8, 4), _rand(rng, 1, 1, 8, 4), _rand(rng, 1, 1, 8, 4)
    lmk = _rand(rng, 1, 1, 2, 4)
    out, idx, lse = ref_forward(q, k, v, lmk, None, chunk_size=4, top_k=2, causal=True,
                                keep_own_chunk=False)
    assert (out[0, 0, :4] == 0).all() and np.isneginf(lse[0, 0, :4]).all()
    assert (idx[0, 0, :4] == -1).all()
    assert np.isfinite(lse[0, 0, 4:]).all() and (idx[0, 0, 4:, 0] == 0).all()


# --------------------------------------------------------------------------- gradients
def _loss(params, R, kw):
    q, k, v, lmk, bias = params
    out, idx, _ = ref_forward(q, k, v, lmk, bias, **kw)
    return float(np.sum(out * R)), idx


@pytest.mark.parametrize("local", [1, 0, 3])
def test_finite_differences(local):
    rng = np.random.default_rng(14 + local)
    B, Hq, Hkv, d, S, L, K = 1, 4, 2, 6, 4, 28, 2
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    R = _rand(rng, B, Hq, L, d)
    kw = dict(chunk_size=S, top_k=K, causal=True, local_chunks=local)
    grads = ref_backward(q, k, v, lmk, bias, R, **kw)
    params = [q, k, v, lmk, bias]
    _, idx0 = _loss(params, R, kw)
    eps = 1e-6
    checked = 0
    for t, (x, gx) in enumerate(zip(params, grads)):
        flat = x.reshape(-1)
        for e in rng.choice(flat.size, size=min(flat.size, 25), replace=False):
            old = flat[e]
            flat[e] = old + eps
            lp, ip = _loss(params, R, kw)
            flat[e] = old - eps
            lm, im = _loss(params, R, kw)
            flat[e] = old
            if not (np.array_equal(ip, idx0) and np.array_equal(im, idx0)):
                continue                      # the perturbation flips a selection: skip
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gx.reshape(-1)[e]) < 1e-7 * max(1.0, abs(fd)), (t, e, fd, gx.reshape(-1)[e])
            checked += 1
    assert checked > 100


def test_fusion_score_gradients_sum_to_zero():
    """Without the own chunk, O is invariant to a common shift of all scores: sum dbias = 0 per query."""
    rng = np.random.default_rng(16)
    B, H, d, S, L, K = 1, 1, 8, 4, 40, 4
    q, k, v = _rand(rng, B, H, 1, d), _rand(rng, B, H, L, d), _rand(rng, B, H, L, d)
    lmk, bias = _rand(rng, B, H, L // S, d), _rand(rng, B, H, L // S)
    dout = _rand(rng, B, H, 1, d)
    _, _, _, _, dbias = ref_backward(q, k, v, lmk, bias, dout, chunk_size=S, top_k=K, causal=True,
                                     keep_own_chunk=False)
    assert abs(dbias.sum()) < 1e-12
    assert np.count_nonzero(dbias) == K


# --------------------------------------------------------------------------- local window
@pytest.mark.parametrize("causal,Lq", [(True, 29), (True, 6), (False, 5)])
def test_window_covering_every_key_is_dense(causal, Lq):
    """A local window wider than the cache leaves no candidates: every visible
    token is attended exactly, i.e. textbook dense attention (and its gradients)."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, d, S, Lkv = 1, 4, 2, 8, 4, 29
    q, k, v = _rand(rng, B, Hq, Lq, d), _rand(rng, B, Hkv, Lkv, d), _rand(rng, B, Hkv, Lkv, d)
    lmk, bias = _rand(rng, B, Hkv, Lkv // S, d), _rand(rng, B, Hkv, Lkv // S)
    kw = dict(chunk_size=S, top_k=3, causal=causal, local_chunks=Lkv // S + 1)
    out, idx, lse = ref_forward(q, k, v, lmk, bias, **kw)
    assert (idx == -1).all()
    if causal:
        mask = np.arange(Lkv)[None, :] <= (Lkv - Lq + np.arange(Lq))[:, None]
    else:
        mask = np.ones((Lq, Lkv), dtype=bool)
    ro, rl = _dense_torch(q, k, v, 1 / math.sqrt(d), mask)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)
    dout = _rand(rng, B, Hq, Lq, d)
    dq, dk, dv, dlmk, dbias = ref_backward(q, k, v, lmk, bias, dout, **kw)
    G = Hq // Hkv
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1),
        attn_mask=torch.tensor(mask))
    (o * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11)
    assert not dlmk.any() and not dbias.any()


def test_window_exact_mass_is_restricted_softmax():
    """Exact-mass scores with a three-chunk window: naive block-sparse attention
    over the top-K chunks before the window plus every window token."""
    rng = np.random.default_rng(22)
    B, H, d, S, NC, K, w = 2, 2, 8, 4, 11, 3, 3
    Lkv = NC * S + 1                                   # own chunk: 2 visible tokens
    q, k, v = _rand(rng, B, H, 1, d), _rand(rng, B, H, Lkv, d), _rand(rng, B, H, Lkv, d)
    lmk = _rand(rng, B, H, NC, d)
    scale = 1 / math.sqrt(d)
    logits = scale * np.einsum("bhd,bhtd->bht", q[:, :, 0], k)
    mass = scipy.special.logsumexp(logits[:, :, :NC * S].reshape(B, H, NC, S), axis=-1)
    bias = mass - scale * np.einsum("bhd,bhcd->bhc", q[:, :, 0], lmk)
    out, idx, lse = ref_decode(q, k, v, lmk, bias, chunk_size=S, top_k=K, local_chunks=w)
    own = (Lkv - 1) // S
    first_local = own - (w - 1)
    for b in range(B):
        for h in range(H):
            best = sorted(np.argsort(-mass[b, h, :first_local], kind="stable")[:K].tolist())
            assert idx[b, h, 0].tolist() == best
            mask = np.zeros((1, Lkv), dtype=bool)
            for c in best:
                mask[0, c * S:(c + 1) * S] = True
            mask[0, first_local * S:Lkv] = True
            ro, rl = _dense_torch(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                  scale, mask)
            np.testing.assert_allclose(out[b, h, 0], ro[0, 0, 0], atol=1e-12)
            np.testing.assert_allclose(lse[b, h, 0], rl[0, 0, 0], atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_window_token_weight_formulation(causal):
    """Token-level second formulation: a retrieved chunk's tokens get
    softmax(scores + window logits)[c] * softmax(chunk logits); a window token j gets
    exp(l_j - LSE) directly, LSE over the retrieval scores and the window logits."""
    rng = np.random.default_rng(23)
    B, Hq, Hkv, d, S, L, K, w = 1, 4, 2, 8, 4, 43, 3, 3
    Lq = L if causal else 6
    q, k, v = _rand(rng, B, Hq, Lq, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    NC = L // S
    lmk, bias = _rand(rng, B, Hkv, NC, d), 0.3 * _rand(rng, B, Hkv, NC)
    out, idx, lse = ref_forward(q, k, v, lmk, bias, chunk_size=S, top_k=K, causal=causal,
                                local_chunks=w)
    scale = 1 / math.sqrt(d)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        logits = scale * q[0, h] @ k[0, g].T
        lscore = scale * q[0, h] @ lmk[0, g].T + bias[0, g][None, :]
        for i in range(Lq):
            t = i if causal else L - 1
            own = t // S if causal else NC
            lo = max(own - (w - 1), 0) * S                 # first window token
            win = np.arange(lo, t + 1)
            sel = [int(c) for c in idx[0, g, i] if c >= 0]
            ncand = max(0, min(own - (w - 1), NC))
            assert len(sel) == min(K, ncand) and all(c < ncand for c in sel)
            ent = [lscore[i, c] for c in sel] + list(logits[i, win])
            LSE = scipy.special.logsumexp(ent)
            a = np.zeros(L)
            for c in sel:
                toks = np.arange(c * S, c * S + S)
                a[toks] += math.exp(lscore[i, c] - LSE) * scipy.special.softmax(logits[i, toks])
            a[win] += np.exp(logits[i, win] - LSE)
            assert abs(a.sum() - 1) < 1e-12
            np.testing.assert_allclose(out[0, h, i], a @ v[0, g], atol=1e-12)
            np.testing.assert_allclose(lse[0, h, i], LSE, atol=1e-12)


def test_window_decode_is_last_prefill_row():
    rng = np.random.default_rng(24)
    B, Hq, Hkv, d, S, L, K = 2, 4, 2, 8, 4, 53, 3
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    kw = dict(chunk_size=S, top_k=K, local_chunks=4)
    o1, i1, l1 = ref_forward(q, k, v, lmk, bias, causal=True, **kw)
    o2, i2, l2 = ref_decode(q[:, :, -1:], k, v, lmk, bias, **kw)
    np.testing.assert_array_equal(i1[:, :, -1:], i2)
    np.testing.assert_allclose(o1[:, :, -1:], o2, atol=1e-13)
    np.testing.assert_allclose(l1[:, :, -1:], l2, atol=1e-13)
    o3, i3, l3 = ref_forward(q, k, v, lmk, bias, causal=True, chunk_size=S, top_k=K,
                             local_chunks=1)
    o4, i4, l4 = ref_forward(q, k, v, lmk, bias, causal=True, chunk_size=S, top_k=K,
                             keep_own_chunk=True)
    np.testing.assert_array_equal(i3, i4)
    np.testing.assert_array_equal(o3, o4)


# --------------------------------------------------------------------------- retrieval query
def test_qret_zero_scores_are_the_biases():
    """q_ret = 0: every chunk score is its bias, so the selection is the top-K
    biases and the fusion weights are a softmax over those biases and the own
    chunk's exact lse of q; the token attention inside chunks still uses q."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, d, S, L, K = 1, 4, 2, 8, 4, 45, 3
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    NC = L // S
    lmk, bias = _rand(rng, B, Hkv, NC, d), _rand(rng, B, Hkv, NC)
    out, idx, lse = ref_forward(q, k, v, lmk, bias, chunk_size=S, top_k=K, causal=True,
                                q_ret=np.zeros_like(q))
    scale = 1 / math.sqrt(d)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        for i in range(L):
            own = i // S
            best = sorted(sorted(range(own), key=lambda c: (-bias[0, g, c], c))[:K])
            assert [c for c in idx[0, g, i] if c >= 0] == best
            parts, scores = [], []
            for c in best:
                m = np.zeros((1, L), dtype=bool)
                m[0, c * S:(c + 1) * S] = True
                o, _ = _dense_torch(q[:, h:h + 1, i:i + 1], k[:, g:g + 1], v[:, g:g + 1], scale, m)
                parts.append(o[0, 0, 0])
                scores.append(bias[0, g, c])
            m = np.zeros((1, L), dtype=bool)
            m[0, own * S:i + 1] = True
            o, lo = _dense_torch(q[:, h:h + 1, i:i + 1], k[:, g:g + 1], v[:, g:g + 1], scale, m)
            parts.append(o[0, 0, 0])
            scores.append(lo[0, 0, 0])
            wts = scipy.special.softmax(scores)
            np.testing.assert_allclose(out[0, h, i], wts @ np.array(parts), atol=1e-12)
            np.testing.assert_allclose(lse[0, h, i], scipy.special.logsumexp(scores), atol=1e-12)


def test_qret_exact_mass_is_restricted_softmax_of_q():
    """Scores made equal to the exact chunk mass of q through q_ret (bias_c =
    lse_c(q) - scale <q_ret, lmk_c>): naive block-sparse attention of q."""
    rng = np.random.default_rng(32)
    B, H, d, S, NC, K = 1, 2, 8, 4, 9, 3
    Lkv = NC * S + 2
    q, k, v = _rand(rng, B, H, 1, d), _rand(rng, B, H, Lkv, d), _rand(rng, B, H, Lkv, d)
    qr = _rand(rng, B, H, 1, d)
    lmk = _rand(rng, B, H, NC, d)
    scale = 1 / math.sqrt(d)
    logits = scale * np.einsum("bhd,bhtd->bht", q[:, :, 0], k)
    mass = scipy.special.logsumexp(logits[:, :, :NC * S].reshape(B, H, NC, S), axis=-1)
    bias = mass - scale * np.einsum("bhd,bhcd->bhc", qr[:, :, 0], lmk)
    out, idx, lse = ref_decode(q, k, v, lmk, bias, chunk_size=S, top_k=K, q_ret=qr)
    own = (Lkv - 1) // S
    for h in range(H):
        best = sorted(np.argsort(-mass[0, h, :own], kind="stable")[:K].tolist())
        assert idx[0, h, 0].tolist() == best
        mask = np.zeros((1, Lkv), dtype=bool)
        for c in best:
            mask[0, c * S:(c + 1) * S] = True
        mask[0, own * S:Lkv] = True
        ro, rl = _dense_torch(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], scale, mask)
        np.testing.assert_allclose(out[0, h, 0], ro[0, 0, 0], atol=1e-12)
        np.testing.assert_allclose(lse[0, h, 0], rl[0, 0, 0], atol=1e-12)


def test_qret_equal_to_q_splits_the_gradient():
    rng = np.random.default_rng(33)
    B, Hq, Hkv, d, S, L, K = 1, 4, 2, 8, 4, 40, 3
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    dout = _rand(rng, B, Hq, L, d)
    kw = dict(chunk_size=S, top_k=K, causal=True, local_chunks=2)
    o1, i1, l1 = ref_forward(q, k, v, lmk, bias, **kw)
    o2, i2, l2 = ref_forward(q, k, v, lmk, bias, q_ret=q.copy(), **kw)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    g1 = ref_backward(q, k, v, lmk, bias, dout, **kw)
    g2 = ref_backward(q, k, v, lmk, bias, dout, q_ret=q.copy(), **kw)
    np.testing.assert_allclose(g1[0], g2[0] + g2[5], atol=1e-12)
    for a, b in zip(g1[1:], g2[1:5]):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_qret_finite_differences():
    rng = np.random.default_rng(34)
    B, Hq, Hkv, d, S, L, K = 1, 4, 2, 6, 4, 28, 2
    q, k, v = _rand(rng, B, Hq, L, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    qr = _rand(rng, B, Hq, L, d)
    lmk, bias = _rand(rng, B, Hkv, L // S, d), _rand(rng, B, Hkv, L // S)
    R = _rand(rng, B, Hq, L, d)
    kw = dict(chunk_size=S, top_k=K, causal=True, local_chunks=2)
    dq, dk, dv, dlmk, dbias, dqr = ref_backward(q, k, v, lmk, bias, R, q_ret=qr, **kw)
    params = [q, k, v, lmk, bias, qr]
    grads = [dq, dk, dv, dlmk, dbias, dqr]

    def loss():
        out, idx, _ = ref_forward(q, k, v, lmk, bias, q_ret=qr, **kw)
        return float(np.sum(out * R)), idx
    _, idx0 = loss()
    eps, checked = 1e-6, 0
    for t, (x, gx) in enumerate(zip(params, grads)):
        flat = x.reshape(-1)
        for e in rng.choice(flat.size, size=min(flat.size, 20), replace=False):
            old = flat[e]
            flat[e] = old + eps
            lp, ip = loss()
            flat[e] = old - eps
            lm, im = loss()
            flat[e] = old
            if not (np.array_equal(ip, idx0) and np.array_equal(im, idx0)):
                continue
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gx.reshape(-1)[e]) < 1e-7 * max(1.0, abs(fd)), (t, e, fd, gx.reshape(-1)[e])
            checked += 1
    assert checked > 90


# --------------------------------------------------------------------------- landmark formation
def _lm_inputs(rng, B=1, Hkv=2, L=192, d=16, S=32):
    k = rng.standard_normal((B, Hkv, L, d))
    lq = rng.standard_normal((B, Hkv, L // S + 1, d))   # one spare row past the chunks
    return lq, k


def test_landmark_surrogate_exact_at_its_query():
    """s(q) = scale <q, lmk_c> + bias_c is the first-order Taylor expansion of the
    chunk's LogSumExp at q = lq_c: value and gradient agree there."""
    rng = np.random.default_rng(41)
    lq, k = _lm_inputs(rng)
    S, d = 32, k.shape[-1]
    sc = 1.0 / math.sqrt(d)
    lmk, bias = landmark_formation(lq, k, chunk_size=S)
    for g in range(2):
        for c in range(k.shape[2] // S):
            kb = k[0, g, c * S:(c + 1) * S]
            q = lq[0, g, c]
            exact = scipy.special.logsumexp(sc * kb @ q)
            assert abs(sc * q @ lmk[0, g, c] + bias[0, g, c] - exact) < 1e-12
            # d/dq logsumexp(sc k q) at q = lq_c equals sc * lmk_c
            eps = 1e-6
            grad = np.array([(scipy.special.logsumexp(sc * kb @ (q + eps * e)) -
                              scipy.special.logsumexp(sc * kb @ (q - eps * e))) / (2 * eps)
                             for e in np.eye(d)])
            assert np.abs(grad - sc * lmk[0, g, c]).max() < 1e-7
    assert np.all(lmk[0, :, -1] == 0) and np.all(bias[0, :, -1] == 0)


def test_landmark_uniform_and_one_hot_limits():
    rng = np.random.default_rng(42)
    S, d = 64, 8
    k = rng.standard_normal((1, 1, S, d))
    lmk, bias = landmark_formation(np.zeros((1, 1, 1, d)), k, chunk_size=S)
    assert abs(bias[0, 0, 0] - math.log(S)) < 1e-12               # uniform: log S
    assert np.abs(lmk[0, 0, 0] - k[0, 0].mean(axis=0)).max() < 1e-12
    k2 = 0.01 * rng.standard_normal((1, 1, S, d))
    k2[0, 0, 5] = 0.0
    k2[0, 0, 5, 0] = 1.0
    lq = np.zeros((1, 1, 1, d))
    lq[0, 0, 0, 0] = 400.0 * math.sqrt(d)                           # key 5 dominates
    lmk, bias = landmark_formation(lq, k2, chunk_size=S)
    assert bias[0, 0, 0] < 1e-6                                     # one-hot: 0
    assert np.abs(lmk[0, 0, 0] - k2[0, 0, 5]).max() < 1e-6


def test_landmark_entropy_matches_scipy():
    rng = np.random.default_rng(43)
    lq, k = _lm_inputs(rng, d=32)
    S = 32
    sc = 1.0 / math.sqrt(32)
    lmk, bias = landmark_formation(lq, k, chunk_size=S)
    for g in range(2):
        for c in range(k.shape[2] // S):
            kb = k[0, g, c * S:(c + 1) * S]
            p = scipy.special.softmax(sc * kb @ lq[0, g, c])
            assert abs(bias[0, g, c] - scipy.stats.entropy(p)) < 1e-12
            assert np.abs(lmk[0, g, c] - p @ kb).max() < 1e-12


def test_landmark_backward_finite_differences():
    rng = np.random.default_rng(44)
    lq, k = _lm_inputs(rng, L=100, d=8, S=32)   # tail keys 96..99 belong to no chunk
    S = 32
    R = rng.standard_normal(lq.shape)
    r = rng.standard_normal(lq.shape[:3])

    def loss(lq_, k_):
        lm, bi = landmark_formation(lq_, k_, chunk_size=S)
        return float((R * lm).sum() + (r * bi).sum())

    dlq, dk = landmark_formation_backward(lq, k, R, r, chunk_size=S)
    eps = 1e-6
    for idx in [(0, 0, 0, 1), (0, 1, 2, 5), (0, 1, 1, 0)]:
        e = np.zeros_like(lq)
        e[idx] = eps
        assert abs((loss(lq + e, k) - loss(lq - e, k)) / (2 * eps) - dlq[idx]) < 1e-6
    for idx in [(0, 0, 3, 2), (0, 1, 40, 7), (0, 0, 95, 0), (0, 1, 97, 3)]:
        e = np.zeros_like(k)
        e[idx] = eps
        assert abs((loss(lq, k + e) - loss(lq, k - e)) / (2 * eps) - dk[idx]) < 1e-6
    assert np.all(dk[:, :, 96:] == 0) and np.all(dlq[:, :, -1] == 0)
