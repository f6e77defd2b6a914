"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before any launch
(so these run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

from chunk_wise_sparse_landmark_amd import hils as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hils.h")

pytestmark = pytest.mark.skipif(not os.path.exists(H.LIB_PATH), reason="libhils.so not built")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(hils_[a-z_]+)\s*\(", src,
                                 flags=re.M)))


def test_header_declares_the_bound_entry_points():
    assert _declared() == sorted(H.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = H.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_params_struct_layout_matches_header():
    assert ctypes.sizeof(H.HilsParams) == 13 * 4


def _p(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=2, head_dim=128, seq_q=256, seq_kv=256,
                chunk_size=64, top_k=2, num_landmarks=4, causal=True, keep_own_chunk=True,
                scale=0.0, dtype=H.HILS_BF16)
    base.update(kw)
    # raw struct: no normalisation of flag values
    return H.HilsParams(base["batch"], base["heads_q"], base["heads_kv"], base["head_dim"],
                        base["seq_q"], base["seq_kv"], base["chunk_size"], base["top_k"],
                        base["num_landmarks"], int(base["causal"]), int(base["keep_own_chunk"]),
                        base["scale"], base["dtype"])


FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: every call below fails validation
MIS = ctypes.c_void_p((1 << 20) + 4)   # not 16-byte aligned


def _fwd(p, q=FAKE, k=FAKE, v=FAKE, lmk=FAKE, bias=None, out=FAKE, idx=FAKE, lse=None, ws=None,
         ws_bytes=0, entry="hils_forward", q_ret=None):
    lib = H.load_library()
    return getattr(lib, entry)(ctypes.byref(p), q, q_ret, k, v, lmk, bias, out, idx, lse, ws,
                               ws_bytes, None)


def _err():
    return H.load_library().hils_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=3), H.HILS_ERR_INVALID_ARG),              # Hq % Hkv != 0
    (dict(chunk_size=0), H.HILS_ERR_INVALID_ARG),
    (dict(top_k=0), H.HILS_ERR_INVALID_ARG),
    (dict(top_k=-3), H.HILS_ERR_INVALID_ARG),
    (dict(num_landmarks=3), H.HILS_ERR_INVALID_ARG),        # < seq_kv / S
    (dict(seq_q=512), H.HILS_ERR_INVALID_ARG),              # causal with seq_q > seq_kv
    (dict(batch=-1), H.HILS_ERR_INVALID_ARG),
    (dict(dtype=7), H.HILS_ERR_INVALID_ARG),
    (dict(causal=2), H.HILS_ERR_INVALID_ARG),
    (dict(keep_own_chunk=-1), H.HILS_ERR_INVALID_ARG),      # the local_chunks field
    (dict(keep_own_chunk=65), H.HILS_ERR_INVALID_ARG),
    (dict(top_k=65), H.HILS_ERR_UNSUPPORTED),
    (dict(head_dim=512), H.HILS_ERR_UNSUPPORTED),
    (dict(chunk_size=512, seq_kv=1024, seq_q=1024, num_landmarks=2), H.HILS_ERR_UNSUPPORTED),
])
def test_forward_rejects(kw, status):
    assert _fwd(_p(**kw)) == status
    assert _err()


def test_null_and_misaligned_pointers():
    assert _fwd(_p(), q=None) == H.HILS_ERR_INVALID_ARG
    assert _fwd(_p(), idx=None) == H.HILS_ERR_INVALID_ARG
    assert _fwd(_p(), k=MIS) == H.HILS_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert _fwd(H.make_params(batch=1, heads_q=32, heads_kv=8, head_dim=128, seq_q=1,
                              seq_kv=4096, chunk_size=64, top_k=8, num_landmarks=64),
                ws=None, entry="hils_decode") == H.HILS_ERR_WORKSPACE


def test_decode_needs_one_query():
    assert _fwd(_p(seq_q=2), entry="hils_decode") == H.HILS_ERR_INVALID_ARG
    assert "seq_q" in _err()


def test_workspace_too_small():
    p = H.make_params(batch=2, heads_q=32, heads_kv=8, head_dim=128, seq_q=1, seq_kv=8192,
                      chunk_size=64, top_k=16, num_landmarks=128)
    need = H.hils_workspace_size(p, H.HILS_OP_DECODE)
    assert need > 0 and need % 256 == 0
    assert _fwd(p, ws=FAKE, ws_bytes=need - 1, entry="hils_decode") == H.HILS_ERR_WORKSPACE
    assert _fwd(p, ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=need,
                entry="hils_decode") == H.HILS_ERR_WORKSPACE


def test_workspace_size_of_invalid_params_is_zero():
    assert H.hils_workspace_size(_p(heads_q=3), H.HILS_OP_FORWARD) == 0
    assert H.hils_workspace_size(_p(), 7) == 0


def _bwd_args(**over):
    names = ["q", "q_ret", "k", "v", "lmk", "lmk_bias", "out", "dout", "sel_idx", "lse", "dq",
             "dq_ret", "dk", "dv", "dlmk", "dlmk_bias", "ws", "ws_bytes", "stream"]
    a = dict(zip(names, [FAKE] * 16 + [FAKE, 1 << 30, None]))
    a.update(q_ret=None, dq_ret=None, lmk_bias=None)
    a.update(over)
    return [a[n] for n in names]


def test_backward_rejections():
    lib = H.load_library()
    p = _p()
    assert lib.hils_backward(ctypes.byref(p), *_bwd_args(lse=None)) == H.HILS_ERR_INVALID_ARG
    assert "null" in _err()
    p2 = _p(chunk_size=128, head_dim=128, num_landmarks=2)
    assert lib.hils_backward(ctypes.byref(p2), *_bwd_args()) == H.HILS_ERR_UNSUPPORTED


def test_retrieval_query_pointer_checks():
    lib = H.load_library()
    assert _fwd(_p(), q_ret=MIS) == H.HILS_ERR_INVALID_ARG
    assert "aligned" in _err()
    # q_ret and dq_ret come together
    assert lib.hils_backward(ctypes.byref(_p()), *_bwd_args(q_ret=FAKE)) == H.HILS_ERR_INVALID_ARG
    assert "together" in _err()
    assert lib.hils_backward(ctypes.byref(_p()), *_bwd_args(dq_ret=FAKE)) == H.HILS_ERR_INVALID_ARG


def test_empty_problem_is_a_no_op():
    assert _fwd(_p(batch=0), q=None, k=None, v=None, lmk=None, out=None, idx=None) == H.HILS_OK
    assert _fwd(_p(seq_q=0), q=None, k=None, v=None, lmk=None, out=None, idx=None) == H.HILS_OK


def test_status_strings():
    lib = H.load_library()
    for s in range(5):
        assert lib.hils_status_string(s).decode().startswith("HILS_")


def _lmk_call(p, lq=FAKE, k=FAKE, lmk=FAKE, bias=None):
    return H.load_library().hils_landmarks(ctypes.byref(p), lq, k, lmk, bias, None)


def _lmk_bwd_call(p, lq=FAKE, k=FAKE, dlmk=FAKE, dbias=None, dlq=FAKE, dk=FAKE):
    return H.load_library().hils_landmarks_backward(ctypes.byref(p), lq, k, dlmk, dbias, dlq, dk,
                                                    None)


@pytest.mark.parametrize("kw,status", [
    (dict(chunk_size=0), H.HILS_ERR_INVALID_ARG),
    (dict(num_landmarks=3), H.HILS_ERR_INVALID_ARG),        # < seq_kv / S
    (dict(seq_kv=-64), H.HILS_ERR_INVALID_ARG),
    (dict(dtype=9), H.HILS_ERR_INVALID_ARG),
    (dict(scale=float("nan")), H.HILS_ERR_INVALID_ARG),
    (dict(head_dim=512), H.HILS_ERR_UNSUPPORTED),
    (dict(chunk_size=128, head_dim=256), H.HILS_ERR_UNSUPPORTED),   # S * d > 16384
])
def test_landmarks_reject(kw, status):
    assert _lmk_call(_p(**kw)) == status
    assert _err()
    assert _lmk_bwd_call(_p(**kw)) == status


def test_landmarks_ignore_attention_only_fields():
    """top_k, causal, local_chunks, seq_q and heads_q take no part in landmark
    formation: values that the attention entry points reject pass its checks
    (the call then fails only on the pointer it is given)."""
    p = _p(top_k=0, causal=5, keep_own_chunk=7, seq_q=-1, heads_q=3)
    assert _lmk_call(p, lq=None) == H.HILS_ERR_INVALID_ARG
    assert "null" in _err()


def test_landmarks_pointer_checks():
    assert _lmk_call(_p(), k=None) == H.HILS_ERR_INVALID_ARG
    assert _lmk_call(_p(), lmk=MIS) == H.HILS_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert _lmk_call(_p(), bias=MIS) == H.HILS_ERR_INVALID_ARG
    assert _lmk_bwd_call(_p(), dk=None) == H.HILS_ERR_INVALID_ARG
    assert _lmk_bwd_call(_p(), dbias=MIS) == H.HILS_ERR_INVALID_ARG


def test_landmarks_empty_is_a_no_op():
    assert _lmk_call(_p(batch=0), lq=None, k=None, lmk=None) == H.HILS_OK
    assert _lmk_call(_p(heads_kv=0, heads_q=0), lq=None, k=None, lmk=None) == H.HILS_OK
    assert _lmk_call(_p(seq_kv=0, num_landmarks=0), lq=None, k=None, lmk=None) == H.HILS_OK
    assert _lmk_bwd_call(_p(batch=0), lq=None, k=None, dlmk=None, dlq=None, dk=None) == H.HILS_OK


# ---- the binding checks every tensor before any call into the library
torch = pytest.importorskip("torch")


def _cpu_inputs(dtype=None):
    dt = dtype or torch.bfloat16
    q = torch.zeros(1, 4, 128, 64, dtype=dt)
    k = torch.zeros(1, 2, 128, 64, dtype=dt)
    v = torch.zeros(1, 2, 128, 64, dtype=dt)
    lmk = torch.zeros(1, 2, 8, 64, dtype=dt)
    return q, k, v, lmk


@pytest.mark.parametrize("case", ["v_dtype", "v_shape", "v_strided", "bias_dtype", "bias_shape",
                                  "out_shape", "sel_dtype", "lse_shape", "qret_dtype"])
def test_binding_rejects_mismatched_forward_tensors(case):
    q, k, v, lmk = _cpu_inputs()
    kw = dict(chunk_size=16, top_k=2)
    if case == "v_dtype":
        v = v.float()
    elif case == "v_shape":
        v = v[:, :, :64]
    elif case == "v_strided":
        v = torch.zeros(1, 2, 64, 128, dtype=q.dtype).transpose(2, 3)
    elif case == "bias_dtype":
        kw["lmk_bias"] = torch.zeros(1, 2, 8, dtype=torch.bfloat16)
    elif case == "bias_shape":
        kw["lmk_bias"] = torch.zeros(1, 2, 9, dtype=torch.float32)
    elif case == "out_shape":
        kw["out"] = torch.zeros(1, 4, 127, 64, dtype=q.dtype)
    elif case == "sel_dtype":
        kw["sel_idx"] = torch.zeros(1, 2, 128, 2, dtype=torch.int64)
    elif case == "lse_shape":
        kw["lse"] = torch.zeros(1, 2, 128, dtype=torch.float32)
    elif case == "qret_dtype":
        kw["q_ret"] = q.float()
    bias = kw.pop("lmk_bias", None)
    with pytest.raises(ValueError):
        H.hils_forward(q, k, v, lmk, bias, **kw)


@pytest.mark.parametrize("case", ["dout_strided", "sel_shape", "lse_dtype", "out_dtype"])
def test_binding_rejects_mismatched_backward_tensors(case):
    q, k, v, lmk = _cpu_inputs()
    out, dout = torch.zeros_like(q), torch.zeros_like(q)
    sel = torch.zeros(1, 2, 128, 2, dtype=torch.int32)
    lse = torch.zeros(1, 4, 128, dtype=torch.float32)
    if case == "dout_strided":
        dout = torch.zeros(1, 4, 64, 128, dtype=q.dtype).transpose(2, 3)
    elif case == "sel_shape":
        sel = torch.zeros(1, 2, 128, 3, dtype=torch.int32)
    elif case == "lse_dtype":
        lse = lse.double()
    elif case == "out_dtype":
        out = out.float()
    with pytest.raises(ValueError):
        H.hils_backward(q, k, v, lmk, None, out, dout, sel, lse, chunk_size=16, top_k=2)


def test_backward_without_queries_needs_gradient_buffers():
    """seq_q = 0 with a non-empty cache zero-fills dk, dv, dlmk: null ones are rejected
    before any launch."""
    p = _p(seq_q=0, causal=False)
    lib = H.load_library()
    st = lib.hils_backward(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                           None, None, None, None, FAKE, FAKE, None, None, 0, None)
    assert st == H.HILS_ERR_INVALID_ARG
    st = lib.hils_backward(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                           None, None, None, FAKE, FAKE, FAKE, MIS, None, 0, None)
    assert st == H.HILS_ERR_INVALID_ARG
