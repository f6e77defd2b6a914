#!/usr/bin/env python3
"""Throughput of the HiLS attention hot path on one MI355X.

Headline workload (the metric's prefill configuration): causal prefill, B=1,
Hq=32, Hkv=8, d=128, L=8192, chunk 64, top-16, own chunk kept, bf16 inputs with
fp32 arithmetic.  One step = one hils_forward call over the whole batch
(retrieval scores, group top-K, per-chunk attention, fusion).  `value` is
algorithmic TFLOP/s: the matmul work the method must do, 2 FLOP per multiply-
add (group score over every candidate, per-head score of every selected chunk,
QK^T and PV over every selected and own-chunk token).

Extra workloads in the same JSON line (`extra`): batch-16 decode over a 128K
cache and batch-1 decode over a 4M cache (algorithmic HBM GB/s: landmarks of
all candidates + K/V of the selected and own tokens + q, out, idx, lse; inputs
rotate over several independent sets so the 256 MB last-level cache cannot hold
them), and the training step (forward + backward, TFLOP/s).

Every input is resident in HBM before timing.  Per-kernel durations come from
HIP events the library records around each launch of the dominant kernel on
its own stream (hils_profile_kernel).
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HiLS decode KV GB/s @128K-4M ctx + prefill TFLOP/s @8K; % of roofline"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


# --------------------------------------------------------------------------- HIP events
class HipEvents:
    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.rt.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.rt.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(ctypes.c_void_p(e))


# --------------------------------------------------------------------------- work counts
def query_counts(cfg):
    """Per query position i: (#candidates, #selected, #own tokens)."""
    import numpy as np
    S, K, Lq, Lkv = cfg["S"], cfg["K"], cfg["Lq"], cfg["Lkv"]
    NC = Lkv // S
    t = Lkv - Lq + np.arange(Lq)
    own = t // S
    ncand = np.minimum(own, NC)
    nsel = np.minimum(ncand, K)
    nown = (t - own * S + 1) if cfg["keep_own"] else np.zeros(Lq, dtype=np.int64)
    return ncand.astype(np.int64), nsel.astype(np.int64), nown.astype(np.int64)


def forward_flops(cfg, queries=None):
    ncand, nsel, nown = query_counts(cfg)
    if queries is not None:
        ncand, nsel, nown = ncand[queries], nsel[queries], nown[queries]
    d, S, G = cfg["d"], cfg["S"], cfg["Hq"] // cfg["Hkv"]
    per_group = (2 * d * ncand).sum() + G * (2 * d * nsel + 4 * d * (S * nsel + nown)).sum()
    return float(cfg["B"] * cfg["Hkv"] * per_group)


def backward_flops(cfg):
    ncand, nsel, nown = query_counts(cfg)
    d, S = cfg["d"], cfg["S"]
    return float(cfg["B"] * cfg["Hq"] * (10 * d * (S * nsel + nown) + 4 * d * nsel).sum())


def decode_bytes(cfg):
    ncand, nsel, nown = query_counts(cfg)
    d, B, Hq, Hkv, K = cfg["d"], cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["K"]
    lmk = B * Hkv * int(ncand[-1]) * d * 2
    kv = B * Hkv * int(nsel[-1] * cfg["S"] + nown[-1]) * d * 2 * 2
    small = 2 * B * Hq * d * 2 + B * Hkv * K * 4 + B * Hq * 4
    return float(lmk + kv + small), float(lmk), float(kv)


# --------------------------------------------------------------------------- runners
def timed(step, steps, warmup, ev, kernel, hl):
    """Run warmup + timed steps; returns (ms per step, avg ms of `kernel` launches)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    starts, stops = ev.create(steps * 4), ev.create(steps * 4)
    keep = hl.hils_profile_kernel(kernel, starts, stops)
    t0, t1 = ev.create(1)[0], ev.create(1)[0]
    torch.cuda.synchronize()
    ev.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    ev.rt.hipEventRecord(ctypes.c_void_p(t0), ctypes.c_void_p(st))
    for i in range(steps):
        step(warmup + i)
    ev.rt.hipEventRecord(ctypes.c_void_p(t1), ctypes.c_void_p(st))
    torch.cuda.synchronize()
    total = ev.elapsed_ms(t0, t1)
    n = hl.hils_profile_count()
    hl.hils_profile_kernel(kernel, [], [])
    del keep
    kms = [ev.elapsed_ms(starts[i], stops[i]) for i in range(n)]
    ev.destroy(starts + stops + [t0, t1])
    return total / steps, (sum(kms) / len(kms) if kms else float("nan")), n


def launched(hl, ev, kernel, fn):
    """True when `fn()` launches kernel family `kernel` (checked with one armed event pair)."""
    import torch
    a, b = ev.create(1), ev.create(1)
    keep = hl.hils_profile_kernel(kernel, a, b)
    fn()
    torch.cuda.synchronize()
    n = hl.hils_profile_count()
    hl.hils_profile_kernel(kernel, [], [])
    del keep
    ev.destroy(a + b)
    return n > 0


def run_prefill(hl, cfg, steps, warmup, ev):
    import torch
    from hils_inputs.device import make_device_inputs
    _, dev = make_device_inputs(cfg)
    out = torch.empty_like(dev["q"])
    idx = torch.empty((cfg["B"], cfg["Hkv"], cfg["Lq"], cfg["K"]), dtype=torch.int32, device="cuda")
    lse = torch.empty((cfg["B"], cfg["Hq"], cfg["Lq"]), dtype=torch.float32, device="cuda")
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]))
    o, i, l = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, **kw)
    ws = None
    p = hl.make_params(batch=cfg["B"], heads_q=cfg["Hq"], heads_kv=cfg["Hkv"], head_dim=cfg["d"],
                       seq_q=cfg["Lq"], seq_kv=cfg["Lkv"], chunk_size=cfg["S"], top_k=cfg["K"],
                       num_landmarks=dev["lmk"].shape[2], causal=True,
                       keep_own_chunk=cfg["keep_own"])
    need = hl.hils_workspace_size(p, hl.HILS_OP_FORWARD)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step(_):
        hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out=out, sel_idx=idx,
                        lse=lse, ws=ws, **kw)

    kern = "prefill_attend" if launched(hl, ev, "prefill_attend", lambda: step(0)) else "generic_attend"
    ms, kms, n = timed(step, steps, warmup, ev, kern, hl)
    flops = forward_flops(cfg)
    ncand, nsel, nown = query_counts(cfg)
    G, d, S = cfg["Hq"] // cfg["Hkv"], cfg["d"], cfg["S"]
    attn_flops = float(cfg["B"] * cfg["Hq"] * (2 * d * nsel + 4 * d * (S * nsel + nown)).sum())
    res = dict(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s", ms_per_step=ms,
               roofline=dict(bound="mfma", kernel=kern, kernel_ms=kms, launches=n,
                             achieved=attn_flops / (kms * 1e-3) / 1e12, peak=PEAK_BF16_TFLOPS,
                             unit="TFLOP/s", traffic=None,
                             per_launch_flops=attn_flops))
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_BF16_TFLOPS
    del dev
    return res


def run_decode(hl, cfg, steps, warmup, ev, nsets):
    import torch
    from hils_inputs.device import make_decode_inputs_on_device
    sets = []
    for r in range(nsets):
        c = dict(cfg, seed=cfg["seed"] + 1000 * r)
        sets.append(make_decode_inputs_on_device(c))
    torch.cuda.synchronize()
    outs = [torch.empty_like(s["q"]) for s in sets]
    idx = torch.empty((cfg["B"], cfg["Hkv"], 1, cfg["K"]), dtype=torch.int32, device="cuda")
    lse = torch.empty((cfg["B"], cfg["Hq"], 1), dtype=torch.float32, device="cuda")
    p = hl.make_params(batch=cfg["B"], heads_q=cfg["Hq"], heads_kv=cfg["Hkv"], head_dim=cfg["d"],
                       seq_q=1, seq_kv=cfg["Lkv"], chunk_size=cfg["S"], top_k=cfg["K"],
                       num_landmarks=cfg["Lkv"] // cfg["S"], keep_own_chunk=cfg["keep_own"])
    ws = torch.empty(max(1, hl.hils_workspace_size(p, hl.HILS_OP_DECODE)), dtype=torch.uint8,
                     device="cuda")
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], keep_own_chunk=bool(cfg["keep_own"]))

    def step(i):
        s = sets[i % nsets]
        hl.hils_decode(s["q"], s["k"], s["v"], s["lmk"], None, out=outs[i % nsets], sel_idx=idx,
                       lse=lse, ws=ws, **kw)

    total, lmk_b, kv_b = decode_bytes(cfg)
    kern, kbytes = ("decode_attend", kv_b) if kv_b >= lmk_b else ("decode_score", lmk_b)
    ms, kms, n = timed(step, steps, warmup, ev, kern, hl)
    res = dict(value=total / (ms * 1e-3) / 1e9, unit="GB/s", ms_per_step=ms, bytes_per_step=total,
               roofline=dict(bound="hbm", kernel=kern, kernel_ms=kms, launches=n,
                             achieved=kbytes / (kms * 1e-3) / 1e9, peak=PEAK_HBM_GBS, unit="GB/s",
                             traffic=None, per_launch_bytes=kbytes))
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_HBM_GBS
    res["frac_of_hbm_peak"] = res["value"] / PEAK_HBM_GBS
    del sets, outs
    torch.cuda.empty_cache()
    return res


def run_train(hl, cfg, steps, warmup, ev):
    import torch
    from hils_inputs.device import make_device_inputs
    _, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]))

    def step(_):
        out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, **kw)
        hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out, dev["dout"], idx,
                         lse, **kw)

    kern = "prefill_bwd_chunks" if launched(hl, ev, "prefill_bwd_chunks", lambda: step(0)) else "generic_bwd_chunks"
    ms, kms, n = timed(step, steps, warmup, ev, kern, hl)
    flops = forward_flops(cfg) + backward_flops(cfg)
    res = dict(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s", ms_per_step=ms,
               frac_of_bf16_peak=flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               dominant_kernel=dict(kernel=kern, kernel_ms=kms, launches=n))
    del dev
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(cfg, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the workload's queries."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from hils_inputs.configs import make_host_inputs
    from oracle.hils_oracle import ref_forward
    host = make_host_inputs(cfg)
    rng = np.random.default_rng(123)
    order = rng.permutation(cfg["Lq"])
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]))
    done, flops, t_used = 0, 0.0, 0.0
    with threadpool_limits(limits=1):
        while t_used < seconds and done < cfg["Lq"]:
            qs = np.sort(order[done:done + 16])
            t0 = time.perf_counter()
            ref_forward(host["q"], host["k"], host["v"], host["lmk"], None, queries=qs, **kw)
            t_used += time.perf_counter() - t0
            flops += forward_flops(cfg, queries=qs)
            done += len(qs)
    return dict(value=flops / t_used / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                sample="%d of %d query positions (random), all %d batch x kv-head groups, "
                       "fp64 numpy, one thread, %.1f s" % (done, cfg["Lq"], cfg["B"] * cfg["Hkv"],
                                                          t_used))


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the decode and training lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", default=None, help="run one workload: prefill_8k, decode_128k, "
                                                     "decode_4m, train_8k, prefill_32k")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import chunk_wise_sparse_landmark_amd as hl
    from hils_inputs.configs import config
    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    hl.load_library()
    ev = HipEvents()

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    if args.only is None:
        main_name = "prefill_8k"
    else:
        main_name = args.only if args.only in ("prefill_8k", "prefill_32k") else None
    extra = []
    line = None
    if main_name is not None:
        cfg = config(main_name)
        log("%s: %d warmup + %d timed steps" % (main_name, args.warmup, args.steps))
        r = run_prefill(hl, cfg, args.steps, args.warmup, ev)
        log("%s: %.3f ms/step, %.1f TFLOP/s" % (main_name, r["ms_per_step"], r["value"]))
        line = {"metric": METRIC, "value": r["value"], "unit": r["unit"], "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded counter generator; landmark = chunk-mean of keys + "
                        "N(0,0.1^2) noise)",
                "config": {"workload": main_name, "batch": cfg["B"], "heads_q": cfg["Hq"],
                           "heads_kv": cfg["Hkv"], "head_dim": cfg["d"], "seq_len": cfg["Lq"],
                           "chunk_size": cfg["S"], "top_k": cfg["K"], "causal": True,
                           "keep_own_chunk": True, "parallelism": "single GPU"},
                "roofline": r["roofline"]}
    todo = []
    if not args.no_extra and args.only is None:
        todo = ["decode_128k", "decode_4m", "train_8k"]
    elif args.only in ("decode_128k", "decode_4m", "train_8k"):
        todo = [args.only]
    for name in todo:
        cfg = config(name)
        if name.startswith("decode"):
            steps, warm = max(args.steps * 10, 100), max(args.warmup, 10)
            nsets = 4 if name == "decode_128k" else 3
            log("%s: %d sets, %d warmup + %d timed steps" % (name, nsets, warm, steps))
            r = run_decode(hl, cfg, steps, warm, ev, nsets)
            log("%s: %.1f us/step, %.0f GB/s" % (name, r["ms_per_step"] * 1e3, r["value"]))
        else:
            steps, warm = max(2, args.steps // 4), max(1, args.warmup // 2)
            log("%s: %d warmup + %d timed steps" % (name, warm, steps))
            r = run_train(hl, cfg, steps, warm, ev)
            log("%s: %.3f ms/step, %.1f TFLOP/s" % (name, r["ms_per_step"], r["value"]))
        r["workload"] = name
        r["steps"] = steps
        extra.append(r)
    if line is None:
        r = extra.pop(0)
        line = {"metric": METRIC, "value": r["value"], "unit": r["unit"], "n_gpus": 1,
                "steps": r["steps"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic", "config": {"workload": r["workload"]},
                "roofline": r.get("roofline")}
    line["extra"] = extra
    if not args.no_cpu and main_name is not None:
        log("cpu baseline: oracle on a sample (~%.0f s)" % args.cpu_seconds)
        line["cpu_baseline"] = cpu_baseline(config(main_name), args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
