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
them), the training step (forward + backward, TFLOP/s), and landmark formation
with its backward over the training batch's keys (algorithmic HBM GB/s, 16
rotating input sets).  The `_swa512` lines repeat prefill_8k, decode_128k and
train_8k with a 512-token chunk-aligned local window (8 chunk slots) beside the
top-K retrieval.  `prefill_8k_corr` repeats prefill_8k with correlated adjacent
queries (first-order autoregressive along the sequence, rho = 0.98), the regime
in which the query-block union kernel saves work; its line reports the measured
share of chunks that adjacent queries have in common.  `train_8k_qcal` repeats the
training step with a separate rank-8 retrieval query (score gradients to it), and
`train_32k` runs it at 32K tokens (batch 1, 512 chunks).

Every input is resident in HBM before timing.  Per-kernel durations come from
HIP events the library records around each launch of the dominant kernel on
its own stream (hils_profile_kernel).
"""
import argparse
import csv
import ctypes
import glob
import hashlib
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
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "chunk_wise_sparse_landmark_amd", "csrc")
# source files whose text fixes each timed kernel's machine code
KERNEL_SOURCES = {
    "prefill_attend": ["hils_prefill.hip", "hils_mfma.h", "hils_common.h"],
    "prefill_select": ["hils_prefill.hip", "hils_mfma.h", "hils_common.h"],
    "decode_attend": ["hils_decode.hip", "hils_mfma.h", "hils_common.h"],
    "decode_score": ["hils_decode.hip", "hils_mfma.h", "hils_common.h"],
    "generic_attend": ["hils_generic.hip", "hils_common.h"],
    "generic_bwd_chunks": ["hils_generic.hip", "hils_common.h"],
    "prefill_bwd_chunks": ["hils_prefill_bwd.hip", "hils_mfma.h", "hils_common.h"],
    "prefill_bwd_rows": ["hils_prefill_bwd.hip", "hils_mfma.h", "hils_common.h"],
    "landmarks": ["hils_landmarks.hip", "hils_common.h"],
    "landmarks_bwd": ["hils_landmarks.hip", "hils_common.h"],
}
# kernel family -> substring of its kernel symbols (default: the family name)
KERNEL_SYMBOLS = {"landmarks": "landmark_forward", "landmarks_bwd": "landmark_backward"}
COPY_MIB = 1024   # size of the plain copy that calibrates the HBM byte counters


# --------------------------------------------------------------------------- HIP events
class HipEvents:
    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    # no system-scope fence at the event record: the default one lengthens the
    # bracketed interval of a short kernel
    FLAGS = 0x20000000   # hipEventDisableSystemFence

    def create(self, n, flags=None):
        out = []
        self.rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        for _ in range(n):
            e = ctypes.c_void_p()
            f = self.FLAGS if flags is None else flags
            assert self.rt.hipEventCreateWithFlags(ctypes.byref(e), f) == 0
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
def local_chunks(cfg):
    """Width of the chunk-aligned local window in chunk slots (1 = own chunk only)."""
    return int(cfg["win"]) if cfg.get("win") is not None else (1 if cfg["keep_own"] else 0)


def query_counts(cfg):
    """Per causal query position i: (#candidates, #selected, #local-window tokens).
    The window is the own chunk's visible tokens and the w - 1 chunks before it;
    candidates are the complete chunks before the window."""
    import numpy as np
    S, K, Lq, Lkv = cfg["S"], cfg["K"], cfg["Lq"], cfg["Lkv"]
    NC = Lkv // S
    w = local_chunks(cfg)
    t = Lkv - Lq + np.arange(Lq)
    own = t // S
    ncand = np.clip(own - max(w - 1, 0), 0, NC)
    nsel = np.minimum(ncand, K)
    if w > 0:
        nloc = (t - own * S + 1) + S * np.minimum(w - 1, own)
    else:
        nloc = np.zeros(Lq, dtype=np.int64)
    return ncand.astype(np.int64), nsel.astype(np.int64), nloc.astype(np.int64)


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


# --------------------------------------------------------------------------- HBM traffic
def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        path = os.path.join(CSRC, f)
        if os.path.exists(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_file(kernel, workload):
    return os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel, workload))


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or the kernel's sources changed since it was taken."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    for ln in open(path):
        if ln.startswith("{"):
            rec = json.loads(ln)
            if rec.get("source_hash") == source_hash(kernel):
                return rec["traffic_bytes_per_launch"]
    return None


def _counter_means(run_dir):
    """{kernel name: {counter: mean over dispatches}} from a rocprofv3 --pmc csv run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under " + run_dir)
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            d = acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], [])
            d.append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def _find(means, key):
    hits = [k for k in means if key in k]
    if not hits:
        raise SystemExit("kernel %r not in counter output (have: %s)" % (key, list(means)[:8]))
    return hits[0]


def summarize_traffic(kernel, workload, fetch_dir, write_dir, commands):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of `kernel`, each scaled by what
    the same counter reads for the plain COPY_MIB copy in the same run."""
    fm, wm = _counter_means(fetch_dir), _counter_means(write_dir)
    copy_bytes = COPY_MIB * 2 ** 20
    ck_f, ck_w = _find(fm, "copy_u4"), _find(wm, "copy_u4")
    f_fetch = copy_bytes / (fm[ck_f]["FETCH_SIZE"] * 1024.0)
    f_write = copy_bytes / (wm[ck_w]["WRITE_SIZE"] * 1024.0)
    sym = KERNEL_SYMBOLS.get(kernel, kernel)
    kf, kw = _find(fm, sym), _find(wm, sym)
    fetch_b = fm[kf]["FETCH_SIZE"] * 1024.0 * f_fetch
    write_b = wm[kw]["WRITE_SIZE"] * 1024.0 * f_write
    rec = dict(kernel=kernel, workload=workload, source_hash=source_hash(kernel),
               fetch_kib_per_dispatch=fm[kf]["FETCH_SIZE"], write_kib_per_dispatch=wm[kw]["WRITE_SIZE"],
               copy_bytes=copy_bytes, copy_fetch_kib=fm[ck_f]["FETCH_SIZE"],
               copy_write_kib=wm[ck_w]["WRITE_SIZE"], fetch_scale=f_fetch, write_scale=f_write,
               fetch_bytes_per_launch=fetch_b, write_bytes_per_launch=write_b,
               traffic_bytes_per_launch=fetch_b + write_b)
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(kernel, workload), "w") as f:
        f.write("HBM traffic of %s on %s (rocprofv3 --pmc, one counter per run)\n" % (kernel, workload))
        for c in commands:
            f.write("command: %s\n" % c)
        f.write("copy calibration: copy_u4 of %d MiB (reads and writes exactly that much); "
                "scale = copy bytes / counter bytes\n" % COPY_MIB)
        f.write("%-28s %14s %14s\n" % ("dispatch mean", "FETCH_SIZE KiB", "WRITE_SIZE KiB"))
        f.write("%-28s %14.1f %14.1f\n" % (kernel, rec["fetch_kib_per_dispatch"],
                                             rec["write_kib_per_dispatch"]))
        f.write("%-28s %14.1f %14.1f\n" % ("copy (%d MiB)" % COPY_MIB, rec["copy_fetch_kib"],
                                             rec["copy_write_kib"]))
        f.write("scaled bytes per launch: fetch %.4g, write %.4g, total %.4g\n"
                % (fetch_b, write_b, fetch_b + write_b))
        f.write(json.dumps(rec) + "\n")
    return rec


def summarize_stats(run_dir, out_name, command):
    """Short text copy of a rocprofv3 --kernel-trace --stats run."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under " + run_dir)
    rows = list(csv.DictReader(open(files[0])))
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, out_name), "w") as f:
        f.write("rocprofv3 kernel statistics\ncommand: %s\n" % command)
        f.write("%-44s %6s %12s %12s %12s %12s %7s\n" % ("kernel", "calls", "total_us", "avg_us",
                                                         "min_us", "max_us", "pct"))
        for r in rows:
            f.write("%-44s %6s %12.1f %12.2f %12.2f %12.2f %7.2f\n" % (
                r["Name"][:44], r["Calls"], float(r["TotalDurationNs"]) / 1e3,
                float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                float(r["Percentage"])))


def copy_calibration():
    """One plain device copy of COPY_MIB MiB (its counters scale FETCH_SIZE/WRITE_SIZE)."""
    import torch
    from hils_inputs.device import device_copy
    src = torch.empty(COPY_MIB * 2 ** 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    device_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def hbm_read_probe(ev, nwg=1024, window_mib=128, total_mib=2048, launches=48):
    """GB/s of a plain streaming read (hils_inputs' read_u4) over rotating 128 MiB
    windows of a 2 GiB buffer: a window is read again only after 1.9 GiB of other
    reads, so the last-level cache cannot serve it.  This is the read rate the part
    sustains by itself, beside the 8 TB/s peak the rooflines use."""
    import torch
    from hils_inputs.device import device_read
    buf = torch.empty(total_mib * 2 ** 20, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(nwg * 256, dtype=torch.int32, device="cuda")
    nwin, wb = total_mib // window_mib, window_mib * 2 ** 20
    ms, n = timed_batch(lambda i: device_read(buf[(i % nwin) * wb:], wb, sink, nwg), launches, ev)
    del buf, sink
    torch.cuda.empty_cache()
    return {"read_GBps": wb / (ms * 1e-3) / 1e9, "bytes_per_launch": wb, "workgroups": nwg,
            "launches": n, "buffer_bytes": total_mib * 2 ** 20,
            "kernel": "read_u4 (hils_inputs): 4 x 16 B loads in flight per thread"}


def mfma_probe(ev, iters=2048, launches=6):
    """TFLOP/s of a plain dense bf16 MFMA loop (hils_inputs' mfma_loop: 256
    workgroups x 8 waves, eight independent 16x16x32 chains per wave, operands
    in registers): the matrix rate the part sustains by itself, beside the
    2.5 PFLOP/s peak the rooflines use."""
    import torch
    from hils_inputs.device import device_mfma_loop
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    ms, n = timed_batch(lambda i: device_mfma_loop(iters, sink), launches, ev)
    flops = 256 * 8 * iters * 8 * 2.0 * 16 * 16 * 32
    return {"TFLOPs": flops / (ms * 1e-3) / 1e12, "flops_per_launch": flops, "launches": n,
            "kernel": "mfma_loop (hils_inputs): 16x16x32 bf16, 8 chains per wave, 2 waves per SIMD"}


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


_SLEEP_CYCLES_PER_MS = None


def _hold(ms, ev):
    """Keep the stream busy for about `ms` (torch's bounded spin kernel), so that
    work enqueued meanwhile by the host runs back to back afterwards."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        t0, t1 = ev.create(1)[0], ev.create(1)[0]
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        ev.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        torch.cuda._sleep(1000)
        ev.rt.hipEventRecord(ctypes.c_void_p(t0), st)
        torch.cuda._sleep(1000000)
        ev.rt.hipEventRecord(ctypes.c_void_p(t1), st)
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1000000 / max(ev.elapsed_ms(t0, t1), 1e-3)
        ev.destroy([t0, t1])
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def timed_batch(fn, n, ev, host_us=60.0):
    """Mean ms per call of `fn(i)`, i < n, between one pair of HIP events.  The
    calls are enqueued while the stream is held busy (host_us per call), so the
    GPU runs them back to back and the mean is their device time, not the
    host's launch rate."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    t0, t1 = ev.create(1)[0], ev.create(1)[0]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ev.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    _hold(n * host_us * 1e-3 + 2.0, ev)
    ev.rt.hipEventRecord(ctypes.c_void_p(t0), st)
    for i in range(n):
        fn(i)
    ev.rt.hipEventRecord(ctypes.c_void_p(t1), st)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(t0, t1) / n
    ev.destroy([t0, t1])
    return ms, n


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


def selection_stats(idx, cfg):
    """From a selection idx [B, Hkv, L, K] (ascending, -1 padded): the mean share of
    chunks a query has in common with the next query of the same chunk (over
    queries with K selections), and the mean union size over 64-query windows."""
    import numpy as np
    B, Hkv, L, K = idx.shape
    NC = cfg["Lkv"] // cfg["S"]
    rows = idx.reshape(-1, K)
    hot = np.zeros((rows.shape[0], NC + 1), dtype=bool)
    hot[np.repeat(np.arange(rows.shape[0]), K), np.where(rows >= 0, rows, NC).reshape(-1)] = True
    hot = hot[:, :NC].reshape(B * Hkv, L, NC)
    full = (idx >= 0).sum(-1).reshape(B * Hkv, L) == K
    pos = np.arange(L - 1)
    same = (pos // cfg["S"]) == ((pos + 1) // cfg["S"])
    pair = full[:, :-1] & full[:, 1:] & same[None, :]
    shared = (hot[:, :-1] & hot[:, 1:]).sum(-1) / K
    union = hot.reshape(B * Hkv, L // 64, 64, NC).any(axis=2).sum(-1)
    return dict(adjacent_sharing=float(shared[pair].mean()) if pair.any() else None,
                union_chunks_per_64_queries=float(union.mean()))


def run_prefill(hl, cfg, steps, warmup, ev):
    import torch
    from hils_inputs.device import make_device_inputs
    _, dev = make_device_inputs(cfg)
    out = torch.empty_like(dev["q"])
    idx = torch.empty((cfg["B"], cfg["Hkv"], cfg["Lq"], cfg["K"]), dtype=torch.int32, device="cuda")
    lse = torch.empty((cfg["B"], cfg["Hq"], cfg["Lq"]), dtype=torch.float32, device="cuda")
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]),
              local_chunks=local_chunks(cfg))
    o, i, l = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, **kw)
    sel_stats = selection_stats(i.cpu().numpy(), cfg)
    ws = None
    p = hl.make_params(batch=cfg["B"], heads_q=cfg["Hq"], heads_kv=cfg["Hkv"], head_dim=cfg["d"],
                       seq_q=cfg["Lq"], seq_kv=cfg["Lkv"], chunk_size=cfg["S"], top_k=cfg["K"],
                       num_landmarks=dev["lmk"].shape[2], causal=True,
                       keep_own_chunk=cfg["keep_own"], local_chunks=local_chunks(cfg))
    need = hl.hils_workspace_size(p, hl.HILS_OP_FORWARD)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step(_):
        hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out=out, sel_idx=idx,
                        lse=lse, ws=ws, **kw)

    kern = "prefill_attend" if launched(hl, ev, "prefill_attend", lambda: step(0)) else "generic_attend"
    ms, kms, n = timed(step, steps, warmup, ev, kern, hl)
    sel = "prefill_select" if kern == "prefill_attend" else "generic_select"
    _, sel_ms, _ = timed(step, steps, 1, ev, sel, hl)
    flops = forward_flops(cfg)
    ncand, nsel, nown = query_counts(cfg)
    G, d, S = cfg["Hq"] // cfg["Hkv"], cfg["d"], cfg["S"]
    attn_flops = float(cfg["B"] * cfg["Hq"] * (2 * d * nsel + 4 * d * (S * nsel + nown)).sum())
    res = dict(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s", ms_per_step=ms,
               roofline=dict(bound="mfma", kernel=kern, kernel_ms=kms, launches=n,
                             achieved=attn_flops / (kms * 1e-3) / 1e12, peak=PEAK_BF16_TFLOPS,
                             unit="TFLOP/s",
                             traffic=recorded_traffic(kern, cfg.get("name", "")),
                             per_launch_flops=attn_flops))
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_BF16_TFLOPS
    res["kernels_ms"] = {kern: kms, sel: sel_ms}
    res["selection"] = sel_stats
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
                       num_landmarks=cfg["Lkv"] // cfg["S"], keep_own_chunk=cfg["keep_own"],
                       local_chunks=local_chunks(cfg))
    ws = torch.empty(max(1, hl.hils_workspace_size(p, hl.HILS_OP_DECODE)), dtype=torch.uint8,
                     device="cuda")
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], keep_own_chunk=bool(cfg["keep_own"]),
              local_chunks=local_chunks(cfg))

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
                             traffic=recorded_traffic(kern, cfg.get("name", "")),
                             per_launch_bytes=kbytes))
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_HBM_GBS
    res["frac_of_hbm_peak"] = res["value"] / PEAK_HBM_GBS
    # the step's other timed launches (the fuse launch after the attention has no hook)
    res["kernels_ms"] = {kern: kms}
    for other in ("decode_score", "decode_merge", "decode_attend"):
        if other != kern and launched(hl, ev, other, lambda: step(0)):
            res["kernels_ms"][other] = timed(step, max(20, steps // 4), 2, ev, other, hl)[1]
    # the generated queries and landmarks of set 0, for the CPU baseline
    res["_host"] = (sets[0]["q"].float().cpu().numpy(), sets[0]["lmk"].float().cpu().numpy())
    del sets, outs
    torch.cuda.empty_cache()
    return res


def run_train(hl, cfg, steps, warmup, ev):
    import torch
    from hils_inputs.device import make_device_inputs
    _, dev = make_device_inputs(cfg)
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]),
              local_chunks=local_chunks(cfg))

    qr = dev.get("q_ret")

    def step(_):
        out, idx, lse = hl.hils_forward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, q_ret=qr,
                                        **kw)
        hl.hils_backward(dev["q"], dev["k"], dev["v"], dev["lmk"], None, out, dev["dout"], idx,
                         lse, q_ret=qr, **kw)

    mfma = launched(hl, ev, "prefill_bwd_rows", lambda: step(0))
    kernels = ["prefill_bwd_rows", "prefill_bwd_chunks"] if mfma else ["generic_bwd_rows", "generic_bwd_chunks"]
    ms, kms0, n0 = timed(step, steps, warmup, ev, kernels[0], hl)
    _, kms1, n1 = timed(step, steps, 1, ev, kernels[1], hl)
    flops = forward_flops(cfg) + backward_flops(cfg)
    res = dict(value=flops / (ms * 1e-3) / 1e12, unit="TFLOP/s", ms_per_step=ms,
               frac_of_bf16_peak=flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               backward_kernels={kernels[0]: dict(kernel_ms=kms0, launches=n0),
                                 kernels[1]: dict(kernel_ms=kms1, launches=n1)})
    del dev
    torch.cuda.empty_cache()
    return res


def landmark_bytes(cfg):
    """Algorithmic HBM bytes of landmark formation (forward, backward) over every
    complete chunk: the forward reads lq and the keys and writes lmk (bf16) and
    bias (fp32); the backward reads lq, keys, dlmk, dbias and writes dlq, dk."""
    B, Hkv, d, S = cfg["B"], cfg["Hkv"], cfg["d"], cfg["S"]
    nc = B * Hkv * (cfg["Lkv"] // S)
    e = 2 if cfg["dtype"] == "bf16" else 4
    keys, rows = nc * S * d * e, nc * d * e
    return keys + 2 * rows + nc * 4, 2 * keys + 3 * rows + nc * 4


def run_landmarks(hl, cfg, steps, warmup, ev, nsets):
    """Landmark formation forward + backward over the keys of one training batch;
    inputs rotate over `nsets` independent sets so the last-level cache cannot
    hold them between steps."""
    import torch
    from hils_inputs.device import fill_normal
    B, Hkv, d, NC = cfg["B"], cfg["Hkv"], cfg["d"], cfg["Lkv"] // cfg["S"]
    sets = []
    for r in range(nsets):
        seed = cfg["seed"] + 1000 * r
        e = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        sets.append(dict(lq=fill_normal(e(B, Hkv, NC, d), seed, "lq"),
                         k=fill_normal(e(B, Hkv, cfg["Lkv"], d), seed, "k"),
                         dlmk=fill_normal(e(B, Hkv, NC, d), seed, "dlmk"),
                         dbias=fill_normal(torch.empty((B, Hkv, NC), device="cuda"), seed, "dbias")))
    torch.cuda.synchronize()

    def step(i):
        s = sets[i % nsets]
        hl.hils_landmarks(s["lq"], s["k"], chunk_size=cfg["S"])
        hl.hils_landmarks_backward(s["lq"], s["k"], s["dlmk"], s["dbias"], chunk_size=cfg["S"])

    def fwd(i):
        s = sets[i % nsets]
        hl.hils_landmarks(s["lq"], s["k"], chunk_size=cfg["S"])

    def bwd(i):
        s = sets[i % nsets]
        hl.hils_landmarks_backward(s["lq"], s["k"], s["dlmk"], s["dbias"], chunk_size=cfg["S"])

    fb, bb = landmark_bytes(cfg)
    for i in range(warmup):
        step(i)
    # these kernels last a few microseconds, less than the host needs to launch
    # them: steps and kernels are timed over back-to-back launches enqueued
    # behind a hold (an event pair around each launch would add its own latency)
    ms, _ = timed_batch(step, steps, ev, host_us=120.0)
    kms, n = timed_batch(bwd, steps, ev)
    fms, fn = timed_batch(fwd, steps, ev)
    res = dict(value=(fb + bb) / (ms * 1e-3) / 1e9, unit="GB/s", ms_per_step=ms,
               bytes_per_step=fb + bb,
               forward_kernel=dict(kernel_ms=fms, launches=fn, per_launch_bytes=fb,
                                   achieved=fb / (fms * 1e-3) / 1e9),
               roofline=dict(bound="hbm", kernel="landmarks_bwd", kernel_ms=kms, launches=n,
                             achieved=bb / (kms * 1e-3) / 1e9, peak=PEAK_HBM_GBS, unit="GB/s",
                             traffic=recorded_traffic("landmarks_bwd", cfg.get("name", "")),
                             per_launch_bytes=bb))
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_HBM_GBS
    del sets
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- CPU baseline
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_pool():
    from oracle.pool import default_workers, make_pool, warm_up
    workers = default_workers()
    pool = make_pool(workers)
    warm_up(pool, workers)
    return pool, workers


def _cpu_meta(workers):
    return dict(cores=workers, host_cpus=os.cpu_count(), cpu_model=cpu_model(),
                blas_threads_per_core=1, kind="oracle")


def cpu_baseline_prefill(pool, workers, cfg, seconds):
    """The CPU oracle, as it stands (fp64 numpy, one BLAS thread per process), on
    all host cores: random blocks of 16 query positions of every (batch, kv head)
    group, handed out to a process pool until ``seconds`` of wall time are spent."""
    import numpy as np
    from hils_inputs.configs import make_host_inputs
    from oracle.pool import forward_tasks
    host = make_host_inputs(cfg)
    rng = np.random.default_rng(123)
    groups = [(b, g) for b in range(cfg["B"]) for g in range(cfg["Hkv"])]
    order = rng.permutation(cfg["Lq"])
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]),
              local_chunks=local_chunks(cfg))
    per_group = 1.0 / (cfg["B"] * cfg["Hkv"])
    done, flops, ntask, t_used = 0, 0.0, 0, 0.0
    nblk = max(1, -(-2 * workers // len(groups)))     # at least two tasks per worker a round
    while t_used < seconds and done < cfg["Lq"]:
        blocks = [np.sort(order[x:x + 16]) for x in range(done, min(done + 16 * nblk, cfg["Lq"]), 16)]
        tasks = [(b, g, qs) for (b, g) in groups for qs in blocks]
        t0 = time.perf_counter()
        forward_tasks(pool, host, tasks, **kw)
        t_used += time.perf_counter() - t0
        for qs in blocks:
            flops += forward_flops(cfg, queries=qs)
            done += len(qs)
        ntask += len(tasks)
    r = dict(value=flops / t_used / 1e12, unit="TFLOP/s",
             sample="%d of %d query positions (random, blocks of 16), all %d batch x kv-head "
                    "groups (%d pool tasks), %.1f s wall" % (done, cfg["Lq"], len(groups), ntask,
                                                              t_used))
    r.update(_cpu_meta(workers))
    return r


def cpu_baseline_decode(pool, workers, cfg, host_q, host_lmk, seconds):
    """The CPU oracle on the decode workload (input set 0: its queries and landmark
    table as generated; K and V regenerated lazily, chunk by chunk): one pool task
    per (batch, kv head) group, repeated until ``seconds`` of wall time are spent.
    Throughput uses the GPU line's algorithmic bytes per step."""
    from hils_inputs.configs import LazyNormalBF16
    from oracle.pool import forward_tasks
    shape = (cfg["B"], cfg["Hkv"], cfg["Lkv"], cfg["d"])
    host = dict(q=host_q, lmk=host_lmk, bias=None, q_ret=None,
                k=LazyNormalBF16(cfg["seed"], "k", shape), v=LazyNormalBF16(cfg["seed"], "v", shape))
    kw = dict(chunk_size=cfg["S"], top_k=cfg["K"], causal=True, keep_own_chunk=bool(cfg["keep_own"]),
              local_chunks=local_chunks(cfg))
    tasks = [(b, g, [0]) for b in range(cfg["B"]) for g in range(cfg["Hkv"])]
    total, _, _ = decode_bytes(cfg)
    steps, t_used = 0, 0.0
    while t_used < seconds and steps < 50:
        t0 = time.perf_counter()
        forward_tasks(pool, host, tasks, **kw)
        t_used += time.perf_counter() - t0
        steps += 1
    r = dict(value=total * steps / t_used / 1e9, unit="GB/s", ms_per_step=1e3 * t_used / steps,
             sample="%d whole decode steps (%d batch x kv-head pool tasks each), %.1f s wall"
                    % (steps, len(tasks), t_used))
    r.update(_cpu_meta(workers))
    return r


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the decode and training lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None, help="run one workload: prefill_8k, decode_128k, "
                                                     "decode_4m, train_8k, landmarks_8k, prefill_32k, "
                                                     "train_32k, train_8k_qcal, prefill_8k_corr, "
                                                     "or prefill_8k, decode_128k, train_8k + _swa512")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain %d MiB device copy (HBM counter calibration)" % COPY_MIB)
    ap.add_argument("--traffic-summary", nargs=4, metavar=("KERNEL", "WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/<kernel>_<workload>_traffic.txt from two --pmc runs")
    ap.add_argument("--stats-summary", nargs=2, metavar=("RUN_DIR", "OUT_NAME"),
                    help="write profiles/OUT_NAME from a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--command", action="append", default=[],
                    help="the profiling command(s) a summary records")
    args = ap.parse_args()
    if args.traffic_summary:
        k, w, fd, wd = args.traffic_summary
        print(json.dumps(summarize_traffic(k, w, fd, wd, args.command)))
        return
    if args.stats_summary:
        summarize_stats(args.stats_summary[0], args.stats_summary[1], " ; ".join(args.command))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
                "roofline": r["roofline"], "kernels_ms": r.get("kernels_ms"),
                "selection": r.get("selection")}
    todo = []
    if not args.no_extra and args.only is None:
        todo = ["decode_128k", "decode_4m", "prefill_32k", "train_8k", "landmarks_8k",
                "prefill_8k_swa512", "decode_128k_swa512", "train_8k_swa512", "prefill_8k_corr",
                "train_8k_qcal", "train_32k"]
    elif args.only in ("decode_128k", "decode_4m", "train_8k", "landmarks_8k", "prefill_8k_swa512",
                       "decode_128k_swa512", "train_8k_swa512", "prefill_8k_corr", "train_8k_qcal",
                       "train_32k"):
        todo = [args.only]
    for name in todo:
        cfg = dict(config("train_8k"), name=name) if name == "landmarks_8k" else config(name)
        if name.startswith("prefill"):
            log("%s: %d warmup + %d timed steps" % (name, args.warmup, args.steps))
            r = run_prefill(hl, cfg, args.steps, args.warmup, ev)
            steps = args.steps
            log("%s: %.3f ms/step, %.1f TFLOP/s" % (name, r["ms_per_step"], r["value"]))
        elif name == "landmarks_8k":
            steps, warm = max(args.steps * 5, 50), max(args.warmup, 5)
            log("%s: 16 sets, %d warmup + %d timed steps" % (name, warm, steps))
            r = run_landmarks(hl, cfg, steps, warm, ev, 16)
            log("%s: %.1f us/step, %.0f GB/s" % (name, r["ms_per_step"] * 1e3, r["value"]))
        elif name.startswith("decode"):
            steps, warm = max(args.steps * 10, 100), max(args.warmup, 10)
            nsets = 4 if name.startswith("decode_128k") else 3
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
        for key in ("kernels_ms", "selection", "backward_kernels", "forward_kernel", "frac_of_hbm_peak",
                    "_host"):
            if key in r:
                line[key] = r[key]
    line["extra"] = extra
    line["hbm_read_probe"] = hbm_read_probe(ev)
    log("hbm read probe: %.0f GB/s" % line["hbm_read_probe"]["read_GBps"])
    line["mfma_probe"] = mfma_probe(ev)
    log("mfma probe: %.0f TFLOP/s" % line["mfma_probe"]["TFLOPs"])
    # each roofline also against the rate the part sustains by itself
    for r in [line] + extra:
        rf = r.get("roofline")
        if not rf or not rf.get("achieved"):
            continue
        ceil = (line["mfma_probe"]["TFLOPs"] if rf.get("bound") == "mfma"
                else line["hbm_read_probe"]["read_GBps"] if rf.get("bound") == "hbm" else None)
        if ceil:
            rf["measured_peak"] = ceil
            rf["frac_of_measured"] = rf["achieved"] / ceil
    if args.calibrate_copy:
        copy_calibration()
    if not args.no_cpu:
        pool, workers = _cpu_pool()
        try:
            if main_name is not None:
                log("cpu baseline: oracle on %d cores, %s (~%.0f s)" % (workers, main_name,
                                                                       args.cpu_seconds))
                line["cpu_baseline"] = cpu_baseline_prefill(pool, workers, config(main_name),
                                                            args.cpu_seconds)
            for r in [line] + extra:
                name = r.get("workload") or r.get("config", {}).get("workload")
                if name in ("decode_128k", "decode_4m") and "_host" in r:
                    log("cpu baseline: oracle on %d cores, %s (~%.0f s)" % (workers, name,
                                                                           args.cpu_seconds / 2))
                    r["cpu_baseline"] = cpu_baseline_decode(pool, workers, config(name),
                                                            *r["_host"], args.cpu_seconds / 2)
        finally:
            pool.shutdown()
    for r in [line] + extra:
        r.pop("_host", None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
