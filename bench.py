#!/usr/bin/env python3
"""Benchmark of the Double Sparsity decode-attention step on one MI355X.

A step is one decode step of one attention layer for the whole batch: label
append of the current token, query gather + approximate scores, top-k select,
exact attention over the selected K/V rows, split merge (all in libds.so).
The metric counts queries: one query is one batch row's decode step on one
layer, so queries/s = batch * steps / time.

Cache residency: a real model runs its other layers between two visits to a
layer, so that layer's label cache and K/V rows are no longer in the 256 MB
Infinity Cache.  The benchmark reproduces that by rotating through `--layers`
independent copies of the layer's K/V cache and label cache (each copy larger
than the Infinity Cache for the default workload); every timed step is real
work and nothing is flushed inside the timed region.

Prints one JSON line (rank 0, N = 1 only; this build runs on one GPU).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode-attn queries/s + achieved HBM GB/s, Llama-2-7B-shaped @4K–128K"
HBM_PEAK_GBS = 8000.0
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def algorithmic_bytes(cfg, S):
    """Bytes one step must move for one layer at length S (all rows): the
    label stream (S * lam per (b, g) row, lam = 2r for fp16 labels, r/2 + 2 for
    int4 codes + fp16 scale), the min(k, S) selected K/V rows of
    (d_k + d_v) * 2 bytes per row, the label append (r K values read, lam
    bytes written per row), the query read and the output written."""
    rows = cfg.B * cfg.Hkv
    lam = 0
    if cfg.k > 0:
        lam = cfg.r // 2 + 2 if cfg.int4 else 2 * cfg.r
    kk = min(cfg.k, S) if cfg.k > 0 else S
    return {"labels": rows * S * lam,
            "append": rows * (2 * cfg.r + lam) if cfg.k > 0 else 0,
            "rows": rows * kk * (cfg.d_k + cfg.d_v) * 2,
            "q": cfg.B * cfg.Hq * cfg.D * 2,
            "out": cfg.B * cfg.Hq * cfg.d_v * 2}


def dominant_kernel(plan, ab, G):
    """The kernel that takes most of a step on this path, its name prefix in
    profiles, and its algorithmic bytes per launch."""
    if plan["path"] == "fused":
        return ("k_decode_fused_g" if G > 1 else "k_decode_fused"), sum(ab.values())
    final = plan["n_split"] == 1
    return "k_attn", ab["rows"] + ab["q"] + (ab["out"] if final else 0)


def pct_us(ms_list):
    """[median, 90th percentile] of a list of durations in ms, in µs."""
    if not ms_list:
        return None
    st = sorted(ms_list)
    return [round(st[len(st) // 2] * 1e3, 3), round(st[min(len(st) - 1, (9 * len(st)) // 10)] * 1e3, 3)]


def copy_ceiling_gbs(torch, mib=1024, reps=5):
    """A plain device copy of `mib` MiB (torch's copy kernel): bytes read plus
    written per second, the box's practical streaming ceiling beside the
    8 TB/s peak."""
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    return 2.0 * mib * (1 << 20) / (ms * 1e-3) / 1e9


def source_hash():
    """Hash of the kernel sources, comments and blank space left out: a stored
    counter record is only used while the code it was taken on is unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sparse_attention_decode_ds_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            text = open(os.path.join(d, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def stored_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the stored counter record, or None
    if there is none or the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(traffic_path(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash() or rec.get("kernel") != kernel:
        return None
    return rec.get("bytes_per_launch")


def _pmc_rows(path):
    import csv
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            yield r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r.get("Dispatch_Id")


def _pmc_mean(path, counter, match):
    """Mean over dispatches whose kernel name contains `match` of the counter
    (values of one dispatch summed, e.g. over XCDs)."""
    per = {}
    for name, cn, v, did in _pmc_rows(path):
        if cn == counter and match in name:
            per[did] = per.get(did, 0.0) + v
    return (sum(per.values()) / len(per), len(per)) if per else (None, 0)


def write_traffic(args):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, each with --calib-copy-mb) into the stored counter record."""
    import sparse_attention_decode_ds_amd as ds
    import synth
    fetch_csv, write_csv = args.traffic_from
    name = synth.CONFIGS[args.workload].name if args.workload in synth.CONFIGS else args.workload
    kern = args.traffic_kernel
    calib_kib = args.calib_copy_mb * 1024.0
    cf, ncf = _pmc_mean(fetch_csv, "FETCH_SIZE", "neg_kernel")
    cw, ncw = _pmc_mean(write_csv, "WRITE_SIZE", "neg_kernel")
    kf, nkf = _pmc_mean(fetch_csv, "FETCH_SIZE", kern)
    kw, nkw = _pmc_mean(write_csv, "WRITE_SIZE", kern)
    if None in (cf, cw, kf, kw):
        print("bench.py: counters missing (calibration %s/%s, kernel %s/%s)" % (cf, cw, kf, kw),
              file=sys.stderr)
        return 1
    f_fetch, f_write = calib_kib / cf, calib_kib / cw
    rec = {"workload": name, "kernel": kern, "source_hash": source_hash(),
           "fetch_kib_per_launch": round(kf, 1), "write_kib_per_launch": round(kw, 1),
           "dispatches": [nkf, nkw],
           "calibration": {"copy_mib": args.calib_copy_mb, "fetch_kib": round(cf, 1),
                           "write_kib": round(cw, 1), "dispatches": [ncf, ncw],
                           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
           "bytes_per_launch": int(round((kf * f_fetch + kw * f_write) * 1024.0)),
           "commands": args.traffic_cmd or []}
    dst = args.traffic_out or traffic_path(name)
    os.makedirs(os.path.dirname(os.path.abspath(dst)), exist_ok=True)
    with open(dst, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return 0


def cpu_baseline(cfg, inp, seconds):
    """The oracle (as it stands) on a bounded sample of the workload: a few
    whole batch rows of one decode step, repeated for about `seconds`."""
    import numpy as np

    import oracle

    S = cfg.S0 + 1
    per_row = cfg.Hkv * (S * (cfg.r + 8) + min(cfg.k if cfg.k > 0 else S, S) * 600)
    n_b = max(1, min(cfg.B, int(2e8 // max(per_row, 1))))
    q = inp.q[:n_b].cpu().numpy()
    K = inp.K[:n_b].cpu().numpy()
    V = inp.V[:n_b].cpu().numpy()
    chan = inp.chan.cpu().numpy() if inp.chan is not None else None
    keep = inp.keep.cpu().numpy() if inp.keep is not None else None
    lab = None
    if cfg.k > 0:
        lab = oracle.Labels.empty(n_b, cfg.Hkv, K.shape[2] + (-K.shape[2]) % 16, cfg.r, cfg.int4)
        oracle.label_build(K, chan, lab, 0, cfg.S0)
    seq = np.full(n_b, S, np.int32)
    pos = seq - 1
    threads = oracle.max_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        if lab is not None:
            oracle.label_append(K, chan, lab, pos)
        oracle.decode(q, K, V, seq, cfg.k, cfg.sm_scale, chan=chan, lab=lab, keep=keep,
                      n_threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": n_b * reps / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d batch rows (all %d KV heads each), one decode step at S=%d "
                      "(label append + scores + top-k + attention), repeated %d times in %.1f s"
                      % (n_b, cfg.B, cfg.Hkv, S, reps, el)}


def counter_reference_copy(torch, mib):
    """A plain streaming kernel of known size (reads and writes mib MiB, five
    times), the reference for the HBM byte counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


CALIB = dict(name="calib_llama2_7b_4k", B=4, Hkv=32, Hq=32, N=4096, D=128, W=64, r=16,
             criterion="qk",
             note="heavy-channel calibration of one Llama-2-7B-shaped layer: 4 sample sequences "
                  "of 4096 tokens, 32 KV heads, a 64-query observation window, QK-outlier, r 16")


def run_calibration(args):
    """Times ds_calibrate_channels on the calibration workload: K of one layer's
    samples and the window queries already in HBM, a rotation of K copies that
    moves well over the Infinity Cache, HIP events on the call's stream."""
    import torch

    import oracle
    import sparse_attention_decode_ds_amd as ds

    c = CALIB
    torch.cuda.set_device(0)
    ds.load()
    if args.calib_copy_mb > 0:
        counter_reference_copy(torch, args.calib_copy_mb)
    g = torch.Generator(device="cuda").manual_seed(1234)
    B, Hkv, N, D, W = c["B"], c["Hkv"], c["N"], c["D"], c["W"]
    k_bytes = B * Hkv * N * D * 2
    L = max(2, int(math.ceil(1.5e9 / k_bytes)))
    Ks = [torch.randn((B, Hkv, N, D), generator=g, device="cuda").half() for _ in range(L)]
    q = torch.randn((B, W, c["Hq"], D), generator=g, device="cuda").half()
    need = ds.calibrate_workspace_size(Ks[0], N, q)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    norms = torch.empty((Hkv, 3, D), device="cuda")
    print("bench: calibration workload %s, %d K copies" % (c["name"], L), flush=True)

    def call(i):
        return ds.calibrate_channels(Ks[i % L], c["r"], c["criterion"], qwin=q, norms=norms,
                                     workspace=ws, validate_tables=False)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        call(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in ev]
    call_mean = sum(call_ms) / len(call_ms)
    alg = k_bytes + q.numel() * 2 + Hkv * c["r"] * 4 + norms.numel() * 4
    achieved = alg / (call_mean * 1e-3) / 1e9
    result = {
        "metric": "heavy-channel calibration layers/s + achieved HBM GB/s",
        "value": round(1e3 / ms, 1), "unit": "layers/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": c["name"], "samples": B, "kv_heads": Hkv, "tokens": N,
                   "head_dim": D, "window": W, "r": c["r"], "criterion": c["criterion"],
                   "k_copies": L, "note": c["note"]},
        "roofline": {"bound": "hbm", "kernel": "k_calib_cols + k_calib_select",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(c["name"], "k_calib_cols"),
                     "traffic_kernel": "k_calib_cols",
                     "algorithmic_bytes_per_launch": alg,
                     "avg_launch_us": round(call_mean * 1e3, 3),
                     "launch_us_p50_p90": pct_us(call_ms),
                     "timing": "torch events on the call's stream around each call (both "
                               "kernels), in a second pass of the same %d calls" % args.steps},
    }
    if not args.no_cpu_baseline:
        # the oracle on a bounded sample: one sequence and four KV heads
        Kc = Ks[0][:1, :4].cpu().numpy()
        qc = q[:1, :, :4].cpu().numpy()
        n, t1 = 0, time.perf_counter()
        while True:
            oracle.calibrate(Kc, oracle.CALIB_QK, c["r"], qwin=qc)
            n += 1
            if time.perf_counter() - t1 > min(args.cpu_seconds, 10.0):
                break
        per = (time.perf_counter() - t1) / n * (B * Hkv / 4)
        result["cpu_baseline"] = {"value": round(1.0 / per, 3), "unit": "layers/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": "1 of 4 sequences x 4 of 32 KV heads, %d calls, "
                                            "scaled by 32" % n}
    print(json.dumps(result), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama2_7b_4k")
    ap.add_argument("--layers", type=int, default=0,
                    help="independent layer caches rotated per step (0: enough that one "
                         "rotation is far larger than the Infinity Cache, 2 to 8)")
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-events", choices=["kernel", "all", "none"], default="kernel",
                    help="second pass of --steps steps with HIP events around the dominant "
                         "kernel only, around every stage, or no second pass")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the stored counter record from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE counter_collection.csv) and exit")
    ap.add_argument("--traffic-kernel", default="k_decode_fused")
    ap.add_argument("--traffic-cmd", action="append", help="command recorded with the counters")
    ap.add_argument("--traffic-out", default=None, help="record path (default: under profiles/)")
    ap.add_argument("--offload", action="store_true",
                    help="K/V in pinned host memory, read over the host link (labels in HBM)")
    ap.add_argument("--calibrate", action="store_true",
                    help="time heavy-channel calibration (%s) instead of the decode step" %
                         CALIB["name"])
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the decode path runs on one GPU; --gpus %d (WORLD_SIZE %d) is not "
              "supported (one GPU holds a whole row set; see the sharding notes)" % (args.gpus, world),
              file=sys.stderr)
        return 2
    if args.traffic_from:
        return write_traffic(args)
    if args.calibrate:
        return run_calibration(args)

    import torch

    import sparse_attention_decode_ds_amd as ds
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    lib = ds.load()
    cfg = synth.CONFIGS[args.workload]
    dev = "cuda"
    # Enough layer copies that one rotation moves well over the 256 MB
    # Infinity Cache (about 1.5 GB of step bytes), 2 to 8 copies.
    step0 = sum(algorithmic_bytes(cfg, cfg.S0 + 1).values())
    L = args.layers if args.layers > 0 else max(2, min(8, int(math.ceil(1.5e9 / step0))))
    if args.offload:
        L = 1  # one K/V copy in pinned host memory; host reads never sit in the Infinity Cache

    if args.calib_copy_mb > 0:
        counter_reference_copy(torch, args.calib_copy_mb)

    print("bench: workload %s (%s), %d layer caches" % (cfg.name, cfg.note, L), flush=True)
    inp = synth.make_inputs(cfg, dev)
    Ks, Vs, labs = [inp.K], [inp.V], []
    for _ in range(1, L):
        Ks.append(inp.K.clone())
        Vs.append(inp.V.clone())
    for l in range(L):
        if cfg.k > 0:
            lab = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4, dev)
            ds.label_build(Ks[l], inp.chan, lab, 0, cfg.S0)
            labs.append(lab)
        else:
            labs.append(None)
    if args.offload:
        # K and V in pinned host memory (mapped into the GPU's address space);
        # the labels and everything else stay in HBM
        Ks = [torch.empty(inp.K.shape, dtype=inp.K.dtype, pin_memory=True)]
        Vs = [torch.empty(inp.V.shape, dtype=inp.V.dtype, pin_memory=True)]
        Ks[0].copy_(inp.K)
        Vs[0].copy_(inp.V)
        hip = ctypes.CDLL("libamdhip64.so")
        for t in (Ks[0], Vs[0]):
            dptr = ctypes.c_void_p()
            rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
            assert rc == 0 and dptr.value == t.data_ptr(), "pinned memory not mapped for the GPU"
    n_q = 16
    qs = [synth.make_q(cfg, dev, s) for s in range(n_q)]
    seqs = [torch.full((cfg.B,), cfg.S0 + j + 1, dtype=torch.int32, device=dev)
            for j in range(cfg.steps)]
    out = torch.empty((cfg.B, cfg.Hq, cfg.d_v), dtype=torch.float16, device=dev)
    ws_bytes = ds.workspace_size(inp.K, inp.V, cfg.Hq, cfg.D, labs[0], cfg.k, cfg.cap)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print("bench: inputs ready (%.1f GB of K/V)" % (
        L * (inp.K.numel() + inp.V.numel()) * 2 / 1e9), flush=True)

    flags = ds.DECODE_APPEND if cfg.k > 0 else 0
    if args.unfused:
        flags |= ds.DECODE_UNFUSED
    S_mid = cfg.S0 + 1 + min(cfg.steps - 1, (args.steps // L) // 2)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labs[0], cfg.k, S_mid, args.n_split, flags)
    ab = algorithmic_bytes(cfg, S_mid)
    dom, dom_bytes = dominant_kernel(plan, ab, cfg.G)
    dom_stage = ds.STAGES.index("attn")  # both dominant kernels run in the attention stage

    # Pre-marshalled ctypes arguments per (layer, step): the timed loops only
    # call into the library.
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_ev = ds.STAGE_COUNT + 1
    total = args.warmup + 2 * args.steps
    if args.stage_events == "all":
        skip = ()
    else:
        skip = [i for i in range(args.steps * n_ev) if i % n_ev not in (dom_stage, dom_stage + 1)]
    events = ds.HipEvents(args.steps * n_ev, skip=skip)
    P = ctypes.c_void_p
    keep = []  # keeps ctypes objects alive

    def make_call(i, ev_base):
        l = i % L
        j = (i // L) % cfg.steps
        kv = ds.kv_desc(Ks[l], Vs[l], cfg.Hq, cfg.D)
        lab = labs[l].desc() if labs[l] is not None else None
        opts = ds.DecodeOpts()
        opts.n_split, opts.flags = args.n_split, flags
        if ev_base is not None:
            opts.stage_events = events.slot_address(ev_base)
        keep.append((kv, lab, opts))
        return (ctypes.byref(kv), P(qs[i % n_q].data_ptr()), P(Ks[l].data_ptr()),
                P(Vs[l].data_ptr()), P(seqs[j].data_ptr()), cfg.S0 + j + 1,
                P(inp.keep.data_ptr()) if inp.keep is not None else None,
                P(inp.chan.data_ptr()) if inp.chan is not None else None,
                ctypes.byref(lab) if lab is not None else None, cfg.k, cfg.sm_scale,
                P(out.data_ptr()), None, P(ws.data_ptr()), ws.numel(), ctypes.byref(opts),
                stream)

    warm = [make_call(i, None) for i in range(args.warmup)]
    timed = [make_call(args.warmup + i, None) for i in range(args.steps)]
    kpass = [make_call(args.warmup + i, i * n_ev) for i in range(args.steps)]
    fn = lib.ds_decode_attn

    for c in warm:
        rc = fn(*c)
        assert rc == 0, ds.STATUS.get(rc, rc)
    torch.cuda.synchronize()

    # Timed region: K steps, nothing but the library calls.
    t0 = time.perf_counter()
    for c in timed:
        fn(*c)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Kernel-timing pass: the same K steps again, HIP events recorded on the
    # library's stream around the dominant kernel (or every stage).
    stage_ms = {name: [] for name in ds.STAGES}
    step_ms = []
    if args.stage_events != "none":
        for c in kpass:
            fn(*c)
        torch.cuda.synchronize()
        for i in range(args.steps):
            b = i * n_ev
            for si, name in enumerate(ds.STAGES):
                if events.handles[b + si] and events.handles[b + si + 1]:
                    stage_ms[name].append(events.elapsed_ms(b + si, b + si + 1))
            if events.handles[b] and events.handles[b + ds.STAGE_COUNT]:
                step_ms.append(events.elapsed_ms(b, b + ds.STAGE_COUNT))
    mean = {k: (sum(v) / len(v) if v else None) for k, v in stage_ms.items()}

    copy_gbs = copy_ceiling_gbs(torch)

    value = cfg.B * args.steps / wall
    ms_step = wall / args.steps * 1e3
    dom_ms = mean["attn"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9 if dom_ms else None
    traffic = stored_traffic(cfg.name, dom)
    step_bytes = sum(ab.values())
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.D, "k_cols": cfg.d_k, "prefill": cfg.S0, "r": cfg.r,
                   "k": cfg.k, "labels": ("int4" if cfg.int4 else "fp16") if cfg.k > 0 else None,
                   "storage": "fp16 q/K/V", "layer_caches": L, "path": plan["path"],
                   "n_split": plan["n_split"], "note": cfg.note},
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": round(achieved, 1) if achieved else None,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "avg_launch_us": round(dom_ms * 1e3, 3) if dom_ms else None,
                     "launch_us_p50_p90": pct_us(stage_ms["attn"]),
                     "copy_gbs": round(copy_gbs, 1),
                     "frac_of_copy": round(achieved / copy_gbs, 4) if achieved else None,
                     "timing": "HIP events recorded by the kernel's own launch at its start "
                               "and end, in a second pass of the same %d steps" % args.steps},
        "step": {"algorithmic_bytes": step_bytes,
                 "hbm_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "bytes": ab,
                 "stage_mean_us": {k: (round(v * 1e3, 3) if v is not None else None)
                                   for k, v in mean.items()}},
    }
    if step_ms:
        result["step"]["us_p50_p90_events"] = pct_us(step_ms)
    if args.offload:
        # the selected K/V rows (and the appended token's K row) cross the host
        # link; the dominant kernel is priced against the link, not HBM
        link = ab["rows"] + (cfg.B * cfg.Hkv * cfg.d_k * 2 if cfg.k > 0 else 0)
        dom_link = ab["rows"]  # the dominant kernel is the one that reads the rows
        ach = dom_link / (dom_ms * 1e-3) / 1e9 if dom_ms else None
        result["config"]["kv_memory"] = "pinned host"
        result["roofline"].update({
            "bound": "host_link", "achieved": round(ach, 2) if ach else None,
            "peak": HOST_LINK_PEAK_GBS, "frac": round(ach / HOST_LINK_PEAK_GBS, 4) if ach else None,
            "traffic": None, "algorithmic_bytes_per_launch": dom_link,
            "copy_gbs": None, "frac_of_copy": None})
        result["offload"] = {"link_bytes_per_step": link,
                             "link_gbs": round(link / (ms_step * 1e-3) / 1e9, 2)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    events.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
