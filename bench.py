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


def algorithmic_bytes(cfg, S):
    """Bytes the step must move for one layer at length S (all rows):
    labels S*lambda per (b, g), lambda = 2r (fp16) or r/2 + 2 (int4 + fp16
    scale); min(k, S) K/V rows of (d_k + d_v) * 2 bytes per (b, g); q and out."""
    rows = cfg.B * cfg.Hkv
    lam = 0
    if cfg.k > 0:
        lam = cfg.r // 2 + 2 if cfg.int4 else 2 * cfg.r
    kk = min(cfg.k, S) if cfg.k > 0 else S
    q_out = cfg.B * cfg.Hq * (cfg.D + cfg.d_v) * 2
    return {"labels": rows * S * lam, "rows": rows * kk * (cfg.d_k + cfg.d_v) * 2, "q_out": q_out}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama2_7b_4k")
    ap.add_argument("--layers", type=int, default=8, help="independent layer caches rotated per step")
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--unfused", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-events", choices=["all", "attn", "none"], default="all",
                    help="HIP events per timed step: every stage boundary, only around the "
                         "attention kernel, or none")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the decode path on one GPU only; "
              "--gpus %d (WORLD_SIZE %d) is not supported" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch

    import sparse_attention_decode_ds_amd as ds
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    lib = ds.load()
    cfg = synth.CONFIGS[args.workload]
    L = max(1, args.layers)
    dev = "cuda"

    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

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

    # Pre-marshalled ctypes arguments per (layer, step): the timed loop only
    # calls into the library.
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flags = ds.DECODE_APPEND if cfg.k > 0 else 0
    if args.unfused:
        flags |= ds.DECODE_UNFUSED
    total = args.warmup + args.steps
    n_ev = ds.STAGE_COUNT + 1
    if args.stage_events == "all":
        skip = ()
    elif args.stage_events == "attn":
        skip = [i for i in range(args.steps * n_ev)
                if i % n_ev not in (ds.STAGES.index("attn"), ds.STAGES.index("attn") + 1)]
    else:
        skip = range(args.steps * n_ev)
    events = ds.HipEvents(args.steps * n_ev, skip=skip)
    calls = []
    keep = []  # keeps ctypes objects alive
    for i in range(total):
        l = i % L
        j = (i // L) % cfg.steps
        kv = ds.kv_desc(Ks[l], Vs[l], cfg.Hq, cfg.D)
        lab = labs[l].desc() if labs[l] is not None else None
        opts = ds.DecodeOpts()
        opts.n_split, opts.flags = args.n_split, flags
        ti = i - args.warmup
        if ti >= 0 and args.stage_events != "none":
            opts.stage_events = events.slot_address(ti * n_ev)
        keep.append((kv, lab, opts))
        P = ctypes.c_void_p
        calls.append((ctypes.byref(kv), P(qs[i % n_q].data_ptr()), P(Ks[l].data_ptr()),
                      P(Vs[l].data_ptr()), P(seqs[j].data_ptr()), cfg.S0 + j + 1, P(
                          inp.keep.data_ptr()) if inp.keep is not None else None,
                      P(inp.chan.data_ptr()) if inp.chan is not None else None,
                      ctypes.byref(lab) if lab is not None else None, cfg.k, cfg.sm_scale,
                      P(out.data_ptr()), None, P(ws.data_ptr()), ws.numel(), ctypes.byref(opts),
                      stream))
    fn = lib.ds_decode_attn

    for i in range(args.warmup):
        rc = fn(*calls[i])
        assert rc == 0, ds.STATUS.get(rc, rc)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        fn(*calls[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    K_steps = args.steps
    value = cfg.B * K_steps / wall
    # per-stage durations from the HIP events recorded inside the timed region
    stage_ms = {name: [] for name in ds.STAGES}
    step_ms = []
    for i in range(K_steps):
        b = i * n_ev
        for s, name in enumerate(ds.STAGES):
            if events.handles[b + s] and events.handles[b + s + 1]:
                stage_ms[name].append(events.elapsed_ms(b + s, b + s + 1))
        if events.handles[b] and events.handles[b + ds.STAGE_COUNT]:
            step_ms.append(events.elapsed_ms(b, b + ds.STAGE_COUNT))
    mean = {k: (sum(v) / len(v) if v else None) for k, v in stage_ms.items()}
    if not step_ms:
        step_ms = [wall / K_steps * 1e3]
    step_ms_sorted = sorted(step_ms)
    med_step = step_ms_sorted[len(step_ms) // 2]
    S_mid = cfg.S0 + 1 + (K_steps // L) // 2
    ab = algorithmic_bytes(cfg, S_mid)
    attn_bytes = ab["rows"] + ab["q_out"]
    dom = "attn"
    attn_ms = mean["attn"] if mean["attn"] else float("nan")
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    step_bytes = ab["labels"] + ab["rows"] + ab["q_out"]
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K_steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.D, "k_cols": cfg.d_k, "prefill": cfg.S0, "r": cfg.r,
                   "k": cfg.k, "labels": ("int4" if cfg.int4 else "fp16") if cfg.k > 0 else None,
                   "storage": "fp16 q/K/V", "layer_caches": L, "note": cfg.note},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "algorithmic_bytes_per_launch": attn_bytes,
                     "avg_launch_us": round(attn_ms * 1e3, 3), "events": args.stage_events},
        "step": {"median_us": round(med_step * 1e3, 3),
                 "p90_us": round(step_ms_sorted[int(0.9 * (len(step_ms) - 1))] * 1e3, 3),
                 "stage_mean_us": {k: (round(v * 1e3, 3) if v is not None else None)
                                   for k, v in mean.items()},
                 "algorithmic_bytes": step_bytes,
                 "hbm_gbs_at_median": round(step_bytes / (med_step * 1e-3) / 1e9, 1),
                 "hbm_frac_at_median": round(step_bytes / (med_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "hbm_gbs_wall": round(step_bytes * K_steps / wall / 1e9, 1)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    events.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
