"""Parity helpers: run the HIP path through the C ABI and the CPU oracle on
the same seeded bytes, and compare them.

Comparison rules:
* label cache (fp16 labels, int4 codes and scales): bit-exact;
* top-k sets: the HIP set and the oracle set may differ only in tokens whose
  oracle score lies within 1e-3 * |s_k| + 1e-6 * max|s| of the oracle's k-th
  score s_k (the two sides rank fp32 and fp64 scores);
* attention output: max |gpu - ref| / max |ref| per (batch, query head) row
  <= 2e-3 (fp32 accumulation of fp16 data, fp16 output); when the sets differ
  the reference is the oracle's attention over the HIP set, so the check
  isolates the arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

ATTN_TOL = 2e-3
TOPK_REL = 1e-3
TOPK_ABS = 1e-6


def rel_err_rows(got, ref):
    """max_i |got - ref| / max_i |ref| over the last axis; rows with ref == 0
    must be exactly zero (returned as 0 or inf)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max(-1)
    num = np.abs(got - ref).max(-1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num == 0, 0.0, np.inf))
    return out


def topk_set_ok(gpu_set, ora_set, scores, k):
    """Sets may differ only in near-ties of the k-th oracle score."""
    g = set(int(x) for x in gpu_set if x >= 0)
    o = set(int(x) for x in ora_set if x >= 0)
    if g == o:
        return True, 0
    if len(g) != len(o):
        return False, -1
    s = np.asarray(scores, np.float64)
    sk = np.sort(s)[::-1][min(k, len(s)) - 1]
    band = TOPK_REL * abs(sk) + TOPK_ABS * np.abs(s).max()
    diff = g.symmetric_difference(o)
    ok = all(abs(s[t] - sk) <= band for t in diff)
    return ok, len(diff)


def sub_problem(cfg, q, K, V, chan, keep, b, g):
    """Host copies of one (batch, KV head) row as a B=1, H_kv=1 problem."""
    G = cfg.G
    qs = q[b, g * G:(g + 1) * G][None].cpu().numpy()
    Ks = K[b, g][None, None].cpu().numpy()
    Vs = V[b, g][None, None].cpu().numpy()
    cs = chan[g][None].cpu().numpy() if chan is not None else None
    ks = keep[g][None].cpu().numpy() if keep is not None else None
    return qs, Ks, Vs, cs, ks


def check_rows(cfg, q, K, V, chan, keep, labels, seq_lens, k, out, topk, rows,
               label_upto=None, strict_sets=False):
    """Compare the HIP results of `rows` with the oracle.  Returns a dict of
    the worst attention error and the set differences seen."""
    worst = 0.0
    n_diff = 0
    seq = seq_lens.cpu().numpy()
    lab_np = None
    if labels is not None:
        lab_np = {"codes": labels.codes.cpu().numpy()}
        if labels.scales is not None:
            lab_np["scales"] = labels.scales.cpu().numpy().view(np.uint16)
    out_np = out.float().cpu().numpy()
    tk_np = topk.cpu().numpy() if topk is not None else None
    for (b, g) in rows:
        S = int(seq[b])
        qs, Ks, Vs, cs, ks = sub_problem(cfg, q, K, V, chan, keep, b, g)
        lab = None
        if k > 0:
            upto = S if label_upto is None else label_upto
            lab = oracle.Labels.empty(1, 1, labels.slots, cfg.r, cfg.int4)
            oracle.label_build(Ks, cs, lab, 0, upto)
            # label cache: bit-exact over the slots in use
            if cfg.int4:
                assert np.array_equal(lab.codes[0, 0, :upto], lab_np["codes"][b, g, :upto]), (b, g)
                assert np.array_equal(lab.scales[0, 0, :upto], lab_np["scales"][b, g, :upto]), (b, g)
            else:
                gl = lab_np["codes"][b, g, :upto].view(np.uint16)
                assert np.array_equal(lab.f16[0, 0, :upto], gl), (b, g)
        res = oracle.decode(qs, Ks, Vs, np.array([S], np.int32), k, cfg.sm_scale, chan=cs,
                            lab=lab, keep=ks, want_scores=k > 0)
        ref = res["out"][0]
        got = out_np[b, g * cfg.G:(g + 1) * cfg.G]
        if k > 0 and tk_np is not None:
            gset = tk_np[b, g]
            oset = res["topk"][0, 0]
            assert np.all(np.diff(gset[gset >= 0]) > 0), "topk not ascending"
            assert np.all(gset[min(k, S):] == -1), "topk padding"
            if S > k:
                ok, nd = topk_set_ok(gset, oset, res["scores"][0, 0, :S], k)
                assert ok, ("topk set", b, g, nd)
                if strict_sets:
                    assert nd == 0, ("topk set differs", b, g, nd)
                if nd:
                    n_diff += nd
                    sets = np.full((1, 1, len(gset)), -1, np.int32)
                    sets[0, 0] = gset
                    ref = oracle.attend_sets(qs, Ks, Vs, sets, cfg.sm_scale, keep=ks)[0]
            else:
                assert np.array_equal(gset[:S], np.arange(S)), "dense fallback set"
        e = rel_err_rows(got, ref).max()
        assert e <= ATTN_TOL, ("attention error", b, g, float(e))
        worst = max(worst, float(e))
    return {"worst_rel_err": worst, "topk_diff_tokens": n_diff}


def sample_rows(cfg, n, seed=0):
    rng = np.random.default_rng(seed)
    allr = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    if n >= len(allr):
        return allr
    pick = rng.choice(len(allr), n, replace=False)
    return [allr[i] for i in sorted(pick)]
