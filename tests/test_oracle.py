"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: numpy's IEEE binary16
conversions, hand-worked fixtures, closed forms, brute force on tiny inputs,
and the textbook softmax attention of ``torch.nn.functional.
scaled_dot_product_attention`` (fp64, CPU) in the cases where the method
reduces to it.  Pages are cited by title and section:

* "Double Sparsity" article (joto.ai blog archive 2025060420469), sections
  "offline calibration" and "online forward computation";
* LeanK article (aitangshan.cn news 1293675), section 2.2;
* grouped-query attention article (trdm.cn news 80600), section 4.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(a):
    return np.asarray(a, dtype=np.float16)


def bits(a):
    return f16(a).view(np.uint16)


def sdpa(q, K, V, scale, mask=None):
    """Textbook softmax attention, fp64 on CPU.  q [B][Hq][D], K/V [B][Hq][S][*]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    kt = torch.from_numpy(np.asarray(K, np.float64))
    vt = torch.from_numpy(np.asarray(V, np.float64))
    m = None if mask is None else torch.from_numpy(mask)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[:, :, 0, :].numpy()


def rand_f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


# --------------------------------------------------------------------------
# binary16 conversions against numpy's IEEE implementation
# --------------------------------------------------------------------------

def test_half_to_double_all_patterns():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    lib = oracle._load()
    got = np.array([lib.oracle_half_to_double(int(b)) for b in allbits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_float_to_half_rn_matches_numpy():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 5, 4000),
        np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0], np.float32),
        # every halfway point between adjacent fp16 values in [1, 2)
        (1.0 + (np.arange(1024) + 0.5) / 1024.0).astype(np.float32),
    ]).astype(np.float32)
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half_rn(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# label cache ("offline calibration": heavy-channel K values copied into a
# contiguous cache at prefill, only the new token appended at decode)
# --------------------------------------------------------------------------

def test_f16_label_is_the_k_columns():
    """Every K element gets a unique bit pattern that encodes (b, g, t, c); each
    label entry must decode back to (b, g, t, chan[g][j])."""
    B, H, cap, D, r = 2, 3, 5, 128, 7
    code = np.arange(B * H * cap * D, dtype=np.int64).reshape(B, H, cap, D)
    K = (code + 0x0400).astype(np.uint16)          # all normal, finite fp16 patterns
    rng = np.random.default_rng(3)
    chan = np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(H)]).astype(np.int32)
    lab = oracle.Labels.empty(B, H, cap + 3, r, False)
    oracle.label_build(K, chan, lab, 0, cap)
    dec = lab.f16[:, :, :cap, :].astype(np.int64) - 0x0400
    b, g, t, j = np.meshgrid(np.arange(B), np.arange(H), np.arange(cap), np.arange(r), indexing="ij")
    expect = ((b * H + g) * cap + t) * D + chan[g, j]
    assert np.array_equal(dec, expect)
    assert not lab.f16[:, :, cap:, :].any()        # slots past the range untouched


def _golden_int4():
    with open(os.path.join(GOLDEN, "int4_label_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_int4(), ids=lambda c: c["id"])
def test_int4_label_golden(case):
    if "x" in case:
        krow = np.zeros(128, np.float16)
        krow[: len(case["x"])] = case["x"]
        chan = np.arange(len(case["x"]), dtype=np.int32)
    else:
        krow = np.zeros(128, np.float16)
        for c, v in case["krow_sparse"].items():
            krow[int(c)] = v
        chan = np.array(case["chan"], np.int32)
    codes, scale = oracle.label_int4_row(krow.view(np.uint16), chan)
    assert scale == case["scale_bits"]
    assert codes.tolist() == case["bytes"]


def _unpack(codes):
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    c = np.stack([lo, hi], -1).reshape(*codes.shape[:-1], -1)
    return np.where(c >= 8, c - 16, c)


def test_int4_label_invariants():
    rng = np.random.default_rng(5)
    B, H, cap, D, r = 2, 4, 64, 128, 16
    K = rand_f16(rng, (B, H, cap, D), 3.0)
    K[0, 0, 3, :] = 0                                  # all-zero token
    chan = np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(H)]).astype(np.int32)
    lab = oracle.Labels.empty(B, H, cap, r, True)
    oracle.label_build(K.view(np.uint16), chan, lab, 0, cap)
    c = _unpack(lab.codes)
    sf = lab.scales.view(np.float16).astype(np.float32)
    x = np.take_along_axis(K.astype(np.float32), chan[None, :, None, :].repeat(B, 0).repeat(cap, 2), 3)
    amax = np.abs(x).max(-1)
    # scale is fp16(amax / 7) with IEEE fp32 division (numpy as the independent reference)
    assert np.array_equal(lab.scales, (amax / np.float32(7)).astype(np.float16).view(np.uint16))
    assert c.min() >= -7 and c.max() <= 7
    nz = sf > 0
    # the absmax channel gets +-7
    arg = np.abs(x).argmax(-1)
    top = np.take_along_axis(c, arg[..., None], -1)[..., 0]
    assert np.all(np.abs(top[nz]) == 7)
    # reconstruction error within half a step where unclamped
    err = np.abs(x - c * sf[..., None])
    assert np.all(err[nz] <= sf[nz][..., None] / 2 + 1e-7 * np.abs(x[nz]))
    assert not c[~nz].any()
    assert not nz[0, 0, 3]


@pytest.mark.parametrize("is_int4", [False, True])
def test_append_equals_build(is_int4):
    """build [0, S+n) == build [0, S) followed by n appends, bit for bit."""
    rng = np.random.default_rng(11)
    B, H, cap, D, r, S = 3, 2, 40, 128, 8, 33
    K = rand_f16(rng, (B, H, cap, D)).view(np.uint16)
    chan = np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(H)]).astype(np.int32)
    full = oracle.label_build(K, chan, oracle.Labels.empty(B, H, cap, r, is_int4), 0, cap)
    inc = oracle.label_build(K, chan, oracle.Labels.empty(B, H, cap, r, is_int4), 0, S)
    for t in range(S, cap):
        oracle.label_append(K, chan, inc, np.full(B, t, np.int32))
    for a in ("f16", "codes", "scales"):
        x, y = getattr(full, a), getattr(inc, a)
        assert (x is None and y is None) or np.array_equal(x, y)


def test_append_skips_out_of_range_rows():
    rng = np.random.default_rng(12)
    B, H, cap, D, r = 3, 2, 10, 128, 4
    K = rand_f16(rng, (B, H, cap, D)).view(np.uint16)
    chan = np.tile(np.arange(r, dtype=np.int32), (H, 1))
    lab = oracle.Labels.empty(B, H, cap, r, False)
    oracle.label_append(K, chan, lab, np.array([-1, 4, cap], np.int32))
    assert not lab.f16[0].any() and not lab.f16[2].any()
    assert np.array_equal(lab.f16[1, :, 4], K[1, :, 4, :r])
    assert not np.delete(lab.f16[1], 4, axis=1).any()


# --------------------------------------------------------------------------
# top-k ("online forward computation", step 3): k largest approximate scores,
# ties to the lower token index (reading), k <= 0 or k >= S -> all tokens
# --------------------------------------------------------------------------

def _is_topk_set(s, T, k):
    """T is the top-k under the order (score desc, index asc) iff every member
    beats every non-member."""
    inside = set(T)
    out = [u for u in range(len(s)) if u not in inside]
    return len(T) == k and all((s[t] > s[u]) or (s[t] == s[u] and t < u) for t in T for u in out)


def test_topk_brute_force_tiny():
    rng = np.random.default_rng(13)
    for trial in range(200):
        S = int(rng.integers(1, 9))
        k = int(rng.integers(1, S + 1))
        s = rng.integers(-3, 4, S).astype(np.float64)     # many ties
        if trial % 3 == 0:
            s = rng.standard_normal(S)
        sets = [c for c in itertools.combinations(range(S), k) if _is_topk_set(s, c, k)]
        assert len(sets) == 1                                # the order makes it unique
        got = oracle.topk(s, k)
        assert got.tolist() == sorted(sets[0])


def test_topk_matches_lexsort_and_edges():
    rng = np.random.default_rng(14)
    s = np.round(rng.standard_normal(5000), 2)               # ties
    for k in (1, 7, 256, 4999):
        ref = np.sort(np.lexsort((np.arange(len(s)), -s))[:k])
        assert np.array_equal(oracle.topk(s, k), ref)
    assert oracle.topk(np.zeros(50), 10).tolist() == list(range(10))   # all equal
    assert oracle.topk(s[:40], 40).tolist() == list(range(40))         # k == S
    assert oracle.topk(s[:40], 99).tolist() == list(range(40))         # k > S
    assert oracle.topk(s[:40], 0).tolist() == list(range(40))          # dense
    assert oracle.topk(np.array([0.0, -0.0, 0.0]), 2).tolist() == [0, 1]


# --------------------------------------------------------------------------
# scores ("online forward computation", steps 1-2)
# --------------------------------------------------------------------------

def _tensors(rng, B, Hq, Hkv, S, D=128, dk=128, dv=128):
    q = rand_f16(rng, (B, Hq, D))
    K = rand_f16(rng, (B, Hkv, S, dk))
    V = rand_f16(rng, (B, Hkv, S, dv))
    return q, K, V


def test_scores_full_channels_are_the_exact_logits():
    """r = D with the identity table and fp16 labels: the approximate score is the
    exact q.K dot product (summed over the group's query heads)."""
    rng = np.random.default_rng(15)
    B, Hq, Hkv, S, D = 2, 4, 2, 50, 128
    q, K, V = _tensors(rng, B, Hq, Hkv, S)
    chan = np.tile(np.arange(D, dtype=np.int32), (Hkv, 1))
    lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, Hkv, S, D, False), 0, S)
    res = oracle.decode(q, K, V, np.full(B, S, np.int32), 5, 0.1, chan=chan, lab=lab,
                        want_scores=True)
    G = Hq // Hkv
    qs = q.astype(np.float64).reshape(B, Hkv, G, D).sum(2)
    ref = np.einsum("bgd,bgtd->bgt", qs, K.astype(np.float64))
    np.testing.assert_allclose(res["scores"], ref, rtol=1e-12, atol=1e-12)


def test_int4_scores_exact_when_labels_are_integers():
    """Heavy-channel values that are integers in [-7, 7] with one +-7 per token
    quantise exactly (scale 1), so the score is the exact dot product."""
    rng = np.random.default_rng(16)
    B, H, S, D, r = 1, 3, 40, 128, 8
    q = rand_f16(rng, (B, H, D))
    K = rand_f16(rng, (B, H, S, D))
    chan = np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(H)]).astype(np.int32)
    ints = rng.integers(-7, 8, (B, H, S, r))
    ints[..., 0] = np.where(rng.random((B, H, S)) < 0.5, 7, -7)
    for g in range(H):
        K[:, g][..., chan[g]] = ints[:, g].astype(np.float16)
    lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, H, S, r, True), 0, S)
    assert np.all(lab.scales == 0x3C00)
    res = oracle.decode(q, K, K, np.full(B, S, np.int32), 3, 0.1, chan=chan, lab=lab,
                        want_scores=True)
    qg = np.stack([q[0, g, chan[g]].astype(np.float64) for g in range(H)])
    ref = np.einsum("gj,gtj->gt", qg, ints[0].astype(np.float64))
    np.testing.assert_allclose(res["scores"][0], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# whole path against textbook attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2), (7, 1)])
def test_dense_reduction(Hq, Hkv):
    """r = D and k = S: Double Sparsity is plain softmax attention."""
    rng = np.random.default_rng(17)
    B, S, D = 2, 37, 128
    q, K, V = _tensors(rng, B, Hq, Hkv, S)
    chan = np.tile(np.arange(D, dtype=np.int32), (Hkv, 1))
    lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, Hkv, S, D, False), 0, S)
    G = Hq // Hkv
    ref = sdpa(q, np.repeat(K, G, 1), np.repeat(V, G, 1), 0.088)
    for k in (S, S + 5, 0, -1):
        res = oracle.decode(q, K, V, np.full(B, S, np.int32), k, 0.088, chan=chan if k > 0 else None,
                            lab=lab if k > 0 else None)
        np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(3, 3), (8, 2)])
def test_exact_topk_attention(Hq, Hkv):
    """r = D, k < S: attention over the k tokens with the largest exact group
    logits (brute-forced with lexsort), i.e. masked textbook attention."""
    rng = np.random.default_rng(18)
    B, S, D, k = 2, 60, 128, 9
    q, K, V = _tensors(rng, B, Hq, Hkv, S)
    chan = np.tile(np.arange(D, dtype=np.int32), (Hkv, 1))
    lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, Hkv, S, D, False), 0, S)
    G = Hq // Hkv
    res = oracle.decode(q, K, V, np.full(B, S, np.int32), k, 0.1, chan=chan, lab=lab)
    qs = q.astype(np.float64).reshape(B, Hkv, G, D).sum(2)
    s = np.einsum("bgd,bgtd->bgt", qs, K.astype(np.float64))
    mask = np.zeros((B, Hkv, S), bool)
    for b in range(B):
        for g in range(Hkv):
            sel = np.lexsort((np.arange(S), -s[b, g]))[:k]
            mask[b, g, sel] = True
            assert res["topk"][b, g].tolist() == sorted(sel.tolist())
    ref = sdpa(q, np.repeat(K, G, 1), np.repeat(V, G, 1), 0.1, mask=np.repeat(mask, G, 1))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_gqa_identical_heads_equal_mha():
    """G identical query heads select the same tokens as MHA with that query and
    give its output on each head (query head h uses KV head h // G)."""
    rng = np.random.default_rng(19)
    B, Hkv, G, S, D, r, k = 2, 3, 4, 80, 128, 8, 11
    qm, K, V = _tensors(rng, B, Hkv, Hkv, S)
    chan = np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    for is_int4 in (False, True):
        lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, Hkv, S, r, is_int4), 0, S)
        mha = oracle.decode(qm, K, V, np.full(B, S, np.int32), k, 0.09, chan=chan, lab=lab)
        qg = np.repeat(qm, G, 1)
        gqa = oracle.decode(qg, K, V, np.full(B, S, np.int32), k, 0.09, chan=chan, lab=lab)
        assert np.array_equal(mha["topk"], gqa["topk"])
        np.testing.assert_allclose(gqa["out"], np.repeat(mha["out"], G, 1), rtol=1e-13, atol=1e-13)


def test_leank_pruned_k_is_masked_dense_attention():
    """LeanK (section 2.2): attention over a static subset of K columns equals
    dense attention with the query zeroed outside the kept channels."""
    rng = np.random.default_rng(20)
    B, Hq, Hkv, S, D, dk = 2, 6, 2, 45, 128, 32
    q, Kfull, V = _tensors(rng, B, Hq, Hkv, S)
    keep = np.stack([np.sort(rng.choice(D, dk, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    Kc = np.stack([Kfull[:, g][..., keep[g]] for g in range(Hkv)], 1)
    G = Hq // Hkv
    qz = np.zeros_like(q)
    for h in range(Hq):
        qz[:, h, keep[h // G]] = q[:, h, keep[h // G]]
    ref = sdpa(qz, np.repeat(Kfull, G, 1), np.repeat(V, G, 1), 0.088)
    res = oracle.decode(q, Kc, V, np.full(B, S, np.int32), 0, 0.088, keep=keep)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)
    # keep = all columns in order is the unpruned path
    ident = np.tile(np.arange(D, dtype=np.int32), (Hkv, 1))
    a = oracle.decode(q, Kfull, V, np.full(B, S, np.int32), 0, 0.088, keep=ident)["out"]
    b = oracle.decode(q, Kfull, V, np.full(B, S, np.int32), 0, 0.088)["out"]
    np.testing.assert_array_equal(a, b)


def test_leank_with_labels_on_compacted_columns():
    """Heavy channels index the compacted K columns; the gathered query reads
    q at keep[chan[j]]."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, S, D, dk, r, k = 1, 4, 2, 70, 128, 32, 32, 6
    q, Kfull, V = _tensors(rng, B, Hq, Hkv, S)
    keep = np.stack([np.sort(rng.choice(D, dk, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    Kc = np.ascontiguousarray(np.stack([Kfull[:, g][..., keep[g]] for g in range(Hkv)], 1))
    chan = np.tile(np.arange(dk, dtype=np.int32), (Hkv, 1))   # all kept columns
    lab = oracle.label_build(Kc.view(np.uint16), chan, oracle.Labels.empty(B, Hkv, S, r, False), 0, S)
    res = oracle.decode(q, Kc, V, np.full(B, S, np.int32), k, 0.1, chan=chan, lab=lab,
                        keep=keep, want_scores=True)
    G = Hq // Hkv
    for g in range(Hkv):
        qs = q[0, g * G:(g + 1) * G][:, keep[g]].astype(np.float64).sum(0)
        np.testing.assert_allclose(res["scores"][0, g], Kc[0, g].astype(np.float64) @ qs,
                                   rtol=1e-12, atol=1e-12)


def test_degenerate_rows():
    rng = np.random.default_rng(22)
    B, H, S, D = 3, 2, 10, 128
    q, K, V = _tensors(rng, B, H, H, S)
    chan = np.tile(np.arange(16, dtype=np.int32), (H, 1))
    lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, H, S, 16, False), 0, S)
    res = oracle.decode(q, K, V, np.array([0, 1, S], np.int32), 1, 0.1, chan=chan, lab=lab,
                        want_scores=True)
    assert not res["out"][0].any()                                    # empty row -> zeros
    np.testing.assert_array_equal(res["out"][1], V[1, :, 0].astype(np.float64))   # one token
    best = res["scores"][2].argmax(-1)                                 # k = 1 -> argmax row
    for g in range(H):
        assert res["topk"][2, g, 0] == best[g]
        np.testing.assert_array_equal(res["out"][2, g], V[2, g, best[g]].astype(np.float64))


def test_synth_config_inputs_are_consistent():
    """The workload tables: heavy channels include the outlier channels, LeanK
    keep tables contain them, shapes are as declared."""
    for name, cfg in synth.CONFIGS.items():
        ht = synth.heavy_table(cfg) if cfg.r > 0 else None
        kt = synth.keep_table(cfg)
        for g in range(cfg.Hkv):
            out = synth.outlier_channels(cfg, g)
            assert len(set(out)) == cfg.n_outlier
            if kt is not None:
                assert len(kt[g]) == cfg.d_k and set(out) <= set(kt[g]) and kt[g] == sorted(kt[g])
            if ht is not None:
                assert len(ht[g]) == cfg.r == len(set(ht[g])) and ht[g] == sorted(ht[g])
                cols = [kt[g][c] for c in ht[g]] if kt is not None else ht[g]
                assert set(out[: cfg.r]) <= set(cols)


def _golden_int4_scores():
    with open(os.path.join(GOLDEN, "int4_score_cases.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("G", [1, 2])
def test_int4_scores_with_per_token_scales_golden(G):
    """Hand-worked int4 scores ("online forward computation", step 2, on the
    4-bit labels of "offline calibration"): tokens whose scales differ and are
    not 1, so dropping the scale, or taking another token's, changes the
    scores and the top-k set.  Values in non-heavy channels of K and q are
    large distractors that must not enter the labels or the gathered query.
    G = 2 splits the gathered query evenly over two query heads of a group."""
    gd = _golden_int4_scores()
    chan = np.array(gd["chan"], np.int32)
    qg = np.array(gd["qg"], np.float64)
    toks = gd["tokens"]
    S, D, r = len(toks), 128, len(chan)
    K = np.full((1, 1, S, D), gd["distractor_k"], np.float16)
    K[0, 0][:, chan] = np.array([t["x"] for t in toks], np.float16)
    q = np.full((1, G, D), gd["distractor_q"], np.float16)
    q[0][:, chan] = (qg / G).astype(np.float16)[None, :].repeat(G, 0)
    assert np.array_equal(q[0][:, chan].astype(np.float64).sum(0), qg)   # exact split
    lab = oracle.label_build(K.view(np.uint16), chan[None], oracle.Labels.empty(1, 1, S, r, True),
                             0, S)
    assert lab.scales[0, 0].tolist() == [t["scale_bits"] for t in toks]
    assert lab.codes[0, 0].tolist() == [t["bytes"] for t in toks]
    V = np.zeros((1, 1, S, D), np.float16)
    for k_str, expect in gd["topk"].items():
        res = oracle.decode(q, K, V, np.array([S], np.int32), int(k_str), 0.1, chan=chan[None],
                            lab=lab, want_scores=True)
        assert res["scores"][0, 0, :S].tolist() == [t["score"] for t in toks]
        assert res["topk"][0, 0].tolist() == expect


# --------------------------------------------------------------------------
# attention over a caller-given token set ("online forward computation",
# step 3: exact softmax attention over the selected tokens' full rows), the
# reference the parity checks fall back to when two selections differ in
# near-ties
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,leank", [(4, 4, False), (6, 2, False), (8, 2, True)])
def test_attend_sets_is_masked_attention(Hq, Hkv, leank):
    """attend_sets over sets padded with -1 and holding out-of-range entries
    (>= capacity, which are ignored) equals textbook attention masked to the
    valid entries; an all-padding set gives zeros.  Under LeanK the pruned K
    is the full K with the query zeroed outside the kept channels."""
    rng = np.random.default_rng(23)
    B, S, D, dk, k_cap = 3, 41, 128, 32, 12
    G = Hq // Hkv
    q, Kfull, V = _tensors(rng, B, Hq, Hkv, S)
    keep = None
    K = Kfull
    qref = q
    if leank:
        keep = np.stack([np.sort(rng.choice(D, dk, replace=False)) for _ in range(Hkv)]).astype(np.int32)
        K = np.ascontiguousarray(np.stack([Kfull[:, g][..., keep[g]] for g in range(Hkv)], 1))
        qref = np.zeros_like(q)
        for h in range(Hq):
            qref[:, h, keep[h // G]] = q[:, h, keep[h // G]]
    sets = np.full((B, Hkv, k_cap), -1, np.int32)
    mask = np.zeros((B, Hkv, S), bool)
    for b in range(B):
        for g in range(Hkv):
            if (b, g) == (B - 1, Hkv - 1):
                continue                                   # all padding
            n = int(rng.integers(1, k_cap - 2))
            sel = rng.choice(S, n, replace=False)
            mask[b, g, sel] = True
            row = np.concatenate([sel, [S + 3, 10 ** 6, -5]]).astype(np.int32)  # junk entries
            rng.shuffle(row)
            sets[b, g, :len(row)] = row
    got = oracle.attend_sets(q, K, V, sets, 0.09, keep=keep)
    m = np.repeat(mask, G, 1)
    ref = sdpa(qref, np.repeat(Kfull, G, 1), np.repeat(V, G, 1), 0.09,
               mask=np.where(m.any(-1, keepdims=True), m, True))
    live = m.any(-1)
    np.testing.assert_allclose(got[live], ref[live], rtol=1e-12, atol=1e-12)
    assert not got[~live].any()
    assert (~live).sum() == G


def test_attend_sets_agrees_with_decode_on_its_own_selection():
    """Fed the oracle's own top-k sets, attend_sets reproduces the decode
    output exactly (same summation)."""
    rng = np.random.default_rng(24)
    B, Hq, Hkv, S, D, r, k = 2, 6, 3, 90, 128, 8, 13
    q, K, V = _tensors(rng, B, Hq, Hkv, S)
    chan = np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    lab = oracle.label_build(K.view(np.uint16), chan, oracle.Labels.empty(B, Hkv, S, r, True), 0, S)
    res = oracle.decode(q, K, V, np.full(B, S, np.int32), k, 0.1, chan=chan, lab=lab)
    got = oracle.attend_sets(q, K, V, res["topk"], 0.1)
    np.testing.assert_array_equal(got, res["out"])


# --------------------------------------------------------------------------
# paged token pool ("use in SGLang": K/V slots pooled across sequences)
# --------------------------------------------------------------------------

def test_gather_pages_inverts_a_page_scatter():
    """A contiguous cache scattered into a pool page by page under a random
    page assignment (written out here slot by slot) is gathered back
    unchanged, and decoding from the gathered cache is decoding the original;
    unused table entries (-1) give zero rows."""
    rng = np.random.default_rng(25)
    B, H, P, max_pages, D = 3, 2, 16, 5, 128
    cap = P * max_pages
    K = rand_f16(rng, (B, H, cap, D))
    n_pages = B * max_pages + 4
    perm = rng.permutation(n_pages)[:B * max_pages].reshape(B, max_pages)
    pool = np.zeros((n_pages, H, P, D), np.float16)
    for b in range(B):
        for t in range(cap):
            pool[perm[b, t // P], :, t % P, :] = K[b, :, t, :]
    back = oracle.gather_pages(pool, perm, P)
    assert np.array_equal(back, K)
    table = perm.copy()
    table[1, 3:] = -1
    part = oracle.gather_pages(pool, table, P)
    assert np.array_equal(part[1, :, :3 * P], K[1, :, :3 * P]) and not part[1, :, 3 * P:].any()
    q = rand_f16(rng, (B, H, D))
    ref = oracle.decode(q, K, K, np.full(B, cap, np.int32), 0, 0.1)["out"]
    got = oracle.decode(q, back, back, np.full(B, cap, np.int32), 0, 0.1)["out"]
    np.testing.assert_array_equal(got, ref)
