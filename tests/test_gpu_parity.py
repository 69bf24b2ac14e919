"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Needs an MI355X and the built libds.so."""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import ds_check

pytestmark = pytest.mark.gpu

ds = pytest.importorskip("sparse_attention_decode_ds_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ds.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _note(msg):
    print(msg, flush=True)


def prefill(cfg, inp, upto):
    labels = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
    ds.label_build(inp.K, inp.chan, labels, 0, upto)
    return labels


def run(cfg, inp, labels, seq_lens, max_seq, k=None, want_idx=True, **kw):
    k = cfg.k if k is None else k
    topk = None
    if k > 0 and want_idx:
        topk = torch.full((cfg.B, cfg.Hkv, k), -7, dtype=torch.int32, device="cuda")
    kw.setdefault("validate_tables", True)
    out = ds.decode_attn(inp.q, inp.K, inp.V, seq_lens, max_seq, k, cfg.sm_scale, chan=inp.chan,
                         labels=labels if k > 0 else None, keep=inp.keep, topk_idx=topk, **kw)
    torch.cuda.synchronize()
    return out, topk


# ---------------------------------------------------------------------------
# label cache
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("r,int4", [(8, True), (16, True), (6, True), (16, False), (8, False),
                                    (5, False), (128, False), (64, True)])
def test_label_build_and_append_bitexact(r, int4):
    cfg = synth.small("lab", B=3, Hq=4, Hkv=4, S0=197, steps=5, r=r, int4=int4, seed=31)
    _note("label r=%d int4=%d" % (r, int4))
    # strided K: the cache lives inside a larger buffer (token stride 136 elements)
    big = synth.normal_tensor((cfg.B, cfg.Hkv, cfg.cap, 136), 5, 2, "cuda")
    K = big[..., :128]
    chan = torch.tensor([sorted(np.random.default_rng(g).choice(128, r, replace=False))
                         for g in range(cfg.Hkv)], dtype=torch.int32, device="cuda")
    labels = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, r, int4)
    ds.label_build(K, chan, labels, 0, 61)
    ds.label_build(K, chan, labels, 61, cfg.S0)
    for t in range(cfg.S0, cfg.cap):
        pos = torch.tensor([t, t if t % 2 else -1, cfg.cap + 3], dtype=torch.int32, device="cuda")
        ds.label_append(K, chan, labels, pos)
    torch.cuda.synchronize()
    Kh = K.cpu().numpy()
    ref = oracle.Labels.empty(cfg.B, cfg.Hkv, labels.slots, r, int4)
    oracle.label_build(Kh, chan.cpu().numpy(), ref, 0, cfg.S0)
    for t in range(cfg.S0, cfg.cap):
        oracle.label_append(Kh, chan.cpu().numpy(), ref,
                            np.array([t, t if t % 2 else -1, cfg.cap + 3], np.int32))
    if int4:
        assert np.array_equal(labels.codes.cpu().numpy(), ref.codes)
        assert np.array_equal(labels.scales.cpu().numpy().view(np.uint16), ref.scales)
    else:
        assert np.array_equal(labels.codes.cpu().numpy().view(np.uint16), ref.f16)


def test_label_int4_golden_rows():
    """The hand-worked int4 rows through the HIP label kernel."""
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "int4_label_cases.json")))["cases"]
    cases = [c for c in cases if "x" in c]
    K = torch.zeros((1, 1, len(cases), 128), dtype=torch.float16)
    for i, c in enumerate(cases):
        K[0, 0, i, :8] = torch.tensor(c["x"], dtype=torch.float16)
    K = K.cuda()
    chan = torch.arange(8, dtype=torch.int32, device="cuda")[None]
    labels = ds.LabelCache.allocate(1, 1, len(cases), 8, True)
    ds.label_build(K, chan, labels, 0, len(cases))
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        assert labels.codes[0, 0, i].cpu().tolist() == c["bytes"], c["id"]
        assert int(labels.scales[0, 0, i].cpu().view(torch.int16).item()) & 0xFFFF == c["scale_bits"]


# ---------------------------------------------------------------------------
# decode step, small shapes (several tiles and ragged tails)
# ---------------------------------------------------------------------------

SMALL = {
    "mha_f16_r16": dict(B=2, Hq=4, Hkv=4, S0=700, r=16, k=48, int4=False),
    "mha_int4_r8": dict(B=3, Hq=4, Hkv=4, S0=1300, r=8, k=100, int4=True),
    "gqa7_f16_r16": dict(B=2, Hq=28, Hkv=4, S0=900, r=16, k=64, int4=False),
    "gqa4_int4_r8": dict(B=2, Hq=16, Hkv=4, S0=513, r=8, k=33, int4=True),
    "gqa2_int4_r16": dict(B=2, Hq=4, Hkv=2, S0=450, r=16, k=40, int4=True),
    "generic_f16_r12": dict(B=2, Hq=6, Hkv=3, S0=333, r=12, k=20, int4=False),
    "generic_int4_r6": dict(B=2, Hq=3, Hkv=3, S0=270, r=6, k=25, int4=True),
    "leank_dense": dict(B=2, Hq=28, Hkv=4, S0=650, r=0, k=0, int4=False, d_k=32),
    "leank_ds": dict(B=2, Hq=28, Hkv=4, S0=650, r=8, k=70, int4=False, d_k=32),
    "leank48_ds": dict(B=2, Hq=8, Hkv=2, S0=400, r=8, k=50, int4=True, d_k=48),
    "g8_dense": dict(B=1, Hq=16, Hkv=2, S0=300, r=0, k=0, int4=False),
}


def check_without_idx(cfg, inp, labels, seq, max_seq, out_idx, rows, **kw):
    """The same decode without the selected-set output (the path that does
    not order the set): every row's output matches the run that returned
    the set, and the sampled rows match the oracle."""
    out, _ = run(cfg, inp, labels, seq, max_seq, want_idx=False, **kw)
    a = out.float()
    b = out_idx.float()
    den = b.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    diff = ((a - b).abs() / den).max().item()
    assert diff <= 1e-3, ("output without the set output", diff)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        None, rows)


def _small_inputs(name, **over):
    kw = dict(SMALL[name])
    kw.update(over)
    cfg = synth.small(name, steps=3, seed=100 + len(name), **kw)
    inp = synth.make_inputs(cfg, "cuda")
    return cfg, inp


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("mode", ["default", "unfused", "stream", "split3", "append_flag"])
def test_decode_small(name, mode):
    cfg, inp = _small_inputs(name)
    _note("decode %s %s" % (name, mode))
    S = cfg.S0 + 1
    labels = None
    kw = {}
    if cfg.k > 0:
        labels = prefill(cfg, inp, cfg.S0 if mode == "append_flag" else S)
        if mode == "append_flag":
            kw["flags"] = ds.DECODE_APPEND
    elif mode == "append_flag":
        pytest.skip("dense: no labels")
    if mode == "unfused":
        kw["flags"] = ds.DECODE_UNFUSED
    if mode == "stream":
        kw["flags"] = ds.DECODE_STREAM
    if mode == "split3":
        kw["n_split"] = 3
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    out, topk = run(cfg, inp, labels, seq, S, **kw)
    rows = ds_check.sample_rows(cfg, 64)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, rows)


@pytest.mark.parametrize("unfused", [False, True])
def test_ragged_lengths_and_degenerate_rows(unfused):
    """Per-row lengths: empty, one token, below/at/just above k, full."""
    cfg, inp = _small_inputs("mha_int4_r8", B=7)
    k = cfg.k
    lens = [0, 1, k - 1, k, k + 1, cfg.S0 // 2 + 3, cfg.S0 + 1]
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0 + 1)
    out, topk = run(cfg, inp, labels, seq, cfg.S0 + 1,
                    flags=ds.DECODE_UNFUSED if unfused else 0)
    assert not out[0].any()
    rows = ds_check.sample_rows(cfg, 1000)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, k, out, topk,
                        rows, label_upto=cfg.S0 + 1)


def test_k_at_least_seq_and_dense_equal():
    """k >= S attends every token: same output as the dense path (k <= 0)."""
    cfg, inp = _small_inputs("gqa4_int4_r8")
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    a, ta = run(cfg, inp, labels, seq, S, k=S + 10)
    b, _ = run(cfg, inp, None, seq, S, k=0)
    assert torch.equal(ta[..., :S].cpu(), torch.arange(S, dtype=torch.int32).expand(cfg.B, cfg.Hkv, S))
    assert (ta[..., S:] == -1).all()
    err = ds_check.rel_err_rows(a.float().cpu().numpy(), b.float().cpu().numpy()).max()
    assert err <= 1e-3


def test_all_equal_scores_pick_lowest_indices():
    """Heavy channels all zero: every approximate score is 0 and the tie rule
    keeps tokens 0 .. k-1 exactly."""
    cfg, inp = _small_inputs("mha_f16_r16")
    for g in range(cfg.Hkv):
        inp.K[:, g][..., inp.chan[g].long()] = 0
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    for unfused in (False, True):
        labels = prefill(cfg, inp, S)
        out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_UNFUSED if unfused else 0)
        assert torch.equal(topk.cpu(), torch.arange(cfg.k, dtype=torch.int32).expand_as(topk.cpu()))
        ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                            topk, ds_check.sample_rows(cfg, 100), strict_sets=True)


def test_integer_ties_exact():
    """Integer-valued labels give exact fp32 ties; sets must match the oracle
    exactly (same scores on both sides, ties to the lower index)."""
    cfg, inp = _small_inputs("mha_f16_r16")
    gen = torch.Generator().manual_seed(3)
    for g in range(cfg.Hkv):
        ints = torch.randint(-2, 3, (cfg.B, cfg.cap, cfg.r), generator=gen).to(torch.float16)
        inp.K[:, g][..., inp.chan[g].long()] = ints.cuda()
    inp.q.copy_(torch.randint(-2, 3, inp.q.shape, generator=gen).to(torch.float16).cuda())
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    for unfused in (False, True):
        out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_UNFUSED if unfused else 0)
        ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                            topk, ds_check.sample_rows(cfg, 100), strict_sets=True)


@pytest.mark.parametrize("S0,r,int4,k", [(2100, 8, True, 200), (4200, 16, False, 1500),
                                         (5500, 8, True, 700), (6140, 16, True, 2048)])
def test_fused_row_lengths(S0, r, int4, k):
    """The one-kernel path at the row lengths of each register budget (8, 20
    and 24 scores per thread), with the label append of the current token."""
    cfg, inp = _small_inputs("mha_int4_r8", B=2, S0=S0, r=r, int4=int4, k=k)
    _note("fused S0=%d r=%d int4=%s k=%d" % (S0, r, int4, k))
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, k, S)
    assert plan["path"] == "fused"
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_APPEND)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 100), label_upto=S)
    check_without_idx(cfg, inp, labels, seq, S, out, ds_check.sample_rows(cfg, 4),
                      flags=ds.DECODE_APPEND)


@pytest.mark.parametrize("sign", [1, -1])
def test_fused_outlier_scores(sign):
    """Ten outlier tokens per row with scores far above (sign 1) or far below
    (sign -1) the rest: the linear bins between the row's smallest and
    largest score crowd the other tokens into a few bins, so the boundary
    bin is resolved among many candidates."""
    cfg, inp = _small_inputs("mha_int4_r8", B=2, S0=4096, r=8, int4=True, k=256)
    _note("fused outlier scores, sign %d" % sign)
    g = torch.Generator().manual_seed(7 + sign)
    q = inp.q.float()
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            ch = inp.chan[h].long()
            sgn = torch.sign(q[b, h, ch]).to(torch.float16)
            sgn[sgn == 0] = 1
            rows = torch.randperm(cfg.S0, generator=g)[:10].to(inp.K.device)
            inp.K[b, h, rows[:, None], ch[None, :]] = (60 * sign) * sgn
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S)
    assert plan["path"] == "fused"
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_APPEND)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 8), label_upto=S, strict_sets=True)
    check_without_idx(cfg, inp, labels, seq, S, out, ds_check.sample_rows(cfg, 4),
                      flags=ds.DECODE_APPEND)


FUSED_GROUP = {
    # tokens per thread 4 (rows up to 4096 tokens)
    "g7_f16_r16_3000": dict(Hq=28, Hkv=4, S0=3000, r=16, int4=False, k=256),
    # just past 4096: the 9-per-thread class with one token in its last round
    "g4_int4_r16_4096": dict(Hq=16, Hkv=4, S0=4096, r=16, int4=True, k=300),
    # the 8K query-group workload's shape, rows nearly filling the class
    "g7_f16_r16_8223": dict(Hq=28, Hkv=4, S0=8223, r=16, int4=False, k=256),
    # four tokens per label vector: the class holds 12288 tokens, filled
    "g2_int4_r8_12287": dict(Hq=4, Hkv=2, S0=12287, r=8, int4=True, k=1024),
    # the longest rows (16384 tokens) with the largest list
    "g8_f16_r8_16383": dict(Hq=16, Hkv=2, S0=16383, r=8, int4=False, k=2048),
    # label width without a specialised vector
    "g3_f16_r12_5000": dict(Hq=6, Hkv=2, S0=5000, r=12, int4=False, k=300),
    # LeanK: 32 stored K columns
    "g7_leank_6000": dict(Hq=28, Hkv=4, S0=6000, r=8, int4=False, k=512, d_k=32),
}


@pytest.mark.parametrize("name", sorted(FUSED_GROUP))
def test_fused_group_rows(name):
    """The one-kernel path for query groups at the row lengths of each
    register budget (4, 9 and 16 tokens per thread), with the label append
    of the current token, with and without the selected-set output."""
    cfg, inp = _small_inputs("gqa7_f16_r16", B=2, **FUSED_GROUP[name])
    _note("fused group %s" % name)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S)
    assert plan["path"] == "fused" and plan["kernels"] == 1
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_APPEND)
    rows = ds_check.sample_rows(cfg, 4)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, rows, label_upto=S)
    check_without_idx(cfg, inp, labels, seq, S, out, ds_check.sample_rows(cfg, 2, seed=1),
                      flags=ds.DECODE_APPEND)


def test_fused_group_ragged_lengths():
    """Per-row lengths on the query-group kernel: empty, one token, below, at
    and just above k, and full rows, with and without the set output."""
    cfg, inp = _small_inputs("gqa7_f16_r16", B=7, S0=5000, k=300)
    k = cfg.k
    lens = [0, 1, k - 1, k, k + 1, 2500, cfg.S0 + 1]
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0 + 1)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, k, cfg.S0 + 1)
    assert plan["path"] == "fused"
    out, topk = run(cfg, inp, labels, seq, cfg.S0 + 1)
    assert not out[0].any()
    rows = ds_check.sample_rows(cfg, 1000)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, k, out, topk,
                        rows, label_upto=cfg.S0 + 1)
    check_without_idx(cfg, inp, labels, seq, cfg.S0 + 1, out, rows)


@pytest.mark.parametrize("sign", [1, -1])
def test_fused_group_outlier_scores(sign):
    """Outlier tokens on the query-group kernel (as test_fused_outlier_scores:
    the boundary bin is crowded), the outliers aligned with the query summed
    over the group."""
    cfg, inp = _small_inputs("gqa7_f16_r16", B=2, S0=8192, r=16, int4=False, k=256)
    _note("fused group outlier scores, sign %d" % sign)
    g = torch.Generator().manual_seed(11 + sign)
    q = inp.q.float()
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            ch = inp.chan[h].long()
            qs = q[b, h * cfg.G:(h + 1) * cfg.G][:, ch].sum(dim=0)
            sgn = torch.sign(qs).to(torch.float16)
            sgn[sgn == 0] = 1
            rows = torch.randperm(cfg.S0, generator=g)[:10].to(inp.K.device)
            inp.K[b, h, rows[:, None], ch[None, :]] = (60 * sign) * sgn
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S)
    assert plan["path"] == "fused"
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_APPEND)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 4), label_upto=S, strict_sets=True)
    check_without_idx(cfg, inp, labels, seq, S, out, ds_check.sample_rows(cfg, 2),
                      flags=ds.DECODE_APPEND)


@pytest.mark.parametrize("mode", [0, 1])
def test_local_select_fallbacks(mode):
    """Long rows are pre-selected per chunk, then merged.  mode 0: the whole
    top k sits in the first chunk (more than its quota), so the merge's
    completeness check fails; mode 1: a whole chunk of equal scores overflows
    its candidate slots.  Both must fall back to the full select and stay
    exact."""
    cfg, inp = _small_inputs("mha_int4_r8", B=2, S0=6000, k=100)
    q = inp.q.float()
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            ch = inp.chan[g].long()
            if mode == 0:
                sgn = torch.sign(q[b, g, ch]).to(torch.float16)
                sgn[sgn == 0] = 1
                inp.K[b, g, :150][:, ch] = 60 * sgn
            else:
                inp.K[b, g, 1024:3072][:, ch] = 0
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S, flags=ds.DECODE_UNFUSED)
    assert plan["path"] == "local" and plan["chunk"] <= 2048   # several chunks, quota 64 < k
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_UNFUSED)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 100))
    if mode == 0:
        assert (topk < 150).all()


@pytest.mark.parametrize("mode,k", [(0, 400), (1, 400), (0, 2048), (1, 2048), (2, 2048)])
def test_local_select_fallbacks_wide_chunks(mode, k):
    """The same two fallbacks with chunks of over 8192 tokens (512-thread
    score workgroups, 20 scores per thread): 256 rows of 32769 tokens in four
    chunks.  k = 400 gives a quota of about 200 per chunk (threshold from the
    chunk's full histogram); k = 2048 a quota of about 1030, whose threshold
    comes from the histogram of every other item.  mode 0: the top k + 50
    tokens all sit in chunk 0; mode 1: chunk 1 holds over 8000 equal scores,
    more than its candidate slots; mode 2: no fallback."""
    cfg, inp = _small_inputs("mha_int4_r8", B=2, Hq=128, Hkv=128, S0=32768, k=k)
    _note("local fallbacks, wide chunks, mode %d, k %d" % (mode, k))
    S = cfg.S0 + 1
    q = inp.q.float()
    top = k + 50
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            ch = inp.chan[g].long()
            if mode == 0:
                sgn = torch.sign(q[b, g, ch]).to(torch.float16)
                sgn[sgn == 0] = 1
                inp.K[b, g, :top][:, ch] = 60 * sgn
            elif mode == 1:
                inp.K[b, g, 8192:16384][:, ch] = 0
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S, flags=ds.DECODE_UNFUSED)
    assert plan["path"] == "local" and plan["chunk"] > 8192
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_UNFUSED)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 24, seed=3))
    if mode == 0:
        assert (topk < top).all()
    del inp, labels, out, topk
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("want_idx", [True, False])
def test_local_select_groups(mode, want_idx):
    """Query groups on the local path (chunk pre-selection, merge, split
    attention).  mode 0: the top k all in chunk 0 (completeness check fails,
    full select); mode 1: a chunk of equal scores overflows its slots; mode
    2: no fallback.  Rows of ragged lengths, one at most k long (every token
    attended); the result does not depend on the split count."""
    cfg, inp = _small_inputs("gqa7_f16_r16", B=3, S0=6000, k=100)
    _note("local select, groups, mode %d, idx %s" % (mode, want_idx))
    q = inp.q.float()
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            ch = inp.chan[g].long()
            if mode == 0:
                qs = q[b, g * cfg.G:(g + 1) * cfg.G][:, ch].sum(dim=0)
                sgn = torch.sign(qs).to(torch.float16)
                sgn[sgn == 0] = 1
                inp.K[b, g, :150][:, ch] = 60 * sgn
            elif mode == 1:
                inp.K[b, g, 1024:3072][:, ch] = 0
    S = cfg.S0 + 1
    seq = torch.tensor([S, 3100, cfg.k - 5], dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S, flags=ds.DECODE_UNFUSED)
    assert plan["path"] == "local" and plan["chunk"] <= 2048
    out, topk = run(cfg, inp, labels, seq, S, want_idx=want_idx, flags=ds.DECODE_UNFUSED)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 100))
    if mode == 0 and want_idx:
        assert (topk[:2] < 150).all()
    ref, _ = run(cfg, inp, labels, seq, S, want_idx=want_idx, flags=ds.DECODE_UNFUSED, n_split=3)
    err = ds_check.rel_err_rows(out.float().cpu().numpy(), ref.float().cpu().numpy()).max()
    assert err <= 1e-3, err


def test_local_leank_long_rows():
    """LeanK + Double Sparsity rows too long for the one-kernel path (17001
    tokens, 32 stored K columns) on the local path, with the label append."""
    cfg, inp = _small_inputs("leank_ds", B=2, S0=17000, k=400)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S)
    assert plan["path"] == "local"
    out, topk = run(cfg, inp, labels, seq, S, flags=ds.DECODE_APPEND)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 4), label_upto=S)
    check_without_idx(cfg, inp, labels, seq, S, out, ds_check.sample_rows(cfg, 2),
                      flags=ds.DECODE_APPEND)


@pytest.mark.parametrize("case", ["dense_5000", "sparse_1500", "leank_dense_3000"])
def test_group_attention_long_splits(case):
    """The split attention for query groups with more than four tiles per
    wave (one split per row: the ring of three tile buffers), including
    splits longer than one token-list batch (2048 positions) and tails of
    one to three tiles."""
    if case == "dense_5000":
        cfg, inp = _small_inputs("g8_dense", B=2, S0=5000)
        k, n_split = 0, 1
    elif case == "sparse_1500":
        cfg, inp = _small_inputs("gqa7_f16_r16", B=2, S0=4000, k=1500)
        k, n_split = 1500, 1
    else:
        cfg, inp = _small_inputs("leank_dense", B=2, S0=3000)
        k, n_split = 0, 1
    _note("group attention, long splits, %s" % case)
    S = cfg.S0 + 1
    seq = torch.tensor([S, S - 37], dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S) if k > 0 else None
    kw = dict(n_split=n_split, flags=ds.DECODE_UNFUSED)
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, k, S, **kw)
    assert plan["n_split"] == 1 and plan["tokens_per_split"] > 256
    out, topk = run(cfg, inp, labels, seq, S, k=k, **kw)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, k, out, topk,
                        ds_check.sample_rows(cfg, 100))


WIDE = {
    # 256-channel queries, 128 stored K columns chosen by the keep table,
    # every stored column a heavy channel (fp16 labels of generic width)
    "mha_q256_r128_f16": dict(B=2, Hq=4, Hkv=4, D=256, d_k=128, S0=1500, r=128, k=64,
                              int4=False),
    # the same for a query group with 64 int4 heavy channels
    "g4_q256_r64_int4": dict(B=2, Hq=16, Hkv=4, D=256, d_k=128, S0=2000, r=64, k=100,
                             int4=True),
}


@pytest.mark.parametrize("name", sorted(WIDE))
@pytest.mark.parametrize("mode", ["default", "unfused", "stream"])
def test_wide_query_and_widest_labels(name, mode):
    """The widest query (256 channels, read through the keep table) and the
    widest labels (every stored column), on the one-kernel, local and
    streaming paths, with the label append."""
    cfg, inp = _small_inputs("mha_f16_r16", **WIDE[name])
    _note("wide %s %s" % (name, mode))
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, cfg.S0)
    flags = ds.DECODE_APPEND | {"default": 0, "unfused": ds.DECODE_UNFUSED,
                                "stream": ds.DECODE_STREAM}[mode]
    plan = ds.decode_plan(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S, flags=flags)
    assert plan["path"] == {"default": "fused", "unfused": "local", "stream": "stream"}[mode]
    out, topk = run(cfg, inp, labels, seq, S, flags=flags)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                        topk, ds_check.sample_rows(cfg, 100), label_upto=S)


@pytest.mark.parametrize("name", ["mha_int4_r8", "gqa7_f16_r16"])
@pytest.mark.parametrize("k", [1, 2, 17])
@pytest.mark.parametrize("mode", ["default", "unfused", "stream"])
def test_smallest_k(name, k, mode):
    """One, two or seventeen heavy tokens per row on every path (the boundary
    bin then holds the whole quota or one item), with the set output."""
    cfg, inp = _small_inputs(name, k=k)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    flags = {"default": 0, "unfused": ds.DECODE_UNFUSED, "stream": ds.DECODE_STREAM}[mode]
    out, topk = run(cfg, inp, labels, seq, S, flags=flags)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, k, out, topk,
                        ds_check.sample_rows(cfg, 100))


def test_split_count_invariance_and_determinism():
    cfg, inp = _small_inputs("mha_int4_r8")
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    base, t0 = run(cfg, inp, labels, seq, S, n_split=1)
    again, t1 = run(cfg, inp, labels, seq, S, n_split=1)
    assert torch.equal(base, again) and torch.equal(t0, t1)       # bitwise repeatable
    for ns in (2, 3, 7):
        o, t = run(cfg, inp, labels, seq, S, n_split=ns)
        assert torch.equal(t, t0)
        err = ds_check.rel_err_rows(o.float().cpu().numpy(), base.float().cpu().numpy()).max()
        assert err <= 1e-3, (ns, err)


def test_workspace_is_not_read_uninitialised():
    """Garbage in the workspace must not change the result."""
    cfg, inp = _small_inputs("gqa7_f16_r16")
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    labels = prefill(cfg, inp, S)
    need = ds.workspace_size(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    a, ta = run(cfg, inp, labels, seq, S, workspace=ws)
    ws.fill_(0x7F)
    b, tb = run(cfg, inp, labels, seq, S, workspace=ws)
    assert torch.equal(a, b) and torch.equal(ta, tb)


def test_decode_steps_with_appends():
    """Several decode steps: append the current token, then decode."""
    cfg, inp = _small_inputs("gqa2_int4_r16")
    labels = prefill(cfg, inp, cfg.S0)
    for step in range(cfg.steps):
        S = cfg.S0 + step + 1
        seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
        ds.label_append(inp.K, inp.chan, labels, seq - 1)
        q = synth.make_q(cfg, "cuda", step)
        inp.q.copy_(q)
        out, topk = run(cfg, inp, labels, seq, cfg.cap)
        ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k, out,
                            topk, ds_check.sample_rows(cfg, 100))


# ---------------------------------------------------------------------------
# the workloads at full size (sampled rows)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,n_rows", [("tiny", 32), ("llama2_7b_4k", 12),
                                         ("qwen25_7b_gqa_8k", 8), ("long_128k", 6),
                                         ("leank_dense", 6), ("leank_ds", 8)])
def test_workload_full_size(name, n_rows):
    cfg = synth.CONFIGS[name]
    _note("workload %s" % name)
    inp = synth.make_inputs(cfg, "cuda")
    labels = prefill(cfg, inp, cfg.S0) if cfg.k > 0 else None
    last = 2 if cfg.steps >= 2 else 0
    for step in range(last + 1):       # decode a few steps, check the last one
        S = cfg.S0 + step + 1
        seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
        inp.q.copy_(synth.make_q(cfg, "cuda", step))
        out, topk = run(cfg, inp, labels, seq, cfg.cap,
                        flags=ds.DECODE_APPEND if cfg.k > 0 else 0)
    rows = ds_check.sample_rows(cfg, n_rows, seed=5)
    res = ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, labels, seq, cfg.k,
                              out, topk, rows)
    _note("workload %s: %s" % (name, res))
    if cfg.k > 0:
        check_without_idx(cfg, inp, labels, seq, cfg.cap, out, rows[:2], flags=ds.DECODE_APPEND)
    del inp, labels, out, topk
    gc.collect()
    torch.cuda.empty_cache()
