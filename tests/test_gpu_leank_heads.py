"""LeanK with a different number of kept K columns per KV head (LeanK
section 2.2: each head keeps a hardware-aligned count, a multiple of 16).

Layout: the K cache is as wide as the largest count; a head's columns past
its own count hold zeros (their keep entries may be any valid channel), so
they add nothing to a logit or to a label score, and the heavy channels of a
head index its own columns.  Each head's output and selected tokens must
match the oracle run on that head alone with only its own columns."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ds = pytest.importorskip("sparse_attention_decode_ds_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ds.load()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("flags", [0, "unfused", "stream"])
def test_per_head_kept_counts(flags):
    fl = {"unfused": ds.DECODE_UNFUSED, "stream": ds.DECODE_STREAM}.get(flags, 0)
    g0 = torch.Generator().manual_seed(41)
    B, Hkv, G, D, cap, S, r, k = 2, 4, 2, 128, 768, 700, 8, 64
    counts = [16, 48, 32, 48]
    d_k = max(counts)
    K = torch.randn((B, Hkv, cap, d_k), generator=g0)
    for g, n in enumerate(counts):
        K[:, g, :, n:] = 0.0
    K = K.half()
    V = torch.randn((B, Hkv, cap, D), generator=g0).half()
    q = torch.randn((B, Hkv * G, D), generator=g0).half()
    keep = torch.stack([torch.randperm(D, generator=g0)[:d_k].sort().values
                        for _ in range(Hkv)]).to(torch.int32)
    chan = torch.stack([torch.randperm(n, generator=g0)[:r].sort().values
                        for n in counts]).to(torch.int32)
    scale = 1.0 / np.sqrt(D)
    print("leank per-head counts %s flags %s" % (counts, flags), flush=True)

    Kd, Vd, qd = K.cuda(), V.cuda(), q.cuda()
    labels = ds.LabelCache.allocate(B, Hkv, cap, r, False)
    ds.label_build(Kd, chan.cuda(), labels, 0, S)
    seq = torch.full((B,), S, dtype=torch.int32, device="cuda")
    topk = torch.full((B, Hkv, k), -7, dtype=torch.int32, device="cuda")
    out = ds.decode_attn(qd, Kd, Vd, seq, S, k, scale, chan=chan.cuda(), labels=labels,
                         keep=keep.cuda(), topk_idx=topk, flags=fl, validate_tables=True)
    torch.cuda.synchronize()
    out, topk = out.cpu().double().numpy(), topk.cpu().numpy()

    for g, n in enumerate(counts):
        qg = q[:, g * G:(g + 1) * G].contiguous().numpy()
        Kg = K[:, g:g + 1, :, :n].contiguous().numpy()
        Vg = V[:, g:g + 1].contiguous().numpy()
        lab = oracle.Labels.empty(B, 1, cap, r, False)
        oracle.label_build(Kg, chan[g:g + 1].numpy(), lab, 0, S)
        res = oracle.decode(qg, Kg, Vg, np.full(B, S, np.int32), k, scale,
                            chan=chan[g:g + 1].numpy(), lab=lab, keep=keep[g:g + 1, :n].numpy(),
                            want_scores=True)
        for b in range(B):
            got, want = set(topk[b, g].tolist()), set(res["topk"][b, 0].tolist())
            w = res["out"][b]
            if got != want:
                s = res["scores"][b, 0, :S]
                sk = np.sort(s)[::-1][k - 1]
                tol = 1e-3 * abs(sk) + 1e-6 * np.abs(s).max()
                for t in got ^ want:
                    assert abs(s[t] - sk) <= tol, (g, b, t, s[t], sk)
                # near-tie swap: the reference is the oracle's attention over
                # the GPU's own set, so the arithmetic is still checked
                sets = np.full((B, 1, k), -1, np.int32)
                sets[b, 0] = topk[b, g]
                w = oracle.attend_sets(qg, Kg, Vg, sets, scale, keep=keep[g:g + 1, :n].numpy(),
                                       rows=[(b, 0)])[b]
            o = out[b, g * G:(g + 1) * G]
            err = (np.abs(o - w).max(axis=1) / np.abs(w).max(axis=1)).max()
            assert err <= 2e-3, (g, b, err)


def test_fully_pruned_head_and_pruned_v_columns():
    # LeanK section 4.4: a head may lose every channel, and V may be pruned
    # too.  With the same zero-padding layout a fully pruned head (K and V all
    # zero) outputs zeros, and pruned V columns give zero output channels;
    # the rest matches the oracle on the same cache.
    g0 = torch.Generator().manual_seed(43)
    B, Hkv, G, D, cap, S, r, k, d_k = 2, 3, 2, 128, 512, 480, 8, 40, 32
    K = torch.randn((B, Hkv, cap, d_k), generator=g0)
    V = torch.randn((B, Hkv, cap, D), generator=g0)
    K[:, 1] = 0.0
    V[:, 1] = 0.0                    # head 1: fully pruned
    V[:, 2, :, 64:] = 0.0            # head 2: V keeps 64 of 128 channels
    K, V = K.half(), V.half()
    q = torch.randn((B, Hkv * G, D), generator=g0).half()
    keep = torch.stack([torch.randperm(D, generator=g0)[:d_k].sort().values
                        for _ in range(Hkv)]).to(torch.int32)
    chan = torch.stack([torch.randperm(d_k, generator=g0)[:r].sort().values
                        for _ in range(Hkv)]).to(torch.int32)
    scale = 1.0 / np.sqrt(D)
    labels = ds.LabelCache.allocate(B, Hkv, cap, r, False)
    ds.label_build(K.cuda(), chan.cuda(), labels, 0, S)
    seq = torch.full((B,), S, dtype=torch.int32, device="cuda")
    out = ds.decode_attn(q.cuda(), K.cuda(), V.cuda(), seq, S, k, scale, chan=chan.cuda(),
                         labels=labels, keep=keep.cuda(), validate_tables=True)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    assert np.all(out[:, 2:4] == 0.0)
    assert np.all(out[:, 4:6, 64:] == 0.0)
    lab = oracle.Labels.empty(B, Hkv, cap, r, False)
    oracle.label_build(K.numpy(), chan.numpy(), lab, 0, S)
    res = oracle.decode(q.numpy(), K.numpy(), V.numpy(), np.full(B, S, np.int32), k, scale,
                        chan=chan.numpy(), lab=lab, keep=keep.numpy())
    for h in (0, 1, 4, 5):
        w = res["out"][:, h, :64]
        err = (np.abs(out[:, h, :64] - w).max(axis=1) / np.abs(w).max(axis=1)).max()
        assert err <= 2e-3, (h, err)


# ---------------------------------------------------------------------------
# Per-head storage (ds_head_layout): every KV head stores only its own kept
# K columns, and a fully pruned head stores neither K nor V (LeanK section
# 2.2: hardware-aligned per-head counts; section 4.4: heads with no K channel
# left drop their V cache too).  Reading: a fully pruned head contributes a
# zero output and selects no token.
# ---------------------------------------------------------------------------

def _per_head_case(B, Hkv, G, D, cap, counts, r, seed, pages_P=0):
    g0 = torch.Generator().manual_seed(seed)
    d_k = max(counts)
    Ks = [torch.randn((B, cap, n), generator=g0).half() for n in counts]
    Vs = [torch.randn((B, cap, D), generator=g0).half() for _ in counts]
    q = torch.randn((B, Hkv * G, D), generator=g0).half()
    keep = torch.stack([torch.randperm(D, generator=g0)[:d_k].sort().values
                        for _ in range(Hkv)]).to(torch.int32)
    chan = torch.stack([torch.randperm(max(n, r), generator=g0)[:r].sort().values
                        for n in counts]).to(torch.int32)
    tokens = pages_P if pages_P else cap
    lay = ds.HeadLayout.packed(counts, tokens)
    if not pages_P:
        Kb = torch.zeros((B, lay.k_row), dtype=torch.float16, device="cuda")
        Vb = torch.zeros((B, max(lay.v_row, 8)), dtype=torch.float16, device="cuda")
        for g, n in enumerate(counts):
            if n:
                lay.head_k(Kb, g).copy_(Ks[g])
                lay.head_v(Vb, g).copy_(Vs[g])
        return q, Ks, Vs, keep, chan, lay, Kb, Vb, None
    # paged: pool of P-token pages, each page holding every head's block
    P = pages_P
    mp = cap // P
    n_pages = B * mp + 2
    perm = torch.randperm(n_pages, generator=g0)[:B * mp].view(B, mp).to(torch.int32)
    Kb = torch.zeros((n_pages, lay.k_row), dtype=torch.float16, device="cuda")
    Vb = torch.zeros((n_pages, max(lay.v_row, 8)), dtype=torch.float16, device="cuda")
    for b in range(B):
        for p in range(mp):
            pg = int(perm[b, p])
            for g, n in enumerate(counts):
                if n:
                    lay.head_k(Kb[pg:pg + 1], g)[0].copy_(Ks[g][b, p * P:(p + 1) * P])
                    lay.head_v(Vb[pg:pg + 1], g)[0].copy_(Vs[g][b, p * P:(p + 1) * P])
    return q, Ks, Vs, keep, chan, lay, Kb, Vb, ds.Pages(perm.cuda(), P)


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("mode", ["fused", "unfused", "stream", "paged", "dense"])
def test_per_head_storage_matches_oracle(mode, G):
    """G = 1 runs the vector-unit kernels, G = 2 the matrix-core ones."""
    B, Hkv, D, cap, S, r = 2, 4, 128, 768, 700, 8
    k = 0 if mode == "dense" else 64
    counts = [16, 48, 0, 32]
    fl = {"unfused": ds.DECODE_UNFUSED, "stream": ds.DECODE_STREAM}.get(mode, 0)
    q, Ks, Vs, keep, chan, lay, Kb, Vb, pages = _per_head_case(
        B, Hkv, G, D, cap, counts, r, 44, pages_P=16 if mode == "paged" else 0)
    print("per-head storage %s G=%d counts %s" % (mode, G, counts), flush=True)
    scale = 1.0 / np.sqrt(D)
    labels = ds.LabelCache.allocate(B, Hkv, cap, r, False)
    ds.label_build(Kb, chan.cuda(), labels, 0, S - 1, pages=pages, heads=lay)
    seq = torch.full((B,), S, dtype=torch.int32, device="cuda")
    topk = torch.full((B, Hkv, max(k, 1)), -7, dtype=torch.int32, device="cuda") if k else None
    out = ds.decode_attn(q.cuda(), Kb, Vb, seq, S, k, scale, chan=chan.cuda(), labels=labels,
                         keep=keep.cuda(), topk_idx=topk, flags=fl | ds.DECODE_APPEND,
                         validate_tables=True, pages=pages, heads=lay)
    torch.cuda.synchronize()
    _check_per_head(out, topk, q, Ks, Vs, keep, chan, labels, counts, G, k, S, scale)


def _check_per_head(out, topk, q, Ks, Vs, keep, chan, labels, counts, G, k, S, scale):
    """Each head's output (and selected set) against the oracle run on that
    head alone with only its own columns; pruned heads give zeros and no
    token.  S: the sequence length of every row, or one per row."""
    out = out.cpu().double().numpy()
    tk = topk.cpu().numpy() if topk is not None else None
    B = out.shape[0]
    r = chan.shape[1]
    seqs = np.broadcast_to(np.asarray(S, np.int32), (B,)).copy()
    for g, n in enumerate(counts):
        o = out[:, g * G:(g + 1) * G]
        if n == 0:  # fully pruned: zero output, no token
            assert np.all(o == 0.0), g
            if tk is not None:
                assert np.all(tk[:, g] == -1), g
            continue
        qg = q[:, g * G:(g + 1) * G].contiguous().numpy()
        Kg = Ks[g][:, None].contiguous().numpy()
        Vg = Vs[g][:, None].contiguous().numpy()
        cg = chan[g:g + 1].numpy()
        lab = oracle.Labels.empty(B, 1, labels.slots, r, False)
        oracle.label_build(Kg, cg, lab, 0, int(seqs.max()))
        got_lab = labels.codes[:, g].cpu().numpy().view(np.uint16)
        for b in range(B):  # appended label included
            assert np.array_equal(lab.f16[b, 0, :seqs[b]], got_lab[b, :seqs[b]]), (g, b)
        res = oracle.decode(qg, Kg, Vg, seqs, k, scale, chan=cg if k else None,
                            lab=lab if k else None, keep=keep[g:g + 1, :n].numpy(),
                            want_scores=k > 0)
        for b in range(B):
            w = res["out"][b]
            if k > 0:
                got, want = set(tk[b, g].tolist()), set(res["topk"][b, 0].tolist())
                if got != want:
                    kk = min(k, int(seqs[b]))
                    s = res["scores"][b, 0, :seqs[b]]
                    sk = np.sort(s)[::-1][kk - 1]
                    tol = 1e-3 * abs(sk) + 1e-6 * np.abs(s).max()
                    for t in got ^ want:
                        assert abs(s[t] - sk) <= tol, (g, b, t)
                    sets = np.full((B, 1, k), -1, np.int32)
                    sets[b, 0] = tk[b, g]
                    w = oracle.attend_sets(qg, Kg, Vg, sets, scale, keep=keep[g:g + 1, :n].numpy(),
                                           rows=[(b, 0)])[b]
            err = (np.abs(o[b] - w).max(axis=1) / np.abs(w).max(axis=1)).max()
            assert err <= 2e-3, (g, b, err)


@pytest.mark.parametrize("mode,G,n_split,counts", [
    ("unfused", 2, 3, [16, 48, 0, 32]),
    ("unfused", 1, 7, [48, 0, 8, 24]),
    ("stream", 4, 5, [0, 32, 16, 0]),
    ("paged", 2, 4, [24, 0, 48, 8]),
    ("dense", 2, 6, [8, 48, 0, 0]),
    ("dense", 1, 9, [32, 16, 40, 0]),
])
def test_per_head_splits_dealt_by_bytes(mode, G, n_split, counts):
    """With a per-head layout and several splits, a batch row's workgroups go
    to its heads in proportion to their bytes per token (pruned heads get
    none) and the combine finds each head's partials again: split counts
    that do not divide evenly, heads of one to several splits, pruned heads
    first, in the middle and last."""
    B, Hkv, D, cap, S, r = 3, 4, 128, 768, 701, 8
    k = 0 if mode == "dense" else 200
    fl = {"unfused": ds.DECODE_UNFUSED, "stream": ds.DECODE_STREAM,
          "paged": ds.DECODE_UNFUSED}.get(mode, 0)
    q, Ks, Vs, keep, chan, lay, Kb, Vb, pages = _per_head_case(
        B, Hkv, G, D, cap, counts, r, 45, pages_P=16 if mode == "paged" else 0)
    print("per-head splits %s G=%d n_split=%d counts %s" % (mode, G, n_split, counts), flush=True)
    scale = 1.0 / np.sqrt(D)
    labels = ds.LabelCache.allocate(B, Hkv, cap, r, False)
    ds.label_build(Kb, chan.cuda(), labels, 0, S - 1, pages=pages, heads=lay)
    seq = torch.tensor([S, 517, 1], dtype=torch.int32, device="cuda")
    topk = torch.full((B, Hkv, max(k, 1)), -7, dtype=torch.int32, device="cuda") if k else None
    out = ds.decode_attn(q.cuda(), Kb, Vb, seq, S, k, scale, chan=chan.cuda(), labels=labels,
                         keep=keep.cuda(), topk_idx=topk, n_split=n_split,
                         flags=fl | ds.DECODE_APPEND, validate_tables=True, pages=pages,
                         heads=lay)
    torch.cuda.synchronize()
    _check_per_head(out, topk, q, Ks, Vs, keep, chan, labels, counts, G, k, seq.cpu().numpy(),
                    scale)


def test_per_head_every_head_pruned_with_splits():
    """No head stores anything: every workgroup of the split pass has no work
    and the combine writes zeros."""
    B, Hkv, G, D, cap, S = 2, 3, 2, 128, 256, 200
    lay = ds.HeadLayout.packed([0, 0, 0], cap)
    Kb = torch.zeros((B, max(lay.k_row, 8)), dtype=torch.float16, device="cuda")
    Vb = torch.zeros((B, max(lay.v_row, 8)), dtype=torch.float16, device="cuda")
    q = torch.randn((B, Hkv * G, D)).half().cuda()
    keep = torch.zeros((Hkv, 8), dtype=torch.int32, device="cuda")
    seq = torch.full((B,), S, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hkv * G, D), 7.0, dtype=torch.float16, device="cuda")
    ds.decode_attn(q, Kb, Vb, seq, S, 0, 0.1, keep=keep, n_split=4, heads=lay, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0.0)
