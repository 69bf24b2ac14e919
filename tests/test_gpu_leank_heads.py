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
