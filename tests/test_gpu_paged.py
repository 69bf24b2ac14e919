"""Paged token pool ("Double Sparsity", section "use in SGLang": the serving
system keeps K/V in a pool of token slots shared by the sequences, and a table
maps each sequence's tokens to slots).  K and V live in pools [n_pages][H_kv]
[page_size][d] under a shuffled page table; the label cache stays one
contiguous stream per (batch row, KV head).  Every path must give, bit for bit,
what it gives on the same data in contiguous rows (the kernels and their
summation order are the same), and match the oracle run on the cache the page
table describes (gathered on the host).  Table entries of pages a row does not
use point at a poison page (large values), so an access through them would
change the results."""
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


def to_pool(X, P, perm, n_pages):
    """Scatter a contiguous cache [B][H][cap][d] into a pool of n_pages pages
    of P tokens: logical page p of row b goes to page perm[b][p]."""
    B, H, cap, d = X.shape
    mp = perm.shape[1]
    Xp = torch.zeros((B, H, mp * P, d), dtype=X.dtype, device=X.device)
    Xp[:, :, :cap] = X
    pool = torch.full((n_pages, H, P, d), 1000.0, dtype=X.dtype, device=X.device)  # poison
    src = Xp.view(B, H, mp, P, d).permute(0, 2, 1, 3, 4).reshape(B * mp, H, P, d)
    pool[perm.reshape(-1).long()] = src
    return pool


def paged_inputs(cfg, inp, P, seed, seq=None):
    """Pools for inp.K / inp.V under a shuffled page table (a few spare pages,
    one of them the poison page that entries of unused pages point at)."""
    B = cfg.B
    mp = (cfg.cap + P - 1) // P
    n_pages = B * mp + 3
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages - 1, generator=g)[:B * mp].view(B, mp).to(torch.int32)
    Kp = to_pool(inp.K, P, perm, n_pages)
    Vp = to_pool(inp.V, P, perm, n_pages)
    table = perm.clone()
    if seq is not None:  # pages past a row's length: the poison page
        for b in range(B):
            used = (int(seq[b]) + P - 1) // P
            table[b, used:] = n_pages - 1
    return Kp, Vp, ds.Pages(table.cuda(), P), mp * P


CASES = {
    # name: (workload overrides, flags, page size)
    "fused_mha_int4": (dict(B=3, Hq=4, Hkv=4, S0=1300, r=8, k=100, int4=True), 0, 16),
    "fused_gqa7_f16": (dict(B=2, Hq=28, Hkv=4, S0=900, r=16, k=64, int4=False), 0, 64),
    "local_mha_int4": (dict(B=2, Hq=4, Hkv=4, S0=1300, r=8, k=100, int4=True), "unfused", 16),
    "local_long_int4": (dict(B=2, Hq=4, Hkv=4, S0=17000, r=8, k=400, int4=True), 0, 64),
    "stream_gqa4_int4": (dict(B=2, Hq=16, Hkv=4, S0=513, r=8, k=33, int4=True), "stream", 16),
    "leank_dense": (dict(B=2, Hq=28, Hkv=4, S0=650, r=0, k=0, int4=False, d_k=32), 0, 16),
    "leank_ds_local": (dict(B=2, Hq=28, Hkv=4, S0=17000, r=8, k=400, int4=False, d_k=32), 0, 64),
    "dense_mha_split": (dict(B=2, Hq=4, Hkv=4, S0=700, r=0, k=0, int4=False), 0, 16),
}


def _run(cfg, q, K, V, seq, S, labels, inp, flags, pages=None, want_idx=True):
    idx = None
    if cfg.k > 0 and want_idx:
        idx = torch.full((cfg.B, cfg.Hkv, cfg.k), -7, dtype=torch.int32, device="cuda")
    out = ds.decode_attn(q, K, V, seq, S, cfg.k, cfg.sm_scale, chan=inp.chan, labels=labels,
                         keep=inp.keep, topk_idx=idx, flags=flags, validate_tables=True,
                         pages=pages)
    torch.cuda.synchronize()
    return out, idx


class PagedRows:
    """Rows of a paged pool for the parity checks, gathered on the host one
    (batch row, KV head) at a time through the oracle's page gather."""

    def __init__(self, pool, pages):
        self.pool, self.table, self.P = pool, pages.table.cpu().numpy(), pages.page_size

    def __getitem__(self, bg):
        b, g = bg
        part = self.pool[:, g:g + 1].cpu().numpy()
        return torch.from_numpy(oracle.gather_pages(part, self.table[b:b + 1], self.P)[0, 0])


def _label_slots_equal(cfg, la, lb, seq):
    for b in range(cfg.B):
        S = int(seq[b])
        assert torch.equal(la.codes[b, :, :S], lb.codes[b, :, :S]), b
        if la.scales is not None:
            assert torch.equal(la.scales[b, :, :S], lb.scales[b, :, :S]), b


def _paged_vs_contiguous(cfg, inp, seq, S, P, flags, n_rows, seed=77):
    Kp, Vp, pages, cap_p = paged_inputs(cfg, inp, P, seed, seq.cpu())
    res = []
    for K, V, pg in ((inp.K, inp.V, None), (Kp, Vp, pages)):
        lab = None
        if cfg.k > 0:
            lab = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cap_p, cfg.r, cfg.int4)
            ds.label_build(K, inp.chan, lab, 0, cfg.S0, pages=pg)
        out, idx = _run(cfg, inp.q, K, V, seq, S, lab, inp, flags, pg)
        res.append((lab, out, idx))
    (lab_c, out_c, idx_c), (lab_p, out_p, idx_p) = res
    assert torch.equal(out_c, out_p)
    if cfg.k > 0:
        assert torch.equal(idx_c, idx_p)
        _label_slots_equal(cfg, lab_c, lab_p, seq)
    # the oracle on the cache the page table describes
    rows = ds_check.sample_rows(cfg, n_rows)
    r = ds_check.check_rows(cfg, inp.q, PagedRows(Kp, pages), PagedRows(Vp, pages), inp.chan,
                            inp.keep, lab_p, seq, cfg.k, out_p, idx_p, rows)
    return r


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_pool_equals_contiguous_rows(name):
    over, mode, P = CASES[name]
    cfg = synth.small(name, steps=2, seed=500 + len(name), **over)
    inp = synth.make_inputs(cfg, "cuda")
    print("paged %s P=%d" % (name, P), flush=True)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    if cfg.B > 1:
        seq[1] = max(1, S - 37)  # a shorter row: pages past it are poison
    flags = {"unfused": ds.DECODE_UNFUSED, "stream": ds.DECODE_STREAM}.get(mode, 0)
    if cfg.k > 0:
        flags |= ds.DECODE_APPEND
    r = _paged_vs_contiguous(cfg, inp, seq, S, P, flags, 6)
    print("paged %s vs oracle: %s" % (name, r), flush=True)


@pytest.mark.parametrize("name", ["llama2_7b_4k", "long_128k"])
def test_paged_pool_full_size(name):
    # the graded workloads at full size in a pool of 16-token pages under a
    # shuffled table: bit-identical to contiguous rows, sampled rows against
    # the oracle
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg, "cuda")
    print("paged full size %s" % name, flush=True)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    r = _paged_vs_contiguous(cfg, inp, seq, S, 16, ds.DECODE_APPEND, 3)
    print("paged full size %s vs oracle: %s" % (name, r), flush=True)
    del inp
    gc.collect()
    torch.cuda.empty_cache()
