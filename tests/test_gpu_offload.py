"""Offloaded K/V ("Double Sparsity", section "experiment details": the
offloading variant keeps the label cache on the GPU and the full K/V cache in
host memory, and fetches only the selected tokens' rows).

Here K and V live in pinned host memory, mapped into the GPU's address space,
and the kernels read the selected rows from there directly: the labels, the
query, the workspace and the output stay on the GPU.  Each step must equal,
bit for bit, the same call with K and V in device memory (the kernels and
their summation order are the same), including the label append, which reads
the current token's K row from host memory.  The offloaded results are also
checked against the CPU oracle on the same bytes: labels bit-exact, selected
sets up to near-ties of the k-th score, attention within 2e-3 per row."""
import ctypes

import pytest
import torch

import synth
from tests import ds_check

pytestmark = pytest.mark.gpu

ds = pytest.importorskip("sparse_attention_decode_ds_amd")

CASES = {
    "mha_int4_r8_fused": (dict(B=3, Hq=4, Hkv=4, S0=1300, r=8, k=100, int4=True), 0),
    "gqa7_f16_r16_fused": (dict(B=2, Hq=28, Hkv=4, S0=900, r=16, k=64, int4=False), 0),
    "mha_int4_r8_local": (dict(B=2, Hq=4, Hkv=4, S0=17000, r=8, k=400, int4=True), 0),
    "leank_ds_local": (dict(B=2, Hq=28, Hkv=4, S0=17000, r=8, k=400, int4=False, d_k=32), 0),
    "gqa4_int4_r8_stream": (dict(B=2, Hq=16, Hkv=4, S0=513, r=8, k=33, int4=True), "stream"),
    "leank_dense": (dict(B=2, Hq=28, Hkv=4, S0=650, r=0, k=0, int4=False, d_k=32), 0),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ds.load()
    yield
    torch.cuda.empty_cache()


def _pinned_copy(t):
    """A new pinned host tensor with t's contents; skips the test unless the
    GPU sees it at the same address (mapped pinned memory)."""
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    hip = ctypes.CDLL("libamdhip64.so")
    dptr = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(h.data_ptr()), 0)
    if rc != 0 or dptr.value != h.data_ptr():
        pytest.skip("pinned host memory not mapped at its host address (status %d)" % rc)
    return h


@pytest.mark.parametrize("name", sorted(CASES))
def test_offloaded_kv_equals_device_kv(name):
    over, mode = CASES[name]
    cfg = synth.small(name, steps=2, seed=300 + len(name), **over)
    inp = synth.make_inputs(cfg, "cuda")
    print("offload %s" % name, flush=True)
    Kh, Vh = _pinned_copy(inp.K), _pinned_copy(inp.V)
    flags = {"stream": ds.DECODE_STREAM}.get(mode, 0) | (ds.DECODE_APPEND if cfg.k > 0 else 0)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    outs, idxs, labs = [], [], []
    for K, V in ((inp.K, inp.V), (Kh, Vh)):
        lab = None
        if cfg.k > 0:
            lab = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
            ds.label_build(inp.K, inp.chan, lab, 0, cfg.S0)
        idx = (torch.full((cfg.B, cfg.Hkv, cfg.k), -7, dtype=torch.int32, device="cuda")
               if cfg.k > 0 else None)
        out = ds.decode_attn(inp.q, K, V, seq, S, cfg.k, cfg.sm_scale, chan=inp.chan, labels=lab,
                             keep=inp.keep, topk_idx=idx, flags=flags, validate_tables=True)
        torch.cuda.synchronize()
        outs.append(out)
        idxs.append(idx)
        labs.append(lab)
    assert torch.equal(outs[0], outs[1])
    if cfg.k > 0:
        assert torch.equal(idxs[0], idxs[1])
        assert torch.equal(labs[0].codes, labs[1].codes)
        if labs[0].scales is not None:
            assert torch.equal(labs[0].scales, labs[1].scales)
    # the offloaded step against the oracle, on the host copies it read
    res = ds_check.check_rows(cfg, inp.q, Kh, Vh, inp.chan, inp.keep, labs[1], seq, cfg.k,
                              outs[1], idxs[1], ds_check.sample_rows(cfg, 8))
    print("offload %s vs oracle: %s" % (name, res), flush=True)


def test_offloaded_kv_full_size_128k():
    # the 128K workload at full size (B4 x 32 KV heads, 131072 + 1 tokens,
    # int4 labels r 8, k 8192): 8.6 GB of K/V in pinned host memory
    cfg = synth.CONFIGS["long_128k"]
    inp = synth.make_inputs(cfg, "cuda")
    print("offload full size %s" % cfg.name, flush=True)
    Kh, Vh = _pinned_copy(inp.K), _pinned_copy(inp.V)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    res = []
    for K, V in ((inp.K, inp.V), (Kh, Vh)):
        lab = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
        ds.label_build(inp.K, inp.chan, lab, 0, cfg.S0)
        idx = torch.full((cfg.B, cfg.Hkv, cfg.k), -7, dtype=torch.int32, device="cuda")
        out = ds.decode_attn(inp.q, K, V, seq, S, cfg.k, cfg.sm_scale, chan=inp.chan, labels=lab,
                             keep=inp.keep, topk_idx=idx, flags=ds.DECODE_APPEND)
        torch.cuda.synchronize()
        res.append((out, idx, lab))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
    assert torch.equal(res[0][2].codes, res[1][2].codes)
    assert torch.equal(res[0][2].scales, res[1][2].scales)
    # sampled rows of the offloaded step against the oracle
    chk = ds_check.check_rows(cfg, inp.q, Kh, Vh, inp.chan, inp.keep, res[1][2], seq, cfg.k,
                              res[1][0], res[1][1], ds_check.sample_rows(cfg, 4, seed=5))
    print("offload full size vs oracle: %s" % chk, flush=True)
