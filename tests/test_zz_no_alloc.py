"""ds_decode_attn_noalloc: the decode step with the library's per-GPU scratch
in place of a caller workspace, for callers that cannot allocate.  Two calls
in a row on one GPU (the second with a smaller input, which reuses the scratch
the first one left behind) must give exactly what ds_decode_attn gives with a
fresh workspace, and agree with the CPU oracle; shapes whose scratch need is
beyond the array are refused before anything is enqueued."""
import ctypes

import pytest
import torch

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
    torch.cuda.empty_cache()


CASES = [
    # larger first: the local path (chunked scores, merge, split attention)
    ("local_gqa", dict(B=2, Hq=16, Hkv=4, S0=17000, r=8, k=400, int4=True), 0),
    # then smaller: the one-kernel path, and a streaming select
    ("fused_mha", dict(B=3, Hq=4, Hkv=4, S0=1300, r=8, k=100, int4=True), 0),
    ("stream_f16", dict(B=2, Hq=8, Hkv=2, S0=700, r=16, k=33, int4=False), ds.DECODE_STREAM),
]


def _step(cfg, inp, flags, noalloc):
    lab = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
    ds.label_build(inp.K, inp.chan, lab, 0, cfg.S0)
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    idx = torch.full((cfg.B, cfg.Hkv, cfg.k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((cfg.B, cfg.Hq, cfg.d_v), 7.0, dtype=torch.float16, device="cuda")
    fl = flags | ds.DECODE_APPEND
    if noalloc:
        ds.decode_attn_noalloc(inp.q, inp.K, inp.V, seq, S, cfg.k, cfg.sm_scale, chan=inp.chan,
                               labels=lab, keep=inp.keep, out=out, topk_idx=idx, flags=fl)
    else:
        ds.decode_attn(inp.q, inp.K, inp.V, seq, S, cfg.k, cfg.sm_scale, chan=inp.chan,
                       labels=lab, keep=inp.keep, out=out, topk_idx=idx, flags=fl)
    torch.cuda.synchronize()
    return out, idx, lab, seq


def test_noalloc_equals_workspace_call_twice():
    for i, (name, over, flags) in enumerate(CASES):
        cfg = synth.small(name, steps=2, seed=900 + i, **over)
        inp = synth.make_inputs(cfg, "cuda")
        print("noalloc call %d: %s" % (i, name), flush=True)
        out_n, idx_n, lab_n, seq = _step(cfg, inp, flags, True)
        out_w, idx_w, lab_w, _ = _step(cfg, inp, flags, False)
        assert torch.equal(out_n, out_w), name
        assert torch.equal(idx_n, idx_w), name
        assert torch.equal(lab_n.codes, lab_w.codes), name
        if lab_n.scales is not None:
            assert torch.equal(lab_n.scales, lab_w.scales), name
        res = ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, lab_n, seq, cfg.k,
                                  out_n, idx_n, ds_check.sample_rows(cfg, 6))
        print("noalloc %s vs oracle: %s" % (name, res), flush=True)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    lib = ds.load()
    kv = ds.KVDesc()
    kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.d_q, kv.d_k, kv.d_v = 64, 64, 8, 128, 128, 128
    kv.capacity = 100000
    for i, s in enumerate((8 * 100000 * 128, 100000 * 128, 128)):
        kv.k_stride[i] = s
        kv.v_stride[i] = s
    lab = ds.LabelDesc()
    lab.r, lab.dtype, lab.slots, lab.codes = 16, ds.LABEL_F16, 100032, 0x100000
    need = lib.ds_decode_attn_workspace_size(ctypes.byref(kv), ctypes.byref(lab), 64, 100000)
    assert need > ds.NOALLOC_SCRATCH_BYTES
    opts = ds.DecodeOpts()
    opts.flags = ds.DECODE_VALIDATE_ONLY
    P = ctypes.c_void_p
    F = 0x100000  # aligned stand-in addresses: validation only, nothing is launched
    rc = lib.ds_decode_attn_noalloc(ctypes.byref(kv), P(F), P(F), P(F), P(F), 100000, None, P(F),
                                    ctypes.byref(lab), 64, 0.088, P(F), None, ctypes.byref(opts),
                                    None)
    assert rc == -5  # DS_ERR_WORKSPACE
    rc = lib.ds_decode_attn_noalloc(ctypes.byref(kv), P(F), P(F), P(F), P(F), 2000, None, P(F),
                                    ctypes.byref(lab), 64, 0.088, P(F), None, ctypes.byref(opts),
                                    None)
    assert rc == 0  # a shorter batch bound fits
