"""A decode step captured in a HIP graph (torch.cuda.graph) and replayed:
the library enqueues kernels only (no allocation, memset or host
synchronisation), so each replay must give the eager result bit for bit.
Replays are separated by eager work and synchronisations."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

ds = pytest.importorskip("sparse_attention_decode_ds_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ds.load()


@pytest.mark.parametrize("name,flags", [("mha_int4", 0), ("gqa_f16", 0), ("mha_int4", 4),
                                        ("gqa_f16", 8)])
def test_graph_replay_matches_eager(name, flags):
    kw = {"mha_int4": dict(B=2, Hq=4, Hkv=4, S0=1500, r=8, k=100, int4=True),
          "gqa_f16": dict(B=2, Hq=28, Hkv=4, S0=3000, r=16, k=256, int4=False)}[name]
    cfg = synth.small(name, steps=3, seed=77, **kw)
    inp = synth.make_inputs(cfg, "cuda")
    labels = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
    S = cfg.S0 + 1
    ds.label_build(inp.K, inp.chan, labels, 0, S)
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    need = ds.workspace_size(inp.K, inp.V, cfg.Hq, cfg.D, labels, cfg.k, S)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.B, cfg.Hq, 128), dtype=torch.float16, device="cuda")
    topk = torch.empty((cfg.B, cfg.Hkv, cfg.k), dtype=torch.int32, device="cuda")

    def step():
        ds.decode_attn(inp.q, inp.K, inp.V, seq, S, cfg.k, cfg.sm_scale, chan=inp.chan,
                       labels=labels, keep=inp.keep, out=out, topk_idx=topk, workspace=ws,
                       flags=flags)

    step()
    torch.cuda.synchronize()
    ref_out, ref_topk = out.clone(), topk.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        out.zero_()
        topk.fill_(-5)
        ws.random_(0, 255)  # the workspace needs no initialisation
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), rep
        assert torch.equal(topk, ref_topk), rep
