"""The sparse-decode threshold ("Double Sparsity", section "use in SGLang"):
a batch whose longest sequence is below the threshold, or whose shortest is
below k, decodes densely.  Such a step equals the dense decode bit for bit
and still appends the current token's label, which then equals what a label
build over the same tokens writes.  Both the dense-by-policy step and the
sparse step at the threshold are checked against the CPU oracle."""
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


@pytest.mark.parametrize("over", [dict(Hq=4, Hkv=4, r=8, int4=True),
                                  dict(Hq=28, Hkv=4, r=16, int4=False)])
def test_threshold_policy(over):
    cfg = synth.small("policy", B=2, S0=600, steps=2, k=64, seed=77, **over)
    inp = synth.make_inputs(cfg, "cuda")
    S = cfg.S0 + 1
    seq = torch.full((cfg.B,), S, dtype=torch.int32, device="cuda")
    print("policy %s" % over, flush=True)

    def prefilled():
        lab = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
        ds.label_build(inp.K, inp.chan, lab, 0, cfg.S0)
        return lab

    args = (inp.q, inp.K, inp.V, seq, S, cfg.k, cfg.sm_scale)
    # below the threshold: dense, with the label append
    lab_a = prefilled()
    out_a = ds.decode_attn(*args, chan=inp.chan, labels=lab_a, flags=ds.DECODE_APPEND,
                           sparse_decode_threshold=S + 1, min_seq_len=S, validate_tables=True)
    dense = ds.decode_attn(inp.q, inp.K, inp.V, seq, S, 0, cfg.sm_scale)
    full = ds.LabelCache.allocate(cfg.B, cfg.Hkv, cfg.cap, cfg.r, cfg.int4)
    ds.label_build(inp.K, inp.chan, full, 0, S)
    # at the threshold: the sparse step
    lab_b = prefilled()
    out_b = ds.decode_attn(*args, chan=inp.chan, labels=lab_b, flags=ds.DECODE_APPEND,
                           sparse_decode_threshold=S, min_seq_len=S, validate_tables=True)
    lab_c = prefilled()
    out_c = ds.decode_attn(*args, chan=inp.chan, labels=lab_c, flags=ds.DECODE_APPEND,
                           validate_tables=True)
    torch.cuda.synchronize()
    assert torch.equal(out_a, dense)
    assert torch.equal(lab_a.codes, full.codes)
    if full.scales is not None:
        assert torch.equal(lab_a.scales, full.scales)
    assert torch.equal(out_b, out_c)
    assert not torch.equal(out_b, dense)  # k = 64 of 601 tokens: a different result
    rows = ds_check.sample_rows(cfg, 8)
    # dense by policy: every token attended (the oracle with k <= 0)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, None, seq, 0, out_a, None,
                        rows)
    # at the threshold: the sparse step, with its appended labels
    idx = torch.full((cfg.B, cfg.Hkv, cfg.k), -7, dtype=torch.int32, device="cuda")
    lab_d = prefilled()
    out_d = ds.decode_attn(*args, chan=inp.chan, labels=lab_d, flags=ds.DECODE_APPEND,
                           sparse_decode_threshold=S, min_seq_len=S, topk_idx=idx,
                           validate_tables=True)
    torch.cuda.synchronize()
    assert torch.equal(out_d, out_b)
    ds_check.check_rows(cfg, inp.q, inp.K, inp.V, inp.chan, inp.keep, lab_d, seq, cfg.k, out_d,
                        idx, rows)
