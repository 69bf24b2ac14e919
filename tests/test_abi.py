"""The C ABI without a GPU: the library loads, exports every function that
include/ds.h declares, and its host-side validation returns the documented
status codes before launching anything."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ds = pytest.importorskip("sparse_attention_decode_ds_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ds.LIB_PATH):
        pytest.skip("libds.so not built")
    return ds.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ds.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(ds.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.ds_abi_version() == 4
    for code in range(0, -7, -1):
        s = lib.ds_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.ds_status_str(-99).decode() == "unknown status"


FAKE = 0x100000  # an aligned address; never dereferenced on these paths


def _kv(**over):
    d = ds.KVDesc()
    vals = dict(batch=2, n_q_heads=28, n_kv_heads=4, d_q=128, d_k=128, d_v=128, capacity=1000)
    vals.update({k: v for k, v in over.items() if not k.endswith("stride")})
    for k, v in vals.items():
        setattr(d, k, v)
    ks = over.get("k_stride", (4 * 1000 * 128, 1000 * 128, 128))
    vs = over.get("v_stride", (4 * 1000 * 128, 1000 * 128, 128))
    for i in range(3):
        d.k_stride[i] = ks[i]
        d.v_stride[i] = vs[i]
    return d


def _lab(**over):
    d = ds.LabelDesc()
    vals = dict(r=16, dtype=ds.LABEL_F16, slots=1024, reserved0=0, codes=FAKE, scales=None)
    vals.update(over)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


def _decode(lib, kv=None, lab=None, k=64, max_seq=900, ws_bytes=1 << 30, flags=ds.DECODE_VALIDATE_ONLY,
            q=FAKE, K=FAKE, V=FAKE, seq=FAKE, out=FAKE, chan=FAKE, keep=None, ws=FAKE,
            n_split=0, scale=0.088):
    kv = kv or _kv()
    lab = lab if lab is not None else _lab()
    opts = ds.DecodeOpts()
    opts.n_split, opts.flags = n_split, flags
    P = ctypes.c_void_p
    return lib.ds_decode_attn(ctypes.byref(kv), P(q), P(K), P(V), P(seq), max_seq, P(keep),
                              P(chan), ctypes.byref(lab) if lab is not False else None, k, scale,
                              P(out), None, P(ws), ws_bytes, ctypes.byref(opts), None)


def test_validate_only_accepts_good_arguments(lib):
    assert _decode(lib) == 0
    # a paged pool: 64 pages of 16 tokens per batch row, 50 pages in the pool
    paged = _kv(page_size=16, capacity=1024, max_pages=64, n_pages=50, page_table=FAKE,
                k_stride=(4 * 16 * 128, 16 * 128, 128), v_stride=(4 * 16 * 128, 16 * 128, 128))
    assert _decode(lib, kv=paged) == 0
    assert _decode(lib, kv=paged, k=0, lab=False, chan=None) == 0
    assert _decode(lib, k=0, lab=False, chan=None) == 0                    # dense, no labels
    assert _decode(lib, lab=_lab(dtype=ds.LABEL_INT4, r=8, scales=FAKE)) == 0
    kv = _kv(d_k=32, k_stride=(4 * 1000 * 32, 1000 * 32, 32))
    assert _decode(lib, kv=kv, keep=FAKE, lab=_lab(r=8)) == 0                # LeanK
    # a dense step that still appends the current token's label
    assert _decode(lib, k=0, flags=ds.DECODE_VALIDATE_ONLY | ds.DECODE_APPEND) == 0


@pytest.mark.parametrize("case,code", [
    (dict(kv=_kv(n_q_heads=30)), -2),                 # heads not divisible
    (dict(kv=_kv(n_q_heads=40, n_kv_heads=4)), -2),   # group of 10 > 8
    (dict(kv=_kv(d_v=64)), -2),
    (dict(kv=_kv(d_k=36)), -2),
    (dict(kv=_kv(capacity=0)), -2),
    (dict(kv=_kv(page_size=16)), -1),                 # paged without a page table
    (dict(kv=_kv(max_pages=3)), -1),                  # paging fields on contiguous rows
    (dict(kv=_kv(page_size=24, capacity=960, max_pages=40, n_pages=50, page_table=FAKE)), -2),
    (dict(kv=_kv(page_size=8, capacity=1024, max_pages=128, n_pages=50, page_table=FAKE)), -2),
    (dict(kv=_kv(page_size=16, capacity=1024, max_pages=63, n_pages=50, page_table=FAKE)), -2),
    (dict(kv=_kv(page_size=16, capacity=1024, max_pages=64, n_pages=0, page_table=FAKE)), -2),
    (dict(kv=_kv(page_size=65536, capacity=65536, max_pages=1, n_pages=32768,
                 page_table=FAKE)), -2),                # physical ids past 2^31
    (dict(kv=_kv(k_stride=(4 * 1000 * 128, 1000 * 128, 132))), -4),
    (dict(lab=_lab(r=0)), -2),
    (dict(lab=_lab(r=129)), -2),
    (dict(lab=_lab(dtype=ds.LABEL_INT4, r=7, scales=FAKE)), -3),
    (dict(lab=_lab(dtype=5)), -3),
    (dict(lab=_lab(slots=999)), -2),
    (dict(lab=_lab(slots=1000 + 4)), -2),
    (dict(lab=_lab(codes=None)), -1),
    (dict(lab=_lab(codes=FAKE + 8)), -4),
    (dict(lab=_lab(dtype=ds.LABEL_INT4, r=8, scales=None)), -1),
    (dict(chan=None), -1),
    (dict(q=None), -1),
    (dict(out=FAKE + 2), -4),
    (dict(K=FAKE + 4), -4),
    (dict(max_seq=1001), -1),
    (dict(max_seq=-1), -1),
    (dict(ws_bytes=16), -5),
    (dict(ws=None), -5),
    (dict(ws=FAKE + 64), -4),
    (dict(flags=ds.DECODE_VALIDATE_ONLY | 64), -1),
    (dict(n_split=-2), -1),
    (dict(k=0, lab=False, chan=None, flags=ds.DECODE_VALIDATE_ONLY | ds.DECODE_APPEND), -1),
    (dict(kv=_kv(d_k=32, k_stride=(4 * 1000 * 32, 1000 * 32, 32)), lab=_lab(r=8)), -2),  # no keep
    (dict(scale=float("nan")), -1),
])
def test_validation_errors(lib, case, code):
    assert _decode(lib, **case) == code


def test_workspace_size(lib):
    kv = _kv()
    lab = _lab()
    n = lib.ds_decode_attn_workspace_size(ctypes.byref(kv), ctypes.byref(lab), 64, 900)
    assert n > 0 and n % 256 == 0
    assert _decode(lib, ws_bytes=n) == 0
    assert _decode(lib, ws_bytes=n - 1) == -5
    assert lib.ds_decode_attn_workspace_size(ctypes.byref(kv), ctypes.byref(lab), 64, 5000) == 0
    assert lib.ds_decode_attn_workspace_size(ctypes.byref(_kv(d_v=7)), ctypes.byref(lab), 64, 9) == 0
    assert lib.ds_decode_attn_workspace_size(ctypes.byref(kv), None, 0, 900) > 0


def _plan(lib, kv, lab, k, max_seq, flags=0, n_split=0):
    opts = ds.DecodeOpts()
    opts.n_split, opts.flags = n_split, flags
    pl = ds.DecodePlan()
    rc = lib.ds_decode_attn_plan(ctypes.byref(kv), ctypes.byref(lab) if lab is not None else None,
                                 k, max_seq, ctypes.byref(opts), ctypes.byref(pl))
    return rc, pl


def _mha(B, H, cap):
    return _kv(batch=B, n_q_heads=H, n_kv_heads=H, capacity=cap,
               k_stride=(H * cap * 128, cap * 128, 128), v_stride=(H * cap * 128, cap * 128, 128))


def test_decode_plan_paths(lib):
    """The plan query names the path each workload shape takes."""
    int4 = dict(dtype=ds.LABEL_INT4, r=8, scales=FAKE)
    # Llama-2-7B-shaped 4K rows, k = 256, single query head per group: one kernel.
    rc, pl = _plan(lib, _mha(32, 32, 4160), _lab(slots=4160, **int4), 256, 4097)
    assert rc == 0 and ds.PATHS[pl.path] == "fused" and pl.kernels == 1 and pl.n_split == 1
    # 128K rows, k = 8192: local top-M + merge, split attention + combine.
    rc, pl = _plan(lib, _mha(4, 32, 131088), _lab(slots=131088, **int4), 8192, 131073)
    assert rc == 0 and ds.PATHS[pl.path] == "local" and pl.n_split > 1 and pl.kernels == 4
    assert 8192 < pl.chunk <= 10240     # 512-thread chunk workgroups, 20 scores per thread
    assert pl.n_split * pl.tokens_per_split >= 8192
    # GQA groups (7 query heads per KV head): one 1024-thread kernel for rows
    # up to 16384 tokens, local top-M + merge beyond.
    rc, pl = _plan(lib, _kv(batch=64, capacity=8224, k_stride=(4 * 8224 * 128, 8224 * 128, 128),
                            v_stride=(4 * 8224 * 128, 8224 * 128, 128)), _lab(slots=8224), 256, 8193)
    assert rc == 0 and ds.PATHS[pl.path] == "fused" and pl.kernels == 1 and pl.n_split == 1
    rc, pl = _plan(lib, _kv(batch=8, capacity=32784, k_stride=(4 * 32784 * 128, 32784 * 128, 128),
                            v_stride=(4 * 32784 * 128, 32784 * 128, 128)), _lab(slots=32784), 1024,
                   32769)
    assert rc == 0 and ds.PATHS[pl.path] == "local"
    # Flags force the other paths; k <= 0 is dense.
    kv, lab = _mha(32, 32, 4160), _lab(slots=4160, **int4)
    rc, pl = _plan(lib, kv, lab, 256, 4097, flags=ds.DECODE_UNFUSED)
    assert rc == 0 and ds.PATHS[pl.path] == "local"
    rc, pl = _plan(lib, kv, lab, 256, 4097, flags=ds.DECODE_STREAM | ds.DECODE_APPEND)
    assert rc == 0 and ds.PATHS[pl.path] == "stream" and pl.kernels >= 4
    rc, pl = _plan(lib, kv, None, 0, 4097)
    assert rc == 0 and ds.PATHS[pl.path] == "dense" and pl.n_split >= 1
    assert pl.workspace_bytes == lib.ds_decode_attn_workspace_size(ctypes.byref(kv), None, 0, 4097)
    rc, pl = _plan(lib, kv, lab, 256, 4097, n_split=4, flags=ds.DECODE_UNFUSED)
    assert rc == 0 and pl.n_split == 4 and pl.tokens_per_split == 64
    # errors
    assert _plan(lib, kv, lab, 256, 5000)[0] == -1
    assert _plan(lib, _kv(d_v=64), lab, 256, 100)[0] == -2
    assert lib.ds_decode_attn_plan(ctypes.byref(kv), ctypes.byref(lab), 256, 4097, None, None) == -1


def test_label_calls_validate_before_launch(lib):
    kv = _kv()
    P = ctypes.c_void_p
    lab = _lab()
    assert lib.ds_label_build(ctypes.byref(kv), P(FAKE), P(FAKE), ctypes.byref(lab), 5, 3, None) == -1
    assert lib.ds_label_build(ctypes.byref(kv), P(FAKE), P(FAKE), ctypes.byref(lab), 0, 1001, None) == -1
    assert lib.ds_label_build(ctypes.byref(kv), None, P(FAKE), ctypes.byref(lab), 0, 10, None) == -1
    assert lib.ds_label_build(ctypes.byref(kv), P(FAKE + 2), P(FAKE), ctypes.byref(lab), 0, 10, None) == -4
    assert lib.ds_label_build(ctypes.byref(kv), P(FAKE), P(FAKE), ctypes.byref(lab), 7, 7, None) == 0
    # label calls read only the K-side fields of the descriptor
    kq = _kv(n_q_heads=1, d_v=32, d_q=7)
    assert lib.ds_label_build(ctypes.byref(kq), P(FAKE), P(FAKE), ctypes.byref(lab), 7, 7, None) == 0
    bad = _lab(dtype=ds.LABEL_INT4, r=3, scales=FAKE)
    assert lib.ds_label_append(ctypes.byref(kv), P(FAKE), P(FAKE), ctypes.byref(bad), P(FAKE), None) == -3
    assert lib.ds_label_append(ctypes.byref(kv), P(FAKE), P(FAKE), ctypes.byref(lab), None, None) == -1


def test_product_has_no_fallback():
    """The binding refuses to run without the HIP library (no CPU path)."""
    import importlib
    mod = importlib.import_module("sparse_attention_decode_ds_amd")
    src = open(mod.__file__).read()
    assert "oracle" not in src.replace("there is no fallback", "")
    assert "import oracle" not in src and "numpy" not in src


def test_check_tables_host_logic():
    """The binding's index-table check (CPU tensors, no GPU needed)."""
    import torch
    chan = torch.tensor([[0, 3, 7], [1, 2, 31]], dtype=torch.int32)
    ds.check_tables(chan, d_k=32, r=3, n_kv_heads=2)
    keep = torch.arange(64, dtype=torch.int32).reshape(2, 32) * 2
    ds.check_tables(chan, d_k=32, r=3, keep=keep, d_q=128, n_kv_heads=2)
    bad = [
        dict(chan=torch.tensor([[0, 3, 32], [1, 2, 3]], dtype=torch.int32), d_k=32),   # column >= d_k
        dict(chan=torch.tensor([[0, -1, 5], [1, 2, 3]], dtype=torch.int32), d_k=32),   # negative
        dict(chan=torch.tensor([[4, 3, 4], [1, 2, 3]], dtype=torch.int32), d_k=32),    # repeated
        dict(chan=chan, d_k=32, r=4),                                                 # wrong r
        dict(chan=chan, d_k=32, n_kv_heads=3),                                        # wrong heads
        dict(chan=chan, d_k=32, keep=keep, d_q=100),                                  # keep >= d_q
        dict(chan=chan, d_k=32, keep=keep[:, :16], d_q=128),                          # keep width
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            ds.check_tables(**kw)


def test_dense_append_step_checks_the_channel_table():
    """A dense step (k <= 0) with DECODE_APPEND still appends the current
    token's label, which reads the heavy-channel table: validate_tables must
    reject a bad table there before anything reaches the library (CPU
    tensors; the check raises before any call)."""
    import torch
    B, Hq, Hkv, cap, D = 1, 2, 2, 64, 128
    q = torch.zeros((B, Hq, D), dtype=torch.float16)
    K = torch.zeros((B, Hkv, cap, D), dtype=torch.float16)
    bad = torch.tensor([[0, 200], [1, 2]], dtype=torch.int32)   # column 200 >= d_k
    lab = ds.LabelCache(2, ds.LABEL_F16, cap, torch.zeros((B, Hkv, cap, 2), dtype=torch.float16),
                        None)
    seq = torch.full((B,), 10, dtype=torch.int32)
    with pytest.raises(ValueError):
        ds.decode_attn(q, K, K, seq, 10, 0, 0.088, chan=bad, labels=lab,
                       flags=ds.DECODE_APPEND, validate_tables=True)


@pytest.mark.parametrize("G,max_seq,path", [
    (1, 6144, "fused"), (1, 6145, "local"),        # 256 threads x 24 scores
    (7, 16384, "fused"), (7, 16385, "local"),      # 1024 threads x 16 scores
    (2, 12288, "fused"), (8, 4096, "fused"),
])
def test_one_kernel_path_bounds(lib, G, max_seq, path):
    """The one-kernel paths hold rows up to their register budget: 6144
    tokens for a single query head, 16384 for a query group."""
    Hkv = 4
    cap = (max_seq + 63) // 64 * 64
    kv = _kv(batch=8, n_q_heads=G * Hkv, n_kv_heads=Hkv, capacity=cap,
             k_stride=(Hkv * cap * 128, cap * 128, 128), v_stride=(Hkv * cap * 128, cap * 128, 128))
    rc, pl = _plan(lib, kv, _lab(slots=cap), 256, max_seq)
    assert rc == 0 and ds.PATHS[pl.path] == path
    if path == "fused":
        assert pl.kernels == 1 and pl.n_split == 1
    # k beyond the LDS token list (2048) leaves the one-kernel path
    rc, pl = _plan(lib, kv, _lab(slots=cap), 2049, max_seq)
    assert rc == 0 and ds.PATHS[pl.path] != "fused"


def test_calibration_rejects_a_paged_pool(lib):
    kv = _kv(page_size=16, capacity=1024, max_pages=64, n_pages=50, page_table=FAKE,
             k_stride=(4 * 16 * 128, 16 * 128, 128))
    assert lib.ds_calibrate_workspace_size(ctypes.byref(kv), 64, 0) == 0
    P = ctypes.c_void_p
    rc = lib.ds_calibrate_channels(ctypes.byref(kv), P(FAKE), 64, None, 0, None, 0, 8, P(FAKE),
                                   None, P(FAKE), 1 << 20, None)
    assert rc == -1


def test_calibrate_workspace_and_argument_errors(lib):
    """Host-side checks of ds_calibrate_channels: every case returns before
    anything is enqueued, so no GPU is needed."""
    P = ctypes.c_void_p
    kv = _kv()
    need = lib.ds_calibrate_workspace_size(ctypes.byref(kv), 900, 4)
    assert need >= 2 * 4 * 128 * 4 * 2 and need % 4 == 0
    assert lib.ds_calibrate_workspace_size(ctypes.byref(kv), 0, 0) == 256
    assert lib.ds_calibrate_workspace_size(ctypes.byref(kv), 0, 4) > 256
    assert lib.ds_calibrate_workspace_size(ctypes.byref(kv), 1001, 4) == 0
    assert lib.ds_calibrate_workspace_size(ctypes.byref(kv), 900, -1) == 0
    assert lib.ds_calibrate_workspace_size(ctypes.byref(_kv(n_q_heads=30)), 900, 4) == 0
    assert lib.ds_calibrate_workspace_size(ctypes.byref(_kv(d_k=12)), 10, 0) == 0

    def call(kv=kv, K=FAKE, n_tok=900, q=FAKE, n_win=4, keep=None, crit=2, r=16, chan=FAKE,
             ws=FAKE, ws_bytes=need):
        return lib.ds_calibrate_channels(ctypes.byref(kv), P(K), n_tok, P(q), n_win,
                                         P(keep) if keep else None, crit, r, P(chan), None,
                                         P(ws) if ws else None, ws_bytes, None)

    assert call(r=0) == -1
    assert call(r=129) == -1
    assert call(crit=3) == -1
    assert call(crit=-1) == -1
    assert call(n_tok=1001) == -1
    assert call(n_tok=-1) == -1
    assert call(n_win=-1) == -1
    assert call(chan=0) == -1
    assert call(q=0) == -1
    assert call(K=0) == -1
    assert call(K=FAKE + 8) == -4
    assert call(ws=0) == -5
    assert call(ws_bytes=need - 4) == -5
    assert call(kv=_kv(n_q_heads=30)) == -2
    assert call(kv=_kv(d_q=64)) == -2  # no keep table and d_k > d_q
    assert call(kv=_kv(d_k=12)) == -2
    assert call(kv=_kv(k_stride=(4 * 1000 * 128, 1000 * 128, 132))) == -4


def test_channel_overlap_host_logic():
    a = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 7]], dtype=torch.int32)
    b = torch.tensor([[3, 2, 9, 8], [4, 5, 6, 7]], dtype=torch.int32)
    assert ds.channel_overlap(a, b) == [0.5, 1.0]
    assert ds.channel_overlap(a, a) == [1.0, 1.0]
    assert ds.channel_overlap([[1, 2]], [[3, 4]]) == [0.0]
    with pytest.raises(ValueError):
        ds.channel_overlap(a, b[:, :2])


def test_channel_overlap_matches_the_oracle(lib):
    """ds_channel_overlap against the oracle on seeded tables: distinct
    sorted channels as calibration writes them, and rows with repeats."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(5)
    for H, r, d in [(1, 1, 4), (4, 8, 16), (32, 16, 128), (7, 32, 40)]:
        a = np.sort(np.stack([rng.choice(d, r, replace=False) for _ in range(H)]), axis=1)
        b = np.sort(np.stack([rng.choice(d, r, replace=False) for _ in range(H)]), axis=1)
        c = rng.integers(0, d, size=(H, r))  # repeats allowed
        for x, y in [(a, b), (a, a), (a, c), (c, b)]:
            got = ds.channel_overlap(torch.from_numpy(x.astype(np.int32)),
                                     torch.from_numpy(y.astype(np.int32)))
            ref = oracle.channel_overlap(x, y)
            assert np.array_equal(np.float32(got), np.float32(ref)), (H, r, got, ref)
    out = (ctypes.c_float * 2)()
    ok = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    assert lib.ds_channel_overlap(None, ok, 2, 2, out) == -1
    assert lib.ds_channel_overlap(ok, ok, 0, 2, out) == -1
    assert lib.ds_channel_overlap(ok, ok, 2, 0, out) == -1
    assert lib.ds_channel_overlap(ok, ok, 2, 2, None) == -1
    assert lib.ds_channel_overlap(ok, ok, 2, 2, out) == 0 and list(out) == [1.0, 1.0]
    bad = (ctypes.c_int32 * 4)(1, 2, 3, 4096)
    assert lib.ds_channel_overlap(ok, bad, 2, 2, out) == -1
    neg = (ctypes.c_int32 * 4)(1, -2, 3, 4)
    assert lib.ds_channel_overlap(neg, ok, 2, 2, out) == -1


def test_sparse_decode_threshold_policy(lib):
    """[DS] "use in SGLang": Double Sparsity decodes a batch only when its
    longest sequence reaches the threshold and its shortest reaches k."""
    en = lib.ds_sparse_decode_enabled
    assert en(4096, 4096, 256, 0) == 1
    assert en(4096, 300, 256, 0) == 1
    assert en(4096, 255, 256, 0) == 0      # a sequence shorter than k
    assert en(4095, 4095, 256, 4096) == 0  # longest below the threshold
    assert en(4096, 1000, 256, 4096) == 1
    assert en(4096, 4096, 0, 0) == 0       # k <= 0 is dense
    assert ds.sparse_decode_enabled(8192, 8192, 256, 8192) is True


def test_calibrate_binding_rejects_a_bad_window():
    K = torch.zeros((2, 4, 16, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        ds.calibrate_channels(K, 8, "qk", qwin=torch.zeros((2, 3, 4, 128), dtype=torch.float32))
    with pytest.raises(ValueError):
        ds.calibrate_channels(K, 8, "qk", qwin=torch.zeros((3, 3, 4, 128), dtype=torch.float16))


def test_check_pages_reads_only_the_pages_in_use():
    # 2 batch rows, 4 logical pages of 16 tokens each, a pool of 6 pages
    table = torch.tensor([[5, 0, 9, -1], [1, 2, 3, 4]], dtype=torch.int32)
    pages = ds.Pages(table, 16)
    ds.check_pages(pages, 6, 32)           # tokens 0..31: pages 0 and 1 of each row
    with pytest.raises(ValueError, match="outside"):
        ds.check_pages(pages, 6, 33)       # page 2 of row 0 is 9 >= 6
    with pytest.raises(ValueError, match="outside"):
        ds.check_pages(ds.Pages(torch.tensor([[0, -1]], dtype=torch.int32), 16), 2, 17)
    with pytest.raises(ValueError, match="needed"):
        ds.check_pages(pages, 16, 65)      # 5 pages per row, the table has 4
    ds.check_pages(pages, 6, 0)            # no token: nothing read
