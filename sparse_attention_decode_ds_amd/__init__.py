"""Python binding of libds.so: Double Sparsity decode attention on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``libds.so`` (see ``include/ds.h`` for the contract); PyTorch only provides
device memory and the current stream.  If the library is missing, every call
raises: there is no fallback path.

Pages (cited by title and section): "Double Sparsity" article (joto.ai blog
archive 2025060420469), sections "offline calibration" (label cache) and
"online forward computation" (steps 1-3); LeanK article (aitangshan.cn news
1293675) section 2.2 (the ``keep`` table); grouped-query attention article
(trdm.cn news 80600) section 4.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libds.so")

DS_OK = 0
STATUS = {0: "DS_OK", -1: "DS_ERR_ARG", -2: "DS_ERR_SHAPE", -3: "DS_ERR_DTYPE",
          -4: "DS_ERR_ALIGN", -5: "DS_ERR_WORKSPACE", -6: "DS_ERR_HIP"}
LABEL_F16 = 0
LABEL_INT4 = 1
STAGE_COUNT = 5
STAGES = ("append", "score", "select", "attn", "combine")
DECODE_APPEND = 1
DECODE_VALIDATE_ONLY = 2
DECODE_UNFUSED = 4
DECODE_STREAM = 8
NOALLOC_SCRATCH_BYTES = 128 << 20  # DS_NOALLOC_SCRATCH_BYTES
PATHS = ("dense", "fused", "local", "stream")
EXPORTS = ("ds_label_build", "ds_label_append", "ds_decode_attn_workspace_size",
           "ds_decode_attn_plan", "ds_decode_attn", "ds_decode_attn_noalloc",
           "ds_calibrate_workspace_size",
           "ds_calibrate_channels", "ds_channel_overlap", "ds_sparse_decode_enabled",
           "ds_status_str",
           "ds_abi_version")


class DsError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(code, "?"), code))


class KVDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("d_q", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
                ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("n_pages", ctypes.c_int32), ("heads", ctypes.c_void_p)]


class LabelDesc(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("dtype", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("n_split", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("stage_events", ctypes.c_void_p)]


class DecodePlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("n_split", ctypes.c_int32),
                ("tokens_per_split", ctypes.c_int32), ("kernels", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None


# DS_ABI_VERSION of include/ds.h this binding's structures follow
ABI_VERSION = 4


def load() -> ctypes.CDLL:
    """Load libds.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libds.so is not built (run __graft_entry__.build()); "
                              "there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        lib.ds_label_build.argtypes = [P, P, P, P, I32, I32, P]
        lib.ds_label_build.restype = ctypes.c_int
        lib.ds_label_append.argtypes = [P, P, P, P, P, P]
        lib.ds_label_append.restype = ctypes.c_int
        lib.ds_decode_attn_workspace_size.argtypes = [P, P, I32, I32]
        lib.ds_decode_attn_workspace_size.restype = ctypes.c_size_t
        lib.ds_decode_attn_plan.argtypes = [P, P, I32, I32, P, P]
        lib.ds_decode_attn_plan.restype = ctypes.c_int
        lib.ds_decode_attn.argtypes = [P, P, P, P, P, I32, P, P, P, I32, ctypes.c_float, P, P, P,
                                       ctypes.c_size_t, P, P]
        lib.ds_decode_attn.restype = ctypes.c_int
        lib.ds_decode_attn_noalloc.argtypes = [P, P, P, P, P, I32, P, P, P, I32, ctypes.c_float,
                                               P, P, P, P]
        lib.ds_decode_attn_noalloc.restype = ctypes.c_int
        lib.ds_channel_overlap.argtypes = [P, P, I32, I32, P]
        lib.ds_channel_overlap.restype = ctypes.c_int
        lib.ds_calibrate_workspace_size.argtypes = [P, I32, I32]
        lib.ds_calibrate_workspace_size.restype = ctypes.c_size_t
        lib.ds_calibrate_channels.argtypes = [P, P, I32, P, I32, P, I32, I32, P, P, P,
                                              ctypes.c_size_t, P]
        lib.ds_calibrate_channels.restype = ctypes.c_int
        lib.ds_sparse_decode_enabled.argtypes = [I32, I32, I32, I32]
        lib.ds_sparse_decode_enabled.restype = I32
        lib.ds_status_str.argtypes = [ctypes.c_int]
        lib.ds_status_str.restype = ctypes.c_char_p
        lib.ds_abi_version.argtypes = []
        lib.ds_abi_version.restype = I32
        if lib.ds_abi_version() != ABI_VERSION:
            raise ImportError("libds.so has ABI %d, this binding expects %d (rebuild)" %
                              (lib.ds_abi_version(), ABI_VERSION))
        _lib = lib
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(0)


def _check(fn, code):
    if code != DS_OK:
        raise DsError(fn, code)


@dataclass
class Pages:
    """A paged K/V pool: ``table`` int32 [batch][max_pages] on the device
    (physical page of each logical page of a batch row); the K and V tensors
    are then pools [n_pages][H_kv][page_size][d]."""
    table: torch.Tensor
    page_size: int


@dataclass
class HeadLayout:
    """LeanK cache whose KV heads keep different numbers of K columns (LeanK
    section 2.2; a head with none is fully pruned and stores no V either,
    section 4.4).  ``table``: int64 [H_kv][3] on the device (k_cols, k_off,
    v_off); every batch row (or page) of ``tokens`` token slots holds the
    heads' K blocks back to back in ``k_row`` halves (rows of k_cols columns)
    and the stored heads' V blocks in ``v_row`` halves (rows of d_v)."""
    table: torch.Tensor
    k_cols: list
    tokens: int
    k_row: int
    v_row: int
    d_v: int = 128

    @staticmethod
    def packed(k_cols, tokens: int, d_v: int = 128, device="cuda"):
        k_cols = [int(c) for c in k_cols]
        if any(c < 0 or c % 8 or c > 128 for c in k_cols):
            raise ValueError("k_cols: multiples of 8 in [0, 128]")
        rows, ko, vo = [], 0, 0
        for c in k_cols:
            rows.append((c, ko, vo if c > 0 else 0))
            ko += tokens * c
            vo += tokens * d_v if c > 0 else 0
        t = torch.tensor(rows, dtype=torch.int64, device=device)
        return HeadLayout(t, k_cols, tokens, ko, vo, d_v)

    def head_k(self, Kbuf, g):
        """Head g's K [B][tokens][k_cols] (a view of the batch-row buffer)."""
        c = self.k_cols[g]
        off = int(self.table[g, 1])
        return Kbuf[:, off:off + self.tokens * c].view(Kbuf.shape[0], self.tokens, c)

    def head_v(self, Vbuf, g):
        off = int(self.table[g, 2])
        return Vbuf[:, off:off + self.tokens * self.d_v].view(Vbuf.shape[0], self.tokens, self.d_v)


def kv_desc(K, V, n_q_heads: int, d_q: int | None = None, pages: Pages | None = None,
            heads: HeadLayout | None = None) -> KVDesc:
    """Describe K [B][H_kv][cap][d_k] and V [B][H_kv][cap][d_v] (fp16, unit
    channel stride), or with ``pages`` the pools K [n_pages][H_kv][P][d_k] and
    V [n_pages][H_kv][P][d_v].  With ``heads``, K and V are the per-head
    buffers [B or n_pages][k_row] and [..][v_row] of that layout."""
    if heads is not None:
        d = KVDesc()
        d0 = K.shape[0]
        Hkv = len(heads.k_cols)
        d_k = max(max(heads.k_cols), 8)
        if pages is not None:
            B, max_pages = pages.table.shape
            d.batch, d.capacity = B, max_pages * pages.page_size
            d.page_size, d.page_table = pages.page_size, pages.table.data_ptr()
            d.max_pages, d.n_pages = max_pages, d0
        else:
            d.batch, d.capacity = d0, heads.tokens
        d.n_q_heads, d.n_kv_heads = n_q_heads, Hkv
        d.d_q = d_k if d_q is None else d_q
        d.d_k, d.d_v = d_k, heads.d_v
        d.k_stride[0], d.k_stride[1], d.k_stride[2] = K.stride(0), 0, d_k
        d.v_stride[0], d.v_stride[1], d.v_stride[2] = V.stride(0), 0, heads.d_v
        d.heads = heads.table.data_ptr()
        return d
    d0, Hkv, d2, d_k = K.shape
    d = KVDesc()
    if pages is not None:
        B, max_pages = pages.table.shape
        d.batch, d.capacity = B, max_pages * pages.page_size
        d.page_size, d.page_table = pages.page_size, pages.table.data_ptr()
        d.max_pages, d.n_pages = max_pages, d0
        if d2 != pages.page_size:
            raise ValueError("pool pages hold %d tokens, page_size is %d" % (d2, pages.page_size))
    else:
        d.batch, d.capacity = d0, d2
    d.n_q_heads, d.n_kv_heads = n_q_heads, Hkv
    d.d_q = d_k if d_q is None else d_q
    d.d_k, d.d_v = d_k, V.shape[3]
    for i in range(3):
        d.k_stride[i] = K.stride(i)
        d.v_stride[i] = V.stride(i)
    return d


@dataclass
class LabelCache:
    """Label-cache storage: fp16 [B][H_kv][slots][r], or int4 codes uint8
    [B][H_kv][slots][r/2] + fp16 scales [B][H_kv][slots]."""
    r: int
    dtype: int
    slots: int
    codes: torch.Tensor
    scales: torch.Tensor | None

    @staticmethod
    def allocate(B, Hkv, capacity, r, int4: bool, device="cuda"):
        slots = (capacity + 63) // 64 * 64
        if int4:
            codes = torch.zeros((B, Hkv, slots, r // 2), dtype=torch.uint8, device=device)
            scales = torch.zeros((B, Hkv, slots), dtype=torch.float16, device=device)
            return LabelCache(r, LABEL_INT4, slots, codes, scales)
        codes = torch.zeros((B, Hkv, slots, r), dtype=torch.float16, device=device)
        return LabelCache(r, LABEL_F16, slots, codes, None)

    def desc(self) -> LabelDesc:
        d = LabelDesc()
        d.r, d.dtype, d.slots, d.reserved0 = self.r, self.dtype, self.slots, 0
        d.codes = self.codes.data_ptr()
        d.scales = self.scales.data_ptr() if self.scales is not None else None
        return d


def check_pages(pages: Pages, n_pages: int, max_seq_len: int):
    """Check the page-table entries a call reads (the pages of tokens below
    max_seq_len of every batch row) against the pool of n_pages pages; the C
    ABI does not read the table on the host.  Copies the entries to the host."""
    P = pages.page_size
    used = (max(max_seq_len, 0) + P - 1) // P
    if used > pages.table.shape[1]:
        raise ValueError("page table: %d pages per row needed, %d given" % (used, pages.table.shape[1]))
    if used == 0:
        return
    t = pages.table[:, :used].to("cpu")
    if int(t.min()) < 0 or int(t.max()) >= n_pages:
        raise ValueError("page table: entries outside [0, %d)" % n_pages)


def check_tables(chan, d_k: int, r: int | None = None, keep=None, d_q: int | None = None,
                 n_kv_heads: int | None = None, head_cols=None):
    """Check the contents of the index tables, which the C ABI does not read
    on the host: chan [H_kv][r] holds distinct stored-K columns in [0, d_k)
    per KV head (with ``head_cols``, a per-head layout: in [0, head_cols[g])
    and not read for a fully pruned head); keep [H_kv][d_k] holds query
    channels in [0, d_q).  Copies the tables to the host (a synchronisation),
    so it suits set-up time, not every decode step.  Raises ValueError."""
    if chan is not None:
        c = chan.detach().to("cpu", torch.int64)
        if c.dim() != 2 or (n_kv_heads is not None and c.shape[0] != n_kv_heads) or (
                r is not None and c.shape[1] != r):
            raise ValueError("chan: expected shape [n_kv_heads][r], got %s" % (tuple(c.shape),))
        if head_cols is not None:
            live = [g for g, n in enumerate(head_cols) if n > 0]
            for g in live:
                if int(c[g].min()) < 0 or int(c[g].max()) >= head_cols[g]:
                    raise ValueError("chan: head %d column outside [0, %d)" % (g, head_cols[g]))
            c = c[live] if live else c[:0]
        elif c.numel() and (int(c.min()) < 0 or int(c.max()) >= d_k):
            raise ValueError("chan: column outside [0, %d)" % d_k)
        if c.shape[1] > 1 and bool((c.sort(dim=1).values.diff(dim=1) == 0).any()):
            raise ValueError("chan: repeated column in a KV head's table")
    if keep is not None:
        k = keep.detach().to("cpu", torch.int64)
        if k.dim() != 2 or k.shape[1] != d_k or (n_kv_heads is not None and k.shape[0] != n_kv_heads):
            raise ValueError("keep: expected shape [n_kv_heads][%d], got %s" % (d_k, tuple(k.shape)))
        hi = d_q if d_q is not None else d_k
        if k.numel() and (int(k.min()) < 0 or int(k.max()) >= hi):
            raise ValueError("keep: query channel outside [0, %d)" % hi)


def label_build(K, chan, labels: LabelCache, t_begin: int, t_end: int, stream=None,
                pages: Pages | None = None, heads: HeadLayout | None = None):
    kv = kv_desc(K, K, 1, pages=pages, heads=heads)
    lab = labels.desc()
    _check("ds_label_build", load().ds_label_build(
        ctypes.byref(kv), _p(K), _p(chan), ctypes.byref(lab), int(t_begin), int(t_end),
        _stream(stream)))


def label_append(K, chan, labels: LabelCache, pos, stream=None, pages: Pages | None = None,
                 heads: HeadLayout | None = None):
    kv = kv_desc(K, K, 1, pages=pages, heads=heads)
    lab = labels.desc()
    _check("ds_label_append", load().ds_label_append(
        ctypes.byref(kv), _p(K), _p(chan), ctypes.byref(lab), _p(pos), _stream(stream)))


CALIB_K, CALIB_Q, CALIB_QK = 0, 1, 2
CALIB_CRITERIA = {"k": CALIB_K, "q": CALIB_Q, "qk": CALIB_QK}


def calibrate_workspace_size(K, n_tok: int, qwin=None) -> int:
    n_win, Hq, d_q = (qwin.shape[1], qwin.shape[2], qwin.shape[3]) if qwin is not None else (
        0, K.shape[1], K.shape[3])
    kv = kv_desc(K, K, Hq, d_q)
    return int(load().ds_calibrate_workspace_size(ctypes.byref(kv), int(n_tok), int(n_win)))


def calibrate_channels(K, r: int, criterion="qk", qwin=None, keep=None, n_tok: int | None = None,
                       norms=None, workspace=None, validate_tables: bool = True, stream=None):
    """Heavy channels per KV head (ds_calibrate_channels; "Double Sparsity",
    section "offline calibration"; LeanK section 1.1).

    K: fp16 cache [B][Hkv][capacity][d_k]; qwin: fp16 [B][n_win][Hq][d_q]
    window queries or None; keep: int32 [Hkv][d_k] or None; criterion "k",
    "q" or "qk".  Returns chan, int32 [Hkv][r] on K's device (ascending
    columns); fills ``norms`` (fp32 [Hkv][3][d_k]) when given."""
    import torch
    crit = CALIB_CRITERIA[criterion] if isinstance(criterion, str) else int(criterion)
    B, Hkv, cap, d_k = K.shape
    n_tok = cap if n_tok is None else int(n_tok)
    if qwin is not None:
        if qwin.dtype != torch.float16 or not qwin.is_contiguous() or qwin.dim() != 4 or \
                qwin.shape[0] != B:
            raise ValueError("qwin: expected a contiguous fp16 [batch][n_win][n_q_heads][d_q] tensor")
        n_win, Hq, d_q = qwin.shape[1], qwin.shape[2], qwin.shape[3]
    else:
        n_win, Hq, d_q = 0, Hkv, d_k
    if validate_tables and keep is not None:
        check_tables(None, d_k, keep=keep, d_q=d_q, n_kv_heads=Hkv)
    kv = kv_desc(K, K, Hq, d_q)
    need = int(load().ds_calibrate_workspace_size(ctypes.byref(kv), n_tok, int(n_win)))
    if need == 0:
        raise DsError("ds_calibrate_workspace_size", -2)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=K.device)
    chan = torch.empty((Hkv, int(r)), dtype=torch.int32, device=K.device)
    _check("ds_calibrate_channels", load().ds_calibrate_channels(
        ctypes.byref(kv), _p(K), n_tok, _p(qwin), int(n_win), _p(keep), crit, int(r), _p(chan),
        _p(norms), _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return chan


def channel_overlap(chan_a, chan_b):
    """Per KV head, the share of heavy channels two tables have in common
    (ds_channel_overlap; "Double Sparsity", section "offline calibration":
    offline-calibrated channels against those found online).  [H_kv][r]
    tables (copied to the host); returns a list of floats."""
    a = chan_a.detach().to("cpu", torch.int32) if hasattr(chan_a, "detach") else torch.as_tensor(chan_a, dtype=torch.int32)
    b = chan_b.detach().to("cpu", torch.int32) if hasattr(chan_b, "detach") else torch.as_tensor(chan_b, dtype=torch.int32)
    if a.dim() != 2 or a.shape != b.shape or a.shape[1] == 0:
        raise ValueError("channel_overlap: two [n_kv_heads][r] tables of one shape expected")
    a, b = a.contiguous(), b.contiguous()
    out = torch.zeros(a.shape[0], dtype=torch.float32)
    _check("ds_channel_overlap", load().ds_channel_overlap(
        _p(a), _p(b), int(a.shape[0]), int(a.shape[1]), _p(out)))
    return out.tolist()


def workspace_size(K, V, n_q_heads, d_q, labels: LabelCache | None, k, max_seq_len,
                   pages: Pages | None = None, heads: HeadLayout | None = None) -> int:
    kv = kv_desc(K, V, n_q_heads, d_q, pages=pages, heads=heads)
    lab = labels.desc() if labels is not None else None
    return int(load().ds_decode_attn_workspace_size(
        ctypes.byref(kv), ctypes.byref(lab) if lab is not None else None, int(k), int(max_seq_len)))


def decode_plan(K, V, n_q_heads, d_q, labels: LabelCache | None, k, max_seq_len,
                n_split: int = 0, flags: int = 0, pages: Pages | None = None,
                heads: HeadLayout | None = None) -> dict:
    """What ds_decode_attn runs for these shapes (ds_decode_attn_plan): the
    path name, attention splits, tokens per split, kernel launches, workspace."""
    kv = kv_desc(K, V, n_q_heads, d_q, pages=pages, heads=heads)
    lab = labels.desc() if labels is not None else None
    opts = DecodeOpts()
    opts.n_split, opts.flags = int(n_split), int(flags)
    pl = DecodePlan()
    _check("ds_decode_attn_plan", load().ds_decode_attn_plan(
        ctypes.byref(kv), ctypes.byref(lab) if lab is not None else None, int(k),
        int(max_seq_len), ctypes.byref(opts), ctypes.byref(pl)))
    return {"path": PATHS[pl.path], "n_split": pl.n_split,
            "tokens_per_split": pl.tokens_per_split, "kernels": pl.kernels, "chunk": pl.chunk,
            "workspace_bytes": int(pl.workspace_bytes)}


def sparse_decode_enabled(max_seq_len: int, min_seq_len: int, k: int, threshold: int) -> bool:
    """The batch policy of the sparse-decode threshold (ds_sparse_decode_enabled)."""
    return bool(load().ds_sparse_decode_enabled(int(max_seq_len), int(min_seq_len), int(k),
                                                int(threshold)))


def decode_attn(q, K, V, seq_lens, max_seq_len: int, k: int, sm_scale: float,
                chan=None, labels: LabelCache | None = None, keep=None, out=None,
                topk_idx=None, workspace=None, n_split: int = 0, flags: int = 0,
                stage_events=None, stream=None, validate_tables: bool = False,
                sparse_decode_threshold: int | None = None, min_seq_len: int | None = None,
                pages: Pages | None = None, heads: HeadLayout | None = None):
    """One decode step (ds_decode_attn).  Returns ``out`` fp16 [B][H_q][d_v].
    ``stage_events``: optional ctypes array of STAGE_COUNT + 1 hipEvent_t.
    ``validate_tables``: check chan and keep first (check_tables; synchronises),
    and with ``pages`` the page-table entries in use (check_pages).
    ``sparse_decode_threshold``: apply the batch policy (needs ``min_seq_len``,
    the host's shortest sequence); a dense step then runs with k = 0 (and
    still appends labels when DECODE_APPEND is set), and ``topk_idx`` is left
    untouched.  ``pages``: K and V are paged pools addressed through its table;
    ``heads``: K and V are the buffers of a per-head LeanK layout."""
    if sparse_decode_threshold is not None and k > 0:
        if min_seq_len is None:
            raise ValueError("sparse_decode_threshold needs min_seq_len")
        if not sparse_decode_enabled(max_seq_len, min_seq_len, k, sparse_decode_threshold):
            k, topk_idx = 0, None
    B, Hq, d_q = q.shape
    if validate_tables:
        # chan is read by the sparse path and by the label append (a dense
        # step with DECODE_APPEND still appends the current token's label)
        uses_chan = k > 0 or bool(flags & DECODE_APPEND)
        if heads is not None:
            check_tables(chan if uses_chan else None, max(heads.k_cols),
                         labels.r if labels is not None else None, keep, d_q,
                         len(heads.k_cols), head_cols=heads.k_cols)
        else:
            check_tables(chan if uses_chan else None, K.shape[3],
                         labels.r if labels is not None else None, keep, d_q, K.shape[1])
    kv = kv_desc(K, V, Hq, d_q, pages=pages, heads=heads)
    if validate_tables and pages is not None:
        check_pages(pages, kv.n_pages, max_seq_len)
    lab = labels.desc() if labels is not None and (k > 0 or flags & DECODE_APPEND) else None
    lib = load()
    need = int(lib.ds_decode_attn_workspace_size(
        ctypes.byref(kv), ctypes.byref(lab) if lab is not None else None, int(k),
        int(max_seq_len)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, kv.d_v), dtype=torch.float16, device=q.device)
    opts = DecodeOpts()
    opts.n_split, opts.flags = int(n_split), int(flags)
    opts.stage_events = ctypes.cast(stage_events, ctypes.c_void_p) if stage_events is not None else None
    _check("ds_decode_attn", lib.ds_decode_attn(
        ctypes.byref(kv), _p(q), _p(K), _p(V), _p(seq_lens), int(max_seq_len), _p(keep), _p(chan),
        ctypes.byref(lab) if lab is not None else None, int(k), float(sm_scale), _p(out),
        _p(topk_idx), _p(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(opts), _stream(stream)))
    return out


def decode_attn_noalloc(q, K, V, seq_lens, max_seq_len: int, k: int, sm_scale: float,
                        chan=None, labels: LabelCache | None = None, keep=None, out=None,
                        topk_idx=None, n_split: int = 0, flags: int = 0, stream=None,
                        pages: Pages | None = None, heads: HeadLayout | None = None):
    """ds_decode_attn_noalloc: the same step as decode_attn with the library's
    per-GPU scratch in place of a workspace (calls on one GPU must not
    overlap).  ``out`` must be given: this call allocates nothing."""
    if out is None:
        raise ValueError("decode_attn_noalloc: pass out (this call allocates nothing)")
    B, Hq, d_q = q.shape
    kv = kv_desc(K, V, Hq, d_q, pages=pages, heads=heads)
    lab = labels.desc() if labels is not None and (k > 0 or flags & DECODE_APPEND) else None
    opts = DecodeOpts()
    opts.n_split, opts.flags = int(n_split), int(flags)
    _check("ds_decode_attn_noalloc", load().ds_decode_attn_noalloc(
        ctypes.byref(kv), _p(q), _p(K), _p(V), _p(seq_lens), int(max_seq_len), _p(keep), _p(chan),
        ctypes.byref(lab) if lab is not None else None, int(k), float(sm_scale), _p(out),
        _p(topk_idx), ctypes.byref(opts), _stream(stream)))
    return out


class HipEvents:
    """Raw hipEvent_t handles (for the stage_events option and kernel timing).
    ``handles`` is a ctypes array of n slots; slots listed in ``skip`` stay NULL."""

    def __init__(self, n: int, skip=()):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        skip = set(skip)
        for i in range(n):
            if i in skip:
                continue
            rc = self._hip.hipEventCreate(ctypes.byref(self.handles, i * ctypes.sizeof(ctypes.c_void_p)))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)

    def slot_address(self, i: int) -> int:
        return ctypes.addressof(self.handles) + i * ctypes.sizeof(ctypes.c_void_p)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def synchronize(self, i: int):
        self._hip.hipEventSynchronize(self.handles[i])

    def close(self):
        for h in self.handles:
            if h:
                self._hip.hipEventDestroy(h)
        self.handles = (ctypes.c_void_p * 0)()
