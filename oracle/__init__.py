"""CPU oracle for Double Sparsity decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  It shares no code
with the HIP path.

The arithmetic lives in ``ds_oracle.c`` (plain C, fp64 from fp16 inputs, the
4-bit quantiser in IEEE fp32); this module only builds that file with gcc and
marshals numpy arrays into it.  Pages (cited by title and section):

* "Double Sparsity" article (joto.ai blog archive 2025060420469), sections
  "offline calibration" (label cache, 4-bit labels) and "online forward
  computation" (gather, approximate score, top-k + exact attention);
* LeanK article (aitangshan.cn news 1293675), section 1.1 (channel importance
  from the query-key product) -- the calibration criteria; section 2.2 (static
  K-channel mask) -- the ``keep`` table;
* grouped-query attention article (trdm.cn news 80600), section 4 -- groups of
  query heads sharing a K/V head.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ds_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build_library(force: bool = True) -> str:
    """Compile ds_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_library(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_float_to_half_rn.argtypes = [ctypes.c_float]
        lib.oracle_float_to_half_rn.restype = ctypes.c_uint16
        lib.oracle_label_int4_row.argtypes = [P, P, I, P, P]
        lib.oracle_label_int4_row.restype = I
        lib.oracle_topk.argtypes = [P, I, I, P]
        lib.oracle_topk.restype = I
        lib.oracle_label_build.argtypes = [P, P, P, P, P, P, I, I]
        lib.oracle_label_build.restype = I
        lib.oracle_label_append.argtypes = [P, P, P, P, P, P, P]
        lib.oracle_label_append.restype = I
        lib.oracle_decode.argtypes = [P, P, P, P, P, P, P, P, P, P, I, ctypes.c_double, P, I,
                                      P, P, I, P, ctypes.c_int64, I]
        lib.oracle_decode.restype = I
        lib.oracle_attend_sets.argtypes = [P, P, P, P, P, P, I, ctypes.c_double, P, I, P, I]
        lib.oracle_attend_sets.restype = I
        lib.oracle_calibrate.argtypes = [P, P, I, I, I, I, P, I, I, I, P, I, I, P, P]
        lib.oracle_calibrate.restype = I
        lib.oracle_channel_overlap.argtypes = [P, P, I, I, P]
        lib.oracle_channel_overlap.restype = I
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d_q", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("ks", ctypes.c_int64 * 3), ("vs", ctypes.c_int64 * 3),
                ("r", ctypes.c_int32), ("is_int4", ctypes.c_int32), ("slots", ctypes.c_int32)]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    """fp16 array viewed as its bit pattern (uint16), C-contiguous."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


def _kv(a):
    """K/V cache as uint16 with unit channel stride (other strides are kept)."""
    if a.strides[-1] != a.itemsize:
        a = np.ascontiguousarray(a)
    return a if a.dtype == np.uint16 else a.view(np.uint16)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


@dataclass
class Labels:
    """Label cache arrays; ``f16`` for fp16 labels, ``codes``+``scales`` for int4."""
    r: int
    is_int4: bool
    slots: int
    f16: np.ndarray | None = None      # uint16 [B][Hkv][slots][r]
    codes: np.ndarray | None = None    # uint8  [B][Hkv][slots][r/2]
    scales: np.ndarray | None = None   # uint16 [B][Hkv][slots]

    @staticmethod
    def empty(B, Hkv, slots, r, is_int4):
        if is_int4:
            return Labels(r, True, slots, codes=np.zeros((B, Hkv, slots, r // 2), np.uint8),
                          scales=np.zeros((B, Hkv, slots), np.uint16))
        return Labels(r, False, slots, f16=np.zeros((B, Hkv, slots, r), np.uint16))


def _shape(K, V, Hq, d_q, lab: Labels | None):
    B, Hkv, cap, d_k = K.shape
    d_v = V.shape[3]
    sh = _Shape()
    sh.B, sh.Hq, sh.Hkv, sh.d_q, sh.d_k, sh.d_v, sh.cap = B, Hq, Hkv, d_q, d_k, d_v, cap
    for i in range(3):
        sh.ks[i] = K.strides[i] // 2
        sh.vs[i] = V.strides[i] // 2
    if lab is not None:
        sh.r, sh.is_int4, sh.slots = lab.r, int(lab.is_int4), lab.slots
    else:
        sh.r, sh.is_int4, sh.slots = 0, 0, cap
    return sh


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(bits)


def float_to_half_rn(x: float) -> int:
    return _load().oracle_float_to_half_rn(x)


def label_int4_row(krow, chan):
    """Quantise one K row's heavy channels; returns (codes uint8[r/2], scale bits)."""
    krow = _u16(krow)
    chan = _i32(chan)
    r = len(chan)
    codes = np.zeros(r // 2, np.uint8)
    scale = np.zeros(1, np.uint16)
    rc = _load().oracle_label_int4_row(_ptr(krow), _ptr(chan), r, _ptr(codes), _ptr(scale))
    if rc:
        raise ValueError("oracle_label_int4_row failed: %d" % rc)
    return codes, int(scale[0])


def topk(scores, k):
    s = np.ascontiguousarray(scores, dtype=np.float64)
    out = np.zeros(max(len(s), 1), np.int32)
    n = _load().oracle_topk(_ptr(s), len(s), int(k), _ptr(out))
    if n < 0:
        raise MemoryError
    return out[:n].copy()


def label_build(K, chan, lab: Labels, t_begin, t_end):
    K = _kv(K)
    chan = _i32(chan)
    sh = _shape(K, K, 1, K.shape[3], lab)
    rc = _load().oracle_label_build(ctypes.byref(sh), _ptr(K), _ptr(chan), _ptr(lab.f16),
                                    _ptr(lab.codes), _ptr(lab.scales), int(t_begin), int(t_end))
    if rc:
        raise ValueError("oracle_label_build failed: %d" % rc)
    return lab


def label_append(K, chan, lab: Labels, pos):
    K = _kv(K)
    chan = _i32(chan)
    pos = _i32(pos)
    sh = _shape(K, K, 1, K.shape[3], lab)
    rc = _load().oracle_label_append(ctypes.byref(sh), _ptr(K), _ptr(chan), _ptr(lab.f16),
                                     _ptr(lab.codes), _ptr(lab.scales), _ptr(pos))
    if rc:
        raise ValueError("oracle_label_append failed: %d" % rc)
    return lab


def all_rows(B, Hkv):
    return [(b, g) for b in range(B) for g in range(Hkv)]


def decode(q, K, V, seq_lens, k, sm_scale, chan=None, lab: Labels | None = None, keep=None,
           rows=None, want_scores=False, n_threads=0):
    """One decode step.  Returns dict(out fp64 [B][Hq][d_v], topk int32 [B][Hkv][k_cap],
    scores fp64 [B][Hkv][cap] or None).  Only ``rows`` (list of (b, g)) are computed."""
    q = _u16(q)
    K = _kv(K)
    V = _kv(V)
    B, Hq, d_q = q.shape
    Hkv, cap = K.shape[1], K.shape[2]
    sh = _shape(K, V, Hq, d_q, lab if k > 0 else None)
    if rows is None:
        rows = all_rows(B, Hkv)
    rows_a = np.ascontiguousarray(np.array(rows, np.int32).reshape(-1, 2))
    seq = _i32(seq_lens)
    k_cap = max(int(k), 1) if k > 0 else 1
    out = np.zeros((B, Hq, V.shape[3]), np.float64)
    tk = np.full((B, Hkv, k_cap), -1, np.int32)
    sc = np.zeros((B, Hkv, cap), np.float64) if (want_scores and k > 0) else None
    use_lab = k > 0
    keep_a, chan_a = _i32(keep), _i32(chan)  # held here: the C call reads them
    rc = _load().oracle_decode(
        ctypes.byref(sh), _ptr(q), _ptr(K), _ptr(V), _ptr(seq), _ptr(keep_a),
        _ptr(chan_a) if use_lab else None,
        _ptr(lab.f16) if use_lab else None, _ptr(lab.codes) if use_lab else None,
        _ptr(lab.scales) if use_lab else None, int(k), float(sm_scale), _ptr(rows_a),
        len(rows_a), _ptr(out), _ptr(tk), k_cap, _ptr(sc), cap, int(n_threads))
    if rc:
        raise ValueError("oracle_decode failed: %d" % rc)
    return {"out": out, "topk": tk if k > 0 else None, "scores": sc}


def attend_sets(q, K, V, sets, sm_scale, keep=None, rows=None, n_threads=0):
    """Attention over given token sets [B][Hkv][k_cap] (entries < 0 ignored)."""
    q = _u16(q)
    K = _kv(K)
    V = _kv(V)
    B, Hq, d_q = q.shape
    Hkv = K.shape[1]
    sh = _shape(K, V, Hq, d_q, None)
    if rows is None:
        rows = all_rows(B, Hkv)
    rows_a = np.ascontiguousarray(np.array(rows, np.int32).reshape(-1, 2))
    sets = _i32(sets)
    out = np.zeros((B, Hq, V.shape[3]), np.float64)
    keep_a = _i32(keep)  # held here: the C call reads it
    rc = _load().oracle_attend_sets(ctypes.byref(sh), _ptr(q), _ptr(K), _ptr(V), _ptr(keep_a),
                                    _ptr(sets), sets.shape[2], float(sm_scale), _ptr(rows_a),
                                    len(rows_a), _ptr(out), int(n_threads))
    if rc:
        raise ValueError("oracle_attend_sets failed: %d" % rc)
    return out


def gather_pages(pool, table, page_size: int):
    """The rows of a paged K/V pool as a contiguous cache: out[b][g][t] =
    pool[table[b][t // page_size]][g][t % page_size] ("Double Sparsity",
    section "use in SGLang": the K/V cache is a pool of token slots shared by
    the sequences, and a table maps each sequence's tokens to slots).  pool:
    [n_pages][H_kv][page_size][d]; table: int [B][max_pages]; entries < 0
    (pages not in use) give zero rows.  Returns [B][H_kv][max_pages *
    page_size][d], the layout every other oracle function reads."""
    pool = np.asarray(pool)
    table = np.asarray(table, dtype=np.int64)
    B, max_pages = table.shape
    n_pages, H, P, d = pool.shape
    assert P == page_size
    out = np.zeros((B, H, max_pages * P, d), dtype=pool.dtype)
    for b in range(B):
        for p in range(max_pages):
            pg = int(table[b, p])
            if pg >= 0:
                out[b, :, p * P:(p + 1) * P, :] = pool[pg]
    return out


def max_threads() -> int:
    return _load().oracle_max_threads()


CALIB_K, CALIB_Q, CALIB_QK = 0, 1, 2


def calibrate(K, criterion, r, qwin=None, Hq=None, keep=None, n_tok=None):
    """Heavy channels per KV head from sample tokens ("Double Sparsity",
    section "offline calibration"; LeanK section 1.1).

    K: fp16 [B][Hkv][cap][d_k] (any token/head/batch strides); qwin: fp16
    [B][n_win][Hq][d_q] or None; keep: int32 [Hkv][d_k] or None.  Returns
    (chan int32 [Hkv][r] ascending, norms float64 [Hkv][3][d_k]: K column
    sums of squares, window query sums of squares, criterion score)."""
    Ku = _kv(K)
    B, Hkv, cap, d_k = Ku.shape
    n_tok = cap if n_tok is None else int(n_tok)
    ks = np.array([s // Ku.itemsize for s in Ku.strides[:3]], np.int64)
    if qwin is not None:
        qu = np.ascontiguousarray(_u16(qwin))
        n_win, d_q = qu.shape[1], qu.shape[3]
        Hq = qu.shape[2]
    else:
        qu, n_win, d_q, Hq = None, 0, 0, Hq or Hkv
    keep_a = _i32(keep)
    chan = np.zeros((Hkv, r), np.int32)
    norms = np.zeros((Hkv, 3, d_k), np.float64)
    rc = _load().oracle_calibrate(_ptr(Ku), _ptr(ks), B, Hkv, d_k, n_tok, _ptr(qu), n_win, Hq,
                                  d_q, _ptr(keep_a), int(criterion), int(r), _ptr(chan),
                                  _ptr(norms))
    if rc != 0:
        raise ValueError("oracle_calibrate: status %d" % rc)
    return chan, norms


def channel_overlap(a, b):
    """Per KV head, the share of a's distinct channels that b also holds
    ("Double Sparsity", section "offline calibration": offline against online
    outlier channels).  a, b: int [Hkv][r].  Returns float64 [Hkv]."""
    aa = np.ascontiguousarray(np.asarray(a), np.int32)
    bb = np.ascontiguousarray(np.asarray(b), np.int32)
    if aa.ndim != 2 or aa.shape != bb.shape:
        raise ValueError("oracle.channel_overlap: two [Hkv][r] tables of one shape expected")
    out = np.zeros(aa.shape[0], np.float64)
    rc = _load().oracle_channel_overlap(_ptr(aa), _ptr(bb), aa.shape[0], aa.shape[1], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_channel_overlap: status %d" % rc)
    return out
