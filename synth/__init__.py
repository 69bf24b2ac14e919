"""Seeded synthetic inputs for Double Sparsity decode attention.

This module holds no part of the method's arithmetic: it only draws the tensors
(q, K cache, V cache, outlier channels, heavy-channel table, LeanK kept-column
table) that the CPU oracle and the HIP path both consume.  Tensors are drawn
once, on one device; the same bytes then go to both sides.

Generator: counter based.  Element i of stream s under seed z is

    u = splitmix64(z * 0xD1B54A32D192ED03 + s * 0x9E3779B97F4A7C15 + i)

(SplitMix64: Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), whose two 32-bit halves give two uniforms that a
Box-Muller transform (Box & Muller, 1958) turns into one N(0, 1) draw in fp64,
rounded to fp16.  Any element can be regenerated from (seed, stream, index).

Input recipe (per KV head): 8 seeded outlier channels whose K values are scaled
by 8 (the pages describe heavy "outlier" channels that an offline calibration
finds); the heavy-channel table is those channels plus seeded extra distinct
channels up to r, sorted.  q and V stay N(0, 1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MASK64 = (1 << 64) - 1

STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_OUTLIER = 6
STREAM_CHAN = 7
STREAM_KEEP = 8

_SEED_MUL = 0xD1B54A32D192ED03
_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(x: int) -> int:
    """Python int in [0, 2^64) as a two's-complement signed 64-bit value."""
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def splitmix64_int(x: int) -> int:
    """Reference SplitMix64 finaliser on Python ints (used for small draws)."""
    z = (x + _GOLDEN) & MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64(x: torch.Tensor) -> torch.Tensor:
    """SplitMix64 finaliser on an int64 tensor (wrapping 64-bit arithmetic)."""
    z = x + _s64(_GOLDEN)
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def stream_base(seed: int, stream: int) -> int:
    return (seed * _SEED_MUL + stream * _GOLDEN) & MASK64


def normal_from_index(idx: torch.Tensor, seed: int, stream: int) -> torch.Tensor:
    """N(0,1) draws (fp64) for int64 element indices ``idx``."""
    z = splitmix64(idx + _s64(stream_base(seed, stream)))
    hi = _lsr(z, 32).to(torch.float64)
    lo = (z & 0xFFFFFFFF).to(torch.float64)
    u1 = (hi + 1.0) * (2.0 ** -32)      # (0, 1]
    u2 = lo * (2.0 ** -32)              # [0, 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def normal_tensor(shape, seed: int, stream: int, device="cpu", offset: int = 0,
                  chunk: int = 1 << 24) -> torch.Tensor:
    """fp16 tensor of N(0,1) draws; element i (row-major) uses counter offset + i."""
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=torch.float16, device=device)
    for start in range(0, n, chunk):
        m = min(chunk, n - start)
        idx = torch.arange(start + offset, start + offset + m, dtype=torch.int64, device=device)
        out[start:start + m] = normal_from_index(idx, seed, stream).to(torch.float16)
    return out.view(*shape)


def uniform_ints(seed: int, stream: int, n: int, salt: int = 0):
    """n 64-bit draws as Python ints (small host-side draws)."""
    base = stream_base(seed, stream) + (salt << 32)
    return [splitmix64_int((base + i) & MASK64) for i in range(n)]


def distinct_channels(seed: int, stream: int, salt: int, count: int, universe: int,
                      exclude=()):
    """``count`` distinct channels from range(universe) minus ``exclude``, by a
    seeded partial Fisher-Yates shuffle; returned in draw order."""
    pool = [c for c in range(universe) if c not in set(exclude)]
    draws = uniform_ints(seed, stream, count, salt)
    for i in range(count):
        j = i + draws[i] % (len(pool) - i)
        pool[i], pool[j] = pool[j], pool[i]
    return pool[:count]


@dataclass
class Config:
    """One workload: shapes, sparsity parameters, label dtype and steps."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int              # full head dim (query width)
    S0: int             # prefilled tokens
    steps: int          # decode steps (capacity = S0 + steps)
    r: int              # heavy channels per KV head (0: no labels)
    k: int              # heavy tokens per KV head (<= 0: dense)
    int4: bool          # label dtype
    d_k: int = 128      # stored K width (LeanK: kept columns)
    d_v: int = 128
    n_outlier: int = 8
    outlier_scale: float = 8.0
    seed: int = 1000
    note: str = ""

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def cap(self):
        return self.S0 + self.steps

    @property
    def sm_scale(self):
        return 1.0 / math.sqrt(self.D)


def _cfg(i, **kw):
    return Config(seed=1000 + i, **kw)


# The workloads: a tiny case, a Llama-2-7B-shaped MHA layer at 4K, a
# Qwen2.5-7B-shaped GQA layer at 8K, a 128K long-context MHA layer, and the
# LeanK pruned-K layer (dense, then with Double Sparsity on top).
CONFIGS = {
    "tiny": _cfg(0, name="tiny", B=1, Hq=32, Hkv=32, D=128, S0=1024, steps=1, r=16, k=64,
                 int4=False, note="B1 MHA 32x128, S 1024+1, r16 fp16 labels, k64"),
    "llama2_7b_4k": _cfg(1, name="llama2_7b_4k", B=32, Hq=32, Hkv=32, D=128, S0=4096, steps=64,
                         r=8, k=256, int4=True,
                         note="B32 MHA 32x128, S 4096+64, r8 int4 labels, k256"),
    "qwen25_7b_gqa_8k": _cfg(2, name="qwen25_7b_gqa_8k", B=64, Hq=28, Hkv=4, D=128, S0=8192,
                             steps=32, r=16, k=256, int4=False,
                             note="B64 GQA 28q/4kv x128, S 8192+32, r16 fp16 labels, k256/group"),
    "long_128k": _cfg(3, name="long_128k", B=4, Hq=32, Hkv=32, D=128, S0=131072, steps=16, r=8,
                      k=8192, int4=True, note="B4 MHA 32x128, S 131072+16, r8 int4 labels, k8192"),
    "leank_dense": _cfg(4, name="leank_dense", B=32, Hq=28, Hkv=4, D=128, S0=32768, steps=16,
                        r=0, k=0, int4=False, d_k=32,
                        note="B32 GQA 28q/4kv, K pruned to 32 of 128 columns, V 128, dense"),
    "leank_ds": _cfg(4, name="leank_ds", B=32, Hq=28, Hkv=4, D=128, S0=32768, steps=16, r=8,
                     k=1024, int4=False, d_k=32,
                     note="LeanK pruned K + Double Sparsity r8 fp16 labels, k1024/group"),
}


@dataclass
class Inputs:
    cfg: Config
    q: torch.Tensor          # [B][Hq][D] fp16
    K: torch.Tensor          # [B][Hkv][cap][d_k] fp16
    V: torch.Tensor          # [B][Hkv][cap][d_v] fp16
    chan: torch.Tensor | None    # [Hkv][r] int32, indexes stored K columns
    keep: torch.Tensor | None    # [Hkv][d_k] int32 (LeanK kept query channels) or None
    outliers: list = field(default_factory=list)


def outlier_channels(cfg: Config, g: int):
    return distinct_channels(cfg.seed, STREAM_OUTLIER, g, cfg.n_outlier, cfg.D)


def keep_table(cfg: Config):
    """LeanK kept channels per KV head: the outliers plus seeded extras, sorted."""
    if cfg.d_k == cfg.D:
        return None
    rows = []
    for g in range(cfg.Hkv):
        out = outlier_channels(cfg, g)
        extra = distinct_channels(cfg.seed, STREAM_KEEP, g, cfg.d_k - len(out), cfg.D, exclude=out)
        rows.append(sorted(out + extra))
    return rows


def heavy_table(cfg: Config, r: int | None = None):
    """Heavy channels per KV head as stored-K column indices, sorted ascending."""
    r = cfg.r if r is None else r
    keep = keep_table(cfg)
    rows = []
    for g in range(cfg.Hkv):
        out = outlier_channels(cfg, g)
        if r <= len(out):
            chosen = out[:r]
        else:
            universe = keep[g] if keep is not None else list(range(cfg.D))
            extra = distinct_channels(cfg.seed, STREAM_CHAN, g, r - len(out), cfg.D,
                                      exclude=[c for c in range(cfg.D) if c not in universe] + out)
            chosen = out + extra
        if keep is not None:
            chosen = [keep[g].index(c) for c in chosen]
        rows.append(sorted(chosen))
    return rows


def make_q(cfg: Config, device="cpu", step: int = 0) -> torch.Tensor:
    n = cfg.B * cfg.Hq * cfg.D
    return normal_tensor((cfg.B, cfg.Hq, cfg.D), cfg.seed, STREAM_Q, device, offset=step * n)


def make_kv(cfg: Config, device="cpu", cap: int | None = None):
    """K [B][Hkv][cap][d_k] and V [B][Hkv][cap][d_v] fp16.  K is drawn over the
    full head dim and the kept columns (all of them unless LeanK) are stored;
    outlier channels are scaled by ``outlier_scale``."""
    cap = cfg.cap if cap is None else cap
    B, H, D = cfg.B, cfg.Hkv, cfg.D
    keep = keep_table(cfg)
    K = torch.empty((B, H, cap, cfg.d_k), dtype=torch.float16, device=device)
    V = torch.empty((B, H, cap, cfg.d_v), dtype=torch.float16, device=device)
    for b in range(B):
        for g in range(H):
            row = (b * H + g)
            kfull = normal_tensor((cap, D), cfg.seed, STREAM_K, device, offset=row * cap * D)
            scale = torch.ones(D, dtype=torch.float16, device=device)
            scale[outlier_channels(cfg, g)] = cfg.outlier_scale
            kfull = kfull * scale
            if keep is not None:
                kfull = kfull[:, torch.tensor(keep[g], device=device)]
            K[b, g] = kfull
            V[b, g] = normal_tensor((cap, cfg.d_v), cfg.seed, STREAM_V, device,
                                    offset=row * cap * cfg.d_v)
    return K, V


def make_inputs(cfg: Config, device="cpu", step: int = 0) -> Inputs:
    K, V = make_kv(cfg, device)
    chan = None
    if cfg.r > 0:
        chan = torch.tensor(heavy_table(cfg), dtype=torch.int32, device=device)
    keep = keep_table(cfg)
    keep_t = torch.tensor(keep, dtype=torch.int32, device=device) if keep is not None else None
    return Inputs(cfg, make_q(cfg, device, step), K, V, chan, keep_t,
                  [outlier_channels(cfg, g) for g in range(cfg.Hkv)])


def small(name: str = "small", **kw) -> Config:
    """A small custom workload (parity cases that the oracle finishes in seconds)."""
    base = dict(name=name, B=2, Hq=4, Hkv=4, D=128, S0=300, steps=4, r=16, k=32, int4=False,
                seed=7)
    base.update(kw)
    return Config(**base)
