"""Workload descriptions and seeded slab generators.

Each workload mirrors one of the decode settings the NOSA pages describe: the
1B model's head layout (16 query heads over 2 KV heads, head_dim 128; aiwiki
"NOSA", Models and training table), the 8B-shaped 32/8 layout, block 64, a
one-block attention sink, a sliding window and a k-block budget split into
k_q query-aware and k_e query-agnostic blocks (aiwiki "NOSA", Main-experiment
configuration).

Recipe (every slab has its own stream, so any (layer, sequence, head) slab can
be regenerated alone):

* stream = PCG64(SeedSequence(seed, spawn_key=(cfg_id, tag, layer, b, h)))
* context K, V elements ~ N(0, 1), drawn as float32 and rounded to bf16 (RNE)
  (values computed in float64 -- hot keys, queries -- are rounded to bf16
  once, directly from float64)
* each (layer, KV head) has a unit direction u (16 of them in the drift
  workload); hot 64-token blocks, drawn without replacement from the blocks
  that start out between the sink and the window, get keys u + 0.3 * N(0, I)
* queries follow an AR(1) walk toward mu*u with mu = sqrt(128):
  q_0 = mu*u + xi_0, q_t = rho*q_{t-1} + (1-rho)*mu*u(t) + sqrt(1-rho^2)*xi_t,
  kept in float64 and rounded to bf16 per step
* forecast heads (SparDA's layer-ahead selection; the trained Forecast
  projection does not exist here): one per (layer, sequence, KV head), the
  same AR(1) walk as a query head of that layer, from a stream of its own
* every decode step appends one token with k, v elements ~ N(0, 1)
* eviction-head weights W1 [128][128] (input-dim major) and W2 [128], one
  pair per (layer, KV head), elements ~ N(0, 0.02^2) (0.02 is the standard
  deviation)

Nothing here implements any step of the method.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128
BLOCK = 64

_TAG = {"K": 0, "V": 1, "HOT": 2, "U": 3, "Q": 4, "KNEW": 5, "VNEW": 6,
        "W1": 7, "W2": 8, "F": 9}


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    context: int            # prefilled tokens per sequence before step 0
    steps: int              # decode steps (one appended token each)
    n_sink_blocks: int
    window_tokens: int
    k_blocks: int
    k_q_blocks: int
    k_e_blocks: int
    rho: float
    n_hot: int              # planted hot blocks per (sequence, KV head)
    n_layers: int = 1
    offload: bool = False   # full KV in pinned host memory
    drift: bool = False     # 16 directions, target changes every 16 steps
    evict_bias: bool = True
    seed: int = 0
    head_dim: int = HEAD_DIM
    block: int = BLOCK

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_context(self) -> int:
        return self.context + self.steps

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _hot_count(context: int, frac: float = 0.01) -> int:
    return max(1, int(round(frac * (context // BLOCK))))


WORKLOADS = {
    1: Workload("tiny-decode-4k", 1, batch=1, n_q_heads=16, n_kv_heads=2,
                context=4096, steps=32, n_sink_blocks=1, window_tokens=256,
                k_blocks=16, k_q_blocks=4, k_e_blocks=12, rho=0.95, n_hot=4),
    2: Workload("nosa1b-layer-16k-b32", 2, batch=32, n_q_heads=16,
                n_kv_heads=2, context=16384, steps=256, n_sink_blocks=1,
                window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                rho=0.95, n_hot=_hot_count(16384)),
    3: Workload("nosa1b-28layer-32k-b64-offload", 3, batch=64, n_q_heads=16,
                n_kv_heads=2, context=32768, steps=128, n_sink_blocks=1,
                window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                rho=0.95, n_hot=_hot_count(32768), n_layers=28, offload=True),
    4: Workload("8b-layer-64k-b32-offload", 4, batch=32, n_q_heads=32,
                n_kv_heads=8, context=65536, steps=64, n_sink_blocks=1,
                window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                rho=0.9, n_hot=_hot_count(65536), offload=True),
    5: Workload("8b-stress-128k-b8-drift-offload", 5, batch=8, n_q_heads=32,
                n_kv_heads=8, context=131072, steps=256, n_sink_blocks=1,
                window_tokens=1024, k_blocks=64, k_q_blocks=32, k_e_blocks=32,
                rho=0.8, n_hot=64, offload=True, drift=True),
}

# Beyond the five benchmark configurations: the pages' own 8B head layout
# (32 query / 2 KV heads, GQA 16; aiwiki "NOSA", Models and training table)
# with the 96-block budget SparDA uses for NOSA-8B (24 query-aware blocks, a
# 1024-token window; aiwiki "NOSA", Adoption in SparDA), at its native 32K.
NEXT_WORKLOADS = {
    "gqa16-k96": Workload("nosa8b-gqa16-k96-32k-b16", 6, batch=16, n_q_heads=32,
                          n_kv_heads=2, context=32768, steps=64, n_sink_blocks=1,
                          window_tokens=1024, k_blocks=96, k_q_blocks=24,
                          k_e_blocks=72, rho=0.9, n_hot=_hot_count(32768)),
}


def small_workload(cfg_id: int = 100, **kw) -> Workload:
    """A small workload for tests; keyword arguments override the defaults."""
    base = dict(name=f"small-{cfg_id}", cfg_id=cfg_id, batch=2, n_q_heads=8,
                n_kv_heads=2, context=1024, steps=8, n_sink_blocks=1,
                window_tokens=128, k_blocks=8, k_q_blocks=2, k_e_blocks=6,
                rho=0.9, n_hot=2)
    base.update(kw)
    return Workload(**base)


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Input rounding for generated tensors only; returns uint16 bit patterns.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("generator produced a non-finite value")
    # finite float32 bit patterns are <= 0xFF7FFFFF, so adding at most
    # 0x8000 cannot wrap a uint32
    u = f.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 once (round to nearest, ties to even),
    with no float32 step in between. Input rounding for generated tensors
    only (their magnitudes are far inside bf16's normal range); returns
    uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float64)
    a = np.abs(f)
    if not np.all(np.isfinite(f)) or np.any((a != 0) & ((a < 2.0 ** -126) | (a >= 2.0 ** 127))):
        raise ValueError("generator produced a value outside bf16's normal range")
    # keep 7 of float64's 52 fraction bits, rounding the other 45 to nearest
    # even; the result has a float32 exponent and 7 fraction bits, so the
    # float32 conversion is exact and its high half is the bf16 pattern
    u = f.view(np.uint64)
    u = (u + np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1))) >> np.uint64(45)
    r = (u << np.uint64(45)).view(np.float64).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- streams

def _rng(wl: Workload, tag: str, layer: int = 0, b: int = 0, h: int = 0):
    ss = np.random.SeedSequence(wl.seed, spawn_key=(wl.cfg_id, _TAG[tag],
                                                   layer, b, h))
    return np.random.Generator(np.random.PCG64(ss))


def _directions(wl: Workload, layer: int, g: int) -> np.ndarray:
    """Unit directions for one (layer, KV head): [n_dir][128] float64."""
    n_dir = 16 if wl.drift else 1
    u = _rng(wl, "U", layer, 0, g).standard_normal((n_dir, wl.head_dim))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def hot_blocks(wl: Workload, layer: int, b: int, g: int) -> np.ndarray:
    """Planted hot block ids for one (layer, sequence, KV head).

    Drawn from the blocks strictly between the sink and the window of the
    prefilled context. In the drift workload direction m is planted in
    blocks [4m, 4m+4) of the returned array.
    """
    n_win = wl.window_tokens // wl.block
    lo, hi = wl.n_sink_blocks, wl.context // wl.block - n_win
    n = 64 if wl.drift else wl.n_hot
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    if hi - lo < n:
        raise ValueError("context too short for the planted blocks")
    return _rng(wl, "HOT", layer, b, g).choice(np.arange(lo, hi), size=n,
                                               replace=False)


def context_kv(wl: Workload, layer: int, b: int, g: int):
    """Prefilled K and V for one (layer, sequence, KV head).

    Returns (K, V) as uint16 bf16 bit patterns, each [context][128] in
    token-major order.
    """
    L, d = wl.context, wl.head_dim
    k = _rng(wl, "K", layer, b, g).standard_normal((L, d), dtype=np.float32)
    v = _rng(wl, "V", layer, b, g).standard_normal((L, d), dtype=np.float32)
    u = _directions(wl, layer, g)
    kb = f32_to_bf16_bits(k)
    for j, blk in enumerate(hot_blocks(wl, layer, b, g)):
        m = j // 4 if wl.drift else 0
        rows = slice(blk * wl.block, (blk + 1) * wl.block)
        kb[rows] = f64_to_bf16_bits(u[m][None, :] + 0.3 * k[rows].astype(np.float64))
    return kb, f32_to_bf16_bits(v)


def queries(wl: Workload, layer: int, b: int, h: int) -> np.ndarray:
    """Per-step queries for one (layer, sequence, q head): uint16 [steps][128]."""
    g = h // wl.group
    xi = _rng(wl, "Q", layer, b, h).standard_normal((wl.steps, wl.head_dim))
    return _ar1_walk(wl, _directions(wl, layer, g), xi)


def forecasts(wl: Workload, layer: int, b: int, g: int) -> np.ndarray:
    """Per-step forecast head that selects layer `layer`'s blocks for one
    (sequence, KV head): uint16 [steps][128], drawn like a query head of that
    layer (toward its direction) from its own stream."""
    xi = _rng(wl, "F", layer, b, g).standard_normal((wl.steps, wl.head_dim))
    return _ar1_walk(wl, _directions(wl, layer, g), xi)


def _ar1_walk(wl: Workload, u: np.ndarray, xi: np.ndarray) -> np.ndarray:
    mu = math.sqrt(wl.head_dim)
    rho = wl.rho
    out = np.empty((wl.steps, wl.head_dim), dtype=np.float64)
    q = None
    for t in range(wl.steps):
        target = u[(t // 16) % len(u)] if wl.drift else u[0]
        if q is None:
            q = mu * target + xi[0]
        else:
            q = rho * q + (1.0 - rho) * mu * target + math.sqrt(
                1.0 - rho * rho) * xi[t]
        out[t] = q
    return f64_to_bf16_bits(out)


def new_tokens(wl: Workload, layer: int, b: int, g: int):
    """Appended (k, v) per decode step: uint16 [steps][128] each."""
    shape = (wl.steps, wl.head_dim)
    k = _rng(wl, "KNEW", layer, b, g).standard_normal(shape, dtype=np.float32)
    v = _rng(wl, "VNEW", layer, b, g).standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def eviction_weights(wl: Workload, layer: int, g: int):
    """Eviction-head weights for one (layer, KV head).

    Returns W1 uint16 [128 inputs][128 hidden] and W2 uint16 [128 hidden].
    """
    d = wl.head_dim
    w1 = 0.02 * _rng(wl, "W1", layer, 0, g).standard_normal((d, d))
    w2 = 0.02 * _rng(wl, "W2", layer, 0, g).standard_normal(d)
    return (f32_to_bf16_bits(w1.astype(np.float32)),
            f32_to_bf16_bits(w2.astype(np.float32)))
