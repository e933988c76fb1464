"""Host-side helpers of bench.py (no GPU): the per-step locality it reports
equals the oracle's gamma(t) on random selections, and the algorithmic byte
count of a decode launch follows its definition."""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import nosa_oracle as o  # noqa: E402
from synth import WORKLOADS, small_workload  # noqa: E402


def test_locality_step_equals_oracle_gamma():
    wl = small_workload(301, batch=3, n_kv_heads=2, k_blocks=8)
    rng = np.random.default_rng(5)
    P, k = wl.batch * wl.n_kv_heads, wl.k_blocks
    for trial in range(50):
        lens = rng.integers(200, 2000, size=wl.batch)
        if trial % 5 == 0:
            lens[0] = 64 * rng.integers(4, 30) + 1          # the token opens a block
        nb = (lens + 63) // 64
        ps = np.full((P, k), -1, np.int32)
        cs = np.full((P, k), -1, np.int32)
        pn = rng.integers(1, k + 1, size=P).astype(np.int32)
        cn = rng.integers(1, k + 1, size=P).astype(np.int32)
        for p in range(P):
            top = int(nb[p // wl.n_kv_heads])
            pn[p], cn[p] = min(pn[p], top), min(cn[p], top)
            ps[p, :pn[p]] = np.sort(rng.choice(top, size=pn[p], replace=False))
            cs[p, :cn[p]] = np.sort(rng.choice(top, size=cn[p], replace=False))
        got = bench.locality_step((ps, pn), (cs, cn), lens, wl)
        want = []
        for p in range(P):
            pos = int(lens[p // wl.n_kv_heads]) - 1
            new_block = pos // 64 if pos % 64 == 0 else None
            want.append(o.locality(ps[p, :pn[p]].tolist(), cs[p, :cn[p]].tolist(), new_block))
        assert np.allclose(got, want, rtol=0, atol=0)


def test_token_locality_step_equals_oracle():
    wl = small_workload(302, batch=3, n_kv_heads=2, k_blocks=8)
    rng = np.random.default_rng(6)
    P, k = wl.batch * wl.n_kv_heads, wl.k_blocks
    for trial in range(60):
        lens = rng.integers(130, 2000, size=wl.batch)
        if trial % 4 == 0:
            lens[1] = 64 * rng.integers(3, 30) + 1          # the token opens a block
        nb = (lens + 63) // 64
        ps = np.full((P, k), -1, np.int32)
        cs = np.full((P, k), -1, np.int32)
        pn = np.zeros(P, np.int32)
        cn = np.zeros(P, np.int32)
        for p in range(P):
            L = int(lens[p // wl.n_kv_heads])
            top = int(nb[p // wl.n_kv_heads])
            prev_top = (L - 1 + 63) // 64                   # blocks at the previous length
            n1 = int(min(rng.integers(1, k + 1), prev_top))
            n2 = int(min(rng.integers(1, k), top - 1))
            ps[p, :n1] = np.sort(rng.choice(prev_top, size=n1, replace=False))
            rest = np.sort(rng.choice(top - 1, size=n2, replace=False))
            cur = np.unique(np.append(rest, top - 1))        # S(t) holds the newest block
            cs[p, :len(cur)] = cur
            pn[p], cn[p] = n1, len(cur)
        got = bench.token_locality_step((ps, pn), (cs, cn), lens, wl)
        want = []
        for p in range(P):
            L = int(lens[p // wl.n_kv_heads])
            want.append(o.token_locality(ps[p, :pn[p]].tolist(), L - 1,
                                         cs[p, :cn[p]].tolist(), L))
        assert np.allclose(got, want, rtol=1e-15, atol=0)


def test_decode_bytes_definition():
    wl = WORKLOADS[2]
    n_att = 4032.44
    want = (n_att * wl.batch * wl.n_kv_heads * (2 * 128 * 2 + 4)
            + wl.batch * wl.n_q_heads * 128 * (2 + 4) + wl.batch * wl.n_kv_heads * wl.k_blocks * 8)
    assert bench.decode_bytes(wl, n_att) == want


def test_generator_rounds_float64_to_bf16_once():
    """Generated values computed in float64 (queries, hot keys) are rounded to
    bf16 once: a value just above a bf16 tie that a float32 step would pull
    onto the tie still rounds up; exact ties go to even."""
    from synth import f64_to_bf16_bits
    x = np.array([1 + 2.0 ** -8,                   # tie -> even (1.0)
                  1 + 3 * 2.0 ** -8,               # tie -> even (1 + 2^-6)
                  1 + 2.0 ** -8 + 2.0 ** -30,      # above the tie; float32 would land on it
                  -(1 + 2.0 ** -8 + 2.0 ** -30),
                  0.0, 3.0, 2.0 ** -126])
    want = [0x3F80, 0x3F82, 0x3F81, 0xBF81, 0x0000, 0x4040, 0x0080]
    assert f64_to_bf16_bits(x).tolist() == want
    with pytest.raises(ValueError):
        f64_to_bf16_bits(np.array([2.0 ** -130]))
