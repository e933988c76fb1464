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


def _oracle_records(wl, n):
    """Selections, kinds and outputs of layer 0 of wl for n steps, computed
    by the oracle itself: records a faultless GPU would produce."""
    from synth import bf16_bits_to_f64, context_kv, eviction_weights, new_tokens, queries
    from trainable_offloadable_block_amd import _lib as L
    to_lib = {o.SINK: L.KIND_SINK, o.WINDOW: L.KIND_WINDOW, o.QUERY: L.KIND_QUERY,
              o.AGNOSTIC: L.KIND_AGNOSTIC}
    G, Hkv, k = wl.group, wl.n_kv_heads, wl.k_blocks
    P = wl.batch * Hkv
    n_w = wl.window_tokens // 64
    sel = np.full((n, P, k), -1, np.int32)
    nsel = np.zeros((n, P), np.int32)
    kind = np.zeros((n, P, k), np.uint8)
    out = np.zeros((n, wl.batch, wl.n_q_heads, 128), np.float32)
    for p in range(P):
        b, g = divmod(p, Hkv)
        K, V = context_kv(wl, 0, b, g)
        w1, w2 = eviction_weights(wl, 0, g)
        Kf, Vf = np.zeros((wl.context + n, 128)), np.zeros((wl.context + n, 128))
        Kf[:wl.context], Vf[:wl.context] = bf16_bits_to_f64(K), bf16_bits_to_f64(V)
        orc = o.PairOracle(Kf, Vf, bf16_bits_to_f64(w1), bf16_bits_to_f64(w2), wl.context,
                           wl.n_sink_blocks, n_w, wl.k_q_blocks,
                           wl.k_e_blocks - wl.n_sink_blocks - n_w, 1.0)
        kn, vn = new_tokens(wl, 0, b, g)
        q = np.stack([queries(wl, 0, b, g * G + h) for h in range(G)])
        for t in range(n):
            r = orc.step(bf16_bits_to_f64(kn[t]), bf16_bits_to_f64(vn[t]),
                         bf16_bits_to_f64(q[:, t]))
            m = len(r.sel.blocks)
            nsel[t, p] = m
            sel[t, p, :m] = r.sel.blocks
            kind[t, p, :m] = [to_lib[r.sel.kinds[x]] for x in r.sel.blocks]
            out[t, b, g * G:(g + 1) * G] = r.out
    return sel, nsel, kind, out


def test_cpu_baseline_parity_check():
    """The bench's full-size parity check (the CPU baseline's oracle run
    against the GPU's records of the same steps): records equal to the
    oracle's pass; a query-aware block swapped for a candidate far from the
    boundary is an unexplained difference, and that pair is followed no
    further; an output off by more than the bar fails the verdict."""
    from trainable_offloadable_block_amd import _lib as L
    wl = WORKLOADS[1]
    n = 3
    sel, nsel, kind, out = _oracle_records(wl, n)
    par, cpu = bench.cpu_baseline(1, 2, n, (sel, nsel, kind, out))
    assert par["verdict"] == "pass" and par["selections_identical"] == 2 * n
    assert par["near_ties"] == 0 and par["unexplained_differences"] == 0
    assert par["attention_max_abs"] < 1e-6 and cpu["cores"] >= 1
    # a planted swap at step 1 of pair 0
    sel2, kind2 = sel.copy(), kind.copy()
    m = int(nsel[1, 0])
    blocks = sel2[1, 0, :m].tolist()
    kinds = kind2[1, 0, :m].tolist()
    i = kinds.index(L.KIND_QUERY)
    blocks[i] = next(x for x in range(wl.n_sink_blocks, 64) if x not in blocks)
    order = np.argsort(blocks)
    sel2[1, 0, :m] = np.array(blocks)[order]
    kind2[1, 0, :m] = np.array(kinds)[order]
    par2, _ = bench.cpu_baseline(1, 2, n, (sel2, nsel, kind2, out))
    assert par2["verdict"] == "fail" and par2["unexplained_differences"] == 1
    assert par2["pair_steps_compared"] == 2 * n - 1
    out3 = out.copy()
    out3[0, 0, 0, 0] += 0.05
    par3, _ = bench.cpu_baseline(1, 2, n, (sel, nsel, kind, out3))
    assert par3["verdict"] == "fail" and par3["unexplained_differences"] == 0
