"""HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Bars: selected blocks and kinds identical (up to the near-tie protocol of
``nosa_harness``), compressed keys bit-identical, attention output within
max-abs 1e-2 and relative L2 2e-3 of the float64 oracle.
"""

import sys

import numpy as np
import pytest
import torch

from synth import NEXT_WORKLOADS, WORKLOADS, small_workload
from nosa_harness import Lockstep, summary
from trainable_offloadable_block_amd import v_to_tiles
from trainable_offloadable_block_amd import _lib as L

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(wl, **kw):
    steps = kw.pop("run_steps", None)
    cache_every = kw.pop("cache_every", 0)
    _say(f"[parity] {wl.name} {kw}")
    ls = Lockstep(wl, **kw)
    ls.check_prefill()
    reps = ls.run(steps, cache_every=cache_every)
    if ls.shape.offload:
        ls.check_cache()
    s = summary(reps)
    _say(f"[parity] {wl.name}: {s}")
    return ls, s


def test_native_library_loaded():
    import trainable_offloadable_block_amd as nosa
    nosa.lib()
    maps = open("/proc/self/maps").read()
    assert "libnosa.so" in maps
    assert torch.cuda.is_available()


@pytest.mark.parametrize("fused", [False, True])
def test_small_resident(fused):
    _run(small_workload(101), fused=fused)


@pytest.mark.parametrize("fused", [False, True])
def test_small_offload(fused):
    _run(small_workload(102, offload=True), cache_every=2, fused=fused)


def test_small_no_bias():
    _run(small_workload(103, evict_bias=False))


def test_ragged_lengths():
    """Different lengths per sequence: ragged last blocks, a sequence with no
    candidates yet, one that opens a block on the first step."""
    wl = small_workload(104, batch=4, steps=70)
    _run(wl, lengths=[1000, 700, 129, 64])


def test_group_16_and_4():
    _run(small_workload(105, n_q_heads=32, n_kv_heads=2))
    _run(small_workload(106, n_q_heads=8, n_kv_heads=2, batch=3))


def test_budget_corner_cases():
    # no query-aware stage
    _run(small_workload(107, k_blocks=6, k_q_blocks=0, k_e_blocks=6))
    # no agnostic dynamic blocks (plain top-k)
    _run(small_workload(108, k_blocks=7, k_q_blocks=4, k_e_blocks=3))
    # no sink, wide window
    _run(small_workload(109, n_sink_blocks=0, window_tokens=256, k_blocks=9,
                        k_q_blocks=3, k_e_blocks=6))


def test_short_context_everything_selected():
    """Contexts shorter than the budget: every block is attended, which is
    full attention (checked against the oracle, itself pinned to SDPA)."""
    _run(small_workload(110, context=200, steps=80, k_blocks=10, k_q_blocks=3,
                        k_e_blocks=7, n_hot=0))


def test_long_run_offload_locality():
    """Many steps in offload mode: misses match the oracle's cache model and
    never exceed k_q per pair after the first step."""
    wl = small_workload(111, offload=True, steps=150, context=2048, k_blocks=12,
                        k_q_blocks=3, k_e_blocks=9, n_hot=4)
    ls, _ = _run(wl, cache_every=25)
    for r in ls.reports[1:]:
        for p, (got, want) in r.misses.items():
            assert got <= wl.k_q_blocks


def test_tiny_decode_workload():
    _run(WORKLOADS[1])


def test_nosa1b_layer_all_pairs():
    """Full-size 1B-shaped layer (batch 32, 16K context, k = 64), the launch
    configuration the benchmark times (append and select in one launch);
    every pair against the oracle."""
    _run(WORKLOADS[2], steps=6, fused=True)


def test_nosa1b_layer_sampled_long():
    """Same layer, 4 sampled pairs over 70 steps: covers the window sliding
    by a block at step 64 and the eligible pool running short."""
    _run(WORKLOADS[2], check_pairs=[0, 12, 47, 63], steps=70)


def _wide_keys(rng, shape):
    """bf16 keys whose magnitudes span far more than 40 binades: mostly N(0,1),
    some entries scaled by 2^+-(40..120), some exact cancelling pairs."""
    import oracle.nosa_oracle as O
    x = rng.standard_normal(shape)
    big = rng.random(shape) < 0.15
    x[big] *= np.ldexp(1.0, rng.integers(40, 120, size=int(big.sum())))
    tiny = rng.random(shape) < 0.15
    x[tiny] *= np.ldexp(1.0, -rng.integers(40, 125, size=int(tiny.sum())))
    return O.bf16_bits(O.bf16_round(x))


def test_chunk_mean_exact_for_any_span():
    """CompressK rounds the exact mean of 32 keys once, also when the keys'
    magnitudes span more binades than a float64 sum keeps exactly: prefilled
    chunks, then 96 appended tokens (six chunk completions per pair), each
    compressed key bit-identical to the oracle's exact (rational) mean."""
    import oracle.nosa_oracle as O
    from synth import bf16_bits_to_f64
    wl = small_workload(195, context=400, steps=96, batch=2)
    rng = np.random.default_rng(195)
    P, steps = wl.batch * wl.n_kv_heads, 96
    ctx = _wide_keys(rng, (P, 400, 128))
    new = _wide_keys(rng, (steps, wl.batch, wl.n_kv_heads, 128))
    Kall = np.concatenate([ctx, new.transpose(1, 2, 0, 3).reshape(P, steps, 128)], axis=1)

    def plant(ls):
        pool = ls.gpu.kv_dev.view(ls.P, ls.gpu.nb_kv, 2, 64, 128)
        for p in range(P):
            kb = np.zeros((7, 64, 128), dtype=np.uint16)
            kb.reshape(-1, 128)[:400] = ctx[p]
            pool[p, :7, 0] = torch.from_numpy(kb.view(np.int16)).to(pool.device)
        torch.cuda.synchronize()

    ls = Lockstep(wl, check_pairs=[], before_prefill=plant, steps=steps)
    g = ls.gpu

    L_end = 400 + steps
    want_all = [O.bf16_bits(O.compress_keys(bf16_bits_to_f64(Kall[p]), L_end)) for p in range(P)]

    def compare(L):
        ck = g.ckey.cpu().numpy().view(np.uint16).reshape(P, ls.shape.c_max, 128)
        C = O.n_chunks(L)
        for p in range(P):
            want = want_all[p][:C]              # chunk i depends on tokens < 16i + 32 only
            bad = np.nonzero(np.any(ck[p, :C] != want, axis=1))[0]
            assert not len(bad), f"L={L} pair {p}: chunks {bad[:8]} differ"

    torch.cuda.synchronize()
    compare(400)
    for t in range(steps):
        _, vd, _ = ls.inputs(t)
        kd = torch.from_numpy(np.ascontiguousarray(new[t]).view(np.int16)).to(g.device)
        g.append(kd, vd)
        if t % 16 == 15:
            torch.cuda.synchronize()
            compare(401 + t)
    assert g.status_bits() == 0


def test_capacity_sets_status():
    wl = small_workload(112, context=120, steps=8, n_hot=0)
    ls = Lockstep(wl, steps=8)
    g = ls.gpu
    # the state was sized for context + steps tokens: fill it, then one more
    for t in range(8):
        kd, vd, qd = ls.inputs(t)
        g.append(kd, vd)
    torch.cuda.synchronize()
    assert g.status_bits() == 0
    assert g.seq_len.cpu().tolist() == [128] * wl.batch
    kd, vd, _ = ls.inputs(0)
    g.max_len = g.shape.max_context - 1        # host bound stays in range
    g.append(kd, vd)
    torch.cuda.synchronize()
    assert g.status_bits() & 1
    assert g.seq_len.cpu().tolist() == [128] * wl.batch


def test_nan_bytes_past_length_are_ignored():
    """The pool holds NaN patterns past each sequence's length when prefill
    runs: prefill clears the tail of the partial block, append clears each
    block it opens, so attention never meets them."""
    wl = small_workload(113, context=1000, steps=80)
    nan = int(np.array([0x7FC0], dtype=np.uint16).view(np.int16)[0])

    def plant(ls):
        pool = ls.gpu.kv_dev.view(ls.P, ls.gpu.nb_kv, 2, 64, 128)
        for p in range(ls.P):
            Lb = int(ls.lengths[p // wl.n_kv_heads])
            blk, r = divmod(Lb, 64)
            pool[p, blk, 0, r:] = nan
            past = np.broadcast_to((np.arange(64) >= r)[:, None], (64, 128))
            mask = torch.from_numpy(v_to_tiles(past).copy()).to(pool.device)
            pool[p, blk, 1].view(-1)[mask] = nan
            pool[p, blk + 1:] = nan
        torch.cuda.synchronize()

    ls = Lockstep(wl, lengths=[1000, 937], before_prefill=plant)
    ls.check_prefill()
    ls.run()


@pytest.mark.parametrize("offload", [False, True])
def test_kv_stride_with_extra_block(offload):
    """A length bound of 129 blocks (a multiple of 129): the pool, the host
    store and the token scores get one block more of stride per pair. Steps
    still match the oracle, and NaN planted in every pair's extra block and
    extra token scores is never read."""
    wl = small_workload(115, context=8190, steps=12, offload=offload)
    nan16 = int(np.array([0x7FC0], dtype=np.uint16).view(np.int16)[0])

    def plant(ls):
        g = ls.gpu
        assert ls.shape.nb_max == 129 and g.nb_kv == 130
        store = g.kv_host if offload else g.kv_dev
        store.view(ls.P, g.nb_kv, 2, 64, 128)[:, 129] = nan16
        g.tok_s.view(ls.P, g.nb_kv * 64)[:, 129 * 64:] = float("nan")
        torch.cuda.synchronize()

    ls = Lockstep(wl, before_prefill=plant)
    ls.check_prefill()
    ls.run(cache_every=4 if offload else 0)
    if offload:
        ls.check_cache()


def test_resident_fetch_is_identity():
    """With resident KV, nosa_fetch_delta only sets phys = sel, n_miss = 0."""
    wl = small_workload(114)
    ls = Lockstep(wl)
    kd, vd, qd = ls.inputs(0)
    g = ls.gpu
    g.append(kd, vd)
    g.select(qd)
    g.phys.fill_(-7)
    g.n_miss.fill_(5)
    g.fetch(force=True)
    torch.cuda.synchronize()
    assert torch.equal(g.phys, g.sel)
    assert int(g.n_miss.abs().sum()) == 0


def test_offload_128k_drift_sampled():
    """Offloaded 128K low-locality workload (8 sequences, 32/8 heads,
    k_q = k_e = 32) at full size: 4 sampled pairs against the oracle over 72
    steps (the hot set moves every 16 steps: four shifts), fetched blocks
    equal the oracle's misses, cache bytes equal the host store."""
    _run(WORKLOADS[5], check_pairs=[0, 21, 42, 63], steps=72, cache_every=8, fused=True)


def test_offload_8b_64k_sampled():
    """Offloaded 8B-shaped 64K layer (32 sequences, 32/8 heads) at full size."""
    _run(WORKLOADS[4], check_pairs=[0, 57, 100, 170, 213, 255], steps=24, cache_every=6)


def test_offload_1b_32k_layer_sampled():
    """One layer (layer 13) of the offloaded 28-layer 32K stack (64 sequences)."""
    _run(WORKLOADS[3], layer=13, check_pairs=[0, 31, 77, 96, 127], steps=24, cache_every=6)


def _state_tensors(g):
    names = ["seq_len", "arrive", "status", "ckey", "tok_s", "chunk_e", "blk_e",
             "eligible", "tail_keys", "kv_dev", "kv_host", "slot_of_block", "block_of_slot"]
    return {n: getattr(g, n) for n in names if getattr(g, n, None) is not None}


@pytest.mark.parametrize("offload", [False, True])
def test_append_select_equals_separate_calls(offload):
    """nosa_append_select leaves the same state and returns the same selection,
    bit for bit, as nosa_compress_append then nosa_select: 80 steps from a
    1000-token context cross chunk completions every 16 tokens, block
    completions, a block opening at 1024 and the window sliding by a block."""
    wl = small_workload(121, context=1000, steps=80, offload=offload)
    a = Lockstep(wl, check_pairs=[], lengths=[1000, 963])
    b = Lockstep(wl, check_pairs=[], lengths=[1000, 963], fused=True)
    for t in range(wl.steps):
        kd, vd, qd = a.inputs(t)
        a.gpu.append(kd, vd)
        a.gpu.select(qd, want_kind=True, want_qscore=True)
        b.gpu.append_select(kd, vd, qd, want_kind=True, want_qscore=True)
        for ls in (a, b):
            ls.gpu.fetch()
        torch.cuda.synchronize()
        for n in ("sel", "n_sel", "kind", "phys", "n_miss"):
            assert torch.equal(getattr(a.gpu, n), getattr(b.gpu, n)), f"step {t}: {n}"
        assert torch.equal(torch.nan_to_num(a.gpu.dbg_q, nan=-7.0),
                           torch.nan_to_num(b.gpu.dbg_q, nan=-7.0)), f"step {t}: qscore"
        sa, sb = _state_tensors(a.gpu), _state_tensors(b.gpu)
        for n in sa:
            assert torch.equal(sa[n], sb[n]), f"step {t}: state {n}"
    assert a.gpu.status_bits() == 0 and b.gpu.status_bits() == 0


def test_append_select_capacity_sets_status():
    wl = small_workload(122, context=120, steps=8, n_hot=0)
    ls = Lockstep(wl, steps=8, fused=True)
    g = ls.gpu
    for t in range(8):
        kd, vd, qd = ls.inputs(t)
        g.append_select(kd, vd, qd)
    torch.cuda.synchronize()
    assert g.status_bits() == 0
    assert g.seq_len.cpu().tolist() == [128] * wl.batch
    kd, vd, qd = ls.inputs(0)
    g.max_len = g.shape.max_context - 1        # host bound stays in range
    g.append_select(kd, vd, qd)
    torch.cuda.synchronize()
    assert g.status_bits() & 1
    assert g.seq_len.cpu().tolist() == [128] * wl.batch


@pytest.mark.parametrize("offload", [False, True])
def test_gqa16_k96_sampled(offload):
    """The pages' 8B head layout (32/2 heads, GQA 16) with SparDA's 96-block
    budget (24 query-aware, window 1024) at 32K, 16 sequences: 3 sampled
    pairs against the oracle; offloaded, the cache must equal the host store."""
    wl = NEXT_WORKLOADS["gqa16-k96"].replace(offload=offload)
    _run(wl, check_pairs=[0, 13, 31], steps=8, cache_every=4, fused=True)


@pytest.mark.parametrize("offload", [False, True])
def test_k128_budget(offload):
    """The largest budget, k = 128 blocks (32 query-aware, 96 agnostic with a
    1024-token window), over 70 steps of a 12K context."""
    wl = small_workload(131, context=12288, steps=70, n_q_heads=16, window_tokens=1024,
                        k_blocks=128, k_q_blocks=32, k_e_blocks=96, offload=offload)
    _run(wl, cache_every=10, fused=True)


@pytest.mark.parametrize("offload", [False, True])
def test_graph_replay_matches_eager(offload):
    """A whole step (append_select, fetch, decode) captured as a HIP graph
    over static input buffers and replayed 40 times, with eager work and
    synchronisations between the replays: every replay's selection, output
    and state equal, bit for bit, those of an identical layer run eagerly,
    and every replay passes the oracle's checks (selection and kinds, scores,
    attention output, misses, eligibility; the full state every 16 replays)
    across chunk completions and a block opening at 1024 tokens."""
    wl = small_workload(141, context=1000, steps=40, offload=offload)
    a = Lockstep(wl, check_pairs=[], lengths=[1000, 990])
    b = Lockstep(wl, lengths=[1000, 990])
    b.check_prefill()
    bound = b.shape.max_context
    for ls in (a, b):
        ls.gpu.max_len = bound - 1          # the same grid sizes on both paths
    kd, vd, qd = b.inputs(0)
    ks, vs, qs = kd.clone(), vd.clone(), qd.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    b.gpu.dbg_q = torch.full((b.shape.pairs * b.shape.nb_max,), float("nan"),
                             dtype=torch.float32, device=b.gpu.device)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            b.gpu.append_select(ks, vs, qs, want_kind=True, want_qscore=True)
            b.gpu.fetch()
            b.gpu.decode(qs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for t in range(wl.steps):
        kd, vd, qd = a.inputs(t)
        a.gpu.max_len = bound - 1
        a.gpu.append_select(kd, vd, qd, want_kind=True, want_qscore=True)
        a.gpu.fetch()
        a.gpu.decode(qd)
        ks.copy_(kd)
        vs.copy_(vd)
        qs.copy_(qd)
        g.replay()
        scratch.add_(1.0)                   # eager work between replays
        torch.cuda.synchronize()
        for n in ("sel", "n_sel", "kind", "phys", "n_miss", "out", "dbg_q"):
            assert torch.equal(torch.nan_to_num(getattr(a.gpu, n), nan=-7.0),
                               torch.nan_to_num(getattr(b.gpu, n), nan=-7.0)), f"replay {t}: {n}"
        sa, sb = _state_tensors(a.gpu), _state_tensors(b.gpu)
        for n in sa:
            assert torch.equal(sa[n], sb[n]), f"replay {t}: state {n}"
        rep = b.compare(t)                  # the replay against the oracle
        assert rep.near_ties == 0, f"replay {t}: near-tie (the eager copy is not re-synchronised)"
        if b.shape.offload and t % 8 == 0:
            b.check_cache()
        if t % 16 == 15 or t == wl.steps - 1:
            b.check_state(f"replay {t}")
    _say(f"[graph] offload={offload}: {summary(b.reports)}")
    assert a.gpu.status_bits() == 0 and b.gpu.status_bits() == 0


# ------------------------------------------------- SparDA layer-ahead order

@pytest.mark.parametrize("offload", [False, True])
def test_forecast_small(offload):
    """Selection one layer ahead with a forecast head (before the append, for
    the length after it) against the oracle over 80 steps from 1000 and 963
    tokens: chunk and block completions, a block opened at 1024 (selected
    before it holds a token: given a slot, not fetched) and the window
    sliding by a block."""
    wl = small_workload(151, context=1000, steps=80, offload=offload)
    _run(wl, lengths=[1000, 963], ahead=True, cache_every=7)


def test_forecast_fetch_wg_long_offload():
    """Layer-ahead selection with the fetch made by 3 looping workgroups
    (many entries each) over 150 steps: copies equal the oracle's misses."""
    wl = small_workload(152, offload=True, steps=150, context=2048, k_blocks=12,
                        k_q_blocks=3, k_e_blocks=9, n_hot=4, batch=3)
    _run(wl, ahead=True, fetch_workgroups=3, cache_every=25)


def test_forecast_1b_32k_sampled():
    """One offloaded layer of the 1B-shaped 32K stack (64 sequences) in the
    layer-ahead order with a 32-workgroup fetch: 3 sampled pairs."""
    _run(WORKLOADS[3], layer=7, check_pairs=[0, 64, 127], steps=8, cache_every=4,
         ahead=True, fetch_workgroups=32)


@pytest.mark.parametrize("n_wg", [1, 7, 64])
def test_fetch_wg_equals_fetch(n_wg):
    """nosa_fetch_delta_wg with any workgroup budget leaves the same slot
    maps, phys, copy counts and cache bytes as nosa_fetch_delta."""
    wl = small_workload(153, context=1500, steps=40, offload=True, k_blocks=12,
                        k_q_blocks=4, k_e_blocks=8, batch=3)
    a = Lockstep(wl, check_pairs=[])
    b = Lockstep(wl, check_pairs=[])
    for t in range(wl.steps):
        kd, vd, qd = a.inputs(t)
        for ls in (a, b):
            ls.gpu.append_select(kd, vd, qd)
        a.gpu.fetch()
        b.gpu.fetch_wg(n_wg)
        torch.cuda.synchronize()
        for n in ("phys", "n_miss"):
            assert torch.equal(getattr(a.gpu, n), getattr(b.gpu, n)), f"step {t}: {n}"
        sa, sb = _state_tensors(a.gpu), _state_tensors(b.gpu)
        for n in sa:
            assert torch.equal(sa[n], sb[n]), f"step {t}: state {n}"


def _stack(wl, n_layers):
    # layer 0 keeps its KV on the GPU (as SparDA does); the rest offload
    return [Lockstep(wl, layer=li, check_pairs=[], ahead=True, offload=li > 0)
            for li in range(n_layers)]


@pytest.mark.parametrize("order", [True, "select"], ids=["beside-decode", "beside-select"])
def test_layer_ahead_stack_overlap_equals_serial(order):
    """The two-stream cross-layer pipeline, in either order (layer l+1's
    selection and fetch on a second stream while layer l appends and
    decodes; or layer l's fetch on the second stream beside layer l+1's
    selection), gives, bit for bit, the outputs, selections and state of the
    same stack run layer by layer on one stream, over 70 steps of 3 layers."""
    from trainable_offloadable_block_amd import LayerAheadStack
    wl = small_workload(154, context=1000, steps=70)
    sa, sb = _stack(wl, 3), _stack(wl, 3)
    pa = LayerAheadStack([ls.gpu for ls in sa], fetch_workgroups=8, overlap=order)
    pb = LayerAheadStack([ls.gpu for ls in sb], fetch_workgroups=8, overlap=False)
    for t in range(wl.steps):
        for pipe, st in ((pa, sa), (pb, sb)):
            ins = []
            for ls in st:
                kd, vd, qd = ls.inputs(t)
                ins.append((ls._dev(ls.f[:, :, t]), kd, vd, qd))
            pipe.step(ins)
        torch.cuda.synchronize()
        for la, lb in zip(sa, sb):
            for n in ("sel", "n_sel", "phys", "n_miss", "out"):
                assert torch.equal(getattr(la.gpu, n), getattr(lb.gpu, n)), f"step {t}: {n}"
            ta, tb = _state_tensors(la.gpu), _state_tensors(lb.gpu)
            for n in ta:
                assert torch.equal(ta[n], tb[n]), f"step {t}: state {n}"
    for st in (sa, sb):
        for ls in st:
            assert ls.gpu.status_bits() == 0


# ------------------------------------------- sparse prefill: bulk block scores

def _prefill_scores_case(wl, T, pos0, check_pairs=None, rows=None):
    import oracle.nosa_oracle as O
    from synth import bf16_bits_to_f64, context_kv, queries
    _say(f"[prefill-scores] {wl.name} T={T} pos0={pos0}")
    ls = Lockstep(wl, check_pairs=[], steps=1)
    B, Hq, Hkv, G = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.group
    wq = wl.replace(steps=T)
    qs = np.stack([np.stack([queries(wq, 0, b, h) for h in range(Hq)], axis=1)
                   for b in range(B)])                                  # [B][T][Hq][128]
    qd = torch.from_numpy(np.ascontiguousarray(qs).view(np.int16)).to(ls.gpu.device)
    out = ls.gpu.prefill_block_scores(qd, T, pos0)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert ls.gpu.status_bits() == 0
    n_s, n_w = wl.n_sink_blocks, wl.window_tokens // 64
    worst = 0.0
    for p in (range(B * Hkv) if check_pairs is None else check_pairs):
        b, g = divmod(p, Hkv)
        K, _ = context_kv(wl, 0, b, g)
        ck = O.compress_keys(bf16_bits_to_f64(K), wl.context)
        Q = bf16_bits_to_f64(qs[b][:, g * G:(g + 1) * G])                # [T][G][128]
        for i in (range(T) if rows is None else rows):
            want = O.prefill_block_scores(Q[i:i + 1], pos0 + i, ck, n_s, n_w)[0]
            got = out[b, g, i, :want.shape[0]]
            fin = np.isfinite(want)
            assert np.array_equal(np.isfinite(got), fin), (p, i)
            assert np.all(out[b, g, i, want.shape[0]:] == -np.inf), (p, i)
            if fin.any():
                rel = np.abs(got[fin] - want[fin]) / np.abs(want[fin])
                worst = max(worst, float(rel.max()))
    _say(f"[prefill-scores] worst relative error {worst:.2e}")
    assert worst < 1e-4


@pytest.mark.parametrize("n_q_heads", [2, 8, 16, 32])
def test_prefill_block_scores_small(n_q_heads):
    """Block scores of 600 prompt queries per sequence at positions 900-1499
    (chunk and block completions, the window moving) for GQA groups of 1, 4,
    8 and 16, every pair and query against the oracle."""
    wl = small_workload(161, context=1500, n_q_heads=n_q_heads, n_kv_heads=2)
    _prefill_scores_case(wl, 600, 900)


def test_prefill_block_scores_from_start():
    """Queries from position 0: rows with no complete chunk or no candidate
    are all -inf."""
    _prefill_scores_case(small_workload(162, context=700), 700, 0)


def test_prefill_block_scores_16k_sampled():
    """The 1B-shaped 16K layer (64 pairs): the last 1024 prompt positions,
    3 pairs x 12 rows against the oracle."""
    rows = [0, 1, 2, 255, 256, 511, 600, 777, 900, 1000, 1022, 1023]
    _prefill_scores_case(WORKLOADS[2], 1024, 16384 - 1024, check_pairs=[0, 33, 63], rows=rows)


def test_prefill_block_scores_short_context_sets_status():
    wl = small_workload(163, context=500)
    ls = Lockstep(wl, check_pairs=[], steps=1)
    q = torch.zeros(wl.batch * 8 * wl.n_q_heads * 128, dtype=torch.int16, device="cuda")
    ls.gpu.prefill_block_scores(q, 8, 493)          # reaches position 501 > 500
    torch.cuda.synchronize()
    assert ls.gpu.status_bits() & 8


# -------------------------------------------- sparse prefill: select + attend

def _prefill_near_tie(Qb, Eb, roles, k_q, k_e_dyn, gsel):
    """True when a prompt query's GPU selection differs from the oracle's only
    at near-ties (the lockstep rule for prompt queries, which have every
    candidate eligible): the sink and window blocks are all there, and some
    set of stage-1 picks -- the oracle's, with blocks whose query-aware score
    lies within TIE_REL of the k_q-th best swapped in and out -- leaves as
    the agnostic picks the oracle's stage 2 over the rest, up to blocks
    within TIE_REL of that stage's k_e'-th best agnostic score."""
    from itertools import combinations
    from nosa_harness import TIE_REL
    cand, gs = roles.candidates, set(gsel)
    base = set(roles.sink) | set(roles.window)
    if not base <= gs:
        return False
    ranked = sorted(cand, key=lambda x: (-Qb[x], x))
    nq = min(k_q, len(cand))
    oq = set(ranked[:nq])
    near = []
    if nq:
        tau_q = Qb[ranked[nq - 1]]
        near = [x for x in cand if abs(Qb[x] - tau_q) <= TIE_REL * abs(tau_q)]
    outs = [x for x in near if x in oq][:6]
    ins = [x for x in near if x not in oq][:6]
    for r in range(min(len(ins), len(outs)) + 1):
        for X in combinations(outs, r):
            for Y in combinations(ins, r):
                qg = (oq - set(X)) | set(Y)
                if not qg <= gs:
                    continue
                pool = sorted((x for x in cand if x not in qg), key=lambda x: (-Eb[x], x))
                ne = min(k_e_dyn, len(pool))
                ag, agn = gs - base - qg, set(pool[:ne])
                if ag == agn:
                    return True
                if ne and len(ag) == ne:
                    tau_e = Eb[pool[ne - 1]]
                    if all(abs(Eb[x] - tau_e) <= TIE_REL * abs(tau_e) for x in ag ^ agn):
                        return True
    return False


def _sparse_prefill_case(wl, T, pos0, check_pairs=None, rows=None):
    import oracle.nosa_oracle as O
    from synth import bf16_bits_to_f64, context_kv, eviction_weights, queries
    _say(f"[sparse-prefill] {wl.name} T={T} pos0={pos0}")
    ls = Lockstep(wl, check_pairs=[], steps=1)
    B, Hq, Hkv, G = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.group
    n_s, n_w = wl.n_sink_blocks, wl.window_tokens // 64
    k_e_dyn = wl.k_e_blocks - n_s - n_w
    wq = wl.replace(steps=T)
    qs = np.stack([np.stack([queries(wq, 0, b, h) for h in range(Hq)], axis=1)
                   for b in range(B)])                                  # [B][T][Hq][128]
    qd = torch.from_numpy(np.ascontiguousarray(qs).view(np.int16)).to(ls.gpu.device)
    out_d, sel_d, nsel_d = ls.gpu.prefill_sparse(qd, T, pos0)
    torch.cuda.synchronize()
    assert ls.gpu.status_bits() == 0
    out, sel, nsel = out_d.cpu().numpy(), sel_d.cpu().numpy(), nsel_d.cpu().numpy()
    got_all, want_all, near = [], [], []
    for p in (range(B * Hkv) if check_pairs is None else check_pairs):
        b, g = divmod(p, Hkv)
        K, V = context_kv(wl, 0, b, g)
        w1, w2 = eviction_weights(wl, 0, g)
        o = O.PairOracle(bf16_bits_to_f64(K), bf16_bits_to_f64(V), bf16_bits_to_f64(w1),
                         bf16_bits_to_f64(w2), wl.context, n_s, n_w, wl.k_q_blocks, k_e_dyn,
                         1.0 if wl.evict_bias else 0.0)
        ck, ec = np.array(o.ckeys), np.array(o.e_chunks)
        Q = bf16_bits_to_f64(qs[b][:, g * G:(g + 1) * G])
        for i in (range(T) if rows is None else rows):
            want, sels = O.prefill_sparse_attend(Q[i:i + 1], pos0 + i, o.K, o.V, o.s, ck, ec,
                                                 n_s, n_w, wl.k_q_blocks, k_e_dyn,
                                                 1.0 if wl.evict_bias else 0.0)
            gsel = [int(x) for x in sel[b, g, i, :nsel[b, g, i]]]
            if gsel != sels[0].blocks:
                L = pos0 + i + 1
                roles = O.block_roles(L, n_s, n_w)
                Qb = O.prefill_block_scores(Q[i:i + 1], pos0 + i, ck, n_s, n_w)[0][:roles.nb]
                Eb = O.block_max_pool(ec[:O.n_chunks(L)], roles.nb)
                assert _prefill_near_tie(Qb, Eb, roles, wl.k_q_blocks, k_e_dyn, gsel), (
                    f"pair {p} query {i}: selection differs beyond near-ties\n"
                    f"gpu {gsel}\noracle {sels[0].blocks}")
                near.append((b, g, i, sels[0].blocks, want[0]))
                continue
            got_all.append(out[b, i, g * G:(g + 1) * G])
            want_all.append(want[0])
    if near:
        # near-tie rows attend again on the oracle's selection
        sel2 = sel.copy()
        nsel2 = nsel.copy()
        for b, g, i, blocks, _ in near:
            sel2[b, g, i] = -1
            sel2[b, g, i, :len(blocks)] = blocks
            nsel2[b, g, i] = len(blocks)
        sel2_d = torch.from_numpy(sel2.reshape(-1)).to(ls.gpu.device)
        nsel2_d = torch.from_numpy(nsel2.reshape(-1)).to(ls.gpu.device)
        out2 = ls.gpu.prefill_attend(qd, T, pos0, sel2_d, nsel2_d, torch.empty_like(out_d))
        torch.cuda.synchronize()
        out2 = out2.cpu().numpy().reshape(out.shape)
        for b, g, i, _, w in near:
            got_all.append(out2[b, i, g * G:(g + 1) * G])
            want_all.append(w)
    got_all, want_all = np.concatenate(got_all), np.concatenate(want_all)
    d = got_all.astype(np.float64) - want_all
    mx = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / np.linalg.norm(want_all))
    _say(f"[sparse-prefill] max-abs {mx:.2e} rel-L2 {rel:.2e} near-ties {len(near)}")
    assert mx <= 1e-2 and rel <= 2e-3


@pytest.mark.parametrize("n_q_heads", [2, 8, 16, 32])
def test_sparse_prefill_small(n_q_heads):
    """Sparse prefill of 300 prompt queries per sequence at positions 700-999:
    per-query selection and attention against the oracle, GQA 1/4/8/16."""
    wl = small_workload(171, context=1000, n_q_heads=n_q_heads, n_kv_heads=2)
    _sparse_prefill_case(wl, 300, 700)


def test_sparse_prefill_from_start_is_full_attention_early():
    """From position 0, queries whose budget covers every block attend
    causally to everything before them."""
    _sparse_prefill_case(small_workload(172, context=600), 600, 0)


def test_sparse_prefill_16k_sampled():
    """The 1B-shaped 16K layer: the last 512 prompt positions, 3 pairs x 8
    rows against the oracle."""
    _sparse_prefill_case(WORKLOADS[2], 512, 16384 - 512, check_pairs=[0, 31, 63],
                         rows=[0, 1, 100, 255, 256, 400, 510, 511])


@pytest.mark.parametrize("context", [24000, 32832, 32896, 36000])
def test_sparse_prefill_long_prompt_sampled(context):
    """Prompt tails past 16K: about 360 candidate blocks per query (one wave
    per query, up to 8 keys a lane), the last prompt length on one wave
    (513 blocks, 510 candidates) and the first past it (the 256-thread
    selection), and about 560 candidates; 64 queries, 2 pairs x 6 rows
    against the oracle."""
    wl = small_workload(173, context=context, k_blocks=40, k_q_blocks=16, k_e_blocks=24)
    _sparse_prefill_case(wl, 64, context - 64, check_pairs=[0, 3], rows=[0, 1, 31, 32, 62, 63])


def test_select_splits_per_workgroup_do_not_change_results():
    """A scoring workgroup that takes several 128-chunk splits one after
    another (the launch shape for large contexts) gives the same selection,
    kinds and scores, bit for bit, as one split per workgroup."""
    # 6000 tokens: 374 chunks in 3 splits; two per workgroup leaves one alone
    wl = small_workload(181, context=6000, steps=20, k_blocks=12, k_q_blocks=4, k_e_blocks=8)
    a = Lockstep(wl, check_pairs=[], fused=True)
    b = Lockstep(wl, check_pairs=[], fused=True)
    for t in range(wl.steps):
        kd, vd, qd = a.inputs(t)
        for ls, subs in ((a, 1), (b, 2)):
            with L.tuning(L.NOSA_TUNE_SELECT_SUBS, subs):
                ls.gpu.append_select(kd, vd, qd, want_kind=True, want_qscore=True)
        torch.cuda.synchronize()
        for n in ("sel", "n_sel", "kind"):
            assert torch.equal(getattr(a.gpu, n), getattr(b.gpu, n)), f"step {t}: {n}"
        assert torch.equal(torch.nan_to_num(a.gpu.dbg_q, nan=-7.0),
                           torch.nan_to_num(b.gpu.dbg_q, nan=-7.0)), f"step {t}: qscore"
        sa, sb = _state_tensors(a.gpu), _state_tensors(b.gpu)
        for n in sa:
            assert torch.equal(sa[n], sb[n]), f"step {t}: state {n}"


@pytest.mark.parametrize("case", ["g4_6k", "g8_boundary_17k", "g8_30k", "g8_boundary_34k",
                                  "tiny_candidates"])
def test_select_pool_paths_agree(case):
    """The selection's two finishing paths -- general (kinds of every block
    in LDS, histogram range refinement, passes over the blocks) and one or
    two candidates per thread (bitonic sorts per wave and binary-search
    ranks) -- give the same selection, kinds, block scores and state, bit
    for bit, step after step. The first decoding step ranks stage 2 (every
    candidate still eligible); the 17K case starts at 255 candidates and
    steps past 256, where a thread takes two candidates; the 30K case has
    about 450; the 34K case starts at 510 and steps past 512, where the
    library leaves the per-thread path; the last case has fewer candidates
    than k_q, and a sequence with none."""
    if case == "g4_6k":
        wl = small_workload(231, context=6000, steps=20, k_blocks=12, k_q_blocks=4, k_e_blocks=8)
        lengths = [6000, 5711]
    elif case == "g8_boundary_17k":
        wl = small_workload(232, batch=1, n_q_heads=16, n_kv_heads=2, context=17350, steps=140,
                            window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                            n_hot=8)
        lengths = None
    elif case == "g8_30k":
        wl = small_workload(234, batch=2, n_q_heads=16, n_kv_heads=2, context=30000, steps=40,
                            window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                            n_hot=8)
        lengths = [30000, 28100]
    elif case == "g8_boundary_34k":
        wl = small_workload(235, batch=1, n_q_heads=16, n_kv_heads=2, context=33700, steps=200,
                            window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                            n_hot=8)
        lengths = None
    else:
        wl = small_workload(233, context=300, steps=40, k_blocks=10, k_q_blocks=4, k_e_blocks=6,
                            n_hot=1)
        lengths = [300, 170]
    runs = [Lockstep(wl, check_pairs=[], lengths=lengths, fused=True) for _ in range(2)]
    for t in range(wl.steps):
        kd, vd, qd = runs[0].inputs(t)
        for ls, mode in zip(runs, (1, 2)):
            with L.tuning(L.NOSA_TUNE_SELECT_POOL, mode):
                ls.gpu.append_select(kd, vd, qd, want_kind=True, want_qscore=True)
        torch.cuda.synchronize()
        a = runs[0].gpu
        for b in (r.gpu for r in runs[1:]):
            for n in ("sel", "n_sel", "kind"):
                assert torch.equal(getattr(a, n), getattr(b, n)), f"{case} step {t}: {n}"
            assert torch.equal(torch.nan_to_num(a.dbg_q, nan=-7.0),
                               torch.nan_to_num(b.dbg_q, nan=-7.0)), f"{case} step {t}: qscore"
            sa, sb = _state_tensors(a), _state_tensors(b)
            for n in sa:
                assert torch.equal(sa[n], sb[n]), f"{case} step {t}: state {n}"


def test_decode_one_split_per_pair():
    """A pair whose whole selection is one workgroup's run (one split: the
    output is normalised and written without the split merge) stays within
    the oracle's tolerance, resident and offloaded."""
    with L.tuning(L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, 64):
        _run(small_workload(191, steps=12), fused=True)
        _run(small_workload(192, steps=12, offload=True), fused=False)


def test_timed_decode_equals_decode():
    """nosa_sparse_decode_timed writes the same output as nosa_sparse_decode,
    bit for bit, and the interval its kernel stamps is positive and inside
    the interval of events recorded around the call."""
    wl = small_workload(193, steps=4)
    ls = Lockstep(wl, check_pairs=[])
    g = ls.gpu
    kd, vd, qd = ls.inputs(0)
    g.append_select(kd, vd, qd, want_kind=True)
    g.fetch()
    g.decode(qd)
    torch.cuda.synchronize()
    ref = g.out.clone()
    g.out.fill_(-1.0)
    e0, e1, a0, a1 = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in (e0, e1):
        e.record()
    a0.record()
    g.decode(qd, events=(e0, e1))
    a1.record()
    torch.cuda.synchronize()
    assert torch.equal(g.out, ref)
    k_ms, c_ms = e0.elapsed_time(e1), a0.elapsed_time(a1)
    assert 0.0 < k_ms <= c_ms + 1e-3, (k_ms, c_ms)
