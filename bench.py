#!/usr/bin/env python3
"""Decode-step benchmark of the NOSA hot path on one MI355X.

Workload: the NOSA-1B-shaped layer (batch 32, 16 query / 2 KV heads,
head_dim 128, 16384-token prefilled context, block 64, 1 sink block, 1024-token
window, k = 64 blocks = 16 query-aware + 48 query-agnostic), KV resident in
HBM, seeded synthetic inputs (see synth/workloads.py). A step is one decode
token through a stack of --layers independent layers of that shape, each
layer running the whole path: compress_append + select (one launch,
nosa_append_select) -> fetch_delta -> sparse_decode. A stack (as in a real
model) keeps one layer's KV from staying in the 256 MB last-level cache
between its steps.

Prints ONE JSON line. value = decode tokens/s per layer = batch * layers *
steps / elapsed. roofline: the sparse-decode kernel's algorithmic bytes per
launch over its HIP-event-timed average duration, against 8 TB/s.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s per layer (batch x steps/s) + % HBM peak, 1B-shape 16K/32K"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA, MI355X


CLOCK_WARM_S = 0.5      # untimed decode launches before each timed region (at least)
CLOCK_WARM_MAX_S = 5.0   # ... and at most, while their launch time has not settled
WARMUPS = []             # what each warm-up took (reported in the JSON line)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--layers", type=int, default=8,
                    help="independent layers of the workload's shape per step")
    ap.add_argument("--cpu-pairs", type=int, default=64)
    ap.add_argument("--cpu-steps", type=int, default=80)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=8)
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the host-link leg (offloaded 128K workload)")
    ap.add_argument("--offload-steps", type=int, default=24)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the many-query block-score (sparse prefill) leg")
    ap.add_argument("--only-next", action="store_true",
                    help="run only the GQA-16 96-block leg and print its JSON")
    ap.add_argument("--phase-workload", type=int, default=2, choices=(1, 2, 3, 4, 5),
                    help="with --phase-clocks: the workload (2: the 16K stack of 8 "
                         "layers; others as stacks of 4)")
    ap.add_argument("--only-32k", action="store_true",
                    help="run only the offloaded 32K stack leg and print its JSON")
    ap.add_argument("--only-8b", action="store_true",
                    help="run only the offloaded 8B-shaped 64K leg and print its JSON")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the many-query block-score leg and print its JSON")
    ap.add_argument("--no-ahead", action="store_true",
                    help="skip the layer-ahead (SparDA order) leg")
    ap.add_argument("--only-ahead", action="store_true",
                    help="run only the layer-ahead leg and print its JSON")
    ap.add_argument("--select-pool", type=int, default=0, choices=(0, 1, 2),
                    help="nosa_set_tuning NOSA_TUNE_SELECT_POOL for the whole run "
                         "(0: the library's choice)")
    ap.add_argument("--select-subs", type=int, default=0,
                    help="nosa_set_tuning NOSA_TUNE_SELECT_SUBS for the whole run "
                         "(0: the library's choice)")
    ap.add_argument("--decode-bps", type=int, default=0,
                    help="nosa_set_tuning NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT for the whole "
                         "run (0: the library's choice)")
    ap.add_argument("--fetch-wg", type=int, default=8,
                    help="workgroup budget of the layer-ahead fetch (8: the budget "
                         "of the fastest two-stream order in the sweep)")
    ap.add_argument("--ahead-steps", type=int, default=64,
                    help="timed steps per order in the layer-ahead leg and its sweep")
    ap.add_argument("--fetch-wg-sweep", type=str, default="", metavar="N,N,...",
                    help="run only the layer-ahead leg, once per workgroup budget, and "
                         "print one JSON list")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the hipGraph replay leg of the same layer stack")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the GQA-16, 96-block leg (beyond the five configs)")
    ap.add_argument("--no-tiny", action="store_true",
                    help="skip the tiny 4K single-layer leg")
    ap.add_argument("--no-microbatch", action="store_true",
                    help="skip the headline stack run as two micro-batches on two streams")
    ap.add_argument("--only-microbatch", action="store_true",
                    help="run only the micro-batch leg and print its JSON")
    ap.add_argument("--mb-workload", type=int, default=2, choices=(2, 3),
                    help="with --only-microbatch: 2 the 16K stack, 3 the offloaded 32K stack")
    ap.add_argument("--mb-count", type=int, default=2, choices=(1, 2, 4),
                    help="with --only-microbatch: micro-batches (1: the plain one-stream run)")
    ap.add_argument("--mb-fetch-wg", type=int, default=0,
                    help="with --only-microbatch and an offloaded workload: looping fetch "
                         "workgroups (0: one workgroup per block)")
    ap.add_argument("--clock-warm", type=float, default=CLOCK_WARM_S, metavar="S",
                    help="least seconds of untimed decode launches before each timed region "
                         "(more while their launch time has not settled)")
    ap.add_argument("--phase-clocks", action="store_true",
                    help="phase breakdown of the append + select and decode launches from the "
                         "timing build's in-kernel clocks (NOSA_LIBRARY=.../libnosa_clocks.so)")
    ap.add_argument("--only-host-link", action="store_true",
                    help="run only the host-link ceiling and the 128K host-link leg, print its JSON")
    ap.add_argument("--only-link", action="store_true",
                    help="run only the host-link ceiling probe and print its JSON")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB first (a known "
                         "byte count for calibrating HBM traffic counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_layer(wl, li, shape, pool, b0=0):
    """Layer li of workload wl holding sequences b0 .. b0 + shape.batch - 1."""
    import numpy as np
    from synth import context_kv, eviction_weights
    from trainable_offloadable_block_amd import NosaLayer
    layer = NosaLayer(shape)
    w = [eviction_weights(wl, li, g) for g in range(wl.n_kv_heads)]
    layer.set_weights(np.stack([x[0] for x in w]), np.stack([x[1] for x in w]))
    P = shape.batch * wl.n_kv_heads
    ctx = list(pool.map(lambda p: context_kv(wl, li, b0 + p // wl.n_kv_heads, p % wl.n_kv_heads),
                        range(P)))
    for p, (K, V) in enumerate(ctx):
        layer.load_pair_context(p, K, V)
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    layer.prefill([wl.context] * shape.batch)
    e1.record()
    torch.cuda.synchronize()
    PREFILL_MS.append((wl.name, e0.elapsed_time(e1)))
    return layer


PREFILL_MS = []          # (workload, ms) of every nosa_prefill_init call


def warm_until_steady(launch_round, label):
    """Untimed rounds of decode launches (launch_round() enqueues one) before
    a timed region: at least CLOCK_WARM_S seconds, then until the last three
    rounds each ran within 2 % of the fastest round so far, at most
    CLOCK_WARM_MAX_S. The GPU idles while the layers are built on the host,
    and its first launches after that run slower; a fixed warm-up cannot
    tell whether they have come back to speed, this one measures it (most
    legs settle within the minimum; the tiny 4K leg, whose rounds last
    0.12 ms, takes about 3 s). Returns the record appended to WARMUPS."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rounds = []
    t0 = time.perf_counter()
    while True:
        e0.record()
        launch_round()
        e1.record()
        torch.cuda.synchronize()
        rounds.append(e0.elapsed_time(e1))
        el = time.perf_counter() - t0
        best = min(rounds)
        settled = len(rounds) >= 3 and max(rounds[-3:]) <= 1.02 * best
        if el >= CLOCK_WARM_MAX_S or (el >= CLOCK_WARM_S and settled):
            break
    rec = {"leg": label, "s": round(el, 2), "rounds": len(rounds),
           "first_round_ms": round(rounds[0], 3), "last_round_ms": round(rounds[-1], 3),
           "settled": bool(settled)}
    WARMUPS.append(rec)
    return rec


def step_inputs(wl, li, n, pool, device, b0=0, nb=None):
    """Per-step q, k_new, v_new for one layer (sequences b0 .. b0 + nb - 1,
    all of them by default), resident on the device: [n][B][Hq][128],
    [n][B][Hkv][128] x2 (bf16 bits as int16)."""
    import numpy as np
    import torch
    from synth import new_tokens, queries
    B, Hq, Hkv = (wl.batch if nb is None else nb), wl.n_q_heads, wl.n_kv_heads
    wl = wl.replace(steps=max(wl.steps, n))     # the same streams, drawn further
    qs = list(pool.map(lambda bh: queries(wl, li, b0 + bh // Hq, bh % Hq)[:n], range(B * Hq)))
    q = np.stack(qs).reshape(B, Hq, n, 128).transpose(2, 0, 1, 3)
    toks = list(pool.map(lambda bg: new_tokens(wl, li, b0 + bg // Hkv, bg % Hkv), range(B * Hkv)))
    k = np.stack([t[0][:n] for t in toks]).reshape(B, Hkv, n, 128).transpose(2, 0, 1, 3)
    v = np.stack([t[1][:n] for t in toks]).reshape(B, Hkv, n, 128).transpose(2, 0, 1, 3)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)  # noqa: E731
    return dev(q), dev(k), dev(v)


def locality_step(prev, cur, seq_len, wl):
    """Per pair: gamma(t), the share of this step's selection S(t) that was in
    S(t-1) or is the block this step's token opened (the oracle's locality()
    definition; bounded below by k_e / k). prev and cur are (sel [P][k],
    n_sel [P]) host arrays; seq_len is the length after the step's append."""
    (ps, pn), (cs, cn) = prev, cur
    g = []
    for p in range(cs.shape[0]):
        if cn[p] <= 0:
            continue
        pos = int(seq_len[p // wl.n_kv_heads]) - 1
        have = set(ps[p, :pn[p]].tolist())
        if pos % 64 == 0:
            have.add(pos // 64)
        g.append(sum(1 for b in cs[p, :cn[p]].tolist() if b in have) / int(cn[p]))
    return g


def token_locality_step(prev, cur, seq_len, wl):
    """Per pair: token-level gamma(t), the share of the tokens of S(t) that
    were also selected at step t-1, leaving out the token this step appended
    (the oracle's token_locality() definition). Arguments as for
    locality_step."""
    (ps, pn), (cs, cn) = prev, cur
    g = []
    for p in range(cs.shape[0]):
        if cn[p] <= 0:
            continue
        L = int(seq_len[p // wl.n_kv_heads])
        have = set(ps[p, :pn[p]].tolist())
        now = kept = 0
        for b in cs[p, :cn[p]].tolist():
            n = max(0, min(64, L - 64 * b))
            if b == (L - 1) // 64:
                n -= 1                               # the step's own token
            now += n
            if b in have:
                kept += max(0, min(64, L - 1 - 64 * b))
        g.append(kept / now if now else 1.0)
    return g


def pct(v, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(v, dtype=float), q)), 2)


def select_bytes(wl, L):
    """Algorithmic bytes of one selection at sequence length L (every
    sequence): each complete chunk's compressed key (bf16), an fp32 score and
    an eviction score per block, the eligibility bits, the group's queries
    (bf16) and the selection list (int32)."""
    B, Hq, Hkv, k = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.k_blocks
    C = (L - 32) // 16 + 1 if L >= 32 else 0
    nb = (L + 63) // 64
    return B * Hkv * (C * 128 * 2 + 2 * nb * 4 + nb / 4) + B * Hq * 128 * 2 + B * Hkv * k * 4


def decode_bytes(wl, n_att_per_pair):
    """Algorithmic bytes of one sparse-decode launch: K, V (bf16) and the
    eviction score (fp32) of every attended token, q (bf16) and out (fp32),
    the selection and slot lists (int32)."""
    B, Hq, Hkv, k = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.k_blocks
    return (n_att_per_pair * B * Hkv * (2 * 128 * 2 + 4) + B * Hq * 128 * (2 + 4)
            + B * Hkv * k * 8)


def attended_tokens(layer, wl):
    """Mean attended tokens per pair of the layer's last decode call."""
    import numpy as np
    k = wl.k_blocks
    sel = layer.sel.cpu().numpy().reshape(-1, k)
    nsel = layer.n_sel.cpu().numpy()
    seq = layer.seq_len.cpu().numpy()
    tot = 0
    for p in range(sel.shape[0]):
        L = int(seq[p // wl.n_kv_heads])
        blocks = sel[p, :nsel[p]].astype(np.int64)
        tot += int(np.minimum(64, L - 64 * blocks).sum())
    return tot / sel.shape[0]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter runs
    (profiles/decode_kernel_traffic.json), or None when the decode kernel's
    sources have changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


_CPU_BARRIER = None
_CPU_BLAS = None


def _oracle_worker_init(barrier):
    """Pool worker set-up: the start barrier, and single-threaded BLAS so that
    the worker processes, not BLAS threads, share the cores."""
    global _CPU_BARRIER, _CPU_BLAS
    _CPU_BARRIER = barrier
    # before numpy loads its BLAS in this process (a spawned interpreter)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401
    try:
        from threadpoolctl import threadpool_limits
        _CPU_BLAS = threadpool_limits(1)
    except Exception:  # pragma: no cover
        _CPU_BLAS = None


def _oracle_pairs(job):
    """One worker's share of the CPU baseline: builds the oracle of its
    pairs (untimed), waits for every worker, then steps them n_steps times.
    Returns (start, end) on the system-wide monotonic clock, and, given the
    GPU's records of the same steps, the parity counts of its pairs."""
    wl_id, pairs, n_steps, gpu = job
    import numpy as np
    import oracle.nosa_oracle as O
    from synth import WORKLOADS, bf16_bits_to_f64, context_kv, eviction_weights, new_tokens, queries
    wl = WORKLOADS[wl_id]
    G, Hkv = wl.group, wl.n_kv_heads
    n_w = wl.window_tokens // 64
    k_e_dyn = wl.k_e_blocks - wl.n_sink_blocks - n_w
    work = []
    for p in pairs:
        b, g = divmod(p, Hkv)
        K, V = context_kv(wl, 0, b, g)
        w1, w2 = eviction_weights(wl, 0, g)
        cap = wl.context + n_steps
        Kf, Vf = np.zeros((cap, 128)), np.zeros((cap, 128))
        Kf[:wl.context], Vf[:wl.context] = bf16_bits_to_f64(K), bf16_bits_to_f64(V)
        o = O.PairOracle(Kf, Vf, bf16_bits_to_f64(w1), bf16_bits_to_f64(w2), wl.context,
                         wl.n_sink_blocks, n_w, wl.k_q_blocks, k_e_dyn, 1.0)
        kn, vn = new_tokens(wl, 0, b, g)
        q = np.stack([queries(wl, 0, b, g * G + h) for h in range(G)])
        work.append((o, bf16_bits_to_f64(kn[:n_steps]), bf16_bits_to_f64(vn[:n_steps]),
                     bf16_bits_to_f64(q[:, :n_steps])))
    _CPU_BARRIER.wait(timeout=900)
    results = [[] for _ in work]
    t0 = time.monotonic()
    for t in range(n_steps):
        for i, (o, kn, vn, q) in enumerate(work):
            results[i].append(o.step(kn[t], vn[t], q[:, t]))
    t1 = time.monotonic()
    return t0, t1, (_parity_pairs(gpu, pairs, results, wl, k_e_dyn) if gpu is not None else None)


def _parity_pairs(gpu, pairs, results, wl, k_e_dyn):
    """The GPU's selections and attention outputs of these pairs, step by
    step, against the oracle's (after the timed stepping). A selection that
    differs must differ only at near-ties -- the sink and window blocks the
    same, every differing query-aware or agnostic block within TIE_REL of
    its stage's boundary score tau -- as the parity tests' protocol
    (tests/nosa_harness.py) decides; a pair is followed until its first
    near-tie (its eligibility then diverges from the oracle's). Outputs are
    compared where the selections are identical."""
    import numpy as np
    import oracle.nosa_oracle as O
    from trainable_offloadable_block_amd import _lib as L
    to_lib = {O.SINK: L.KIND_SINK, O.WINDOW: L.KIND_WINDOW, O.QUERY: L.KIND_QUERY,
              O.AGNOSTIC: L.KIND_AGNOSTIC}
    sel, n_sel, kind, out = gpu
    st = {"pair_steps": 0, "exact": 0, "near_ties": 0, "unexplained": 0,
          "max_abs": 0.0, "sq_diff": 0.0, "sq_want": 0.0}
    for i in range(len(pairs)):
        for t, res in enumerate(results[i]):
            st["pair_steps"] += 1
            gb = [int(x) for x in sel[i][t][:n_sel[i][t]]]
            gk = {int(x): int(c) for x, c in zip(sel[i][t][:n_sel[i][t]], kind[i][t][:n_sel[i][t]])}
            if gb == res.sel.blocks and gk == {x: to_lib[c] for x, c in res.sel.kinds.items()}:
                st["exact"] += 1
                d = out[i][t].astype(np.float64) - res.out
                st["max_abs"] = max(st["max_abs"], float(np.abs(d).max()))
                st["sq_diff"] += float((d * d).sum())
                st["sq_want"] += float((res.out * res.out).sum())
                continue
            gq = {x for x, c in gk.items() if c == L.KIND_QUERY}
            ga = {x for x, c in gk.items() if c == L.KIND_AGNOSTIC}
            base_ok = ({x for x, c in gk.items() if c in (L.KIND_SINK, L.KIND_WINDOW)}
                       == set(res.roles.sink) | set(res.roles.window))
            if base_ok and _near_tie(res, gq, ga, wl.k_q_blocks, k_e_dyn):
                st["near_ties"] += 1
            else:
                st["unexplained"] += 1
            break                                      # the pair's later steps diverge
    return st


TIE_REL = 1e-5                # near-tie band, relative to the stage's boundary score


def _near_tie(res, gq, ga, k_q, k_e_dyn):
    """True when the GPU's query-aware picks gq and agnostic picks ga differ
    from the oracle's result res only among candidates whose score lies
    within TIE_REL of the stage's k-th best score."""
    import oracle.nosa_oracle as O
    cand = res.roles.candidates
    oq = set(res.sel.query)
    if gq != oq:
        ranked = sorted(cand, key=lambda x: (-res.Qb[x], x))
        tau = res.Qb[ranked[min(len(ranked), k_q) - 1]]
        if any(abs(res.Qb[x] - tau) > TIE_REL * abs(tau) for x in gq ^ oq):
            return False
    pool = [x for x in cand if x in res.eligible and x not in gq]
    agn = set(O.top_by_score(pool, res.Eb, k_e_dyn))
    if ga != agn:
        ranked = sorted(pool, key=lambda x: (-res.Eb[x], x))
        tau = res.Eb[ranked[min(len(ranked), k_e_dyn) - 1]]
        if any(abs(res.Eb[x] - tau) > TIE_REL * abs(tau) for x in ga ^ agn):
            return False
    return True


def gpu_records(dev, wl_id, n_steps, workers):
    """Layer 0 of workload wl_id on the GPU for n_steps decode steps (append +
    select, decode), each step's selections, kinds and attention output
    copied to the host: what the CPU baseline's oracle run is checked
    against."""
    import numpy as np
    import torch
    from synth import WORKLOADS
    from trainable_offloadable_block_amd import LayerShape
    wl = WORKLOADS[wl_id]
    shape = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                       wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                       wl.context + n_steps, offload=wl.offload)
    with cf.ThreadPoolExecutor(workers) as pool:
        layer = build_layer(wl, 0, shape, pool)
        q, kn, vn = step_inputs(wl, 0, n_steps, pool, dev)
    P, k = wl.batch * wl.n_kv_heads, wl.k_blocks
    sel, n_sel, kind, out = [], [], [], []
    for t in range(n_steps):
        layer.append_select(kn[t], vn[t], q[t], want_kind=True)
        layer.fetch()
        layer.decode(q[t])
        torch.cuda.synchronize()
        sel.append(layer.sel.cpu().numpy().reshape(P, k))
        n_sel.append(layer.n_sel.cpu().numpy().reshape(P))
        kind.append(layer.kind.cpu().numpy().reshape(P, k))
        out.append(layer.out.float().cpu().numpy().reshape(wl.batch, wl.n_q_heads, 128))
    assert layer.status_bits() == 0
    del layer
    torch.cuda.empty_cache()
    return np.stack(sel), np.stack(n_sel), np.stack(kind), np.stack(out)


def cpu_baseline(wl_id, n_pairs, n_steps, gpu=None):
    """The oracle as it stands, on a bounded sample (n_pairs pairs of layer
    0, n_steps decode steps each: append + select + attend), spread over one
    single-threaded process per host core (at most 16, the GPU's share of a
    box), every process starting together. With gpu (gpu_records of the
    same steps), the oracle's results are then checked against the GPU's:
    the headline configuration's parity at full size."""
    import multiprocessing as mp
    import numpy as np
    from synth import WORKLOADS
    wl = WORKLOADS[wl_id]
    P = wl.batch * wl.n_kv_heads
    pairs = sorted({int(x) for x in np.linspace(0, P - 1, n_pairs)})
    n_proc = max(1, min(16, len(os.sched_getaffinity(0)), len(pairs)))
    shares = [pairs[i::n_proc] for i in range(n_proc)]
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(n_proc)
    G, Hkv = wl.group, wl.n_kv_heads

    def share_records(sh):
        if gpu is None:
            return None
        sel, n_sel, kind, out = gpu
        return ([sel[:, p] for p in sh], [n_sel[:, p] for p in sh], [kind[:, p] for p in sh],
                [out[:, p // Hkv, (p % Hkv) * G:(p % Hkv + 1) * G] for p in sh])
    with ctx.Pool(n_proc, initializer=_oracle_worker_init, initargs=(barrier,)) as pool:
        spans = pool.map(_oracle_pairs, [(wl_id, sh, n_steps, share_records(sh)) for sh in shares],
                         chunksize=1)
    el = max(b for _, b, _ in spans) - min(a for a, _, _ in spans)
    step_s = el / n_steps * (P / len(pairs))          # all P pairs of one layer
    parity = None
    if gpu is not None:
        agg = {}
        for _, _, st in spans:
            for key, v in st.items():
                agg[key] = max(agg.get(key, 0.0), v) if key == "max_abs" else agg.get(key, 0) + v
        rel_l2 = (agg["sq_diff"] / agg["sq_want"]) ** 0.5 if agg["sq_want"] > 0 else 0.0
        ok = agg["unexplained"] == 0 and agg["max_abs"] <= 1e-2 and rel_l2 <= 2e-3
        parity = {"workload": wl.name, "layer": 0, "pairs": len(pairs), "steps": n_steps,
                  "pair_steps_compared": agg["pair_steps"], "selections_identical": agg["exact"],
                  "near_ties": agg["near_ties"], "unexplained_differences": agg["unexplained"],
                  "attention_max_abs": round(agg["max_abs"], 8), "attention_rel_l2": rel_l2,
                  "bars": {"max_abs": 1e-2, "rel_l2": 2e-3, "near_tie_rel": TIE_REL},
                  "verdict": "pass" if ok else "fail",
                  "protocol": "GPU against the float64 oracle over the CPU baseline's steps; "
                              "a pair is followed until its first near-tie; outputs compared "
                              "where selections are identical"}
    return parity, {
        "value": wl.batch / step_s,
        "unit": "tokens/s/layer",
        "cores": n_proc,
        "host_cores": len(os.sched_getaffinity(0)),
        "threads_per_process": 1,
        "kind": "oracle",
        "seconds": round(el, 2),
        "sample": (f"{len(pairs)} of {P} (sequence, KV head) pairs of layer 0 of {wl.name} x "
                   f"{n_steps} decode steps (append+select+attend, float64 numpy), split over "
                   f"{n_proc} single-threaded processes; per-layer step time = wall time of "
                   f"the parallel stepping / steps x {P} / {len(pairs)} pairs"),
    }


def host_link_peak(dev, nbytes=1 << 30, reps=5):
    """The host-to-device link ceiling, measured in this process on a
    contiguous pinned buffer of nbytes: the best of reps DMA copies
    (hipMemcpyAsync through torch) and the best compute-unit read of the
    same buffer through its device alias with nosa_link_copy (the delta
    fetch's load path) over several workgroup counts. The peak is the larger
    of the two."""
    import ctypes
    import torch
    from trainable_offloadable_block_amd import _lib as L

    def ev():
        return torch.cuda.Event(enable_timing=True)
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    memcpy = 0.0
    for _ in range(reps):
        a, b = ev(), ev()
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        memcpy = max(memcpy, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    alias = ctypes.c_void_p()
    L.check(L.lib().nosa_host_alias(ctypes.c_void_p(src.data_ptr()), ctypes.byref(alias)),
            "host_alias")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    cu = {}
    for n_wg in (32, 128, 512, 2048):
        best = 0.0
        for _ in range(reps):
            a, b = ev(), ev()
            a.record()
            L.check(L.lib().nosa_link_copy(alias, ctypes.c_void_p(dst.data_ptr()), nbytes,
                                           n_wg, stream), "link_copy")
            b.record()
            torch.cuda.synchronize()
            best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        cu[n_wg] = round(best, 2)
    assert bool((dst[:4096] == 1).all()) and bool((dst[-4096:] == 1).all())
    del src, dst
    torch.cuda.empty_cache()
    peak = max(memcpy, max(cu.values()))
    return {"bytes": nbytes, "h2d_memcpy_GBps": round(memcpy, 2),
            "cu_read_GBps_by_workgroups": {str(k): v for k, v in cu.items()},
            "peak_GBps": round(peak, 2),
            "peak_from": "memcpy" if memcpy >= max(cu.values()) else "cu_read"}


def hbm_read_ceiling(dev, nbytes=2 << 30, reps=3, launches=5):
    """The practical HBM read rate of this GPU: nosa_hbm_read (a streaming
    read that does nothing else) over nbytes of device memory at several
    workgroup counts, the best of reps runs of `launches` back-to-back
    launches between two events. Reported beside the published peak, which
    stays the roofline's peak."""
    import ctypes
    import torch
    from trainable_offloadable_block_amd import _lib as L
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.fill_(0x01010101)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    by_wg = {}
    for n_wg in (64, 128, 256, 512, 1024):     # 64, 128: what one workgroup streams
        sink = torch.empty(n_wg * 256 * 4, dtype=torch.int32, device=dev)
        best = 0.0
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(launches):
                L.check(L.lib().nosa_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, n_wg,
                                              ctypes.c_void_p(sink.data_ptr()), stream),
                        "hbm_read")
            b.record()
            torch.cuda.synchronize()
            best = max(best, launches * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        by_wg[n_wg] = round(best, 1)
        del sink
    del buf
    torch.cuda.empty_cache()
    best_wg = max(by_wg, key=by_wg.get)
    return {"GBps": by_wg[best_wg], "workgroups": best_wg, "bytes": nbytes,
            "GBps_by_workgroups": {str(k): v for k, v in by_wg.items()},
            "GBps_per_workgroup_at_64": round(by_wg[64] / 64, 2),
            "frac_of_peak": round(by_wg[best_wg] / HBM_PEAK_GBS, 4)}


def fetch_stats(fetched, wl, link_peak):
    """Delta-fetch record of a leg: bytes and time summed over the calls
    (GB/s = total bytes / total time), per-call median and p90, and the time
    the same bytes need at the host-link peak."""
    import numpy as np
    b_tot = float(sum(f[0] for f in fetched))
    us_tot = float(sum(f[1] for f in fetched))
    gbps = b_tot / (us_tot * 1e-6) / 1e9 if us_tot else 0.0
    out = {"calls": len(fetched), "bytes_per_call": int(b_tot / max(1, len(fetched))),
           "us_mean": round(us_tot / max(1, len(fetched)), 1),
           "us_median": pct([f[1] for f in fetched], 50),
           "us_p90": pct([f[1] for f in fetched], 90),
           "GBps": round(gbps, 2),
           "bound_bytes_per_call": wl.batch * wl.n_kv_heads * wl.k_q_blocks * 32768}
    if link_peak:
        out["link_peak_GBps"] = link_peak
        out["us_at_link_peak"] = round(b_tot / max(1, len(fetched)) / (link_peak * 1e9) * 1e6, 1)
        out["frac_of_link_peak"] = round(gbps / link_peak, 4)
    return out


def host_link_leg(n_steps, pool, dev, link):
    """Delta fetch over the host link on the offloaded low-locality 128K
    workload (8 sequences, 32 query / 8 KV heads, k_q = k_e = 32): fetch
    GB/s on the cold first step and in steady state, against the host-link
    peak measured in the same process (host_link_peak), and a per-32-KiB
    hipMemcpy baseline for fragmented copies."""
    import numpy as np
    import torch
    from synth import WORKLOADS
    from trainable_offloadable_block_amd import LayerShape
    wl = WORKLOADS[5]
    shape = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                       wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                       wl.context + n_steps, offload=True)
    layer = build_layer(wl, 0, shape, pool)
    q, kn, vn = step_inputs(wl, 0, n_steps, pool, dev)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # fragmented: 2048 copies of 32 KiB from scattered offsets of 1 GiB
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nb, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(0)
    offs = rng.choice(nb // 32768, size=2048, replace=False) * 32768
    a, b = ev(), ev()
    a.record()
    for o in offs:
        dst[o:o + 32768].copy_(src[o:o + 32768], non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    frag = 2048 * 32768 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    # delta fetch per step
    recs = []
    k = wl.k_blocks
    prev, gammas, tgammas, hits = None, [], [], []
    for t in range(n_steps):
        layer.append_select(kn[t], vn[t], q[t], want_kind=False)
        a, b = ev(), ev()
        a.record()
        layer.fetch()
        b.record()
        layer.decode(q[t])
        torch.cuda.synchronize()
        miss = layer.n_miss.cpu().numpy()
        cur = (layer.sel.cpu().numpy().reshape(-1, k), layer.n_sel.cpu().numpy())
        if t >= 4:
            seq = layer.seq_len.cpu().numpy()
            gammas += locality_step(prev, cur, seq, wl)
            tgammas += token_locality_step(prev, cur, seq, wl)
            hits += [1.0 - m / n for m, n in zip(miss.tolist(), cur[1].tolist()) if n > 0]
        prev = cur
        recs.append((int(miss.sum()) * 32768, a.elapsed_time(b) * 1e3))
    status = layer.status_bits()
    assert not status, f"device status bits set: {status}"
    cold_b, cold_us = recs[0]
    peak = link["peak_GBps"]
    cold_gbps = cold_b / (cold_us * 1e-6) / 1e9
    steady = fetch_stats(recs[4:], wl, peak)
    steady["cache_hit_rate"] = round(float(np.mean(hits)), 4)
    return {
        "workload": wl.name, "pairs": wl.batch * wl.n_kv_heads,
        "link": link,
        "fragmented_32KiB_memcpy_GBps": round(frag, 2),
        "fetch_cold": {"bytes": cold_b, "us": round(cold_us, 1), "GBps": round(cold_gbps, 2),
                       "frac_of_link_peak": round(cold_gbps / peak, 4)},
        "fetch_steady": steady,
        "locality": {"gamma_min": round(float(np.min(gammas)), 4),
                     "gamma_mean": round(float(np.mean(gammas)), 4),
                     "token_gamma_min": round(float(np.min(tgammas)), 4),
                     "token_gamma_mean": round(float(np.mean(tgammas)), 4),
                     "bound": round((k - wl.k_q_blocks) / k, 4), "samples": len(gammas)},
    }


def time_stack(wl, R, W, K, n_bd, dev, workers, graph_steps=0, link_peak=None):
    """Times K decode steps (after W warm-up steps) of a stack of R
    independent layers of workload wl, as plain stream launches. K more
    steps give the decode's launch time: each runs every layer's append +
    select (and fetch) first, then the R decode launches back to back
    between two HIP events on their stream, so a decode follows a kernel
    with no idle gap, as in the timed steps, and the events' own cost is
    shared by R launches (a pair of events stamped by every launch, kept out
    of the first K steps, cost the step about 9 % and each launch about
    2 us); n_bd further steps give a per-call breakdown
    (events recorded around each call) and the exact
    number of attended tokens. With graph_steps, the same stack then runs
    that many steps (after 4 untimed ones) as replays of one captured HIP
    graph of a whole step, each step's inputs copied into the graph's static
    buffer first."""
    import numpy as np
    import torch
    from trainable_offloadable_block_amd import LayerShape
    n_graph = graph_steps + 4 if graph_steps else 0
    n_tok = W + 2 * K + n_bd + n_graph
    shape = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                       wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                       wl.context + n_tok, offload=wl.offload)
    t_setup = time.perf_counter()
    layers, inputs = [], []
    with cf.ThreadPoolExecutor(workers) as pool:
        for li in range(R):
            layers.append(build_layer(wl, li, shape, pool))
            inputs.append(step_inputs(wl, li, n_tok, pool, dev))
            log(f"{wl.name}: layer {li} ready ({time.perf_counter() - t_setup:.1f}s)")
    torch.cuda.synchronize()

    def run_step(t, events=None):
        if events is None:
            for li, layer in enumerate(layers):
                q, kn, vn = inputs[li][0][t], inputs[li][1][t], inputs[li][2][t]
                layer.append_select(kn, vn, q, want_kind=False)
                layer.fetch()
                layer.decode(q)
            return
        i = t - W - K
        if len(layers) == 1:       # one layer: the launch stamps its own events
            layer = layers[0]
            q, kn, vn = inputs[0][0][t], inputs[0][1][t], inputs[0][2][t]
            layer.append_select(kn, vn, q, want_kind=False)
            layer.fetch()
            layer.decode(q, events=(events[0][i], events[1][i]))
            return
        events[2][i].record()                       # every layer's selection, then
        for li, layer in enumerate(layers):
            q, kn, vn = inputs[li][0][t], inputs[li][1][t], inputs[li][2][t]
            layer.append_select(kn, vn, q, want_kind=False)
            layer.fetch()
        events[0][i].record()                       # the R decodes between two events
        for li, layer in enumerate(layers):
            layer.decode(inputs[li][0][t])
        events[1][i].record()

    for t in range(W):
        run_step(t)
    # repeated decode launches (they read the state and rewrite only the
    # output and workspace) bring the GPU to a steady speed before the timed
    # steps

    def warm_round():
        for _ in range(16):
            for li, layer in enumerate(layers):
                layer.decode(inputs[li][0][W - 1] if W > 0 else inputs[li][0][0])
    warm_until_steady(warm_round, wl.name)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(W, W + K):
        run_step(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # the decode's launch time: K more steps with each step's R decodes back
    # to back between two events (created, by a first record, beforehand)
    ev = tuple([torch.cuda.Event(enable_timing=True) for _ in range(K)] for _ in range(3))
    for lst in ev:
        for e in lst:
            e.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for t in range(W + K, W + 2 * K):
        run_step(t, ev)
    torch.cuda.synchronize()
    el_stamped = time.perf_counter() - t1
    dec_ms = [a.elapsed_time(b) / R for a, b in zip(ev[0], ev[1])]   # per launch, step by step
    # the R selections (+ fetches) back to back before them, the same way
    sel_ms = [a.elapsed_time(b) / R for a, b in zip(ev[2], ev[0])] if R > 1 else []

    # per-call breakdown on a few extra steps (untimed region); these steps
    # also give the exact number of attended tokens per decode launch (the
    # stage-2 pool can run short, so a selection may hold fewer than k blocks)
    names = ("append_select", "fetch", "decode")
    bd = {n: [] for n in names}
    layer_step = []                               # us per layer-step (the three calls)
    n_att_samples = []
    fetched = []                                  # (bytes, us) per fetch call
    gammas, tgammas, hits = [], [], []
    k = wl.k_blocks

    def selection(layer):
        return (layer.sel.cpu().numpy().reshape(-1, k), layer.n_sel.cpu().numpy())
    prev = [selection(ly) for ly in layers]
    for t in range(W + 2 * K, W + 2 * K + n_bd):
        for li, layer in enumerate(layers):
            q, kn, vn = inputs[li][0][t], inputs[li][1][t], inputs[li][2][t]
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            evs[0].record()
            layer.append_select(kn, vn, q, want_kind=False)
            evs[1].record()
            layer.fetch()
            evs[2].record()
            layer.decode(q)
            evs[3].record()
            torch.cuda.synchronize()
            for i, n in enumerate(names):
                bd[n].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)
            layer_step.append(evs[0].elapsed_time(evs[3]) * 1e3)
            n_att_samples.append(attended_tokens(layer, wl))
            cur = selection(layer)
            seq = layer.seq_len.cpu().numpy()
            gammas += locality_step(prev[li], cur, seq, wl)
            tgammas += token_locality_step(prev[li], cur, seq, wl)
            prev[li] = cur
            if wl.offload:
                miss = layer.n_miss.cpu().numpy()
                hits += [1.0 - m / n for m, n in zip(miss.tolist(), cur[1].tolist()) if n > 0]
                fetched.append((int(miss.sum()) * 32768, evs[1].elapsed_time(evs[2]) * 1e3))
    graph = None
    if graph_steps:
        graph = graph_replays(layers, inputs, W + 2 * K + n_bd, graph_steps, shape)
    status = [ly.status_bits() for ly in layers]
    assert not any(status), f"device status bits set: {status}"
    dec_us = [x * 1e3 for x in dec_ms]
    out = {"value": wl.batch * R * K / el, "elapsed": el,
           "decode_timing_steps": {"steps": K, "ms_per_step": round(el_stamped / K * 1e3, 4)},
           "n_att": float(np.mean(n_att_samples)),
           "dec_avg_s": float(np.mean(dec_ms)) / 1e3,
           "dec_launch_us": {"median": pct(dec_us, 50), "p90": pct(dec_us, 90),
                             "launches": len(dec_us) * R,
                             "samples": ("per launch" if R == 1 else
                                         f"{len(dec_us)} step means of {R} launches")},
           "sel_launch_us": ({"mean": round(float(np.mean(sel_ms)) * 1e3, 2),
                              "median": pct([x * 1e3 for x in sel_ms], 50),
                              "p90": pct([x * 1e3 for x in sel_ms], 90),
                              "launches": len(sel_ms) * R,
                              "samples": f"{len(sel_ms)} step means of {R} calls"}
                             if sel_ms else None),
           "breakdown": {n: round(float(np.median(v)), 2) for n, v in bd.items()},
           "breakdown_p90": {n: pct(v, 90) for n, v in bd.items()},
           "layer_step_us": {"median": pct(layer_step, 50), "p90": pct(layer_step, 90),
                             "samples": len(layer_step)}}
    out["locality"] = {"gamma_min": round(float(np.min(gammas)), 4),
                       "gamma_mean": round(float(np.mean(gammas)), 4),
                       "token_gamma_min": round(float(np.min(tgammas)), 4),
                       "token_gamma_mean": round(float(np.mean(tgammas)), 4),
                       "bound": round((k - wl.k_q_blocks) / k, 4),
                       "samples": len(gammas), "steps": n_bd}
    if fetched:
        out["fetch"] = fetch_stats(fetched, wl, link_peak)
        out["fetch"]["cache_hit_rate"] = round(float(np.mean(hits)), 4)
    if graph is not None:
        out["graph"] = {"steps": graph_steps, "ms_per_step": round(graph * 1e3 / graph_steps, 4),
                        "value": round(wl.batch * R * graph_steps / graph, 1)}
    layers.clear()
    inputs.clear()
    torch.cuda.empty_cache()
    return out


def graph_replays(layers, inputs, t0, n, shape):
    """Captures one step of every layer (append_select, fetch, decode) as a
    HIP graph over a static input buffer, then replays it for steps t0 + 4 ..
    t0 + 4 + n - 1 (4 untimed first); returns the timed seconds. The length
    hint is the layers' capacity, so the baked grid sizes hold for every
    replay."""
    import torch
    R = len(layers)
    parts = [[inputs[li][j] for j in range(3)] for li in range(R)]
    sizes = [x[0].numel() for row in parts for x in row]
    static = torch.empty(sum(sizes), dtype=torch.int16, device=parts[0][0].device)
    views, off = [], 0
    for row in parts:
        v = []
        for x in row:
            v.append(static[off:off + x[0].numel()].view(x[0].shape))
            off += x[0].numel()
        views.append(v)
    packed = torch.stack([torch.cat([x[t].reshape(-1) for row in parts for x in row])
                          for t in range(t0, t0 + n + 4)])
    saved = [ly.max_len for ly in layers]
    for ly in layers:
        ly.max_len = shape.max_context - 1       # becomes the bound inside
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for li, ly in enumerate(layers):
                q, kn, vn = views[li]
                ly.append_select(kn, vn, q, want_kind=False)
                ly.fetch()
                ly.decode(q)
    torch.cuda.current_stream().wait_stream(side)
    for ly, m in zip(layers, saved):
        ly.max_len = m
    for t in range(4):
        static.copy_(packed[t])
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for t in range(4, n + 4):
        static.copy_(packed[t])
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t1
    for ly in layers:                            # the lengths moved on by n + 4
        ly.max_len = min(ly.max_len + n + 4, shape.max_context)
    return el


def offload_32k_leg(dev, workers, R=4, W=4, K=24, n_bd=8, link_peak=None):
    """The offloaded 32K 1B-shaped stack (64 sequences, 16/2 heads, k = 64,
    full KV in pinned host memory; R of its 28 layers): decode tokens/s per
    layer with the delta fetch on the step path, and the decode kernel
    (reading the device block cache) against the HBM roofline."""
    from synth import WORKLOADS
    wl = WORKLOADS[3]
    m = time_stack(wl, R, W, K, n_bd, dev, workers, link_peak=link_peak)
    dbytes = decode_bytes(wl, m["n_att"])
    ach = dbytes / m["dec_avg_s"] / 1e9
    return {"workload": wl.name, "layers_per_step": R, "steps": K,
            "value": round(m["value"], 1), "unit": "tokens/s/layer",
            "ms_per_step": round(m["elapsed"] * 1e3 / K, 4),
            "decode": {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": int(dbytes),
                       "avg_launch_us": round(m["dec_avg_s"] * 1e6, 2),
                       "attended_tokens_per_pair": round(m["n_att"], 2)},
            "breakdown_us": m["breakdown"], "breakdown_p90_us": m["breakdown_p90"],
            "layer_step_us": m["layer_step_us"], "delta_fetch": m.get("fetch"),
            "locality": m["locality"]}


def offload_8b_64k_leg(dev, workers, W=4, K=32, n_bd=8, link_peak=None):
    """The offloaded 8B-shaped 64K layer (32 sequences, 32/8 heads, k = 64,
    full KV in pinned host memory), one layer timed repeatedly: decode
    tokens/s with the delta fetch on the step path, and the decode kernel
    (256 pairs, one workgroup each, reading the device block cache) against
    the HBM roofline."""
    from synth import WORKLOADS
    wl = WORKLOADS[4]
    m = time_stack(wl, 1, W, K, n_bd, dev, workers, link_peak=link_peak)
    dbytes = decode_bytes(wl, m["n_att"])
    ach = dbytes / m["dec_avg_s"] / 1e9
    return {"workload": wl.name, "layers_per_step": 1, "steps": K,
            "value": round(m["value"], 1), "unit": "tokens/s/layer",
            "ms_per_step": round(m["elapsed"] * 1e3 / K, 4),
            "decode": {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": int(dbytes),
                       "avg_launch_us": round(m["dec_avg_s"] * 1e6, 2),
                       "attended_tokens_per_pair": round(m["n_att"], 2)},
            "breakdown_us": m["breakdown"], "breakdown_p90_us": m["breakdown_p90"],
            "layer_step_us": m["layer_step_us"], "delta_fetch": m.get("fetch"),
            "locality": m["locality"]}


def forecast_inputs(wl, li, n, pool, device):
    """Per-step forecast heads that select layer li: [n][B][Hkv][128]."""
    import numpy as np
    import torch
    from synth import forecasts
    B, Hkv = wl.batch, wl.n_kv_heads
    wl = wl.replace(steps=max(wl.steps, n))
    fs = list(pool.map(lambda bg: forecasts(wl, li, *divmod(bg, Hkv))[:n], range(B * Hkv)))
    f = np.stack(fs).reshape(B, Hkv, n, 128).transpose(2, 0, 1, 3)
    return torch.from_numpy(np.ascontiguousarray(f).view(np.int16)).to(device)


def layer_ahead_leg(dev, workers, R=4, W=4, K=64, n_bd=4, n_wg=8, sweep=None):
    """SparDA's layer-ahead order on the 1B-shaped 32K stack (64 sequences,
    16/2 heads, k = 64; R of its 28 layers, layer 0's KV on the GPU and the
    rest in pinned host memory, as SparDA keeps layer 0 resident): each
    layer's blocks are selected by a forecast head before its append, and
    fetched with n_wg looping workgroups. The same layers run K steps
    layer by layer on one stream, then K steps with layer l+1's selection and
    fetch on a second stream beside layer l's append and decode, then K steps
    with layer l's fetch on the second stream beside layer l+1's selection
    (overlap_beside_select). With sweep
    (a list of workgroup budgets), the same built stack is timed once per
    budget and the result holds one record per budget."""
    import numpy as np
    import torch
    from synth import WORKLOADS
    from trainable_offloadable_block_amd import LayerAheadStack, LayerShape
    wl = WORKLOADS[3]
    budgets = list(sweep) if sweep else [n_wg]
    n_tok = len(budgets) * (3 * W + 3 * K + n_bd)
    t_setup = time.perf_counter()
    layers, ins = [], []
    with cf.ThreadPoolExecutor(workers) as pool:
        for li in range(R):
            shape = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                               wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                               wl.context + n_tok, offload=li > 0)
            layers.append(build_layer(wl, li, shape, pool))
            q, k, v = step_inputs(wl, li, n_tok, pool, dev)
            ins.append((forecast_inputs(wl, li, n_tok, pool, dev), k, v, q))
            log(f"layer-ahead: layer {li} ready ({time.perf_counter() - t_setup:.1f}s)")
    torch.cuda.synchronize()

    def run(pipe, t0, n):
        for t in range(t0, t0 + n):
            pipe.step([tuple(x[t] for x in ins[li]) for li in range(R)])

    records = []
    t = 0
    for nw in budgets:
        serial = LayerAheadStack(layers, fetch_workgroups=nw, overlap=False)
        overlap = LayerAheadStack(layers, fetch_workgroups=nw, overlap=True)
        beside_select = LayerAheadStack(layers, fetch_workgroups=nw, overlap="select")
        res = {"workload": wl.name + "-layer-ahead", "layers_per_step": R, "steps": K,
               "fetch_workgroups": nw, "unit": "tokens/s/layer",
               "layer0": "resident (SparDA keeps layer 0 on the GPU)"}
        for name, pipe in (("serial", serial), ("overlap", overlap),
                           ("overlap_beside_select", beside_select)):
            run(pipe, t, W)
            torch.cuda.synchronize()
            t += W
            t0 = time.perf_counter()
            run(pipe, t, K)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            t += K
            res[name] = {"value": round(wl.batch * R * K / el, 1),
                         "ms_per_step": round(el * 1e3 / K, 4)}
        res["speedup"] = round(res["overlap"]["value"] / res["serial"]["value"], 3)
        res["speedup_beside_select"] = round(
            res["overlap_beside_select"]["value"] / res["serial"]["value"], 3)
        # per-call breakdown of the offloaded layers, serial order (untimed)
        names = ("select_forecast", "fetch_wg", "append", "decode")
        bd = {n: [] for n in names}
        fetched = []
        for _ in range(n_bd):
            for li in range(1, R):
                f, k, v, q = (x[t] for x in ins[li])
                ly = layers[li]
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                evs[0].record()
                ly.select_forecast(f, want_kind=False)
                evs[1].record()
                ly.fetch_wg(nw)
                evs[2].record()
                ly.append(k, v)
                evs[3].record()
                ly.decode(q)
                evs[4].record()
                torch.cuda.synchronize()
                for i, n in enumerate(names):
                    bd[n].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)
                fetched.append((int(ly.n_miss.sum().item()) * 32768,
                                evs[1].elapsed_time(evs[2]) * 1e3))
            t += 1
        res["breakdown_us"] = {n: round(float(np.median(v)), 2) for n, v in bd.items()}
        b_ = float(np.mean([x[0] for x in fetched]))
        us = float(np.mean([x[1] for x in fetched]))
        res["fetch"] = {"bytes_per_call": int(b_), "us_mean": round(us, 1),
                        "GBps": round(b_ / (us * 1e-6) / 1e9, 2)}
        res["decode_beside_us"] = decode_beside(layers[1], ins[1][3][t - 1], layers[2], nw)
        records.append(res)
    status = [ly.status_bits() for ly in layers]
    assert not any(status), f"device status bits set: {status}"
    layers.clear()
    ins.clear()
    torch.cuda.empty_cache()
    return records if sweep else records[0]


def decode_beside(dec_layer, q, fetch_layer, n_wg, n=6):
    """Median decode-launch time (us) of dec_layer alone, beside a large
    delta fetch of fetch_layer on a second stream (its cache emptied first,
    so every selected block is copied by n_wg workgroups reading host
    memory), and beside a 256 MiB pinned-host-to-device copy on the DMA
    engines. Emptying fetch_layer's cache drops the tokens its newest block
    holds only there, so that layer's later outputs are not meaningful (its
    timings still are; a budget sweep goes on stepping it)."""  
    import numpy as np
    import torch
    side = torch.cuda.Stream()
    pin = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dec_layer.device)

    def decodes():
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record()
            dec_layer.decode(q)
            b.record()
        return evs

    out = {}
    for mode in ("alone", "fetch_wg", "dma_copy"):
        torch.cuda.synchronize()
        if mode == "fetch_wg":
            fetch_layer.slot_of_block.fill_(-1)
            fetch_layer.block_of_slot.fill_(-1)
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                fetch_layer.fetch_wg(n_wg)
        elif mode == "dma_copy":
            with torch.cuda.stream(side):
                dst.copy_(pin, non_blocking=True)
        evs = decodes()
        torch.cuda.synchronize()
        out[mode] = round(float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs])), 1)
    return out


def attend_roofline(head_tokens, us):
    """The prompt attention against the bf16 MFMA peak: 4 x 128 flop per
    (query head, attended token) -- the Q K^T logit and the P V product --
    over the launch time (the kernel splits P into bf16 hi + lo for P V,
    which doubles that product's MFMA work; the algorithmic count is the
    plain one)."""
    tf = 4 * 128 * head_tokens / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "flop_per_launch": int(4 * 128 * head_tokens)}


def prefill_scores_leg(dev, workers, T=4096, K=10):
    """Block scores of T prompt queries per sequence at once (the selection
    side of NOSA_S's sparse prefill) on the 16K 1B-shaped layer: the last T
    positions of the 16K prompt, all 64 pairs; MFMA rate of the logits."""
    import numpy as np
    import torch
    from synth import WORKLOADS, queries
    from trainable_offloadable_block_amd import LayerShape
    wl = WORKLOADS[2]
    pos0 = wl.context - T
    shape = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                       wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                       wl.context + 1)
    with cf.ThreadPoolExecutor(workers) as pool:
        layer = build_layer(wl, 0, shape, pool)
        wq = wl.replace(steps=T)
        B, Hq = wl.batch, wl.n_q_heads
        qs = list(pool.map(lambda bh: queries(wq, 0, *divmod(bh, Hq)), range(B * Hq)))
    q = np.stack(qs).reshape(B, Hq, T, 128).transpose(0, 2, 1, 3)
    qd = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to(dev)
    del qs, q
    layer.prefill_block_scores(qd, T, pos0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in evs:
        a.record()
        layer.prefill_block_scores(qd, T, pos0)
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))
    assert layer.status_bits() == 0
    chunks = sum((pos0 + i + 1 - 32) // 16 + 1 for i in range(T))          # per (query, head)
    flops = 2.0 * 128 * chunks * wl.n_q_heads * wl.batch                    # one logit pass
    nb = -(-(pos0 + T) // 64)
    out_bytes = wl.batch * wl.n_kv_heads * T * nb * 4
    res = {"workload": wl.name + "-prompt-scores", "queries_per_sequence": T, "pos0": pos0,
           "us": round(us, 1), "queries_per_s": round(wl.batch * T / (us * 1e-6), 1),
           "logit_TFLOPs": round(flops / (us * 1e-6) / 1e12, 1), "peak_TFLOPs": 2500.0,
           "frac": round(flops / (us * 1e-6) / 1e12 / 2500.0, 4),
           "out_bytes": out_bytes}
    # the whole sparse prefill of the same queries: scores, per-query
    # selection, attention (each query attends as a decode step would)
    import ctypes
    from trainable_offloadable_block_amd import _lib as L
    P, k = layer.shape.pairs, layer.shape.k_blocks
    scores = layer.prefill_block_scores(qd, T, pos0)
    sel = torch.empty(P * T * k, dtype=torch.int32, device=dev)
    nsel = torch.empty(P * T, dtype=torch.int32, device=dev)
    out = torch.empty(wl.batch * T * wl.n_q_heads * 128, dtype=torch.float32, device=dev)
    lib = L.lib()

    def sel_call():
        L.check(lib.nosa_prefill_select(ctypes.byref(layer.cfg), ctypes.byref(layer.state),
                                        ctypes.c_void_p(scores.data_ptr()), T, pos0,
                                        ctypes.c_void_p(sel.data_ptr()),
                                        ctypes.c_void_p(nsel.data_ptr()), layer.stream), "sel")

    def att_call():
        L.check(lib.nosa_prefill_attend(ctypes.byref(layer.cfg), ctypes.byref(layer.state),
                                        ctypes.c_void_p(qd.data_ptr()), T, pos0,
                                        ctypes.c_void_p(sel.data_ptr()),
                                        ctypes.c_void_p(nsel.data_ptr()),
                                        ctypes.c_void_p(out.data_ptr()), layer.stream), "att")

    times = {}
    for name, fn in (("select", sel_call), ("attend", att_call)):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(3)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        times[name] = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
    n_att = float(nsel.float().mean().item()) * 64            # tokens per (query, pair), about
    assert layer.status_bits() == 0
    total = us + times["select"] + times["attend"]
    res["sparse_prefill"] = {
        "select_us": round(times["select"], 1), "attend_us": round(times["attend"], 1),
        "total_us": round(total, 1), "prompt_tokens_per_s": round(wl.batch * T / (total * 1e-6), 1),
        "attended_tokens_per_query_pair": round(n_att, 1),
        "attend_kv_GBps_if_unshared": round(wl.batch * wl.n_kv_heads * T * n_att * 516 /
                                            (times["attend"] * 1e-6) / 1e9, 1),
        # the attention's own roofline: its contractions on MFMA, 2 x 128
        # flop per (query head, attended token) for Q K^T and as many for P V
        "attend_roofline": attend_roofline(wl.batch * wl.n_q_heads * T * n_att, times["attend"])}
    del layer, qd, scores, sel, nsel, out
    torch.cuda.empty_cache()
    return res


def next_leg(dev, workers, R=4, W=8, K=48):
    """The GQA-16, 96-block workload (beyond the five benchmark configs):
    step throughput and the decode kernel against the HBM roofline."""
    from synth import NEXT_WORKLOADS
    wl = NEXT_WORKLOADS["gqa16-k96"]
    m = time_stack(wl, R, W, K, 2, dev, workers)
    dbytes = decode_bytes(wl, m["n_att"])
    ach = dbytes / m["dec_avg_s"] / 1e9
    return {"workload": wl.name, "layers_per_step": R, "steps": K,
            "value": round(m["value"], 1), "unit": "tokens/s/layer",
            "ms_per_step": round(m["elapsed"] * 1e3 / K, 4),
            "decode": {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": int(dbytes),
                       "avg_launch_us": round(m["dec_avg_s"] * 1e6, 2),
                       "attended_tokens_per_pair": round(m["n_att"], 2)},
            "breakdown_us": m["breakdown"], "locality": m["locality"]}


def microbatch_leg(dev, workers, R=8, W=12, K=120, n_mb=2, wl_id=2, fetch_wg=None):
    """A stack of R layers of workload wl_id (by default the headline: the
    16K workload's 32 sequences, 8 layers) run as n_mb micro-batches of
    batch / n_mb sequences, each on its own HIP stream
    (default priority) and its own layers, a step issuing every
    micro-batch's whole R-layer step in turn: the sequences are independent,
    so one micro-batch's latency-bound selection runs beside another's
    HBM-bound decode. Every sequence still goes through every layer in order
    (append + select, then decode), as in the headline's single stream. An
    offloaded workload fetches each layer's missing blocks between the two
    (with fetch_wg, by that many looping workgroups, which leave the CUs to
    the other stream's kernels, instead of one workgroup per block).
    value = decode tokens/s per layer over K timed steps."""
    import torch
    from synth import WORKLOADS
    from trainable_offloadable_block_amd import LayerShape
    wl = WORKLOADS[wl_id]
    nb = wl.batch // n_mb
    n_tok = W + K
    shape = LayerShape(nb, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks, wl.window_tokens,
                       wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks, wl.context + n_tok,
                       offload=wl.offload)
    mbs = []
    with cf.ThreadPoolExecutor(workers) as pool:
        for m in range(n_mb):
            layers = [build_layer(wl, li, shape, pool, b0=m * nb) for li in range(R)]
            inputs = [step_inputs(wl, li, n_tok, pool, dev, b0=m * nb, nb=nb) for li in range(R)]
            mbs.append((layers, inputs))
    streams = [torch.cuda.Stream(dev) for _ in range(n_mb)]
    torch.cuda.synchronize()

    def step(t):
        for (layers, inputs), s in zip(mbs, streams):
            with torch.cuda.stream(s):
                for li, layer in enumerate(layers):
                    q, kn, vn = inputs[li][0][t], inputs[li][1][t], inputs[li][2][t]
                    layer.append_select(kn, vn, q, want_kind=False)
                    if fetch_wg:
                        layer.fetch_wg(fetch_wg)
                    else:
                        layer.fetch()
                    layer.decode(q)

    for t in range(W):
        step(t)
    torch.cuda.synchronize()

    def warm_round():
        for _ in range(4):
            for layers, inputs in mbs:
                for li, layer in enumerate(layers):
                    layer.decode(inputs[li][0][W - 1])
    warm_until_steady(warm_round, f"microbatch-{wl.name}")
    t0 = time.perf_counter()
    for t in range(W, W + K):
        step(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return {"workload": wl.name, "micro_batches": n_mb, "sequences_each": nb, "streams": n_mb,
            "fetch_workgroups": fetch_wg, "layers_per_step": R, "steps": K, "unit": "tokens/s/layer",
            "value": round(wl.batch * R * K / el, 1), "ms_per_step": round(el * 1e3 / K, 4)}


def tiny_leg(dev, workers, W=4, K=32):
    """The tiny single-layer 4K workload (batch 1, 16/2 heads, k = 16 blocks:
    4 query-aware + 12 agnostic, window 256): its 32 decode steps, a
    latency-bound launch chain, as stream launches and as replays of one
    captured HIP graph of a whole step."""
    from synth import WORKLOADS
    wl = WORKLOADS[1]
    m = time_stack(wl, 1, W, K, K, dev, workers, graph_steps=K)
    dbytes = decode_bytes(wl, m["n_att"])
    return {"workload": wl.name, "layers_per_step": 1, "steps": K,
            "value": round(m["value"], 1), "unit": "tokens/s/layer",
            "ms_per_step": round(m["elapsed"] * 1e3 / K, 4),
            "decode": {"bytes_per_launch": int(dbytes), "launch_us": m["dec_launch_us"],
                       "achieved": round(dbytes / m["dec_avg_s"] / 1e9, 1), "unit": "GB/s",
                       "bound": "latency (about 1 MB per launch)"},
            "breakdown_us": m["breakdown"], "breakdown_p90_us": m["breakdown_p90"],
            "layer_step_us": m["layer_step_us"], "graph_replay": m.get("graph"),
            "locality": m["locality"]}


def warm_leg(dev, workers, W=8, K=120):
    """The headline 16K layer alone, stepped repeatedly: its ~150 MB working
    set partly stays in the 256 MB last-level cache between steps, so these
    are warm numbers, labelled as such (the headline stack of 8 layers is the
    cold case)."""
    from synth import WORKLOADS
    wl = WORKLOADS[2]
    m = time_stack(wl, 1, W, K, 2, dev, workers)
    dbytes = decode_bytes(wl, m["n_att"])
    ach = dbytes / m["dec_avg_s"] / 1e9
    return {"workload": wl.name, "cache": "warm (one layer repeated)", "layers_per_step": 1,
            "steps": K, "value": round(m["value"], 1), "unit": "tokens/s/layer",
            "ms_per_step": round(m["elapsed"] * 1e3 / K, 4),
            "decode": {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(ach / HBM_PEAK_GBS, 4),
                       "avg_launch_us": round(m["dec_avg_s"] * 1e6, 2)},
            "breakdown_us": m["breakdown"]}


def phase_clocks(dev, workers, R=8, W=12, samples=24, wl_id=2):
    """Phase breakdown of the fused append + select and the decode launches
    on a stack of R layers of workload wl_id (the 16K stack by default; an
    offloaded workload runs its delta fetch between the two), from the
    timing build's in-kernel clocks (load it with
    NOSA_LIBRARY=trainable_offloadable_block_amd/libnosa_clocks.so). Every
    other sampled step stops after the last layer's append + select (its
    clocks copied out, the earlier launches having run back to back); the
    others run whole and copy out the last layer's decode clocks. Times in
    us from the launch's first workgroup start (100 MHz counter)."""
    import ctypes
    import numpy as np
    import torch
    from synth import WORKLOADS
    from trainable_offloadable_block_amd import LayerShape
    from trainable_offloadable_block_amd import _lib as L
    lib = L.lib()
    if not hasattr(lib, "nosa_phase_clocks_decode"):
        raise SystemExit("--phase-clocks needs the timing build: python -m "
                         "trainable_offloadable_block_amd.build --phase-clocks, then "
                         "NOSA_LIBRARY=trainable_offloadable_block_amd/libnosa_clocks.so")
    readers = {}
    for name in ("append_select", "decode"):
        fn = getattr(lib, f"nosa_phase_clocks_{name}")
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        readers[name] = fn
    NP, ROWS, SLOTS = 512, 40, 16
    wl = WORKLOADS[wl_id]
    P = wl.batch * wl.n_kv_heads
    n_tok = W + samples
    shape = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                       wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                       wl.context + n_tok, offload=wl.offload)
    layers, inputs = [], []
    with cf.ThreadPoolExecutor(workers) as pool:
        for li in range(R):
            layers.append(build_layer(wl, li, shape, pool))
            inputs.append(step_inputs(wl, li, n_tok, pool, dev))
    torch.cuda.synchronize()

    def read(name):
        buf = np.zeros(NP * ROWS * SLOTS, dtype=np.uint64)
        L.check(readers[name](ctypes.c_void_p(buf.ctypes.data), buf.nbytes, 1), name)
        return buf.reshape(NP, ROWS, SLOTS)[:P].astype(np.float64)

    for t in range(W):
        for li, ly in enumerate(layers):
            q, kn, vn = (x[t] for x in inputs[li])
            ly.append_select(kn, vn, q, want_kind=False)
            ly.fetch()
            ly.decode(q)
    def warm_round():
        for _ in range(16):
            for li, ly in enumerate(layers):
                ly.decode(inputs[li][0][W - 1])
    warm_until_steady(warm_round, f"phase-clocks-{wl.name}")
    sel_runs, dec_runs = [], []
    for sidx in range(samples):
        t = W + sidx
        for name in readers:
            readers[name](None, 0, 1)
        for li, ly in enumerate(layers):
            q, kn, vn = (x[t] for x in inputs[li])
            ly.append_select(kn, vn, q, want_kind=False)
            if li == R - 1 and sidx % 2 == 0:
                torch.cuda.synchronize()
                sel_runs.append(read("append_select"))
            ly.fetch()
            ly.decode(q)
        torch.cuda.synchronize()
        if sidx % 2 == 1:
            dec_runs.append(read("decode"))

    def us(a, t0):
        return (a - t0) / 100.0

    def stat(v):
        v = np.asarray(v, dtype=float)
        return {"mean": round(float(v.mean()), 2), "max": round(float(v.max()), 2)}

    sel = {k: [] for k in ("start", "score_done", "score_done_max", "score_landed",
                           "append_done", "append_done_max", "append_landed", "last_arrival",
                           "last_arrival_max", "pool_loads", "pool_factors", "pool_chunk_scores",
                           "pool_stage1", "pool_stage2", "pool_list", "pool_eligibility",
                           "pool_eligibility_max", "end", "stage1_keys", "stage1_r0_minmax",
                           "stage1_r0_hist", "stage1_r0_end", "stage1_rounds", "stage2_rounds",
                           "stage2_ranked")}
    for a in sel_runs:
        rows = np.nonzero((a[:, :, 0] > 0).any(axis=0))[0]
        n_wg = int(rows[rows < ROWS - 1].max())          # the append workgroup's row
        t0 = a[:, :n_wg + 1, 0].min()
        sel["start"].append(stat(us(a[:, :n_wg + 1, 0], t0))["max"])
        sel["score_done"].append(float(us(a[:, :n_wg, 1], t0).mean()))
        sel["score_done_max"].append(float(us(a[:, :n_wg, 1], t0).max()))
        sel["score_landed"].append(float(us(a[:, :n_wg, 2], t0).mean()))
        sel["append_done"].append(float(us(a[:, n_wg, 1], t0).mean()))
        sel["append_done_max"].append(float(us(a[:, n_wg, 1], t0).max()))
        sel["append_landed"].append(float(us(a[:, n_wg, 2], t0).mean()))
        arr = us(a[:, :n_wg, 3].max(axis=1), t0)            # the pool's start, per pair
        sel["last_arrival"].append(float(arr.mean()))
        sel["last_arrival_max"].append(float(arr.max()))
        for k, slot in (("pool_loads", 4), ("pool_factors", 5), ("pool_chunk_scores", 6),
                        ("stage1_keys", 0), ("stage1_r0_minmax", 1), ("stage1_r0_hist", 2),
                        ("stage1_r0_end", 3),
                        ("pool_stage1", 7), ("pool_stage2", 8), ("pool_list", 9),
                        ("pool_eligibility", 10)):
            col = a[:P, ROWS - 1, slot]
            if (col > 0).all():        # slots 1-3: stamped by the range refinement only
                sel[k].append(float(us(col, t0).mean()))
        sel["pool_eligibility_max"].append(float(us(a[:, ROWS - 1, 10], t0).max()))
        sel["end"].append(float(max(us(a[:, ROWS - 1, 11], t0).max(),
                                    us(a[:, n_wg, 2], t0).max())))
        # counts, not clocks: refinement rounds of each top-k stage and the
        # candidates stage 2 ranks (eligible and not taken by stage 1)
        for k, slot in (("stage1_rounds", 12), ("stage2_rounds", 13), ("stage2_ranked", 14)):
            sel[k].append(float(a[:, ROWS - 1, slot].mean()))
    dec = {k: [] for k in ("start", "wave_loop_end_mean", "wave_loop_end_max", "lds_merge",
                           "published", "last_arrival", "merge_end", "slowest_pair_vs_median",
                           "wave_spread_in_wg", "wg_spread_in_xcd")}
    xcd_loop = []             # per launch: mean over each XCD's workgroups of their slowest wave
    for a in dec_runs:
        rows = np.nonzero((a[:, :, 0] > 0).any(axis=0))[0]
        ns = int(rows.max()) + 1
        t0 = a[:, :ns, 0].min()
        dec["start"].append(float(us(a[:, :ns, 0], t0).max()))
        loops = us(a[:, :ns, 6:10], t0)
        dec["wave_loop_end_mean"].append(float(loops.mean()))
        dec["wave_loop_end_max"].append(float(loops.max()))
        dec["lds_merge"].append(float(us(a[:, :ns, 2], t0).mean()))
        dec["published"].append(float(us(a[:, :ns, 3], t0).mean()))
        arr = us(a[:, :ns, 4].max(axis=1), t0)
        dec["last_arrival"].append(float(arr.mean()))
        dec["merge_end"].append(float(us(a[:, :ns, 5].max(axis=1), t0).max()))
        dec["slowest_pair_vs_median"].append(float(arr.max() - np.median(arr)))
        # the step kernels deal a pair's workgroups to one XCD: unit p * ns + split
        # of the total sits on XCD (p * ns + split) // (total / 8)
        wg_end = loops.max(axis=2)                       # [P][ns]
        unit = np.arange(P)[:, None] * ns + np.arange(ns)[None, :]
        xcd = unit // max(1, (P * ns) // 8) if (P * ns) % 8 == 0 else unit % 8
        xcd_loop.append([float(wg_end[xcd == x].mean()) for x in range(8)])
        # slowest minus fastest wave of a workgroup, and slowest minus fastest
        # workgroup (by its slowest wave) of an XCD: means
        dec["wave_spread_in_wg"].append(float((loops.max(axis=2) - loops.min(axis=2)).mean()))
        dec["wg_spread_in_xcd"].append(float(np.mean(
            [wg_end[xcd == x].max() - wg_end[xcd == x].min() for x in range(8)])))
    out = {"workload": wl.name, "layers": R, "sampled_launches": {"append_select": len(sel_runs),
                                                                 "decode": len(dec_runs)},
           "unit": "us from the launch's first workgroup start; mean over sampled launches",
           "append_select": {k: round(float(np.mean(v)), 2) for k, v in sel.items() if v},
           "decode": {k: round(float(np.mean(v)), 2) for k, v in dec.items()}}
    if xcd_loop:
        out["decode"]["xcd_wg_loop_end_mean"] = [round(float(x), 2) for x in np.mean(xcd_loop, axis=0)]
        out["decode"]["xcd_wg_loop_end_mean_by_launch_spread"] = round(
            float(np.mean([max(r) - min(r) for r in xcd_loop])), 2)
    return out


def main():
    args = parse()
    global CLOCK_WARM_S
    CLOCK_WARM_S = args.clock_warm
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the NOSA "
              "decode path has no cross-GPU step; pairs would shard by sequence "
              "or KV head with no exchange.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from synth import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    workers = min(16, len(os.sched_getaffinity(0)))
    from trainable_offloadable_block_amd import _lib as L
    for knob, v in ((L.NOSA_TUNE_SELECT_POOL, args.select_pool),
                    (L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, args.decode_bps),
                    (L.NOSA_TUNE_SELECT_SUBS, args.select_subs)):
        if v:
            L.check(L.lib().nosa_set_tuning(knob, v), "set_tuning")
    if args.phase_clocks:
        print(json.dumps(phase_clocks(dev, workers, R=8 if args.phase_workload == 2 else 4,
                                      wl_id=args.phase_workload)), flush=True)
        return
    if args.only_host_link:
        link = host_link_peak(dev)
        with cf.ThreadPoolExecutor(workers) as pool:
            print(json.dumps(host_link_leg(args.offload_steps, pool, dev, link)), flush=True)
        return
    if args.only_link:
        print(json.dumps(host_link_peak(dev)), flush=True)
        return
    if args.fetch_wg_sweep:
        budgets = [int(x) for x in args.fetch_wg_sweep.split(",") if x]
        print(json.dumps(layer_ahead_leg(dev, workers, K=args.ahead_steps, sweep=budgets)),
              flush=True)
        return
    if args.only_ahead:
        print(json.dumps(layer_ahead_leg(dev, workers, K=args.ahead_steps, n_wg=args.fetch_wg)),
              flush=True)
        return
    if args.only_prefill:
        print(json.dumps(prefill_scores_leg(dev, workers)), flush=True)
        return
    if args.only_32k:
        link = host_link_peak(dev)
        print(json.dumps(offload_32k_leg(dev, workers, link_peak=link["peak_GBps"])), flush=True)
        return
    if args.only_8b:
        print(json.dumps(offload_8b_64k_leg(dev, workers)), flush=True)
        return
    if args.only_next:
        print(json.dumps(next_leg(dev, workers)), flush=True)
        return
    if args.only_microbatch:
        if args.mb_workload == 3:        # the offloaded 32K stack: 4 of its layers
            leg = microbatch_leg(dev, workers, R=4, W=4, K=24, n_mb=args.mb_count, wl_id=3,
                                 fetch_wg=args.mb_fetch_wg or None)
        else:
            leg = microbatch_leg(dev, workers, n_mb=args.mb_count)
        print(json.dumps(leg), flush=True)
        return
    wl = WORKLOADS[2]
    R, W, K = args.layers, args.warmup, args.steps
    m = time_stack(wl, R, W, K, args.breakdown_steps, dev, workers,
                   graph_steps=0 if args.no_graph else K)
    value, el, n_att, dec_avg_s, bd = m["value"], m["elapsed"], m["n_att"], m["dec_avg_s"], m["breakdown"]
    dbytes = decode_bytes(wl, n_att)
    achieved = dbytes / dec_avg_s / 1e9
    log("HBM read ceiling")
    ceiling = hbm_read_ceiling(dev)
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(el * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "n_q_heads": wl.n_q_heads,
            "n_kv_heads": wl.n_kv_heads, "head_dim": 128, "context": wl.context,
            "block": 64, "n_sink_blocks": wl.n_sink_blocks,
            "window_tokens": wl.window_tokens, "k_blocks": wl.k_blocks,
            "k_q_blocks": wl.k_q_blocks, "k_e_blocks": wl.k_e_blocks,
            "kv": "hbm", "layers_per_step": R, "evict_bias": True,
        },
        "roofline": {
            "kernel": "nosa_sparse_decode", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "bytes_per_launch": int(dbytes), "avg_launch_us": round(dec_avg_s * 1e6, 2),
            "timing": "HIP events around each step's 8 decode launches, run back to back "
                      "after the step's selections, over the K steps that follow the value's "
                      "timed region (the same stack; that region runs without events)",
            "launch_us": m["dec_launch_us"],
            "call_us_events_around": bd["decode"],
            "attended_tokens_per_pair": round(n_att, 2),
            # beside the published peak: what a streaming read that does
            # nothing else reaches on this GPU (nosa_hbm_read)
            "practical_read_ceiling": ceiling,
            "frac_of_practical_read_ceiling": round(achieved / ceiling["GBps"], 4),
        },
        "decode_timing_steps": m["decode_timing_steps"],
        "breakdown_us": bd,
        "breakdown_p90_us": m["breakdown_p90"],
        "layer_step_us": m["layer_step_us"],
        "locality": m["locality"],
    }
    # the selection against the same roofline: its algorithmic bytes over the
    # fused append + select launch's time, the step's 8 calls back to back
    # between two events (as the decode; events around a single call add
    # their own cost, kept as call_us_events_around); the pool after the
    # scoring splits is latency-bound
    L_mid = wl.context + W + K
    sb = select_bytes(wl, L_mid)
    sel_us = m["sel_launch_us"]["mean"]
    res["select_roofline"] = {
        "kernel": "nosa_append_select", "bound": "hbm", "bytes_per_launch": int(sb),
        "avg_launch_us": sel_us,
        "timing": "HIP events around each step's 8 append + select calls, run back to "
                  "back before the step's decodes, over the same K steps as the decode's",
        "launch_us": m["sel_launch_us"],
        "call_us_events_around": bd["append_select"],
        "achieved": round(sb / (sel_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(sb / (sel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if "graph" in m:
        res["graph_replay"] = m["graph"]
    pf = [ms for name, ms in PREFILL_MS if name == wl.name]
    if pf:
        # the state build reads every context token's K and V once (512 B)
        ms = float(np.median(pf))
        byt = wl.batch * wl.n_kv_heads * wl.context * 512
        res["state_build"] = {"call": "nosa_prefill_init", "ms_per_layer": round(ms, 3),
                              "context_tokens_per_s": round(wl.batch * wl.context / (ms * 1e-3), 1),
                              "kv_GBps": round(byt / (ms * 1e-3) / 1e9, 1)}
    if not args.no_microbatch:
        log("two micro-batches on two streams")
        res["microbatch_2x16"] = microbatch_leg(dev, workers)
    log("warm single-layer leg")
    res["warm_1layer"] = warm_leg(dev, workers)
    if not args.no_tiny:
        log("tiny 4K leg")
        res["tiny_4k"] = tiny_leg(dev, workers)
    if not args.no_prefill:
        log("prefill block-score leg")
        res["prefill_scores"] = prefill_scores_leg(dev, workers)
    if not args.no_next:
        log("GQA-16 96-block leg")
        res["gqa16_k96"] = next_leg(dev, workers)
    if not args.no_offload:
        log("host-link ceiling")
        link = host_link_peak(dev)
        log("offloaded 32K stack leg")
        res["offload_32k"] = offload_32k_leg(dev, workers, link_peak=link["peak_GBps"])
        log("offloaded 8B-shaped 64K leg")
        res["offload_8b_64k"] = offload_8b_64k_leg(dev, workers, link_peak=link["peak_GBps"])
        if not args.no_ahead:
            log("layer-ahead leg (SparDA order, offloaded 32K stack)")
            res["layer_ahead"] = layer_ahead_leg(dev, workers, K=args.ahead_steps,
                                                 n_wg=args.fetch_wg)
        log("host-link leg (offloaded 128K workload)")
        with cf.ThreadPoolExecutor(workers) as pool:
            res["host_link"] = host_link_leg(args.offload_steps, pool, dev, link)
    if not args.no_cpu:
        log("timing the CPU oracle")
        log("GPU records of layer 0 for the oracle's parity check")
        gpu = gpu_records(dev, 2, args.cpu_steps, workers)
        res["parity"], res["cpu_baseline"] = cpu_baseline(2, args.cpu_pairs, args.cpu_steps, gpu)
    else:
        res["cpu_baseline"] = None
    res["clock_warm"] = WARMUPS
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
