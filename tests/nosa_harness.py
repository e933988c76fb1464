"""Lockstep runner: the HIP path and the CPU oracle on the same inputs.

The GPU layer runs every pair of a workload through the C ABI; the oracle
runs a chosen subset of pairs (all of them for small workloads, a sample at
full size). After each step the harness compares, per checked pair:

* the selection: block ids and kinds exactly, except near-ties (below);
* the attention output: max-abs <= 1e-2 and relative L2 <= 2e-3 over the
  checked heads;
* compressed keys bit for bit, eviction and block scores to float32 error:
  after the prefill, and (``check_state``) every 16 steps and at the end of
  a run for every complete chunk and block, so the chunks that appends
  complete are compared too.

Layer-ahead mode (``ahead=True``, SparDA's order): each step selects with
the synthetic forecast head before the append (nosa_select_forecast against
PairOracle.step_ahead), then fetches (optionally with a workgroup budget),
appends and decodes. Forecast scores are plain logits that can sit near 0, so
their ties and score errors are measured against max(|tau|, rms of the
candidates' scores) instead of |tau| alone.

Near-tie protocol: when the GPU and the oracle pick different blocks, the
step still passes if every block in the symmetric difference of the
query-aware picks scores within 1e-5 (relative) of the oracle's k_q-th best
query-aware score, and every block in the symmetric difference of the
agnostic picks (recomputed by the oracle from the GPU's query-aware picks)
within 1e-5 of the k_e'-th best agnostic score. The GPU is then re-run on
the oracle's selection (decode output checked against the oracle), and its
eligibility bits (and cache, in offload mode) are re-synchronised to the
oracle's state.
"""

from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle.nosa_oracle as O
from synth import (bf16_bits_to_f64, context_kv, eviction_weights, forecasts,
                   new_tokens, queries)
from trainable_offloadable_block_amd import LayerShape, NosaLayer, v_from_tiles
from trainable_offloadable_block_amd import _lib as L

TIE_REL = 1e-5
MAX_ABS = 1e-2
REL_L2 = 2e-3
# Score diagnostics: float32 accumulation against the float64 oracle. The
# eviction score is a sum of 128 softplus terms of either sign, so a single
# token's score can sit near zero while its error does not; its errors (and
# those of the chunk and block means built from it) are taken relative to
# the root-mean-square score of the pair. Query-aware block scores are
# positive softmax sums and are taken relative to themselves.
SCORE_REL = 1e-5
KIND_OF = {O.SINK: L.KIND_SINK, O.WINDOW: L.KIND_WINDOW, O.QUERY: L.KIND_QUERY,
           O.AGNOSTIC: L.KIND_AGNOSTIC}


def shape_of(wl, offload=None, max_context=None) -> LayerShape:
    return LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                      wl.window_tokens, wl.k_blocks, wl.k_q_blocks, wl.k_e_blocks,
                      max_context or wl.max_context,
                      wl.offload if offload is None else offload, wl.evict_bias)


@dataclass
class StepReport:
    t: int
    near_ties: int = 0
    max_abs: float = 0.0
    rel_l2: float = 0.0
    qscore_rel: float = 0.0
    escore_rel: float = 0.0
    misses: dict = field(default_factory=dict)


class Lockstep:
    def __init__(self, wl, layer=0, check_pairs=None, lengths=None,
                 offload=None, steps=None, before_prefill=None, fused=False,
                 ahead=False, fetch_workgroups=0):
        self.wl = wl
        self.fused = fused          # nosa_append_select instead of the two calls
        self.ahead = ahead          # layer-ahead selection with a forecast head
        self.fetch_workgroups = fetch_workgroups
        self.layer_idx = layer
        B, Hkv, G = wl.batch, wl.n_kv_heads, wl.group
        self.lengths = np.full(B, wl.context, dtype=np.int64) if lengths is None \
            else np.asarray(lengths, dtype=np.int64)
        self.steps = wl.steps if steps is None else steps
        self.shape = shape_of(wl, offload, int(self.lengths.max()) + self.steps)
        self.gpu = NosaLayer(self.shape)
        self.P = B * Hkv
        self.check = list(range(self.P)) if check_pairs is None else list(check_pairs)
        w1 = np.stack([eviction_weights(wl, layer, g)[0] for g in range(Hkv)])
        w2 = np.stack([eviction_weights(wl, layer, g)[1] for g in range(Hkv)])
        self.gpu.set_weights(w1, w2)
        self.n_w = wl.window_tokens // 64
        self.k_e_dyn = wl.k_e_blocks - wl.n_sink_blocks - self.n_w
        self.oracles = {}
        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as pool:
            ctx = list(pool.map(lambda p: context_kv(wl, layer, *divmod(p, Hkv)),
                                range(self.P)))
        for p in range(self.P):
            b, g = divmod(p, Hkv)
            K, V = ctx[p]
            ctx[p] = None
            Lb = int(self.lengths[b])
            K, V = K[:Lb], V[:Lb]
            self.gpu.load_pair_context(p, K, V)
            if p in self.check:
                cap = Lb + self.steps
                Kf = np.zeros((cap, 128))
                Vf = np.zeros((cap, 128))
                Kf[:Lb] = bf16_bits_to_f64(K)
                Vf[:Lb] = bf16_bits_to_f64(V)
                self.oracles[p] = O.PairOracle(
                    Kf, Vf, bf16_bits_to_f64(w1[g]), bf16_bits_to_f64(w2[g]), Lb,
                    wl.n_sink_blocks, self.n_w, wl.k_q_blocks, self.k_e_dyn,
                    1.0 if wl.evict_bias else 0.0)
        if before_prefill is not None:
            before_prefill(self)
        self.gpu.prefill(self.lengths)
        # per-step inputs for every pair / head
        Hq = wl.n_q_heads
        self.q = np.stack([np.stack([queries(wl, layer, b, h)[:self.steps]
                                     for h in range(Hq)]) for b in range(B)])
        kn, vn = [], []
        for b in range(B):
            kk, vv = zip(*[new_tokens(wl, layer, b, g) for g in range(Hkv)])
            kn.append(np.stack([x[:self.steps] for x in kk]))
            vn.append(np.stack([x[:self.steps] for x in vv]))
        self.knew = np.stack(kn)   # [B][Hkv][steps][128]
        self.vnew = np.stack(vn)
        self.f = None
        if ahead:
            self.f = np.stack([np.stack([forecasts(wl, layer, b, g)[:self.steps]
                                         for g in range(Hkv)]) for b in range(B)])
        self.reports = []

    # ---------------------------------------------------------------- inputs
    def _dev(self, arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(
            self.gpu.device)

    def inputs(self, t):
        k = self._dev(self.knew[:, :, t])
        v = self._dev(self.vnew[:, :, t])
        q = self._dev(self.q[:, :, t])
        return k, v, q

    # ---------------------------------------------------------------- checks
    def check_prefill(self):
        """The state after the prefill (see check_state)."""
        self.check_state("prefill")

    def check_state(self, where=""):
        """Every complete chunk's compressed key bit for bit against the
        oracle's (incrementally built) keys; the eviction score of every
        token, the mean score of every complete chunk and the agnostic score
        of every block whose chunks are all complete within SCORE_REL of
        the pair's RMS score; the lengths equal."""
        g = self.gpu
        ck = g.ckey.cpu().numpy().view(np.uint16).reshape(self.P, self.shape.c_max, 128)
        ts = g.tok_s.cpu().numpy().reshape(self.P, -1)
        ce = g.chunk_e.cpu().numpy().reshape(self.P, -1)
        be = g.blk_e.cpu().numpy().reshape(self.P, -1)
        seq = g.seq_len.cpu().numpy()
        worst = 0.0
        for p, o in self.oracles.items():
            assert int(seq[p // self.wl.n_kv_heads]) == o.L, f"{where} pair {p}: length"
            C = len(o.ckeys)
            assert C == O.n_chunks(o.L)
            want = O.bf16_bits(np.array(o.ckeys)) if C else np.zeros((0, 128), np.uint16)
            bad = np.nonzero(np.any(ck[p, :C] != want, axis=1))[0]
            assert not len(bad), f"{where} pair {p}: compressed keys of chunks {bad[:8]} differ"
            s_ref = o.s[:o.L]
            scale = math.sqrt(float(np.mean(s_ref ** 2)))
            err = float((np.abs(ts[p, :o.L] - s_ref) / scale).max())
            if C:
                e_ref = np.array(o.e_chunks)
                err = max(err, float((np.abs(ce[p, :C] - e_ref) / scale).max()))
                nbc = sum(1 for b in range(O.n_blocks(o.L)) if 4 * b + 3 < C)
                if nbc:
                    b_ref = O.block_max_pool(e_ref, O.n_blocks(o.L))[:nbc]
                    err = max(err, float((np.abs(be[p, :nbc] - b_ref) / scale).max()))
            worst = max(worst, err)
            assert err < SCORE_REL, f"{where} pair {p}: eviction/chunk/block score rel err {err}"
        return worst

    def _near_tie(self, res, gq, ga):
        """True when the GPU's query-aware / agnostic picks differ from the
        oracle's only at near-ties (see module docstring)."""
        cand = res.roles.candidates
        oq = set(res.sel.query)
        if gq != oq:
            ranked = sorted(cand, key=lambda b: (-res.Qb[b], b))
            tau = res.Qb[ranked[min(len(ranked), self.wl.k_q_blocks) - 1]]
            ref = abs(tau)
            if self.ahead:
                ref = max(ref, math.sqrt(float(np.mean(res.Qb[cand] ** 2))))
            for b in gq ^ oq:
                if abs(res.Qb[b] - tau) > TIE_REL * ref:
                    return False
        pool = [b for b in cand if b in res.eligible and b not in gq]
        agn = set(O.top_by_score(pool, res.Eb, self.k_e_dyn))
        if ga != agn:
            ranked = sorted(pool, key=lambda b: (-res.Eb[b], b))
            tau = res.Eb[ranked[min(len(ranked), self.k_e_dyn) - 1]]
            for b in ga ^ agn:
                if abs(res.Eb[b] - tau) > TIE_REL * abs(tau):
                    return False
        return True

    def _elig_words(self, o, res):
        words = (self.shape.nb_max + 31) // 32
        bits = np.full(words * 32, 1, dtype=np.uint64)
        for b in res.roles.candidates:
            bits[b] = 1 if b in o.carry else 0
        w = np.zeros(words, dtype=np.uint64)
        for j in range(32):
            w |= bits[j::32][:words] << np.uint64(j)
        return w.astype(np.uint32)

    def step(self, t, check_scores=True) -> StepReport:
        """Runs step t on the GPU, then compares it with the oracle."""
        self.launch(t, check_scores)
        return self.compare(t, check_scores)

    def launch(self, t, check_scores=True):
        kd, vd, qd = self.inputs(t)
        g = self.gpu
        if self.ahead:
            g.select_forecast(self._dev(self.f[:, :, t]), want_kind=True,
                              want_fscore=check_scores)
            if self.fetch_workgroups:
                g.fetch_wg(self.fetch_workgroups)
            else:
                g.fetch()
            g.append(kd, vd)
        elif self.fused:
            g.append_select(kd, vd, qd, want_kind=True, want_qscore=check_scores)
            g.fetch()
        else:
            g.append(kd, vd)
            g.select(qd, want_kind=True, want_qscore=check_scores)
            g.fetch()
        g.decode(qd)

    def compare(self, t, check_scores=True) -> StepReport:
        """Steps the oracle of every checked pair and compares the GPU's
        results of step t (already computed) with them."""
        wl, G, Hkv, k = self.wl, self.wl.group, self.wl.n_kv_heads, self.wl.k_blocks
        g = self.gpu
        qd = self.inputs(t)[2]
        torch.cuda.synchronize()
        sel = g.sel.cpu().numpy().reshape(self.P, k)
        nsel = g.n_sel.cpu().numpy()
        kind = g.kind.cpu().numpy().reshape(self.P, k)
        out = g.out.cpu().numpy().reshape(wl.batch, wl.n_q_heads, 128)
        nmiss = g.n_miss.cpu().numpy()
        rep = StepReport(t)
        results = {}
        resync = []
        for p, o in self.oracles.items():
            b, gg = divmod(p, Hkv)
            qg = bf16_bits_to_f64(self.q[b, gg * G:(gg + 1) * G, t])
            if self.ahead:
                res = o.step_ahead(bf16_bits_to_f64(self.f[b, gg, t]),
                                   bf16_bits_to_f64(self.knew[b, gg, t]),
                                   bf16_bits_to_f64(self.vnew[b, gg, t]), qg)
            else:
                res = o.step(bf16_bits_to_f64(self.knew[b, gg, t]),
                             bf16_bits_to_f64(self.vnew[b, gg, t]), qg)
            results[p] = res
            gb = [int(x) for x in sel[p, :nsel[p]]]
            gk = {int(x): int(c) for x, c in zip(sel[p, :nsel[p]], kind[p, :nsel[p]])}
            ok_kinds = {bb: KIND_OF[c] for bb, c in res.sel.kinds.items()}
            if gb != res.sel.blocks or gk != ok_kinds:
                gq = {bb for bb, c in gk.items() if c == L.KIND_QUERY}
                ga = {bb for bb, c in gk.items() if c == L.KIND_AGNOSTIC}
                base_ok = ({bb for bb, c in gk.items() if c in (L.KIND_SINK, L.KIND_WINDOW)}
                           == set(res.roles.sink) | set(res.roles.window))
                assert base_ok and self._near_tie(res, gq, ga), (
                    f"step {t} pair {p}: selection differs beyond near-ties\n"
                    f"gpu    {sorted(gk.items())}\noracle {sorted(ok_kinds.items())}")
                rep.near_ties += 1
                resync.append(p)
            elif self.shape.offload:
                rep.misses[p] = (int(nmiss[p]), len(res.misses))
                assert int(nmiss[p]) == len(res.misses), (
                    f"step {t} pair {p}: {nmiss[p]} blocks fetched, oracle {len(res.misses)}")
        if resync:
            self._resync(t, qd, resync, results)
            out = g.out.cpu().numpy().reshape(wl.batch, wl.n_q_heads, 128)
        # attention output over the checked heads
        got, want = [], []
        for p, res in results.items():
            b, gg = divmod(p, Hkv)
            got.append(out[b, gg * G:(gg + 1) * G])
            want.append(res.out)
        got, want = np.concatenate(got), np.concatenate(want)
        diff = got.astype(np.float64) - want
        rep.max_abs = float(np.abs(diff).max())
        rep.rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30))
        assert rep.max_abs <= MAX_ABS and rep.rel_l2 <= REL_L2, (
            f"step {t}: attention max-abs {rep.max_abs:.3e} rel-L2 {rep.rel_l2:.3e}")
        if check_scores:
            dq = g.dbg_q.cpu().numpy().reshape(self.P, -1)
            be = g.blk_e.cpu().numpy().reshape(self.P, -1)
            for p, res in results.items():
                c = res.roles.candidates
                if not c:
                    continue
                if wl.k_q_blocks > 0:
                    den = np.abs(res.Qb[c])
                    if self.ahead:
                        den = np.maximum(den, math.sqrt(float(np.mean(res.Qb[c] ** 2))))
                    qr = np.abs(dq[p, c] - res.Qb[c]) / den
                    rep.qscore_rel = max(rep.qscore_rel, float(qr.max()))
                scale = math.sqrt(float(np.mean(res.Eb[c] ** 2)))
                er = np.abs(be[p, c] - res.Eb[c]) / scale
                rep.escore_rel = max(rep.escore_rel, float(er.max()))
            assert rep.qscore_rel < SCORE_REL, f"step {t}: query score rel err {rep.qscore_rel}"
            assert rep.escore_rel < SCORE_REL, f"step {t}: agnostic score rel err {rep.escore_rel}"
        if not resync:
            self.check_eligibility(results)
        self.reports.append(rep)
        return rep

    def check_eligibility(self, results):
        words = self.gpu.eligible_words()
        for p, res in results.items():
            want = self._elig_words(self.oracles[p], res)
            assert np.array_equal(words[p], want), f"pair {p}: eligibility bits differ"

    def _resync(self, t, qd, pairs, results):
        """Runs fetch + decode on the oracle's selection for the given pairs and
        overwrites their eligibility bits with the oracle's."""
        g, k = self.gpu, self.wl.k_blocks
        sel = g.sel.cpu().numpy().reshape(self.P, k).copy()
        nsel = g.n_sel.cpu().numpy().copy()
        elig = g.eligible_words().copy()
        for p in pairs:
            blocks = results[p].sel.blocks
            sel[p] = -1
            sel[p, :len(blocks)] = blocks
            nsel[p] = len(blocks)
            elig[p] = self._elig_words(self.oracles[p], results[p])
        g.eligible.copy_(torch.from_numpy(elig.view(np.int32).reshape(-1)))
        sel_t = torch.from_numpy(sel.reshape(-1)).to(g.device)
        nsel_t = torch.from_numpy(nsel).to(g.device)
        # the wrongly fetched blocks are simply cached extra; fetching the
        # oracle's selection now evicts them
        g.fetch(sel_t, nsel_t)
        g.decode(qd, sel_t, g.phys if self.shape.offload else sel_t, nsel_t)
        torch.cuda.synchronize()

    def check_cache(self):
        """Offload mode: each selected block's cache slot holds the oracle's
        K and V for the block's existing tokens, and a complete block's host
        copy equals its cache slot (the host store receives a block when its
        last token arrives; until then the cache holds the newest tokens)."""
        g, k = self.gpu, self.wl.k_blocks
        sel = g.sel.cpu().numpy().reshape(self.P, k)
        phys = g.phys.cpu().numpy().reshape(self.P, k)
        nsel = g.n_sel.cpu().numpy()
        seq = g.seq_len.cpu().numpy()
        cache = g.kv_dev.view(self.P, k + 1, 2, 64, 128)
        host = g.kv_host.view(self.P, g.nb_kv, 2, 64, 128)
        for p in self.check:
            Lb = int(seq[p // self.wl.n_kv_heads])
            o = self.oracles.get(p)
            for i in range(nsel[p]):
                blk = int(sel[p, i])
                n = min(64, Lb - 64 * blk)        # tokens that exist
                a = cache[p, phys[p, i]].cpu()
                ak = a[0, :n].numpy().view(np.uint16)
                av = v_from_tiles(a[1].reshape(-1).numpy())[:n].view(np.uint16)
                if o is not None:
                    rows = slice(64 * blk, 64 * blk + n)
                    assert np.array_equal(ak, O.bf16_bits(o.K[rows])), \
                        f"pair {p} block {blk}: cached K differs from the oracle"
                    assert np.array_equal(av, O.bf16_bits(o.V[rows])), \
                        f"pair {p} block {blk}: cached V differs from the oracle"
                if n == 64:
                    h = host[p, blk]
                    assert torch.equal(a, h), f"pair {p} block {blk}: host copy differs"

    def run(self, steps=None, check_scores=True, cache_every=0, state_every=16):
        n = self.steps if steps is None else steps
        for t in range(n):
            self.step(t, check_scores)
            if cache_every and self.shape.offload and t % cache_every == 0:
                self.check_cache()
            if state_every and (t % state_every == state_every - 1 or t == n - 1):
                self.check_state(f"step {t}")
        return self.reports


def summary(reports):
    return dict(steps=len(reports),
                near_ties=sum(r.near_ties for r in reports),
                max_abs=max(r.max_abs for r in reports),
                rel_l2=max(r.rel_l2 for r in reports),
                qscore_rel=max(r.qscore_rel for r in reports),
                escore_rel=max(r.escore_rel for r in reports))


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


__all__ = ["Lockstep", "shape_of", "summary", "rel_l2", "math"]
