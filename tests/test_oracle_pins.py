"""The oracle against its pins, and planted mistakes against the pins.

CPU only. A planted mistake lives in a private copy of the oracle module (never
in the HIP path); each one must make at least one pin fail, which shows the
pins would catch that kind of slip in the oracle itself.
"""

import importlib.util
import math
import os
import sys

import numpy as np
import pytest

import oracle.nosa_oracle as real
import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(real.__file__), "nosa_oracle.py")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(real)


_copies = 0


def _fresh_oracle():
    global _copies
    _copies += 1
    name = f"nosa_oracle_copy_{_copies}"
    spec = importlib.util.spec_from_file_location(name, ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod          # dataclasses look their module up here
    spec.loader.exec_module(mod)
    return mod


# ------------------------------------------------------------ planted mistakes

def _chunks_by_start(o):
    def chunks_of_block(b, C):               # only chunks starting in b
        lo = min(C, 4 * b)
        return range(lo, min(C, 4 * b + 4))
    o.chunks_of_block = chunks_of_block


def _no_score_scale(o):
    def query_chunk_scores(q, ckeys):
        logits = q @ ckeys.T
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        return (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
    o.query_chunk_scores = query_chunk_scores


def _softmax_over_heads(o):
    def query_chunk_scores(q, ckeys):
        logits = (q @ ckeys.T) / math.sqrt(q.shape[1])
        e = np.exp(logits - logits.max(axis=0, keepdims=True))
        return (e / e.sum(axis=0, keepdims=True)).sum(axis=0)
    o.query_chunk_scores = query_chunk_scores


def _transposed_w1(o):
    def eviction_scores(V, W1, W2):
        return o.softplus(V @ W1.T) @ W2
    o.eviction_scores = eviction_scores


def _swapped_pool(o):
    o.POOL_KERNEL, o.POOL_STRIDE = 16, 32


def _sum_not_mean(o):
    def chunk_means(s, L=None):
        L = s.shape[0] if L is None else L
        return np.array([s[16 * i:16 * i + 32].sum()
                         for i in range(o.n_chunks(L))])
    o.chunk_means = chunk_means


def _ties_high_index(o):
    def top_by_score(ids, scores, k):
        return sorted(ids, key=lambda b: (-scores[b], -b))[:max(0, k)]
    o.top_by_score = top_by_score


def _bias_sign(o):
    orig = o.attend

    def attend(q, K, V, s, blocks, L, beta):
        return orig(q, K, V, s, blocks, L, -beta)
    o.attend = attend


def _window_without_partial(o):
    orig = o.block_roles

    def block_roles(L, n_sink, n_win):
        r = orig(L, n_sink, n_win)
        if L % 64 and r.window:
            r.window = r.window[:-1]
        return r
    o.block_roles = block_roles


def _double_rounding(o):
    def bf16_round(x):
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        return u.astype(np.uint32).view(np.float32).astype(np.float64)
    o.bf16_round = bf16_round


def _float_sum_compress(o):
    def compress_chunk(rows):
        return o.bf16_round(rows.astype(np.float32).sum(axis=0,
                                                        dtype=np.float32) / 32)
    o.compress_chunk = compress_chunk


def _evict_on_agnostic_only(o):
    orig = o.select_blocks

    def select_blocks(Qb, Eb, eligible, roles, k_q, k_e_dyn):
        sel = orig(Qb, Eb, eligible, roles, k_q, k_e_dyn)
        # a Q pick of an eligible block now costs it its eligibility
        eligible.difference_update(set(sel.query))
        return sel
    o.select_blocks = select_blocks


def _fill_shortfall(o):
    orig = o.select_blocks

    def select_blocks(Qb, Eb, eligible, roles, k_q, k_e_dyn):
        everything = set(roles.candidates)
        return orig(Qb, Eb, everything, roles, k_q, k_e_dyn)
    o.select_blocks = select_blocks


def _forecast_softmax(o):
    def forecast_chunk_scores(f, ckeys):
        x = (ckeys @ f) / math.sqrt(f.shape[0])
        e = np.exp(x - x.max())
        return e / e.sum()
    o.forecast_chunk_scores = forecast_chunk_scores


def _forecast_unscaled(o):
    o.forecast_chunk_scores = lambda f, ckeys: ckeys @ f


def _ahead_at_current_length(o):
    def select_ahead(self, f):
        ck = self._ckeys()
        a = o.forecast_chunk_scores(f, ck) if len(ck) else np.zeros(0)
        return self._select_at(self.L, a, self.L)
    o.PairOracle.select_ahead = select_ahead


def _prefill_off_by_one(o):
    orig = o.prefill_block_scores

    def prefill_block_scores(Q, pos0, ckeys, n_sink, n_win):
        return orig(Q, pos0 - 1, ckeys, n_sink, n_win)[:, :o.n_blocks(pos0 + Q.shape[0])] \
            if pos0 > 0 else orig(Q, pos0, ckeys, n_sink, n_win)
    o.prefill_block_scores = prefill_block_scores


def _prefill_not_causal(o):
    def prefill_block_scores(Q, pos0, ckeys, n_sink, n_win):
        T = Q.shape[0]
        out = np.full((T, o.n_blocks(pos0 + T)), -np.inf)
        C = o.n_chunks(pos0 + T)                  # every chunk, for every row
        for i in range(T):
            roles = o.block_roles(pos0 + i + 1, n_sink, n_win)
            if C and roles.candidates:
                a = o.query_chunk_scores(Q[i], ckeys[:C])
                Qb = o.block_max_pool(a, roles.nb)
                out[i, roles.candidates] = Qb[roles.candidates]
        return out
    o.prefill_block_scores = prefill_block_scores


def _prefill_attend_not_causal(o):
    orig = o.attend

    def prefill_sparse_attend(Q, pos0, K, V, s, ckeys, e_chunks, n_sink, n_win, k_q,
                              k_e_dyn, beta):
        T = Q.shape[0]
        scores = o.prefill_block_scores(Q, pos0, ckeys, n_sink, n_win)
        outs, sels = [], []
        for i in range(T):
            L = pos0 + i + 1
            roles = o.block_roles(L, n_sink, n_win)
            Eb = o.block_max_pool(np.asarray(e_chunks[:o.n_chunks(L)]), roles.nb)
            sel = o.select_blocks(scores[i, :roles.nb], Eb, set(roles.candidates), roles,
                                  k_q, k_e_dyn)
            outs.append(orig(Q[i], K, V, s, sel.blocks, pos0 + T, beta))   # sees the future
            sels.append(sel)
        return np.stack(outs), sels
    o.prefill_sparse_attend = prefill_sparse_attend


def _append_half_chunk_mean(o):
    def append(self, k_new, v_new):
        j = self.L
        self.K[j] = k_new
        self.V[j] = v_new
        self.s[j] = o.eviction_scores(v_new[None, :], self.W1, self.W2)[0]
        self.L += 1
        while len(self.ckeys) < o.n_chunks(self.L):
            i = len(self.ckeys)
            self.ckeys.append(o.compress_chunk(self.K[16 * i:16 * i + 32]))
            self.e_chunks.append(self.s[16 * i:16 * i + 16].mean())   # half the chunk
        return j
    o.PairOracle.append = append


def _locality_newest_always_present(o):
    def locality(prev, cur, new_block):
        have = set(prev) | {max(cur)}
        if new_block is not None:
            have.add(new_block)
        return sum(1 for b in cur if b in have) / len(cur)
    o.locality = locality


def _locality_previous_denominator(o):
    def locality(prev, cur, new_block):
        have = set(prev)
        if new_block is not None:
            have.add(new_block)
        return sum(1 for b in cur if b in have) / len(prev)
    o.locality = locality


def _token_locality_counts_new_token(o):
    def token_locality(prev, L_prev, cur, L_cur):
        now = o.selected_tokens(cur, L_cur)
        before = o.selected_tokens(prev, L_prev)
        return len(now & before) / len(now)
    o.token_locality = token_locality


def _token_locality_whole_blocks(o):
    def token_locality(prev, L_prev, cur, L_cur):
        now = {j for b in cur for j in range(64 * b, 64 * b + 64) if j != L_cur - 1}
        before = {j for b in prev for j in range(64 * b, 64 * b + 64)}
        return len(now & before) / len(now)
    o.token_locality = token_locality


MUTATIONS = [_chunks_by_start, _no_score_scale, _softmax_over_heads,
             _transposed_w1, _swapped_pool, _sum_not_mean, _ties_high_index,
             _bias_sign, _window_without_partial, _double_rounding,
             _float_sum_compress, _evict_on_agnostic_only, _fill_shortfall,
             _forecast_softmax, _forecast_unscaled, _ahead_at_current_length,
             _prefill_off_by_one, _prefill_not_causal, _prefill_attend_not_causal,
             _append_half_chunk_mean, _locality_newest_always_present,
             _locality_previous_denominator, _token_locality_counts_new_token,
             _token_locality_whole_blocks]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mutate):
    o = _fresh_oracle()
    mutate(o)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutate.__name__}"
