"""Pins of the CPU oracle against facts it does not compute itself.

Each ``pin_*`` takes an oracle module and raises AssertionError when the
module disagrees with a closed form, a brute-force count on a tiny input, an
independent library routine, a printed value of the pages, or an invariant
the pages state. ``test_oracle_pins.py`` runs them on the real oracle and on
copies of it with planted mistakes (each planted mistake must trip a pin).
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_vals(rng, shape, scale=1.0):
    """Random bf16-representable float64 values (truncated float32)."""
    x = (scale * rng.standard_normal(shape)).astype(np.float32)
    bits = x.view(np.uint32) & np.uint32(0xFFFF0000)
    return bits.view(np.float32).astype(np.float64)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


# ------------------------------------------------------------------ bf16

def pin_bf16_golden(o):
    """Hand-derived roundings (bf16 = 1 sign, 8 exponent, 7 fraction bits)."""
    for expr, bits in read_golden("bf16_rne.txt"):
        x = float(eval(expr, {"__builtins__": {}}, {}))  # arithmetic only
        got = int(o.bf16_bits(o.bf16_round(np.array([x])))[0])
        assert got == int(bits, 16), (expr, hex(got), bits)


def pin_bf16_vs_torch(o):
    """Library routine: torch's float32 -> bfloat16 conversion rounds to
    nearest even; on float32 inputs direct rounding must agree with it."""
    import torch
    rng = _rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
    ])
    # exact halfway points between neighbouring bf16 values
    base = x.view(np.uint32) & np.uint32(0xFFFF0000)
    half = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, half[np.isfinite(half)]])
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16)
    ref = ref.numpy().view(np.uint16)
    got = o.bf16_bits(o.bf16_round(x.astype(np.float64)))
    assert np.array_equal(got, ref)


def pin_bf16_exact_path(o):
    """The rational-input rounding agrees with the float64 one."""
    rng = _rng(2)
    for v in rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300):
        assert o.bf16_round_exact(Fraction(float(v))) == float(
            o.bf16_round(np.array([v]))[0])


# ------------------------------------------------------------------ CompressK

def pin_chunk_count(o):
    """Chunk i covers tokens [16i, 16i+32): brute-force count of complete
    windows."""
    for L in range(0, 300):
        brute = sum(1 for i in range(L) if 16 * i + 32 <= L)
        assert o.n_chunks(L) == brute, L


def pin_compress_exact_means(o):
    """Keys that are small integers: the chunk mean is an exact dyadic value
    with at most 8 significant bits, so CompressK must return it exactly."""
    rng = _rng(3)
    K = rng.integers(-4, 5, size=(96, 8)).astype(np.float64)
    c = o.compress_keys(K)
    assert c.shape == (5, 8)
    for i in range(5):
        for d in range(8):
            exact = Fraction(int(K[16 * i:16 * i + 32, d].sum()), 32)
            assert Fraction(c[i, d]) == exact, (i, d)


def pin_compress_single_rounding(o):
    """The mean is rounded once, directly: 31 ones and one 1.125 average to
    1 + 2^-8, an exact tie between 1 and 1 + 2^-7 that rounds to even (1)."""
    rows = np.ones((32, 2))
    rows[5, 0] = 1.125
    rows[7, 1] = 1.125 + 2.0 ** -4   # mean 1 + 2^-8 + 2^-9: rounds up
    c = o.compress_chunk(rows)
    assert c[0] == 1.0
    assert c[1] == 1.0 + 2.0 ** -7


def pin_compress_wide_range(o):
    """Exact sum even when float64 accumulation would lose a term:
    2^60 + 2^-60 - 2^60 averages to 2^-65, a bf16 value."""
    rows = np.zeros((32, 1))
    rows[0, 0], rows[1, 0], rows[2, 0] = 2.0 ** 60, 2.0 ** -60, -(2.0 ** 60)
    assert o.compress_chunk(rows)[0] == 2.0 ** -65


def pin_pool_identity(o):
    """Mean pooling commutes with the dot product: for keys whose chunk means
    are bf16-exact, q . c_i equals the mean of q . k_j over chunk i."""
    rng = _rng(4)
    K = rng.integers(-3, 4, size=(160, 16)).astype(np.float64)
    q = rng.standard_normal(16)
    c = o.compress_keys(K)
    tok = K @ q
    for i in range(c.shape[0]):
        assert math.isclose(c[i] @ q, tok[16 * i:16 * i + 32].mean(),
                            rel_tol=1e-12, abs_tol=1e-12)


# ------------------------------------------------------------------ eviction

def pin_eviction_closed_form(o):
    """softplus(0) = ln 2 and softplus(ln(e - 1)) = 1; W1 is input-major, so a
    one-hot value vector at input e reads row e of W1."""
    d = 4
    W1 = np.zeros((d, d))
    W1[0, 0] = math.log(math.e - 1.0)      # row 0 -> hidden 0 gets 1
    W1[1, 2] = 50.0                          # row 1 -> hidden 2 ~ linear
    W2 = np.array([2.0, 3.0, 5.0, 0.0])
    V = np.eye(d)[:2]
    s = o.eviction_scores(V, W1, W2)
    ln2 = math.log(2.0)
    assert math.isclose(s[0], 2.0 * 1.0 + 3.0 * ln2 + 5.0 * ln2, rel_tol=1e-13)
    assert math.isclose(s[1], 2.0 * ln2 + 3.0 * ln2 + 5.0 * 50.0,
                        rel_tol=1e-13)
    # very negative pre-activations contribute nothing
    W1n = np.full((d, d), -800.0)
    assert abs(o.eviction_scores(V, W1n, W2)[0]) < 1e-300


def pin_chunk_means_closed_form(o):
    """Mean of s_j = j over chunk i is 16i + 15.5."""
    s = np.arange(200, dtype=np.float64)
    m = o.chunk_means(s)
    assert len(m) == o.n_chunks(200)
    assert np.allclose(m, 16 * np.arange(len(m)) + 15.5, rtol=0, atol=0)


def pin_block_pool_brute(o):
    """Brute force over tokens: block b takes the max over every chunk that
    shares at least one token with it."""
    rng = _rng(5)
    for L in (32, 47, 64, 100, 128, 200, 511, 640):
        C = o.n_chunks(L)
        nb = -(-L // 64)
        x = rng.standard_normal(C)
        got = o.block_max_pool(x, nb)
        for b in range(nb):
            members = [i for i in range(C)
                       if set(range(16 * i, 16 * i + 32))
                       & set(range(64 * b, 64 * b + 64))]
            want = max(x[i] for i in members) if members else -np.inf
            assert got[b] == want, (L, b)


# ------------------------------------------------------------------ query-aware

def pin_query_scores_closed_form(o):
    """Two chunks whose scaled logits differ by ln 3 get softmax weights 1/4
    and 3/4; the scale is 1/sqrt(d)."""
    d = 128
    c = np.zeros((2, d))
    c[1, 0] = 1.0
    q = np.zeros((1, d))
    q[0, 0] = math.log(3.0) * math.sqrt(d)
    a = o.query_chunk_scores(q, c)
    assert np.allclose(a, [0.25, 0.75], rtol=1e-14, atol=0)


def pin_query_scores_scipy(o):
    """Library routine: scipy's softmax per head, summed over the group."""
    from scipy.special import softmax
    rng = _rng(6)
    for G, C in ((1, 7), (4, 33), (8, 100)):
        q = _bf16_vals(rng, (G, 128), 3.0)
        c = _bf16_vals(rng, (C, 128))
        want = softmax((q @ c.T) / math.sqrt(128), axis=1).sum(axis=0)
        got = o.query_chunk_scores(q, c)
        assert np.allclose(got, want, rtol=1e-12, atol=0)
        assert math.isclose(got.sum(), G, rel_tol=1e-12)


# ------------------------------------------------------------------ selection

def pin_roles(o):
    """Sink, window and candidates partition the blocks, by brute force."""
    for L in range(1, 1200, 7):
        for n_s, n_w in ((1, 2), (1, 4), (2, 3), (0, 2)):
            r = o.block_roles(L, n_s, n_w)
            nb = -(-L // 64)
            assert r.nb == nb
            allb = sorted(r.sink + r.window + r.candidates)
            assert allb == list(range(nb)), (L, n_s, n_w)
            assert r.sink == [b for b in range(nb) if b < n_s]
            assert r.window == [b for b in range(nb)
                                if b >= n_s and b >= nb - n_w]
            for b in r.candidates:                     # complete blocks only
                assert 64 * (b + 1) <= L


def pin_topk_lexsort(o):
    """Library routine: numpy's lexsort on (score descending, id ascending),
    with many exact ties."""
    rng = _rng(7)
    for n, k in ((1, 1), (10, 3), (50, 50), (300, 16), (300, 0), (40, 64)):
        scores = rng.integers(0, 6, size=n).astype(np.float64)
        ids = list(range(n))
        want = list(np.lexsort((np.arange(n), -scores))[:max(0, k)])
        assert o.top_by_score(ids, scores, k) == want


def pin_select_reduces_to_plain_topk(o):
    """With k_e' = 0 the selection is sink + window + top-k_q (InfLLM-V2's
    plain selection)."""
    rng = _rng(8)
    r = o.block_roles(64 * 40 + 5, 1, 4)
    Qb = rng.standard_normal(r.nb)
    Eb = rng.standard_normal(r.nb)
    sel = o.select_blocks(Qb, Eb, set(r.candidates), r, 6, 0)
    top = sorted(r.candidates, key=lambda b: -Qb[b])[:6]
    assert sel.blocks == sorted(set(r.sink) | set(r.window) | set(top))
    assert sel.agnostic == []


def _run_pair(o, rng, L0, steps, n_s, n_w, k_q, k_e_dyn, G=2, d=8,
              hot=False, ahead=False):
    cap = L0 + steps
    K = _bf16_vals(rng, (cap, d))
    V = _bf16_vals(rng, (cap, d))
    W1 = _bf16_vals(rng, (d, d), 0.5)
    W2 = _bf16_vals(rng, (d,), 0.5)
    if hot:
        u = rng.standard_normal(d)
        for b in rng.choice(np.arange(n_s, max(n_s + 1, L0 // 64 - n_w)),
                            size=2):
            K[64 * b:64 * b + 64] += u
    p = o.PairOracle(K.copy(), V.copy(), W1, W2, L0, n_s, n_w, k_q, k_e_dyn,
                     1.0)
    out = []
    for t in range(steps):
        qg = _bf16_vals(rng, (G, d), 2.0)
        if ahead:
            f = _bf16_vals(rng, (d,), 2.0)
            out.append(p.step_ahead(f, K[L0 + t], V[L0 + t], qg))
        else:
            out.append(p.step(K[L0 + t], V[L0 + t], qg))
    return out


def pin_agnostic_only_is_streaming_topk(o):
    """With k_q = 0 the agnostic part is a streaming top-k over a fixed
    score: A(t) = top-k_e' of A(t-1) plus the blocks that just left the
    window (closed form of the never-reselect rule)."""
    rng = _rng(9)
    res = _run_pair(o, rng, 64 * 30, 140, 1, 3, 0, 5)
    for t in range(1, len(res)):
        prev, cur = res[t - 1], res[t]
        fresh = set(cur.roles.candidates) - set(prev.roles.candidates)
        pool = set(prev.sel.agnostic) | fresh
        want = sorted(sorted(pool, key=lambda b: (-cur.Eb[b], b))[:5])
        assert cur.sel.agnostic == want, t


def pin_invariants(o, seed=10, cases=12, ahead=False):
    """Theorem 2's bound gamma(t) >= k_e / k, the eligible set only shrinking
    or extending forward in time ([W] How NOSA works), and the bookkeeping
    facts that follow from the construction."""
    rng = _rng(seed)
    for case in range(cases):
        n_s = int(rng.integers(0, 3))
        n_w = int(rng.integers(2, 5))
        k_q = int(rng.integers(0, 5))
        k_e_dyn = int(rng.integers(0, 6))
        L0 = 64 * int(rng.integers(1, 25)) + int(rng.integers(0, 64))
        res = _run_pair(o, rng, L0, 150, n_s, n_w, k_q, k_e_dyn,
                        hot=bool(case % 2), ahead=ahead)
        k = n_s + n_w + k_q + k_e_dyn
        k_e = n_s + n_w + k_e_dyn
        E0 = len(res[0].roles.candidates)
        for t, r in enumerate(res):
            S = r.sel.blocks
            assert len(S) <= k
            assert not set(r.sel.query) & set(r.sel.agnostic)        # I4
            assert set(r.sel.agnostic) <= r.eligible                   # I4
            assert len(r.sel.query) == min(k_q, len(r.roles.candidates))
            assert len(r.eligible) >= min(k_e_dyn, E0)                 # I5
            if t == 0:
                continue
            p = res[t - 1]
            fresh = set(r.roles.candidates) - set(p.roles.candidates)
            assert r.eligible - fresh <= p.eligible                    # I2
            assert r.eligible <= set(p.sel.blocks)                     # I3
            gamma = o.locality(p.sel.blocks, S, r.new_block)
            assert gamma >= k_e / k - 1e-12, (case, t, gamma)          # I1
            assert len(r.misses) <= k_q                                # I7
            have = set(p.sel.blocks) | ({r.new_block} - {None})
            assert r.misses == [b for b in S if b not in have]


def pin_incremental_state_equals_bulk(o):
    """Appending tokens one at a time leaves the state that building it in
    bulk from the whole prefix gives: compressed keys equal compress_keys (the
    pinned mean pooling of [B1B] 核心组件一), chunk means of the eviction score
    equal chunk_means ([L189] 2.1, eqs. 5-6) and the per-token scores equal
    eviction_scores over all values at once. Runs start from no token, from
    just below chunk and block completions, and cross block and window
    boundaries."""
    rng = _rng(18)
    d = 8
    for L0, steps in ((0, 150), (31, 90), (64 * 3 + 15, 120), (64 * 5 + 63, 140)):
        cap = L0 + steps
        K = _bf16_vals(rng, (cap, d), 2.0)
        V = _bf16_vals(rng, (cap, d))
        W1 = _bf16_vals(rng, (d, d), 0.5)
        W2 = _bf16_vals(rng, (d,), 0.5)
        K0, V0 = np.zeros((cap, d)), np.zeros((cap, d))
        K0[:L0], V0[:L0] = K[:L0], V[:L0]
        p = o.PairOracle(K0, V0, W1, W2, L0, 1, 2, 2, 2, 1.0)
        for t in range(steps):
            p.append(K[L0 + t], V[L0 + t])
            L = p.L
            assert L == L0 + t + 1
            if t % 7 and t != steps - 1:
                continue
            ck = np.array(p.ckeys).reshape(-1, d)
            assert np.array_equal(ck, o.compress_keys(K, L)), (L0, t)
            s_bulk = o.eviction_scores(V[:L], W1, W2)
            assert np.allclose(p.s[:L], s_bulk, rtol=1e-12, atol=1e-300), (L0, t)
            e_bulk = o.chunk_means(p.s, L)
            assert len(p.e_chunks) == len(e_bulk) == o.n_chunks(L), (L0, t)
            assert np.allclose(p.e_chunks, e_bulk, rtol=1e-14, atol=0), (L0, t)


def pin_locality_closed_form(o):
    """Hand-counted block-level gamma(t) = |S(t) kept| / |S(t)| ([W] How NOSA
    works, Theorem 2), with the block this step's token opened counted as
    present."""
    # S(t-1) = {0,1,2,5,7}, S(t) = {0,1,2,6,7,8}: kept 0,1,2,7 (+8 if new)
    assert o.locality([0, 1, 2, 5, 7], [0, 1, 2, 6, 7, 8], 8) == 5 / 6
    assert o.locality([0, 1, 2, 5, 7], [0, 1, 2, 6, 7, 8], None) == 4 / 6
    # the newest selected block is neither kept nor new: not counted
    assert o.locality([0, 1, 2], [0, 1, 3], None) == 2 / 3
    # an opened block that is not selected adds nothing
    assert o.locality([0, 1], [0, 1, 4], 5) == 2 / 3
    assert o.locality([4, 9], [4, 9], None) == 1.0


def pin_token_locality_closed_form(o):
    """Hand-counted token-level gamma(t): the share of the selected tokens
    that were selected one step earlier, leaving out the token appended at
    this step ([W] How NOSA works: locality as a fraction of selected
    tokens)."""
    # S(t-1) = {0, 2} at L = 150: tokens 0..63 and 128..149 (86).
    # S(t) = {0, 1, 2} at L = 151: tokens 0..150 less the new 150 (150).
    assert o.token_locality([0, 2], 150, [0, 1, 2], 151) == 86 / 150
    # the new token opens block 2: everything else was selected
    assert o.token_locality([0, 1], 128, [0, 2], 129) == 1.0
    # block 3 dropped, block 1 added: kept 0..63 and 256..299 (108) of
    # 0..127 and 256..299 (172)
    assert o.token_locality([0, 3, 4], 300, [0, 1, 4], 301) == 108 / 172
    # block-level and token-level agree when every block is full and kept
    assert o.token_locality([1, 2], 640, [1, 2], 641) == 1.0


def pin_invariants_ahead(o):
    """The same bound and bookkeeping when every step selects one layer ahead
    with a forecast head (SparDA's order: select and fetch, then append):
    the never-reselect rule and Theorem 2 do not depend on what ranks the
    query-aware stage."""
    pin_invariants(o, seed=12, cases=8, ahead=True)


# ------------------------------------------------------------------ forecast

def pin_forecast_closed_form(o):
    """A forecast head against hand-built compressed keys: the plain logit
    f . c / sqrt(d) per chunk, no normalisation (a softmax would make the
    values sum to 1)."""
    d = 128
    f = np.zeros(d)
    f[0], f[1] = 2.0 * math.sqrt(d), -math.sqrt(d)
    c = np.zeros((3, d))
    c[0, 0] = 1.5                      # 2 * 1.5
    c[1, 1] = 4.0                      # -1 * 4
    c[2, 0], c[2, 1] = 0.25, 0.5       # 0.5 - 0.5
    got = o.forecast_chunk_scores(f, c)
    assert np.allclose(got, [3.0, -4.0, 0.0], rtol=0, atol=1e-12), got


def pin_ahead_equals_single_head_select(o):
    """Selecting one step ahead with forecast head f picks what NOSA's own
    selection picks after the append with f as a one-head group: a softmax
    over one head is increasing in the logit, max-pooling commutes with an
    increasing map, and the chunk the appended token may complete lies in
    the window. Started just below block boundaries, so the length used
    (after the coming token, not before) decides the window and candidates
    at some steps."""
    import copy
    rng = _rng(13)
    d = 8
    for case in range(6):
        n_s, n_w = int(rng.integers(0, 3)), int(rng.integers(2, 5))
        k_q, k_e_dyn = int(rng.integers(1, 5)), int(rng.integers(0, 5))
        L0 = 64 * int(rng.integers(4, 20)) + 62 - case
        cap = L0 + 80
        K = _bf16_vals(rng, (cap, d))
        V = _bf16_vals(rng, (cap, d))
        W1 = _bf16_vals(rng, (d, d), 0.5)
        W2 = _bf16_vals(rng, (d,), 0.5)
        a = o.PairOracle(K.copy(), V.copy(), W1, W2, L0, n_s, n_w, k_q,
                         k_e_dyn, 1.0)
        b = copy.deepcopy(a)
        for t in range(70):
            f = _bf16_vals(rng, (d,), 2.0)
            ra = a.select_ahead(f)
            a.append(K[L0 + t], V[L0 + t])
            b.append(K[L0 + t], V[L0 + t])
            rb = b.select(f[None, :])
            assert ra.L == rb.L == L0 + t + 1
            assert ra.sel.blocks == rb.sel.blocks, (case, t)
            assert ra.sel.kinds == rb.sel.kinds, (case, t)
            assert ra.eligible == rb.eligible, (case, t)
            assert ra.misses == rb.misses, (case, t)


# ------------------------------------------------------------------ prefill

def pin_prefill_scores_match_decode(o):
    """A prompt query at position L - 1 gets the block scores NOSA's decode
    selection computes at length L for the same query (the decode path is
    pinned above), over 150 steps crossing chunk, block and window
    boundaries."""
    rng = _rng(14)
    d, G = 8, 2
    L0, steps = 64 * 6 + 5, 150
    K = _bf16_vals(rng, (L0 + steps, d))
    V = _bf16_vals(rng, (L0 + steps, d))
    W1 = _bf16_vals(rng, (d, d), 0.5)
    W2 = _bf16_vals(rng, (d,), 0.5)
    p = o.PairOracle(K.copy(), V.copy(), W1, W2, L0, 1, 2, 3, 2, 1.0)
    for t in range(steps):
        qg = _bf16_vals(rng, (G, d), 2.0)
        p.append(K[L0 + t], V[L0 + t])
        r = p.select(qg)
        got = o.prefill_block_scores(qg[None], p.L - 1, np.array(p.ckeys), 1, 2)
        c = r.roles.candidates
        assert np.array_equal(got[0, c], r.Qb[c]), t
        others = [b for b in range(got.shape[1]) if b not in set(c)]
        assert np.all(got[0, others] == -np.inf), t


def pin_prefill_scores_causal(o):
    """Row i depends only on tokens up to position pos0 + i: rewriting every
    later key leaves it unchanged, while the last row sees them."""
    rng = _rng(15)
    d, G, T, pos0 = 8, 4, 70, 64 * 5 + 3
    K = _bf16_vals(rng, (pos0 + T, d))
    Q = _bf16_vals(rng, (T, G, d), 2.0)
    base = o.prefill_block_scores(Q, pos0, o.compress_keys(K, pos0 + T), 1, 2)
    for i in (0, 17, 40, T - 2):
        K2 = K.copy()
        K2[pos0 + i + 1:] = _bf16_vals(rng, (T - i - 1, d), 3.0)
        got = o.prefill_block_scores(Q, pos0, o.compress_keys(K2, pos0 + T), 1, 2)
        assert np.array_equal(got[:i + 1], base[:i + 1]), i
        if T - 1 - i >= 48:                   # a complete chunk of the last row changed
            assert not np.array_equal(got[T - 1], base[T - 1]), i


def pin_prefill_full_budget_is_causal_attention(o):
    """With a budget that covers every block, sparse prefill is full causal
    attention: torch's scaled_dot_product_attention in float64 with the
    eviction-score bias, over the tokens up to each query's position."""
    import torch
    rng = _rng(16)
    d, G, T, pos0 = 128, 2, 90, 200
    L = pos0 + T
    K = _bf16_vals(rng, (L, d))
    V = _bf16_vals(rng, (L, d))
    s = rng.standard_normal(L) * 0.3
    Q = _bf16_vals(rng, (T, G, d), 2.0)
    ck = o.compress_keys(K, L)
    ec = o.chunk_means(s, L)
    nb = -(-L // 64)
    out, sels = o.prefill_sparse_attend(Q, pos0, K, V, s, ck, ec, 1, 2, nb, nb, 1.0)
    for i in (0, 37, T - 1):
        Li = pos0 + i + 1
        assert sels[i].blocks == list(range(-(-Li // 64))), i
        tq = torch.from_numpy(Q[i])[None]                       # [1][G][d]
        tk = torch.from_numpy(K[:Li])[None]
        tv = torch.from_numpy(V[:Li])[None]
        mask = torch.from_numpy(s[:Li])[None, None, :].expand(1, G, Li)
        want = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=mask)[0].numpy()
        assert np.allclose(out[i], want, rtol=1e-12, atol=1e-13), i


def pin_prefill_last_query_is_first_decode_step(o):
    """The prompt's last query, selected and attended at the prompt's length,
    is the first decode step after that prompt (every candidate still
    eligible there, R9)."""
    rng = _rng(17)
    d, G, pos0, T = 8, 2, 64 * 9 + 20, 30
    L = pos0 + T
    K = _bf16_vals(rng, (L + 1, d))
    V = _bf16_vals(rng, (L + 1, d))
    W1 = _bf16_vals(rng, (d, d), 0.5)
    W2 = _bf16_vals(rng, (d,), 0.5)
    Q = _bf16_vals(rng, (T, G, d), 2.0)
    p = o.PairOracle(K.copy(), V.copy(), W1, W2, L - 1, 1, 2, 2, 3, 1.0)
    r = p.step(K[L - 1], V[L - 1], Q[-1])                    # length L
    out, sels = o.prefill_sparse_attend(
        Q, pos0, p.K, p.V, p.s, np.array(p.ckeys), np.array(p.e_chunks), 1, 2, 2, 3, 1.0)
    assert sels[-1].blocks == r.sel.blocks and sels[-1].kinds == r.sel.kinds
    assert np.allclose(out[-1], r.out, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ attention

def pin_attention_full_coverage_sdpa(o):
    """When the selection covers every block, sparse attention is full
    attention: torch's scaled_dot_product_attention in float64 with the
    eviction score as an additive mask (and without it for beta = 0)."""
    import torch
    rng = _rng(11)
    for L in (1, 63, 64, 65, 200, 511):
        G, d = 4, 128
        q = _bf16_vals(rng, (G, d), 2.0)
        K = _bf16_vals(rng, (L, d))
        V = _bf16_vals(rng, (L, d))
        s = rng.standard_normal(L) * 0.3
        blocks = list(range(-(-L // 64)))
        for beta in (1.0, 0.0):
            got = o.attend(q, K, V, s, blocks, L, beta)
            tq, tk, tv = (torch.from_numpy(a)[None] for a in (q, K, V))
            mask = torch.from_numpy(beta * s)[None, None, :].expand(1, G, L)
            want = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=mask)[0].numpy()
            assert np.allclose(got, want, rtol=1e-12, atol=1e-13), (L, beta)


def pin_attention_closed_form(o):
    """Two tokens whose logits (bias included) differ by ln 3 mix their
    values 1:3; tokens past L and unselected blocks are ignored."""
    d = 128
    q = np.zeros((1, d))
    K = np.zeros((130, d))
    V = np.zeros((130, d))
    V[0, 0], V[64, 0], V[129, 0] = 4.0, 8.0, 1000.0
    s = np.zeros(130)
    s[64] = math.log(3.0)
    o_ = o.attend(q, K, V, s, [0, 1, 2], 65, 1.0)
    # block 0: 64 tokens of logit 0 (only token 0 has a nonzero value);
    # block 1: token 64 with logit ln 3; block 2 and token 129 lie past L
    w64 = 3.0 / (64.0 + 3.0)
    w0 = 1.0 / (64.0 + 3.0)
    assert math.isclose(o_[0, 0], w0 * 4.0 + w64 * 8.0, rel_tol=1e-13)


# ------------------------------------------------------------------ budget

def pin_budget_golden(o):
    """The main-experiment budget printed in the aiwiki article."""
    want = {k: v for k, v in read_golden("main_experiment_budget.txt")}
    b = o.budget(int(want["k_tokens"]), int(want["k_q_tokens"]),
                 int(want["n_sink_blocks"]), int(want["window_tokens"]))
    assert b["k"] == int(want["k_blocks"])
    assert b["k_q"] == int(want["k_q_blocks"])
    assert b["k_e"] == int(want["k_e_blocks"])
    assert b["k_e_dyn"] == int(want["k_e_dynamic_blocks"])
    assert b["dynamic"] == int(want["dynamic_blocks"])
    assert math.isclose(b["bound"], float(want["locality_bound"]))
    assert b["transfer_unit"] == int(want["transfer_unit_bytes"])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
