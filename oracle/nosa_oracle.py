"""Plain float64 CPU oracle of NOSA's batched decode step.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's
CPU-baseline leg use this module. It is written from the pages' description
of the method and shares no code with the HIP library.

Sources (the pages are web text; each function names the passage it follows):
  [W]     aiwiki article "NOSA (Native and Offloadable Sparse Attention)"
  [B1B]   "NOSA-1B 核心组件揭秘" (blog post on the NOSA-1B repository)
  [SPARDA] aliyun article on SparDA ("提前预测下一层 KV 访问范围")
  [L189]  "NOSA原生可卸载稀疏注意力机制解析" (l189.com)
  [AIW-S] aiwiki "NOSA", section Adoption in SparDA

Everything is float64 except where a rounding is part of the definition
(compressed keys are bf16, see ``compress_keys``). Inputs are the bf16 bit
patterns the generators produce, lifted exactly to float64.

Readings taken where the pages are silent or ambiguous (each is one branch or
constant below):
  R1  mean-pool kernel 32, stride 16 ([W] Main-experiment configuration note;
      [B1B] 核心组件一; [SPARDA] 轻量化设计与训练).
  R2  a chunk is max-pooled into every 64-token block it overlaps.
  R3  query-aware score: per-q-head softmax over chunks, summed over the GQA
      group, then max-pooled ([B1B] 核心组件三; [SPARDA] 轻量化设计与训练).
  R4  softmax scale 1/sqrt(d), over all complete chunks.
  R5  only complete chunks are scored; candidates are the complete blocks
      between the sink and the window.
  R6  the window is the last n_w blocks, the partial current block included.
  R7  k_e counts sink + window + agnostic dynamic blocks ([W] table).
  R8  "not selected at step t" means not in S(t) at all.
  R9  E(0) = all candidates at the first decode step.
  R10 a stage-2 shortfall is left empty.
  R11 ties: higher score first, then the lower block index.
  R12 the eviction score is an additive logit bias on every attended token
      (beta = 1); beta = 0 gives plain attention.
  R13 one (W1, W2) per KV head, no biases.
  R14 compressed keys are stored in bf16, rounded once from the exact mean.
  R19 SparDA's forecast score: one forecast head per KV group, the logit
      f . c / sqrt(d) against each compressed key, with neither the softmax
      nor a sum over heads, max-pooled to blocks like the query-aware score.
  R20 the layer-ahead selection is taken before the step's token is appended,
      for the length after that append, from the compressed keys that exist
      then; the blocks a forecast picks replace stage 1 (query-aware), and
      stage 2 and the never-reselect rule are NOSA's own.
  R21 a selected block that holds no token yet (the one the coming token
      opens) is not fetched: the append creates it on the device.
  R22 sparse prefill (NOSA_S, sparse in both phases): a prompt query at
      position i is scored exactly as a decode step at length i + 1 would
      score it -- over the chunks complete at that length, candidates between
      the sink and that length's window -- so many queries' scores are one
      causal product against the compressed keys.
  R23 sparse prefill selects per prompt query with both of NOSA's stages and
      every candidate eligible (the never-reselect state starts at decode,
      R9), and attends like a decode step at the query's own length: sink,
      window and selected blocks, tokens up to the query's position, with the
      eviction-score bias.
All functions are pinned by tests (closed forms, brute force, invariants);
the readings themselves are definitional, not fixed by the pages.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

POOL_KERNEL = 32   # R1
POOL_STRIDE = 16   # R1
BLOCK = 64         # [W] Main-experiment configuration: block size 64

SINK, WINDOW, QUERY, AGNOSTIC = 1, 2, 3, 4   # kind codes of selected blocks


# ----------------------------------------------------------------- bf16

def bf16_round(x) -> np.ndarray:
    """Round float64 values directly to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and float32's exponent range: for
    2^(e-1) <= |x| < 2^e the spacing is 2^(e-8), never below 2^-133
    (subnormals); magnitudes that round to 2^128 or more become infinite.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e_q = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(x, -e_q))          # exact scaling, ties to even
    y = np.ldexp(r, e_q)
    return np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, x), y)


def bf16_round_exact(v: Fraction) -> float:
    """Same rounding for an exact rational value."""
    if v == 0:
        return 0.0
    a = abs(v)
    e = math.floor(math.log2(a.numerator)) - math.floor(
        math.log2(a.denominator))
    # settle e so that 2^(e-1) <= a < 2^e
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    while Fraction(2) ** e <= a:
        e += 1
    q = Fraction(2) ** max(e - 8, -133)
    r = round(v / q)                         # Fraction rounds ties to even
    y = r * q
    if abs(y) >= Fraction(2) ** 128:
        return math.copysign(math.inf, v)
    return float(y)


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of bf16-representable float64 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------- CompressK

def n_chunks(L: int) -> int:
    """Complete pooling chunks among L tokens: chunk i is tokens
    [16i, 16i+32) and exists once all of them do ([B1B] 核心组件一)."""
    count = 0
    while count * POOL_STRIDE + POOL_KERNEL <= L:
        count += 1
    return count


def _exact_mean_is_safe(rows: np.ndarray) -> np.ndarray:
    """Per column: True where the float64 sum of these bf16 values is exact.

    Each value has 8 significant bits; a sum of 32 of them needs at most
    8 + 5 bits beyond the span of their exponents, so a span of at most 40
    binades keeps the float64 sum exact.
    """
    nz = rows != 0
    _, e = np.frexp(rows)
    hi = np.where(nz, e, -10_000).max(axis=0)
    lo = np.where(nz, e, 10_000).min(axis=0)
    return (hi - lo <= 40) | (~nz.any(axis=0))


def compress_chunk(rows: np.ndarray) -> np.ndarray:
    """CompressK for one chunk: the mean of its 32 keys, rounded once to bf16.

    [B1B] 核心组件一 (mean pooling of 32-token windows, stride 16); [SPARDA]
    KV 预取的运行时实现 (compressed keys are 1/16 of K, hence K's dtype).
    """
    assert rows.shape[0] == POOL_KERNEL
    total = rows.sum(axis=0)
    out = bf16_round(total / POOL_KERNEL)
    safe = _exact_mean_is_safe(rows)
    for col in np.nonzero(~safe)[0]:
        exact = sum((Fraction(float(v)) for v in rows[:, col]), Fraction(0))
        out[col] = bf16_round_exact(exact / POOL_KERNEL)
    return out


def compress_keys(K: np.ndarray, L: int | None = None) -> np.ndarray:
    """All complete compressed keys of K[:L]: [C][d], bf16-valued float64."""
    L = K.shape[0] if L is None else L
    C = n_chunks(L)
    out = np.empty((C, K.shape[1]), dtype=np.float64)
    for i in range(C):
        start = i * POOL_STRIDE
        out[i] = compress_chunk(K[start:start + POOL_KERNEL])
    return out


# ----------------------------------------------------------------- eviction

def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, x)


def eviction_scores(V: np.ndarray, W1: np.ndarray, W2: np.ndarray):
    """Per-token eviction score s_j = softplus(v_j W1) W2.

    [W] How NOSA works (eviction head adapted from DMA, tau = softplus);
    [L189] 2.1, eq. 4. W1 is [d_in][hidden], W2 is [hidden]; ED-DMA ranks on
    s itself, before any exponential ([W] How NOSA works).
    """
    hidden = softplus(V @ W1)
    return hidden @ W2


def chunk_means(s: np.ndarray, L: int | None = None) -> np.ndarray:
    """Mean of the eviction score over each complete chunk: the first of the
    two poolings that turn per-token agnostic scores into block scores
    ([L189] 2.1, eqs. 5-6; [B1B] 核心组件二)."""
    L = s.shape[0] if L is None else L
    C = n_chunks(L)
    return np.array([s[i * POOL_STRIDE:i * POOL_STRIDE + POOL_KERNEL].mean()
                     for i in range(C)], dtype=np.float64)


def chunks_of_block(b: int, C: int) -> range:
    """Chunks overlapping block b's tokens [64b, 64b+64) (reading R2).

    Chunk i spans tokens [16i, 16i+32); it overlaps the block when
    16i + 32 > 64b and 16i < 64b + 64.
    """
    lo = max(0, (b * BLOCK - POOL_KERNEL) // POOL_STRIDE + 1)
    hi = min(C, -(-((b + 1) * BLOCK) // POOL_STRIDE))
    return range(lo, max(lo, hi))


def block_max_pool(x: np.ndarray, nb: int) -> np.ndarray:
    """Max of the chunk values over the chunks overlapping each block;
    -inf where a block has no complete chunk ([L189] 2.1, eqs. 5-6)."""
    C = x.shape[0]
    out = np.full(nb, -np.inf)
    for b in range(nb):
        r = chunks_of_block(b, C)
        if len(r):
            out[b] = x[r.start:r.stop].max()
    return out


# ----------------------------------------------------------------- query-aware

def query_chunk_scores(q: np.ndarray, ckeys: np.ndarray) -> np.ndarray:
    """Query-aware chunk score a_i for one GQA group.

    q is [G][d] (the group's query heads), ckeys is [C][d]. A lightweight
    attention of each head over the compressed keys ([B1B] 核心组件三), a
    softmax per head over the chunks, summed over the group's heads
    ([SPARDA] 轻量化设计与训练 names that softmax aggregation). R3, R4.
    """
    d = q.shape[1]
    logits = (q @ ckeys.T) / math.sqrt(d)          # [G][C]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


def forecast_chunk_scores(f: np.ndarray, ckeys: np.ndarray) -> np.ndarray:
    """SparDA's forecast score of each chunk (R19): the KV group's single
    forecast head against the compressed keys, as a plain scaled logit --
    SparDA keeps one forecast head per KV head and drops the softmax used to
    combine a group's query heads ([SPARDA] 解耦选块与注意力计算, 轻量化设计与训练).
    f is [d], ckeys is [C][d]."""
    d = f.shape[0]
    return (ckeys @ f) / math.sqrt(d)


def prefill_block_scores(Q: np.ndarray, pos0: int, ckeys: np.ndarray,
                         n_sink: int, n_win: int) -> np.ndarray:
    """Query-aware block scores of many prompt queries at once (R22; the
    query-aware score of [B1B] 核心组件三 and R3, applied per query with
    causal chunk sets; NOSA_S is sparse in both phases, [W] Results).

    Q is [T][G][d]: query i sits at position pos0 + i. ckeys holds at least
    every chunk complete at length pos0 + T. Returns [T][nb] with nb the block
    count at length pos0 + T: row i holds Q_b for the candidate blocks of
    length pos0 + i + 1 and -inf elsewhere.
    """
    T = Q.shape[0]
    nb_all = n_blocks(pos0 + T)
    out = np.full((T, nb_all), -np.inf)
    for i in range(T):
        L = pos0 + i + 1
        C = n_chunks(L)
        roles = block_roles(L, n_sink, n_win)
        if C == 0 or not roles.candidates:
            continue
        a = query_chunk_scores(Q[i], ckeys[:C])
        Qb = block_max_pool(a, roles.nb)
        out[i, roles.candidates] = Qb[roles.candidates]
    return out


def prefill_sparse_attend(Q: np.ndarray, pos0: int, K: np.ndarray,
                          V: np.ndarray, s: np.ndarray, ckeys: np.ndarray,
                          e_chunks: np.ndarray, n_sink: int, n_win: int,
                          k_q: int, k_e_dyn: int, beta: float):
    """NOSA_S-style sparse prefill of T prompt queries of one pair (R22, R23;
    [W] Results: sparse in both phases). Q is [T][G][d]; query i sits at
    position pos0 + i; K, V, s hold the prompt's tokens, ckeys and e_chunks
    its complete chunks. Returns (outputs [T][G][d], selections)."""
    scores = prefill_block_scores(Q, pos0, ckeys, n_sink, n_win)
    outs, sels = [], []
    for i in range(Q.shape[0]):
        L = pos0 + i + 1
        roles = block_roles(L, n_sink, n_win)
        Eb = block_max_pool(np.asarray(e_chunks[:n_chunks(L)]), roles.nb)
        sel = select_blocks(scores[i, :roles.nb], Eb, set(roles.candidates),
                            roles, k_q, k_e_dyn)
        outs.append(attend(Q[i], K, V, s, sel.blocks, L, beta))
        sels.append(sel)
    return np.stack(outs), sels


# ----------------------------------------------------------------- selection

def n_blocks(L: int) -> int:
    return -(-L // BLOCK)


@dataclass
class Roles:
    nb: int
    sink: list
    window: list
    candidates: list


def block_roles(L: int, n_sink: int, n_win: int) -> Roles:
    """Sink, sliding window and the dynamic candidates ([W] How NOSA works:
    NOSA keeps InfLLM-V2's attention sink and sliding window; R5, R6)."""
    nb = n_blocks(L)
    sink = list(range(min(n_sink, nb)))
    win_lo = max(n_sink, nb - n_win)
    window = list(range(win_lo, nb))
    candidates = list(range(n_sink, max(n_sink, nb - n_win)))
    return Roles(nb, sink, window, candidates)


def top_by_score(ids, scores, k: int) -> list:
    """The first min(k, len(ids)) ids by descending score, then ascending id
    (R11)."""
    order = sorted(ids, key=lambda b: (-scores[b], b))
    return order[:max(0, k)]


@dataclass
class Selection:
    blocks: list          # ascending
    kinds: dict           # block -> SINK / WINDOW / QUERY / AGNOSTIC
    query: list
    agnostic: list


def select_blocks(Qb, Eb, eligible: set, roles: Roles, k_q: int,
                  k_e_dyn: int) -> Selection:
    """Two-stage selection ([W] How NOSA works; [L189] 2.1).

    Stage 1 takes the k_q candidates with the highest query-aware score.
    Their combined score is then +inf, so the final arg-top-k keeps them and
    fills the remaining k_e' dynamic slots from the highest query-agnostic
    scores of the other eligible candidates -- the same as excluding the
    stage-1 blocks from stage 2. A stage-2 shortfall stays empty (R10).
    """
    cand = roles.candidates
    query = top_by_score(cand, Qb, k_q)
    qset = set(query)
    pool = [b for b in cand if b in eligible and b not in qset]
    agn = top_by_score(pool, Eb, k_e_dyn)
    kinds = {}
    for b in roles.sink:
        kinds[b] = SINK
    for b in roles.window:
        kinds[b] = WINDOW
    for b in query:
        kinds[b] = QUERY
    for b in agn:
        kinds[b] = AGNOSTIC
    return Selection(sorted(kinds), kinds, sorted(query), sorted(agn))


# ----------------------------------------------------------------- attention

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, s: np.ndarray,
           blocks, L: int, beta: float) -> np.ndarray:
    """Sparse attention over the selected blocks' existing tokens.

    o_h = sum_j softmax_j(q_h . k_j / sqrt(d) + beta * s_j) v_j over the
    tokens of the selected blocks ([B1B] 解码阶段如何只用 64 个 KV 块; the
    eviction score enters as an additive logit bias, [W] How NOSA works;
    [L189] 2.1, eq. 8). The page's V-scaling plus all-ones-V denominator is
    the same quantity.
    """
    d = q.shape[1]
    J = [j for b in sorted(blocks)
         for j in range(b * BLOCK, min((b + 1) * BLOCK, L))]
    J = np.array(J, dtype=np.int64)
    logits = (q @ K[J].T) / math.sqrt(d) + beta * s[J][None, :]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    w /= w.sum(axis=1, keepdims=True)
    return w @ V[J]


# ----------------------------------------------------------------- one pair

@dataclass
class StepResult:
    L: int
    roles: Roles
    sel: Selection
    Qb: np.ndarray
    Eb: np.ndarray
    eligible: set          # E(t), the eligible candidates used at this step
    misses: list           # blocks fetched from host this step
    new_block: int | None  # block opened by this step's token, if any
    out: np.ndarray | None = None


@dataclass
class PairOracle:
    """State of one (sequence, KV head) pair across decode steps.

    K, V are float64 [capacity][d]; q heads of the group are passed per step.
    """
    K: np.ndarray
    V: np.ndarray
    W1: np.ndarray
    W2: np.ndarray
    L: int
    n_sink: int
    n_win: int
    k_q: int
    k_e_dyn: int
    beta: float
    s: np.ndarray = field(init=False)
    ckeys: list = field(init=False)
    e_chunks: list = field(init=False)
    carry: set | None = field(init=False, default=None)   # E(t-1) ∩ S(t-1)
    prev_cand: list | None = field(init=False, default=None)
    prev_sel: list | None = field(init=False, default=None)

    def __post_init__(self):
        cap = self.K.shape[0]
        self.s = np.zeros(cap)
        self.s[:self.L] = eviction_scores(self.V[:self.L], self.W1, self.W2)
        c = compress_keys(self.K, self.L)
        self.ckeys = [row for row in c]
        self.e_chunks = list(chunk_means(self.s, self.L))

    # -- steps of one decode step, in order --------------------------------
    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """Append the new token; extend CompressK and the eviction scores."""
        j = self.L
        self.K[j] = k_new
        self.V[j] = v_new
        self.s[j] = eviction_scores(v_new[None, :], self.W1, self.W2)[0]
        self.L += 1
        C = n_chunks(self.L)
        while len(self.ckeys) < C:
            i = len(self.ckeys)
            rows = self.K[i * POOL_STRIDE:i * POOL_STRIDE + POOL_KERNEL]
            self.ckeys.append(compress_chunk(rows))
            self.e_chunks.append(
                self.s[i * POOL_STRIDE:i * POOL_STRIDE + POOL_KERNEL].mean())
        return j

    def _ckeys(self) -> np.ndarray:
        C = len(self.ckeys)
        return np.array(self.ckeys) if C else np.zeros((0, self.K.shape[1]))

    def select(self, q_group: np.ndarray) -> StepResult:
        """NOSA's selection at the current length (after the append)."""
        ck = self._ckeys()
        a = query_chunk_scores(q_group, ck) if len(ck) else np.zeros(0)
        return self._select_at(self.L, a, self.L - 1)

    def select_ahead(self, f: np.ndarray) -> StepResult:
        """SparDA's layer-ahead selection (R19, R20; [SPARDA]
        解耦选块与注意力计算, KV 预取的运行时实现): taken before the step's
        token is appended, for the length L + 1 it will have, with the
        forecast head f [d] in place of the group's queries."""
        ck = self._ckeys()
        a = forecast_chunk_scores(f, ck) if len(ck) else np.zeros(0)
        return self._select_at(self.L + 1, a, self.L)

    def _select_at(self, L: int, a: np.ndarray, newest: int) -> StepResult:
        """Both stages and the eligibility update at length L, from the
        chunk scores a; `newest` is the position of the step's token."""
        roles = block_roles(L, self.n_sink, self.n_win)
        Qb = block_max_pool(a, roles.nb)
        Eb = block_max_pool(np.array(self.e_chunks), roles.nb)
        # eligibility, [W] How NOSA works: a block not selected at step t is
        # never again picked by the query-agnostic part (R8, R9)
        if self.carry is None:
            eligible = set(roles.candidates)
        else:
            fresh = set(roles.candidates) - set(self.prev_cand)
            eligible = (self.carry | fresh) & set(roles.candidates)
        sel = select_blocks(Qb, Eb, eligible, roles, self.k_q, self.k_e_dyn)
        self.carry = eligible & set(sel.blocks)
        self.prev_cand = roles.candidates
        new_block = newest // BLOCK if newest % BLOCK == 0 else None
        if self.prev_sel is None:
            misses = [b for b in sel.blocks if b != new_block]
        else:
            have = set(self.prev_sel)
            misses = [b for b in sel.blocks
                      if b not in have and b != new_block]
        self.prev_sel = list(sel.blocks)
        return StepResult(L, roles, sel, Qb, Eb, eligible, misses, new_block)

    def attend(self, q_group: np.ndarray, blocks) -> np.ndarray:
        return attend(q_group, self.K, self.V, self.s, blocks, self.L,
                      self.beta)

    def step(self, k_new, v_new, q_group) -> StepResult:
        """append -> select -> fetch model -> attend, as one decode step."""
        self.append(k_new, v_new)
        r = self.select(q_group)
        r.out = self.attend(q_group, r.sel.blocks)
        return r

    def step_ahead(self, f, k_new, v_new, q_group) -> StepResult:
        """SparDA's order: layer-ahead selection (and fetch) -> append ->
        attend over the selected blocks with the layer's own queries."""
        r = self.select_ahead(f)
        self.append(k_new, v_new)
        assert self.L == r.L
        r.out = self.attend(q_group, r.sel.blocks)
        return r


def locality(prev: list, cur: list, new_block) -> float:
    """Block-level gamma(t): the share of S(t) already in S(t-1), counting the
    block opened by this step's token as already present ([W] How NOSA works,
    Theorem 2)."""
    have = set(prev)
    if new_block is not None:
        have.add(new_block)
    return sum(1 for b in cur if b in have) / len(cur)


def selected_tokens(blocks, L: int) -> set:
    """Positions of the existing tokens (< L) of the given blocks."""
    return {j for b in blocks for j in range(b * BLOCK, min((b + 1) * BLOCK, L))}


def token_locality(prev: list, L_prev: int, cur: list, L_cur: int) -> float:
    """Token-level gamma(t), as [W] How NOSA works measures locality: the share
    of the tokens selected at step t that were also selected at step t-1.
    The token appended at this step (position L_cur - 1) could not have been
    selected before, so it is left out of the count."""
    now = selected_tokens(cur, L_cur)
    now.discard(L_cur - 1)
    if not now:
        return 1.0
    before = selected_tokens(prev, L_prev)
    return len(now & before) / len(now)


# ----------------------------------------------------------------- budget

def budget(k_tokens: int, k_q_tokens: int, n_sink: int, window_tokens: int,
           block: int = BLOCK) -> dict:
    """Budget arithmetic of the main experiment ([W] Main-experiment
    configuration): k = k_q + k_e, with k_e counting sink + window +
    query-agnostic dynamic blocks (R7); the locality bound is k_e / k."""
    k = k_tokens // block
    k_q = k_q_tokens // block
    n_w = window_tokens // block
    k_e = k - k_q
    return dict(k=k, k_q=k_q, k_e=k_e, k_e_dyn=k_e - n_sink - n_w,
                dynamic=k - n_sink - n_w, bound=k_e / k,
                transfer_unit=block * 128 * 2)
