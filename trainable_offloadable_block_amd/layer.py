"""One layer's NOSA decode state on one GPU, driven through the C ABI.

Torch supplies device memory, pinned host memory and the stream; every step
of the decode path runs in libnosa's HIP kernels.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L

BLOCK = 64
HEAD_DIM = 128
BLOCK_ELEMS = 2 * BLOCK * HEAD_DIM


@dataclass(frozen=True)
class LayerShape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    n_sink_blocks: int
    window_tokens: int
    k_blocks: int
    k_q_blocks: int
    k_e_blocks: int
    max_context: int
    offload: bool = False
    evict_bias: bool = True

    def config(self) -> L.NosaConfig:
        c = L.NosaConfig()
        c.batch, c.n_q_heads, c.n_kv_heads = self.batch, self.n_q_heads, self.n_kv_heads
        c.head_dim, c.block_size, c.pool_kernel, c.pool_stride = HEAD_DIM, BLOCK, 32, 16
        c.n_sink_blocks, c.window_tokens = self.n_sink_blocks, self.window_tokens
        c.k_blocks, c.k_q_blocks, c.k_e_blocks = self.k_blocks, self.k_q_blocks, self.k_e_blocks
        c.max_context, c.evict_hidden = self.max_context, 128
        c.flags = (L.NOSA_EVICT_BIAS if self.evict_bias else 0) | (
            L.NOSA_OFFLOAD if self.offload else 0)
        return c

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def pairs(self):
        return self.batch * self.n_kv_heads

    @property
    def nb_max(self):
        return -(-self.max_context // BLOCK)

    @property
    def c_max(self):
        return (self.max_context - 32) // 16 + 1


def _ptr(t):
    # a plain int: the bound functions declare their pointer arguments as
    # c_void_p, which ctypes fills from an int (or None for NULL) directly
    return t.data_ptr() if t is not None else None


# the current stream's handle as an int, through torch's direct accessor
# where it has one (about 10x cheaper per call than current_stream())
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def v_to_tiles(v: np.ndarray) -> np.ndarray:
    """V of whole blocks, [..., 64 tokens, 128 dims] -> the blocks' V parts
    in tile order [..., 2 halves, 8 dim tiles, 4 token groups, 16 dims,
    8 tokens], flattened per block."""
    lead = v.shape[:-2]
    t = v.reshape(*lead, 2, 4, 8, 8, 16)          # half, group, tok, tile, dim
    n = len(lead)
    t = t.transpose(*range(n), n, n + 3, n + 1, n + 4, n + 2)
    return t.reshape(*lead, BLOCK * HEAD_DIM)


def v_from_tiles(flat: np.ndarray) -> np.ndarray:
    """Inverse of v_to_tiles: [..., 64*128] tile order -> [..., 64, 128]."""
    lead = flat.shape[:-1]
    t = flat.reshape(*lead, 2, 8, 4, 16, 8)       # half, tile, group, dim, tok
    n = len(lead)
    t = t.transpose(*range(n), n, n + 2, n + 4, n + 1, n + 3)
    return t.reshape(*lead, BLOCK, HEAD_DIM)


def to_block_layout(K: np.ndarray, V: np.ndarray, nb: int) -> np.ndarray:
    """Token-major K, V ([L][128] uint16 bf16 bits) -> nb blocks of 32 KiB:
    K rows [64][128], then V in tile order (v_to_tiles); zero past L."""
    Lt = K.shape[0]
    out = np.zeros((nb, 2, BLOCK * HEAD_DIM), dtype=np.uint16)
    full = min(nb, Lt // BLOCK)
    if full:
        out[:full, 0] = K[:full * BLOCK].reshape(full, BLOCK * HEAD_DIM)
        out[:full, 1] = v_to_tiles(V[:full * BLOCK].reshape(full, BLOCK, HEAD_DIM))
    rest = Lt - full * BLOCK
    if rest and full < nb:
        kb = np.zeros((BLOCK, HEAD_DIM), dtype=np.uint16)
        vb = np.zeros((BLOCK, HEAD_DIM), dtype=np.uint16)
        kb[:rest] = K[full * BLOCK:]
        vb[:rest] = V[full * BLOCK:]
        out[full, 0] = kb.reshape(-1)
        out[full, 1] = v_to_tiles(vb)
    return out


class NosaLayer:
    """Decode state of one layer: buffers, workspaces and the four calls."""

    def __init__(self, shape: LayerShape, device: str = "cuda"):
        self.shape = shape
        self.device = torch.device(device)
        self._dev_index = (self.device.index if self.device.index is not None
                           else torch.cuda.current_device())
        self.cfg = shape.config()
        lib = L.lib()
        L.check(lib.nosa_validate_config(ctypes.byref(self.cfg)), "validate_config")
        sizes = (ctypes.c_size_t * len(L.BUFFERS))()
        L.check(lib.nosa_state_bytes(ctypes.byref(self.cfg), sizes), "state_bytes")
        self.sizes = dict(zip(L.BUFFERS, list(sizes)))
        # blocks per pair in the KV pool / host store (NB_max, or one more
        # where that stride would crowd the HBM channels): tok_s holds one
        # row of nb_kv * 64 scores per pair
        self.nb_kv = self.sizes["tok_s"] // (shape.pairs * BLOCK * 4)
        dev = self.device
        P, nbm = shape.pairs, shape.nb_max

        def buf(name, dtype, elem):
            n = self.sizes[name] // elem
            return torch.zeros(n, dtype=dtype, device=dev) if n else None

        self.seq_len = buf("seq_len", torch.int32, 4)
        self.arrive = buf("arrive", torch.int32, 4)
        self.status = buf("status", torch.int32, 4)
        self.ckey = buf("ckey", torch.int16, 2)
        self.tok_s = buf("tok_s", torch.float32, 4)
        self.chunk_e = buf("chunk_e", torch.float32, 4)
        self.blk_e = buf("blk_e", torch.float32, 4)
        self.eligible = buf("eligible", torch.int32, 4)
        self.tail_keys = buf("tail_keys", torch.int16, 2)
        self.kv_dev = buf("kv_dev", torch.int16, 2)
        self.slot_of_block = buf("slot_of_block", torch.int32, 4)
        self.block_of_slot = buf("block_of_slot", torch.int32, 4)
        self.w1 = buf("w1", torch.int16, 2)
        self.w2 = buf("w2", torch.int16, 2)
        self.kv_host = None
        self.kv_host_alias = ctypes.c_void_p(0)
        if shape.offload:
            n = self.sizes["kv_host"] // 2
            self.kv_host = torch.zeros(n, dtype=torch.int16, pin_memory=True)
            alias = ctypes.c_void_p()
            L.check(lib.nosa_host_alias(ctypes.c_void_p(self.kv_host.data_ptr()),
                                        ctypes.byref(alias)), "host_alias")
            self.kv_host_alias = alias
        st = L.NosaState()
        for name in L.BUFFERS:
            if name == "kv_host":
                st.kv_host = self.kv_host_alias.value
            else:
                t = getattr(self, name)
                setattr(st, name, t.data_ptr() if t is not None else None)
        self.state = st
        mc = shape.max_context
        self.ws_select = self._ws(L.NOSA_WS_SELECT, mc)
        self.ws_fetch = self._ws(L.NOSA_WS_FETCH, mc)
        self.ws_decode = self._ws(L.NOSA_WS_DECODE, mc)
        k = shape.k_blocks
        self.sel = torch.full((P * k,), -1, dtype=torch.int32, device=dev)
        self.n_sel = torch.zeros(P, dtype=torch.int32, device=dev)
        self.kind = torch.zeros(P * k, dtype=torch.uint8, device=dev)
        self.phys = torch.full((P * k,), -1, dtype=torch.int32, device=dev)
        self.n_miss = torch.zeros(P, dtype=torch.int32, device=dev)
        self.out = torch.zeros(shape.batch * shape.n_q_heads * HEAD_DIM,
                               dtype=torch.float32, device=dev)
        self.dbg_q = None
        self.max_len = 0
        del nbm

    def _ws(self, which, max_len):
        n = L.lib().nosa_workspace_bytes(ctypes.byref(self.cfg), which, max_len)
        # 256-byte alignment: torch's caching allocator hands out 512-byte
        # aligned blocks
        t = torch.zeros(max(n, 256), dtype=torch.uint8, device=self.device)
        assert t.data_ptr() % 256 == 0
        return t

    @property
    def stream(self):
        if _raw_stream is not None:
            return _raw_stream(self._dev_index)
        return torch.cuda.current_stream(self.device).cuda_stream

    # ------------------------------------------------------------ set-up
    def set_weights(self, w1: np.ndarray, w2: np.ndarray):
        """w1 uint16 [Hkv][128][128] (input-major), w2 uint16 [Hkv][128]."""
        self.w1.copy_(torch.from_numpy(np.ascontiguousarray(w1).view(np.int16).reshape(-1)))
        self.w2.copy_(torch.from_numpy(np.ascontiguousarray(w2).view(np.int16).reshape(-1)))

    def load_pair_context(self, p: int, K: np.ndarray, V: np.ndarray):
        """Writes pair p's prefilled K, V (token-major uint16 bf16 bits) into
        the pool (resident) or the pinned host store (offload)."""
        blocks = to_block_layout(K, V, -(-K.shape[0] // BLOCK)).view(np.int16)
        nb = blocks.shape[0]
        flat = blocks.reshape(-1)
        base = p * self.nb_kv * BLOCK_ELEMS
        if self.shape.offload:
            self.kv_host.numpy()[base:base + flat.size] = flat
        else:
            self.kv_dev[base:base + flat.size].copy_(torch.from_numpy(flat))
        del nb

    def prefill(self, lengths):
        """Sets seq_len and builds the decode state from the loaded context."""
        lengths = np.asarray(lengths, dtype=np.int32)
        self.seq_len.copy_(torch.from_numpy(lengths))
        self.max_len = int(lengths.max())
        L.check(L.lib().nosa_prefill_init(ctypes.byref(self.cfg), ctypes.byref(self.state),
                                          self.max_len, self.stream), "prefill_init")

    # ------------------------------------------------------------ the step
    def append(self, k_new: torch.Tensor, v_new: torch.Tensor):
        self.max_len = min(self.max_len + 1, self.shape.max_context)
        L.check(L.lib().nosa_compress_append(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(k_new), _ptr(v_new),
            self.max_len, self.stream), "compress_append")

    def select(self, q: torch.Tensor, want_kind=True, want_qscore=False):
        if want_qscore and self.dbg_q is None:
            self.dbg_q = torch.full((self.shape.pairs * self.shape.nb_max,), float("nan"),
                                    dtype=torch.float32, device=self.device)
        L.check(L.lib().nosa_select(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(q), _ptr(self.sel),
            _ptr(self.n_sel), _ptr(self.kind) if want_kind else ctypes.c_void_p(0),
            _ptr(self.dbg_q) if want_qscore else ctypes.c_void_p(0),
            _ptr(self.ws_select), self.ws_select.numel(), self.max_len, self.stream),
            "select")

    def append_select(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      want_kind=True, want_qscore=False):
        """append then select, in one launch (same results as the two calls)."""
        if want_qscore and self.dbg_q is None:
            self.dbg_q = torch.full((self.shape.pairs * self.shape.nb_max,), float("nan"),
                                    dtype=torch.float32, device=self.device)
        self.max_len = min(self.max_len + 1, self.shape.max_context)
        L.check(L.lib().nosa_append_select(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(k_new), _ptr(v_new),
            _ptr(q), _ptr(self.sel), _ptr(self.n_sel),
            _ptr(self.kind) if want_kind else ctypes.c_void_p(0),
            _ptr(self.dbg_q) if want_qscore else ctypes.c_void_p(0),
            _ptr(self.ws_select), self.ws_select.numel(), self.max_len, self.stream),
            "append_select")

    def fetch(self, sel=None, n_sel=None, force=False):
        """Offload: brings the selection's missing blocks into the cache.
        Resident KV needs no fetch (decode reads each block at its own
        index), so the call is skipped unless force=True."""
        if not self.shape.offload and not force:
            return
        sel = self.sel if sel is None else sel
        n_sel = self.n_sel if n_sel is None else n_sel
        L.check(L.lib().nosa_fetch_delta(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(sel), _ptr(n_sel),
            _ptr(self.phys), _ptr(self.n_miss), _ptr(self.ws_fetch), self.ws_fetch.numel(),
            self.stream), "fetch_delta")

    def select_forecast(self, f: torch.Tensor, want_kind=True, want_fscore=False):
        """SparDA's layer-ahead selection, taken before this step's append
        for the length it will give: stage 1 ranked by the forecast head f
        (dev bf16 [B][Hkv][128]); stage 2 and eligibility as select()."""
        if want_fscore and self.dbg_q is None:
            self.dbg_q = torch.full((self.shape.pairs * self.shape.nb_max,), float("nan"),
                                    dtype=torch.float32, device=self.device)
        L.check(L.lib().nosa_select_forecast(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(f), _ptr(self.sel),
            _ptr(self.n_sel), _ptr(self.kind) if want_kind else ctypes.c_void_p(0),
            _ptr(self.dbg_q) if want_fscore else ctypes.c_void_p(0),
            _ptr(self.ws_select), self.ws_select.numel(),
            min(self.max_len + 1, self.shape.max_context), self.stream), "select_forecast")

    def fetch_wg(self, n_workgroups: int, force=False):
        """fetch() with the copies made by n_workgroups looping workgroups
        (for a fetch that runs beside compute on another stream)."""
        if not self.shape.offload and not force:
            return
        L.check(L.lib().nosa_fetch_delta_wg(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(self.sel), _ptr(self.n_sel),
            _ptr(self.phys), _ptr(self.n_miss), int(n_workgroups), _ptr(self.ws_fetch),
            self.ws_fetch.numel(), self.stream), "fetch_delta_wg")

    def decode(self, q: torch.Tensor, sel=None, phys=None, n_sel=None, events=None):
        """Sparse attention of the step into self.out. With events = (start,
        stop), two torch.cuda.Event(enable_timing=True) objects, the kernel
        stamps its own start and end into them (nosa_sparse_decode_timed)."""
        sel = self.sel if sel is None else sel
        if phys is None:
            phys = self.phys if self.shape.offload else sel
        n_sel = self.n_sel if n_sel is None else n_sel
        args = (ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(q), _ptr(sel),
                _ptr(phys), _ptr(n_sel), _ptr(self.out), _ptr(self.ws_decode),
                self.ws_decode.numel(), self.max_len, self.stream)
        if events is None:
            L.check(L.lib().nosa_sparse_decode(*args), "sparse_decode")
            return
        handles = []
        for ev in events:
            if not ev.cuda_event:          # torch creates the HIP event on first record
                ev.record()
            handles.append(ctypes.c_void_p(ev.cuda_event))
        L.check(L.lib().nosa_sparse_decode_timed(*args, *handles), "sparse_decode_timed")

    def decode_static(self, q: torch.Tensor, sel=None, phys=None, n_sel=None):
        """decode() through nosa_sparse_decode_static: the library's own
        scratch in place of this layer's decode workspace (nothing
        allocated by the call)."""
        sel = self.sel if sel is None else sel
        if phys is None:
            phys = self.phys if self.shape.offload else sel
        n_sel = self.n_sel if n_sel is None else n_sel
        L.check(L.lib().nosa_sparse_decode_static(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(q), _ptr(sel), _ptr(phys),
            _ptr(n_sel), _ptr(self.out), self.max_len, self.stream), "sparse_decode_static")

    def step(self, k_new, v_new, q, want_kind=False, want_qscore=False):
        """append + select (one launch) -> fetch -> decode, all enqueued on
        one stream."""
        self.append_select(k_new, v_new, q, want_kind=want_kind, want_qscore=want_qscore)
        self.fetch()
        self.decode(q)
        return self.out

    def step_ahead(self, f, k_new, v_new, q, fetch_workgroups=0, want_kind=False):
        """One layer in SparDA's order, on one stream: layer-ahead selection
        -> fetch -> append -> decode."""
        self.select_forecast(f, want_kind=want_kind)
        if fetch_workgroups:
            self.fetch_wg(fetch_workgroups)
        else:
            self.fetch()
        self.append(k_new, v_new)
        self.decode(q)
        return self.out

    def prefill_block_scores(self, q: torch.Tensor, n_queries: int, pos0: int) -> torch.Tensor:
        """Block scores of n_queries prompt queries per sequence (q: dev bf16
        [B][n_queries][Hq][128], query i at position pos0 + i): fp32
        [B][Hkv][n_queries][ceil((pos0 + n_queries) / 64)], -inf off the
        candidates."""
        nb = -(-(pos0 + n_queries) // BLOCK)
        out = torch.empty(self.shape.pairs * n_queries * nb, dtype=torch.float32,
                          device=self.device)
        L.check(L.lib().nosa_prefill_block_scores(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(q), int(n_queries),
            int(pos0), _ptr(out), self.stream), "prefill_block_scores")
        return out.view(self.shape.batch, self.shape.n_kv_heads, n_queries, nb)

    def prefill_sparse(self, q: torch.Tensor, n_queries: int, pos0: int):
        """NOSA_S-style sparse prefill of n_queries prompt queries per sequence
        (q: dev bf16 [B][n_queries][Hq][128], query i at position pos0 + i):
        block scores, per-query selection, attention. Returns (out fp32
        [B][n_queries][Hq][128], sel [B][Hkv][n_queries][k], n_sel)."""
        scores = self.prefill_block_scores(q, n_queries, pos0)
        P, k = self.shape.pairs, self.shape.k_blocks
        sel = torch.empty(P * n_queries * k, dtype=torch.int32, device=self.device)
        n_sel = torch.empty(P * n_queries, dtype=torch.int32, device=self.device)
        out = torch.empty(self.shape.batch * n_queries * self.shape.n_q_heads * HEAD_DIM,
                          dtype=torch.float32, device=self.device)
        lib = L.lib()
        L.check(lib.nosa_prefill_select(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(scores), int(n_queries),
            int(pos0), _ptr(sel), _ptr(n_sel), self.stream), "prefill_select")
        self.prefill_attend(q, n_queries, pos0, sel, n_sel, out)
        B, Hkv = self.shape.batch, self.shape.n_kv_heads
        return (out.view(B, n_queries, self.shape.n_q_heads, HEAD_DIM),
                sel.view(B, Hkv, n_queries, k), n_sel.view(B, Hkv, n_queries))

    def prefill_attend(self, q: torch.Tensor, n_queries: int, pos0: int, sel: torch.Tensor,
                       n_sel: torch.Tensor, out: torch.Tensor):
        """Attention of n_queries prompt queries per sequence over the given
        selections (sel dev int32 [B][Hkv][n_queries][k], n_sel [B][Hkv][n_queries])
        into out (dev fp32 [B][n_queries][Hq][128])."""
        L.check(L.lib().nosa_prefill_attend(
            ctypes.byref(self.cfg), ctypes.byref(self.state), _ptr(q), int(n_queries),
            int(pos0), _ptr(sel), _ptr(n_sel), _ptr(out), self.stream), "prefill_attend")
        return out

    # ------------------------------------------------------------ views
    def status_bits(self) -> int:
        return int(self.status.cpu().item()) & 0xFFFFFFFF

    def eligible_words(self) -> np.ndarray:
        words = (self.shape.nb_max + 31) // 32
        return self.eligible.cpu().numpy().view(np.uint32).reshape(self.shape.pairs, words)


class LayerAheadStack:
    """SparDA's cross-layer pipeline over a stack of layers (aliyun article,
    KV 预取的运行时实现): when layer l starts, its forecast head selects layer
    l+1's blocks and the fetch of those blocks starts on a second stream,
    while layer l appends and attends on the main stream; layer l+1 waits for
    its fetch before its append. The first layer selects with its own
    forecast head and fetches (when offloaded) on the main stream. Both
    streams keep the default priority.

    Ordering: the side stream starts layer l+1's work after an event the main
    stream records once layer l-1's decode is enqueued, so it follows layer
    l+1's previous decode (which reads the slots it refills) and append
    (which moved its length); the main stream's append of layer l+1 follows
    the fetch that reassigns its cache slots.

    overlap="select" is the other order the two streams allow: the main
    stream runs each layer's selection one layer ahead (layer l+1's right
    after layer l's fetch is issued) and layer l's append and decode once
    layer l's fetch is done; the side stream runs the fetches back to back,
    each as soon as its selection is done. The chain of fetches is then the
    step's critical path, and the appends and decodes (slowed beside a
    gather, which reads host memory from compute units) fit under it; with
    a small gather budget (8 workgroups, which slow a decode beside them
    about 4x where 32 slow it about 8x) this order ran 1.13-1.16x the
    one-stream step on the 32K stack, where the first order ran 0.95-1.00x.
    Holding each fetch until the previous decode was done (so that a gather
    met only a selection) measured slower than one stream (0.94-0.97x).
    """

    def __init__(self, layers, fetch_workgroups: int = 32, overlap=True):
        self.layers = list(layers)
        self.fetch_workgroups = int(fetch_workgroups)
        self.overlap = overlap              # False, True (beside the decode) or "select"
        dev = self.layers[0].device
        self.side = torch.cuda.Stream(device=dev)
        n = len(self.layers)
        self.ev_start = [torch.cuda.Event() for _ in range(n)]
        self.ev_fetch = [torch.cuda.Event() for _ in range(n)]
        self.ev_sel = [torch.cuda.Event() for _ in range(n)]

    def _select_fetch(self, layer, f):
        layer.select_forecast(f, want_kind=False)
        if self.fetch_workgroups:
            layer.fetch_wg(self.fetch_workgroups)
        else:
            layer.fetch()

    def step(self, inputs):
        """inputs[l] = (f, k_new, v_new, q) of layer l for this step, where f
        is the forecast head that selects layer l (made by layer l-1, or
        layer 0's own). Enqueues the whole step; returns the layers' outputs
        (written when the main stream reaches them)."""
        main = torch.cuda.current_stream(self.layers[0].device)
        n = len(self.layers)
        if not self.overlap:
            for layer, (f, k, v, q) in zip(self.layers, inputs):
                self._select_fetch(layer, f)
                layer.append(k, v)
                layer.decode(q)
            return [layer.out for layer in self.layers]
        if self.overlap == "select":
            self.layers[0].select_forecast(inputs[0][0], want_kind=False)
            self.ev_sel[0].record(main)
            for li in range(n):
                layer = self.layers[li]
                with torch.cuda.stream(self.side):      # layer li's fetch ...
                    self.side.wait_event(self.ev_sel[li])
                    if self.fetch_workgroups:
                        layer.fetch_wg(self.fetch_workgroups)
                    else:
                        layer.fetch()
                    self.ev_fetch[li].record(self.side)
                if li + 1 < n:                          # ... beside layer li+1's selection
                    self.layers[li + 1].select_forecast(inputs[li + 1][0], want_kind=False)
                    self.ev_sel[li + 1].record(main)
                main.wait_event(self.ev_fetch[li])
                _, k, v, q = inputs[li]
                layer.append(k, v)
                layer.decode(q)
            return [layer.out for layer in self.layers]
        self._select_fetch(self.layers[0], inputs[0][0])
        for li in range(n):
            if li + 1 < n:
                self.ev_start[li].record(main)
                with torch.cuda.stream(self.side):
                    self.side.wait_event(self.ev_start[li])
                    self._select_fetch(self.layers[li + 1], inputs[li + 1][0])
                    self.ev_fetch[li + 1].record(self.side)
            if li > 0:
                main.wait_event(self.ev_fetch[li])
            _, k, v, q = inputs[li]
            self.layers[li].append(k, v)
            self.layers[li].decode(q)
        return [layer.out for layer in self.layers]
