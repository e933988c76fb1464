"""C-ABI checks that need no GPU: the library loads, exports every function
include/nosa.h declares, and rejects bad arguments in host code before any
HIP call."""

import ctypes

import pytest

import trainable_offloadable_block_amd as nosa
from trainable_offloadable_block_amd import _lib as L
from trainable_offloadable_block_amd.layer import LayerShape


def _cfg(**kw):
    base = dict(batch=2, n_q_heads=16, n_kv_heads=2, n_sink_blocks=1,
                window_tokens=1024, k_blocks=64, k_q_blocks=16, k_e_blocks=48,
                max_context=16640)
    base.update(kw)
    return LayerShape(**base).config()


def test_exports_every_declared_function():
    lib = nosa.lib()
    names = L.header_functions()
    assert len(names) >= 11
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_valid_configs_of_the_workloads():
    from synth import WORKLOADS
    for wl in WORKLOADS.values():
        c = LayerShape(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.n_sink_blocks,
                       wl.window_tokens, wl.k_blocks, wl.k_q_blocks,
                       wl.k_e_blocks, wl.max_context, wl.offload).config()
        assert nosa.lib().nosa_validate_config(ctypes.byref(c)) == 0, wl.name


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=15), L.NOSA_ERR_INVALID),           # not a multiple
    (dict(n_q_heads=64, n_kv_heads=2), L.NOSA_ERR_UNSUPPORTED),  # G = 32
    (dict(k_blocks=63), L.NOSA_ERR_INVALID),             # k != k_q + k_e
    (dict(k_e_blocks=10, k_blocks=26), L.NOSA_ERR_INVALID),  # < sink + window
    (dict(window_tokens=1000), L.NOSA_ERR_INVALID),      # not block-aligned
    (dict(window_tokens=64, k_e_blocks=2, k_blocks=18), L.NOSA_ERR_UNSUPPORTED),
    (dict(k_blocks=144, k_q_blocks=96), L.NOSA_ERR_UNSUPPORTED),  # k > 128
    (dict(max_context=1 << 20), L.NOSA_ERR_UNSUPPORTED),
    (dict(max_context=32), L.NOSA_ERR_UNSUPPORTED),
    (dict(batch=0), L.NOSA_ERR_INVALID),
])
def test_validate_rejects(kw, code):
    c = _cfg(**kw)
    assert nosa.lib().nosa_validate_config(ctypes.byref(c)) == code
    assert nosa.lib().nosa_last_error()


def test_validate_accepts_k_up_to_128():
    """The 8B shape with GQA 16 and a 96-block budget (24 query-aware,
    window 1024), and the largest budget, 128 blocks."""
    lib = nosa.lib()
    for kw in (dict(n_q_heads=32, n_kv_heads=2, k_blocks=96, k_q_blocks=24, k_e_blocks=72),
               dict(k_blocks=128, k_q_blocks=64, k_e_blocks=64)):
        c = _cfg(**kw)
        assert lib.nosa_validate_config(ctypes.byref(c)) == L.NOSA_OK, kw


def test_validate_rejects_bad_fields():
    lib = nosa.lib()
    for field, value, code in (("head_dim", 64, L.NOSA_ERR_UNSUPPORTED),
                               ("pool_stride", 32, L.NOSA_ERR_UNSUPPORTED),
                               ("block_size", 128, L.NOSA_ERR_UNSUPPORTED),
                               ("evict_hidden", 64, L.NOSA_ERR_UNSUPPORTED),
                               ("flags", 8, L.NOSA_ERR_INVALID)):
        c = _cfg()
        setattr(c, field, value)
        assert lib.nosa_validate_config(ctypes.byref(c)) == code, field
    assert lib.nosa_validate_config(None) == L.NOSA_ERR_INVALID


def test_state_bytes_layout():
    lib = nosa.lib()
    c = _cfg()
    sizes = (ctypes.c_size_t * len(L.BUFFERS))()
    assert lib.nosa_state_bytes(ctypes.byref(c), sizes) == 0
    s = dict(zip(L.BUFFERS, sizes))
    P, NB, C = 4, 16640 // 64, (16640 - 32) // 16 + 1
    assert s["kv_dev"] == P * NB * 32768          # resident pool
    assert s["kv_host"] == 0 and s["slot_of_block"] == 0
    assert s["ckey"] == P * C * 256
    assert s["tok_s"] == P * NB * 64 * 4
    assert s["eligible"] == P * ((NB + 31) // 32) * 4
    c.flags |= L.NOSA_OFFLOAD
    assert lib.nosa_state_bytes(ctypes.byref(c), sizes) == 0
    s = dict(zip(L.BUFFERS, sizes))
    assert s["kv_dev"] == P * 65 * 32768          # k + 1 cache slots
    assert s["kv_host"] == P * NB * 32768
    assert s["block_of_slot"] == P * 65 * 4
    # a block count that is a multiple of 129 gets one more block of stride
    # in the pool, the host store and the token scores (not elsewhere)
    for nb, nb_kv in ((258, 259), (257, 257), (387, 388), (516, 517)):
        c = _cfg(max_context=64 * nb)
        for flags in (0, L.NOSA_OFFLOAD):
            c.flags = flags
            assert lib.nosa_state_bytes(ctypes.byref(c), sizes) == 0
            s = dict(zip(L.BUFFERS, sizes))
            assert s["tok_s"] == P * nb_kv * 64 * 4
            assert s["blk_e"] == P * nb * 4
            assert s["eligible"] == P * ((nb + 31) // 32) * 4
            if flags:
                assert s["kv_host"] == P * nb_kv * 32768
                assert s["slot_of_block"] == P * nb * 4
            else:
                assert s["kv_dev"] == P * nb_kv * 32768


def test_workspace_sizes():
    lib = nosa.lib()
    c = _cfg()
    for which in (L.NOSA_WS_SELECT, L.NOSA_WS_FETCH, L.NOSA_WS_DECODE):
        n = lib.nosa_workspace_bytes(ctypes.byref(c), which, 16640)
        assert n > 0 and n % 256 == 0
    assert lib.nosa_workspace_bytes(ctypes.byref(c), 99, 16640) == 0
    assert lib.nosa_workspace_bytes(ctypes.byref(c), L.NOSA_WS_SELECT, 10 ** 6) == 0
    # select workspace grows with the length bound
    small = lib.nosa_workspace_bytes(ctypes.byref(c), L.NOSA_WS_SELECT, 1024)
    big = lib.nosa_workspace_bytes(ctypes.byref(c), L.NOSA_WS_SELECT, 16640)
    assert small < big


def test_calls_reject_before_any_hip_call():
    """Bad arguments come back as error codes without touching a device."""
    lib = nosa.lib()
    c = _cfg()
    st = L.NosaState()                      # all NULL
    null = ctypes.c_void_p(0)
    assert lib.nosa_prefill_init(ctypes.byref(c), ctypes.byref(st), 16, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_compress_append(ctypes.byref(c), None, null, null, 16, null) == L.NOSA_ERR_INVALID
    # a state with every pointer set (never dereferenced by host code)
    for name in L.BUFFERS:
        setattr(st, name, 256)
    assert lib.nosa_compress_append(ctypes.byref(c), ctypes.byref(st), null, null, 16,
                                    null) == L.NOSA_ERR_INVALID
    assert lib.nosa_compress_append(ctypes.byref(c), ctypes.byref(st), 256, 256,
                                    c.max_context + 1, null) == L.NOSA_ERR_CAPACITY
    # select: workspace too small / misaligned
    assert lib.nosa_select(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, null, null,
                           256, 16, 16640, null) == L.NOSA_ERR_WORKSPACE
    assert lib.nosa_select(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, null, null,
                           260, 1 << 40, 16640, null) == L.NOSA_ERR_WORKSPACE
    assert lib.nosa_sparse_decode(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, 256,
                                  256, null, 0, 16640, null) == L.NOSA_ERR_WORKSPACE
    # timed decode: both events required; then the same checks as the plain call
    for evs in ((null, null), (256, null), (null, 256)):
        assert lib.nosa_sparse_decode_timed(ctypes.byref(c), ctypes.byref(st), 256, 256, 256,
                                            256, 256, 256, 1 << 20, 16640, null,
                                            *evs) == L.NOSA_ERR_INVALID
    assert lib.nosa_sparse_decode_timed(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, 256,
                                        256, null, 0, 16640, null, 256,
                                        256) == L.NOSA_ERR_WORKSPACE
    # forecast selection: workspace too small; budgeted fetch: bad budget
    assert lib.nosa_select_forecast(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, null,
                                    null, 256, 16, 16640, null) == L.NOSA_ERR_WORKSPACE
    for n_wg in (0, -3, L.NOSA_MAX_FETCH_WORKGROUPS + 1):
        assert lib.nosa_fetch_delta_wg(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, 256,
                                       n_wg, 256, 1 << 20, null) == L.NOSA_ERR_INVALID
    # prefill scores: no queries, negative position, past max_context, NULL out
    assert lib.nosa_prefill_block_scores(ctypes.byref(c), ctypes.byref(st), 256, 0, 0, 256,
                                         null) == L.NOSA_ERR_INVALID
    assert lib.nosa_prefill_block_scores(ctypes.byref(c), ctypes.byref(st), 256, 4, -1, 256,
                                         null) == L.NOSA_ERR_INVALID
    assert lib.nosa_prefill_block_scores(ctypes.byref(c), ctypes.byref(st), 256, 64,
                                         c.max_context - 10, 256, null) == L.NOSA_ERR_CAPACITY
    assert lib.nosa_prefill_block_scores(ctypes.byref(c), ctypes.byref(st), 256, 4, 0, None,
                                         null) == L.NOSA_ERR_INVALID
    # sparse prefill: bad sizes, NULLs; attention rejects offloaded KV
    assert lib.nosa_prefill_select(ctypes.byref(c), ctypes.byref(st), 256, 0, 0, 256, 256,
                                   null) == L.NOSA_ERR_INVALID
    assert lib.nosa_prefill_select(ctypes.byref(c), ctypes.byref(st), None, 4, 0, 256, 256,
                                   null) == L.NOSA_ERR_INVALID
    assert lib.nosa_prefill_attend(ctypes.byref(c), ctypes.byref(st), 256, 4, c.max_context,
                                   256, 256, 256, null) == L.NOSA_ERR_CAPACITY
    c_off = _cfg()
    c_off.flags |= L.NOSA_OFFLOAD
    assert lib.nosa_prefill_attend(ctypes.byref(c_off), ctypes.byref(st), 256, 4, 0, 256, 256,
                                   256, null) == L.NOSA_ERR_UNSUPPORTED
    # offload without a host store
    c.flags |= L.NOSA_OFFLOAD
    st.kv_host = None
    assert lib.nosa_fetch_delta(ctypes.byref(c), ctypes.byref(st), 256, 256, 256, 256,
                                256, 1 << 20, null) == L.NOSA_ERR_INVALID


def test_strerror():
    lib = nosa.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.nosa_strerror(code)
    assert b"unknown" in lib.nosa_strerror(42)


def test_v_tile_order_matches_the_header_formula():
    """The block's V part: token t, dim c at element
    ((((t/32)*8 + c/16)*4 + (t%32)/8)*16 + c%16)*8 + t%8 (include/nosa.h)."""
    import numpy as np
    v = (np.arange(64)[:, None] * 1000 + np.arange(128)[None, :]).astype(np.int64)
    flat = nosa.v_to_tiles(v)
    for t in range(64):
        for c in range(128):
            i = ((((t // 32) * 8 + c // 16) * 4 + (t % 32) // 8) * 16 + c % 16) * 8 + t % 8
            assert flat[i] == t * 1000 + c
    assert np.array_equal(nosa.v_from_tiles(flat), v)
    many = np.random.default_rng(3).integers(0, 1 << 16, (5, 64, 128))
    assert np.array_equal(nosa.v_from_tiles(nosa.v_to_tiles(many)), many)


def test_tuning_knobs():
    """nosa_set_tuning: range checks, the previous value returned, 0 restores
    the library's choice; the decode workspace follows the split size."""
    lib = nosa.lib()
    c = _cfg()
    for knob, bad in ((L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, 3),
                      (L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, 65),
                      (L.NOSA_TUNE_SELECT_SUBS, -1),
                      (L.NOSA_TUNE_GATHER_VPT, 3), (L.NOSA_TUNE_SELECT_POOL, 3),
                      (7, 1), (-1, 0)):
        assert lib.nosa_set_tuning(knob, bad) == L.NOSA_ERR_INVALID, (knob, bad)
    default = lib.nosa_workspace_bytes(ctypes.byref(c), L.NOSA_WS_DECODE, 16640)
    with L.tuning(L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, 64):
        one_split = lib.nosa_workspace_bytes(ctypes.byref(c), L.NOSA_WS_DECODE, 16640)
        assert lib.nosa_set_tuning(L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, 64) == 64
    assert lib.nosa_set_tuning(L.NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, 0) == 0
    assert one_split < default
    assert lib.nosa_workspace_bytes(ctypes.byref(c), L.NOSA_WS_DECODE, 16640) == default


def test_link_copy_rejects_before_any_hip_call():
    lib = nosa.lib()
    null = ctypes.c_void_p(0)
    assert lib.nosa_link_copy(None, 256, 4096, 8, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_link_copy(256, None, 4096, 8, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_link_copy(256, 256, 4100, 8, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_link_copy(264, 256, 4096, 8, null) == L.NOSA_ERR_INVALID
    for n_wg in (0, L.NOSA_MAX_FETCH_WORKGROUPS + 1):
        assert lib.nosa_link_copy(256, 256, 4096, n_wg, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_link_copy(256, 256, 0, 8, null) == L.NOSA_OK


def test_hbm_read_rejects_before_any_hip_call():
    lib = nosa.lib()
    null = ctypes.c_void_p(0)
    assert lib.nosa_hbm_read(None, 4096, 8, 256, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_hbm_read(256, 4096, 8, None, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_hbm_read(256, 4100, 8, 256, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_hbm_read(264, 4096, 8, 256, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_hbm_read(256, 4096, 8, 264, null) == L.NOSA_ERR_INVALID
    for n_wg in (0, L.NOSA_MAX_READ_WORKGROUPS + 1):
        assert lib.nosa_hbm_read(256, 4096, n_wg, 256, null) == L.NOSA_ERR_INVALID


def test_static_decode_rejects_before_any_hip_call():
    """nosa_sparse_decode_static: NULL arguments, and a config whose decode
    workspace exceeds the static scratch, come back as errors before any HIP
    call."""
    lib = nosa.lib()
    null = ctypes.c_void_p(0)
    c = _cfg()
    st = L.NosaState()
    for name in L.BUFFERS:
        setattr(st, name, 256)
    assert lib.nosa_sparse_decode_static(ctypes.byref(c), ctypes.byref(st), None, 256, 256, 256,
                                         256, 16640, null) == L.NOSA_ERR_INVALID
    assert lib.nosa_sparse_decode_static(ctypes.byref(c), None, 256, 256, 256, 256, 256, 16640,
                                         null) == L.NOSA_ERR_INVALID
    big = _cfg(batch=8192, n_q_heads=32, n_kv_heads=2, max_context=4096, k_blocks=64)
    need = lib.nosa_workspace_bytes(ctypes.byref(big), L.NOSA_WS_DECODE, 4096)
    assert need > L.NOSA_DECODE_STATIC_SCRATCH_BYTES
    assert lib.nosa_sparse_decode_static(ctypes.byref(big), ctypes.byref(st), 256, 256, 256, 256,
                                         256, 4096, null) == L.NOSA_ERR_WORKSPACE
    assert b"STATIC_SCRATCH" in lib.nosa_last_error()
