"""ctypes binding of libnosa.so (argument marshalling only).

torch is imported first on purpose: it loads the HIP runtime that libnosa.so
links against by soname, so torch's allocations and these kernels share one
runtime. Nothing here computes any step of the method.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (provides the HIP runtime; see module docstring)

PKG = os.path.dirname(os.path.abspath(__file__))
# NOSA_LIBRARY may name another build of the same library (e.g. a tuning
# variant); by default the in-tree build is used.
LIB_PATH = os.environ.get("NOSA_LIBRARY") or os.path.join(PKG, "libnosa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "nosa.h")

NOSA_OK = 0
NOSA_ERR_INVALID = -1
NOSA_ERR_UNSUPPORTED = -2
NOSA_ERR_CAPACITY = -3
NOSA_ERR_WORKSPACE = -4
NOSA_ERR_HIP = -5

NOSA_STATUS_CAPACITY = 1
NOSA_STATUS_BAD_SEL = 2
NOSA_STATUS_LEN_HINT = 4
NOSA_STATUS_SHORT_CONTEXT = 8

NOSA_MAX_FETCH_WORKGROUPS = 4096
NOSA_MAX_READ_WORKGROUPS = 65536
NOSA_DECODE_STATIC_SCRATCH_BYTES = 8 << 20

NOSA_EVICT_BIAS = 1
NOSA_OFFLOAD = 2

NOSA_WS_SELECT, NOSA_WS_FETCH, NOSA_WS_DECODE = 1, 2, 3
NOSA_TUNE_DECODE_BLOCKS_PER_SPLIT, NOSA_TUNE_SELECT_SUBS, NOSA_TUNE_GATHER_VPT = 0, 1, 2
NOSA_TUNE_SELECT_POOL = 3
KIND_NONE, KIND_SINK, KIND_WINDOW, KIND_QUERY, KIND_AGNOSTIC = range(5)

BUFFERS = ["seq_len", "arrive", "status", "ckey", "tok_s", "chunk_e", "blk_e",
           "eligible", "tail_keys", "kv_dev", "kv_host", "slot_of_block",
           "block_of_slot", "w1", "w2"]


class NosaConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "block_size",
        "pool_kernel", "pool_stride", "n_sink_blocks", "window_tokens",
        "k_blocks", "k_q_blocks", "k_e_blocks", "max_context",
        "evict_hidden")] + [("flags", ctypes.c_uint32)]


class NosaState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFERS]


class NosaError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().nosa_last_error().decode(errors="replace")
        text = lib().nosa_strerror(code).decode()
        super().__init__(f"{where}: {text} ({code}): {msg}")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m trainable_offloadable_block_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    cfgp = ctypes.POINTER(NosaConfig)
    stp = ctypes.POINTER(NosaState)
    sig = {
        "nosa_validate_config": (ctypes.c_int, [cfgp]),
        "nosa_state_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(ctypes.c_size_t)]),
        "nosa_workspace_bytes": (ctypes.c_size_t, [cfgp, ctypes.c_int, _I32]),
        "nosa_prefill_init": (ctypes.c_int, [cfgp, stp, _I32, _P]),
        "nosa_compress_append": (ctypes.c_int, [cfgp, stp, _P, _P, _I32, _P]),
        "nosa_select": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _I32, _P]),
        "nosa_append_select": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_size_t, _I32, _P]),
        "nosa_fetch_delta": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P,
                                            ctypes.c_size_t, _P]),
        "nosa_select_forecast": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P, _P,
                                                ctypes.c_size_t, _I32, _P]),
        "nosa_fetch_delta_wg": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _I32, _P,
                                               ctypes.c_size_t, _P]),
        "nosa_sparse_decode": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P,
                                              _P, ctypes.c_size_t, _I32, _P]),
        "nosa_sparse_decode_timed": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P,
                                                    _P, ctypes.c_size_t, _I32, _P, _P, _P]),
        "nosa_sparse_decode_static": (ctypes.c_int, [cfgp, stp, _P, _P, _P, _P, _P, _I32, _P]),
        "nosa_prefill_block_scores": (ctypes.c_int, [cfgp, stp, _P, _I32, _I32, _P, _P]),
        "nosa_prefill_select": (ctypes.c_int, [cfgp, stp, _P, _I32, _I32, _P, _P, _P]),
        "nosa_prefill_attend": (ctypes.c_int, [cfgp, stp, _P, _I32, _I32, _P, _P, _P, _P]),
        "nosa_host_alias": (ctypes.c_int, [_P, ctypes.POINTER(_P)]),
        "nosa_link_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _I32, _P]),
        "nosa_hbm_read": (ctypes.c_int, [_P, ctypes.c_size_t, _I32, _P, _P]),
        "nosa_set_tuning": (ctypes.c_int, [ctypes.c_int, _I32]),
        "nosa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "nosa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/nosa.h declares."""
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nosa_[a-z_]+)\s*\(", text)))


def check(code: int, where: str):
    if code != NOSA_OK:
        raise NosaError(code, where)


class tuning:
    """Context manager that sets one nosa_set_tuning knob and restores its
    previous value on exit."""

    def __init__(self, knob: int, value: int):
        self.knob, self.value, self.prev = knob, int(value), None

    def __enter__(self):
        prev = lib().nosa_set_tuning(self.knob, self.value)
        if prev < 0:
            raise NosaError(prev, "set_tuning")
        self.prev = prev
        return self

    def __exit__(self, *exc):
        lib().nosa_set_tuning(self.knob, self.prev)
        return False
