"""The two measuring probes of the C ABI on the GPU: nosa_link_copy (the
host-link ceiling's copy) moves the bytes it is given, and nosa_hbm_read
(the HBM read ceiling's streaming read) reads every byte once, at several
workgroup counts and with a ragged tail."""

import ctypes
import sys

import numpy as np
import pytest
import torch

from trainable_offloadable_block_amd import _lib as L

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("n16,n_wg", [(1, 1), (1000003, 7), (1 << 20, 256), (4099, 1024)])
def test_hbm_read_xor_covers_every_word(n16, n_wg):
    print(f"[probe] hbm_read n16={n16} n_wg={n_wg}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(n16 + n_wg)
    host = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((n_wg * 256, 4), -1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.check(L.lib().nosa_hbm_read(_ptr(src), n16 * 16, n_wg, _ptr(sink), stream), "hbm_read")
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32), axis=0)
    want = np.bitwise_xor.reduce(host, axis=0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n16,n_wg", [(1, 1), (300007, 5), (1 << 18, 64)])
def test_link_copy_moves_the_bytes(n16, n_wg):
    print(f"[probe] link_copy n16={n16} n_wg={n_wg}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(7 * n16 + n_wg)
    host = rng.integers(-2**31, 2**31, size=(n16, 4), dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).pin_memory()
    alias = ctypes.c_void_p()
    L.check(L.lib().nosa_host_alias(ctypes.c_void_p(src.data_ptr()), ctypes.byref(alias)),
            "host_alias")
    dst = torch.zeros((n16, 4), dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.check(L.lib().nosa_link_copy(alias, _ptr(dst), n16 * 16, n_wg, stream), "link_copy")
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), host)
