"""nosa_sparse_decode_static -- the sparse decode for callers that cannot
allocate, with its workspace in the library's own scratch -- against
nosa_sparse_decode with a caller workspace, through the C ABI: the same
output bit for bit, over consecutive calls whose sizes shrink and grow
(the scratch keeps the previous call's contents)."""

import pytest
import torch

from nosa_harness import Lockstep
from synth import small_workload

pytestmark = pytest.mark.gpu


def _compare(wl, steps, lengths=None):
    ls = Lockstep(wl, check_pairs=[], steps=steps, lengths=lengths)
    g = ls.gpu
    for t in range(steps):
        kd, vd, qd = ls.inputs(t)
        g.append_select(kd, vd, qd)
        g.fetch()
        g.decode(qd)
        torch.cuda.synchronize()
        ref = g.out.clone()
        g.out.fill_(float("nan"))
        g.decode_static(qd)
        torch.cuda.synchronize()
        assert torch.equal(g.out, ref), f"{wl.name} step {t}: static-scratch decode differs"
    assert g.status_bits() == 0
    print(f"[no-alloc] {wl.name}: {steps} steps equal", flush=True)


def test_static_decode_equals_workspace_decode():
    # larger first: 4 sequences x 2 KV heads, k = 64 over a 3000-token context
    _compare(small_workload(211, batch=4, context=3000, steps=6, window_tokens=1024,
                            k_blocks=40, k_q_blocks=8, k_e_blocks=32), 6)
    # then a smaller input: 2 sequences, ragged lengths, k = 12
    _compare(small_workload(212, batch=2, context=700, steps=5), 5, lengths=[700, 650])
    # then larger again, offloaded, 72 pairs: its arrival counters reach past
    # the bytes the previous calls kept at zero (the library clears them)
    _compare(small_workload(213, batch=36, context=900, steps=4, offload=True), 4)
    # and GQA 4 with 6 KV heads
    _compare(small_workload(214, batch=5, n_q_heads=24, n_kv_heads=6, context=2000, steps=4), 4)
