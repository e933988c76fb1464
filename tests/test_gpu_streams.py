"""Independent layers on concurrent HIP streams (the two-micro-batch leg of
bench.py): each layer owns its state and workspace, so two layers stepped on
two streams at once, with no synchronisation between their steps, give the
same selections, kinds, block ids and attention outputs, bit for bit, as
the same layers stepped one after another on one stream."""

import sys

import pytest
import torch

from synth import small_workload
from nosa_harness import Lockstep

pytestmark = pytest.mark.gpu


def _record(ls, t, outs):
    k, v, q = ls.inputs(t)
    ls.gpu.append_select(k, v, q, want_kind=True)
    ls.gpu.fetch()
    ls.gpu.decode(q)
    outs.append(tuple(x.clone() for x in (ls.gpu.sel, ls.gpu.n_sel, ls.gpu.kind, ls.gpu.phys,
                                          ls.gpu.out)))


@pytest.mark.parametrize("offload", [False, True])
def test_two_streams_match_one(offload):
    print(f"[streams] offload={offload}", flush=True)
    sys.stdout.flush()
    steps = 24
    # two micro-batches: different sequences (seeds) and lengths, so their
    # selections and kernels differ; both cross a chunk completion
    wls = [small_workload(171, batch=3, context=1500, steps=steps, offload=offload),
           small_workload(172, batch=2, context=2100, steps=steps, offload=offload)]
    serial = [Lockstep(wl, check_pairs=[]) for wl in wls]
    conc = [Lockstep(wl, check_pairs=[]) for wl in wls]
    ref = [[], []]
    for t in range(steps):
        for i, ls in enumerate(serial):
            _record(ls, t, ref[i])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [[], []]
    for t in range(steps):
        for i, (ls, s) in enumerate(zip(conc, streams)):
            with torch.cuda.stream(s):
                _record(ls, t, got[i])
    torch.cuda.synchronize()
    for i in range(2):
        for t in range(steps):
            for name, a, b in zip(("sel", "n_sel", "kind", "phys", "out"), ref[i][t], got[i][t]):
                assert torch.equal(a, b), f"micro-batch {i} step {t}: {name} differs"
    for ls_a, ls_b in zip(serial, conc):
        assert ls_a.gpu.status_bits() == 0 and ls_b.gpu.status_bits() == 0
