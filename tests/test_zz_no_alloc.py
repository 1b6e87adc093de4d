"""pa_append_decode_noalloc: the allocation-free variant of pa_append_decode.

It must leave the pools and out bit-identical to pa_append_decode with its own
workspace, call after call on the one scratch array it shares: a first call on
a larger batch, then a smaller batch with another split size (its counters sit
where the first call's partials were, so they must be cleared), then the first
batch again.  Outputs are also checked against the FP64 oracle.  A call whose
workspace would not fit in the scratch array is refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_205_amd import ops, synth
from tests.helpers import Device, check_close, oracle_sequence, say


def test_oversized_call_is_refused_on_the_host():
    """B = 1024 at 128 table entries under the automatic split needs about 138 MB
    of partials: PA_ERR_SCRATCH, before any device call (no GPU needed)."""
    lib = ops.load()
    A = 0x10000
    need = lib.pa_decode_workspace_bytes(1024, 32, 64, 128, 0)
    assert need > (64 << 20)
    st = lib.pa_append_decode_noalloc(A, A, A, A, A, A, 128, A, ctypes.c_float(0.125), A, 1024, 32, 8, 64, 1 << 20,
                                      0, None)
    assert st == -10
    assert lib.pa_status_string(-10).decode().startswith("PA_ERR_SCRATCH")
    # bad sizes are still shape errors
    assert lib.pa_append_decode_noalloc(A, A, A, A, A, A, 0, A, ctypes.c_float(0.125), A, 4, 32, 8, 64, 16, 0,
                                        None) == -2


def _run_pair(lay, partition, refs_for=()):
    """One layer through pa_append_decode (own workspace) and through the
    allocation-free call, on two copies of the same state."""
    d1 = Device(lay)
    d2 = Device(lay)
    refs = {b: oracle_sequence(d1, 0, b) for b in refs_for}
    x = d1.inputs[0]
    o1 = ops.pa_append_decode(x["k_new"], x["v_new"], d1.k_pool, d1.v_pool, x["q"], d1.bt[0], d1.seq_lens,
                              lay.scale, partition_tokens=partition)
    o2 = torch.full_like(o1, float("nan"))
    ops.pa_append_decode_noalloc(x["k_new"], x["v_new"], d2.k_pool, d2.v_pool, x["q"], d2.bt[0], d2.seq_lens,
                                 lay.scale, o2, partition_tokens=partition)
    torch.cuda.synchronize()
    assert torch.equal(d1.k_pool.view(torch.int16), d2.k_pool.view(torch.int16)), "K pool differs"
    assert torch.equal(d1.v_pool.view(torch.int16), d2.v_pool.view(torch.int16)), "V pool differs"
    assert torch.equal(o1, o2), "out differs"
    got = o2.cpu().numpy()
    for b, r in refs.items():
        check_close(got[b], r, f"{lay.name} sequence {b}")


@pytest.mark.gpu
def test_noalloc_matches_append_decode_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()
    big = synth.fragmented(B=48, n_layers=1)
    small = synth.skewed(B=20, n_layers=1)
    say("noalloc: fragmented B=48, automatic split")
    _run_pair(big, 0, refs_for=range(0, 48, 5))
    say("noalloc: skewed B=20, one-page splits (queue in use)")
    _run_pair(small, 16, refs_for=range(20))
    say("noalloc: fragmented B=48 again, automatic split")
    _run_pair(big, 0)
    say("noalloc: headline shape B=64 x 2048, one layer")
    _run_pair(synth.full(B=64, n_layers=1), 0, refs_for=(0, 31, 63))
