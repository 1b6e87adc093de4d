"""Concurrent calls: decode steps of two different batches issued on two streams
at once, each with its own pools, workspace and plan, leave exactly the outputs
and pools the same calls give one after the other.  Nothing of a call's state
lives outside its arguments (besides which devices have had their LDS limit
raised, the library's only process-wide state is the per-device scratch array
of the allocation-free entry point, not called here), so work that overlaps on
the GPU cannot see another call's counters, queue or partials.  The batches take the
in-kernel work queue and the per-head merge (more items than workgroups,
several splits per sequence) and the planned path.
"""
import pytest
import torch

from paged_kv_cache_205_amd import ops, synth
from tests.helpers import Device, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()


def _run_step(d, planned, part, ws, plan, outs, stream):
    lay = d.lay
    with torch.cuda.stream(stream):
        if planned:
            ops.pa_decode_plan(d.seq_lens, lay.max_blocks, part, plan=plan, stream=stream)
        for l in range(lay.n_layers):
            x = d.inputs[l]
            if planned:
                ops.pa_decode_planned(x["q"], d.k_pool, d.v_pool, d.bt[l], plan, lay.scale, k_new=x["k_new"],
                                      v_new=x["v_new"], out=outs[l], partition_tokens=part, workspace=ws,
                                      stream=stream)
            else:
                ops.pa_append_decode(x["k_new"], x["v_new"], d.k_pool, d.v_pool, x["q"], d.bt[l], d.seq_lens,
                                     lay.scale, out=outs[l], partition_tokens=part, workspace=ws, stream=stream)


def _buffers(lay, part, planned):
    ws = ops.workspace_for(lay.B, lay.max_blocks, part)
    plan = (torch.empty(ops.pa_decode_plan_bytes(lay.B, lay.max_blocks, part), dtype=torch.uint8, device="cuda")
            if planned else None)
    outs = [torch.full((lay.B, 32, 64), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(lay.n_layers)]
    return ws, plan, outs


@pytest.mark.parametrize("planned", [False, True])
def test_two_streams_match_sequential(planned):
    lays = [synth.fragmented(B=48, n_layers=3), synth.skewed(B=600, n_layers=3)]
    parts = [16, 0]  # one-page splits: queue in use and many splits per sequence; automatic
    say(f"concurrent steps planned={planned}: {[l.B for l in lays]} sequences")
    # one after the other on the current stream
    seq = []
    for lay, part in zip(lays, parts):
        d = Device(lay)
        ws, plan, outs = _buffers(lay, part, planned)
        _run_step(d, planned, part, ws, plan, outs, torch.cuda.current_stream())
        torch.cuda.synchronize()
        seq.append((d.k_pool.clone(), d.v_pool.clone(), [o.clone() for o in outs]))
        del d
    # at once, launches interleaved on two side streams
    devs = [Device(lay) for lay in lays]
    bufs = [_buffers(lay, part, planned) for lay, part in zip(lays, parts)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(2):
        if rep:  # the second round runs on pools restored to their starting state
            devs = [Device(lay) for lay in lays]
            torch.cuda.synchronize()
        for i in (0, 1):
            d, (ws, plan, outs) = devs[i], bufs[i]
            _run_step(d, planned, parts[i], ws, plan, outs, streams[i])
        torch.cuda.synchronize()
        for i in (0, 1):
            k_ref, v_ref, o_ref = seq[i]
            d, (_, _, outs) = devs[i], bufs[i]
            for l, (o, r) in enumerate(zip(outs, o_ref)):
                assert torch.equal(o, r), f"batch {i} layer {l} round {rep}: out differs from the sequential call"
            assert torch.equal(d.k_pool.view(torch.int16), k_ref.view(torch.int16)), f"batch {i}: K pool"
            assert torch.equal(d.v_pool.view(torch.int16), v_ref.view(torch.int16)), f"batch {i}: V pool"
