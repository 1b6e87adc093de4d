"""GPU tests of the binding's stream handling and of pa_merge's split rule.

Decode calls that get no workspace or out allocate them on the launch stream:
run on a side stream while the current stream is still busy (and a freed block
full of non-zero bytes waits in the current stream's cache), a multi-split
batch whose items go through the work queue still matches the oracle.

pa_merge takes the split rule pa_decode uses, where partition_tokens above 2048
act as 2048: partial states cut at 2048 tokens merge to the oracle's output
under partition_tokens = 4096 too.
"""
import math

import numpy as np
import pytest
import torch

from oracle import decode_ref, partial_ref
from paged_kv_cache_205_amd import ops, synth
from tests.helpers import Device, check_close, oracle_sequence, say
from tests.test_oracle import random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()


def _busy_current_stream():
    """Queue a few hundred microseconds of work on the current stream and leave a
    freed block of non-zero bytes in its cache."""
    junk = torch.full((1 << 22,), 0x7F, dtype=torch.uint8, device="cuda")
    del junk
    big = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(4):
        big.mul_(1.0001)
    return big


@pytest.mark.parametrize("fused", [False, True])
def test_decode_on_side_stream_without_workspace(fused):
    lay = synth.fragmented(B=16, n_layers=1)
    d = Device(lay)
    x = d.inputs[0]
    refs = [oracle_sequence(d, 0, b) for b in range(lay.B)]  # pre-append pages, the oracle appends
    if not fused:
        d.append(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for part in (16, 0):  # one-page splits: more items than workgroups, the queue in use
        say(f"side-stream decode fused={fused} partition={part}")
        if fused:
            d2 = Device(lay)
            torch.cuda.synchronize()
            big = _busy_current_stream()
            out = ops.pa_append_decode(x["k_new"], x["v_new"], d2.k_pool, d2.v_pool, x["q"], d2.bt[0], d2.seq_lens,
                                       lay.scale, partition_tokens=part, stream=side)
        else:
            big = _busy_current_stream()
            out = ops.pa_decode(x["q"], d.k_pool, d.v_pool, d.bt[0], d.seq_lens, lay.scale,
                                partition_tokens=part, stream=side)
        side.synchronize()
        torch.cuda.synchronize()
        del big
        got = out.cpu().numpy()
        for b in range(lay.B):
            check_close(got[b], refs[b], f"side stream, sequence {b}, partition {part}")


def test_merge_partition_above_2048():
    lens = [4800, 2049, 2048, 100, 0]
    q, kp, vp, bt, L = random_case(77, Hq=32, Hkv=8, D=64, max_blocks=300, lens=lens)
    scale = 0.125
    part = 2048
    S = 3
    B = len(lens)
    po = np.zeros((B, 32, S, 64), np.float32)
    pm = np.zeros((B, 32, S), np.float32)
    pl = np.zeros((B, 32, S), np.float32)
    for b in range(B):
        for h in range(32):
            for s in range(S):
                t0, t1 = s * part, min(int(L[b]), (s + 1) * part)
                if t0 >= t1:
                    continue
                m, l, o = partial_ref(q, kp, vp, bt, L, scale, b, h, t0, t1)
                pm[b, h, s] = m * math.log2(math.e)
                pl[b, h, s] = l
                po[b, h, s] = o
    ref = decode_ref(q, kp, vp, bt, L, scale)
    dev = lambda a: torch.from_numpy(a).cuda()
    for pt in (2048, 4096, 1 << 20):
        out = ops.pa_merge(dev(po), dev(pm), dev(pl), dev(L), pt).cpu().numpy()
        assert np.all(out[L == 0] == 0.0)
        check_close(out[L > 0], ref[L > 0], f"pa_merge partition_tokens={pt}")
