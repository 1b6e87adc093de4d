"""The library's launches captured in a HIP graph (through torch.cuda.CUDAGraph)
replay to the eager results: each graph is replayed several times with eager
work of the program's own and synchronisations in between, and every replay is
compared with the eager call bit for bit (both paths are deterministic: the
decode merges its splits in split order and resets its own counters, so no
memset sits in the graph).  Also checked against the FP64 oracle once."""
import numpy as np
import pytest
import torch

from oracle import decode_ref, prefill_ref
from paged_kv_cache_205_amd import ops, synth
from tests.helpers import check_close, say
from tests.test_oracle import rand_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()


def capture(fn):
    """Capture fn() on a side stream after one eager warm-up call; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def test_fused_append_decode_replays():
    lay = synth.small()
    l = 5
    k_pool, v_pool = synth.make_pools(lay, "cuda", layers=[l])
    x = synth.step_inputs(lay, l, "cuda")
    bt = torch.from_numpy(lay.block_tables[l]).cuda()
    sl = torch.from_numpy(lay.seq_lens).cuda()
    ws = ops.workspace_for(lay.B, lay.max_blocks)
    out = torch.empty((lay.B, 32, 64), device="cuda")

    def step():
        ops.pa_append_decode(x["k_new"], x["v_new"], k_pool, v_pool, x["q"], bt, sl, lay.scale, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    pool_k, pool_v = synth.bits(k_pool), synth.bits(v_pool)
    ref = decode_ref(synth.bits(x["q"]), pool_k, pool_v, lay.block_tables[l], lay.seq_lens, lay.scale)
    check_close(eager.cpu().numpy(), ref, "eager fused step")
    g = capture(step)
    other = torch.empty_like(out)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"fused decode graph replay {rep}")
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        # the appends replayed onto the same slots: the pool is unchanged
        assert np.array_equal(synth.bits(k_pool), pool_k) and np.array_equal(synth.bits(v_pool), pool_v)
        # eager work of the program's own between replays (same workspace, other output)
        ops.pa_decode(x["q"], k_pool, v_pool, bt, sl, lay.scale, out=other, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


@pytest.mark.parametrize("weights", ["bf16x2", "fp16"])
def test_prefill_replays(weights):
    rng = np.random.default_rng(40)
    lens = [1, 70, 0, 130, 33]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qh, kh, vh = rand_bits(rng, (T, 32, 64)), rand_bits(rng, (T, 8, 64)), rand_bits(rng, (T, 8, 64))
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, cud = dev(qh), dev(kh), dev(vh), torch.from_numpy(cu).cuda()
    out = torch.empty((T, 32, 64), device="cuda")

    def step():
        ops.pa_prefill(q, k, v, cud, 0.125, out=out, weights=weights)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    check_close(eager.cpu().numpy(), prefill_ref(qh, kh, vh, cu, 0.125), f"eager prefill {weights}")
    g = capture(step)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"prefill ({weights}) graph replay {rep}")
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        ops.pa_prefill(q, k, v, cud, 0.125, weights=weights)  # eager work in between, fresh output
        torch.cuda.synchronize()


def test_queued_decode_replays():
    """A mixed batch whose items exceed the workgroups that take them (300
    sequences, one workgroup per CU, the rest from the queue): every replay
    equals the eager call bit for bit, so the queue and the split counters are
    back at zero after each call, also inside a graph."""
    lay = synth.fragmented(B=300, n_layers=1)
    k_pool, v_pool = synth.make_pools(lay, "cuda")
    x = synth.step_inputs(lay, 0, "cuda")
    bt = torch.from_numpy(lay.block_tables[0]).cuda()
    sl = torch.from_numpy(lay.seq_lens).cuda()
    ws = ops.workspace_for(lay.B, lay.max_blocks)
    out = torch.empty((lay.B, 32, 64), device="cuda")

    def step():
        ops.pa_append_decode(x["k_new"], x["v_new"], k_pool, v_pool, x["q"], bt, sl, lay.scale, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    sample = [0, 1, 2, 3, int(np.argmax(lay.seq_lens)), lay.B - 1]
    pool_k, pool_v = synth.bits(k_pool), synth.bits(v_pool)
    ref = decode_ref(synth.bits(x["q"]), pool_k, pool_v, lay.block_tables[0], lay.seq_lens, lay.scale, batch=sample)
    check_close(eager.cpu().numpy()[sample], ref[sample], "eager queued step")
    g = capture(step)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"queued decode graph replay {rep}")
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        other = ops.pa_decode(x["q"], k_pool, v_pool, bt, sl, lay.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


def test_rope_append_replays():
    """RoPE + append captured in a graph: between replays the program's own eager
    work overwrites the rotated queries and the appended slots; every replay
    restores them bit for bit, equal to the eager call and to the oracle."""
    from oracle.rope import rope_append_ref
    lay = synth.small()
    l = 2
    k_pool, v_pool = synth.make_pools(lay, "cuda", layers=[l])
    x = synth.step_inputs(lay, l, "cuda")
    table = synth.rope_table(2048, device="cuda")
    bt = torch.from_numpy(lay.block_tables[l]).cuda()
    sl = torch.from_numpy(lay.seq_lens).cuda()
    q_out = torch.empty_like(x["q"])
    kp0, vp0 = synth.bits(k_pool), synth.bits(v_pool)

    def step():
        ops.pa_rope_append(x["q"], x["k_new"], x["v_new"], table, k_pool, v_pool, bt, sl, q_out=q_out)

    step()
    torch.cuda.synchronize()
    eager_q, eager_k, eager_v = q_out.clone(), k_pool.clone(), v_pool.clone()
    qr, kr, vr = rope_append_ref(synth.bits(x["q"]), synth.bits(x["k_new"]), synth.bits(x["v_new"]),
                                 table.cpu().numpy(), kp0, vp0, lay.block_tables[l], lay.seq_lens,
                                 np.zeros((lay.B, 32, 64), np.uint16))
    assert np.array_equal(synth.bits(eager_q), qr)
    assert np.array_equal(synth.bits(eager_k), kr) and np.array_equal(synth.bits(eager_v), vr)
    g = capture(step)
    junk_k = torch.full_like(x["k_new"], 3.0)
    junk_v = torch.full_like(x["v_new"], -5.0)
    for rep in range(3):
        q_out.fill_(7.0)
        ops.pa_append(junk_k, junk_v, k_pool, v_pool, bt, sl)  # clobbers every appended slot
        torch.cuda.synchronize()
        assert not torch.equal(k_pool.view(torch.int16), eager_k.view(torch.int16))
        say(f"rope_append graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_out.view(torch.int16), eager_q.view(torch.int16)), f"replay {rep}: q_out"
        assert torch.equal(k_pool.view(torch.int16), eager_k.view(torch.int16)), f"replay {rep}: k_pool"
        assert torch.equal(v_pool.view(torch.int16), eager_v.view(torch.int16)), f"replay {rep}: v_pool"
