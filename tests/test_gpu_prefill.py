"""pa_prefill (causal GQA attention of whole prompts over their own K and V) on
the GPU against the FP64 oracle: ragged prompt batches spanning several 64-row
blocks with ragged tails, prompt boundaries inside and at the edges of 16-row
groups, empty and one-token prompts, scale extremes, scores that raise the
running maximum in every tile, the largest batch, and
the full 64 x 2047-row prompt workload (one whole prompt plus sampled rows of
every other).  Tolerance: 2e-3 absolute, 1e-2 row-relative (tests/helpers)."""
import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, prefill_ref, prefill_rows_ref
from paged_kv_cache_205_amd import ops, synth
from tests.helpers import check_close, say
from tests.test_oracle import rand_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def inputs(seed, lens, sigma_q=1.0, sigma_k=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return (rand_bits(rng, (T, 32, 64), sigma_q), rand_bits(rng, (T, 8, 64), sigma_k), rand_bits(rng, (T, 8, 64)), cu)


def run(q, k, v, cu, scale, weights="bf16x2"):
    say(f"pa_prefill: B={len(cu) - 1} T={q.shape[0]} scale={scale} weights={weights}")
    out = ops.pa_prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(cu).cuda(), scale, weights=weights)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def v_spread(v: np.ndarray, cu: np.ndarray, rows=None) -> np.ndarray:
    """max - min of V over the keys each row attends (its prompt up to itself), per KV head and dim,
    expanded to the 32 query heads: [R][32][64]."""
    V = bf16_to_f64(v)
    hi = np.empty_like(V)
    lo = np.empty_like(V)
    for b in range(len(cu) - 1):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        hi[sl] = np.maximum.accumulate(V[sl], axis=0)
        lo[sl] = np.minimum.accumulate(V[sl], axis=0)
    spread = hi - lo if rows is None else hi[rows] - lo[rows]
    return np.repeat(spread, 4, axis=1)


def check_fp16_weights(got, ref, spread, what=""):
    """fp16 weights (2^-11 each, the row sum over the same rounded weights) move an
    output by at most 2^-10 times the spread of the V values it averages; 1e-5 more
    for FP32 accumulation."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = 2.0 ** -10 * spread + 1e-5
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"{what}: fp16 weights, max abs {float(err.max()) if err.size else 0:.2e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the fp16-weight bound"
    # on these N(0, 1) inputs the errors also stay inside the decode tolerance
    check_close(got, ref, what)


CASES = {
    "one_token": [1],
    "one_block": [64],
    "block_plus_one": [65],
    "short": [5],
    "ragged": [3, 61, 1, 0, 130, 17],
    "group_edges": [31, 33, 16, 16, 200, 15],
    "tiny_prompts": [1] * 40 + [2] * 20 + [7],
    "two_long": [700, 513],
    "empty_ends": [0, 90, 0],
}


@pytest.mark.parametrize("weights", ["bf16x2", "fp16"])
@pytest.mark.parametrize("name", list(CASES))
def test_ragged_prompts(name, weights):
    lens = CASES[name]
    q, k, v, cu = inputs(list(CASES).index(name), lens)
    got = run(q, k, v, cu, 0.125, weights)
    ref = prefill_ref(q, k, v, cu, 0.125)
    if weights == "fp16":
        check_fp16_weights(got, ref, v_spread(v, cu), name)
    else:
        mx = check_close(got, ref, name)
        say(f"{name}: max abs {mx[0]:.2e}, row-rel {mx[1]:.2e}")


def test_full_length_prompt():
    q, k, v, cu = inputs(11, [2047])
    check_close(run(q, k, v, cu, 0.125), prefill_ref(q, k, v, cu, 0.125), "2047-row prompt")


@pytest.mark.parametrize("weights", ["bf16x2", "fp16"])
@pytest.mark.parametrize("scale,sigma_k", [(0.0, 1.0), (0.125, 3.0), (1.0, 1.0), (4.0, 1.0), (-0.5, 1.0)])
def test_scales(scale, sigma_k, weights):
    q, k, v, cu = inputs(12, [77, 200, 9], sigma_k=sigma_k)
    got, ref = run(q, k, v, cu, scale, weights), prefill_ref(q, k, v, cu, scale)
    if weights == "fp16":
        check_fp16_weights(got, ref, v_spread(v, cu), f"scale {scale} sigma_k {sigma_k}")
    else:
        check_close(got, ref, f"scale {scale} sigma_k {sigma_k}")


@pytest.mark.parametrize("weights", ["bf16x2", "fp16"])
def test_running_maximum_raised_every_tile(weights):
    """Scores that grow along each prompt by about 11 (base 2) per 32-key tile,
    more than the lazy maximum's slack of 8: every tile raises the running
    maximum and rescales what the rows have accumulated."""
    lens = [300, 97, 1, 64]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.float32)

    def bits(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    q = bits(np.full((T, 32, 64), 0.125))  # q . k = 0.24 pos, 0.35 pos in base-2 logits at scale 1
    k = bits(np.broadcast_to((0.03 * pos)[:, None, None], (T, 8, 64)))
    v = rand_bits(np.random.default_rng(15), (T, 8, 64))
    got, ref = run(q, k, v, cu, 1.0, weights), prefill_ref(q, k, v, cu, 1.0)
    if weights == "fp16":
        check_fp16_weights(got, ref, v_spread(v, cu), "raised every tile")
    else:
        check_close(got, ref, "raised every tile")


def test_scale_zero_gives_running_means():
    q, k, v, cu = inputs(13, [150])
    got = run(q, k, v, cu, 0.0)
    V = bf16_to_f64(v)
    means = np.cumsum(V, axis=0) / np.arange(1, 151)[:, None, None]
    check_close(got, np.repeat(means, 4, axis=1), "running means")


@pytest.mark.parametrize("weights", ["bf16x2", "fp16"])
def test_first_row_of_each_prompt_is_its_v_row(weights):
    lens = [1, 16, 17, 40, 3]
    q, k, v, cu = inputs(14, lens)
    got = run(q, k, v, cu, 0.125, weights)
    for b in range(len(lens)):
        r = cu[b]
        for h in range(32):
            # one weight: its bf16 pair is within 2^-16 of it, and the row sum is that weight
            assert np.allclose(got[r, h], bf16_to_f64(v[r, h // 4]), rtol=2.0 ** -15, atol=0)


def test_deterministic():
    q, k, v, cu = inputs(15, [300, 45])
    a = run(q, k, v, cu, 0.125)
    b = run(q, k, v, cu, 0.125)
    assert np.array_equal(a, b)


def test_neighbouring_prompt_values_do_not_reach_across_group_edges():
    # prompts that start on 16-row boundaries: non-finite K and V in one prompt
    # leave the other prompt's rows untouched
    q, k, v, cu = inputs(16, [32, 48, 16])
    k2, v2 = k.copy(), v.copy()
    k2[32:80] = 0x7FC0
    v2[32:80] = 0x7F80  # +inf
    got = run(q, k2, v2, cu, 0.125)
    ref = prefill_ref(q, k, v, cu, 0.125)
    check_close(got[:32], ref[:32], "before the poisoned prompt")
    check_close(got[80:], ref[80:], "after the poisoned prompt")


def test_largest_batch():
    lens = [0, 1, 2, 3] * 1024
    q, k, v, cu = inputs(17, lens)
    assert len(cu) - 1 == 4096
    check_close(run(q, k, v, cu, 0.125), prefill_ref(q, k, v, cu, 0.125), "4096 prompts")


def test_output_buffer_and_stream():
    q, k, v, cu = inputs(18, [100, 28])
    out = torch.full((128, 32, 64), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    qd, kd, vd, cd = dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(cu).cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ops.pa_prefill(qd, kd, vd, cd, 0.125, out=out, stream=s)
    s.synchronize()
    check_close(out.cpu().numpy(), prefill_ref(q, k, v, cu, 0.125), "given out, side stream")


@pytest.mark.parametrize("weights", ["bf16x2", "fp16"])
def test_full_workload_sampled(weights):
    # the 64 x 2047-row prompt batch of the prefill benchmark (one layer): one
    # whole prompt against the full oracle, and sampled rows of every prompt
    lay = synth.full()
    layer = 3
    k, v, cu = synth.prefill_inputs(lay, layer, "cuda")
    q = synth.prefill_queries(lay, layer, "cuda")
    T = q.shape[0]
    assert T == 64 * 2047
    say(f"full workload: T={T}")
    out = ops.pa_prefill(q, k, v, cu, lay.scale, weights=weights)
    torch.cuda.synchronize()
    cu_h = cu.cpu().numpy()
    qh, kh, vh = host_bits(q), host_bits(k), host_bits(v)
    got = out.cpu().numpy()
    b = 63
    sl = slice(int(cu_h[b]), int(cu_h[b + 1]))
    one = np.array([0, 2047], np.int32)
    ref = prefill_ref(qh[sl], kh[sl], vh[sl], one, lay.scale)
    if weights == "fp16":
        check_fp16_weights(got[sl], ref, v_spread(vh[sl], one), "last prompt, every row")
    else:
        check_close(got[sl], ref, "last prompt, every row")
    rng = np.random.default_rng(19)
    rows = np.concatenate([cu_h[:-1], cu_h[1:] - 1, rng.integers(0, T, 256)]).astype(np.int64)
    starts = cu_h[np.searchsorted(cu_h, rows, side="right") - 1]
    ref = prefill_rows_ref(qh[rows], kh, vh, starts, rows, lay.scale)
    if weights == "fp16":
        check_fp16_weights(got[rows], ref, v_spread(vh, cu_h, rows), "sampled rows")
    else:
        check_close(got[rows], ref, "sampled rows")
