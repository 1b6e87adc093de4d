"""The error bound the fp16-weight prefill mode is tested against, checked on
the CPU from its derivation.  The kernel's weights are 2^(x - m) with the
lazy running maximum m, so the largest weight of a row lies in [1, 2^8].
Each weight rounded to fp16 (relative error u = 2^-11 in the normal range,
absolute 2^-25 below it), with the average taken over the sum of the same
rounded weights, moves an output by at most 2^-10 times the spread of the V
values averaged.  Normalised weights sum to one before and after rounding, so
the error is sum_j (w~_j - w_j)(v_j - c) for any c; with c at mid-spread it is
at most sum_j |w~_j - w_j| * spread / 2, and sum_j |w~_j - w_j| <= 2u/(1 - u)
plus n 2^-25 / (sum of weights >= 1), below 2^-9 for n <= 2^11."""
import numpy as np
import pytest


def rounded_average(w: np.ndarray, v: np.ndarray) -> np.ndarray:
    wr = w.astype(np.float16).astype(np.float64)
    return (wr[:, None] * v).sum(axis=0) / wr.sum()


@pytest.mark.parametrize("seed", range(40))
def test_bound_holds(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 2049))
    s = rng.normal(size=n) * rng.choice([0.1, 1.0, 4.0, 20.0])
    # weights relative to a stale maximum: the largest is anywhere in [1, 2^8]
    w = np.exp2(s - s.max() + rng.uniform(0, 8))
    v = rng.normal(size=(n, 64)) * rng.choice([0.01, 1.0, 30.0])
    exact = (w[:, None] * v).sum(axis=0) / w.sum()
    got = rounded_average(w, v)
    spread = v.max(axis=0) - v.min(axis=0)
    assert (np.abs(got - exact) <= 2.0 ** -10 * spread + 1e-12).all()


def test_two_key_case_is_near_the_bound():
    # two near-equal weights that round in opposite directions, V values far
    # apart: the error reaches a fair part of the bound (it is not loose by orders)
    w = np.array([1 + 2.0 ** -11 * 0.999, 1 - 2.0 ** -12 * 0.999])
    v = np.array([[4.0], [-4.0]])
    exact = (w[:, None] * v).sum(axis=0) / w.sum()
    err = abs(rounded_average(w, v) - exact)[0]
    assert 0.1 * 2.0 ** -10 * 8 < err <= 2.0 ** -10 * 8
