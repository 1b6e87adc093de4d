"""Pins of the oracle's causal prefill attention (prefill_ref) against facts
that do not come from it: the first position returning its own V row, scale 0
giving running means of V (a cumulative sum), causality, each row equalling the
separately pinned paged decode over the prefix, scipy softmax on an explicitly
masked score matrix, the hardmax limit, GQA isolation, and planted slips in a
copy of it that each fail a pin."""
import numpy as np
import pytest
import scipy.special

from oracle import bf16_to_f64, decode_ref, prefill_ref, prefill_rows_ref
from tests.test_oracle import PT, rand_bits, to_bits


def case(seed, lens, Hq=8, Hkv=2, D=16, sigma_k=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return rand_bits(rng, (T, Hq, D)), rand_bits(rng, (T, Hkv, D), sigma_k), rand_bits(rng, (T, Hkv, D)), cu


def test_first_position_returns_its_v_row():
    q, k, v, cu = case(0, [5, 1, 9])
    out = prefill_ref(q, k, v, cu, 0.25)
    for b in range(3):
        r = cu[b]
        for h in range(8):
            assert np.array_equal(out[r, h], bf16_to_f64(v[r, h // 4]))


def test_scale_zero_gives_running_means():
    q, k, v, cu = case(1, [13, 40])
    out = prefill_ref(q, k, v, cu, 0.0)
    for b in range(2):
        V = bf16_to_f64(v[cu[b]:cu[b + 1]])
        means = np.cumsum(V, axis=0) / np.arange(1, len(V) + 1)[:, None, None]
        for h in range(8):
            assert np.allclose(out[cu[b]:cu[b + 1], h], means[:, h // 4], rtol=1e-13, atol=1e-14)


def test_causality():
    q, k, v, cu = case(2, [30])
    base = prefill_ref(q, k, v, cu, 0.3)
    for i in (0, 7, 29):
        k2, v2 = k.copy(), v.copy()
        rng = np.random.default_rng(i)
        k2[i + 1:] = rand_bits(rng, k2[i + 1:].shape)
        v2[i + 1:] = rand_bits(rng, v2[i + 1:].shape)
        got = prefill_ref(q, k2, v2, cu, 0.3)
        assert np.array_equal(got[:i + 1], base[:i + 1])


def test_rows_equal_paged_decode_over_the_prefix():
    q, k, v, cu = case(3, [37])
    out = prefill_ref(q, k, v, cu, 0.125)
    n = 37
    kp = np.full(((n + PT - 1) // PT, PT, 2, 16), 0x7FC0, np.uint16)
    vp = kp.copy()
    for t in range(n):
        kp[t // PT, t % PT] = k[t]
        vp[t // PT, t % PT] = v[t]
    bt = np.arange(kp.shape[0], dtype=np.int32)[None]
    for i in (0, 15, 16, 36):
        ref = decode_ref(q[i:i + 1], kp, vp, bt, np.array([i + 1], np.int32), 0.125)[0]
        assert np.allclose(out[i], ref, rtol=1e-12, atol=1e-13)


def test_scipy_softmax_on_a_masked_matrix():
    q, k, v, cu = case(4, [3, 50, 17], sigma_k=3.0)
    out = prefill_ref(q, k, v, cu, 0.2)
    for b in range(3):
        Q, K, V = (bf16_to_f64(x[cu[b]:cu[b + 1]]) for x in (q, k, v))
        n = len(Q)
        mask = np.tril(np.ones((n, n)))
        for h in range(8):
            s = 0.2 * np.einsum("id,jd->ij", Q[:, h], K[:, h // 4])
            p = scipy.special.softmax(np.where(mask > 0, s, -np.inf), axis=1)
            assert np.allclose(out[cu[b]:cu[b + 1], h], p @ V[:, h // 4], rtol=1e-12, atol=1e-13)


def test_hardmax_picks_the_largest_visible_score():
    n = 20
    q = np.zeros((n, 4, 8), np.uint16)
    q[:] = to_bits([1, 0, 0, 0, 0, 0, 0, 0])
    k = np.zeros((n, 1, 8), np.uint16)
    keys = [1.0 + (j % 7) / 8 if j != 12 else 4.0 for j in range(n)]
    for j in range(n):
        k[j, 0] = to_bits([keys[j], 0, 0, 0, 0, 0, 0, 0])
    v = rand_bits(np.random.default_rng(5), (n, 1, 8))
    out = prefill_ref(q, k, v, np.array([0, n], np.int32), 1000.0)
    for i in range(n):
        j = int(np.argmax(keys[:i + 1]))
        assert np.array_equal(out[i, 0], bf16_to_f64(v[j, 0]))


def test_gqa_isolation():
    q, k, v, cu = case(6, [25])
    base = prefill_ref(q, k, v, cu, 0.125)
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] = 0x7FC0
    v2[:, 1] = 0x7FC0
    got = prefill_ref(q, k2, v2, cu, 0.125)
    assert np.array_equal(got[:, :4], base[:, :4]) and np.isnan(got[:, 4:]).all()


def test_rows_ref_equals_prefill_ref_row_by_row():
    # prefill_rows_ref (one row at a time, for sampled rows of large inputs) gives
    # the rows of the pinned prefill_ref, prompt boundaries included
    q, k, v, cu = case(7, [1, 16, 0, 33, 9], sigma_k=2.0)
    full = prefill_ref(q, k, v, cu, 0.3)
    T = int(cu[-1])
    rows = np.arange(T)
    starts = cu[np.searchsorted(cu, rows, side="right") - 1]
    got = prefill_rows_ref(q, k, v, starts, rows, 0.3)
    assert np.allclose(got, full, rtol=1e-13, atol=1e-14)
    pick = np.array([0, 1, 16, 17, 50, T - 1])
    assert np.array_equal(prefill_rows_ref(q[pick], k, v, starts[pick], pick, 0.3), got[pick])


# ---------------------------------------------------------------- planted slips


def make_prefill(mistake):
    def prefill(q, k, v, cu, scale):
        T, Hq, D = q.shape
        G = Hq // k.shape[1]
        out = np.zeros((T, Hq, D))
        for b in range(len(cu) - 1):
            r0, r1 = int(cu[b]), int(cu[b + 1])
            n = r1 - r0
            Q, K, V = bf16_to_f64(q[r0:r1]), bf16_to_f64(k[r0:r1]), bf16_to_f64(v[r0:r1])
            if mistake == "no_mask":
                later = np.zeros((n, n), dtype=bool)
            elif mistake == "strict_mask":  # i does not attend itself
                later = np.triu(np.ones((n, n), dtype=bool), 0)
                later[0, 0] = False
            else:
                later = np.triu(np.ones((n, n), dtype=bool), 1)
            for h in range(Hq):
                g = h % k.shape[1] if mistake == "gqa_modulo" else h // G
                s = (1.0 if mistake == "no_scale" else scale) * (Q[:, h] @ K[:, g].T)
                s[later] = -np.inf
                w = np.exp(s - s.max(axis=1, keepdims=True))
                out[r0:r1, h] = (w @ (K if mistake == "k_as_v" else V)[:, g]) / w.sum(axis=1, keepdims=True)
        return out

    return prefill


MUTANTS = ["no_mask", "strict_mask", "gqa_modulo", "no_scale", "k_as_v"]


def pins_hold(fn) -> bool:
    q, k, v, cu = case(0, [5, 1, 9])
    out = fn(q, k, v, cu, 0.25)
    ok = all(np.array_equal(out[cu[b], h], bf16_to_f64(v[cu[b], h // 4])) for b in range(3) for h in range(8))
    q, k, v, cu = case(4, [3, 50, 17], sigma_k=3.0)
    out = fn(q, k, v, cu, 0.2)
    for b in range(3):
        Q, K, V = (bf16_to_f64(x[cu[b]:cu[b + 1]]) for x in (q, k, v))
        n = len(Q)
        mask = np.tril(np.ones((n, n)))
        for h in range(8):
            s = 0.2 * np.einsum("id,jd->ij", Q[:, h], K[:, h // 4])
            p = scipy.special.softmax(np.where(mask > 0, s, -np.inf), axis=1)
            ok &= bool(np.allclose(out[cu[b]:cu[b + 1], h], p @ V[:, h // 4], rtol=1e-12, atol=1e-13))
    return ok


def test_real_and_unmutated_pass():
    assert pins_hold(prefill_ref) and pins_hold(make_prefill("none"))


@pytest.mark.parametrize("mistake", MUTANTS)
def test_prefill_mutant_is_caught(mistake):
    with np.errstate(all="ignore"):
        assert not pins_hold(make_prefill(mistake)), f"no pin catches {mistake!r}"
