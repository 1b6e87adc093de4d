"""Pins of the FP64 oracle against facts that do not come from the oracle itself.

The pages print no worked example or values, so every pin is a closed form, an
invariant of softmax attention, a library routine on a gathered (contiguous)
copy, or brute force on a tiny case.  Each is chosen so that a plausible slip in
the oracle (a dropped scale, a wrong sign, a wrong head or page index, an
off-by-one in the length, a transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import append_ref, bf16_to_f64, decode_ref, merge_ref, partial_ref
from paged_kv_cache_205_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PT = 16


def to_bits(x) -> np.ndarray:
    """FP64 values that are exact in BF16 -> uint16 bit patterns (asserts exactness)."""
    x = np.asarray(x, dtype=np.float64)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.to(torch.float64).numpy(), x, equal_nan=True), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_bits(rng, shape, sigma=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * np.float32(sigma))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_case(seed, B=3, Hq=8, Hkv=2, D=16, max_blocks=6, lens=None, sigma_k=1.0, poison=True):
    """A small random paged state: shuffled pages, NaN in every unreferenced slot."""
    rng = np.random.default_rng(seed)
    lens = np.array(lens if lens is not None else rng.integers(1, max_blocks * PT + 1, size=B), np.int32)
    B = len(lens)
    need = sum((int(L) + PT - 1) // PT for L in lens)
    num_pages = need + 3
    free = rng.permutation(num_pages)
    bt = np.full((B, max_blocks), -1, np.int32)
    k = 0
    for b, L in enumerate(lens):
        n = (int(L) + PT - 1) // PT
        bt[b, :n] = free[k:k + n]
        k += n
    kp = np.full((num_pages, PT, Hkv, D), 0x7FC0 if poison else 0, np.uint16)
    vp = kp.copy()
    for b, L in enumerate(lens):
        for t in range(int(L)):
            kp[bt[b, t // PT], t % PT] = rand_bits(rng, (Hkv, D), sigma_k)
            vp[bt[b, t // PT], t % PT] = rand_bits(rng, (Hkv, D))
    q = rand_bits(rng, (B, Hq, D))
    return q, kp, vp, bt, lens


# ---------------------------------------------------------------- conversion


def test_bf16_conversion_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4049, 0x3E00], np.uint16)
    got = bf16_to_f64(pats)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 3.140625, 0.125]
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[3])
    assert np.isnan(bf16_to_f64(np.array([0x7FC0], np.uint16)))[0]


def test_bf16_conversion_matches_torch():
    u = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_to_f64(u), t, equal_nan=True)


# ---------------------------------------------------------------- append (P1)


def test_append_tiny_hand_position():
    lay = synth.tiny()
    bt = lay.block_tables[0]
    rng = np.random.default_rng(0)
    kp = rng.integers(0, 1 << 16, size=(8, PT, 8, 64)).astype(np.uint16)
    vp = rng.integers(0, 1 << 16, size=(8, PT, 8, 64)).astype(np.uint16)
    kn = rng.integers(0, 1 << 16, size=(1, 8, 64)).astype(np.uint16)
    vn = rng.integers(0, 1 << 16, size=(1, 8, 64)).astype(np.uint16)
    k2, v2 = append_ref(kp, vp, kn, vn, bt, np.array([38], np.int32))
    # position 37 = block 2, slot 5, worked by hand
    page = int(bt[0, 2])
    assert np.array_equal(k2[page, 5], kn[0]) and np.array_equal(v2[page, 5], vn[0])
    dk = (k2 != kp).any(axis=(2, 3))
    dv = (v2 != vp).any(axis=(2, 3))
    assert set(zip(*np.nonzero(dk))) <= {(page, 5)} and set(zip(*np.nonzero(dv))) <= {(page, 5)}
    assert kp is not k2 and np.array_equal(kp[page, 4], k2[page, 4])


@pytest.mark.parametrize("L,slot,blk", [(1, 0, 0), (16, 15, 0), (17, 0, 1), (32, 15, 1), (2048, 15, 127)])
def test_append_boundaries(L, slot, blk):
    bt = np.arange(128, dtype=np.int32)[None, ::-1].copy()
    kp = np.zeros((128, PT, 1, 2), np.uint16)
    vp = np.zeros_like(kp)
    kn = np.full((1, 1, 2), 0x1234, np.uint16)
    vn = np.full((1, 1, 2), 0x4321, np.uint16)
    k2, v2 = append_ref(kp, vp, kn, vn, bt, np.array([L], np.int32))
    assert np.argwhere(k2 != 0).tolist() == [[127 - blk, slot, 0, 0], [127 - blk, slot, 0, 1]]
    assert np.argwhere(v2 != 0).tolist() == [[127 - blk, slot, 0, 0], [127 - blk, slot, 0, 1]]


def test_append_skips_empty_and_changes_exactly_2B_rows():
    q, kp, vp, bt, lens = random_case(3, B=5, lens=[0, 5, 16, 33, 96])
    rng = np.random.default_rng(1)
    kn = rng.integers(0, 0x7F00, size=(5, 2, 16)).astype(np.uint16)
    vn = rng.integers(0, 0x7F00, size=(5, 2, 16)).astype(np.uint16)
    k2, v2 = append_ref(kp, vp, kn, vn, bt, lens)
    changed = (k2 != kp).any(axis=(2, 3))
    assert changed.sum() == 4  # 4 non-empty sequences, sequence 0 skipped
    for b, L in enumerate(lens):
        if L:
            p, s = bt[b, (L - 1) // PT], (L - 1) % PT
            assert np.array_equal(k2[p, s], kn[b]) and np.array_equal(v2[p, s], vn[b])


def test_append_rejects_shared_slot():
    bt = np.array([[0], [0]], np.int32)
    kp = np.zeros((1, PT, 1, 1), np.uint16)
    kn = np.ones((2, 1, 1), np.uint16)
    with pytest.raises(AssertionError):
        append_ref(kp, kp, kn, kn, bt, np.array([3, 3], np.int32))


# ---------------------------------------------------------------- decode


def gather_softmax(q, kp, vp, bt, lens, scale):
    """Independent route: gather to contiguous [L][Hkv][D] by flat row index, then
    scipy's softmax and a matmul per head (query head h -> kv head h // G)."""
    B, Hq, D = q.shape
    Hkv = kp.shape[2]
    G = Hq // Hkv
    kflat = bf16_to_f64(kp).reshape(-1, Hkv, D)
    vflat = bf16_to_f64(vp).reshape(-1, Hkv, D)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        rows = bt[b, pos // PT].astype(np.int64) * PT + pos % PT
        Kc, Vc = kflat[rows], vflat[rows]  # [L][Hkv][D]
        Q = bf16_to_f64(q[b])  # [Hq][D]
        for g in range(Hkv):
            S = scale * (Q[g * G:(g + 1) * G] @ Kc[:, g, :].T)  # [G][L]
            out[b, g * G:(g + 1) * G] = scipy.special.softmax(S, axis=1) @ Vc[:, g, :]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_decode_matches_gathered_scipy_softmax(seed):
    q, kp, vp, bt, lens = random_case(seed, lens=[1, 15, 16, 17, 40, 96] if seed == 0 else None,
                                      sigma_k=3.0 if seed % 2 else 1.0)
    got = decode_ref(q, kp, vp, bt, lens, 0.25)
    want = gather_softmax(q, kp, vp, bt, lens, 0.25)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_two_token_golden():
    with open(os.path.join(GOLDEN, "two_token.json")) as f:
        gd = json.load(f)
    Hq, Hkv, D = gd["Hq"], gd["Hkv"], gd["D"]
    q = np.stack([to_bits(gd["q_row"])] * Hq)[None]
    kp = np.full((2, PT, Hkv, D), 0x7FC0, np.uint16)
    vp = kp.copy()
    # tokens live on page 1 (block table [1, 0]); page 0 stays poisoned and unreferenced
    kp[1, 0, 0], kp[1, 1, 0] = to_bits(gd["K"][0]), to_bits(gd["K"][1])
    vp[1, 0, 0], vp[1, 1, 0] = to_bits(gd["V"][0]), to_bits(gd["V"][1])
    out = decode_ref(q, kp, vp, np.array([[1, 0]], np.int32), np.array([2], np.int32), gd["scale"])
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], gd["expected"], rtol=1e-15, atol=1e-15)


def test_length_one_returns_v_row_exactly():
    q, kp, vp, bt, lens = random_case(11, lens=[1, 1, 1])
    out = decode_ref(q, kp, vp, bt, lens, 0.125)
    for b in range(3):
        for h in range(8):
            assert np.array_equal(out[b, h], bf16_to_f64(vp[bt[b, 0], 0, h // 4]))


def test_empty_sequence_gives_zeros():
    q, kp, vp, bt, lens = random_case(12, lens=[0, 20])
    out = decode_ref(q, kp, vp, bt, lens, 0.125)
    assert (out[0] == 0).all() and np.isfinite(out[1]).all() and (out[1] != 0).any()


def test_constant_keys_give_mean_of_v():
    q, kp, vp, bt, lens = random_case(13, lens=[37, 64])
    for b, L in enumerate(lens):
        for t in range(L):
            kp[bt[b, t // PT], t % PT] = kp[bt[b, 0], 0]
    out = decode_ref(q, kp, vp, bt, lens, 0.125)
    for b, L in enumerate(lens):
        V = np.stack([bf16_to_f64(vp[bt[b, t // PT], t % PT]) for t in range(L)])
        for h in range(8):
            np.testing.assert_allclose(out[b, h], V[:, h // 4].mean(axis=0), rtol=1e-14, atol=1e-15)


def test_scale_zero_gives_mean_of_v():
    q, kp, vp, bt, lens = random_case(14, lens=[50])
    out = decode_ref(q, kp, vp, bt, lens, 0.0)
    V = np.stack([bf16_to_f64(vp[bt[0, t // PT], t % PT]) for t in range(50)])
    for h in range(8):
        np.testing.assert_allclose(out[0, h], V[:, h // 4].mean(axis=0), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("target", [0, 15, 16, 33, 49])
def test_large_scale_picks_the_argmax_token(target):
    """Hardmax limit: the token with the largest q.k wins (a sign error would pick the smallest)."""
    L = 50
    q, kp, vp, bt, lens = random_case(15, B=1, Hq=4, Hkv=1, D=8, lens=[L])
    q[0, :] = to_bits([1, 0, 0, 0, 0, 0, 0, 0])
    for t in range(L):
        val = 4.0 if t == target else (-8.0 if t == (target + 1) % L else 1.0 - t / 64)
        kp[bt[0, t // PT], t % PT, 0] = to_bits([val, 0, 0, 0, 0, 0, 0, 0])
    out = decode_ref(q, kp, vp, bt, lens, 1000.0)
    want = bf16_to_f64(vp[bt[0, target // PT], target % PT, 0])
    for h in range(4):
        assert np.array_equal(out[0, h], want)


def test_last_appended_position_is_attended():
    """seq_lens counts the new token: with it as the hardmax winner the output is its V row."""
    for L in (16, 17, 38):
        q, kp, vp, bt, lens = random_case(16, B=1, Hq=4, Hkv=1, D=8, lens=[L])
        q[0, :] = to_bits([1, 0, 0, 0, 0, 0, 0, 0])
        for t in range(L):
            kp[bt[0, t // PT], t % PT, 0] = to_bits([2.0 if t == L - 1 else 0.0] + [0] * 7)
        out = decode_ref(q, kp, vp, bt, lens, 1000.0)
        assert np.array_equal(out[0, 0], bf16_to_f64(vp[bt[0, (L - 1) // PT], (L - 1) % PT, 0]))


def test_page_permutation_invariance():
    q, kp, vp, bt, lens = random_case(17, B=4, max_blocks=8)
    base = decode_ref(q, kp, vp, bt, lens, 0.125)
    perm = np.random.default_rng(5).permutation(kp.shape[0])
    kq = np.empty_like(kp)
    vq = np.empty_like(vp)
    kq[perm] = kp
    vq[perm] = vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    assert np.array_equal(decode_ref(q, kq, vq, bt2, lens, 0.125), base)


def test_gqa_isolation_and_shared_group():
    q, kp, vp, bt, lens = random_case(18, B=2, Hq=8, Hkv=2, D=16, lens=[30, 45])
    base = decode_ref(q, kp, vp, bt, lens, 0.125)
    for g in range(2):
        kq, vq = kp.copy(), vp.copy()
        other = [x for x in range(2) if x != g]
        kq[:, :, other] = 0x7FC0
        vq[:, :, other] = 0x7FC0
        got = decode_ref(q, kq, vq, bt, lens, 0.125)
        heads = slice(4 * g, 4 * g + 4)
        assert np.isfinite(got[:, heads]).all()
        assert np.array_equal(got[:, heads], base[:, heads])
        assert np.isnan(got[:, [h for h in range(8) if h // 4 != g]]).all()
    q2 = q.copy()
    q2[:, 4:8] = q2[:, 4:5]
    out = decode_ref(q2, kp, vp, bt, lens, 0.125)
    for h in range(5, 8):
        assert np.array_equal(out[:, h], out[:, 4])


def test_token_order_invariance():
    """No positional bias inside decode: shuffling the token order (K and V together) is a no-op."""
    q, kp, vp, bt, lens = random_case(19, B=1, lens=[70])
    L = 70
    perm = np.random.default_rng(2).permutation(L)
    kq, vq = kp.copy(), vp.copy()
    for t in range(L):
        s = perm[t]
        kq[bt[0, t // PT], t % PT] = kp[bt[0, s // PT], s % PT]
        vq[bt[0, t // PT], t % PT] = vp[bt[0, s // PT], s % PT]
    np.testing.assert_allclose(decode_ref(q, kq, vq, bt, lens, 0.125),
                               decode_ref(q, kp, vp, bt, lens, 0.125), rtol=1e-13, atol=1e-14)


def test_linearity_in_v():
    q, kp, vp, bt, lens = random_case(20, B=2, lens=[33, 9])
    rng = np.random.default_rng(3)
    ref_pages = np.unique(bt[bt >= 0])
    V = rng.integers(-8, 9, size=vp.shape).astype(np.float64)
    c = rng.integers(-4, 5, size=vp.shape[-1]).astype(np.float64)
    v1 = vp.copy()
    v2 = vp.copy()
    v1[ref_pages] = to_bits(V[ref_pages])
    v2[ref_pages] = to_bits(2 * V[ref_pages] + c)
    o1 = decode_ref(q, kp, v1, bt, lens, 0.125)
    o2 = decode_ref(q, kp, v2, bt, lens, 0.125)
    np.testing.assert_allclose(o2, 2 * o1 + c, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny_config():
    """The tiny workload (37 then 38 tokens, 32 heads) by a scalar triple loop with math.fsum."""
    lay = synth.tiny()
    kp_t, vp_t = synth.make_pools(lay, "cpu")
    inp = synth.step_inputs(lay, 0, "cpu")
    kp, vp = synth.bits(kp_t), synth.bits(vp_t)
    q = synth.bits(inp["q"])
    bt = lay.block_tables[0]
    k2, v2 = append_ref(kp, vp, synth.bits(inp["k_new"]), synth.bits(inp["v_new"]), bt, lay.seq_lens)
    for L, (K, V) in ((37, (kp, vp)), (38, (k2, v2))):
        out = decode_ref(q, K, V, bt, np.array([L], np.int32), lay.scale)
        assert np.isfinite(out).all()
        for h in range(32):
            g = h // 4
            qh = [float(x) for x in bf16_to_f64(q[0, h])]
            s = []
            for t in range(L):
                kr = bf16_to_f64(K[bt[0, t // 16], t % 16, g])
                s.append(lay.scale * math.fsum(qh[d] * float(kr[d]) for d in range(64)))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = math.fsum(w)
            for d in range(0, 64, 7):
                num = math.fsum(w[t] * float(bf16_to_f64(V[bt[0, t // 16], t % 16, g, d])) for t in range(L))
                assert abs(out[0, h, d] - num / den) <= 1e-14 * max(1.0, abs(num / den))


# ---------------------------------------------------------------- split / merge (P7)


def test_merge_closed_form():
    o1, o2 = np.array([1.0, 0.0]), np.array([0.0, 2.0])
    # equal maxima: weights proportional to l
    np.testing.assert_allclose(merge_ref([0.5, 0.5], [3.0, 1.0], [o1, o2]), [0.75, 0.5], rtol=1e-15)
    # m differs by ln 2: weight ratio 2 * (l1 / l2)
    np.testing.assert_allclose(merge_ref([math.log(2.0), 0.0], [1.0, 1.0], [o1, o2]), [2 / 3, 2 / 3], rtol=1e-15)
    # empty states are skipped, all-empty gives zeros
    np.testing.assert_allclose(merge_ref([-math.inf, 0.0], [0.0, 1.0], [o1 * np.nan, o2]), o2)
    assert (merge_ref([-math.inf], [0.0], [o1]) == 0).all()


@pytest.mark.parametrize("part", [16, 32, 48, 64, 256, 7])
def test_split_merge_equals_full(part):
    q, kp, vp, bt, lens = random_case(21, B=3, lens=[1, 77, 96], sigma_k=3.0)
    full = decode_ref(q, kp, vp, bt, lens, 0.125)
    for b, L in enumerate(lens):
        for h in range(8):
            states = [partial_ref(q, kp, vp, bt, lens, 0.125, b, h, t0, min(L, t0 + part))
                      for t0 in range(0, L, part)]
            states.append(partial_ref(q, kp, vp, bt, lens, 0.125, b, h, L, L))  # an empty split
            ms, ls, os_ = zip(*states)
            np.testing.assert_allclose(merge_ref(ms, ls, os_), full[b, h], rtol=1e-13, atol=1e-14)


def test_partial_of_whole_range_is_decode():
    q, kp, vp, bt, lens = random_case(22, B=2, lens=[40, 3])
    full = decode_ref(q, kp, vp, bt, lens, 0.125)
    m, l, o = partial_ref(q, kp, vp, bt, lens, 0.125, 0, 5, 0, 40)
    np.testing.assert_allclose(o, full[0, 5], rtol=1e-14)
    assert l >= 1.0  # the maximum term contributes exp(0) = 1


def test_poison_never_leaks():
    q, kp, vp, bt, lens = random_case(23, B=4, lens=[1, 16, 17, 95])
    assert np.isnan(bf16_to_f64(kp)).any()
    assert np.isfinite(decode_ref(q, kp, vp, bt, lens, 0.125)).all()
