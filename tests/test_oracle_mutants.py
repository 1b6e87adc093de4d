"""The oracle's pins catch plausible slips.

Each mutant below is a copy of the oracle's decode with one planted mistake (run
on the CPU only).  The pin suite used here (gathered scipy softmax, the
hand-worked two-token case, length one, constant keys, hardmax argmax, the
appended position attended, page permutation, GQA isolation, linearity in V)
must reject every mutant and accept the real oracle.
"""
import json
import os

import numpy as np
import pytest

from oracle import bf16_to_f64, decode_ref
from tests.test_oracle import GOLDEN, PT, gather_softmax, random_case, to_bits


def make_decode(mistake: str):
    """A decode with one planted mistake (same page walk as the oracle otherwise)."""

    def decode(q, kp, vp, bt, lens, scale):
        B, Hq, D = q.shape
        Hkv = kp.shape[2]
        G = Hq // Hkv
        out = np.zeros((B, Hq, D))
        for b in range(B):
            L = int(lens[b])
            if mistake == "off_by_one_short":
                L -= 1
            if mistake == "off_by_one_long":
                L += 1
            if L <= 0:
                continue
            for h in range(Hq):
                g = h % Hkv if mistake == "gqa_modulo" else h // G
                qh = bf16_to_f64(q[b, h])
                s, V = [], []
                for j in range((L + PT - 1) // PT):
                    page = j if mistake == "no_block_table" else int(bt[b, j])
                    n = min(PT, L - PT * j)
                    lo = 1 if (mistake == "slot_shift" and j == (L - 1) // PT and n < PT) else 0
                    K = bf16_to_f64(kp[page, lo:lo + n, g])
                    Vr = bf16_to_f64(vp[page, lo:lo + n, g])
                    sc = K @ qh
                    if mistake == "no_scale":
                        pass
                    elif mistake == "sign":
                        sc = -scale * sc
                    else:
                        sc = scale * sc
                    s.append(sc)
                    V.append(K if mistake == "k_as_v" else Vr)
                s = np.concatenate(s)
                V = np.concatenate(V)
                with np.errstate(over="ignore", invalid="ignore"):
                    w = np.exp(s) if mistake == "no_max" else np.exp(s - s.max())
                    out[b, h] = (w @ V) if mistake == "no_normalise" else (w @ V) / w.sum()
        return out

    return decode


MUTANTS = ["no_scale", "sign", "gqa_modulo", "off_by_one_short", "off_by_one_long", "no_block_table",
           "slot_shift", "k_as_v", "no_max", "no_normalise"]


# ---- the pins, each taking a decode function; True means the pin holds


def pin_gather(decode):
    q, kp, vp, bt, lens = random_case(0, lens=[1, 15, 16, 17, 40, 96])
    got = decode(q, kp, vp, bt, lens, 0.25)
    return bool(np.isfinite(got).all() and np.allclose(got, gather_softmax(q, kp, vp, bt, lens, 0.25),
                                                       rtol=1e-12, atol=1e-13))


def pin_two_token(decode):
    with open(os.path.join(GOLDEN, "two_token.json")) as f:
        gd = json.load(f)
    q = np.stack([to_bits(gd["q_row"])] * gd["Hq"])[None]
    kp = np.full((2, PT, gd["Hkv"], gd["D"]), 0x7FC0, np.uint16)
    vp = kp.copy()
    kp[1, 0, 0], kp[1, 1, 0] = to_bits(gd["K"][0]), to_bits(gd["K"][1])
    vp[1, 0, 0], vp[1, 1, 0] = to_bits(gd["V"][0]), to_bits(gd["V"][1])
    out = decode(q, kp, vp, np.array([[1, 0]], np.int32), np.array([2], np.int32), gd["scale"])
    return bool(np.allclose(out[0], np.array(gd["expected"])[None], rtol=1e-14, atol=1e-14))


def pin_length_one(decode):
    q, kp, vp, bt, lens = random_case(11, lens=[1, 1, 1])
    out = decode(q, kp, vp, bt, lens, 0.125)
    return all(np.array_equal(out[b, h], bf16_to_f64(vp[bt[b, 0], 0, h // 4])) for b in range(3) for h in range(8))


def pin_hardmax(decode):
    L = 50
    ok = True
    for target in (0, 17, 49):
        q, kp, vp, bt, lens = random_case(15, B=1, Hq=4, Hkv=1, D=8, lens=[L])
        q[0, :] = to_bits([1, 0, 0, 0, 0, 0, 0, 0])
        for t in range(L):
            val = 4.0 if t == target else (-8.0 if t == (target + 1) % L else 1.0 - t / 64)
            kp[bt[0, t // PT], t % PT, 0] = to_bits([val, 0, 0, 0, 0, 0, 0, 0])
        with np.errstate(all="ignore"):
            out = decode(q, kp, vp, bt, lens, 1000.0)
        ok &= bool(np.array_equal(out[0, 0], bf16_to_f64(vp[bt[0, target // PT], target % PT, 0])))
    return ok


def pin_last_attended(decode):
    ok = True
    for L in (16, 17, 38):
        q, kp, vp, bt, lens = random_case(16, B=1, Hq=4, Hkv=1, D=8, lens=[L])
        q[0, :] = to_bits([1, 0, 0, 0, 0, 0, 0, 0])
        for t in range(L):
            kp[bt[0, t // PT], t % PT, 0] = to_bits([2.0 if t == L - 1 else 0.0] + [0] * 7)
        with np.errstate(all="ignore"):
            out = decode(q, kp, vp, bt, lens, 1000.0)
        ok &= bool(np.array_equal(out[0, 0], bf16_to_f64(vp[bt[0, (L - 1) // PT], (L - 1) % PT, 0])))
    return ok


def pin_page_permutation(decode):
    q, kp, vp, bt, lens = random_case(17, B=4, max_blocks=8)
    base = decode(q, kp, vp, bt, lens, 0.125)
    perm = np.random.default_rng(5).permutation(kp.shape[0])
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    got = decode(q, kq, vq, bt2, lens, 0.125)
    return bool(np.isfinite(base).all() and np.array_equal(got, base))


def pin_gqa_isolation(decode):
    q, kp, vp, bt, lens = random_case(18, B=2, Hq=8, Hkv=2, D=16, lens=[30, 45])
    base = decode(q, kp, vp, bt, lens, 0.125)
    kq, vq = kp.copy(), vp.copy()
    kq[:, :, 1] = 0x7FC0
    vq[:, :, 1] = 0x7FC0
    got = decode(q, kq, vq, bt, lens, 0.125)
    return bool(np.isfinite(got[:, 0:4]).all() and np.array_equal(got[:, 0:4], base[:, 0:4]))


def pin_linearity(decode):
    q, kp, vp, bt, lens = random_case(20, B=2, lens=[33, 9])
    rng = np.random.default_rng(3)
    ref_pages = np.unique(bt[bt >= 0])
    V = rng.integers(-8, 9, size=vp.shape).astype(np.float64)
    c = rng.integers(-4, 5, size=vp.shape[-1]).astype(np.float64)
    v1, v2 = vp.copy(), vp.copy()
    v1[ref_pages] = to_bits(V[ref_pages])
    v2[ref_pages] = to_bits(2 * V[ref_pages] + c)
    o1 = decode(q, kp, v1, bt, lens, 0.125)
    o2 = decode(q, kp, v2, bt, lens, 0.125)
    return bool(np.isfinite(o1).all() and np.allclose(o2, 2 * o1 + c, rtol=1e-12, atol=1e-12))


PINS = [pin_gather, pin_two_token, pin_length_one, pin_hardmax, pin_last_attended, pin_page_permutation,
        pin_gqa_isolation, pin_linearity]


def test_real_oracle_passes_every_pin():
    for pin in PINS:
        assert pin(decode_ref), pin.__name__


def test_unmutated_copy_passes_every_pin():
    dec = make_decode("none")
    for pin in PINS:
        assert pin(dec), pin.__name__


def holds(pin, decode) -> bool:
    """A pin holds if it runs and its check passes (an exception is a failed pin)."""
    try:
        return pin(decode)
    except (IndexError, ValueError, FloatingPointError):
        return False


@pytest.mark.parametrize("mistake", MUTANTS)
def test_mutant_is_caught(mistake):
    dec = make_decode(mistake)
    failed = [pin.__name__ for pin in PINS if not holds(pin, dec)]
    assert failed, f"no pin catches the mutant {mistake!r}"
