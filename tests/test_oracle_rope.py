"""Pins of the RoPE + append oracle (oracle/rope.py) against facts that do not
come from it: a hand-worked row with two rounding ties, brute-force BF16
rounding, the identity table, the FP64 rotation within the BF16 rounding,
preserved pair norms, the inverse rotation, and the append's placement.  Each
is chosen so that a plausible slip (a wrong sign, interleaved instead of
half-split pairs, cos and sin swapped, rounding by truncation, the wrong
position) fails at least one of them; planted versions of those slips are
checked below to fail."""
import json
import os

import numpy as np
import pytest

from oracle import append_ref
from oracle.rope import (bf16_bits_to_f32, f32_to_bf16_rne, rope_append_ref, rope_f64, rope_rows_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    with open(os.path.join(GOLDEN, "rope_pair.json")) as f:
        g = json.load(f)
    x = np.zeros(64, np.float32)
    cs = np.zeros(64, np.float32)
    cs[:32] = 1.0
    for k, v in g["x"].items():
        x[int(k)] = v
    for k, v in g["cos"].items():
        cs[int(k)] = v
    for k, v in g["sin"].items():
        cs[32 + int(k)] = v
    want = np.zeros(64, np.float32)
    for k, v in g["expected"].items():
        want[int(k)] = v
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f32(xb), x), "fixture inputs exact in bf16"
    return xb, cs, (want.view(np.uint32) >> 16).astype(np.uint16)


def rand_bf16(rng, shape, sigma=1.0):
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do


def rotation_table(max_pos, base=10000.0):
    """cos/sin of p * base^(-2i/64), from FP64 (a proper rotation per pair)."""
    inv = base ** (-np.arange(32, dtype=np.float64) * 2.0 / 64.0)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def test_golden_row():
    xb, cs, want = golden()
    assert np.array_equal(rope_rows_ref(xb, cs), want)


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact ties: a bf16 value plus half an ulp (low 16 bits 0x8000)
    ties = ((rng.integers(0, 0x4000, 2000).astype(np.uint32) + 0x3000) << 16 | 0x8000).view(np.float32)  # finite
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-40, -1e-40, 3.3e38])])
    got = f32_to_bf16_rne(x)
    for xv, gv in zip(x.tolist(), got.tolist()):
        u = int(np.float32(xv).view(np.uint32))
        lo = u >> 16
        cands = [lo, lo + 1]  # truncation and the next pattern up in magnitude
        val = [float(np.uint32(c << 16).view(np.float32)) for c in cands]
        err = [abs(v - float(xv)) for v in val]
        pick = cands[0] if err[0] < err[1] else cands[1] if err[1] < err[0] else (cands[0] if cands[0] % 2 == 0 else cands[1])
        assert gv == pick, (xv, hex(gv), hex(pick))
    special = f32_to_bf16_rne(np.float32([np.inf, -np.inf, np.nan, 3.4e38, -3.4e38]))
    assert special[0] == 0x7F80 and special[1] == 0xFF80
    # past the largest BF16 value plus half an ulp (3.3961e38) rounding gives infinity
    assert special[3] == 0x7F80 and special[4] == 0xFF80
    assert (special[2] & 0x7F80) == 0x7F80 and (special[2] & 0x007F) != 0  # still a NaN


def test_identity_table_keeps_bits():
    rng = np.random.default_rng(1)
    x = rand_bf16(rng, (40, 64))
    cs = np.concatenate([np.ones(32, np.float32), np.zeros(32, np.float32)])
    assert np.array_equal(rope_rows_ref(x, cs), x)


def test_matches_fp64_within_bf16_rounding():
    rng = np.random.default_rng(2)
    table = rotation_table(2048)
    for pos in (0, 1, 37, 1000, 2047):
        x = rand_bf16(rng, (40, 64), sigma=3.0)
        xf = bf16_bits_to_f32(x).astype(np.float64)
        c = table[pos, :32].astype(np.float64)
        s = table[pos, 32:].astype(np.float64)
        ref = rope_f64(xf, c, s)
        got = bf16_bits_to_f32(rope_rows_ref(x, table[pos])).astype(np.float64)
        lo, hi = xf[:, :32], xf[:, 32:]
        mag = np.concatenate([np.abs(lo * c) + np.abs(hi * s), np.abs(hi * c) + np.abs(lo * s)], axis=1)
        # BF16 rounding (half an ulp, <= 2^-8 relative) of the FP32 result, plus the FP32 roundings
        bound = 2.0 ** -8 * (np.abs(ref) + 2.0 ** -22 * mag) + 2.0 ** -22 * mag
        assert np.all(np.abs(got - ref) <= bound)


def test_pair_norms_preserved():
    rng = np.random.default_rng(3)
    table = rotation_table(512)
    x = rand_bf16(rng, (64, 64))
    xf = bf16_bits_to_f32(x).astype(np.float64)
    got = bf16_bits_to_f32(rope_rows_ref(x, table[311])).astype(np.float64)
    n0 = np.hypot(xf[:, :32], xf[:, 32:])
    n1 = np.hypot(got[:, :32], got[:, 32:])
    assert np.all(np.abs(n1 - n0) <= 2.0 ** -7 * n0 + 1e-30)


def test_inverse_rotation_returns_input():
    rng = np.random.default_rng(4)
    table = rotation_table(300)
    x = rand_bf16(rng, (64, 64))
    fwd = rope_rows_ref(x, table[299])
    inv = table[299].copy()
    inv[32:] = -inv[32:]
    back = bf16_bits_to_f32(rope_rows_ref(fwd, inv)).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    scale = np.hypot(xf[:, :32], xf[:, 32:])
    scale = np.concatenate([scale, scale], axis=1)
    assert np.all(np.abs(back - xf) <= 2.0 ** -6 * scale + 1e-30)


def _case(seed, B=5, Hq=32, Hkv=8, max_blocks=4, num_pages=24, max_pos=64):
    rng = np.random.default_rng(seed)
    q = rand_bf16(rng, (B, Hq, 64))
    k_new = rand_bf16(rng, (B, Hkv, 64))
    v_new = rand_bf16(rng, (B, Hkv, 64))
    k_pool = rand_bf16(rng, (num_pages, 16, Hkv, 64))
    v_pool = rand_bf16(rng, (num_pages, 16, Hkv, 64))
    perm = rng.permutation(num_pages)[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    table = rotation_table(max_pos)
    q_out = rand_bf16(rng, (B, Hq, 64))
    return q, k_new, v_new, table, k_pool, v_pool, perm, q_out


def test_rope_append_rotates_and_places():
    """Every live sequence: q and k rotated at position L - 1, the rotated k and
    the plain v at that position's slot (the append oracle's placement); skipped
    sequences keep their q_out rows and append nothing."""
    q, k_new, v_new, table, k_pool, v_pool, bt, q_out = _case(5)
    lens = np.array([1, 16, 17, 0, 64], np.int32)  # pos 0, a page's last slot, a page's first, empty, the last row
    bt[4, 3] = -1  # the last sequence's page entry is invalid: skipped
    lens2 = lens.copy()
    lens2[4] = 0
    qo, ko, vo = rope_append_ref(q, k_new, v_new, table, k_pool, v_pool, bt, lens, q_out)
    k_rot = np.stack([rope_rows_ref(k_new[b], table[max(int(lens[b]) - 1, 0)]) for b in range(5)])
    k_want, v_want = append_ref(k_pool, v_pool, k_rot, v_new, bt, lens2)
    assert np.array_equal(ko, k_want) and np.array_equal(vo, v_want)
    for b in range(5):
        if lens2[b] > 0:
            assert np.array_equal(qo[b], rope_rows_ref(q[b], table[lens2[b] - 1]))
        else:
            assert np.array_equal(qo[b], q_out[b])
    # position 0 of a proper table is the identity
    assert np.array_equal(qo[0], q[0]) and np.array_equal(ko[bt[0, 0], 0], k_new[0])


def test_rope_append_skips_positions_past_the_table():
    q, k_new, v_new, table, k_pool, v_pool, bt, q_out = _case(6, max_pos=20)
    lens = np.array([21, 20, 3, 40, 5], np.int32)
    qo, ko, vo = rope_append_ref(q, k_new, v_new, table, k_pool, v_pool, bt, lens, q_out)
    live = np.array([0, 20, 3, 0, 5], np.int32)
    k_rot = np.stack([rope_rows_ref(k_new[b], table[max(int(live[b]) - 1, 0)]) for b in range(5)])
    k_want, v_want = append_ref(k_pool, v_pool, k_rot, v_new, bt, live)
    assert np.array_equal(ko, k_want) and np.array_equal(vo, v_want)
    assert np.array_equal(qo[0], q_out[0]) and np.array_equal(qo[3], q_out[3])


# Planted slips: each must be caught by the pins above.
def _interleaved(x_bits, cs):
    x = bf16_bits_to_f32(x_bits)
    c, s = cs[:32], cs[32:]
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return f32_to_bf16_rne(out)


def _sign_swapped(x_bits, cs):
    x = bf16_bits_to_f32(x_bits)
    c, s = cs[:32], cs[32:]
    lo, hi = x[..., :32], x[..., 32:]
    return f32_to_bf16_rne(np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1))


def _cos_sin_swapped(x_bits, cs):
    return rope_rows_ref(x_bits, np.concatenate([cs[32:], cs[:32]]))


def _truncating(x_bits, cs):
    x = bf16_bits_to_f32(x_bits)
    c, s = cs[:32], cs[32:]
    lo, hi = x[..., :32], x[..., 32:]
    out = np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1).astype(np.float32)
    return (out.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("mutant", [_interleaved, _sign_swapped, _cos_sin_swapped, _truncating])
def test_planted_slips_fail_the_golden_row(mutant):
    xb, cs, want = golden()
    assert not np.array_equal(mutant(xb, cs), want)
