"""Pins of the oracle's prefill fill (fill_ref) against facts that do not come from it.

A fill writes a run of consecutive tokens of each sequence into its pages.  The
pins: a placement worked out by hand, the one-token fill being exactly the
append (whose own pins are in test_oracle.py), a gather through the block table
returning the source rows, attention over filled pages equalling attention over
the source rows with no pages at all, invariance under a permutation of the
physical pages, and planted slips in a copy of the fill that each fail a pin.
"""
import numpy as np
import pytest
import scipy.special

from oracle import append_ref, bf16_to_f64, decode_ref, fill_ref
from tests.test_oracle import PT, rand_bits, random_case

NAN = 0x7FC0


def fill_case(seed, lens, starts=None, Hkv=2, D=16, max_blocks=8, spare=3):
    """Tables for runs [start, start + n) per sequence, a NaN-poisoned pool, source rows."""
    rng = np.random.default_rng(seed)
    lens = [int(n) for n in lens]
    starts = [0] * len(lens) if starts is None else [int(s) for s in starts]
    B = len(lens)
    need = [(s + n + PT - 1) // PT for s, n in zip(starts, lens)]
    num_pages = sum(need) + spare
    free = rng.permutation(num_pages)
    bt = np.full((B, max_blocks), -1, np.int32)
    k = 0
    for b in range(B):
        bt[b, :need[b]] = free[k:k + need[b]]
        k += need[b]
    kp = np.full((num_pages, PT, Hkv, D), NAN, np.uint16)
    vp = kp.copy()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ks = rand_bits(rng, (int(cu[-1]), Hkv, D))
    vs = rand_bits(rng, (int(cu[-1]), Hkv, D))
    return kp, vp, ks, vs, bt, np.array(starts, np.int32), cu


def test_fill_hand_worked_placement():
    # table row [2, 0, 3]; 4 tokens from position 14: positions 14 and 15 are slots 14
    # and 15 of block 0 (page 2), positions 16 and 17 are slots 0 and 1 of block 1 (page 0)
    bt = np.array([[2, 0, 3]], np.int32)
    kp = np.zeros((4, PT, 1, 2), np.uint16)
    vp = np.zeros_like(kp)
    ks = np.array([[[1, 2]], [[3, 4]], [[5, 6]], [[7, 8]]], np.uint16)
    vs = ks + 100
    k2, v2 = fill_ref(kp, vp, ks, vs, bt, np.array([14], np.int32), np.array([0, 4], np.int32))
    placed = {(2, 14): 0, (2, 15): 1, (0, 0): 2, (0, 1): 3}
    for (page, slot), i in placed.items():
        assert np.array_equal(k2[page, slot], ks[i]) and np.array_equal(v2[page, slot], vs[i])
    changed = {tuple(x) for x in np.argwhere((k2 != 0).any(axis=(2, 3)))}
    assert changed == set(placed)
    assert np.array_equal(kp, np.zeros_like(kp)), "input pool modified"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_token_fill_is_the_append(seed):
    q, kp, vp, bt, lens = random_case(seed, B=6, lens=[1, 15, 16, 17, 0, 96])
    rng = np.random.default_rng(seed + 10)
    kn = rand_bits(rng, (6, 2, 16))
    vn = rand_bits(rng, (6, 2, 16))
    live = lens > 0
    cu = np.concatenate([[0], np.cumsum(live)]).astype(np.int32)
    k1, v1 = append_ref(kp, vp, kn, vn, bt, lens)
    k2, v2 = fill_ref(kp, vp, kn[live], vn[live], bt, np.maximum(lens - 1, 0), cu)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


@pytest.mark.parametrize("seed", [3, 4])
def test_gather_through_the_table_returns_the_source(seed):
    lens, starts = [0, 1, 15, 16, 17, 40, 128], [0, 0, 3, 16, 15, 31, 0]
    kp, vp, ks, vs, bt, st, cu = fill_case(seed, lens, starts, max_blocks=9)
    k2, v2 = fill_ref(kp, vp, ks, vs, bt, st, cu)
    for b, (s, n) in enumerate(zip(starts, lens)):
        pos = np.arange(s, s + n)
        rows_k = k2[bt[b, pos // PT], pos % PT]
        rows_v = v2[bt[b, pos // PT], pos % PT]
        assert np.array_equal(rows_k, ks[cu[b]:cu[b + 1]]) and np.array_equal(rows_v, vs[cu[b]:cu[b + 1]])
    # exactly sum(n) slots changed, every other byte kept
    assert int(((k2 != kp).any(axis=(2, 3))).sum()) == sum(lens)
    assert int(((v2 != vp).any(axis=(2, 3))).sum()) == sum(lens)


def test_attention_over_filled_pages_is_attention_over_the_prompt():
    lens = [1, 16, 29, 70]
    kp, vp, ks, vs, bt, st, cu = fill_case(5, lens, Hkv=2, D=16)
    k2, v2 = fill_ref(kp, vp, ks, vs, bt, None, cu)
    rng = np.random.default_rng(6)
    q = rand_bits(rng, (len(lens), 8, 16))
    out = decode_ref(q, k2, v2, bt, np.array(lens, np.int32), 0.25)
    for b, n in enumerate(lens):  # no pages: the source rows as one contiguous sequence
        K = bf16_to_f64(ks[cu[b]:cu[b + 1]])
        V = bf16_to_f64(vs[cu[b]:cu[b + 1]])
        for h in range(8):
            s = 0.25 * K[:, h // 4] @ bf16_to_f64(q[b, h])
            ref = scipy.special.softmax(s) @ V[:, h // 4]
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)


def test_fill_page_permutation():
    lens, starts = [5, 33, 18], [0, 2, 14]
    kp, vp, ks, vs, bt, st, cu = fill_case(7, lens, starts)
    k1, v1 = fill_ref(kp, vp, ks, vs, bt, st, cu)
    perm = np.random.default_rng(8).permutation(kp.shape[0])
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    k2, v2 = fill_ref(kp, vp, ks, vs, bt2, st, cu)  # the poisoned pool is the same under any permutation
    assert np.array_equal(k2[perm], k1) and np.array_equal(v2[perm], v1)


def test_fill_empty_and_rejections():
    kp = np.zeros((2, PT, 1, 1), np.uint16)
    src = np.zeros((0, 1, 1), np.uint16)
    k2, v2 = fill_ref(kp, kp, src, src, np.zeros((0, 1), np.int32), None, np.array([0], np.int32))
    assert np.array_equal(k2, kp)
    one = np.ones((2, 1, 1), np.uint16)
    with pytest.raises(AssertionError):  # two sequences into one slot
        fill_ref(kp, kp, one, one, np.array([[0], [0]], np.int32), np.array([3, 3], np.int32),
                 np.array([0, 1, 2], np.int32))
    with pytest.raises(AssertionError):  # beyond the table
        fill_ref(kp, kp, one, one, np.array([[0]], np.int32), np.array([15], np.int32), np.array([0, 2], np.int32))


# ---------------------------------------------------------------- planted slips


def make_fill(mistake):
    """A copy of the fill with one planted mistake (same loop structure otherwise)."""

    def fill(kp, vp, ks, vs, bt, start, cu):
        k2, v2 = kp.copy(), vp.copy()
        B = len(cu) - 1
        st = np.zeros(B, np.int64) if start is None else np.asarray(start, np.int64)
        for b in range(B):
            for i in range(int(cu[b + 1] - cu[b])):
                pos = (0 if mistake == "ignore_start" else int(st[b])) + i
                blk = (pos + 1) // PT if mistake == "block_of_next" else pos // PT
                slot = (pos + 1) % PT if mistake == "slot_shift" else pos % PT
                page = int(bt[b, min(blk, bt.shape[1] - 1)])
                row = int(cu[b]) + i + (1 if mistake == "row_shift" and i + 1 < cu[b + 1] - cu[b] else 0)
                k2[page, slot] = (vs if mistake == "k_from_v" else ks)[row]
                v2[page, slot] = vs[row]
        return k2, v2

    return fill


FILL_MUTANTS = ["ignore_start", "block_of_next", "slot_shift", "row_shift", "k_from_v"]


def pins_hold(fill):
    """The hand-worked placement and the gather round trip, run against a fill function."""
    bt = np.array([[2, 0, 3]], np.int32)
    kp = np.zeros((4, PT, 1, 2), np.uint16)
    ks = np.array([[[1, 2]], [[3, 4]], [[5, 6]], [[7, 8]]], np.uint16)
    vs = ks + 100
    k2, v2 = fill(kp, kp.copy(), ks, vs, bt, np.array([14], np.int32), np.array([0, 4], np.int32))
    placed = {(2, 14): 0, (2, 15): 1, (0, 0): 2, (0, 1): 3}
    ok = all(np.array_equal(k2[p, s], ks[i]) and np.array_equal(v2[p, s], vs[i]) for (p, s), i in placed.items())
    lens, starts = [3, 17, 40], [0, 15, 5]
    kq, vq, ks2, vs2, bt2, st2, cu2 = fill_case(9, lens, starts)
    k3, v3 = fill(kq, vq, ks2, vs2, bt2, st2, cu2)
    for b, (s, n) in enumerate(zip(starts, lens)):
        pos = np.arange(s, s + n)
        ok &= bool(np.array_equal(k3[bt2[b, pos // PT], pos % PT], ks2[cu2[b]:cu2[b + 1]]))
        ok &= bool(np.array_equal(v3[bt2[b, pos // PT], pos % PT], vs2[cu2[b]:cu2[b + 1]]))
    return ok


def test_unmutated_copy_passes_the_fill_pins():
    assert pins_hold(make_fill("none")) and pins_hold(fill_ref)


@pytest.mark.parametrize("mistake", FILL_MUTANTS)
def test_fill_mutant_is_caught(mistake):
    assert not pins_hold(make_fill(mistake)), f"no pin catches the fill mutant {mistake!r}"
