"""Decode at the limits of the C ABI, against the FP64 oracle in full.

- Block tables longer than 128 entries: the kernel then reads each split's own
  table entries instead of the whole row (the path the five workloads, with
  their 128-entry tables, never take).  Lengths straddle the 2048-token context
  of the workloads, up to the whole table.
- The longest table the library takes (PA_MAX_BLOCKS_LIMIT = 4096 pages,
  65,536 tokens), with a sequence that fills it.
- The largest batch (PA_MAX_DECODE_BATCH = 4096 sequences) of short lengths,
  empty sequences included.

Each case appends (bit-exact against append_ref over the whole pool) and then
decodes under several split sizes.  Inputs follow the workloads' recipe:
standard-normal BF16 values, NaN in every slot that is not a filled position,
pages dealt one block at a time from a shuffled free list with spare pages.
"""
import numpy as np
import pytest
import torch

from oracle import append_ref, decode_ref
from paged_kv_cache_205_amd import ops, synth
from tests.helpers import Device, check_close, say

pytestmark = pytest.mark.gpu

MAX_BLOCKS_LIMIT = 4096
MAX_DECODE_BATCH = 4096


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def layout(name: str, seed_id: int, lens, max_blocks: int, spare: int = 5) -> synth.Layout:
    """One layer; block j of every sequence is assigned before block j + 1 of any."""
    lens = np.asarray(lens, np.int32)
    need = [synth.nblocks(x) for x in lens]
    num_pages = sum(need) + spare
    free = np.random.default_rng(seed_id).permutation(num_pages).astype(np.int32)
    bt = np.full((1, len(lens), max_blocks), -1, np.int32)
    k = 0
    for j in range(max(need)):
        for b, n in enumerate(need):
            if j < n:
                bt[0, b, j] = free[k]
                k += 1
    lay = synth.Layout(name, seed_id, 0, B=len(lens), n_layers=1, max_blocks=max_blocks,
                       num_pages=num_pages, seq_lens=lens, block_tables=bt)
    lay.check_invariants()
    return lay


def append_then_decode(lay: synth.Layout, partitions):
    d = Device(lay)
    kp0, vp0 = synth.bits(d.k_pool), synth.bits(d.v_pool)
    x = d.inputs[0]
    d.append(0)
    k2, v2 = append_ref(kp0, vp0, synth.bits(x["k_new"]), synth.bits(x["v_new"]), lay.block_tables[0], lay.seq_lens)
    assert np.array_equal(synth.bits(d.k_pool), k2) and np.array_equal(synth.bits(d.v_pool), v2), "append"
    ref = decode_ref(synth.bits(x["q"]), k2, v2, lay.block_tables[0], lay.seq_lens, lay.scale)
    for part in partitions:
        say(f"{lay.name}: B={lay.B} max_blocks={lay.max_blocks} partition {part}")
        out = d.decode(0, partition_tokens=part)
        torch.cuda.synchronize()
        ea, er = check_close(out.cpu().numpy(), ref, f"{lay.name} partition {part}")
        say(f"{lay.name} partition {part}: max abs {ea:.2e} rel {er:.2e}")


def test_tables_longer_than_128_entries():
    lay = layout("long_tables", 61, [4800, 2049, 4799, 1, 0, 3007, 16, 17, 2048, 4785], max_blocks=300)
    append_then_decode(lay, [0, 16, 256, 2048])


def test_longest_table():
    lay = layout("longest_table", 62, [16 * MAX_BLOCKS_LIMIT, 12345, 1], max_blocks=MAX_BLOCKS_LIMIT)
    append_then_decode(lay, [0, 2048])


def test_largest_batch():
    rng = np.random.default_rng(63)
    lens = rng.integers(0, 49, size=MAX_DECODE_BATCH)
    lens[:6] = [0, 1, 16, 17, 48, 32]
    lay = layout("largest_batch", 63, lens, max_blocks=3)
    append_then_decode(lay, [0, 16])
