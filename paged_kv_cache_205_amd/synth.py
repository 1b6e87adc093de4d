"""Seeded synthetic inputs for paged decode attention.

This module is shared by the tests, the benchmark and the oracle harness.  It
holds none of the attention arithmetic: it only draws sequence lengths, block
tables (page assignments), query/key/value values and the NaN poison that marks
unreferenced pool slots.

Sources (web pages describing the samir-vllm teaching engine):
  [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
           Inference - Start here" (memedata.com copy of the project README).
  [ARCH]   "samir-vllm: Build LLM Inference From Scratch in C++ and CUDA"
           (wpnews.pro), section "Architecture walkthrough".

Facts used from them: pages hold 16 tokens of K and V of one layer ([ARCH] KV
cache paragraph; [README] feature list, KV page pool item); there is one block
table per sequence and layer ([README] same item); the pool is BF16 and shared
and defaults to 128 MiB ([README] paragraph on the KV pool size); the model has
16 layers and a fixed 2048-token context ([README] admission paragraph and the
paragraph on fixed model dimensions).  Head counts (32 query heads, 8 KV heads,
head dim 64) are not stated on the pages; they are the reading that makes
32 x 64 equal the 2048-wide hidden state the README names.

Layout of one plane of the pool: bf16 [num_pages][16 tokens][8 kv heads][64].
The K plane and the V plane are two tensors indexed by the same page id.

Length convention: ``seq_lens[b]`` is the length *after* this step's append.
Positions 0 .. L-2 of every (layer, sequence) hold random values; position L-1
is written by the append from ``k_new``/``v_new``; every other slot of the
pool (tail of the last page, free pages, the append target before the append)
holds BF16 NaN (0x7FC0) so that any stray read shows up in the output.

Random values: float32 standard normals from a seeded torch generator, times
sigma, rounded to BF16 by torch's round-to-nearest-even conversion.  Lengths and
page assignments come from numpy PCG64 generators seeded by
``SeedSequence([205, config_id, draw, stream])``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

PAGE_TOKENS = 16
HQ = 32
HKV = 8
HEAD_DIM = 64
MAX_CONTEXT = 2048
BF16_NAN_BITS = 0x7FC0
ROW_ELEMS = HKV * HEAD_DIM  # bf16 elements in one token row of one plane

# numpy streams
_S_LENS, _S_ALLOC = 0, 1
# torch streams
_S_Q, _S_K, _S_V, _S_KNEW, _S_VNEW = 2, 3, 4, 5, 6
_S_PQ = 7  # prefill queries


def _np_rng(config_id: int, draw: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([205, config_id, draw, stream])))


def _torch_seed(config_id: int, draw: int, stream: int, layer: int) -> int:
    state = np.random.SeedSequence([205, config_id, draw, stream, layer]).generate_state(1, np.uint64)[0]
    return int(state & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _torch_gen(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def nblocks(L: int) -> int:
    return (int(L) + PAGE_TOKENS - 1) // PAGE_TOKENS


@dataclass
class Layout:
    """Host-side description of one synthetic workload (no tensor data)."""

    name: str
    config_id: int
    draw: int
    B: int
    n_layers: int
    max_blocks: int
    num_pages: int
    seq_lens: np.ndarray  # int32 [B], length after the append
    block_tables: np.ndarray  # int32 [n_layers][B][max_blocks], -1 = unassigned
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    scale: float = 0.125  # 1/sqrt(64), exact in binary
    notes: str = ""

    @property
    def kv_bytes_per_layer(self) -> int:
        """Bytes of K and V the attention must read per layer (attended tokens only)."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * ROW_ELEMS * 2

    @property
    def kv_bytes_per_step(self) -> int:
        return self.kv_bytes_per_layer * self.n_layers

    @property
    def pool_bytes(self) -> int:
        return self.num_pages * PAGE_TOKENS * ROW_ELEMS * 2 * 2

    def check_invariants(self) -> None:
        """Allocator invariants every generated layout must satisfy."""
        L = self.seq_lens.astype(np.int64)
        assert self.block_tables.shape == (self.n_layers, self.B, self.max_blocks)
        assert (L >= 0).all() and (L <= self.max_blocks * PAGE_TOKENS).all()
        owned = []
        for l in range(self.n_layers):
            for b in range(self.B):
                n = nblocks(L[b])
                row = self.block_tables[l, b]
                assert ((row[:n] >= 0) & (row[:n] < self.num_pages)).all(), (l, b)
                owned.append(row[:n])
        allp = np.concatenate(owned) if owned else np.zeros(0, np.int64)
        assert len(np.unique(allp)) == len(allp), "a page is owned by two (layer, sequence) pairs"

    def filled_slots(self, layer: int) -> Tuple[np.ndarray, np.ndarray]:
        """(page, slot) of every pre-filled position 0..L-2 of ``layer``, in (b, pos) order."""
        pages, slots = [], []
        for b in range(self.B):
            n = int(self.seq_lens[b]) - 1
            if n <= 0:
                continue
            pos = np.arange(n, dtype=np.int64)
            pages.append(self.block_tables[layer, b, pos // PAGE_TOKENS].astype(np.int64))
            slots.append(pos % PAGE_TOKENS)
        if not pages:
            return np.zeros(0, np.int64), np.zeros(0, np.int64)
        return np.concatenate(pages), np.concatenate(slots)


# ----------------------------------------------------------------------------
# page assignment helpers


def _alloc_layer_seq_block(lens: np.ndarray, n_layers: int, max_blocks: int, free: np.ndarray) -> np.ndarray:
    """Assign pages layer -> sequence -> block from the ``free`` list, in order."""
    B = len(lens)
    bt = np.full((n_layers, B, max_blocks), -1, np.int32)
    k = 0
    for l in range(n_layers):
        for b in range(B):
            n = nblocks(lens[b])
            bt[l, b, :n] = free[k:k + n]
            k += n
    return bt


def _alloc_round_robin(lens: np.ndarray, n_layers: int, max_blocks: int, free: np.ndarray) -> np.ndarray:
    """Assign one block at a time, round-robin over (layer, sequence), as lazy growth would."""
    B = len(lens)
    need = np.array([nblocks(x) for x in lens])
    bt = np.full((n_layers, B, max_blocks), -1, np.int32)
    k = 0
    for j in range(max_blocks):
        for l in range(n_layers):
            for b in range(B):
                if j < need[b]:
                    bt[l, b, j] = free[k]
                    k += 1
    return bt


# ----------------------------------------------------------------------------
# the workloads


def tiny() -> Layout:
    """1 sequence, 1 layer, decode at 37 then append position 37 and decode at 38."""
    rng = _np_rng(1, 0, _S_ALLOC)
    bt = np.full((1, 1, 8), -1, np.int32)
    bt[0, 0] = rng.permutation(8).astype(np.int32)
    return Layout("tiny", 1, 0, B=1, n_layers=1, max_blocks=8, num_pages=8,
                  seq_lens=np.array([38], np.int32), block_tables=bt,
                  notes="pre-filled 37 tokens; decode at 37, append position 37, decode at 38")


def small() -> Layout:
    """8 sequences, 16 layers, L ~ U{1..512}, 128 MiB pool (4096 pages), shuffled free list."""
    lens = _np_rng(2, 0, _S_LENS).integers(1, 513, size=8).astype(np.int32)
    free = _np_rng(2, 0, _S_ALLOC).permutation(4096).astype(np.int32)
    bt = _alloc_layer_seq_block(lens, 16, 128, free)
    return Layout("small", 2, 0, B=8, n_layers=16, max_blocks=128, num_pages=4096,
                  seq_lens=lens, block_tables=bt)


def full(B: int = 64, n_layers: int = 16) -> Layout:
    """Every sequence at 2048 tokens; pages contiguous by sequence: (b*16 + l)*128 + j."""
    lens = np.full(B, MAX_CONTEXT, np.int32)
    mb = MAX_CONTEXT // PAGE_TOKENS
    bt = np.empty((n_layers, B, mb), np.int32)
    for l in range(n_layers):
        for b in range(B):
            bt[l, b] = (b * n_layers + l) * mb + np.arange(mb)
    return Layout("full" if (B, n_layers) == (64, 16) else f"full_b{B}_l{n_layers}", 3, 0,
                  B=B, n_layers=n_layers, max_blocks=mb, num_pages=B * n_layers * mb,
                  seq_lens=lens, block_tables=bt)


def fragmented(B: int = 256, n_layers: int = 16) -> Layout:
    """Log-uniform lengths in [16, 2048] with forced page-boundary cases; pool at ~50% occupancy."""
    rng = _np_rng(4, 0, _S_LENS)
    lens = np.rint(np.exp(rng.uniform(np.log(16.0), np.log(2048.0), size=B)))
    lens = np.clip(lens, 16, 2048).astype(np.int32)
    forced = [16, 17, 1025, 2048]
    lens[:min(B, len(forced))] = forced[:min(B, len(forced))]
    need = int(sum(nblocks(x) for x in lens)) * n_layers
    num_pages = 2 * need
    free = _np_rng(4, 0, _S_ALLOC).permutation(num_pages).astype(np.int32)
    bt = _alloc_round_robin(lens, n_layers, 128, free)
    return Layout("fragmented" if (B, n_layers) == (256, 16) else f"fragmented_b{B}_l{n_layers}", 4, 0,
                  B=B, n_layers=n_layers, max_blocks=128, num_pages=num_pages,
                  seq_lens=lens, block_tables=bt)


def skewed(B: int = 1024, n_layers: int = 16) -> Layout:
    """One sequence at 2048, the rest U{1..64}; keys with sigma 3; pool = exact need, shuffled."""
    rng = _np_rng(5, 0, _S_LENS)
    lens = rng.integers(1, 65, size=B).astype(np.int32)
    lens[int(rng.integers(B))] = 2048
    need = int(sum(nblocks(x) for x in lens)) * n_layers
    free = _np_rng(5, 0, _S_ALLOC).permutation(need).astype(np.int32)
    bt = _alloc_layer_seq_block(lens, n_layers, 128, free)
    return Layout("skewed" if (B, n_layers) == (1024, 16) else f"skewed_b{B}_l{n_layers}", 5, 0,
                  B=B, n_layers=n_layers, max_blocks=128, num_pages=need,
                  seq_lens=lens, block_tables=bt, sigma_k=3.0)


def large(B: int = 1024, n_layers: int = 16) -> Layout:
    """L ~ U{1..2048}, keys with sigma 3; each layer's pages form one contiguous shuffled band."""
    lens = _np_rng(5, 1, _S_LENS).integers(1, 2049, size=B).astype(np.int32)
    per_layer = int(sum(nblocks(x) for x in lens))
    rng = _np_rng(5, 1, _S_ALLOC)
    bt = np.full((n_layers, B, 128), -1, np.int32)
    for l in range(n_layers):
        band = (l * per_layer + rng.permutation(per_layer)).astype(np.int32)
        bt[l] = _alloc_layer_seq_block(lens, 1, 128, band)[0]
    return Layout("large" if (B, n_layers) == (1024, 16) else f"large_b{B}_l{n_layers}", 5, 1,
                  B=B, n_layers=n_layers, max_blocks=128, num_pages=per_layer * n_layers,
                  seq_lens=lens, block_tables=bt, sigma_k=3.0)


CONFIGS = {
    "tiny": tiny,
    "small": small,
    "full": full,
    "fragmented": fragmented,
    "skewed": skewed,
    "large": large,
}


def get(name: str) -> Layout:
    return CONFIGS[name]()


# ----------------------------------------------------------------------------
# tensor data


def _randn_bf16(shape, sigma: float, device, seed: int) -> torch.Tensor:
    g = _torch_gen(torch.device(device), seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def step_inputs(lay: Layout, layer: int, device="cpu") -> Dict[str, torch.Tensor]:
    """q [B][32][64], k_new / v_new [B][8][64] (bf16) for one layer of the decode step."""
    cid, d = lay.config_id, lay.draw
    return {
        "q": _randn_bf16((lay.B, HQ, HEAD_DIM), lay.sigma_q, device, _torch_seed(cid, d, _S_Q, layer)),
        "k_new": _randn_bf16((lay.B, HKV, HEAD_DIM), lay.sigma_k, device, _torch_seed(cid, d, _S_KNEW, layer)),
        "v_new": _randn_bf16((lay.B, HKV, HEAD_DIM), lay.sigma_v, device, _torch_seed(cid, d, _S_VNEW, layer)),
    }


def _layer_values(lay: Layout, l: int, n: int, c: int, dev) -> Tuple[torch.Tensor, torch.Tensor]:
    """Values of chunk c (n token rows) of layer l's pre-filled positions."""
    return (_randn_bf16((n, ROW_ELEMS), lay.sigma_k, dev, _torch_seed(lay.config_id, lay.draw, _S_K, (l << 16) | c)),
            _randn_bf16((n, ROW_ELEMS), lay.sigma_v, dev, _torch_seed(lay.config_id, lay.draw, _S_V, (l << 16) | c)))


def rope_table(max_pos: int = 2048, base: float = 500000.0, device="cpu") -> torch.Tensor:
    """A RoPE table fp32 [max_pos][64] for the rotation's input: row p holds
    cos(p w_i) for i < 32, then sin(p w_i), with w_i = base^(-2i/64), computed
    in FP64.  (The pages give no base; 500000 is a synthetic choice.)"""
    w = base ** (-torch.arange(32, dtype=torch.float64) * 2.0 / 64.0)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * w[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).to(device)


def make_pools(lay: Layout, device="cpu", layers: Optional[List[int]] = None,
               chunk_rows: int = 1 << 22) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V planes, bf16 [num_pages][16][8][64], NaN everywhere except positions 0..L-2.

    Values are drawn per layer in (sequence, position) order, in chunks of at most
    ``chunk_rows`` token rows, each chunk from its own seeded generator.
    """
    dev = torch.device(device)
    shape = (lay.num_pages, PAGE_TOKENS, HKV, HEAD_DIM)
    k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    kf = k_pool.view(lay.num_pages * PAGE_TOKENS, ROW_ELEMS)
    vf = v_pool.view(lay.num_pages * PAGE_TOKENS, ROW_ELEMS)
    for l in (range(lay.n_layers) if layers is None else layers):
        pages, slots = lay.filled_slots(l)
        rows = torch.from_numpy(pages * PAGE_TOKENS + slots).to(dev)
        for c, start in enumerate(range(0, len(rows), chunk_rows)):
            r = rows[start:start + chunk_rows]
            kf[r], vf[r] = _layer_values(lay, l, r.numel(), c, dev)
    return k_pool, v_pool


def prefill_inputs(lay: Layout, layer: int, device="cpu", chunk_rows: int = 1 << 22):
    """One layer's prompt rows packed as a prefill fill takes them.

    Returns (k_src, v_src, cu_tokens): bf16 [T][8][64] holding the values that
    ``make_pools`` puts at positions 0..L-2 of every sequence (same generators,
    same (sequence, position) order), and int32 [B+1] run boundaries with
    run b of length max(L_b - 1, 0).
    """
    dev = torch.device(device)
    n = np.maximum(lay.seq_lens.astype(np.int64) - 1, 0)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(cu[-1])
    ks, vs = [], []
    for c, start in enumerate(range(0, T, chunk_rows)):
        k, v = _layer_values(lay, layer, min(chunk_rows, T - start), c, dev)
        ks.append(k)
        vs.append(v)
    empty = torch.empty((0, ROW_ELEMS), dtype=torch.bfloat16, device=dev)
    k_src = (torch.cat(ks) if ks else empty).view(T, HKV, HEAD_DIM)
    v_src = (torch.cat(vs) if vs else empty).view(T, HKV, HEAD_DIM)
    return k_src, v_src, torch.from_numpy(cu).to(dev)


def prefill_queries(lay: Layout, layer: int, device="cpu", chunk_rows: int = 1 << 20) -> torch.Tensor:
    """Queries of one layer's prompt rows, bf16 [T][32][64] in the row order of
    ``prefill_inputs`` (T = sum of max(L_b - 1, 0)), N(0, sigma_q) values drawn in
    chunks of ``chunk_rows`` rows, each chunk from its own seeded generator."""
    dev = torch.device(device)
    T = int(np.maximum(lay.seq_lens.astype(np.int64) - 1, 0).sum())
    parts = [_randn_bf16((min(chunk_rows, T - start), HQ, HEAD_DIM), lay.sigma_q, dev,
                         _torch_seed(lay.config_id, lay.draw, _S_PQ, (layer << 16) | c))
             for c, start in enumerate(range(0, T, chunk_rows))]
    return torch.cat(parts) if parts else torch.empty((0, HQ, HEAD_DIM), dtype=torch.bfloat16, device=dev)


def layer_pages(lay: Layout, layer: int, device="cpu", chunk_rows: int = 1 << 22):
    """Only the pages of one layer, renumbered 0..n-1: (k_pages, v_pages, block_table).

    Holds the same values ``make_pools`` puts in those pages (same generators,
    same order), without materialising the rest of the pool.  The returned
    block table is int32 [B][max_blocks] in the local numbering (-1 kept).
    """
    dev = torch.device(device)
    bt = lay.block_tables[layer]
    used = np.unique(np.concatenate([bt[b, :nblocks(lay.seq_lens[b])] for b in range(lay.B)] or [np.zeros(0, np.int32)]))
    local = np.full(lay.num_pages, -1, np.int64)
    local[used] = np.arange(len(used))
    bt_local = np.where(bt >= 0, local[np.maximum(bt, 0)], -1).astype(np.int32)
    shape = (len(used), PAGE_TOKENS, HKV, HEAD_DIM)
    k_pages = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pages = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    kf = k_pages.view(-1, ROW_ELEMS)
    vf = v_pages.view(-1, ROW_ELEMS)
    pages, slots = lay.filled_slots(layer)
    rows = torch.from_numpy(local[pages] * PAGE_TOKENS + slots).to(dev)
    for c, start in enumerate(range(0, len(rows), chunk_rows)):
        r = rows[start:start + chunk_rows]
        kf[r], vf[r] = _layer_values(lay, layer, r.numel(), c, dev)
    return k_pages, v_pages, bt_local


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw BF16 bit patterns of ``t`` as a host numpy uint16 array."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def sequence_pages(k_pool: torch.Tensor, v_pool: torch.Tensor, lay: Layout, layer: int, b: int):
    """Host copies of the pages that (layer, b) owns, and a block table row over them.

    Returns (k_pages, v_pages, bt_row) where the page arrays are uint16
    [n][16][8][64] and ``bt_row`` maps logical block j to local page j.  Used to
    feed the oracle a single sequence of a large pool without copying the pool.
    """
    n = nblocks(int(lay.seq_lens[b]))
    ids = torch.from_numpy(lay.block_tables[layer, b, :n].astype(np.int64)).to(k_pool.device)
    kp = bits(k_pool.index_select(0, ids))
    vp = bits(v_pool.index_select(0, ids))
    return kp, vp, np.arange(n, dtype=np.int32)
