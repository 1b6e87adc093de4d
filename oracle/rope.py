"""CPU oracle for RoPE at the absolute position fused with the one-token append.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library; inputs are numpy arrays of BF16 bit patterns (uint16), FP32 tables and
int32 tables.

What the pages fix
------------------
* RoPE is the position encoding applied to the queries and keys before
  attention ([README] feature list: the kernels include RoPE, and dense causal
  prefill runs Q/K/V projection, then RoPE, then grouped-query attention).
* Decode appends the one new token of a sequence into its page slot "at its
  absolute RoPE position": the new token's position is its absolute index in
  the sequence ([README] KV page pool item; [ARCH] KV cache paragraph).

Readings where the pages are silent (none of these is printed on the pages)
-------------------------------------------------------------------------
* The rotation constants (base, frequency scaling) are not given, so they are
  an input: ``cos_sin[p]`` holds, for position p, c_i = cos_sin[p][i] and
  s_i = cos_sin[p][32 + i] (i < 32) as FP32.  Any base or scaling is a choice
  of this table.
* Pairing: dimension i is rotated together with dimension i + 32 (the
  "rotate half" convention of the Llama models the pages name):

      x'[i]      = x[i] c_i - x[i + 32] s_i
      x'[i + 32] = x[i + 32] c_i + x[i] s_i,      i = 0 .. 31.

* The new token of sequence b sits at position L - 1 (L = seq_lens[b], the
  length after the append); q[b] is the query of that token, so it is rotated
  at the same position.
* Precision: the result is stored as BF16, so the rounding decides a stored
  code.  The oracle takes that decision in the precision of the kernel: each
  product and the difference / sum are single FP32 operations (rounded to
  nearest, no fused multiply-add), and the FP32 result is rounded to BF16 to
  nearest, ties to even.  A NaN keeps its sign and upper payload with the quiet
  bit set.  The FP64 rotation is within the BF16 rounding of this (tested).
* A sequence with L <= 0, or whose position has no row in the table
  (L - 1 >= max_pos), or whose page entry is outside [0, num_pages), is
  skipped: its q_out rows are left as they were and nothing is appended.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .oracle import append_ref

HALF = 32  # rotation pairs (i, i + HALF) of a 64-wide head


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact BF16 -> FP32: a BF16 value is the upper half of an FP32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 bits, rounded to nearest with ties to even; NaN stays a
    quiet NaN with its sign and upper payload."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = (u >> np.uint64(16)) | np.uint64(0x0040)
    return np.where(nan, quiet, rounded).astype(np.uint16)


def rope_rows_ref(x_bits: np.ndarray, cs_row: np.ndarray) -> np.ndarray:
    """Rotate the rows x[..., 64] (BF16 bits) by one position's table row
    cs_row[64] (FP32: 32 cosines then 32 sines); returns BF16 bits."""
    x = bf16_bits_to_f32(x_bits)
    c = np.asarray(cs_row[:HALF], dtype=np.float32)
    s = np.asarray(cs_row[HALF:2 * HALF], dtype=np.float32)
    lo, hi = x[..., :HALF], x[..., HALF:]
    with np.errstate(invalid="ignore", over="ignore"):
        out_lo = np.subtract(np.multiply(lo, c, dtype=np.float32), np.multiply(hi, s, dtype=np.float32),
                             dtype=np.float32)
        out_hi = np.add(np.multiply(hi, c, dtype=np.float32), np.multiply(lo, s, dtype=np.float32),
                        dtype=np.float32)
    return f32_to_bf16_rne(np.concatenate([out_lo, out_hi], axis=-1))


def rope_f64(x: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The same rotation in FP64 on real inputs (no rounding), for pins."""
    lo, hi = x[..., :HALF], x[..., HALF:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_append_ref(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, cos_sin: np.ndarray,
                    k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                    q_out: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Return (q_out, k_pool, v_pool) after RoPE at position L - 1 and the append.

    q: uint16 [B][Hq][64]; k_new, v_new: uint16 [B][Hkv][64]; cos_sin: float32
    [max_pos][64]; pools uint16 [num_pages][16][Hkv][64]; block_table int32
    [B][max_blocks]; seq_lens int32 [B]; q_out: uint16 [B][Hq][64], the rows
    of skipped sequences are kept.  Inputs are not modified.
    """
    B = int(q.shape[0])
    max_pos = int(cos_sin.shape[0])
    num_pages = int(k_pool.shape[0])
    q_res = np.array(q_out, dtype=np.uint16, copy=True)
    k_rot = np.array(k_new, dtype=np.uint16, copy=True)
    lens = np.zeros(B, dtype=np.int32)  # 0 = skipped by the append below
    for b in range(B):
        L = int(seq_lens[b])
        pos = L - 1
        if L <= 0 or pos >= max_pos or (pos >> 4) >= block_table.shape[1]:
            continue
        page = int(block_table[b][pos >> 4])
        if page < 0 or page >= num_pages:
            continue
        q_res[b] = rope_rows_ref(q[b], cos_sin[pos])
        k_rot[b] = rope_rows_ref(k_new[b], cos_sin[pos])
        lens[b] = L
    k_out, v_out = append_ref(k_pool, v_pool, k_rot, v_new, block_table, lens)
    return q_res, k_out, v_out
