"""Plain FP64 CPU oracle for paged decode attention and the one-token KV append.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it; inputs are plain numpy arrays holding BF16
bit patterns (uint16) and int32 tables.

What it computes, and where the pages say so
--------------------------------------------
Sources (web pages describing the samir-vllm teaching engine):
  [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
           Inference - Start here" (memedata.com copy of the project README),
           feature list.
  [ARCH]   "samir-vllm: Build LLM Inference From Scratch in C++ and CUDA"
           (wpnews.pro), section "Architecture walkthrough", KV cache paragraph.
  [NF]     news-factory.app article on the free LLM-inference course, section
           "How does the engine manage KV cache memory?".

* Pool and tables: one shared BF16 pool of physical pages, each holding 16
  tokens of K and V of one layer, and a block table per (sequence, layer) that
  maps logical 16-token blocks to pages ([README] KV page pool item; [ARCH]).
* Append: each decode step writes the one new token of a sequence into its
  page slot at its absolute position ([README] KV page pool item; [ARCH]).
* Prefill fill: prefill writes the K and V rows of a sequence's prompt tokens
  into that sequence's pages, through the same block table ([README] KV page
  pool item: prefill fills prompt pages).
* Prefill attention: dense causal grouped-query attention over a prompt's own
  contiguous K and V ([README] feature list: dense causal prefill runs
  grouped-query attention in all 16 layers): position i of a prompt attends
  positions 0..i,

      out[i, h] = sum_{j <= i} softmax_j(scale * q[i, h] . k[j, g]) * v[j, g].
* Decode attention: every query head reads its sequence's cached pages directly
  (no contiguous gather) and forms softmax-weighted sums of V ([README] paged
  decode attention item; [NF]).  The pages compute it with an FP32 online
  softmax; online softmax and the split/merge over page ranges are exact
  rewrites of the plain softmax, so the oracle is the plain definition

      out[b, h] = sum_t softmax_t(scale * q[b, h] . K_t[g]) * V_t[g],
      t = 0 .. L-1,  g = h // (Hq / Hkv),

  evaluated in FP64 by walking the block table page by page.

Readings where the pages are silent:
  * ``seq_lens[b]`` is the length after the append; decode attends every
    position t < L, including the one just appended.
  * query head h uses KV head h // G with G = Hq / Hkv (contiguous groups).
  * in-page layout per plane: [16 tokens][Hkv][D].
  * L = 0: append skips the sequence; decode returns zeros for it.
  * prefill fill writes n_b consecutive tokens of sequence b at positions
    start_b .. start_b + n_b - 1; the pages' prefill is start_b = 0, and a
    one-token fill at start_b = L - 1 is the append.
  * the split partial state is (m, l, o): m the maximum scaled score of the
    split in natural-log units, l = sum exp(s - m), o = (sum exp(s - m) v) / l.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

import numpy as np

PAGE_TOKENS = 16


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact BF16 -> FP64 conversion: a BF16 value is the top half of an FP32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def append_ref(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
               block_table: np.ndarray, seq_lens: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with token L-1 of every sequence written (bit copy).

    k_pool/v_pool: uint16 [num_pages][16][Hkv][D]; k_new/v_new: uint16 [B][Hkv][D];
    block_table: int32 [B][max_blocks] of one layer; seq_lens: int32 [B].
    """
    k_out = np.array(k_pool, dtype=np.uint16, copy=True)
    v_out = np.array(v_pool, dtype=np.uint16, copy=True)
    num_pages, max_blocks = k_pool.shape[0], block_table.shape[1]
    written = set()
    for b, L in enumerate(np.asarray(seq_lens).tolist()):
        if L <= 0:
            continue
        pos = L - 1
        blk, slot = pos // PAGE_TOKENS, pos % PAGE_TOKENS
        assert blk < max_blocks, "sequence longer than its block table"
        page = int(block_table[b, blk])
        assert 0 <= page < num_pages, "block table entry outside the pool"
        assert (page, slot) not in written, "two sequences append into the same slot"
        written.add((page, slot))
        k_out[page, slot] = k_new[b]
        v_out[page, slot] = v_new[b]
    return k_out, v_out


def fill_ref(k_pool: np.ndarray, v_pool: np.ndarray, k_src: np.ndarray, v_src: np.ndarray,
             block_table: np.ndarray, start, cu_tokens) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with each sequence's run of tokens written (bit copy).

    k_src/v_src: uint16 [T][Hkv][D], the tokens of all sequences one after another:
    sequence b owns rows cu_tokens[b] .. cu_tokens[b+1]-1.  Row i of that range is the
    token at position start[b] + i (start None: every start is 0), which lives in page
    block_table[b][position // 16], slot position % 16.
    """
    k_out = np.array(k_pool, dtype=np.uint16, copy=True)
    v_out = np.array(v_pool, dtype=np.uint16, copy=True)
    num_pages, max_blocks = k_pool.shape[0], block_table.shape[1]
    cu = np.asarray(cu_tokens, dtype=np.int64)
    B = len(cu) - 1
    st = np.zeros(B, np.int64) if start is None else np.asarray(start, dtype=np.int64)
    written = set()
    for b in range(B):
        for i in range(int(cu[b + 1] - cu[b])):
            pos = int(st[b]) + i
            blk, slot = pos // PAGE_TOKENS, pos % PAGE_TOKENS
            assert blk < max_blocks, "position beyond the block table"
            page = int(block_table[b, blk])
            assert 0 <= page < num_pages, "block table entry outside the pool"
            assert (page, slot) not in written, "two tokens written into the same slot"
            written.add((page, slot))
            k_out[page, slot] = k_src[cu[b] + i]
            v_out[page, slot] = v_src[cu[b] + i]
    return k_out, v_out


def prefill_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_tokens, scale: float) -> np.ndarray:
    """Causal attention of each prompt over its own tokens, in FP64.

    q: uint16 [T][Hq][D]; k, v: uint16 [T][Hkv][D] (BF16 bits), prompts one after
    another: prompt b is rows cu_tokens[b] .. cu_tokens[b+1]-1.  Returns
    float64 [T][Hq][D].  Query head h uses KV head h // (Hq / Hkv).
    """
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    cu = np.asarray(cu_tokens, dtype=np.int64)
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        Q, K, V = bf16_to_f64(q[r0:r1]), bf16_to_f64(k[r0:r1]), bf16_to_f64(v[r0:r1])
        later = np.triu(np.ones((n, n), dtype=bool), 1)  # j > i: not attended
        for h in range(Hq):
            g = h // G
            s = scale * (Q[:, h] @ K[:, g].T)
            s[later] = -np.inf
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[r0:r1, h] = (w @ V[:, g]) / w.sum(axis=1, keepdims=True)
    return out


def prefill_rows_ref(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, starts, rows, scale: float) -> np.ndarray:
    """Selected rows of the causal prefill attention, in FP64, one at a time.

    q_rows: uint16 [R][Hq][D], the queries of packed rows ``rows``; k, v: uint16
    [T][Hkv][D] (all prompts); starts[r]: first row of the prompt that rows[r]
    belongs to.  Row r attends keys starts[r] .. rows[r], as in prefill_ref.
    Returns float64 [R][Hq][D].
    """
    R, Hq, D = q_rows.shape
    G = Hq // k.shape[1]
    out = np.zeros((R, Hq, D))
    for r in range(R):
        j0, j1 = int(starts[r]), int(rows[r]) + 1
        K, V = bf16_to_f64(k[j0:j1]), bf16_to_f64(v[j0:j1])
        Q = bf16_to_f64(q_rows[r])
        for h in range(Hq):
            s = scale * (K[:, h // G] @ Q[h])
            w = np.exp(s - s.max())
            out[r, h] = (w @ V[:, h // G]) / w.sum()
    return out


def _walk(k_pool, v_pool, block_table_row, L, g, t0=0, t1=None):
    """Yield (K rows, V rows) as FP64 arrays for the tokens [t0, t1) of one sequence, page by page."""
    t1 = L if t1 is None else t1
    for j in range(t0 // PAGE_TOKENS, (t1 + PAGE_TOKENS - 1) // PAGE_TOKENS):
        page = int(block_table_row[j])
        lo = max(t0, j * PAGE_TOKENS) - j * PAGE_TOKENS
        hi = min(t1, (j + 1) * PAGE_TOKENS) - j * PAGE_TOKENS
        yield bf16_to_f64(k_pool[page, lo:hi, g, :]), bf16_to_f64(v_pool[page, lo:hi, g, :])


def scores_and_values(q, k_pool, v_pool, block_table, seq_lens, scale, b, h, t0=0, t1=None):
    """Scaled scores s_t = scale * q[b,h].K_t and the matching V rows for tokens [t0, t1)."""
    Hq, Hkv = q.shape[1], k_pool.shape[2]
    g = h // (Hq // Hkv)
    L = int(seq_lens[b])
    qh = bf16_to_f64(q[b, h])
    s_parts: List[np.ndarray] = []
    v_parts: List[np.ndarray] = []
    for K, V in _walk(k_pool, v_pool, block_table[b], L, g, t0, t1):
        s_parts.append(scale * (K @ qh))
        v_parts.append(V)
    if not s_parts:
        return np.zeros(0), np.zeros((0, q.shape[2]))
    return np.concatenate(s_parts), np.concatenate(v_parts)


def decode_ref(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
               seq_lens: np.ndarray, scale: float, batch: Iterable[int] = None) -> np.ndarray:
    """FP64 decode attention for one layer.  Returns float64 [B][Hq][D].

    q: uint16 [B][Hq][D]; pools uint16 [num_pages][16][Hkv][D]; block_table int32
    [B][max_blocks]; seq_lens int32 [B].  ``batch`` restricts the work to some
    sequences (the other rows are left at zero).
    """
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), np.float64)
    for b in (range(B) if batch is None else batch):
        if int(seq_lens[b]) == 0:
            continue
        for h in range(Hq):
            s, V = scores_and_values(q, k_pool, v_pool, block_table, seq_lens, scale, b, h)
            m = s.max()
            w = np.exp(s - m)
            out[b, h] = (w @ V) / w.sum()
    return out


def partial_ref(q, k_pool, v_pool, block_table, seq_lens, scale, b, h, t0, t1):
    """Partial state (m, l, o) of one (sequence, query head) over tokens [t0, t1).

    An empty range returns (-inf, 0, zeros).
    """
    s, V = scores_and_values(q, k_pool, v_pool, block_table, seq_lens, scale, b, h, t0, t1)
    if s.size == 0:
        return -math.inf, 0.0, np.zeros(q.shape[2])
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return m, l, (w @ V) / l


def merge_ref(ms: Sequence[float], ls: Sequence[float], os: Sequence[np.ndarray]) -> np.ndarray:
    """Combine partial states of disjoint token ranges into the full softmax average.

    M = max m_i, w_i = l_i exp(m_i - M), out = sum w_i o_i / sum w_i.  States with
    l_i = 0 or m_i = -inf hold no tokens and are skipped; if none is left the
    result is zero.
    """
    live = [i for i in range(len(ms)) if ls[i] > 0 and ms[i] != -math.inf]
    if not live:
        return np.zeros_like(np.asarray(os[0], dtype=np.float64))
    M = max(ms[i] for i in live)
    num = 0.0
    den = 0.0
    for i in live:
        w = ls[i] * math.exp(ms[i] - M)
        num = num + w * np.asarray(os[i], dtype=np.float64)
        den += w
    return num / den
