"""Shared helpers for the GPU parity tests: oracle inputs and the tolerance check."""
import sys

import numpy as np
import torch

from oracle import append_ref, bf16_to_f64, decode_ref
from paged_kv_cache_205_amd import ops, synth

# Tolerance for the FP32 attention output against the FP64 oracle, for BF16
# N(0,1) inputs and scale 1/sqrt(64): element-wise absolute error, and a
# row-wise (per sequence and head) relative error normalised by the row's
# largest reference magnitude.
ABS_TOL = 2e-3
REL_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Assert no NaN/Inf, max |got-ref| <= 2e-3 and row-wise relative error <= 1e-2."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = np.abs(ref).max(axis=-1)
    rowerr = err.max(axis=-1)
    live = denom > 0
    max_rel = float((rowerr[live] / denom[live]).max()) if live.any() else 0.0
    assert max_abs <= ABS_TOL, f"{what}: max abs error {max_abs:.3g}"
    assert max_rel <= REL_TOL, f"{what}: max row-relative error {max_rel:.3g}"
    return max_abs, max_rel


class Device:
    """A workload resident on the GPU: pools, tables, lengths and per-layer step inputs."""

    def __init__(self, lay: synth.Layout, dev="cuda"):
        self.lay = lay
        self.dev = dev
        self.k_pool, self.v_pool = synth.make_pools(lay, dev)
        self.bt = torch.from_numpy(lay.block_tables).to(dev)  # [layers][B][max_blocks]
        self.seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
        self.inputs = [synth.step_inputs(lay, l, dev) for l in range(lay.n_layers)]

    def append(self, l, seq_lens=None):
        x = self.inputs[l]
        ops.pa_append(x["k_new"], x["v_new"], self.k_pool, self.v_pool, self.bt[l],
                      self.seq_lens if seq_lens is None else seq_lens)

    def decode(self, l, partition_tokens=0, seq_lens=None, out=None):
        return ops.pa_decode(self.inputs[l]["q"], self.k_pool, self.v_pool, self.bt[l],
                             self.seq_lens if seq_lens is None else seq_lens, self.lay.scale,
                             out=out, partition_tokens=partition_tokens)


def oracle_sequence(d: Device, l: int, b: int, k_pages=None, v_pages=None):
    """FP64 oracle output [32][64] for sequence b of layer l, from host copies of
    its pages taken before the append (the oracle applies the append itself)."""
    lay = d.lay
    if k_pages is None:
        k_pages, v_pages, _ = synth.sequence_pages(d.k_pool, d.v_pool, lay, l, b)
    n = k_pages.shape[0]
    bt = np.arange(max(n, 1), dtype=np.int32)[None]
    L = np.array([lay.seq_lens[b]], np.int32)
    x = d.inputs[l]
    k2, v2 = append_ref(k_pages, v_pages, synth.bits(x["k_new"][b:b + 1]), synth.bits(x["v_new"][b:b + 1]), bt, L)
    q = synth.bits(x["q"][b:b + 1])
    return decode_ref(q, k2, v2, bt, L, lay.scale)[0]
