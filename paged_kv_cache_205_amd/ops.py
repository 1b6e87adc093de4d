"""Thin ctypes binding over libpa.so (the C ABI of include/pa.h).

Argument marshalling only: torch tensors become device pointers and the current
HIP stream becomes the ``hipStream_t``; every step of the computation runs in
the library's kernels.  If the library is missing the calls raise; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK = 0
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
          -4: "PA_ERR_WORKSPACE", -5: "PA_ERR_LAUNCH", -6: "PA_ERR_ALIGN", -7: "PA_ERR_REJECTED",
          -8: "PA_ERR_BUDGET", -9: "PA_ERR_STATE", -10: "PA_ERR_SCRATCH"}
EXPORTS = ("pa_status_string", "pa_append", "pa_rope_append", "pa_fill", "pa_prefill", "pa_decode_workspace_bytes",
           "pa_default_partition_tokens", "pa_decode", "pa_append_decode", "pa_rope_append_decode",
           "pa_append_decode_noalloc", "pa_decode_plan_bytes", "pa_decode_plan", "pa_decode_planned", "pa_merge",
           "pa_sched_budget_pages", "pa_sched_create", "pa_sched_destroy", "pa_sched_submit", "pa_sched_admit",
           "pa_sched_grow", "pa_sched_block_table", "pa_sched_finish", "pa_sched_decode_batch",
           "pa_sched_get_stats")

_lib = None


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} returned {status} ({text})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with paged_kv_cache_205_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_append.argtypes = [P, P, P, P, P, I32, P, I32, I32, I32, I64, P]
    lib.pa_append.restype = ctypes.c_int
    lib.pa_fill.argtypes = [P, P, P, P, P, I32, P, P, I32, I64, I32, I32, I64, P]
    lib.pa_rope_append.argtypes = [P, P, P, P, I32, P, P, P, P, I32, P, I32, I32, I32, I32, I64, P]
    lib.pa_rope_append.restype = ctypes.c_int
    lib.pa_fill.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [P, P, P, P, I32, I64, I32, I32, I32, F32, I32, P, P]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.pa_decode_workspace_bytes.restype = SZ
    lib.pa_default_partition_tokens.argtypes = []
    lib.pa_default_partition_tokens.restype = I32
    lib.pa_decode.argtypes = [P, P, P, P, I32, P, F32, P, I32, I32, I32, I32, I64, I32, P, SZ, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_append_decode.argtypes = [P, P, P, P, P, P, I32, P, F32, P, I32, I32, I32, I32, I64, I32, P, SZ, P]
    lib.pa_append_decode.restype = ctypes.c_int
    lib.pa_rope_append_decode.argtypes = [P, P, P, P, P, P, I32, P, I32, P, F32, P, I32, I32, I32, I32, I64, I32, P,
                                          SZ, P]
    lib.pa_rope_append_decode.restype = ctypes.c_int
    lib.pa_append_decode_noalloc.argtypes = [P, P, P, P, P, P, I32, P, F32, P, I32, I32, I32, I32, I64, I32, P]
    lib.pa_append_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_plan_bytes.argtypes = [I32, I32, I32]
    lib.pa_decode_plan_bytes.restype = SZ
    lib.pa_decode_plan.argtypes = [P, I32, I32, I32, P, SZ, P]
    lib.pa_decode_plan.restype = ctypes.c_int
    lib.pa_decode_planned.argtypes = [P, P, P, P, I32, P, P, P, I32, F32, P, I32, I32, I32, I32, I64, I32, P, SZ, P,
                                      SZ, P]
    lib.pa_decode_planned.restype = ctypes.c_int
    lib.pa_merge.argtypes = [P, P, P, P, I32, P, I32, I32, I32, I32, P]
    lib.pa_merge.restype = ctypes.c_int
    lib.pa_sched_budget_pages.argtypes = [I32, I32, I32, I32, ctypes.POINTER(I64)]
    lib.pa_sched_budget_pages.restype = ctypes.c_int
    lib.pa_sched_create.argtypes = [I64, I32, I32, I32, ctypes.POINTER(P)]
    lib.pa_sched_create.restype = ctypes.c_int
    lib.pa_sched_destroy.argtypes = [P]
    lib.pa_sched_destroy.restype = None
    lib.pa_sched_submit.argtypes = [P, I32, I32, ctypes.POINTER(I64)]
    lib.pa_sched_submit.restype = ctypes.c_int
    lib.pa_sched_admit.argtypes = [P, ctypes.POINTER(I64), I32, ctypes.POINTER(I32)]
    lib.pa_sched_admit.restype = ctypes.c_int
    lib.pa_sched_grow.argtypes = [P, I64, I32]
    lib.pa_sched_grow.restype = ctypes.c_int
    lib.pa_sched_block_table.argtypes = [P, I64, I32, ctypes.POINTER(I32), I32]
    lib.pa_sched_block_table.restype = ctypes.c_int
    lib.pa_sched_finish.argtypes = [P, I64]
    lib.pa_sched_finish.restype = ctypes.c_int
    lib.pa_sched_decode_batch.argtypes = [P, I32]
    lib.pa_sched_decode_batch.restype = ctypes.c_int
    lib.pa_sched_get_stats.argtypes = [P, ctypes.POINTER(SchedStats)]
    lib.pa_sched_get_stats.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(fn, status, load().pa_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor], dtype, name: str) -> Optional[int]:
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(dev: torch.device, stream):
    """The launch stream as a torch stream object (the current one when None)."""
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=dev)


def _decode_buffers(q, block_table, partition_tokens, out, workspace, stream):
    """out and workspace for a decode call, allocated (and the workspace zero-filled)
    on the launch stream when the caller passes none, so that the fill is ordered
    before the kernel and the caching allocator recycles the blocks only after
    work on that stream.  (Every binding that allocates an output does so on the
    launch stream for the same reason.)"""
    B, Hq, D = q.shape
    if out is not None and workspace is not None:
        return out, workspace
    if q.device.type != "cuda":
        raise ValueError("q must be a device tensor")
    with torch.cuda.stream(_torch_stream(q.device, stream)):
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = workspace_for(B, block_table.shape[1], partition_tokens, q.device)
    return out, workspace


def _bf16(t, name):
    return _ptr(t, torch.bfloat16, name)


def pa_append(k_new, v_new, k_pool, v_pool, block_table, seq_lens, stream=None) -> None:
    """k_new/v_new bf16 [B][8][64]; pools bf16 [num_pages][16][8][64]; block_table int32 [B][max_blocks]."""
    B, Hkv, D = k_new.shape
    lib = load()
    st = lib.pa_append(_bf16(k_new, "k_new"), _bf16(v_new, "v_new"), _bf16(k_pool, "k_pool"),
                       _bf16(v_pool, "v_pool"), _ptr(block_table, torch.int32, "block_table"),
                       block_table.shape[1], _ptr(seq_lens, torch.int32, "seq_lens"), B, Hkv, D,
                       k_pool.shape[0], _stream(k_pool.device, stream))
    _check("pa_append", st)


def pa_rope_append(q, k_new, v_new, cos_sin, k_pool, v_pool, block_table, seq_lens, q_out=None,
                   stream=None) -> torch.Tensor:
    """RoPE of q and k_new at position seq_lens - 1 (cos_sin fp32 [max_pos][64]: 32 cosines then 32
    sines), then the append of the rotated key and the value; returns q_out bf16 [B][32][64]."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if q_out is None:
        with torch.cuda.stream(_torch_stream(q.device, stream)):
            q_out = torch.empty_like(q)
    lib = load()
    st = lib.pa_rope_append(_bf16(q, "q"), _bf16(k_new, "k_new"), _bf16(v_new, "v_new"),
                            _ptr(cos_sin, torch.float32, "cos_sin"), cos_sin.shape[0], _bf16(q_out, "q_out"),
                            _bf16(k_pool, "k_pool"), _bf16(v_pool, "v_pool"), _ptr(block_table, torch.int32, "block_table"),
                            block_table.shape[1], _ptr(seq_lens, torch.int32, "seq_lens"), B, Hq, Hkv, D,
                            k_pool.shape[0], _stream(q.device, stream))
    _check("pa_rope_append", st)
    return q_out


def pa_fill(k_src, v_src, k_pool, v_pool, block_table, cu_tokens, start=None, stream=None) -> None:
    """k_src/v_src bf16 [T][8][64] (runs one after another); cu_tokens int32 [B+1] on the device,
    with T = cu_tokens[B] (the host's T is the rows of k_src); start int32 [B] or None (all 0)."""
    T, Hkv, D = k_src.shape
    B = cu_tokens.shape[0] - 1
    lib = load()
    st = lib.pa_fill(_bf16(k_src, "k_src"), _bf16(v_src, "v_src"), _bf16(k_pool, "k_pool"), _bf16(v_pool, "v_pool"),
                     _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
                     _ptr(start, torch.int32, "start"), _ptr(cu_tokens, torch.int32, "cu_tokens"), B, T, Hkv, D,
                     k_pool.shape[0], _stream(k_pool.device, stream))
    _check("pa_fill", st)


PREFILL_WEIGHTS = {"bf16x2": 0, "fp16": 1}


def pa_prefill(q, k, v, cu_tokens, scale: float, out=None, weights: str = "bf16x2", stream=None) -> torch.Tensor:
    """Causal attention of each prompt over its own rows: q bf16 [T][32][64], k/v bf16 [T][8][64]
    (prompts one after another), cu_tokens int32 [B+1] on the device -> out fp32 [T][32][64].
    weights: "bf16x2" (each weight as a bf16 pair, 2^-16) or "fp16" (fp16 weights and V, 2^-11)."""
    if weights not in PREFILL_WEIGHTS:
        raise ValueError(f"weights must be one of {sorted(PREFILL_WEIGHTS)}")
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    B = cu_tokens.shape[0] - 1
    if k.shape[0] != T or v.shape != k.shape:
        raise PAError("pa_prefill", -2, "q, k and v must have the same rows, k and v the same shape")
    if out is None:
        with torch.cuda.stream(_torch_stream(q.device, stream)):
            out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (T, Hq, D):
        raise PAError("pa_prefill", -2, f"out must be [{T}][{Hq}][{D}]")
    lib = load()
    st = lib.pa_prefill(_bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _ptr(cu_tokens, torch.int32, "cu_tokens"), B, T,
                        Hq, Hkv, D, float(scale), PREFILL_WEIGHTS[weights], _ptr(out, torch.float32, "out"),
                        _stream(q.device, stream))
    _check("pa_prefill", st)
    return out


def pa_decode_workspace_bytes(B: int, max_blocks: int, partition_tokens: int = 0, Hq: int = 32, D: int = 64) -> int:
    return int(load().pa_decode_workspace_bytes(B, Hq, D, max_blocks, partition_tokens))


def pa_default_partition_tokens() -> int:
    return int(load().pa_default_partition_tokens())


def workspace_for(B: int, max_blocks: int, partition_tokens: int = 0, device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled workspace for pa_decode / pa_append_decode (None when none is needed),
    allocated and filled on the current stream."""
    n = pa_decode_workspace_bytes(B, max_blocks, partition_tokens)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def pa_decode(q, k_pool, v_pool, block_table, seq_lens, scale: float, out=None,
              partition_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
    """q bf16 [B][32][64] -> out fp32 [B][32][64] (allocated if not given)."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    out, workspace = _decode_buffers(q, block_table, partition_tokens, out, workspace, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib = load()
    st = lib.pa_decode(_bf16(q, "q"), _bf16(k_pool, "k_pool"), _bf16(v_pool, "v_pool"),
                       _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
                       _ptr(seq_lens, torch.int32, "seq_lens"), float(scale),
                       _ptr(out, torch.float32, "out"), B, Hq, Hkv, D, k_pool.shape[0],
                       partition_tokens, ws_ptr, ws_n, _stream(q.device, stream))
    _check("pa_decode", st)
    return out


def pa_append_decode(k_new, v_new, k_pool, v_pool, q, block_table, seq_lens, scale: float, out=None,
                     partition_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
    """pa_append then pa_decode in one launch; returns out fp32 [B][32][64]."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    out, workspace = _decode_buffers(q, block_table, partition_tokens, out, workspace, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib = load()
    st = lib.pa_append_decode(_bf16(k_new, "k_new"), _bf16(v_new, "v_new"), _bf16(k_pool, "k_pool"),
                              _bf16(v_pool, "v_pool"), _bf16(q, "q"), _ptr(block_table, torch.int32, "block_table"),
                              block_table.shape[1], _ptr(seq_lens, torch.int32, "seq_lens"), float(scale),
                              _ptr(out, torch.float32, "out"), B, Hq, Hkv, D, k_pool.shape[0],
                              partition_tokens, ws_ptr, ws_n, _stream(q.device, stream))
    _check("pa_append_decode", st)
    return out


def pa_rope_append_decode(k_new, v_new, k_pool, v_pool, q, cos_sin, block_table, seq_lens, scale: float, out=None,
                          partition_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
    """RoPE of q and k_new at position L-1, the append and the decode in one launch; returns out fp32 [B][32][64]."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    out, workspace = _decode_buffers(q, block_table, partition_tokens, out, workspace, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib = load()
    st = lib.pa_rope_append_decode(_bf16(k_new, "k_new"), _bf16(v_new, "v_new"), _bf16(k_pool, "k_pool"),
                                   _bf16(v_pool, "v_pool"), _bf16(q, "q"), _ptr(cos_sin, torch.float32, "cos_sin"),
                                   cos_sin.shape[0], _ptr(block_table, torch.int32, "block_table"),
                                   block_table.shape[1], _ptr(seq_lens, torch.int32, "seq_lens"), float(scale),
                                   _ptr(out, torch.float32, "out"), B, Hq, Hkv, D, k_pool.shape[0],
                                   partition_tokens, ws_ptr, ws_n, _stream(q.device, stream))
    _check("pa_rope_append_decode", st)
    return out


def pa_decode_plan_bytes(B: int, max_blocks: int, partition_tokens: int = 0) -> int:
    return int(load().pa_decode_plan_bytes(B, max_blocks, partition_tokens))


def pa_decode_plan(seq_lens, max_blocks: int, partition_tokens: int = 0, plan=None, stream=None) -> torch.Tensor:
    """The work plan of one decode step (seq_lens int32 [B] on the device), for every
    layer's pa_decode_planned call of that step; returns the plan buffer (uint8)."""
    B = seq_lens.shape[0]
    if plan is None:
        with torch.cuda.stream(_torch_stream(seq_lens.device, stream)):
            plan = torch.empty(max(pa_decode_plan_bytes(B, max_blocks, partition_tokens), 16), dtype=torch.uint8,
                               device=seq_lens.device)
    st = load().pa_decode_plan(_ptr(seq_lens, torch.int32, "seq_lens"), B, max_blocks, partition_tokens,
                               _ptr(plan, torch.uint8, "plan"), plan.numel(), _stream(seq_lens.device, stream))
    _check("pa_decode_plan", st)
    return plan


def pa_decode_planned(q, k_pool, v_pool, block_table, plan, scale: float, k_new=None, v_new=None, cos_sin=None,
                      out=None, partition_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
    """Decode (with the append when k_new / v_new are given, and RoPE when cos_sin is)
    from a plan of pa_decode_plan; returns out fp32 [B][32][64]."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    out, workspace = _decode_buffers(q, block_table, partition_tokens, out, workspace, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().pa_decode_planned(_bf16(q, "q"), _bf16(k_new, "k_new"), _bf16(v_new, "v_new"),
                                  _ptr(cos_sin, torch.float32, "cos_sin"),
                                  cos_sin.shape[0] if cos_sin is not None else 0, _bf16(k_pool, "k_pool"),
                                  _bf16(v_pool, "v_pool"), _ptr(block_table, torch.int32, "block_table"),
                                  block_table.shape[1], float(scale), _ptr(out, torch.float32, "out"), B, Hq, Hkv, D,
                                  k_pool.shape[0], partition_tokens, _ptr(plan, torch.uint8, "plan"), plan.numel(),
                                  ws_ptr, ws_n, _stream(q.device, stream))
    _check("pa_decode_planned", st)
    return out


def pa_append_decode_noalloc(k_new, v_new, k_pool, v_pool, q, block_table, seq_lens, scale: float, out,
                             partition_tokens: int = 0, stream=None) -> torch.Tensor:
    """pa_append_decode without a workspace (the library's fixed per-GPU scratch array).
    out fp32 [B][32][64] must be given: this call allocates nothing."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    lib = load()
    st = lib.pa_append_decode_noalloc(_bf16(k_new, "k_new"), _bf16(v_new, "v_new"), _bf16(k_pool, "k_pool"),
                                      _bf16(v_pool, "v_pool"), _bf16(q, "q"),
                                      _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
                                      _ptr(seq_lens, torch.int32, "seq_lens"), float(scale),
                                      _ptr(out, torch.float32, "out"), B, Hq, Hkv, D, k_pool.shape[0],
                                      partition_tokens, _stream(q.device, stream))
    _check("pa_append_decode_noalloc", st)
    return out


def pa_merge(part_o, part_m, part_l, seq_lens=None, partition_tokens: int = 0, out=None, stream=None):
    """part_o fp32 [B][32][S][64], part_m / part_l fp32 [B][32][S] (base-2 maxima) -> out fp32 [B][32][64]."""
    B, Hq, S, D = part_o.shape
    if out is None:
        with torch.cuda.stream(_torch_stream(part_o.device, stream)):
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=part_o.device)
    lib = load()
    st = lib.pa_merge(_ptr(part_o, torch.float32, "part_o"), _ptr(part_m, torch.float32, "part_m"),
                      _ptr(part_l, torch.float32, "part_l"),
                      _ptr(seq_lens, torch.int32, "seq_lens") if seq_lens is not None else None,
                      partition_tokens, _ptr(out, torch.float32, "out"), B, Hq, D, S,
                      _stream(part_o.device, stream))
    _check("pa_merge", st)
    return out


# ----------------------------------------------------------------------------
# page-budget admission and lazy page assignment (include/pa_sched.h; host only)


class SchedStats(ctypes.Structure):
    _fields_ = [("pool_pages", ctypes.c_int64), ("free_pages", ctypes.c_int64), ("assigned_pages", ctypes.c_int64),
                ("peak_assigned_pages", ctypes.c_int64), ("credits_free", ctypes.c_int64),
                ("active", ctypes.c_int32), ("waiting", ctypes.c_int32), ("peak_active", ctypes.c_int32),
                ("largest_decode_batch", ctypes.c_int32), ("admission_waits", ctypes.c_int64),
                ("rejected", ctypes.c_int64), ("completed", ctypes.c_int64)]


def sched_budget_pages(prompt_tokens: int, max_new_tokens: int, context: int = 2048, n_layers: int = 16) -> int:
    out = ctypes.c_int64()
    _check("pa_sched_budget_pages", load().pa_sched_budget_pages(prompt_tokens, max_new_tokens, context, n_layers,
                                                                 ctypes.byref(out)))
    return out.value


class Scheduler:
    """Thin owner of a pa_sched object: arguments are passed through as they are."""

    def __init__(self, pool_pages: int, n_layers: int = 16, context: int = 2048, static: bool = False):
        self._h = None
        self._lib = load()
        h = ctypes.c_void_p()
        _check("pa_sched_create", self._lib.pa_sched_create(pool_pages, n_layers, context, int(static), ctypes.byref(h)))
        self._h = h
        self.n_layers = n_layers

    def close(self) -> None:
        if self._h:
            self._lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def submit(self, prompt_tokens: int, max_new_tokens: int) -> Optional[int]:
        """The request id, or None when its budget exceeds the whole pool (rejected)."""
        rid = ctypes.c_int64()
        st = self._lib.pa_sched_submit(self._h, prompt_tokens, max_new_tokens, ctypes.byref(rid))
        if st == -7:
            return None
        _check("pa_sched_submit", st)
        return rid.value

    def admit(self, capacity: int = 1 << 16):
        ids = (ctypes.c_int64 * max(capacity, 1))()
        n = ctypes.c_int32()
        _check("pa_sched_admit", self._lib.pa_sched_admit(self._h, ids, capacity, ctypes.byref(n)))
        return [ids[i] for i in range(n.value)]

    def grow(self, rid: int, new_length: int) -> bool:
        """False when new_length is beyond the request's budget (nothing assigned)."""
        st = self._lib.pa_sched_grow(self._h, rid, new_length)
        if st == -8:
            return False
        _check("pa_sched_grow", st)
        return True

    def block_table(self, rid: int, layer: int, max_blocks: int):
        import numpy as np
        row = np.empty(max_blocks, np.int32)
        _check("pa_sched_block_table", self._lib.pa_sched_block_table(
            self._h, rid, layer, row.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), max_blocks))
        return row

    def finish(self, rid: int) -> None:
        _check("pa_sched_finish", self._lib.pa_sched_finish(self._h, rid))

    def decode_batch(self, n: int) -> None:
        _check("pa_sched_decode_batch", self._lib.pa_sched_decode_batch(self._h, n))

    def stats(self) -> dict:
        st = SchedStats()
        _check("pa_sched_get_stats", self._lib.pa_sched_get_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in SchedStats._fields_}
