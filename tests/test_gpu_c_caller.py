"""The library driven from plain C on the GPU (C11, gcc, include/pa.h,
hipMalloc'd buffers, the default stream).  tests/c/gpu_append_decode.c calls
pa_append_decode under the automatic split and under one page per split, then
the same through a plan (pa_decode_plan, pa_decode_planned) and through the
allocation-free entry point (pa_append_decode_noalloc): the pools must equal
the oracle's append bit for bit, every output must match the FP64 decode of the
appended pools, and each planned or allocation-free output must equal the
unplanned one of the same split bit for bit.  tests/c/gpu_prefill.c fills three packed prompts
into their pages with pa_fill and runs pa_prefill in both weight modes: the
pools must equal the oracle's fill bit for bit and the outputs must match the
FP64 prefill (fp16 weights to their bound)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import append_ref, decode_ref, fill_ref, prefill_ref
from paged_kv_cache_205_amd import ops
from tests.helpers import check_close, say
from tests.test_gpu_prefill import check_fp16_weights, v_spread

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
B, HQ, HKV, D, MAXB, PAGES, PT = 3, 32, 8, 64, 4, 12, 16


def read_dump(path):
    raw = open(path, "rb").read()
    pos = 0

    def take(dtype, shape):
        nonlocal pos
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        a = np.frombuffer(raw, dtype=dtype, count=int(np.prod(shape)), offset=pos).reshape(shape)
        pos += n
        return a

    d = dict(q=take(np.uint16, (B, HQ, D)), k_new=take(np.uint16, (B, HKV, D)), v_new=take(np.uint16, (B, HKV, D)),
             bt=take(np.int32, (B, MAXB)), lens=take(np.int32, (B,)),
             kp=take(np.uint16, (PAGES, PT, HKV, D)), vp=take(np.uint16, (PAGES, PT, HKV, D)),
             kp_after=take(np.uint16, (PAGES, PT, HKV, D)), vp_after=take(np.uint16, (PAGES, PT, HKV, D)),
             out=take(np.float32, (6, B, HQ, D)))
    assert pos == len(raw), f"dump holds {len(raw)} bytes, expected {pos}"
    return d


def build_and_run(tmp_path, name):
    """Compile tests/c/<name>.c against libpa.so with gcc, run it, return its dump's path."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load()  # raises if libpa.so is missing
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe, dump = str(tmp_path / name), str(tmp_path / f"{name}.bin")
    libdir = os.path.dirname(ops.LIB_PATH)
    cmd = [gcc, "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", f"{name}.c"),
           "-L", libdir, "-lpa", "-L", "/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe, dump], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, f"exit {run.returncode}: {run.stderr}"
    return dump


def test_c_program_drives_append_decode(tmp_path):
    say("C caller: pa_append_decode, the planned decode and the allocation-free call, two split sizes")
    dump = build_and_run(tmp_path, "gpu_append_decode")
    d = read_dump(dump)
    k_ref, v_ref = append_ref(d["kp"], d["vp"], d["k_new"], d["v_new"], d["bt"], d["lens"])
    assert np.array_equal(d["kp_after"], k_ref), "K pool after the C calls differs from the oracle's append"
    assert np.array_equal(d["vp_after"], v_ref), "V pool after the C calls differs from the oracle's append"
    ref = decode_ref(d["q"], k_ref, v_ref, d["bt"], d["lens"], 0.125)
    names = ("automatic", "one page", "planned automatic", "planned one page", "allocation-free automatic",
             "allocation-free one page")
    for c, part in enumerate(names):
        check_close(d["out"][c], ref, f"C caller, {part} split")
    for c in range(2, 6):
        assert np.array_equal(d["out"][c].view(np.uint32), d["out"][c % 2].view(np.uint32)), \
            f"{names[c]} output differs from the unplanned one"


def test_c_program_drives_fill_and_prefill(tmp_path):
    say("C caller: pa_fill and pa_prefill in both weight modes")
    dump = build_and_run(tmp_path, "gpu_prefill")
    T, MB, NP = 111, 8, 16
    raw = open(dump, "rb").read()
    pos = 0

    def take(dtype, shape):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=int(np.prod(shape)), offset=pos).reshape(shape)
        pos += a.nbytes
        return a

    q, k, v = take(np.uint16, (T, HQ, D)), take(np.uint16, (T, HKV, D)), take(np.uint16, (T, HKV, D))
    bt, cu = take(np.int32, (3, MB)), take(np.int32, (4,))
    kp, vp = take(np.uint16, (NP, PT, HKV, D)), take(np.uint16, (NP, PT, HKV, D))
    kp_after, vp_after = take(np.uint16, (NP, PT, HKV, D)), take(np.uint16, (NP, PT, HKV, D))
    out = take(np.float32, (2, T, HQ, D))
    assert pos == len(raw), f"dump holds {len(raw)} bytes, expected {pos}"
    k_ref, v_ref = fill_ref(kp, vp, k, v, bt, None, cu)
    assert np.array_equal(kp_after, k_ref), "K pool after pa_fill differs from the oracle's fill"
    assert np.array_equal(vp_after, v_ref), "V pool after pa_fill differs from the oracle's fill"
    ref = prefill_ref(q, k, v, cu, 0.125)
    check_close(out[0], ref, "C caller, prefill with bf16-pair weights")
    check_fp16_weights(out[1], ref, v_spread(v, cu), "C caller, prefill with fp16 weights")
