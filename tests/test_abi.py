"""The C-ABI library loads, exports every symbol pa.h declares, and rejects bad
arguments on the host before launching anything (no GPU needed: each call below
fails a host-side check, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_205_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("pa.h", "pa_sched.h")]

# Fake device addresses: 256-byte aligned, never dereferenced because every call
# in this file is rejected by a host-side check first.
A = 0x10000
MIS = A + 8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libpa.so not built (run __graft_entry__.build())")
    return ops.load()


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(ops.EXPORTS), names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {ops.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings(lib):
    for code, name in ops.STATUS.items():
        assert lib.pa_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.pa_status_string(-99)


def test_default_partition_and_workspace_sizes(lib):
    assert lib.pa_default_partition_tokens() == 0  # automatic split size
    # single split: no partials, only the (sequence, KV head) counters and the queue counter
    assert lib.pa_decode_workspace_bytes(64, 32, 64, 128, 2048) == 64 * 8 * 4 + 256
    assert lib.pa_decode_workspace_bytes(512, 32, 64, 8, 0) == 512 * 8 * 4 + 256  # automatic splits have >= 8 pages
    # automatic: partial rows for up to ceil(128 / 4) = 32 splits for up to 64 sequences, ceil(128 / 8) = 16 above
    assert lib.pa_decode_workspace_bytes(64, 32, 64, 128, 0) == lib.pa_decode_workspace_bytes(64, 32, 64, 128, 64)
    assert lib.pa_decode_workspace_bytes(65, 32, 64, 128, 0) == lib.pa_decode_workspace_bytes(65, 32, 64, 128, 128)
    assert lib.pa_decode_workspace_bytes(5000, 32, 64, 128, 0) == 0  # batch above the plan limit
    # 8 splits of 256 tokens: part_o + part_m + part_l + one counter per (sequence, KV head) + the
    # queue, each padded to 256 bytes
    rows = 64 * 32 * 8
    want = rows * 64 * 4 + 2 * (((rows * 4) + 255) // 256 * 256) + 64 * 8 * 4 + 256
    assert lib.pa_decode_workspace_bytes(64, 32, 64, 128, 256) == want
    # partitions above 2048 tokens act as 2048
    assert lib.pa_decode_workspace_bytes(4, 32, 64, 256, 4096) == lib.pa_decode_workspace_bytes(4, 32, 64, 256, 2048) > 0
    # invalid sizes report 0
    assert lib.pa_decode_workspace_bytes(64, 32, 64, 128, 24) == 0
    assert lib.pa_decode_workspace_bytes(0, 32, 64, 128, 256) == 0
    assert lib.pa_decode_workspace_bytes(64, 16, 64, 128, 256) == 0


def _append(lib, **kw):
    args = dict(k_new=A, v_new=A, k_pool=A, v_pool=A, bt=A, max_blocks=128, seq_lens=A, B=4,
                Hkv=8, D=64, num_pages=1024, stream=None)
    args.update(kw)
    return lib.pa_append(args["k_new"], args["v_new"], args["k_pool"], args["v_pool"], args["bt"],
                         args["max_blocks"], args["seq_lens"], args["B"], args["Hkv"], args["D"],
                         args["num_pages"], args["stream"])


def test_append_validation(lib):
    assert _append(lib, k_new=None) == -1
    assert _append(lib, seq_lens=None) == -1
    assert _append(lib, bt=None) == -1
    assert _append(lib, B=-1) == -2
    assert _append(lib, max_blocks=0) == -2
    assert _append(lib, max_blocks=5000) == -2
    assert _append(lib, num_pages=0) == -2
    assert _append(lib, num_pages=1 << 40) == -2
    assert _append(lib, Hkv=4) == -3
    assert _append(lib, D=128) == -3
    assert _append(lib, k_pool=MIS) == -6
    assert _append(lib, B=0) == 0  # empty batch: nothing launched


def _decode(lib, **kw):
    args = dict(q=A, k=A, v=A, bt=A, max_blocks=128, sl=A, scale=0.125, out=A, B=4, Hq=32, Hkv=8,
                D=64, num_pages=1024, part=256, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    return lib.pa_decode(args["q"], args["k"], args["v"], args["bt"], args["max_blocks"], args["sl"],
                         args["scale"], args["out"], args["B"], args["Hq"], args["Hkv"], args["D"],
                         args["num_pages"], args["part"], args["ws"], args["ws_bytes"], args["stream"])


def test_decode_validation(lib):
    need = lib.pa_decode_workspace_bytes(4, 32, 64, 128, 256)
    assert need > 0
    assert _decode(lib, q=None) == -1
    assert _decode(lib, out=None) == -1
    assert _decode(lib, sl=None) == -1
    assert _decode(lib, B=-3) == -2
    assert _decode(lib, part=24) == -2
    assert _decode(lib, part=-16) == -2
    assert _decode(lib, scale=float("nan")) == -2
    assert _decode(lib, scale=float("inf")) == -2
    assert _decode(lib, max_blocks=0) == -2
    assert _decode(lib, Hq=30) == -2  # not a multiple of Hkv
    assert _decode(lib, Hq=16) == -3
    assert _decode(lib, Hkv=4, Hq=16) == -3
    assert _decode(lib, D=128) == -3
    assert _decode(lib, ws=None, ws_bytes=0) == -4
    assert _decode(lib, ws=A, ws_bytes=need - 1) == -4
    assert _decode(lib, ws=MIS, ws_bytes=need) == -6
    assert _decode(lib, q=MIS, ws=A, ws_bytes=need) == -6
    assert _decode(lib, B=0) == 0
    assert _decode(lib, B=4097) == -2


def _append_decode(lib, **kw):
    args = dict(kn=A, vn=A, k=A, v=A, q=A, bt=A, max_blocks=128, sl=A, scale=0.125, out=A, B=4, Hq=32,
                Hkv=8, D=64, num_pages=1024, part=256, ws=A, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.pa_append_decode(args["kn"], args["vn"], args["k"], args["v"], args["q"], args["bt"],
                                args["max_blocks"], args["sl"], args["scale"], args["out"], args["B"],
                                args["Hq"], args["Hkv"], args["D"], args["num_pages"], args["part"],
                                args["ws"], args["ws_bytes"], args["stream"])


def test_append_decode_validation(lib):
    assert _append_decode(lib, kn=None) == -1
    assert _append_decode(lib, vn=None) == -1
    assert _append_decode(lib, q=None) == -1
    assert _append_decode(lib, kn=MIS) == -6
    assert _append_decode(lib, part=40) == -2
    assert _append_decode(lib, D=32) == -3
    assert _append_decode(lib, ws=None, ws_bytes=0) == -4
    assert _append_decode(lib, B=0) == 0


def _merge(lib, **kw):
    args = dict(o=A, m=A, l=A, sl=A, part=256, out=A, B=4, Hq=32, D=64, S=8, stream=None)
    args.update(kw)
    return lib.pa_merge(args["o"], args["m"], args["l"], args["sl"], args["part"], args["out"],
                        args["B"], args["Hq"], args["D"], args["S"], args["stream"])


def test_merge_validation(lib):
    assert _merge(lib, o=None) == -1
    assert _merge(lib, out=None) == -1
    assert _merge(lib, S=0) == -2
    assert _merge(lib, part=0) == -2
    assert _merge(lib, part=20) == -2
    assert _merge(lib, D=32) == -3
    assert _merge(lib, o=MIS) == -6
    assert _merge(lib, B=0) == 0


def test_binding_requires_device_tensors(lib):
    import torch
    x = torch.zeros(2, 32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.pa_decode(x, torch.zeros(1, 16, 8, 64, dtype=torch.bfloat16),
                      torch.zeros(1, 16, 8, 64, dtype=torch.bfloat16), torch.zeros(2, 1, dtype=torch.int32),
                      torch.zeros(2, dtype=torch.int32), 0.125, out=torch.zeros(2, 32, 64))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "libpa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ops.load()


def _fill(lib, **kw):
    args = dict(ks=A, vs=A, k=A, v=A, bt=A, max_blocks=128, start=None, cu=A, B=4, T=100, Hkv=8, D=64,
                num_pages=1024, stream=None)
    args.update(kw)
    return lib.pa_fill(args["ks"], args["vs"], args["k"], args["v"], args["bt"], args["max_blocks"], args["start"],
                       args["cu"], args["B"], args["T"], args["Hkv"], args["D"], args["num_pages"], args["stream"])


def test_fill_validation(lib):
    assert _fill(lib, B=-1) == -2
    assert _fill(lib, B=4097) == -2
    assert _fill(lib, T=-1) == -2
    assert _fill(lib, T=1 << 31) == -2
    assert _fill(lib, max_blocks=0) == -2
    assert _fill(lib, max_blocks=4097) == -2
    assert _fill(lib, num_pages=0) == -2
    assert _fill(lib, Hkv=4) == -3
    assert _fill(lib, D=128) == -3
    assert _fill(lib, ks=None) == -1
    assert _fill(lib, cu=None) == -1
    assert _fill(lib, bt=None) == -1
    assert _fill(lib, ks=MIS) == -6
    assert _fill(lib, v=MIS) == -6
    # nothing to do: no launch
    assert _fill(lib, B=0) == 0
    assert _fill(lib, T=0) == 0
    assert _fill(lib, B=0, ks=None, cu=None) == 0


def _prefill(lib, **kw):
    args = dict(q=A, k=A, v=A, cu=A, B=4, T=100, Hq=32, Hkv=8, D=64, scale=0.125, weights=0, out=A, stream=None)
    args.update(kw)
    return lib.pa_prefill(args["q"], args["k"], args["v"], args["cu"], args["B"], args["T"], args["Hq"], args["Hkv"],
                          args["D"], args["scale"], args["weights"], args["out"], args["stream"])


def test_prefill_validation(lib):
    assert _prefill(lib, B=0) == -2
    assert _prefill(lib, B=-1) == -2
    assert _prefill(lib, B=4097) == -2
    assert _prefill(lib, T=-1) == -2
    assert _prefill(lib, T=(1 << 30) + 1) == -2
    assert _prefill(lib, Hq=30) == -2
    assert _prefill(lib, Hq=16, Hkv=4) == -3
    assert _prefill(lib, D=128) == -3
    assert _prefill(lib, scale=float("inf")) == -2
    assert _prefill(lib, scale=float("nan")) == -2
    assert _prefill(lib, weights=2) == -2
    assert _prefill(lib, weights=-1) == -2
    assert _prefill(lib, q=None) == -1
    assert _prefill(lib, cu=None) == -1
    assert _prefill(lib, out=None) == -1
    assert _prefill(lib, k=MIS) == -6
    assert _prefill(lib, out=MIS) == -6
    # nothing to do: no launch
    assert _prefill(lib, T=0) == 0
    assert _prefill(lib, T=0, q=None, out=None) == 0


def _rope(lib, **kw):
    args = dict(q=A, k_new=A, v_new=A, cs=A, max_pos=2048, q_out=A, k=A, v=A, bt=A, max_blocks=128, sl=A, B=4,
                Hq=32, Hkv=8, D=64, num_pages=1024, stream=None)
    args.update(kw)
    return lib.pa_rope_append(args["q"], args["k_new"], args["v_new"], args["cs"], args["max_pos"], args["q_out"],
                              args["k"], args["v"], args["bt"], args["max_blocks"], args["sl"], args["B"], args["Hq"],
                              args["Hkv"], args["D"], args["num_pages"], args["stream"])


def test_rope_append_validation(lib):
    assert _rope(lib, B=-1) == -2
    assert _rope(lib, B=4097) == -2
    assert _rope(lib, max_pos=0) == -2
    assert _rope(lib, max_blocks=0) == -2
    assert _rope(lib, max_blocks=4097) == -2
    assert _rope(lib, num_pages=0) == -2
    assert _rope(lib, num_pages=1 << 31) == -2
    assert _rope(lib, Hq=30) == -2
    assert _rope(lib, Hkv=4, Hq=16) == -3
    assert _rope(lib, D=128) == -3
    assert _rope(lib, q=None) == -1
    assert _rope(lib, cs=None) == -1
    assert _rope(lib, q_out=None) == -1
    assert _rope(lib, sl=None) == -1
    assert _rope(lib, cs=MIS) == -6
    assert _rope(lib, q_out=MIS) == -6
    assert _rope(lib, v=MIS) == -6
    # nothing to do: no launch
    assert _rope(lib, B=0) == 0
    assert _rope(lib, B=0, q=None, cs=None) == 0


def _rope_decode(lib, **kw):
    args = dict(k_new=A, v_new=A, k=A, v=A, q=A, cs=A, max_pos=2048, bt=A, max_blocks=128, sl=A, scale=0.125, out=A,
                B=4, Hq=32, Hkv=8, D=64, num_pages=1024, part=0, ws=A, ws_n=1 << 30, stream=None)
    args.update(kw)
    return lib.pa_rope_append_decode(args["k_new"], args["v_new"], args["k"], args["v"], args["q"], args["cs"],
                                     args["max_pos"], args["bt"], args["max_blocks"], args["sl"], args["scale"],
                                     args["out"], args["B"], args["Hq"], args["Hkv"], args["D"], args["num_pages"],
                                     args["part"], args["ws"], args["ws_n"], args["stream"])


def test_rope_append_decode_validation(lib):
    assert _rope_decode(lib, max_pos=0) == -2
    assert _rope_decode(lib, max_pos=2047) == -2  # the table must cover 16 x 128 positions
    assert _rope_decode(lib, max_pos=64, max_blocks=5) == -2
    assert _rope_decode(lib, cs=None) == -1
    assert _rope_decode(lib, cs=MIS) == -6
    assert _rope_decode(lib, k_new=None) == -1
    assert _rope_decode(lib, Hq=16, Hkv=4) == -3
    assert _rope_decode(lib, ws=None) == -4
    assert _rope_decode(lib, B=0) == 0  # nothing to do: no launch
