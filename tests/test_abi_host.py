"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/pda.h declares, and rejects bad arguments on the host before
any HIP call; the split policy and workspace sizes are pure host logic."""

import ctypes
import os
import re

import pytest

import paged_split_decode_amd as pda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "pda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pda_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = pda.load_library()
    names = _declared_functions()
    assert "pda_paged_decode_attention" in names and "pda_split_combine" in names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pda_version().startswith(b"pda ")


def _dims(**kw):
    base = dict(batch=8, num_tokens=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                page_size=16, num_pages=2049, max_pages_per_seq=257, max_q_len=1, kv_dtype=0)
    base.update(kw)
    return pda.DecodeDims(**base)


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def _call(dims, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, ql=None, scale=0.1, window=0,
                splits=1, out=FAKE, ks=None, vs=None, ws=None, wsb=0)
    args.update(over)
    lib = pda.load_library()
    return lib.pda_paged_decode_attention(
        args["q"], args["k"], args["v"], args["bt"], args["sl"], args["ql"], args["scale"],
        args["window"], args["splits"], args["out"], args["ks"], args["vs"],
        None if dims is None else ctypes.byref(dims), args["ws"], args["wsb"], None)


@pytest.mark.parametrize("dims_kw,over,status", [
    (dict(head_dim=64), {}, -4),
    (dict(page_size=48), {}, -4),
    (dict(page_size=512), {}, -4),
    (dict(page_size=8), {}, -4),
    (dict(kv_layout=2), {}, -4),
    (dict(kernel=1, page_size=32), {}, -4),  # the vector kernel reads 16-key pages
    (dict(kernel=1, kv_layout=1), {}, -4),   # ... in the NHD layout
    (dict(num_q_heads=30), {}, -2),
    (dict(num_kv_heads=0), {}, -2),
    (dict(kv_dtype=7), {}, -4),
    (dict(max_q_len=0), {}, -2),
    (dict(num_q_heads=64, num_kv_heads=1, kernel=2), {}, -4),  # decode kernels: <= 32 rows
    (dict(num_q_heads=64, num_kv_heads=1, kernel=1), {}, -4),
    (dict(num_q_heads=256, num_kv_heads=1), {}, -4),  # group > PDA_MAX_GROUP
    (dict(num_q_heads=64, num_kv_heads=1), dict(splits=4), -4),  # prefill: one split
    (dict(kernel=3), dict(splits=2), -4),
    (dict(kernel=4), {}, -4),
    (dict(num_pages=0), {}, -2),
    ({}, dict(q=None), -1),
    ({}, dict(out=None), -1),
    ({}, dict(q=ctypes.c_void_p(0x100004)), -3),
    ({}, dict(out=ctypes.c_void_p(0x100008)), -3),
    ({}, dict(splits=-1), -2),
    ({}, dict(splits=257), -2),
    (dict(kv_dtype=1), {}, -1),  # fp8 without scales
    ({}, dict(ks=FAKE, vs=FAKE), -2),  # scales with fp16
    (dict(num_tokens=9), {}, -2),  # no q_lens: T must equal B
    ({}, dict(splits=4), -5),  # 4 splits need a workspace
    ({}, dict(splits=4, ws=FAKE, wsb=16), -5),
])
def test_validation_errors(dims_kw, over, status):
    st = _call(_dims(**dims_kw), **over)
    assert st == status, (st, pda.load_library().pda_last_error())
    assert pda.load_library().pda_last_error()


def test_null_dims():
    assert _call(None) == -1


def test_empty_batch_is_ok_without_launch():
    assert _call(_dims(batch=0, num_tokens=0)) == 0


def test_split_policy_and_workspace():
    d = _dims()
    # matrix kernel: 8 sequences x 2 groups of 4 KV heads per split; 2 wave
    # slots per SIMD on 256 CUs -> 512 four-wave workgroups -> 32 splits
    assert pda.resolve_splits(d, 0, 0, 256) == 32
    assert pda.resolve_splits(d, 0, 0, 128) == 16
    # v_dot2 kernel: 64 (sequence, KV head) units, about one workgroup per CU
    assert pda.resolve_splits(_dims(kernel=1), 0, 0, 256) == 4
    assert pda.resolve_splits(d, 0, 3, 256) == 3
    d3 = _dims(batch=1, num_tokens=1, num_q_heads=24, num_kv_heads=4, head_dim=256,
               max_pages_per_seq=1025, num_pages=1025)
    s = pda.resolve_splits(d3, 0, 0, 256)
    assert 64 <= s <= 256
    s_win = pda.resolve_splits(d3, 4096, 0, 256)
    assert 1 <= s_win <= s
    assert pda.workspace_bytes(d, 0, 1) == 0
    assert pda.workspace_bytes(d, 0, 8) == 8 * 32 * 8 * (128 + 2) * 4
    assert pda.partials_bytes(d, 0, 1) == 8 * 32 * 1 * (128 + 2) * 4
    tiny = _dims(batch=1, num_tokens=1, max_pages_per_seq=1)
    assert pda.resolve_splits(tiny, 0, 0, 256) == 1


def _cdims(**kw):
    base = dict(num_tokens=4, num_kv_heads=8, head_dim=128, page_size=16, num_pages=64,
                kv_dtype=0)
    base.update(kw)
    return pda.CacheDims(**base)


def _wcall(dims, **over):
    args = dict(key=FAKE, value=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None)
    args.update(over)
    return pda.load_library().pda_write_kv_cache(
        args["key"], args["value"], args["slots"], args["kc"], args["vc"], args["ks"],
        args["vs"], None if dims is None else ctypes.byref(dims), None)


@pytest.mark.parametrize("dims_kw,over,status", [
    (dict(head_dim=100), {}, -4),               # not a multiple of 8
    (dict(kv_dtype=5), {}, -4),
    (dict(kv_layout=3), {}, -4),
    (dict(num_kv_heads=0), {}, -2),
    (dict(page_size=0), {}, -2),
    (dict(num_tokens=-1), {}, -2),
    (dict(num_pages=1 << 28, page_size=16), {}, -2),  # slots would overflow int32
    ({}, dict(slots=None), -1),
    ({}, dict(kc=None), -1),
    (dict(kv_dtype=1), {}, -1),                 # fp8 without scales
    (dict(kv_dtype=2), dict(ks=FAKE), -1),      # int8 with one scale missing
    ({}, dict(ks=FAKE, vs=FAKE), -2),           # scales with fp16
    ({}, dict(key=ctypes.c_void_p(0x100008)), -3),
    ({}, dict(kc=ctypes.c_void_p(0x100008)), -3),  # fp16 cache needs 16 bytes
])
def test_writer_validation_errors(dims_kw, over, status):
    st = _wcall(_cdims(**dims_kw), **over)
    assert st == status, (st, pda.load_library().pda_last_error())
    assert pda.load_library().pda_last_error()


def test_writer_null_dims_and_empty_batch():
    assert _wcall(None) == -1
    # no tokens: nothing to write, no pointer is looked at
    assert _wcall(_cdims(num_tokens=0), key=None, value=None, slots=None, kc=None, vc=None) == 0


def test_prefill_split_policy_and_no_partials():
    d = _dims(num_q_heads=64, num_kv_heads=1)   # 64 rows per KV head: prefill kernel
    assert pda.resolve_splits(d, 0, 0, 256) == 1
    assert pda.resolve_splits(d, 0, 1, 256) == 1
    assert pda.workspace_bytes(d, 0, 0) == 0
    lib = pda.load_library()
    st = lib.pda_paged_decode_partials(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, 0, 0, None, None,
                                       ctypes.byref(d), FAKE, 1 << 20, None)
    assert st == -4 and b"decode kernels" in lib.pda_last_error()


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No fallback: a missing libpda.so is an error, not a silent CPU path."""
    monkeypatch.setattr(pda, "_lib", None)
    monkeypatch.setattr(pda, "_LIB_PATH", str(tmp_path / "libpda.so"))
    with pytest.raises(RuntimeError, match="missing"):
        pda.load_library()
