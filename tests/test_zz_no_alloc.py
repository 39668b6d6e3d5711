"""The no-allocation entry point (pda_paged_decode_attention_noalloc, the
library's per-device scratch array in place of a workspace) against the
entry point with a caller workspace, through the C ABI: two calls in a row,
the second smaller, each equal bit for bit to the workspace path and within
the oracle's tolerance."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import WORKLOADS, Workload, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f16": 2e-3, "fp8_e4m3": 2e-2, "int8": 2e-2}


def _abi_call(fn_name, c, num_splits, out, workspace=None):
    """One call through the C ABI (ctypes, no binding logic)."""
    lib = pda.load_library()
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, c.max_q_len,
                           c.kv_dtype, "auto", c.kv_layout)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [P(c.q), P(c.k_cache), P(c.v_cache), P(c.block_table), P(c.seq_lens), P(c.q_lens),
            ctypes.c_float(c.scale), ctypes.c_int32(c.window), ctypes.c_int32(num_splits),
            P(out), P(c.k_scale), P(c.v_scale), ctypes.byref(dims)]
    if workspace is not None:
        args += [P(workspace), ctypes.c_size_t(workspace.numel())]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = getattr(lib, fn_name)(*args, stream)
    assert st == 0, lib.pda_last_error().decode()
    return dims


def _both(c, num_splits):
    T, Hq, D = c.q.shape
    ref = torch.full((T, Hq, D), float("nan"), dtype=torch.float16, device=DEV)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, c.max_q_len,
                           c.kv_dtype, "auto", c.kv_layout)
    need = pda.workspace_bytes(dims, c.window, num_splits)
    assert 0 <= need <= pda.noalloc_scratch_bytes()
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    _abi_call("pda_paged_decode_attention", c, num_splits, ref, ws)
    got = torch.full((T, Hq, D), float("nan"), dtype=torch.float16, device=DEV)
    _abi_call("pda_paged_decode_attention_noalloc", c, num_splits, got)
    torch.cuda.synchronize()
    return got, ref, need


def _check(got, ref, c):
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    want = oracle.paged_decode_attention(**c.host())
    g = got.cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all()
    assert np.abs(g - want).max() <= TOL[c.kv_dtype]


@pytest.mark.parametrize("first,second,splits", [
    # automatic (balanced) splits: a large ragged batch, then a smaller one
    (dict(seq_lens=(5000, 3, 0, 900, 64, 2500), q_len=3), dict(seq_lens=(700, 20), q_len=2), 0),
    # a caller's split count
    (dict(seq_lens=(4000, 4000, 1, 300), q_len=1), dict(seq_lens=(33,), q_len=1), 5),
    # D=256, 1-byte KV
    (dict(seq_lens=(3000, 77, 6000), q_len=1, head_dim=256, kv_dtype="fp8_e4m3",
          num_q_heads=16, num_kv_heads=4),
     dict(seq_lens=(100, 9), q_len=1, head_dim=256, kv_dtype="fp8_e4m3", num_q_heads=16,
          num_kv_heads=4), 0),
])
def test_noalloc_equals_workspace_path(first, second, splits):
    sizes = []
    for i, kw in enumerate((first, second)):
        base = dict(name="noalloc", batch=len(kw["seq_lens"]), num_q_heads=8, num_kv_heads=2,
                    head_dim=128, seed=300 + i, num_splits=splits)
        base.update(kw)
        c = make_case(Workload(**base), device=DEV)
        got, ref, need = _both(c, splits)
        _check(got, ref, c)
        sizes.append(need)
    assert sizes[1] < sizes[0]


def test_noalloc_headline_workload_twice():
    """The D=128 8 x 4096 workload (automatic splits), then the tiny one."""
    c = make_case(WORKLOADS["gqa4_d128_b8_l4096"], device=DEV)
    got, ref, big = _both(c, 0)
    _check(got, ref, c)
    t = make_case(WORKLOADS["tiny_d128"], device=DEV)
    got, ref, small = _both(t, 3)
    _check(got, ref, t)
    assert 0 < small < big


def test_noalloc_refuses_a_call_larger_than_its_scratch():
    """A call whose partials exceed the scratch array gets PDA_ERR_WORKSPACE
    before any launch (its out stays as it was)."""
    w = Workload("big", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=256, seq_len=16,
                 q_len=1, num_splits=256, seed=9)
    c = make_case(w, device=DEV)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, 1, "f16")
    assert pda.workspace_bytes(dims, 0, 256) > pda.noalloc_scratch_bytes()
    out = torch.full(tuple(c.q.shape), 7.0, dtype=torch.float16, device=DEV)
    with pytest.raises(pda.PdaError, match="PDA_ERR_WORKSPACE"):
        pda.paged_decode_attention_noalloc(c.q, c.k_cache, c.v_cache, c.block_table,
                                           c.seq_lens, c.q_lens, c.scale, 0, 256, out,
                                           max_q_len=1)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0).item()
