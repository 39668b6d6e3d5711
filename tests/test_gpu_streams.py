"""Stream semantics of the C ABI: every launch (attention and cache writer)
goes on the caller's stream, and the library keeps no device state between
calls (two calls in flight at once on two streams, each with its own
workspace, do not interfere).

A call is queued behind a bounded GPU sleep and an asynchronous copy of its
queries on the same side stream: it gives the oracle's answer only if its
kernels run after the copy, i.e. on that stream (the default stream would not
wait for it). Tolerances as in test_gpu_parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import Workload, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3
SLEEP_CYCLES = 1 << 24  # a few ms of GPU time at the shader clock


def case(seed, lens, **kw):
    base = dict(name="streams", batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                seq_lens=tuple(lens), seed=seed, num_splits=0)
    base.update(kw)
    return make_case(Workload(**base), device=DEV)


def enqueue(c, stream, num_splits=0, kernel="auto", q_src=None):
    """On `stream`: sleep, copy q (from `q_src`, ready on the device) into a
    fresh buffer, run the attention on that buffer. Returns the output tensor
    (valid once `stream` is done)."""
    if q_src is None:
        q_src = c.q.clone()
        torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        q = torch.zeros_like(q_src)
        out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=DEV)
        torch.cuda._sleep(SLEEP_CYCLES)
        q.copy_(q_src, non_blocking=True)
        pda.paged_decode_attention(q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.q_lens,
                                   c.scale, c.window, num_splits, out, k_scale=c.k_scale,
                                   v_scale=c.v_scale, kv_dtype=c.kv_dtype, max_q_len=c.max_q_len,
                                   kernel=kernel, kv_layout=c.kv_layout)
    return out


def check(out, c, what):
    g = out.cpu().numpy().astype(np.float64)
    want = oracle.paged_decode_attention(**c.host())
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - want).max()
    assert err <= TOL, f"{what}: max |err| {err:.3g} > {TOL}"


@pytest.mark.parametrize("kernel,splits", [("matrix", 0), ("matrix", 3), ("vector", 2),
                                           ("auto", 1)])
def test_runs_on_the_callers_stream(kernel, splits):
    c = case(5, (700, 0, 33, 2500), q_len=2)
    s = torch.cuda.Stream()
    out = enqueue(c, s, splits, kernel)
    s.synchronize()
    check(out, c, f"side stream {kernel} S={splits}")


def test_prefill_runs_on_the_callers_stream():
    c = case(6, (300, 90), q_len=64)
    s = torch.cuda.Stream()
    out = enqueue(c, s, 1)
    s.synchronize()
    check(out, c, "side stream prefill")


def test_two_streams_in_flight():
    """Two ragged batches (automatic, balanced splits: chunk lists and
    partials in each call's own workspace) queued on two streams at once."""
    a = case(7, (5000, 3, 0, 900, 64), q_len=3)
    b = case(8, (40, 6000, 1200), q_len=1, num_q_heads=12, num_kv_heads=4)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    qa, qb = a.q.clone(), b.q.clone()
    torch.cuda.synchronize()
    out_a = enqueue(a, s1, q_src=qa)
    out_b = enqueue(b, s2, q_src=qb)
    torch.cuda.synchronize()
    check(out_a, a, "stream 1")
    check(out_b, b, "stream 2")


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
def test_writer_runs_on_the_callers_stream(kv):
    """The cache writer behind a sleep and a copy of its key rows on a side
    stream: the cache bytes equal the writer oracle's."""
    from synth import make_write_case
    c = make_write_case(300, 4, 128, 16, num_pages=40, kv_dtype=kv, seed=11, device=DEV)
    h = c.host()
    key_src = c.key.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        key = torch.zeros_like(key_src)
        torch.cuda._sleep(SLEEP_CYCLES)
        key.copy_(key_src, non_blocking=True)
        pda.write_kv_cache(key, c.value, c.slot_mapping, c.k_cache, c.v_cache,
                           k_scale=c.k_scale, v_scale=c.v_scale, kv_dtype=c.kv_dtype,
                           kv_layout=c.kv_layout)
    s.synchronize()
    want_k, want_v = oracle.write_kv_cache(h["key"], h["value"], h["slot_mapping"], h["k_cache"],
                                           h["v_cache"], h["kv_dtype"], h["k_scale"],
                                           h["v_scale"], h["kv_layout"])
    assert c.k_cache.cpu().numpy().tobytes() == want_k.tobytes(), "K cache bytes differ"
    assert c.v_cache.cpu().numpy().tobytes() == want_v.tobytes(), "V cache bytes differ"


def test_own_workspace_on_a_non_current_stream():
    """A call that names a stream other than the current one and brings no
    workspace: the binding's temporary workspace must not go to new work on
    the current stream while the call's kernels (queued behind a sleep on
    their own stream) still use it. Allocations right after the call, on the
    current stream and of the workspace's size, are filled with NaN bytes."""
    c = case(9, (5000, 3, 900, 64), q_len=2)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, c.max_q_len,
                           "f16")
    need = pda.workspace_bytes(dims, c.window, 0)
    assert need > 0
    s = torch.cuda.Stream()
    q_src = c.q.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        q = torch.zeros_like(q_src)
        out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=DEV)
        torch.cuda._sleep(SLEEP_CYCLES)
        q.copy_(q_src, non_blocking=True)
    assert torch.cuda.current_stream() != s
    pda.paged_decode_attention(q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.q_lens,
                               c.scale, c.window, 0, out, max_q_len=c.max_q_len, stream=s)
    junk = [torch.empty(need, dtype=torch.uint8, device=DEV).fill_(0xFF) for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    check(out, c, "own workspace, named stream")
