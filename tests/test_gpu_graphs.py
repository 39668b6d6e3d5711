"""The one-call path captured in a HIP graph (torch.cuda.CUDAGraph): its two
launches take no allocation, memset or host synchronization, so a serving
loop can capture a decode step once and replay it.

With automatic splits the work is balanced on the device from seq_lens, so
one captured graph serves changing lengths: between replays the test writes
new lengths (at most the captured table's capacity) and new queries into the
same device buffers, with eager work and synchronizations in between, and
checks every replay against the oracle on those inputs and, bit for bit,
against an eager call. Tolerances as in test_gpu_parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import Workload, make_case

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f16": 2e-3, "fp8_e4m3": 2e-2, "int8": 2e-2}


def case(seed, lens, **kw):
    base = dict(name="graphs", batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                seq_lens=tuple(lens), seed=seed, num_splits=0)
    base.update(kw)
    return make_case(Workload(**base), device=DEV)


def call(c, out, ws, num_splits, kernel):
    pda.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.q_lens,
                               c.scale, c.window, num_splits, out, k_scale=c.k_scale,
                               v_scale=c.v_scale, kv_dtype=c.kv_dtype, max_q_len=c.max_q_len,
                               workspace=ws, kernel=kernel, kv_layout=c.kv_layout)


@pytest.mark.parametrize("kernel,splits,kv,Q", [("matrix", 0, "f16", 3), ("matrix", 0, "fp8_e4m3", 1),
                                                ("matrix", 4, "f16", 2), ("vector", 3, "int8", 1),
                                                ("auto", 1, "f16", 48)])
def test_graph_replays_with_new_lengths(kernel, splits, kv, Q):
    # Every table row maps 4100 keys; the replays' lengths stay within that.
    cap = (4100,) * 6
    c = case(21, cap, q_len=Q, kv_dtype=kv)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, c.max_q_len,
                           c.kv_dtype, kernel, c.kv_layout)
    ws = torch.empty(max(1, pda.workspace_bytes(dims, c.window, splits)), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty(c.q.shape, dtype=torch.float16, device=DEV)
    eager = torch.empty_like(out)

    # Warm up on a side stream (the first call queries the device), then
    # capture.
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(c, out, ws, splits, kernel)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(c, out, ws, splits, kernel)

    r = np.random.default_rng(5)
    for rep, lens in enumerate([cap, (3000, 17, 0, 1200, 640, 4100), (40, 4100, 2999, 0, 15, 1),
                                (1, 1, 1, 1, 1, 1), (4000, 3900, 64, 700, 2222, 4096), cap]):
        # New lengths and queries in the captured buffers (eager work).
        c.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        c.q.copy_(torch.from_numpy(r.standard_normal(tuple(c.q.shape)).astype(np.float16)))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        h = c.host()
        want = oracle.paged_decode_attention(**h)
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), f"replay {rep}: non-finite output"
        err = np.abs(got - want).max()
        assert err <= TOL[kv], f"replay {rep} lens={lens}: max |err| {err:.3g}"
        # The eager call on the same inputs gives the same bits.
        call(c, eager, ws, splits, kernel)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), out.view(torch.int16)), f"replay {rep}"
