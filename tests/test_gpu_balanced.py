"""Length-balanced automatic splits (num_splits 0, matrix kernel) against the
fp64 oracle, and the one-call path's two stages.

With automatic splits the decode kernel reads seq_lens / q_lens and cuts every
sequence into chunks of one common size, so a ragged batch's long sequences
get many splits, short ones one (written straight to `out`), and the combine
merges a per-sequence number of partials. Tolerances as in
test_gpu_parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import WORKLOADS, Workload, make_case
from tests.test_gpu_parity import all_units, units_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f16": 2e-3, "fp8_e4m3": 2e-2, "int8": 2e-2}


def run(c, num_splits=0, kernel="matrix", workspace=None, stage="one-call", out=None):
    T, Hq, D = c.q.shape
    if out is None:
        out = torch.full((T, Hq, D), float("nan"), dtype=torch.float16, device=DEV)
    args = (c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.q_lens, c.scale,
            c.window, num_splits, out)
    kw = dict(k_scale=c.k_scale, v_scale=c.v_scale, kv_dtype=c.kv_dtype,
              max_q_len=c.max_q_len, kernel=kernel, kv_layout=c.kv_layout, workspace=workspace)
    if stage == "one-call":
        pda.paged_decode_attention(*args, **kw)
    else:
        pda.attention_stages(*args, **kw, stage="both")
    torch.cuda.synchronize()
    return out


def check(got, want, kv, what):
    g = got.cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    zero_rows = np.all(want == 0, axis=-1)
    assert np.all(g[zero_rows] == 0), f"{what}: rows that see no key are not zero"
    err = np.abs(g - want).max()
    assert err <= TOL[kv], f"{what}: max |err| {err:.3g} > {TOL[kv]}"
    return err


def ragged(seed, lens, **kw):
    base = dict(name="ragged", batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                seq_lens=tuple(lens), seed=seed, pool_pages=0, num_splits=0)
    base.update(kw)
    return Workload(**base)


# One long sequence among short and empty ones: the long one is cut into many
# chunks, the others get one chunk each (written by the decode kernel).
LENS = (0, 1, 15, 16, 17, 6000, 40, 2200, 5, 700, 0, 129)


@pytest.mark.parametrize("D,kv,G,Q,W", [(128, "f16", 4, 1, 0), (128, "f16", 7, 3, 0),
                                        (256, "f16", 6, 1, 0), (256, "fp8_e4m3", 4, 1, 0),
                                        (128, "int8", 7, 3, 100), (256, "f16", 6, 1, 1000),
                                        (128, "f16", 8, 4, 0), (256, "int8", 2, 2, 0)])
@pytest.mark.parametrize("Hkv", [1, 4, 6])
def test_balanced_ragged_vs_oracle(D, kv, G, Q, W, Hkv):
    w = ragged(61 + Hkv, LENS, head_dim=D, kv_dtype=kv, num_q_heads=G * Hkv,
               num_kv_heads=Hkv, q_len=Q, window=W)
    c = make_case(w, device=DEV)
    check(run(c), oracle.paged_decode_attention(**c.host()), kv, repr(w))


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("P", [16, 64, 256])
def test_balanced_layouts_and_page_sizes(layout, P):
    w = ragged(67, (3 * P + 5, 0, P, 4000, P - 1), layout=layout, page_size=P, q_len=2,
               num_q_heads=12, num_kv_heads=3)
    c = make_case(w, device=DEV)
    check(run(c), oracle.paged_decode_attention(**c.host()), "f16", repr(w))


@pytest.mark.parametrize("lens", [(0,), (0, 0, 0), (1,), (1, 0, 2), (20000,), (7, 20000)])
@pytest.mark.parametrize("Q", [1, 3])
def test_balanced_degenerate_batches(lens, Q):
    """All sequences empty, single-key sequences, one sequence holding the
    whole grid (the most chunks a row can get), and rows with no visible key
    (q_len above seq_len)."""
    w = ragged(71, lens, q_len=Q, num_q_heads=4, num_kv_heads=4, head_dim=256)
    c = make_case(w, device=DEV)
    check(run(c), oracle.paged_decode_attention(**c.host()), "f16", repr(w))


@pytest.mark.parametrize("lens,Q", [(LENS, 3), ((4096,) * 8, 1), ((20000,), 1)])
def test_stages_equal_one_call(lens, Q):
    """Decode stage then combine stage is the one-call path, bit for bit."""
    c = make_case(ragged(73, lens, q_len=Q), device=DEV)
    a = run(c)
    b = run(c, stage="stages")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name,over", [("gqa4_d128_b8_l4096", {}),
                                       ("gqa6_d256_l16384", dict(batch=3, window=4096)),
                                       ("verify_q3_d128_b32", dict(ragged_max=None, seq_len=3000,
                                                                   forced_zero=0))])
def test_balanced_uniform_batch_matches_fixed_split(name, over):
    """A uniform batch (same length and q_len everywhere) takes the fixed
    split: automatic splits give the output of the automatic count given
    explicitly, bit for bit."""
    c = make_case(WORKLOADS[name].with_(**over), device=DEV)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, c.max_q_len,
                           c.kv_dtype, "matrix")
    S = pda.resolve_splits(dims, c.window, 0)
    auto = run(c, num_splits=0)
    fixed = run(c, num_splits=S)
    assert torch.equal(auto.view(torch.int16), fixed.view(torch.int16))


def test_balanced_large_batch_uses_one_count():
    """A batch as large as the grid's slot count keeps one split count per
    sequence (balancing has no room); short ragged sequences."""
    lens = tuple(int(x) for x in np.random.default_rng(3).integers(0, 90, size=300))
    w = ragged(79, lens, num_q_heads=8, num_kv_heads=8, pool_pages=0)
    c = make_case(w, device=DEV)
    check(run(c), oracle.paged_decode_attention(**c.host()), "f16", "B=300")


def test_balanced_workspace_reuse_poisoned():
    """The chunk lists and partials are rewritten by every call: a workspace
    filled with NaN, then reused for batches of different raggedness, gives
    the oracle's answer each time."""
    c1 = make_case(ragged(83, LENS, q_len=2), device=DEV)
    c2 = make_case(ragged(84, (5000, 3, 0, 900), q_len=2), device=DEV)
    dims = pda.decode_dims(c1.q, c1.k_cache, c1.block_table, c1.seq_lens, c1.q_lens,
                           c1.max_q_len, "f16", "matrix")
    dims2 = pda.decode_dims(c2.q, c2.k_cache, c2.block_table, c2.seq_lens, c2.q_lens,
                            c2.max_q_len, "f16", "matrix")
    n = max(pda.workspace_bytes(dims, 0, 0), pda.workspace_bytes(dims2, 0, 0))
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    ws.view(torch.float32).fill_(float("nan"))
    first = None
    for c in (c1, c2, c1):
        got = run(c, workspace=ws)
        check(got, oracle.paged_decode_attention(**c.host()), "f16", "reused")
        if c is c1:
            if first is None:
                first = got
            else:
                assert torch.equal(got.view(torch.int16), first.view(torch.int16))


def test_full_verify_q3_d128_b32_balanced():
    """The ragged multi-token verify workload at full size with automatic
    (balanced) splits; every (sequence, KV head) unit."""
    c = make_case(WORKLOADS["verify_q3_d128_b32"].with_(num_splits=0), device=DEV)
    got = run(c, kernel="auto")
    units_parity(c, got, all_units(c))


@pytest.mark.parametrize("B,Q", [(65, 1), (100, 3), (255, 1)])
@pytest.mark.parametrize("kind", ["ragged", "uniform"])
def test_balanced_batches_over_64(B, Q, kind):
    """65 to 255 sequences: each lane of the search holds up to four
    sequences; ragged lengths (with empty ones) and a uniform batch."""
    r = np.random.default_rng(B)
    if kind == "ragged":
        lens = [int(x) for x in r.integers(0, 1200, size=B)]
        lens[3] = 0
        lens[B - 1] = 5000
    else:
        lens = [700] * B
    w = ragged(89 + B, tuple(lens), q_len=Q, num_q_heads=8, num_kv_heads=2)
    c = make_case(w, device=DEV)
    check(run(c), oracle.paged_decode_attention(**c.host()), "f16", f"B={B} {kind}")


@pytest.mark.parametrize("seed", range(6))
def test_balanced_ragged_near_page_edges(seed):
    """Seeded ragged batches whose lengths sit at, just below and just past
    16-key tile edges, a few sequences long and many short, so that chunk
    counts round up unevenly."""
    r = np.random.default_rng(1000 + seed)
    B = int(r.integers(2, 40))
    tiles = r.choice([1, 2, 3, 5, 8, 33, 64, 130], size=B)
    lens = tuple(int(16 * t + r.choice([-1, 0, 1])) for t in tiles)
    c = make_case(ragged(97 + seed, lens, q_len=int(r.choice([1, 2])), num_q_heads=4,
                         num_kv_heads=1), device=DEV)
    check(run(c), oracle.paged_decode_attention(**c.host()), "f16", repr(lens))


@pytest.mark.parametrize("kernel,splits,Q", [("matrix", 5, 2), ("matrix", 1, 1), ("vector", 0, 1),
                                             ("vector", 3, 2), ("auto", 0, 40)])
def test_stages_equal_one_call_every_path(kernel, splits, Q):
    """The two stage calls reproduce the one-call path bit for bit on the
    fixed-count path, one split (no combine), the vector kernel and the
    prefill kernel (40 new tokens: one split, nothing to combine)."""
    c = make_case(ragged(101, (300, 0, 77, 1000), q_len=Q, num_q_heads=8, num_kv_heads=2),
                  device=DEV)
    a = run(c, num_splits=splits, kernel=kernel)
    b = run(c, num_splits=splits, kernel=kernel, stage="stages")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check(a, oracle.paged_decode_attention(**c.host()), "f16", f"{kernel} S={splits} Q={Q}")


@pytest.mark.parametrize("L,W,S,Q", [(1 << 18, 0, 0, 1), (1 << 18, 0, 256, 1), (1 << 18, 0, 0, 3),
                                     (1 << 20, 70000, 0, 3)])
def test_very_long_sequence(L, W, S, Q):
    """One sequence of 2^18 keys (8 times the longest benchmark) with
    automatic splits and with the most splits a call takes, and one of 2^20
    keys (65536 pages) with a window far inside it, against the oracle."""
    w = ragged(103, (L,), q_len=Q, window=W, num_q_heads=4, num_kv_heads=1)
    c = make_case(w, device=DEV)
    check(run(c, num_splits=S), oracle.paged_decode_attention(**c.host()), "f16",
          f"L={L} W={W} S={S} Q={Q}")
