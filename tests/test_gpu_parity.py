"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: max |gpu - oracle| <= 2e-3 for fp16 KV and <= 2e-2 against the
dequantized-KV oracle for fp8-e4m3 / int8 KV. Rows that see no key must be
exactly zero; every output must be finite. Cases mirror the decode cells the
pages list (writer layout, empty rows, custom scale into out, sliding window,
multi-token queries, split decode) plus page-permutation and uniform-V
bit-exactness, and the benchmark workloads at full size on sampled
(sequence, KV head) units.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import WORKLOADS, Workload, make_case, unit_subcase

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f16": 2e-3, "fp8_e4m3": 2e-2, "int8": 2e-2}


KERNELS = ["vector", "matrix"]


def run_gpu(case, num_splits=None, scale=None, window=None, out=None, use_q_lens=True,
            kernel="auto"):
    T, Hq, D = case.q.shape
    if out is None:
        out = torch.full((T, Hq, D), float("nan"), dtype=torch.float16, device=DEV)
    ql = case.q_lens if use_q_lens else None
    pda.paged_decode_attention(
        case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens, ql,
        case.scale if scale is None else scale,
        case.window if window is None else window,
        case.workload.num_splits if num_splits is None else num_splits, out,
        k_scale=case.k_scale, v_scale=case.v_scale, kv_dtype=case.kv_dtype,
        max_q_len=case.max_q_len if use_q_lens else None, kernel=kernel,
        kv_layout=case.kv_layout)
    torch.cuda.synchronize()
    return out


def oracle_full(case, **over):
    h = case.host()
    h.update(over)
    return oracle.paged_decode_attention(**h)


def assert_parity(got, want, kv, what=""):
    g = got.detach().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    zero_rows = np.all(want == 0, axis=-1)
    assert np.all(g[zero_rows] == 0), f"{what}: rows that see no key are not zero"
    err = np.abs(g - want).max() if g.size else 0.0
    assert err <= TOL[kv], f"{what}: max |err| {err:.3g} > {TOL[kv]}"
    return err


def case_on_gpu(w):
    return make_case(w, device=DEV)


def vector_takes(D, kv, rows):
    """Whether the vector kernel covers G * max_q_len query rows per KV head:
    up to 8 waves of its largest compiled row count (5 rows per wave for fp16
    at D=128, 6 for 1-byte KV at D=128, 4 at D=256, 3 for int8 at D=256)."""
    per_wave = {(128, "f16"): 5, (128, "fp8_e4m3"): 6, (128, "int8"): 6,
                (256, "f16"): 4, (256, "fp8_e4m3"): 4, (256, "int8"): 3}[(D, kv)]
    return rows <= 8 * per_wave


def small(seed, **kw):
    base = dict(name="small", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                seq_lens=(1, 77, 300), seed=seed, pool_pages=48)
    base.update(kw)
    base["batch"] = len(base["seq_lens"])
    return Workload(**base)


# ---------------------------------------------------------------------------
# The tiny workload and small random cases (full comparison)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("kernel", KERNELS)
def test_tiny_workload(splits, kernel):
    c = case_on_gpu(WORKLOADS["tiny_d128"])
    assert_parity(run_gpu(c, kernel=kernel, num_splits=splits), oracle_full(c), "f16", f"tiny S={splits}")


def _random_case(seed):
    r = np.random.default_rng(500 + seed)
    D = int(r.choice([128, 256]))
    kv = str(r.choice(["f16", "fp8_e4m3", "int8"]))
    Hkv = int(r.choice([1, 2, 3, 4, 5, 8, 12]))
    Q = int(r.choice([1, 1, 2, 3, 4]))
    max_g = max(1, 32 // Q)
    G = int(r.choice([g for g in (1, 2, 3, 4, 5, 6, 7, 8) if g <= max_g]))
    B = int(r.integers(1, 5))
    lens = tuple(int(x) for x in r.integers(0, 700, size=B))
    W = int(r.choice([0, 0, 1, 17, 100, 5000]))
    S = int(r.choice([0, 1, 2, 3, 5, 8, 32]))
    return Workload("rand", batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                    kv_dtype=kv, q_len=Q, seq_lens=lens, window=W, num_splits=S,
                    seed=seed, table_pad=int(r.integers(0, 3)))


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("kernel", KERNELS)
def test_random_small_cases(seed, kernel):
    w = _random_case(seed)
    c = case_on_gpu(w)
    G = w.num_q_heads // w.num_kv_heads
    if kernel == "vector" and not vector_takes(w.head_dim, w.kv_dtype, G * w.q_len):
        with pytest.raises(pda.PdaError, match="PDA_ERR_UNSUPPORTED"):
            run_gpu(c, kernel=kernel)
        return
    assert_parity(run_gpu(c, kernel=kernel), oracle_full(c), w.kv_dtype, repr(w))


@pytest.mark.parametrize("Hkv", [1, 3, 4, 5, 6, 8, 12, 16])
@pytest.mark.parametrize("D,kv,G,Q", [(128, "f16", 4, 1), (256, "f16", 6, 1),
                                      (256, "fp8_e4m3", 4, 1), (128, "int8", 7, 3),
                                      (256, "f16", 5, 4)])
@pytest.mark.parametrize("splits", [1, 4])
def test_kv_head_groups(Hkv, D, kv, G, Q, splits):
    """KV heads are grouped into workgroups (one or several waves per head,
    the last group possibly short); every head's rows must come out right,
    written directly (one split) or through partials."""
    w = small(23, head_dim=D, kv_dtype=kv, num_q_heads=G * Hkv, num_kv_heads=Hkv, q_len=Q,
              seq_lens=(0, 45, 700, 129), num_splits=splits)
    c = case_on_gpu(w)
    assert_parity(run_gpu(c, kernel="matrix"), oracle_full(c), kv, repr(w))


@pytest.mark.parametrize("D,kv,G,Q", [(128, "f16", 4, 1), (256, "f16", 6, 1),
                                      (256, "fp8_e4m3", 4, 2), (128, "int8", 7, 3)])
@pytest.mark.parametrize("splits", [1, 4, 0])
def test_streaming_loads_give_the_same_output(D, kv, G, Q, splits):
    """The matrix kernel streams K and V (non-temporal loads) when the K/V a
    call can read, judged from the block table's capacity, exceed the
    last-level cache. The same small case with its table padded by unused
    columns (never read: past every sequence's pages) takes that variant;
    both outputs equal the oracle's. (Not bit for bit each other's: the
    capacity also sets the split and key-wave plan, hence the order of the
    fp32 sums. No window: a window bounds the keys a call can read whatever
    the table.)"""
    import dataclasses
    w = small(29, head_dim=D, kv_dtype=kv, num_q_heads=G * 2, num_kv_heads=2, q_len=Q,
              seq_lens=(0, 45, 700, 129), num_splits=splits)
    c = case_on_gpu(w)
    elem = 2 if kv == "f16" else 1
    cols = (256 << 20) // (c.workload.page_size * 4 * 2 * D * elem * 2) + 16  # capacity past the cache
    bt = torch.zeros((c.block_table.shape[0], cols), dtype=c.block_table.dtype, device=DEV)
    bt[:, :c.block_table.shape[1]] = c.block_table
    want = oracle_full(c)
    assert_parity(run_gpu(c, kernel="matrix"), want, kv, repr(w))
    assert_parity(run_gpu(dataclasses.replace(c, block_table=bt), kernel="matrix"), want, kv,
                  f"{w!r}, table of {cols} columns")


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("P", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("D,kv,G,Q,W", [(128, "f16", 4, 1, 0), (256, "fp8_e4m3", 6, 2, 100),
                                        (128, "int8", 7, 3, 0), (256, "f16", 1, 1, 37)])
@pytest.mark.parametrize("splits", [1, 5])
def test_layouts_and_page_sizes(layout, P, D, kv, G, Q, W, splits):
    """Pages of 16 * 2^k keys and the HND layout ([page, head, slot, dim])
    on the matrix kernel; lengths end inside, at and across page edges."""
    w = small(41 + P, head_dim=D, kv_dtype=kv, num_q_heads=G * 3, num_kv_heads=3, q_len=Q,
              seq_lens=(0, P - 1, P, 2 * P + 17, 700), page_size=P, layout=layout,
              window=W, num_splits=splits, pool_pages=0)
    c = case_on_gpu(w)
    assert_parity(run_gpu(c, kernel="matrix"), oracle_full(c), kv, repr(w))


@pytest.mark.parametrize("layout,kernel", [("NHD", "auto"), ("HND", "auto"), ("NHD", "vector")])
def test_identity_table(layout, kernel):
    """Pages in pool order (the "dense" reading of the pages' layout flag)."""
    w = small(43, seq_lens=(300, 17, 129), layout=layout, num_splits=3, identity_table=True)
    c = case_on_gpu(w)
    assert_parity(run_gpu(c, kernel=kernel), oracle_full(c), "f16", repr(w))


@pytest.mark.parametrize("D,kv,G,Q", [(128, "f16", 7, 3), (256, "f16", 6, 1),
                                      (256, "int8", 4, 1)])
@pytest.mark.parametrize("splits", [64, 200])
def test_longest_first_order(D, kv, G, Q, splits):
    """Grids of several rounds order their rows by sequence length (ragged
    lengths with ties and empty sequences); every sequence must still get its
    own rows."""
    lens = (900, 0, 33, 900, 1, 410, 0, 77, 900, 256, 16, 17, 640, 5, 129, 900, 2, 300, 31, 64)
    w = small(31, head_dim=D, kv_dtype=kv, num_q_heads=G * 4, num_kv_heads=4, q_len=Q,
              seq_lens=lens, num_splits=splits, pool_pages=1024)
    c = case_on_gpu(w)
    assert_parity(run_gpu(c, kernel="matrix"), oracle_full(c), kv, repr(w))


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("G,Q", [(1, 1), (4, 1), (6, 1), (8, 1), (7, 3), (8, 4), (5, 2)])
@pytest.mark.parametrize("kernel", KERNELS)
def test_head_dims_dtypes_groups(kv, D, G, Q, kernel):
    w = small(11, head_dim=D, kv_dtype=kv, num_q_heads=2 * G, num_kv_heads=2, q_len=Q,
              num_splits=3)
    c = case_on_gpu(w)
    if kernel == "vector" and not vector_takes(D, kv, G * Q):
        # more rows than the vector kernel's spill-free shapes cover: refused
        with pytest.raises(pda.PdaError, match="PDA_ERR_UNSUPPORTED"):
            run_gpu(c, kernel=kernel)
        return
    assert_parity(run_gpu(c, kernel=kernel), oracle_full(c), kv, repr(w))


# ---------------------------------------------------------------------------
# The pages' decode cells
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("kernel", KERNELS)
def test_writer_layout_identity_and_permuted_tables(kernel):
    # The kernel reads [page, slot, KV head, dim] pages through the table,
    # whether the table is an identity (dense layout) or a permutation.
    w = small(12, seq_lens=(64, 160), pool_pages=0, table_pad=0)
    c = case_on_gpu(w)
    want = oracle_full(c)
    assert_parity(run_gpu(c, kernel=kernel), want, "f16", "permuted")
    n = c.k_cache.shape[0]
    bt = c.block_table.long()
    order = torch.cat([bt[0, :4], bt[1, :10]])
    rest = torch.tensor([p for p in range(n) if p not in set(order.tolist())], device=DEV)
    order = torch.cat([order, rest])
    c.k_cache = c.k_cache[order].contiguous()
    c.v_cache = c.v_cache[order].contiguous()
    c.block_table = torch.tensor([[0, 1, 2, 3] + [n - 1] * 6, list(range(4, 14))],
                                 dtype=torch.int32, device=DEV)
    assert_parity(run_gpu(c, kernel=kernel), want, "f16", "identity table")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("kernel", KERNELS)
def test_empty_rows_are_zero(D, kernel):
    w = small(13, head_dim=D, q_len=3, seq_lens=(0, 2, 1, 40, 0), num_splits=4)
    c = case_on_gpu(w)
    got = run_gpu(c, kernel=kernel)
    want = oracle_full(c)
    assert_parity(got, want, "f16", "empty rows")
    g = got.cpu().numpy()
    # L=0: rows 0-2; L=2, q_len 3: row 3; L=1: rows 6-7 (row 8 sees key 0); L=0: rows 12-14
    for t in (0, 1, 2, 3, 6, 7, 12, 13, 14):
        assert np.all(g[t] == 0), t
    assert np.any(g[8] != 0)


@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("kernel", KERNELS)
def test_custom_scale_into_out(splits, kernel):
    c = case_on_gpu(small(14, num_splits=splits))
    out = torch.full(tuple(c.q.shape), float("nan"), dtype=torch.float16, device=DEV)
    got = run_gpu(c, kernel=kernel, scale=0.37, out=out)
    assert got.data_ptr() == out.data_ptr()
    assert_parity(out, oracle_full(c, scale=0.37), "f16", "scale 0.37")


@pytest.mark.parametrize("W", [1, 2, 15, 16, 17, 64, 299, 300, 10000])
@pytest.mark.parametrize("Q", [1, 3])
@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_paged_sliding_window(W, Q, kernel):
    c = case_on_gpu(small(15, window=W, q_len=Q, num_q_heads=4, num_splits=0))
    assert_parity(run_gpu(c, kernel=kernel), oracle_full(c), "f16", f"W={W} Q={Q}")


@pytest.mark.parametrize("Q", [2, 3, 4])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_multi_token_queries(Q, D, kernel):
    c = case_on_gpu(small(16, q_len=Q, head_dim=D, seq_lens=(3, 50, 257, 2), num_splits=2))
    assert_parity(run_gpu(c, kernel=kernel), oracle_full(c), "f16", f"Q={Q} D={D}")


@pytest.mark.parametrize("kv", ["f16", "int8"])
@pytest.mark.parametrize("kernel", KERNELS)
def test_forward_split_decode_counts_agree(kv, kernel):
    c = case_on_gpu(small(17, kv_dtype=kv, seq_lens=(5, 123, 700, 0), q_len=2, window=250))
    want = oracle_full(c)
    outs = {}
    for S in (1, 2, 3, 8, 0, 64, 256):
        outs[S] = run_gpu(c, kernel=kernel, num_splits=S)
        assert_parity(outs[S], want, kv, f"S={S}")
    base = outs[1].float()
    for S, o in outs.items():
        assert (o.float() - base).abs().max().item() <= 2 * TOL[kv]


@pytest.mark.parametrize("kernel", KERNELS)
def test_page_permutation_is_bit_exact_on_gpu(kernel):
    c = case_on_gpu(small(18, seq_lens=(40, 333), q_len=2, num_splits=3))
    base = run_gpu(c, kernel=kernel).clone()
    n = c.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5)).to(DEV)
    k2 = torch.empty_like(c.k_cache)
    v2 = torch.empty_like(c.v_cache)
    k2[perm] = c.k_cache
    v2[perm] = c.v_cache
    c.k_cache, c.v_cache = k2, v2
    c.block_table = perm[c.block_table.long()].to(torch.int32)
    got = run_gpu(c, kernel=kernel)
    assert torch.equal(got.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("splits", [1, 5])
@pytest.mark.parametrize("kernel", KERNELS)
def test_uniform_v_returns_v_bit_exact(splits, kernel):
    c = case_on_gpu(small(19, seq_lens=(9, 300), num_splits=splits))
    c.v_cache = torch.full_like(c.v_cache, 0.7)
    got = run_gpu(c, kernel=kernel)
    assert torch.all(got == torch.tensor(0.7, dtype=torch.float16)).item()


def _shape_scores(c, a_of_j):
    """Keys k_j = a_j * ones and queries 0.25 * ones, so that key j scores
    scale * 0.25 * D * a_j for every row: the running maximum can be made to
    climb page after page (a rescale of the accumulators on every page), to
    fall (none after the first), or to jump between pages."""
    P = c.workload.page_size
    D = c.q.shape[-1]
    c.q = torch.full_like(c.q, 0.25)
    for b, L in enumerate(c.seq_lens_host.tolist()):
        j = torch.arange(L)
        pages = c.block_table[b].cpu()[j // P].long()
        a = torch.tensor([a_of_j(int(x), L) for x in j], dtype=torch.float32)
        rows = (a[:, None, None] * torch.ones(1, c.k_cache.shape[2], D)).to(torch.float16)
        c.k_cache[pages.to(DEV), (j % P).to(DEV)] = rows.to(DEV)


@pytest.mark.parametrize("pattern", ["rising", "falling", "zigzag"])
@pytest.mark.parametrize("splits", [1, 5])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("kernel", KERNELS)
def test_score_ramps_exercise_the_rescale(pattern, splits, D, kernel):
    # about 150 natural-log units of score over the sequence: 8 or more per
    # 16-key page when rising, beyond the lazy reference's slack of 8 (base 2)
    top = 150.0 / (0.25 * D / np.sqrt(D))
    fn = {"rising": lambda j, L: top * j / L,
          "falling": lambda j, L: top * (1 - j / L),
          "zigzag": lambda j, L: top * ((j // 16) % 2) * (0.5 + 0.5 * j / L)}[pattern]
    c = case_on_gpu(small(23, seq_lens=(300, 47, 1), head_dim=D, q_len=2, num_splits=splits))
    _shape_scores(c, fn)
    assert_parity(run_gpu(c, kernel=kernel), oracle_full(c), "f16", f"{pattern} D={D}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_q_lens_null_equals_ones(kernel):
    c = case_on_gpu(small(20, num_splits=2))
    a = run_gpu(c, kernel=kernel, use_q_lens=False)
    b = run_gpu(c, kernel=kernel, use_q_lens=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
@pytest.mark.parametrize("kernel", KERNELS)
def test_partials_then_combine_equals_attention(kv, kernel):
    c = case_on_gpu(small(21, kv_dtype=kv, q_len=2, seq_lens=(0, 90, 500), num_splits=6))
    ref = run_gpu(c, kernel=kernel)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens,
                           c.max_q_len, kv, kernel)
    nbytes = pda.partials_bytes(dims, c.window, 6)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    S = pda.paged_decode_partials(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                  c.q_lens, c.scale, c.window, 6, ws, c.k_scale, c.v_scale,
                                  kv_dtype=kv, max_q_len=c.max_q_len, kernel=kernel)
    T, Hq, D = c.q.shape
    po, pml = pda.partials_views(ws, T, Hq, S, D)
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float16, device=DEV)
    pda.split_combine(po, pml, out, S)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # the partials themselves combine, in the oracle, to the oracle's answer
    mixed = oracle.split_combine(po.cpu().numpy(), pml[..., 0].cpu().numpy(),
                                 pml[..., 1].cpu().numpy(), base=2.0)
    assert_parity(torch.from_numpy(mixed), oracle_full(c), kv, "oracle-combined partials")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("D", [128, 256])
def test_workspace_reuse(kernel, D):
    """One workspace serves repeated calls, whatever it held before (here:
    NaN partials); results repeat bit for bit."""
    c = case_on_gpu(small(22, head_dim=D, q_len=2, seq_lens=(0, 70, 600, 33), num_splits=5))
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens,
                           c.max_q_len, "f16", kernel)
    nbytes = pda.workspace_bytes(dims, c.window, 5)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    # Poison the partials: a merge that read them before they were written
    # would produce NaN.
    ws.view(torch.float32).fill_(float("nan"))
    outs = []
    for _ in range(3):
        out = torch.full(tuple(c.q.shape), float("nan"), dtype=torch.float16, device=DEV)
        pda.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                   c.q_lens, c.scale, c.window, 5, out, workspace=ws,
                                   max_q_len=c.max_q_len, kernel=kernel)
        torch.cuda.synchronize()
        outs.append(out)
    assert_parity(outs[0], oracle_full(c), "f16", "reused workspace")
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("T", [5, 90])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("S", [1, 2, 7, 16, 17, 64, 65, 200, 256])
def test_split_combine_vs_oracle(D, S, T):
    # 15 rows: each row's dims are cut into the most slices (2 at D=128, 4 at
    # D=256); 270 rows (more than the compute units): one slice per row
    g = torch.Generator(device=DEV).manual_seed(S * D + T)
    Hq = 3
    m = torch.randn(T, Hq, S, generator=g, device=DEV) * 4
    l = torch.rand(T, Hq, S, generator=g, device=DEV) * 3 + 0.1
    # o_s = l_s * (a softmax-weighted mean of N(0,1) values), as a split writes it
    po = l[..., None] * torch.randn(T, Hq, S, D, generator=g, device=DEV)
    empty = torch.rand(T, Hq, S, generator=g, device=DEV) < 0.3
    empty[0, 0] = True  # a row with every split empty
    m[empty] = float("-inf")
    l[empty] = 0.0
    po[empty] = float("nan")  # never read
    pml = torch.stack([m, l], dim=-1).contiguous()
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float16, device=DEV)
    pda.split_combine(po, pml, out, S)
    torch.cuda.synchronize()
    want = oracle.split_combine(po.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), base=2.0)
    assert np.all(out[0, 0].cpu().numpy() == 0)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
    assert err <= 2e-3, err


# ---------------------------------------------------------------------------
# Benchmark workloads at full size, in the bench's launch configuration
# ---------------------------------------------------------------------------


def units_parity(c, got, units, workers=16):
    """Compare the (sequence, KV head) units of a full-size output with the
    oracle run on each unit alone (its pages gathered from the pool). The
    oracle runs in a pool of host threads (its numpy work releases the
    interpreter lock), up to `workers` units at a time, each with a
    single-threaded BLAS."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    assert torch.isfinite(got.float()).all()
    G = c.q.shape[1] // c.workload.num_kv_heads
    host = got.cpu()
    worst = 0.0
    # one BLAS thread per worker: nested BLAS threads oversubscribe the cores
    with threadpool_limits(limits=1), ThreadPoolExecutor(
            max_workers=max(1, min(workers, os.cpu_count() or 1))) as ex:
        futs = []
        for b, g in units:
            sub = unit_subcase(c, b, g)  # device gathers stay on this thread
            futs.append(((b, g), ex.submit(oracle.paged_decode_attention, **sub)))
        for (b, g), f in futs:
            want = f.result()  # [Q, G, D]
            off = int(c.q_lens_host[:b].sum())
            Q = int(c.q_lens_host[b])
            part = host[off:off + Q, g * G:(g + 1) * G]
            worst = max(worst, assert_parity(part, want, c.kv_dtype, f"unit ({b},{g})"))
    return worst


def all_units(c):
    return [(b, g) for b in range(c.workload.batch) for g in range(c.workload.num_kv_heads)]


def sampled_parity(c, units, kernel):
    got = run_gpu(c, kernel=kernel)
    return got, units_parity(c, got, units)


@pytest.mark.parametrize("kernel", KERNELS)
def test_full_gqa4_d128_b8_l4096(kernel):
    c = case_on_gpu(WORKLOADS["gqa4_d128_b8_l4096"])
    got = run_gpu(c, kernel=kernel)
    assert_parity(got, oracle_full(c), "f16", "gqa4 full")


@pytest.mark.parametrize("over", [dict(layout="HND"), dict(page_size=64),
                                  dict(identity_table=True), dict(num_splits=8)])
def test_full_gqa4_d128_b8_l4096_variants(over):
    """The headline shape in the bench's variant cells (HND layout, 64-key
    pages, identity table, a caller's 8 splits), full comparison."""
    c = case_on_gpu(WORKLOADS["gqa4_d128_b8_l4096"].with_(**over))
    assert_parity(run_gpu(c), oracle_full(c), "f16", f"gqa4 {over}")


@pytest.mark.parametrize("window", [0, 4096])
@pytest.mark.parametrize("B", [1, 2, 3, 8, 32])
@pytest.mark.parametrize("kernel", KERNELS)
def test_full_gqa6_d256_l16384(B, window, kernel):
    """Every (sequence, KV head) unit of every batch of the sweep."""
    w = WORKLOADS["gqa6_d256_l16384"].with_(batch=B, window=window)
    c = case_on_gpu(w)
    sampled_parity(c, all_units(c), kernel)


@pytest.mark.parametrize("kernel", KERNELS)
def test_full_verify_q3_d128_b32(kernel):
    """Every unit of the ragged verify batch (two empty sequences among
    them), at its stated 8 splits."""
    c = case_on_gpu(WORKLOADS["verify_q3_d128_b32"])
    sampled_parity(c, all_units(c), kernel)


@pytest.mark.parametrize("name", ["quant_fp8_d256_b64_l32768", "quant_int8_d256_b64_l32768"])
def test_full_quantized_d256_b64_l32768(name):
    """Every unit of the quantized long-context batch on the default path,
    at its stated 8 splits."""
    c = case_on_gpu(WORKLOADS[name])
    sampled_parity(c, all_units(c), "auto")


@pytest.mark.parametrize("name", ["quant_fp8_d256_b64_l32768", "quant_int8_d256_b64_l32768"])
def test_full_quantized_d256_b64_l32768_vector(name):
    """The vector kernel on the same batch: 32 units, every KV head of 8
    sequences spread over the batch."""
    c = case_on_gpu(WORKLOADS[name])
    sampled_parity(c, [(b, g) for b in range(0, 64, 9) for g in range(4)][:32], "vector")
