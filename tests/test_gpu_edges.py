"""Edge cases of the HIP path against the fp64 oracle, through the C ABI:
scale 0 (every visible key weighs the same: the mean of the visible V rows)
and negative scales on the matrix, vector and prefill kernels, quantized KV
with negative per-head scales, automatic balanced splits on batches whose
sequences read the same number of 16-key tiles but hold different lengths,
and the softmax weights of the matrix kernels (numerator and denominator
must weigh each key alike, which only a V with a large common offset shows).

Tolerances as in test_gpu_parity.py: 2e-3 for fp16 KV, 2e-2 against the
dequantized-KV oracle for fp8 / int8 KV."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import Workload, make_case
from tests.test_gpu_parity import DEV, TOL, assert_parity, oracle_full, run_gpu

pytestmark = pytest.mark.gpu


def _case(seed, lens, q_len=1, **kw):
    base = dict(name="edge", batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                seq_lens=tuple(lens), q_len=q_len, seed=seed, pool_pages=0, num_splits=0)
    base.update(kw)
    return make_case(Workload(**base), device=DEV)


# Kernel families and the query count that routes a call to each: the
# prefill kernel takes calls with more than 32 query rows per KV head.
FAMILIES = [("matrix", 2), ("vector", 2), ("prefill", 40)]


@pytest.mark.parametrize("kernel,Q", FAMILIES)
@pytest.mark.parametrize("D,kv", [(128, "f16"), (256, "f16"), (256, "fp8_e4m3"), (128, "int8")])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_zero_scale_gives_the_mean_of_visible_v(kernel, Q, D, kv, splits):
    """scale = 0: every score is 0, so each row is the plain mean of the V
    rows it sees (the closed form the oracle is pinned to)."""
    if kernel == "prefill" and splits > 1:
        pytest.skip("the prefill kernel runs one split")
    c = _case(201 + D, (0, 1, 45, 300), q_len=Q, head_dim=D, kv_dtype=kv, window=0)
    want = oracle_full(c, scale=0.0)
    got = run_gpu(c, scale=0.0, num_splits=splits, kernel=kernel)
    assert_parity(got, want, kv, f"{kernel} scale 0")
    # the closed form itself, on one row: token Q-1 of sequence 2 sees its
    # 45 keys
    h = c.host()
    t = int(c.q_lens_host[:2].sum()) + Q - 1
    keys = oracle.attention._gather_keys(oracle.as_nhd(h["v_cache"]), h["block_table"][2], 45, 0,
                                         kv, None if h["v_scale"] is None else h["v_scale"][0])
    np.testing.assert_allclose(want[t, 0], keys.mean(axis=0), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kernel,Q", FAMILIES)
@pytest.mark.parametrize("D,kv", [(128, "f16"), (256, "f16"), (256, "fp8_e4m3"),
                                  (128, "int8"), (256, "int8")])
@pytest.mark.parametrize("scale", [-0.37, -1.0 / 16])
def test_negative_scale(kernel, Q, D, kv, scale):
    """A negative scale reverses the order of the scores: the kernels fold
    its sign into q so that the running maximum is that of the scaled
    scores."""
    c = _case(211 + D, (3, 77, 300, 1), q_len=Q, head_dim=D, kv_dtype=kv)
    assert_parity(run_gpu(c, scale=scale, num_splits=3 if kernel != "prefill" else 1,
                          kernel=kernel), oracle_full(c, scale=scale), kv,
                  f"{kernel} scale {scale}")


@pytest.mark.parametrize("kernel,Q", FAMILIES)
@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("sign", [(-1, 1), (1, -1), (-1, -1)])
def test_negative_kv_scales(kernel, Q, kv, sign):
    """Per-head K and V scales below zero (a code's value is code * scale):
    a negative K scale flips the scores like a negative attention scale, a
    negative V scale the output."""
    c = _case(223, (5, 140, 260), q_len=Q, head_dim=256, kv_dtype=kv, num_q_heads=8,
              num_kv_heads=2)
    ks = c.k_scale.clone()
    ks[0] *= sign[0]  # head 0 flipped, head 1 not
    vs = c.v_scale.clone()
    vs[1] *= sign[1]
    c = dataclasses.replace(c, k_scale=ks, v_scale=vs)
    assert_parity(run_gpu(c, num_splits=2 if kernel != "prefill" else 1, kernel=kernel),
                  oracle_full(c), kv, f"{kernel} signs {sign}")


# ---------------------------------------------------------------------------
# Balanced splits: equal tile counts, different lengths
# ---------------------------------------------------------------------------


def _tiles(L, Q, W):
    lo = max(0, L - Q + 1 - W) if W > 0 else 0
    return max(0, -(-L // 16) - lo // 16)


@pytest.mark.parametrize("lens,Q,W", [
    ((4097, 4100, 4111), 1, 0),
    ((4097, 4100, 4111), 3, 0),
    ((4111, 4097, 4100, 4098), 2, 0),
    ((16385, 16390, 16398), 1, 4096),
    ((16386, 16391, 16399), 3, 4096),
])
@pytest.mark.parametrize("D", [128, 256])
def test_balanced_equal_tiles_different_lengths(lens, Q, W, D):
    """Automatic splits see a uniform batch when every sequence reads as many
    16-key tiles with as many new tokens; each workgroup must still take its
    own sequence's length (masks and key range)."""
    assert len({_tiles(L, Q, W) for L in lens}) == 1
    c = _case(231, lens, q_len=Q, window=W, head_dim=D, num_q_heads=4 * (D // 64),
              num_kv_heads=D // 64)
    dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens, c.max_q_len,
                           "f16", "matrix")
    assert pda.resolve_splits(dims, W, 0) >= 2  # balanced mode is on
    assert_parity(run_gpu(c, num_splits=0, kernel="matrix"), oracle_full(c), "f16",
                  f"lens {lens} Q={Q} W={W}")


@pytest.mark.parametrize("B", [65, 130])
def test_balanced_equal_tiles_different_lengths_over_64(B):
    """The same with more than 64 sequences (a lane of the search holds
    several sequences): lengths 16 k + 1 .. 16 k + 16 all read k + 1 tiles."""
    r = np.random.default_rng(B)
    lens = tuple(int(x) for x in 16 * 40 + 1 + r.integers(0, 16, size=B))
    assert len({_tiles(L, 1, 0) for L in lens}) == 1
    c = _case(239, lens, num_q_heads=4, num_kv_heads=1)
    assert_parity(run_gpu(c, num_splits=0, kernel="matrix"), oracle_full(c), "f16",
                  f"B={B} equal tiles")


# ---------------------------------------------------------------------------
# Softmax weights: numerator and denominator weigh each key alike
# ---------------------------------------------------------------------------


def _f16_round_up_exponents(qk, count, rng):
    """fp16 values a in (-1, 0) whose weight p = 2^(a * qk) (fp32 product,
    exponential to fp32, as the kernels compute it with a row maximum of 0)
    rounds UP to fp16 by 0.3 to 0.45 of an fp16 ulp: every key's rounded
    weight then errs the same way."""
    h = np.arange(0x8001, 0xBC00, dtype=np.uint16).view(np.float16)  # -2^-24 .. -1 (excl.)
    a = h.astype(np.float32)
    x = (a * np.float32(qk)).astype(np.float32)
    p = np.exp2(x.astype(np.float64)).astype(np.float32)
    ulp = np.spacing(p.astype(np.float16)).astype(np.float64)  # fp16 ulp at p
    lo = p.astype(np.float16).astype(np.float64)
    lo = np.where(lo > p, lo - ulp, lo)  # fp16 value just below p
    frac = (p.astype(np.float64) - lo) / ulp
    ok = (frac > 0.55) & (frac < 0.7) & (p > 0.5)
    pick = a[ok]
    assert len(pick) > 50
    return rng.choice(pick, size=count)


@pytest.mark.parametrize("kernel,Q", [("matrix", 1), ("matrix", 3), ("prefill", 40)])
@pytest.mark.parametrize("D", [128, 256])
def test_weights_agree_between_numerator_and_denominator(kernel, Q, D):
    """V = 3.9 + 0.01 N(0,1) and scores whose fp16-rounded weights all err
    upward. The matrix kernels round each weight p to fp16 for P.V; the
    result stays a weighted mean of the V rows (error far below the output's
    own fp16 rounding) only if the denominator adds the same rounded
    weights. The test first shows, on the host, that a denominator of the
    unrounded weights misses the bound it then holds the GPU to."""
    L = 700
    scale = float(np.float32(0.6931471805599453))  # ln 2: scale * log2 e is about 1
    qk = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    c = _case(241 + D + Q, (L,), q_len=Q, head_dim=D, num_q_heads=2, num_kv_heads=1,
              num_splits=1)
    rng = np.random.default_rng(D + Q)
    a = _f16_round_up_exponents(qk, L, rng)
    # The first key of every page has the largest score (0, so p = 1): every
    # wave's first page then sets its reference maximum to 0, and all waves
    # and splits form the same weights.
    a[::16] = 0.0
    bt = c.block_table[0].long()
    j = torch.arange(L)
    pages, slots = bt[(j // 16).to(DEV)], (j % 16).to(DEV)
    k = torch.zeros((L, D), dtype=torch.float16)
    k[:, 0] = torch.from_numpy(a.astype(np.float16))
    v = (3.9 + 0.01 * torch.from_numpy(rng.standard_normal((L, D)))).to(torch.float16)
    kc, vc = c.k_cache.clone(), c.v_cache.clone()
    kc[pages, slots, 0] = k.to(DEV)
    vc[pages, slots, 0] = v.to(DEV)
    q = torch.zeros_like(c.q)
    q[..., 0] = 1.0  # score of key j: a_j (exact)
    c = dataclasses.replace(c, q=q, k_cache=kc, v_cache=vc, scale=scale)
    want = oracle_full(c)

    # Host model of the last token's rows (it sees every key): weights as
    # the kernels form them, rounded to fp16 for P.V.
    p = np.exp2((a.astype(np.float32) * qk).astype(np.float64)).astype(np.float32)
    p16 = p.astype(np.float16).astype(np.float64)
    vv = v.numpy().astype(np.float64)
    half_ulp = lambda x: np.spacing(np.abs(x).astype(np.float16)).astype(np.float64) / 2  # noqa
    ref = want[-1, 0]
    bound = half_ulp(ref) + 1e-4
    consistent = ((p16 @ vv) / p16.sum()).astype(np.float16).astype(np.float64)
    mixed = ((p16 @ vv) / p.astype(np.float64).sum()).astype(np.float16).astype(np.float64)
    assert np.all(np.abs(consistent - ref) <= bound)
    assert np.any(np.abs(mixed - ref) > bound), "the case does not separate the two"

    got = run_gpu(c, num_splits=1, kernel=kernel)
    assert_parity(got, want, "f16", f"{kernel} offset V")
    g = got.cpu().numpy().astype(np.float64)
    err = np.abs(g - want)
    lim = half_ulp(want) + 1e-4
    assert np.all(err <= lim), f"max excess {np.max(err - lim):.3g}"
