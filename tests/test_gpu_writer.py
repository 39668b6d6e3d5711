"""The KV-cache writer through the C ABI against the writer oracle: cache
bytes must be bit-identical (codes are bytes; both sides quantize with the
same fp32 division and round-to-nearest-even). Then the decode must read what
the writer wrote: decode of the GPU-written cache against the attention
oracle on the oracle-written cache (the writer-layout cell of the decode
tests)."""

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import Workload, make_case, make_write_case

pytestmark = pytest.mark.gpu

DEV = "cuda"


def run_writer(c):
    pda.write_kv_cache(c.key, c.value, c.slot_mapping, c.k_cache, c.v_cache,
                       k_scale=c.k_scale, v_scale=c.v_scale, kv_dtype=c.kv_dtype,
                       kv_layout=c.kv_layout)
    torch.cuda.synchronize()


def assert_cache_equal(c, h):
    want_k, want_v = oracle.write_kv_cache(h["key"], h["value"], h["slot_mapping"], h["k_cache"],
                                           h["v_cache"], h["kv_dtype"], h["k_scale"], h["v_scale"],
                                           h["kv_layout"])
    got_k = c.k_cache.cpu().numpy()
    got_v = c.v_cache.cpu().numpy()
    assert got_k.tobytes() == want_k.tobytes(), "K cache bytes differ"
    assert got_v.tobytes() == want_v.tobytes(), "V cache bytes differ"


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("D,P,Hkv", [(128, 16, 8), (256, 16, 4), (64, 1, 3), (256, 5, 2)])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_writer_bit_exact(kv, D, P, Hkv, T):
    c = make_write_case(T, Hkv, D, P, num_pages=64 + T, kv_dtype=kv, seed=T * 7 + D + P,
                        device=DEV)
    h = c.host()
    run_writer(c)
    assert_cache_equal(c, h)


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("P", [16, 64, 3])
def test_writer_hnd_layout(kv, P):
    c = make_write_case(200, 4, 128, P, num_pages=200 // P + 9, kv_dtype=kv, seed=P + 3,
                        device=DEV, layout="HND")
    h = c.host()
    run_writer(c)
    assert_cache_equal(c, h)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("scale", [2.0 ** -3, 1.0, 2.0 ** 4, 0.37, 3.1e-5])
def test_writer_every_fp16_value(kv, scale):
    """All 63,488 finite fp16 values (plus zeros for the rest), so every code,
    tie, subnormal and the saturation edge is hit; power-of-two scales make
    the quotients exact, so ties are real ties."""
    vals = np.arange(1 << 16, dtype=np.uint16).view(np.float16).copy()
    vals[~np.isfinite(vals)] = 0
    rng = np.random.default_rng(5)
    rng.shuffle(vals)
    c = make_write_case(64, 4, 256, 16, num_pages=8, kv_dtype=kv, seed=9, skip_frac=0.0,
                        values=vals, scale=scale, device=DEV)
    c.slot_mapping.copy_(torch.arange(64, dtype=torch.int32, device=DEV))
    h = c.host()
    run_writer(c)
    assert_cache_equal(c, h)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("scale", [1.0 / 3.0, 0.1, 0.0123, 7.7e-4, 2.9e-3])
def test_writer_every_fp16_value_inexact_scales(kv, scale):
    """Every fp16 value again at scales whose quotients are rarely exact: the
    writer first takes x * (1 / scale) and falls back to the IEEE division
    only where the codes at the two ends of a small bracket around that
    product differ; many values land next to a rounding boundary here."""
    test_writer_every_fp16_value(kv, float(np.float32(scale)))


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("Hkv,D,layout", [(16, 256, "NHD"), (32, 128, "HND"), (3, 1000, "NHD")])
def test_writer_wide_tokens(kv, Hkv, D, layout):
    """Tokens of more than 256 16-byte chunks (all heads of K): a token takes
    several workgroups."""
    c = make_write_case(45, Hkv, D, 16, num_pages=8, kv_dtype=kv, seed=Hkv + D, device=DEV,
                        layout=layout)
    h = c.host()
    run_writer(c)
    assert_cache_equal(c, h)


def test_writer_no_tokens_is_a_no_op():
    c = make_write_case(0, 2, 128, 16, num_pages=4, kv_dtype="fp8_e4m3", seed=1, device=DEV)
    before = c.k_cache.clone()
    run_writer(c)
    assert torch.equal(c.k_cache, before)


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("D,G,Q", [(128, 4, 1), (256, 6, 1), (128, 7, 3)])
def test_decode_reads_what_the_writer_wrote(kv, D, G, Q):
    """Write every sequence's keys through the GPU writer into a fresh poisoned
    pool following the case's block tables, then decode on the GPU; compare
    with the attention oracle on the oracle-written pool."""
    w = Workload("writer_layout", batch=4, num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                 q_len=Q, seq_lens=(130, 0, 47, 301), kv_dtype=kv, num_splits=3, seed=D + G)
    case = make_case(w, device=DEV)
    P = case.k_cache.shape[1]
    lens = case.seq_lens_host
    bt = case.block_table.cpu().numpy()
    slots = np.concatenate([bt[b, np.arange(L) // P] * P + np.arange(L) % P
                            for b, L in enumerate(lens)]).astype(np.int32)
    T = len(slots)
    rng = np.random.default_rng(D * G)
    dense_k = rng.standard_normal((T, 2, D)).astype(np.float16)
    dense_v = rng.standard_normal((T, 2, D)).astype(np.float16)
    scales = {}
    if kv != "f16":
        top = 448.0 if kv == "fp8_e4m3" else 127.0
        scales = dict(k_scale=(np.abs(dense_k).max(axis=(0, 2)).astype(np.float32) / top),
                      v_scale=(np.abs(dense_v).max(axis=(0, 2)).astype(np.float32) / top))
    kc = case.k_cache.clone()
    vc = case.v_cache.clone()
    h = case.host()
    ks = None if kv == "f16" else torch.from_numpy(scales["k_scale"]).to(DEV)
    vs = None if kv == "f16" else torch.from_numpy(scales["v_scale"]).to(DEV)
    pda.write_kv_cache(torch.from_numpy(dense_k).to(DEV), torch.from_numpy(dense_v).to(DEV),
                       torch.from_numpy(slots).to(DEV), kc, vc, k_scale=ks, v_scale=vs,
                       kv_dtype=kv)
    want_k, want_v = oracle.write_kv_cache(dense_k, dense_v, slots, h["k_cache"], h["v_cache"],
                                           kv, scales.get("k_scale"), scales.get("v_scale"))
    assert kc.cpu().numpy().tobytes() == want_k.tobytes()
    assert vc.cpu().numpy().tobytes() == want_v.tobytes()

    out = torch.full(case.q.shape, float("nan"), dtype=torch.float16, device=DEV)
    pda.paged_decode_attention(case.q, kc, vc, case.block_table, case.seq_lens, case.q_lens,
                               case.scale, 0, 3, out, k_scale=ks, v_scale=vs, kv_dtype=kv,
                               max_q_len=Q)
    torch.cuda.synchronize()
    h.update(k_cache=want_k, v_cache=want_v, k_scale=scales.get("k_scale"),
             v_scale=scales.get("v_scale"))
    ref = oracle.paged_decode_attention(**h)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    tol = 2e-3 if kv == "f16" else 2e-2
    assert np.abs(got - ref).max() <= tol
