"""Pools larger than 4 GiB per cache: page byte offsets past 2^32 in every
kernel family (matrix and vector decode, the prefill kernel, both layouts,
the cache writer). The sequences' pages are drawn from a 140000-page fp16
pool (4.6 GB per cache), so some sit above 2^32 bytes. Each (sequence, KV
head) unit is checked against the oracle on a compact copy of its pages.
Tolerances as in test_gpu_parity.py."""

import numpy as np
import pytest
import torch

import oracle
import paged_split_decode_amd as pda
from synth import Workload, make_case, unit_subcase

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3
POOL = 140000  # pages of 16 x 8 heads x 128 dims fp16 = 32 KiB: 4.6 GB per cache


@pytest.fixture(scope="module", params=["NHD", "HND"])
def big(request):
    w = Workload(name="big", batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 seq_lens=(2000, 777, 3001), pool_pages=POOL, seed=31, layout=request.param)
    c = make_case(w, device=DEV)
    page_bytes = c.k_cache[0].numel() * c.k_cache.element_size()
    assert int(c.block_table.max()) * page_bytes >= 1 << 32, "no page past 4 GiB"
    yield c
    del c
    torch.cuda.empty_cache()


def with_q_len(c, Q, seed):
    """The same cache with Q new tokens per sequence (fresh queries)."""
    import dataclasses
    B, Hq, D = len(c.seq_lens_host), c.q.shape[1], c.q.shape[2]
    ql = np.full(B, Q, np.int32)
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B * Q, Hq, D), generator=g, device=DEV).to(torch.float16)
    return dataclasses.replace(c, q=q, q_lens=torch.from_numpy(ql).to(DEV), q_lens_host=ql)


def check_units(c, out, what):
    Hkv = c.k_cache.shape[1 if c.kv_layout == "HND" else 2]
    G = c.q.shape[1] // Hkv
    for b in range(len(c.seq_lens_host)):
        off, Q = int(c.q_lens_host[:b].sum()), int(c.q_lens_host[b])
        for g in range(Hkv):
            want = oracle.paged_decode_attention(**unit_subcase(c, b, g))
            got = out[off:off + Q, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
            err = np.abs(got - want).max()
            assert np.isfinite(got).all() and err <= TOL, f"{what} unit ({b},{g}): {err:.3g}"


def call(c, splits, kernel):
    out = torch.full(c.q.shape, float("nan"), dtype=torch.float16, device=DEV)
    pda.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.q_lens,
                               c.scale, c.window, splits, out, max_q_len=c.max_q_len,
                               kernel=kernel, kv_layout=c.kv_layout)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kernel,splits,Q", [("matrix", 0, 3), ("matrix", 5, 1), ("auto", 1, 40)])
def test_pages_past_4gib(big, kernel, splits, Q):
    c = with_q_len(big, Q, seed=Q + splits)
    check_units(c, call(c, splits, kernel), f"{kernel} S={splits} Q={Q} {c.kv_layout}")


def test_vector_kernel_pages_past_4gib(big):
    """The vector kernel reads NHD pages of 16 keys; an HND cache is refused
    with an error before any launch."""
    c = with_q_len(big, 1, seed=2)
    if c.kv_layout == "HND":
        with pytest.raises(pda.PdaError):
            call(c, 2, "vector")
        return
    check_units(c, call(c, 2, "vector"), "vector S=2 NHD")


def test_writer_past_4gib(big):
    """fp16 rows written to slots of the highest pages read back unchanged."""
    c = big
    hnd = c.kv_layout == "HND"
    P = c.k_cache.shape[2 if hnd else 1]
    Hkv, D = c.k_cache.shape[1 if hnd else 2], c.k_cache.shape[3]
    T = 200
    used = set()
    for b, L in enumerate(c.seq_lens_host):
        used.update(c.block_table[b, :-(-int(L) // P)].tolist())
    free = [p for p in range(POOL - 1, 0, -1) if p not in used][:T]  # the highest unused pages
    pages = torch.tensor(free, device=DEV)
    assert int(pages.min()) * c.k_cache[0].numel() * 2 >= 1 << 32
    slots = (pages * P + (torch.arange(T, device=DEV) % P)).to(torch.int32)
    g = torch.Generator(device=DEV).manual_seed(9)
    key = torch.randn((T, Hkv, D), generator=g, device=DEV).to(torch.float16)
    value = torch.randn((T, Hkv, D), generator=g, device=DEV).to(torch.float16)
    pda.write_kv_cache(key, value, slots, c.k_cache, c.v_cache, kv_layout=c.kv_layout)
    torch.cuda.synchronize()
    pos = slots.long() % P
    for cache, rows in ((c.k_cache, key), (c.v_cache, value)):
        got = cache[pages, :, pos] if hnd else cache[pages, pos]
        assert torch.equal(got.view(torch.int16), rows.view(torch.int16))
