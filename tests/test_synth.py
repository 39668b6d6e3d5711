"""The seeded generator lays inputs out as documented: tables reach only the
sequence's own pages, everything else is poison, quantization scales are
per KV head, and the same seed gives the same bytes."""

import numpy as np
import torch

from synth import WORKLOADS, Workload, algorithmic_bytes, make_case, unit_subcase


def test_tiny_workload_layout():
    c = make_case(WORKLOADS["tiny_d128"])
    assert tuple(c.k_cache.shape) == (32, 16, 2, 128)
    assert c.seq_lens_host.tolist() == [0, 37, 200]
    bt = c.block_table.numpy()
    owned = [set(bt[b, : -(-L // 16)].tolist()) for b, L in enumerate(c.seq_lens_host)]
    flat = [p for s in owned for p in s]
    assert len(flat) == len(set(flat)) == 0 + 3 + 13
    assert c.poison_page not in flat
    # padding entries point at the poison page
    for b, L in enumerate(c.seq_lens_host):
        assert set(bt[b, -(-L // 16):].tolist()) == {c.poison_page}
    k = c.k_cache.float()
    assert torch.isnan(k[c.poison_page]).all()
    unused = set(range(32)) - set(flat)
    assert all(torch.isnan(k[p]).all() for p in unused)
    last = bt[1, 37 // 16]
    assert torch.isnan(k[last, 37 % 16:]).all() and not torch.isnan(k[last, :37 % 16]).any()


def test_seeded_reproducible():
    a = make_case(WORKLOADS["tiny_d128"])
    b = make_case(WORKLOADS["tiny_d128"])
    assert torch.equal(a.q, b.q) and torch.equal(a.block_table, b.block_table)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))


def test_quantized_codes_and_scales():
    w = Workload("q", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=128,
                 seq_lens=(20, 33), kv_dtype="int8", seed=3)
    c = make_case(w)
    assert c.k_cache.dtype == torch.uint8 and c.k_scale.shape == (2,)
    codes = c.k_cache.view(torch.int8)[c.block_table[0, 0].long()]
    assert codes.abs().max() <= 127
    w8 = w.with_(kv_dtype="fp8_e4m3")
    c8 = make_case(w8)
    vals = c8.k_cache.view(torch.float8_e4m3fn)[c8.block_table[1, 0].long()].float()
    assert torch.isfinite(vals).all() and vals.abs().max() <= 448


def test_ragged_forced_zero():
    c = make_case(WORKLOADS["verify_q3_d128_b32"].with_(ragged_max=300))
    assert (c.seq_lens_host == 0).sum() >= 2
    assert c.num_tokens == 96 and c.max_q_len == 3


def test_algorithmic_bytes_formula():
    c = make_case(WORKLOADS["tiny_d128"])
    # keys: 0 + 37 + 200, 2 KV heads, D=128, fp16 K and V; q and out fp16
    assert algorithmic_bytes(c) == 237 * 2 * 128 * 2 * 2 + 3 * 4 * 128 * 2 * 2


def test_unit_subcase_identity_table():
    c = make_case(WORKLOADS["tiny_d128"])
    u = unit_subcase(c, 2, 1)
    assert u["k_cache"].shape == (13, 16, 1, 128)
    assert u["block_table"].tolist() == [list(range(13))]
    np.testing.assert_array_equal(u["q"], c.q[2:3, 2:4].numpy())


def test_workload_sizes_without_a_pool():
    """The pool-free byte and pair counts equal those of the built case."""
    from synth import (visible_pairs, workload_algorithmic_bytes, workload_lengths,
                       workload_visible_pairs)
    for w in (WORKLOADS["tiny_d128"], WORKLOADS["verify_q3_d128_b32"].with_(ragged_max=900),
              WORKLOADS["gqa6_d256_l16384"].with_(batch=2, seq_len=700, window=300)):
        c = make_case(w)
        assert workload_lengths(w).tolist() == c.seq_lens_host.tolist()
        assert workload_algorithmic_bytes(w) == algorithmic_bytes(c)
        assert workload_visible_pairs(w) == visible_pairs(c)
