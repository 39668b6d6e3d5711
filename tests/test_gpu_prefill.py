"""The long-query (prefill) kernel through the C ABI against the fp64 oracle.
It computes the same function as the decode kernels: multi-token causal
attention over the paged cache, here with hundreds of new tokens per
sequence. Tolerances as for decode (2e-3 fp16 KV, 2e-2 fp8/int8)."""

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, Workload, make_case, unit_subcase
from tests.test_gpu_parity import DEV, TOL, assert_parity, oracle_full, run_gpu

pytestmark = pytest.mark.gpu




def _ragged(seed, q_lens, ctx, **kw):
    """Sequences with their own query counts (q_lens ragged)."""
    lens = [int(c + q) for c, q in zip(ctx, q_lens)]
    base = dict(name="prefill", batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                seq_lens=tuple(lens), q_len=max(q_lens), seed=seed, num_splits=1)
    base.update(kw)
    c = make_case(Workload(**base), device=DEV)
    ql = np.array(q_lens, np.int32)
    G, D = c.q.shape[1], c.q.shape[2]
    q = torch.randn((int(ql.sum()), G, D), generator=torch.Generator(device=DEV).manual_seed(seed),
                    device=DEV).to(torch.float16)
    import dataclasses
    return dataclasses.replace(c, q=q, q_lens=torch.from_numpy(ql).to(DEV), q_lens_host=ql)


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("G", [1, 4, 7])
def test_prefill_parity(kv, D, G):
    # ragged query runs; the second sequence has fewer keys than queries
    # (its first rows see nothing), the third a long cached context
    c = _ragged(3 * G + D, q_lens=[37, 130, 300], ctx=[0, -100, 900], head_dim=D, kv_dtype=kv,
                num_q_heads=2 * G, num_kv_heads=2)
    assert_parity(run_gpu(c, num_splits=1), oracle_full(c), kv, f"prefill D={D} {kv} G={G}")


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
@pytest.mark.parametrize("table_pad,G", [(1, 1), (200, 1), (1, 4)])
def test_prefill_both_workgroup_shapes(kv, table_pad, G):
    # The same batch through a tight block table (capacity 320 keys < 4 x 300
    # new tokens) with 300 query rows per KV head: 4-wave workgroups; through
    # a roomy table (3504 keys) or with 1200 rows per KV head: 8-wave
    # workgroups at D=128, with two steps of loads in flight.
    c = _ragged(77, q_lens=[300, 61, 190], ctx=[0, 40, 10], kv_dtype=kv, table_pad=table_pad,
                num_q_heads=4 * G, num_kv_heads=4)
    cap = c.block_table.shape[1] * c.workload.page_size
    assert (4 * 300 <= cap) == (table_pad == 200)
    assert_parity(run_gpu(c, num_splits=1), oracle_full(c), kv,
                  f"prefill pad={table_pad} G={G} {kv}")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("G", [16, 48, 128])
@pytest.mark.parametrize("table_pad", [1, 300])
def test_prefill_large_groups(D, G, table_pad):
    # Workgroups whose last waves have some or no rows (G = 48: 240 of 256
    # rows with 8 waves, 96 of 128 with 4 waves or with D=256's wave pairs;
    # G = 128: two tokens per workgroup, one with the pairs).
    c = _ragged(G + table_pad + D, q_lens=[70, 9], ctx=[30, 200], table_pad=table_pad,
                num_q_heads=2 * G, num_kv_heads=2, head_dim=D)
    assert_parity(run_gpu(c, num_splits=1), oracle_full(c), "f16", f"prefill D={D} G={G}")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("window", [1, 64, 300])
@pytest.mark.parametrize("layout,P", [("NHD", 16), ("HND", 64)])
def test_prefill_window_layouts(D, window, layout, P):
    c = _ragged(window + P + D, q_lens=[200, 50], ctx=[500, 7], window=window, layout=layout,
                page_size=P, num_q_heads=12, num_kv_heads=3, head_dim=D)
    assert_parity(run_gpu(c, num_splits=1), oracle_full(c), "f16",
                  f"prefill D={D} W={window} {layout}")


@pytest.mark.parametrize("kv", ["f16", "int8"])
def test_prefill_kernel_on_short_queries_matches_decode(kv):
    """Forced on a decode-sized call, the prefill kernel must give the decode
    kernel's function."""
    w = Workload("short", batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=3,
                 seq_lens=(1, 40, 300, 0, 999), kv_dtype=kv, seed=12, num_splits=1)
    c = make_case(w, device=DEV)
    want = oracle_full(c)
    a = run_gpu(c, kernel="prefill", num_splits=1)
    b = run_gpu(c, kernel="matrix", num_splits=1)
    assert_parity(a, want, kv, "prefill kernel")
    assert (a.float() - b.float()).abs().max().item() <= 2 * TOL[kv]


def _with_seq_lens(c, lens):
    """The case with fewer keys per sequence than its block table holds, so
    that the first new tokens of a sequence may sit at negative positions and
    see no key."""
    import dataclasses
    L = np.array(lens, np.int32)
    return dataclasses.replace(c, seq_lens=torch.from_numpy(L).to(DEV), seq_lens_host=L)


@pytest.mark.parametrize("cus", [1, 3, 8])
@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
@pytest.mark.parametrize("shape", ["wide", "narrow", "negative", "window", "negative_d256"])
def test_prefill_many_items_per_workgroup(shape, kv, cus, monkeypatch):
    """The persistent grid sized for 1, 3 or 8 CUs (PDA_PREFILL_CUS), so that
    each workgroup takes many (token block, KV head, sequence) items in turn,
    as on the whole device at full size: items of other sequences and KV heads
    follow each other, token blocks past a short sequence's new tokens are
    skipped, some items have one 64-key step, and (negative) some have tokens
    that all precede the sequence's keys, hence no step at all; 8-wave (wide,
    negative, window) and 4-wave (narrow) workgroups, fp16 KV (direct loads
    into LDS) and fp8 (staged through registers). D=256 (one item per
    workgroup, whatever the CU count) takes the negative case as well. The
    output equals the oracle's, and bit for bit the output of the grid sized
    for the device."""
    if shape == "narrow":
        # 4-wave workgroups: 4 x 100 new tokens exceed the table's capacity,
        # and a KV head has 4 x 100 < 512 rows
        c = _ragged(300 + cus, q_lens=[100, 3, 40, 77], ctx=[20, 0, 90, 30], kv_dtype=kv)
    else:
        # 8-wave workgroups: a KV head has 4 x 300 >= 512 rows
        d256 = shape == "negative_d256"
        c = _ragged(310 + cus, q_lens=[300, 1, 17, 130, 64], ctx=[200, 0, 5, 700, 64], kv_dtype=kv,
                    window=40 if shape == "window" else 0, head_dim=256 if d256 else 128,
                    num_q_heads=12 if d256 else 8)
        if shape.startswith("negative"):
            c = _with_seq_lens(c, [150, 1, 10, 830, 20])
    monkeypatch.delenv("PDA_PREFILL_CUS", raising=False)
    full = run_gpu(c, num_splits=1)
    monkeypatch.setenv("PDA_PREFILL_CUS", str(cus))
    got = run_gpu(c, num_splits=1)
    assert_parity(got, oracle_full(c), kv, f"prefill {shape} {kv} on {cus} CUs")
    assert torch.equal(got, full), "the output depends on the grid size"


def test_prefill_rejects_splits():
    import paged_split_decode_amd as pda
    c = _ragged(5, q_lens=[100], ctx=[10])
    with pytest.raises(pda.PdaError):
        run_gpu(c, num_splits=4)


def sampled_tokens(c, n_per_seq, seed):
    """GPU rows of sampled (sequence, KV head, token) triples against the
    oracle on the single-token problem each one is: token i of sequence b
    attends like a one-token decode of the sequence cut at its position."""
    got = run_gpu(c, num_splits=1)
    assert torch.isfinite(got.float()).all()
    r = np.random.default_rng(seed)
    Hkv = c.workload.num_kv_heads
    G = c.q.shape[1] // Hkv
    worst = 0.0
    for b in range(len(c.seq_lens_host)):
        Q, L = int(c.q_lens_host[b]), int(c.seq_lens_host[b])
        off = int(c.q_lens_host[:b].sum())
        for i in r.choice(Q, size=min(n_per_seq, Q), replace=False):
            g = int(r.integers(Hkv))
            sub = unit_subcase(c, b, g)
            p = L - Q + int(i)
            sub.update(q=sub["q"][i:i + 1], seq_lens=np.array([p + 1], np.int32),
                       q_lens=np.array([1], np.int32))
            want = oracle.paged_decode_attention(**sub)
            part = got[off + i:off + i + 1, g * G:(g + 1) * G]
            worst = max(worst, assert_parity(part, want, c.kv_dtype, f"({b},{g},{i})"))
    return worst


@pytest.mark.parametrize("name", ["prefill_d128_b4_q2048", "chunked_d128_b8_l8192_q512",
                                  "prefill_d256_b4_q2048"])
def test_prefill_workloads_sampled(name):
    c = make_case(WORKLOADS[name], device=DEV)
    sampled_tokens(c, 12, seed=len(name))


@pytest.mark.parametrize("pattern", ["rising", "zigzag", "window_edge"])
@pytest.mark.parametrize("D", [128, 256])
def test_prefill_score_ramps_move_the_maximum(pattern, D):
    """Scores shaped so that the running maximum of a row jumps by more than
    the lazy reference's slack (8, base 2) between the two 32-key halves of a
    64-key step and across steps: rising over the sequence (about 16 base-2
    units per 32 keys), alternating per 16-key tile, and, under a window, the
    first 3 keys of every 32 scoring low. The rescale of o and l must cover
    every weight not yet multiplied into o."""
    import dataclasses
    from tests.test_gpu_parity import _shape_scores
    W = 70 if pattern == "window_edge" else 0
    c = _ragged(211 + D, q_lens=[150, 70], ctx=[400, 30], window=W, num_q_heads=16,
                num_kv_heads=4, head_dim=D)
    top = 150.0 / (0.25 * D / np.sqrt(D))
    fn = {"rising": lambda j, L: top * j / L,
          "zigzag": lambda j, L: top * ((j // 16) % 2) * (0.5 + 0.5 * j / L),
          "window_edge": lambda j, L: top * (0.2 if (j % 32) < 3 else 1.0) * (j / L)}[pattern]
    _shape_scores(c, fn)
    assert_parity(run_gpu(c, num_splits=1), oracle_full(c), "f16", f"prefill {pattern} D={D}")
