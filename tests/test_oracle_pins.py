"""Pins of the fp64 oracle against things other than itself.

- brute force: a key-by-key pure-Python evaluation on tiny cases, walking the
  block table one key at a time, with the masks written as per-key predicates
  and sums taken with math.fsum;
- torch's scaled_dot_product_attention in float64 on the dense-equivalent
  problem (GQA by repeat_interleave, an explicit boolean mask);
- invariants: empty rows are zero, page-permutation bit-exactness, split-count
  independence, window == truncation, uniform V returns V, multi-token rows
  equal single-token decodes of truncated sequences;
- closed forms: one key, zero scale (mean of V), window 1, a dominant key,
  distinct per-KV-head constants (the GQA mapping), the golden two-key case.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import Workload, make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed, **kw):
    base = dict(name="tiny", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=8,
                page_size=4, seq_lens=(0, 9, 23), seed=seed)
    base.update(kw)
    base["batch"] = len(base["seq_lens"])
    return make_case(Workload(**base)).host()


def _random_tiny(seed):
    r = np.random.default_rng(1000 + seed)
    Hkv = int(r.integers(1, 3))
    G = int(r.choice([1, 2, 3, 7]))
    B = int(r.integers(1, 4))
    P = int(r.choice([4, 16]))
    Q = int(r.choice([1, 2, 3]))
    lens = tuple(int(x) for x in r.integers(0, 40, size=B))
    D = int(r.choice([4, 8, 16]))
    W = int(r.choice([0, 0, 1, 5, 100]))
    kv = str(r.choice(["f16", "f16", "fp8_e4m3", "int8"]))
    return Workload("rand", batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                    head_dim=D, page_size=P, q_len=Q, seq_lens=lens, window=W,
                    kv_dtype=kv, seed=seed, table_pad=int(r.integers(0, 3)))


# ---------------------------------------------------------------------------
# Independent evaluators
# ---------------------------------------------------------------------------


def _value_torch(codes, kv, scale):
    """Element value via torch's casts (not the oracle's decoders)."""
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if kv == "f16":
        return t.view(torch.float16).to(torch.float64) if t.dtype != torch.float16 \
            else t.to(torch.float64)
    if kv == "fp8_e4m3":
        return t.view(torch.float8_e4m3fn).to(torch.float64) * float(scale)
    return t.view(torch.int8).to(torch.float64) * float(scale)


def brute_force(h):
    q = h["q"].astype(np.float64)
    kc, vc, bt = h["k_cache"], h["v_cache"], h["block_table"]
    P, Hkv, D = kc.shape[1], kc.shape[2], kc.shape[3]
    T, Hq, _ = q.shape
    G = Hq // Hkv
    kv, W = h["kv_dtype"], h["window"]
    scale = float(np.float32(h["scale"]))
    out = np.zeros((T, Hq, D))
    t = 0
    for b, (L, Q) in enumerate(zip(h["seq_lens"], h["q_lens"])):
        L, Q = int(L), int(Q)
        for i in range(Q):
            pos = L - Q + i
            for hq in range(Hq):
                g = hq // G
                ks = 1.0 if h["k_scale"] is None else h["k_scale"][g]
                vs = 1.0 if h["v_scale"] is None else h["v_scale"][g]
                seen, scores = [], []
                for j in range(L):
                    if j > pos:
                        continue
                    if W > 0 and pos - j >= W:
                        continue
                    page, slot = int(bt[b][j // P]), j % P
                    kvec = _value_torch(kc[page, slot, g], kv, ks).tolist()
                    scores.append(scale * math.fsum(q[t, hq, d] * kvec[d] for d in range(D)))
                    seen.append((page, slot))
                if not seen:
                    continue
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                Z = math.fsum(ws)
                vals = [_value_torch(vc[pg, sl, g], kv, vs).tolist() for pg, sl in seen]
                for d in range(D):
                    out[t, hq, d] = math.fsum(w * v[d] for w, v in zip(ws, vals)) / Z
            t += 1
    return out


def sdpa_reference(h):
    """torch float64 SDPA on the dense-equivalent problem, per sequence."""
    q = torch.from_numpy(h["q"].astype(np.float64))
    kc, vc, bt = h["k_cache"], h["v_cache"], h["block_table"]
    P, Hkv, D = kc.shape[1], kc.shape[2], kc.shape[3]
    T, Hq, _ = q.shape
    G = Hq // Hkv
    kv, W = h["kv_dtype"], h["window"]
    ks = np.ones(Hkv) if h["k_scale"] is None else h["k_scale"].astype(np.float64)
    vs = np.ones(Hkv) if h["v_scale"] is None else h["v_scale"].astype(np.float64)
    out = torch.zeros(T, Hq, D, dtype=torch.float64)
    t = 0
    for b, (L, Q) in enumerate(zip(h["seq_lens"], h["q_lens"])):
        L, Q = int(L), int(Q)
        if L == 0:
            t += Q
            continue
        pages = torch.from_numpy(bt[b][: -(-L // P)].astype(np.int64))
        kd = _value_torch(kc, kv, 1.0)[pages].reshape(-1, Hkv, D)[:L]
        vd = _value_torch(vc, kv, 1.0)[pages].reshape(-1, Hkv, D)[:L]
        kd = kd * torch.from_numpy(ks)[None, :, None]
        vd = vd * torch.from_numpy(vs)[None, :, None]
        pos = torch.arange(L - Q, L)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= pos
        if W > 0:
            mask &= j > pos - W
        qq = q[t:t + Q].permute(1, 0, 2)[None]  # [1, Hq, Q, D]
        kk = kd.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        vv = vd.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, scale=float(np.float32(h["scale"])))
        o = o[0].permute(1, 0, 2)
        empty = ~mask.any(dim=1)
        o[empty] = 0.0
        out[t:t + Q] = o
        t += Q
    return out.numpy()


def run_oracle(h, **over):
    args = dict(h)
    args.update(over)
    return oracle.paged_decode_attention(**args)


# ---------------------------------------------------------------------------
# Brute force and library cross-checks
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(60))
def test_oracle_vs_brute_force_random(seed):
    h = make_case(_random_tiny(seed)).host()
    got = run_oracle(h)
    want = brute_force(h)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(60, 120))
def test_oracle_vs_torch_sdpa_random(seed):
    h = make_case(_random_tiny(seed)).host()
    np.testing.assert_allclose(run_oracle(h), sdpa_reference(h), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("D", [128, 256])
def test_oracle_vs_sdpa_full_head_dims(kv, D):
    h = _tiny(7, head_dim=D, kv_dtype=kv, q_len=2, window=6, seq_lens=(3, 40))
    np.testing.assert_allclose(run_oracle(h), sdpa_reference(h), rtol=0, atol=1e-12)


def test_tiny_workload_vs_sdpa():
    from synth import WORKLOADS
    h = make_case(WORKLOADS["tiny_d128"]).host()
    np.testing.assert_allclose(run_oracle(h), sdpa_reference(h), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------


def test_empty_rows_are_zero():
    h = _tiny(3, q_len=3, seq_lens=(0, 2, 9))
    out = run_oracle(h)
    assert np.all(out[0:3] == 0)  # L = 0
    assert np.all(out[3] == 0)  # L = 2, q_len 3: token 0 sits at position -1
    assert np.all(np.isfinite(out))
    assert np.any(out[4] != 0)


def test_page_permutation_is_bit_exact():
    h = _tiny(4, seq_lens=(17, 30, 5), pool_pages=40, q_len=2, window=7)
    base = run_oracle(h)
    r = np.random.default_rng(9)
    n = h["k_cache"].shape[0]
    perm = r.permutation(n)  # new position of old page p is perm[p]
    k2 = np.empty_like(h["k_cache"])
    v2 = np.empty_like(h["v_cache"])
    k2[perm] = h["k_cache"]
    v2[perm] = h["v_cache"]
    bt2 = perm[h["block_table"]].astype(np.int32)
    got = run_oracle(h, k_cache=k2, v_cache=v2, block_table=bt2)
    assert np.array_equal(got, base)


@pytest.mark.parametrize("kv", ["f16", "int8"])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 64])
def test_split_count_independence(S, kv):
    h = _tiny(5, q_len=3, window=11, seq_lens=(0, 2, 25, 40), batch=4, kv_dtype=kv)
    one = run_oracle(h)
    split = oracle.paged_decode_attention_split(**h, num_splits=S)
    np.testing.assert_allclose(split, one, rtol=0, atol=1e-13)


def test_window_equals_truncation():
    L, W, P = 37, 9, 4
    h = _tiny(6, batch=1, seq_lens=(L,), window=W, page_size=P)
    got = run_oracle(h)
    # Same keys, re-paged: a sequence holding only the last W keys.
    kc, vc = h["k_cache"], h["v_cache"]
    pages = h["block_table"][0]
    keys_k = np.stack([kc[pages[j // P], j % P] for j in range(L - W, L)])
    keys_v = np.stack([vc[pages[j // P], j % P] for j in range(L - W, L)])
    npg = -(-W // P)
    k2 = np.full((npg, P) + kc.shape[2:], np.nan, kc.dtype)
    v2 = np.full_like(k2, np.nan)
    k2.reshape(npg * P, *kc.shape[2:])[:W] = keys_k
    v2.reshape(npg * P, *kc.shape[2:])[:W] = keys_v
    want = run_oracle(h, k_cache=k2, v_cache=v2, seq_lens=np.array([W], np.int32),
                      block_table=np.arange(npg, dtype=np.int32)[None], window=0)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    # A window covering every key is no window.
    np.testing.assert_array_equal(run_oracle(h, window=L), run_oracle(h, window=0))


def test_uniform_v_returns_v():
    h = _tiny(8, q_len=2, seq_lens=(5, 33, 2))
    vc = np.full_like(h["v_cache"], np.float16(0.7))
    out = run_oracle(h, v_cache=vc)
    np.testing.assert_allclose(out, float(np.float16(0.7)), rtol=1e-15, atol=0)


def test_multi_token_rows_equal_truncated_single_token():
    Q, W = 3, 6
    h = _tiny(10, q_len=Q, window=W, seq_lens=(4, 19, 2))
    out = run_oracle(h)
    t = 0
    for b, L in enumerate(h["seq_lens"]):
        for i in range(Q):
            Li = int(L) - Q + i + 1  # keys token i sees, itself included
            if Li <= 0:
                assert np.all(out[t] == 0)
            else:
                sub = run_oracle(h, q=h["q"][t:t + 1], seq_lens=np.array([Li], np.int32),
                                 q_lens=np.array([1], np.int32),
                                 block_table=h["block_table"][b:b + 1])
                np.testing.assert_allclose(out[t], sub[0], rtol=0, atol=1e-15)
            t += 1


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------


def _dense_kv(h, b, g):
    P = h["k_cache"].shape[1]
    L = int(h["seq_lens"][b])
    v = [h["v_cache"][h["block_table"][b][j // P], j % P, g].astype(np.float64)
         for j in range(L)]
    return np.stack(v)


def test_single_key_returns_v0():
    h = _tiny(11, seq_lens=(1, 1), batch=2)
    out = run_oracle(h)
    for b in range(2):
        for hq in range(4):
            np.testing.assert_array_equal(out[b, hq], _dense_kv(h, b, hq // 2)[0])


def test_zero_scale_is_mean_of_visible_v():
    h = _tiny(12, seq_lens=(13, 30), batch=2, window=5, scale=0.0)
    out = run_oracle(h)
    for b, L in enumerate(h["seq_lens"]):
        for hq in range(4):
            vis = _dense_kv(h, b, hq // 2)[int(L) - 5:]
            np.testing.assert_allclose(out[b, hq], vis.mean(axis=0), rtol=0, atol=1e-15)


def test_window_one_returns_own_v():
    h = _tiny(13, q_len=2, window=1, seq_lens=(7, 20), batch=2)
    out = run_oracle(h)
    t = 0
    for b, L in enumerate(h["seq_lens"]):
        V = _dense_kv(h, b, 0), _dense_kv(h, b, 1)
        for i in range(2):
            pos = int(L) - 2 + i
            for hq in range(4):
                np.testing.assert_array_equal(out[t, hq], V[hq // 2][pos])
            t += 1


def test_dominant_key_returns_its_v():
    h = _tiny(14, batch=1, seq_lens=(20,), num_q_heads=2, num_kv_heads=1)
    kc = h["k_cache"].copy()
    q = np.zeros_like(h["q"])
    q[0, :, 0] = 1.0
    page, slot = h["block_table"][0][11 // 4], 11 % 4
    kc[h["block_table"][0][:5], :, :, 0] = 0.0
    kc[page, slot, 0, 0] = 60000.0  # score gap of 60000 * scale: exp underflows
    out = run_oracle(h, q=q, k_cache=kc, scale=1.0)
    np.testing.assert_array_equal(out[0, 0], h["v_cache"][page, slot, 0].astype(np.float64))


def test_gqa_mapping_consecutive_heads_share_kv_head():
    h = _tiny(15, num_q_heads=6, num_kv_heads=3, seq_lens=(10,), batch=1)
    vc = h["v_cache"].copy()
    for g in range(3):
        vc[:, :, g, :] = np.float16(g + 1)
    out = run_oracle(h, v_cache=vc)
    for hq in range(6):
        np.testing.assert_allclose(out[0, hq], np.full(8, float(hq // 2 + 1)), rtol=1e-15)


def test_query_head_permutation_within_group_permutes_output():
    h = _tiny(16, num_q_heads=6, num_kv_heads=2, seq_lens=(12, 7), batch=2)
    base = run_oracle(h)
    perm = [2, 0, 1, 4, 5, 3]  # stays inside each group of 3
    got = run_oracle(h, q=h["q"][:, perm])
    np.testing.assert_array_equal(got, base[:, perm])


def test_golden_two_key_example():
    with open(os.path.join(GOLDEN, "two_key_softmax.txt")) as f:
        want = [float(x) for ln in f if not ln.startswith("#") for x in ln.split()]
    P = 16
    kc = np.full((2, P, 1, 2), np.nan, np.float16)
    vc = np.full_like(kc, np.nan)
    kc[1, 0, 0] = (0, 0)
    kc[1, 1, 0] = (1, 0)
    vc[1, 0, 0] = (1, 0)
    vc[1, 1, 0] = (0, 1)
    out = oracle.paged_decode_attention(
        q=np.array([[[1, 0]]], np.float16), k_cache=kc, v_cache=vc,
        block_table=np.array([[1]], np.int32), seq_lens=np.array([2], np.int32),
        q_lens=None, scale=1.0)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-16)


# ---------------------------------------------------------------------------
# Split combine (the merge of per-split partials)
# ---------------------------------------------------------------------------


def test_split_combine_equals_one_shot_softmax():
    r = np.random.default_rng(3)
    s = r.normal(size=50) * 3
    v = r.normal(size=(50, 4))
    cuts = [0, 7, 7, 30, 50]  # the third split is empty
    m, l, o = [], [], []
    for a, z in zip(cuts[:-1], cuts[1:]):
        if a == z:
            m.append(-np.inf), l.append(0.0), o.append(np.zeros(4))
            continue
        mx = s[a:z].max()
        w = np.exp2(s[a:z] - mx)
        m.append(mx), l.append(w.sum()), o.append(w @ v[a:z])
    got = oracle.split_combine(np.array(o), np.array(m), np.array(l), base=2.0)
    w = np.exp2(s - s.max())
    np.testing.assert_allclose(got, w @ v / w.sum(), rtol=0, atol=1e-14)


def test_split_combine_all_empty_is_zero():
    got = oracle.split_combine(np.full((3, 5), np.nan), np.full(3, -np.inf), np.zeros(3))
    assert np.array_equal(got, np.zeros(5))


# ---------------------------------------------------------------------------
# Layout and page-size variants
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("P", [32, 64])
@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3"])
def test_large_pages_vs_sdpa(P, kv):
    h = _tiny(71 + P, page_size=P, seq_lens=(0, 5, 100, 200), q_len=3, window=70,
              head_dim=16, kv_dtype=kv)
    np.testing.assert_allclose(run_oracle(h), sdpa_reference(h), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv", ["f16", "int8"])
def test_hnd_layout_against_dense_attention(kv):
    """Keys placed into an HND pool ([page, head, slot, dim]) by explicit
    index arithmetic must give dense attention."""
    r = np.random.default_rng(8)
    B, Hkv, G, D, P, Q = 2, 3, 2, 8, 4, 2
    lens = [13, 6]
    num_pages = 8
    perm = r.permutation(num_pages)
    table = np.zeros((B, 4), np.int32)
    table[0, :4], table[1, :2] = perm[:4], perm[4:6]
    shape = (num_pages, Hkv, P, D)
    if kv == "f16":
        kc = np.full(shape, np.nan, np.float16)
        vc = kc.copy()
        dk = [r.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
        dv = [r.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
        ks = vs = None
        val = lambda x, s: x.astype(np.float64)  # noqa: E731
    else:
        kc = np.full(shape, 127, np.uint8)
        vc = kc.copy()
        dk = [r.integers(-127, 128, (L, Hkv, D)).astype(np.int8).view(np.uint8) for L in lens]
        dv = [r.integers(-127, 128, (L, Hkv, D)).astype(np.int8).view(np.uint8) for L in lens]
        ks, vs = np.float32([0.02, 0.03, 0.05]), np.float32([0.1, 0.07, 0.04])
        val = lambda x, s: x.view(np.int8).astype(np.float64) * s[:, None]  # noqa: E731
    for b, L in enumerate(lens):
        for j in range(L):
            for g in range(Hkv):
                kc[table[b, j // P], g, j % P] = dk[b][j, g]
                vc[table[b, j // P], g, j % P] = dv[b][j, g]
    q = r.standard_normal((B * Q, Hkv * G, D)).astype(np.float16)
    got = oracle.paged_decode_attention(q, kc, vc, table, np.int32(lens), np.int32([Q, Q]), 0.3,
                                        kv_dtype=kv, k_scale=ks, v_scale=vs, kv_layout="HND")
    for b, L in enumerate(lens):
        K, V = val(dk[b], ks), val(dv[b], vs)
        for i in range(Q):
            t, p = b * Q + i, L - Q + i
            for h in range(Hkv * G):
                sc = float(np.float32(0.3))  # the caller's fp32 scale, widened
                s = [sc * float(np.dot(q[t, h].astype(np.float64), K[j, h // G]))
                     for j in range(p + 1)]
                m = max(s)
                w = np.array([math.exp(x - m) for x in s])
                ref = (w[:, None] * V[:p + 1, h // G]).sum(0) / w.sum()
                np.testing.assert_allclose(got[t, h], ref, rtol=1e-12, atol=1e-13)


def test_hnd_writer_places_rows_by_index():
    r = np.random.default_rng(9)
    num_pages, Hkv, P, D, T = 5, 2, 4, 8, 11
    key = r.standard_normal((T, Hkv, D)).astype(np.float16)
    val = r.standard_normal((T, Hkv, D)).astype(np.float16)
    slots = r.choice(num_pages * P, T, replace=False)
    slots[3] = -1
    kc0 = np.zeros((num_pages, Hkv, P, D), np.float16)
    kc, vc = oracle.write_kv_cache(key, val, slots, kc0, kc0.copy(), kv_layout="HND")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        for g in range(Hkv):
            assert kc[s // P, g, s % P].tobytes() == key[t, g].tobytes()
            assert vc[s // P, g, s % P].tobytes() == val[t, g].tobytes()
    assert np.count_nonzero(kc) == np.count_nonzero(key[slots >= 0])
