"""Pins of the KV-cache writer oracle (oracle/kv_writer.py) against things
other than itself: torch's e4m3fn cast, the format's own decoder over every
code, Python's round-half-even, fp64 arithmetic, a flat-index formulation of
the slot writes, and attention read back through the page table. Planted
mistakes at the end check that these pins catch plausible errors."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.kv_writer as kw
from tests.test_oracle_pins import sdpa_reference

FINITE_CODES = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_matches_torch_cast_inside_range():
    # every finite fp16 value below torch's NaN threshold (464), plus random fp32
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float32)
    h = h[np.abs(h) < 464.0]
    r = np.random.default_rng(0)
    f = (r.standard_normal(200_000) * np.exp2(r.integers(-14, 9, 200_000))).astype(np.float32)
    f = f[np.abs(f) < 464.0]
    for x in (h, f):
        np.testing.assert_array_equal(oracle.encode_e4m3fn(x), _torch_e4m3(x))


def test_e4m3_saturates_and_never_emits_nan():
    x = np.array([448.0, 448.5, 463.9, 464.0, 464.1, 500.0, 1e4, 3e38], np.float32)
    codes = oracle.encode_e4m3fn(np.concatenate([x, -x]))
    assert codes.tolist() == [0x7E] * len(x) + [0xFE] * len(x)


def test_e4m3_roundtrip_every_code():
    vals = oracle.decode_e4m3fn(np.array(FINITE_CODES))
    np.testing.assert_array_equal(oracle.encode_e4m3fn(vals), np.array(FINITE_CODES, np.uint8))


def test_e4m3_ties_to_even_at_every_midpoint():
    # positive codes are ordered like their values; the midpoint of codes c
    # and c + 1 must go to the one with an even mantissa (the even code)
    for c in range(0, 0x7E):
        a, b = oracle.decode_e4m3fn(np.array([c, c + 1]))
        mid = (a + b) / 2
        got = int(oracle.encode_e4m3fn(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), (c, mid, got)
        # just off the midpoint it goes to the nearer code
        assert int(oracle.encode_e4m3fn(np.array([np.nextafter(mid, 0)]))[0]) == c
        assert int(oracle.encode_e4m3fn(np.array([np.nextafter(mid, 1e9)]))[0]) == c + 1


def test_int8_rounding_matches_python_round():
    r = np.random.default_rng(1)
    x = np.concatenate([np.arange(-140, 140, 0.25), r.standard_normal(5000) * 60,
                        [126.5, 127.5, -127.5, -128.5, 1e9, -1e9]])
    want = [max(-127, min(127, round(float(v)))) for v in x]  # Python rounds half to even
    assert oracle.encode_int8(x).view(np.int8).tolist() == want


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
def test_quantize_divides_in_fp32(kv):
    r = np.random.default_rng(2)
    x = (r.standard_normal((3, 5, 16)) * 3).astype(np.float16)
    scale = (r.random(5) * 0.05 + 0.001).astype(np.float32)
    got = oracle.quantize(x, scale, kv)
    # fp32 quotient through exact fp64 division rounded once to fp32 (no
    # double-rounding issue: 53 >= 2 * 24 + 2)
    q = np.array([[[np.float32(float(x[t, h, d]) / float(scale[h])) for d in range(16)]
                   for h in range(5)] for t in range(3)], np.float32)
    enc = kw.encode_e4m3fn if kv == "fp8_e4m3" else kw.encode_int8
    np.testing.assert_array_equal(got, enc(q))


def _pool(num_pages, P, Hkv, D, kv):
    if kv == "f16":
        return np.full((num_pages, P, Hkv, D), np.nan, np.float16)
    return np.full((num_pages, P, Hkv, D), 0x7F if kv == "fp8_e4m3" else 127, np.uint8)


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
def test_writes_land_at_their_flat_slot(kv):
    r = np.random.default_rng(3)
    num_pages, P, Hkv, D, T = 9, 4, 3, 8, 20
    key = r.standard_normal((T, Hkv, D)).astype(np.float16)
    val = r.standard_normal((T, Hkv, D)).astype(np.float16)
    slots = r.choice(num_pages * P, size=T, replace=False).astype(np.int64)
    slots[[2, 7, 11]] = -1
    ks = vs = None
    if kv != "f16":
        ks, vs = (r.random(Hkv) * 0.02 + 0.005).astype(np.float32), np.full(Hkv, 0.01, np.float32)
    kc0, vc0 = _pool(num_pages, P, Hkv, D, kv), _pool(num_pages, P, Hkv, D, kv)
    kc, vc = oracle.write_kv_cache(key, val, slots, kc0, vc0, kv, ks, vs)
    flat_k, flat_v = kc.reshape(num_pages * P, Hkv, D), vc.reshape(num_pages * P, Hkv, D)
    written = set()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        written.add(int(s))
        if kv == "f16":
            assert flat_k[s].tobytes() == key[t].tobytes()
            assert flat_v[s].tobytes() == val[t].tobytes()
        else:
            assert np.array_equal(flat_k[s], oracle.quantize(key[t:t + 1], ks, kv)[0])
            assert np.array_equal(flat_v[s], oracle.quantize(val[t:t + 1], vs, kv)[0])
    untouched = [i for i in range(num_pages * P) if i not in written]
    assert kc0.reshape(num_pages * P, Hkv, D)[untouched].tobytes() == flat_k[untouched].tobytes()


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
def test_slots_past_the_pool_leave_both_caches_untouched(kv, layout):
    """A token whose slot is at or past num_pages * P (the first slot that
    does not exist, and ones far beyond it) writes nothing: both caches keep
    their bytes. The tokens of the same call with in-pool slots are written,
    so the call is not a no-op."""
    r = np.random.default_rng(5)
    num_pages, P, Hkv, D, T = 5, 4, 2, 8, 9
    n_slots = num_pages * P
    key = r.standard_normal((T, Hkv, D)).astype(np.float16)
    val = r.standard_normal((T, Hkv, D)).astype(np.float16)
    slots = np.array([n_slots, n_slots + 1, 3, n_slots + P, 2 * n_slots, 17, 1 << 30,
                      n_slots + 7, 0], np.int64)
    ks = vs = None
    if kv != "f16":
        ks, vs = np.full(Hkv, 0.02, np.float32), np.full(Hkv, 0.03, np.float32)
    kc0, vc0 = _pool(num_pages, P, Hkv, D, kv), _pool(num_pages, P, Hkv, D, kv)
    if layout == "HND":
        kc0, vc0 = np.ascontiguousarray(kc0.swapaxes(1, 2)), np.ascontiguousarray(vc0.swapaxes(1, 2))
    # only the out-of-pool tokens: nothing may change
    out = slots >= n_slots
    kc, vc = oracle.write_kv_cache(key[out], val[out], slots[out], kc0, vc0, kv, ks, vs,
                                   kv_layout=layout)
    assert kc.tobytes() == kc0.tobytes() and vc.tobytes() == vc0.tobytes()
    # the whole call: exactly the in-pool slots change (each row of D elements)
    kc, vc = oracle.write_kv_cache(key, val, slots, kc0, vc0, kv, ks, vs, kv_layout=layout)
    to_flat = (lambda c: c.swapaxes(1, 2).reshape(n_slots, Hkv, D)) if layout == "HND" else (
        lambda c: c.reshape(n_slots, Hkv, D))
    changed = {i for i in range(n_slots)
               if to_flat(kc)[i].tobytes() != to_flat(kc0)[i].tobytes()}
    assert changed == {int(x) for x in slots if x < n_slots}
    changed_v = {i for i in range(n_slots)
                 if to_flat(vc)[i].tobytes() != to_flat(vc0)[i].tobytes()}
    assert changed_v == changed


def _written_case(kv, seed=4):
    """A batch written token by token through the writer into a poisoned
    pool, following a random page table; returns the decode inputs."""
    r = np.random.default_rng(seed)
    B, Hkv, G, D, P = 3, 2, 3, 16, 4
    lens = np.array([11, 0, 7])
    num_pages = 12
    perm = r.permutation(num_pages)
    table = np.zeros((B, 3), np.int32)
    cur = 0
    for b in range(B):
        n = -(-lens[b] // P)
        table[b, :n] = perm[cur:cur + n]
        cur += n
    dense_k = [r.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    dense_v = [r.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    ks = vs = None
    if kv != "f16":
        ks = (r.random(Hkv) * 0.01 + 0.01).astype(np.float32)
        vs = (r.random(Hkv) * 0.01 + 0.01).astype(np.float32)
    kc, vc = _pool(num_pages, P, Hkv, D, kv), _pool(num_pages, P, Hkv, D, kv)
    for b in range(B):
        slots = np.array([table[b, j // P] * P + j % P for j in range(lens[b])], np.int64)
        kc, vc = oracle.write_kv_cache(dense_k[b], dense_v[b], slots, kc, vc, kv, ks, vs)
    q = r.standard_normal((B, Hkv * G, D)).astype(np.float16)
    h = dict(q=q, k_cache=kc, v_cache=vc, block_table=table, seq_lens=lens.astype(np.int32),
             q_lens=np.ones(B, np.int32), scale=0.25, window=0, kv_dtype=kv, k_scale=ks,
             v_scale=vs)
    return h, dense_k, dense_v


@pytest.mark.parametrize("kv", ["f16", "fp8_e4m3", "int8"])
def test_written_cache_reads_back_through_the_table(kv):
    h, dk, dv = _written_case(kv)
    got = oracle.paged_decode_attention(**h)
    np.testing.assert_allclose(got, sdpa_reference(h), rtol=0, atol=1e-12)
    if kv == "f16":
        # attention over the dense fp16 rows, written directly in fp64
        G = h["q"].shape[1] // dk[0].shape[1]
        for b, L in enumerate(h["seq_lens"]):
            for qh in range(h["q"].shape[1]):
                if L == 0:
                    assert np.all(got[b, qh] == 0)
                    continue
                s = [h["scale"] * float(np.dot(h["q"][b, qh].astype(np.float64),
                                               dk[b][j, qh // G].astype(np.float64)))
                     for j in range(L)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                ref = sum(wj * dv[b][j, qh // G].astype(np.float64) for j, wj in enumerate(w))
                np.testing.assert_allclose(got[b, qh], ref / sum(w), rtol=1e-12, atol=1e-13)
    else:
        # every written key sits, quantized, at its table position
        for b, L in enumerate(h["seq_lens"]):
            for j in range(L):
                page, pos = h["block_table"][b, j // 4], j % 4
                want = oracle.quantize(dk[b][j:j + 1], h["k_scale"], kv)[0]
                assert np.array_equal(h["k_cache"][page, pos], want)


# --- planted mistakes -------------------------------------------------------


def _swapped_page_slot(key, value, slot_mapping, k_cache, v_cache, kv_dtype="f16",
                       k_scale=None, v_scale=None):
    P = k_cache.shape[1]
    num_pages = k_cache.shape[0]
    remap = [(s % num_pages) * P + s // num_pages if s >= 0 else s for s in slot_mapping]
    return _ORIG_WRITE(key, value, np.array(remap), k_cache, v_cache, kv_dtype, k_scale, v_scale)


def _ties_away(x):
    v = np.asarray(x, np.float64)
    return _ORIG_E4M3(np.sign(v) * (np.abs(v) + 1e-12 * np.abs(v)))


def _no_saturation(x):
    v = np.asarray(x, np.float64)
    return np.where(np.abs(v) >= 448.0, np.uint8(0x7F) | (np.signbit(v) * 0x80).astype(np.uint8),
                    _ORIG_E4M3(np.clip(v, -448, 448)))


def _slots_wrap_around(key, value, slot_mapping, k_cache, v_cache, kv_dtype="f16",
                       k_scale=None, v_scale=None, kv_layout="NHD"):
    n = as_nhd_shape(k_cache, kv_layout)
    wrapped = np.array([s % n if s >= 0 else s for s in np.asarray(slot_mapping).tolist()])
    return _ORIG_WRITE(key, value, wrapped, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                       kv_layout=kv_layout)


def as_nhd_shape(cache, kv_layout):
    """Slots of a cache: num_pages * P."""
    return cache.shape[0] * (cache.shape[2] if kv_layout == "HND" else cache.shape[1])


def _int8_truncates(x):
    return np.clip(np.trunc(np.asarray(x, np.float64)), -127, 127).astype(np.int8).view(np.uint8)


_ORIG_WRITE = kw.write_kv_cache
_ORIG_E4M3 = kw.encode_e4m3fn


@pytest.mark.parametrize("name,target,mutant,pin", [
    ("page and slot swapped", "write_kv_cache", _swapped_page_slot,
     lambda: test_writes_land_at_their_flat_slot("f16")),
    ("slots past the pool wrap around", "write_kv_cache", _slots_wrap_around,
     lambda: test_slots_past_the_pool_leave_both_caches_untouched("int8", "HND")),
    ("ties away from zero", "encode_e4m3fn", _ties_away, test_e4m3_ties_to_even_at_every_midpoint),
    ("no saturation", "encode_e4m3fn", _no_saturation, test_e4m3_saturates_and_never_emits_nan),
    ("int8 truncation", "encode_int8", _int8_truncates, test_int8_rounding_matches_python_round),
])
def test_planted_writer_mistakes_are_caught(monkeypatch, name, target, mutant, pin):
    monkeypatch.setattr(kw, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    with pytest.raises(AssertionError):
        pin()
