"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the independent pins catch each one. A pin set that let one of
these through would not be pinning the oracle."""

import numpy as np
import pytest

import oracle.attention as oa
from synth import Workload, make_case
from tests.test_oracle_pins import brute_force, sdpa_reference


def _cases():
    ws = [
        Workload("m1", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=4,
                 q_len=3, seq_lens=(9, 22), window=5, seed=21),
        Workload("m2", batch=2, num_q_heads=6, num_kv_heads=2, head_dim=8, page_size=4,
                 seq_lens=(13, 6), kv_dtype="fp8_e4m3", seed=22),
        Workload("m3", batch=1, num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=4,
                 seq_lens=(17,), kv_dtype="int8", seed=23),
    ]
    return [make_case(w).host() for w in ws]


def _caught(h):
    got = oa.paged_decode_attention(**h)
    for ref in (sdpa_reference(h), brute_force(h)):
        if not np.allclose(got, ref, rtol=0, atol=1e-9, equal_nan=False):
            return True
    return False


def _vr_causal_off_by_one(seq_len, q_len, i, window):
    lo, hi = _ORIG_VR(seq_len, q_len, i, window)
    return lo, hi + 1 if hi + 1 < seq_len else hi  # lets a token see the next key


def _vr_window_off_by_one(seq_len, q_len, i, window):
    lo, hi = _ORIG_VR(seq_len, q_len, i, window)
    return (max(0, lo - 1) if window > 0 else lo), hi


def _deq_no_scale(codes, kv_dtype, scale=None):
    return _ORIG_DEQ(codes, kv_dtype, None if kv_dtype == "f16" else np.float32(1.0))


def _e4m3_bias8(codes):
    return _ORIG_E4M3(codes) * 0.5


def _gather_slot_reversed(cache, row, seq_len, g, kv_dtype, scale):
    P = cache.shape[1]
    return _ORIG_GATHER(cache[:, ::-1], row, seq_len, g, kv_dtype, scale) if P > 1 else None


_ORIG_VR = oa.visible_range
_ORIG_DEQ = oa.dequantize
_ORIG_E4M3 = oa.decode_e4m3fn
_ORIG_GATHER = oa._gather_keys

MUTANTS = {
    "causal_off_by_one": ("visible_range", _vr_causal_off_by_one),
    "window_off_by_one": ("visible_range", _vr_window_off_by_one),
    "scale_dropped": ("dequantize", _deq_no_scale),
    "e4m3_bias": ("decode_e4m3fn", _e4m3_bias8),
    "slot_order": ("_gather_keys", _gather_slot_reversed),
}


def test_unmutated_oracle_passes_pins():
    for h in _cases():
        assert not _caught(h)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    assert any(_caught(h) for h in _cases()), name
