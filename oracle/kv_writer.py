"""Plain definition of the paged KV-cache writer: new tokens' K and V rows go
into their page slots, quantized to fp8-e4m3 or int8 codes with one fp32
scale per KV head.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources. The decode kernel of vllm-rdna pull request #33 ("perf(rocm):
FA-RDNA2 decode, scores on every wave and 4 barriers per tile") reads the
cache in the layout the cache writer produces; its "Test Plan" runs a writer
layout test file and a writer-layout decode cell, and its "Purpose" section
gives fp8 and int8 decode wrappers over the same bodies. The pages show no
writer code. The readings used here are the plainest ones that agree with
what the decode side reads:

  * layout [num_pages, P, Hkv, D] per cache; token t's rows go to page
    slot_mapping[t] // P, slot slot_mapping[t] % P; a negative slot means the
    token is not written (padding), and so does a slot past the pool's end;
  * fp16 caches store the fp16 inputs unchanged;
  * a quantized code is q = x / scale[h] computed in fp32 (the fp16 input
    widened exactly, IEEE division), then rounded to the nearest code with
    ties to even, saturating at the largest finite magnitude (448 for
    e4m3fn, 127 for int8: symmetric, -128 is never produced). Inputs are
    finite.
"""

from __future__ import annotations

import numpy as np

from .attention import as_nhd

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6  # smallest normal exponent (bias 7, exponent field 1)
E4M3_MANT_BITS = 3


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Finite float values to OCP E4M3 ('fn') codes, round to nearest with
    ties to even, saturating at +-448. Written from the format: a normal
    value is (-1)^s 2^(e-7) (1 + m/8) for exponent field e in 1..15, a
    subnormal is (-1)^s 2^-6 (m/8). Within binade 2^k (k >= -6) the spacing
    is 2^(k-3); below 2^-6 it is 2^-9."""
    v = np.asarray(x, dtype=np.float64)
    assert np.isfinite(v).all(), "inputs must be finite"
    sign = np.signbit(v)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    nz = a > 0
    # exponent of the binade (floor(log2 a)), never below the normal minimum
    k = np.full(v.shape, E4M3_MIN_NORMAL_EXP, dtype=np.int64)
    k[nz] = np.maximum(np.frexp(a[nz])[1].astype(np.int64) - 1, E4M3_MIN_NORMAL_EXP)
    step = np.exp2((k - E4M3_MANT_BITS).astype(np.float64))
    n = np.rint(a / step)  # multiples of the spacing; ties to even (exact division)
    r = np.minimum(n * step, E4M3_MAX)  # rounded magnitude, saturated
    # encode the rounded magnitude r (it may have moved up a binade)
    sub = r < 2.0 ** E4M3_MIN_NORMAL_EXP
    out[sub] = np.rint(r[sub] / 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANT_BITS)).astype(np.int64)
    rn = r[~sub]
    e = np.frexp(rn)[1].astype(np.int64) - 1  # a = f 2^x with f in [0.5, 1)
    mant = np.rint((rn / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    out[~sub] = ((e + 7) << 3) | mant
    out = np.where(sign, out | 0x80, out)
    return out.astype(np.uint8)


def encode_int8(x: np.ndarray) -> np.ndarray:
    """Finite float values to symmetric int8 codes (as uint8 bytes): nearest
    integer with ties to even, saturating at +-127."""
    v = np.asarray(x, dtype=np.float64)
    assert np.isfinite(v).all(), "inputs must be finite"
    q = np.clip(np.rint(v), -127, 127).astype(np.int8)
    return q.view(np.uint8)


def quantize(x_f16: np.ndarray, scale: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Codes of fp16 values x [..., Hkv, D] with per-KV-head scales [Hkv]:
    q = x / scale in fp32, then the format's rounding."""
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32)[:, None]
    q = (x / s).astype(np.float32)  # IEEE fp32 division
    if kv_dtype == "fp8_e4m3":
        return encode_e4m3fn(q)
    if kv_dtype == "int8":
        return encode_int8(q)
    raise ValueError(kv_dtype)


def write_kv_cache(key, value, slot_mapping, k_cache, v_cache, kv_dtype="f16",
                   k_scale=None, v_scale=None, kv_layout="NHD"):
    """Returns copies of (k_cache, v_cache) [num_pages, P, Hkv, D] with token
    t's rows key[t], value[t] ([T, Hkv, D] fp16) stored at slot
    slot_mapping[t] (page = slot // P, position in page = slot % P); tokens
    with a negative slot, or one past the pool's num_pages * P slots, are
    skipped. fp16 caches take the values as they
    are; fp8/int8 caches take quantize(row, scale, kv_dtype) as uint8 codes.
    With kv_layout="HND" the caches are [num_pages, Hkv, P, D] and are
    written through the slot/head-swapped view."""
    kc_out = np.array(k_cache, copy=True)
    vc_out = np.array(v_cache, copy=True)
    kc, vc = as_nhd(kc_out, kv_layout), as_nhd(vc_out, kv_layout)  # views
    P = kc.shape[1]
    key = np.asarray(key, dtype=np.float16)
    value = np.asarray(value, dtype=np.float16)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= kc.shape[0] * P:
            continue
        page, pos = divmod(int(slot), P)
        if kv_dtype == "f16":
            kc[page, pos] = key[t].view(kc.dtype) if kc.dtype != np.float16 else key[t]
            vc[page, pos] = value[t].view(vc.dtype) if vc.dtype != np.float16 else value[t]
        else:
            kc[page, pos] = quantize(key[t][None], k_scale, kv_dtype)[0]
            vc[page, pos] = quantize(value[t][None], v_scale, kv_dtype)[0]
    return kc_out, vc_out
