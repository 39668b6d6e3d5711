"""Plain fp64 definition of paged decode attention, with GQA, multi-token
causal queries, an optional sliding window and quantized KV.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed. For sequence b with L_b cached keys (the new tokens
included) and Q_b new query tokens, token i sits at absolute position
p = L_b - Q_b + i and sees keys j with lo <= j <= p, where lo = 0 without a
window and lo = max(0, p - W + 1) with a window of W keys. Query head h reads
KV head h // G, G = Hq / Hkv (consecutive query heads share a KV head). Key j
of sequence b lives in slot j % P of physical page block_table[b][j // P].
For each (token, query head) row the result is

    out = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),   s_j = scale * q . k_j,

over the visible keys (m = max_j s_j), i.e. one-shot softmax attention over
the gathered keys, and exactly 0 for a row that sees no key.

Sources. The operation is the per-head paged split-K decode attention kernel
of vllm-rdna pull request #33 ("perf(rocm): FA-RDNA2 decode, scores on every
wave and 4 barriers per tile"), section "Purpose": softmax(q.K^T).V per query
head over a paged KV cache, with fp16, fp8 and int8 KV. Its "Test Plan"
section names the behaviours checked here: empty rows are zero, a custom
scale, a sliding window, multi-token queries and split decode. Its "Test
Result" section measures the split-K schedule against a one-shot fp64
reference, which is what this module is. The pages give no formula for the
window or the multi-token mask; the readings used (a window of W keys ending
at the token's own position; token i of Q_b seeing L_b - Q_b + i + 1 keys)
are the plainest ones, and every one of them is pinned by tests against
brute force, torch's attention and invariants.

Layouts (all contiguous):
    q            float16 [T, Hq, D], T = sum(q_lens), sequences packed in order
    k_cache      [num_pages, P, Hkv, D] ("NHD": page, slot, KV head, dim), or
                 [num_pages, Hkv, P, D] ("HND": page, KV head, slot, dim) with
                 kv_layout="HND": float16, or uint8 codes for fp8/int8. The
                 pages name the cache writer's layout and a "dense" layout
                 without defining either (pull request #33, "Test Plan"); NHD
                 is the plainest reading of the writer's, HND the other common
                 paged layout. Both hold the same key: HND is NHD with the
                 slot and head axes exchanged, which is how it is read here.
    v_cache      same as k_cache
    block_table  int32 [B, max_pages_per_seq]
    seq_lens     int32 [B]
    q_lens       int32 [B] or None (every sequence has one new token)
    k_scale/v_scale  float32 [Hkv] (quantized KV only)
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Element formats (exact decoders)
# ---------------------------------------------------------------------------


def decode_f16(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 values (np.float16, or their uint16 bit patterns) to
    float64. Exact: every binary16 value is a binary64 value."""
    x = np.asarray(x)
    if x.dtype == np.uint16 or x.dtype == np.int16:
        x = x.view(np.float16)
    assert x.dtype == np.float16, x.dtype
    return x.astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 (the 'fn' flavour: exponent bias 7, no infinities,
    S.1111.111 is NaN, largest finite value 448) to float64, written from the
    format definition: normal codes are (-1)^s 2^(e-7) (1 + m/8), codes with
    e = 0 are the subnormals (-1)^s 2^-6 (m/8)."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def decode_int8(codes: np.ndarray) -> np.ndarray:
    """Symmetric signed int8 codes (stored as uint8 bytes) to float64."""
    return np.asarray(codes).view(np.int8).astype(np.float64)


def dequantize(codes: np.ndarray, kv_dtype: str, scale=None) -> np.ndarray:
    """KV element -> float64 value: fp16 as is; fp8-e4m3 and int8 codes times
    the per-KV-head float32 scale (widened exactly to float64). The fp8 and
    int8 decode wrappers of the pages' kernel share the fp16 bodies
    (pull request #33, "Purpose"), so the value is the only thing that
    changes."""
    if kv_dtype == "f16":
        return decode_f16(codes)
    if kv_dtype == "fp8_e4m3":
        return np.float64(np.float32(scale)) * decode_e4m3fn(codes)
    if kv_dtype == "int8":
        return np.float64(np.float32(scale)) * decode_int8(codes)
    raise ValueError(kv_dtype)


# ---------------------------------------------------------------------------
# Masks
# ---------------------------------------------------------------------------


def visible_range(seq_len: int, q_len: int, i: int, window: int):
    """Inclusive key range [lo, hi] seen by new token i of a sequence that
    holds seq_len keys (its q_len new tokens included). Empty when hi < lo,
    which covers tokens whose position is negative (q_len > seq_len)."""
    pos = seq_len - q_len + i
    hi = pos
    lo = max(0, pos - window + 1) if window > 0 else 0
    return lo, hi


def _token_offsets(q_lens: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(q_lens)[:-1]]).astype(np.int64)


def _gather_keys(cache, block_table_row, seq_len, g, kv_dtype, scale):
    """Logical keys 0..seq_len-1 of KV head g, gathered page by page through
    the block table, as float64 [seq_len, D]."""
    P = cache.shape[1]
    n_pages = -(-seq_len // P)
    pages = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    rows = cache[pages, :, g, :]  # [n_pages, P, D]: key j is rows[j // P, j % P]
    rows = rows.reshape(-1, cache.shape[3])[:seq_len]
    return dequantize(rows, kv_dtype, scale)


def as_nhd(cache, kv_layout="NHD"):
    """The cache seen as [num_pages, P, Hkv, D] (a view; HND swaps the slot
    and head axes)."""
    if kv_layout == "NHD":
        return cache
    if kv_layout == "HND":
        return np.swapaxes(cache, 1, 2)
    raise ValueError(kv_layout)


def _check(q, k_cache, v_cache, block_table, seq_lens, q_lens):
    T, Hq, D = q.shape
    num_pages, P, Hkv, Dk = k_cache.shape
    assert v_cache.shape == k_cache.shape and Dk == D and Hq % Hkv == 0
    B = len(seq_lens)
    q_lens = np.ones(B, np.int64) if q_lens is None else np.asarray(q_lens, np.int64)
    assert int(q_lens.sum()) == T, (int(q_lens.sum()), T)
    assert block_table.shape[0] == B
    return T, Hq, D, P, Hkv, Hq // Hkv, B, q_lens


# ---------------------------------------------------------------------------
# One-shot attention (the parity oracle)
# ---------------------------------------------------------------------------


def paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, q_lens,
                           scale, window=0, kv_dtype="f16", k_scale=None,
                           v_scale=None, units=None, kv_layout="NHD"):
    """One-shot masked softmax attention over the gathered keys, in float64.

    Returns float64 [T, Hq, D]. ``units`` optionally restricts the work to a
    set of (b, g) pairs (sequence, KV head); rows of other units are NaN.
    """
    k_cache, v_cache = as_nhd(k_cache, kv_layout), as_nhd(v_cache, kv_layout)
    T, Hq, D, P, Hkv, G, B, q_lens = _check(q, k_cache, v_cache, block_table,
                                             seq_lens, q_lens)
    q64 = decode_f16(q)
    scale64 = np.float64(np.float32(scale))
    offs = _token_offsets(q_lens)
    out = np.zeros((T, Hq, D), np.float64)
    for b in range(B):
        L, Q, off = int(seq_lens[b]), int(q_lens[b]), int(offs[b])
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            if units is not None and (b, g) not in units:
                out[off:off + Q, heads] = np.nan
                continue
            ks = None if k_scale is None else k_scale[g]
            vs = None if v_scale is None else v_scale[g]
            K = _gather_keys(k_cache, block_table[b], L, g, kv_dtype, ks)
            V = _gather_keys(v_cache, block_table[b], L, g, kv_dtype, vs)
            for i in range(Q):
                t = off + i
                lo, hi = visible_range(L, Q, i, window)
                if hi < lo:
                    out[t, heads] = 0.0  # a row that sees no key is zero
                    continue
                s = scale64 * (K[lo:hi + 1] @ q64[t, heads].T)  # [n, G]
                w = np.exp(s - s.max(axis=0))
                out[t, heads] = (w.T @ V[lo:hi + 1]) / w.sum(axis=0)[:, None]
    return out


# ---------------------------------------------------------------------------
# Split-K model and split combine (for invariants and for the combine step)
# ---------------------------------------------------------------------------


def paged_decode_attention_split(q, k_cache, v_cache, block_table, seq_lens,
                                 q_lens, scale, window=0, num_splits=1,
                                 kv_dtype="f16", k_scale=None, v_scale=None,
                                 kv_layout="NHD"):
    """Split-K form of the same attention: the keys any token of a sequence
    can see, [lo of token 0, L), are cut into ``num_splits`` contiguous
    chunks (chunks may be empty); each chunk yields, per row, its running
    max m_c, its sum l_c = sum exp(s - m_c) and o_c = sum exp(s - m_c) v over
    the row's visible keys inside the chunk, and the chunks are merged by
    ``split_combine`` in base e. The pages' schedule splits the key axis
    across workgroups and merges the splits (pull request #33, "Purpose" and
    "Test Result"); this model exists to show that the result does not
    depend on the split count."""
    k_cache, v_cache = as_nhd(k_cache, kv_layout), as_nhd(v_cache, kv_layout)
    T, Hq, D, P, Hkv, G, B, q_lens = _check(q, k_cache, v_cache, block_table,
                                             seq_lens, q_lens)
    S = int(num_splits)
    q64 = decode_f16(q)
    scale64 = np.float64(np.float32(scale))
    offs = _token_offsets(q_lens)
    part_o = np.zeros((T, Hq, S, D))
    part_m = np.full((T, Hq, S), -np.inf)
    part_l = np.zeros((T, Hq, S))
    for b in range(B):
        L, Q, off = int(seq_lens[b]), int(q_lens[b]), int(offs[b])
        lo0 = visible_range(L, Q, 0, window)[0]
        n = max(0, L - lo0)
        bounds = [lo0 + (c * n) // S for c in range(S + 1)]
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            ks = None if k_scale is None else k_scale[g]
            vs = None if v_scale is None else v_scale[g]
            K = _gather_keys(k_cache, block_table[b], L, g, kv_dtype, ks)
            V = _gather_keys(v_cache, block_table[b], L, g, kv_dtype, vs)
            for i in range(Q):
                t = off + i
                lo, hi = visible_range(L, Q, i, window)
                for c in range(S):
                    a, z = max(lo, bounds[c]), min(hi + 1, bounds[c + 1])
                    if a >= z:
                        continue  # empty chunk: m = -inf, l = 0, o = 0
                    s = scale64 * (K[a:z] @ q64[t, heads].T)  # [n_c, G]
                    m = s.max(axis=0)
                    w = np.exp(s - m)
                    part_m[t, heads, c] = m
                    part_l[t, heads, c] = w.sum(axis=0)
                    part_o[t, heads, c] = w.T @ V[a:z]
    return split_combine(part_o, part_m, part_l, base=np.e)


def split_combine(part_o, part_m, part_l, base=2.0):
    """Merge per-split partials: with M = max over non-empty splits of m_s,
    out = sum_s base^(m_s - M) o_s / sum_s base^(m_s - M) l_s, where o_s is
    the split's unnormalized output and l_s its softmax denominator, both
    relative to its own max m_s (in units of log base). Splits with l_s = 0
    are empty and drop out; a row whose splits are all empty is 0.

    part_o [..., S, D], part_m and part_l [..., S]; returns float64 [..., D].
    """
    part_o = np.asarray(part_o, np.float64)
    part_m = np.asarray(part_m, np.float64)
    part_l = np.asarray(part_l, np.float64)
    live = part_l > 0
    M = np.where(live, part_m, -np.inf).max(axis=-1, keepdims=True)
    any_live = live.any(axis=-1, keepdims=True)
    M = np.where(any_live, M, 0.0)
    w = np.where(live, np.power(base, np.where(live, part_m, 0.0) - M), 0.0)
    num = (w[..., None] * np.where(live[..., None], part_o, 0.0)).sum(axis=-2)
    den = (w * part_l).sum(axis=-1, keepdims=True)
    return np.where(any_live, num / np.where(den > 0, den, 1.0), 0.0)
