"""Workload definitions and the seeded generator.

Every value is drawn from a seeded generator: numpy's PCG64 for lengths and
page permutations, torch's generator (on the device the case is built on)
for the N(0, 1) query and KV values. The same bytes go to the HIP path and to
the oracle.

Pool layout: K and V caches are [num_pages, P, Hkv, D] (page, slot, KV head,
dim), contiguous. Sequence b owns ceil(L_b / P) pages, taken in logical order
from a seeded permutation of the pool; its block-table row lists them and is
padded with the index of a poison page. Unused pages, the poison page and
the slots past L_b in a sequence's last page are filled with NaN (fp16 and
fp8-e4m3) or with the int8 code 127, so that any read of them shows.

Quantized KV: fp32 N(0, 1) values, one scale per KV head for K and one for V
(amax over the pool / 448 for fp8-e4m3, amax / 127 for int8), codes rounded
to nearest-even by torch's casts (int8 saturated to [-127, 127]).
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

F16_NAN_BITS = 0x7E00
FP8_NAN_CODE = 0x7F
INT8_POISON_CODE = 0x7F


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16
    kv_dtype: str = "f16"  # "f16" | "fp8_e4m3" | "int8"
    q_len: int = 1
    seq_lens: Optional[Tuple[int, ...]] = None  # explicit lengths
    seq_len: Optional[int] = None  # one length for every sequence
    ragged_max: Optional[int] = None  # lengths uniform in [0, ragged_max]
    forced_zero: int = 0  # that many seeded sequences forced to length 0
    window: int = 0  # <= 0: no sliding window
    num_splits: int = 0  # 0: the library's automatic choice
    pool_pages: int = 0  # total pool size (0: what the sequences need + 1)
    table_pad: int = 1  # extra block-table columns past the longest sequence
    scale: Optional[float] = None  # default 1/sqrt(D)
    seed: int = 0
    layout: str = "NHD"  # "NHD": [pages, P, Hkv, D]; "HND": [pages, Hkv, P, D]
    identity_table: bool = False  # pages in pool order instead of a permutation

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five synthetic workloads of the decode-attention benchmark.
WORKLOADS = {
    # Tiny paged decode: three sequences of 0, 37 and 200 keys in a pool of
    # 32 pages, 4 query heads over 2 KV heads, D=128; run with 1 and 3 splits.
    "tiny_d128": Workload("tiny_d128", batch=3, num_q_heads=4, num_kv_heads=2,
                          head_dim=128, seq_lens=(0, 37, 200), pool_pages=32,
                          num_splits=1, seed=1),
    # fp16 KV, D=128, 32/8 heads, 8 sequences of 4096 keys, automatic splits.
    "gqa4_d128_b8_l4096": Workload("gqa4_d128_b8_l4096", batch=8,
                                   num_q_heads=32, num_kv_heads=8,
                                   head_dim=128, seq_len=4096, seed=2),
    # fp16 KV, D=256, 24/4 heads (6 per KV head), 16384 keys; batch swept over
    # {1, 2, 3, 8, 32}, with no window and with a 4096-key window.
    "gqa6_d256_l16384": Workload("gqa6_d256_l16384", batch=8, num_q_heads=24,
                                 num_kv_heads=4, head_dim=256, seq_len=16384,
                                 seed=3),
    # Ragged multi-token verify: 32 sequences with lengths uniform in
    # [0, 32768], two of them forced to 0, three causal query tokens each,
    # 28/4 heads, D=128, 8 splits.
    "verify_q3_d128_b32": Workload("verify_q3_d128_b32", batch=32,
                                   num_q_heads=28, num_kv_heads=4,
                                   head_dim=128, q_len=3, ragged_max=32768,
                                   forced_zero=2, num_splits=8, seed=4),
    # Long query runs on the same paged cache (the prefill kernel): a fresh
    # prefill of 4 x 2048 tokens, and chunked prefill of 512 new tokens on
    # 8 sequences of 8192 keys, fp16 KV, D=128, 32/8 heads; and the fresh
    # prefill at D=256 with 24/4 heads.
    "prefill_d128_b4_q2048": Workload("prefill_d128_b4_q2048", batch=4, num_q_heads=32,
                                      num_kv_heads=8, head_dim=128, q_len=2048, seq_len=2048,
                                      num_splits=1, seed=7),
    "chunked_d128_b8_l8192_q512": Workload("chunked_d128_b8_l8192_q512", batch=8,
                                           num_q_heads=32, num_kv_heads=8, head_dim=128,
                                           q_len=512, seq_len=8192, num_splits=1, seed=8),
    "prefill_d256_b4_q2048": Workload("prefill_d256_b4_q2048", batch=4, num_q_heads=24,
                                      num_kv_heads=4, head_dim=256, q_len=2048, seq_len=2048,
                                      num_splits=1, seed=9),
    # Quantized long context: D=256, 16/4 heads, 64 sequences of 32768 keys,
    # K/V as fp8-e4m3 or int8 codes with per-KV-head fp32 scales, 8 splits.
    "quant_fp8_d256_b64_l32768": Workload("quant_fp8_d256_b64_l32768",
                                          batch=64, num_q_heads=16,
                                          num_kv_heads=4, head_dim=256,
                                          seq_len=32768, kv_dtype="fp8_e4m3",
                                          num_splits=8, seed=5),
    "quant_int8_d256_b64_l32768": Workload("quant_int8_d256_b64_l32768",
                                           batch=64, num_q_heads=16,
                                           num_kv_heads=4, head_dim=256,
                                           seq_len=32768, kv_dtype="int8",
                                           num_splits=8, seed=6),
}


@dataclass
class Case:
    """One generated input set. Tensors live on ``device``; q is float16
    [T, Hq, D]; caches are float16 or uint8 codes [num_pages, P, Hkv, D]
    (or [num_pages, Hkv, P, D] for the HND layout)."""
    workload: Workload
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq]
    seq_lens: torch.Tensor  # int32 [B]
    q_lens: torch.Tensor  # int32 [B]
    k_scale: Optional[torch.Tensor]  # float32 [Hkv] or None
    v_scale: Optional[torch.Tensor]
    scale: float
    window: int
    poison_page: int
    seq_lens_host: np.ndarray = field(repr=False, default=None)
    q_lens_host: np.ndarray = field(repr=False, default=None)

    @property
    def kv_dtype(self) -> str:
        return self.workload.kv_dtype

    @property
    def kv_layout(self) -> str:
        return self.workload.layout

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens_host.max()) if len(self.q_lens_host) else 1

    def to(self, device) -> "Case":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return dataclasses.replace(
            self, q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
            block_table=mv(self.block_table), seq_lens=mv(self.seq_lens),
            q_lens=mv(self.q_lens), k_scale=mv(self.k_scale), v_scale=mv(self.v_scale))

    def host(self) -> dict:
        """numpy views of every input, in the oracle's argument layout."""
        np_ = lambda t: None if t is None else t.detach().cpu().numpy()  # noqa: E731
        return dict(q=np_(self.q), k_cache=np_(self.k_cache), v_cache=np_(self.v_cache),
                    block_table=np_(self.block_table), seq_lens=np_(self.seq_lens),
                    q_lens=np_(self.q_lens), scale=self.scale, window=self.window,
                    kv_dtype=self.kv_dtype, k_scale=np_(self.k_scale),
                    v_scale=np_(self.v_scale), kv_layout=self.kv_layout)


def _seq_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.seq_lens is not None:
        lens = np.array(w.seq_lens, np.int64)
    elif w.seq_len is not None:
        lens = np.full(w.batch, w.seq_len, np.int64)
    else:
        lens = rng.integers(0, w.ragged_max, size=w.batch, endpoint=True)
    if w.forced_zero:
        lens[rng.choice(w.batch, size=w.forced_zero, replace=False)] = 0
    assert len(lens) == w.batch
    return lens


def _normal(shape, gen, device, dtype=torch.float32):
    return torch.randn(shape, generator=gen, device=device, dtype=dtype)


def _draw_cache(shape, w: Workload, gen, device):
    """N(0,1) values for one cache, as fp16 or as quantized codes + scales."""
    num_pages, P, Hkv, D = shape
    if w.kv_dtype == "f16":
        out = torch.empty(shape, dtype=torch.float16, device=device)
        chunk = max(1, (1 << 28) // (P * Hkv * D))  # bound the fp32 temporary
        for p0 in range(0, num_pages, chunk):
            p1 = min(num_pages, p0 + chunk)
            out[p0:p1] = _normal((p1 - p0, P, Hkv, D), gen, device).to(torch.float16)
        return out, None
    x = _normal(shape, gen, device)
    amax = x.abs().amax(dim=(0, 1, 3))  # per KV head
    if w.kv_dtype == "fp8_e4m3":
        sc = (amax / 448.0).to(torch.float32)
        codes = (x / sc[None, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    elif w.kv_dtype == "int8":
        sc = (amax / 127.0).to(torch.float32)
        codes = torch.round(x / sc[None, None, :, None]).clamp_(-127, 127)
        codes = codes.to(torch.int8).view(torch.uint8)
    else:
        raise ValueError(w.kv_dtype)
    del x
    return codes.contiguous(), sc


def _poison_value(kv_dtype):
    if kv_dtype == "f16":
        return torch.tensor(F16_NAN_BITS, dtype=torch.int16).view(torch.float16).item()
    return FP8_NAN_CODE if kv_dtype == "fp8_e4m3" else INT8_POISON_CODE


def make_case(w: Workload, device="cpu") -> Case:
    rng = np.random.default_rng(w.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    B, Hq, Hkv, D, P = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    lens = _seq_lens(w, rng)
    q_lens = np.full(B, w.q_len, np.int64)
    pages_per_seq = -(-lens // P)
    needed = int(pages_per_seq.sum())
    num_pages = max(w.pool_pages, needed + 1)
    max_pages = int(max(1, pages_per_seq.max(initial=0))) + w.table_pad

    perm = rng.permutation(num_pages)
    if w.identity_table:
        perm = np.arange(num_pages)
    poison_page = int(perm[-1])
    table = np.full((B, max_pages), poison_page, np.int64)
    cursor = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        table[b, :n] = perm[cursor:cursor + n]
        cursor += n
    used = perm[:needed]

    T = int(q_lens.sum())
    q = _normal((T, Hq, D), gen, device).to(torch.float16)
    shape = (num_pages, P, Hkv, D)
    k_cache, k_scale = _draw_cache(shape, w, gen, device)
    v_cache, v_scale = _draw_cache(shape, w, gen, device)

    # Poison: every page not owned by a sequence, and the tail slots of each
    # sequence's last page.
    poison = _poison_value(w.kv_dtype)
    unused = np.setdiff1d(np.arange(num_pages), used)
    if len(unused):
        idx = torch.from_numpy(unused).to(device)
        k_cache[idx] = poison
        v_cache[idx] = poison
    for b in range(B):
        L = int(lens[b])
        if L % P:
            last = int(table[b, L // P])
            k_cache[last, L % P:] = poison
            v_cache[last, L % P:] = poison

    if w.layout == "HND":
        k_cache = k_cache.permute(0, 2, 1, 3).contiguous()
        v_cache = v_cache.permute(0, 2, 1, 3).contiguous()
    elif w.layout != "NHD":
        raise ValueError(w.layout)
    scale = w.scale if w.scale is not None else 1.0 / math.sqrt(D)
    return Case(
        workload=w, q=q, k_cache=k_cache, v_cache=v_cache,
        block_table=torch.from_numpy(table.astype(np.int32)).to(device),
        seq_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        q_lens=torch.from_numpy(q_lens.astype(np.int32)).to(device),
        k_scale=k_scale, v_scale=v_scale, scale=float(np.float32(scale)),
        window=int(w.window), poison_page=poison_page,
        seq_lens_host=lens.astype(np.int32), q_lens_host=q_lens.astype(np.int32))


def unit_subcase(case: Case, b: int, g: int) -> dict:
    """Inputs of one (sequence b, KV head g) unit as a self-contained host
    problem for the oracle: that sequence's pages of KV head g only, an
    identity block table, and its G query heads, always in the NHD layout.
    Lets the oracle check sampled outputs of a full-size case without copying
    the whole pool."""
    hnd = case.kv_layout == "HND"
    P = case.k_cache.shape[2 if hnd else 1]
    Hq, Hkv = case.q.shape[1], case.k_cache.shape[1 if hnd else 2]
    G = Hq // Hkv
    L = int(case.seq_lens_host[b])
    Q = int(case.q_lens_host[b])
    off = int(case.q_lens_host[:b].sum())
    n = -(-L // P)
    pages = case.block_table[b, :n].long()
    def head(cache, idx):
        x = cache.index_select(0, idx)
        x = x[:, g:g + 1].transpose(1, 2) if hnd else x[:, :, g:g + 1]
        return x.contiguous().cpu().numpy()

    first = torch.zeros(1, dtype=torch.long, device=case.k_cache.device)
    k = head(case.k_cache, pages if n else first)  # one (unread) page if empty
    v = head(case.v_cache, pages if n else first)
    q = case.q[off:off + Q, g * G:(g + 1) * G].cpu().numpy()
    sel = lambda t: None if t is None else t[g:g + 1].cpu().numpy()  # noqa: E731
    return dict(q=q, k_cache=k, v_cache=v,
                block_table=np.arange(max(n, 1), dtype=np.int32)[None, :],
                seq_lens=np.array([L], np.int32), q_lens=np.array([Q], np.int32),
                scale=case.scale, window=case.window, kv_dtype=case.kv_dtype,
                k_scale=sel(case.k_scale), v_scale=sel(case.v_scale))


def visible_keys_of_sequence(L: int, Q: int, window: int) -> int:
    """Number of cached keys some new token of the sequence can see (the
    union of their ranges): what a decode step must read for it."""
    if window > 0:
        lo = max(0, L - Q + 1 - window)
    else:
        lo = 0
    return max(0, L - lo)


def workload_lengths(w: Workload) -> np.ndarray:
    """The seeded sequence lengths of a workload, as make_case draws them
    (the first draw of its generator), without building the pool."""
    return _seq_lens(w, np.random.default_rng(w.seed))


def workload_algorithmic_bytes(w: Workload) -> int:
    """algorithmic_bytes of the case make_case(w) builds, from the lengths
    alone (no pool)."""
    e = 2 if w.kv_dtype == "f16" else 1
    keys = sum(visible_keys_of_sequence(int(L), w.q_len, w.window) for L in workload_lengths(w))
    return keys * w.num_kv_heads * w.head_dim * e * 2 + w.batch * w.q_len * w.num_q_heads * w.head_dim * 4


def workload_visible_pairs(w: Workload) -> int:
    """visible_pairs of the case make_case(w) builds, from the lengths alone."""
    total = 0
    for L in workload_lengths(w).tolist():
        for i in range(w.q_len):
            p = int(L) - w.q_len + i
            if p < 0:
                continue
            lo = max(0, p - w.window + 1) if w.window > 0 else 0
            total += p - lo + 1
    return total * w.num_q_heads


def algorithmic_bytes(case: Case) -> int:
    """Bytes one call must move: every visible key of K and V once, plus q
    and out (fp16). Scales, block table and split partials are excluded."""
    w = case.workload
    e = 2 if w.kv_dtype == "f16" else 1
    D, Hkv, Hq = w.head_dim, w.num_kv_heads, w.num_q_heads
    keys = sum(visible_keys_of_sequence(int(L), int(Q), case.window)
               for L, Q in zip(case.seq_lens_host, case.q_lens_host))
    return keys * Hkv * D * e * 2 + case.num_tokens * Hq * D * 2 * 2


# ---------------------------------------------------------------------------
# Cache-writer inputs
# ---------------------------------------------------------------------------


@dataclass
class WriteCase:
    """Inputs of one cache write: new rows, their slots, poisoned caches."""
    key: torch.Tensor           # fp16 [T, Hkv, D]
    value: torch.Tensor         # fp16 [T, Hkv, D]
    slot_mapping: torch.Tensor  # int32 [T]
    k_cache: torch.Tensor       # [num_pages, P, Hkv, D] fp16 or uint8 codes
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]  # fp32 [Hkv] or None
    v_scale: Optional[torch.Tensor]
    kv_dtype: str
    kv_layout: str = "NHD"  # "HND": caches [num_pages, Hkv, P, D]

    def host(self) -> dict:
        np_ = lambda t: None if t is None else t.detach().cpu().numpy()  # noqa: E731
        return dict(key=np_(self.key), value=np_(self.value), slot_mapping=np_(self.slot_mapping),
                    k_cache=np_(self.k_cache), v_cache=np_(self.v_cache), kv_dtype=self.kv_dtype,
                    k_scale=np_(self.k_scale), v_scale=np_(self.v_scale),
                    kv_layout=self.kv_layout)


def make_write_case(num_tokens, num_kv_heads, head_dim, page_size, num_pages, kv_dtype,
                    seed, skip_frac=0.1, values=None, scale=None, device="cpu",
                    layout="NHD") -> WriteCase:
    """Seeded writer inputs. Rows are N(0,1) fp16 (or `values`, an fp16 array
    of T*Hkv*D elements laid out in order); slots are distinct and random in
    the pool, with about `skip_frac` of them negative and a few past the
    pool's end. Scales for quantized caches are `scale` (a number) or the
    per-KV-head amax of the rows over the format's largest code. Caches start
    poisoned (NaN / code 0x7F / 127)."""
    rng = np.random.default_rng(seed)
    T, Hkv, D, P = num_tokens, num_kv_heads, head_dim, page_size
    if values is None:
        key = rng.standard_normal((T, Hkv, D)).astype(np.float16)
        value = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    else:
        key = np.asarray(values, np.float16).reshape(T, Hkv, D)
        value = key[::-1].copy()
    n_slots = num_pages * P
    assert T <= n_slots, "distinct slots need num_pages * page_size >= num_tokens"
    slots = rng.choice(n_slots, size=T, replace=False).astype(np.int64)
    if T:
        slots[rng.random(T) < skip_frac] = -1
        slots[rng.random(T) < skip_frac / 4] = n_slots + int(rng.integers(0, 5))
    k_scale = v_scale = None
    if kv_dtype != "f16":
        top = 448.0 if kv_dtype == "fp8_e4m3" else 127.0
        if scale is None:
            amax = lambda x: np.abs(x.astype(np.float32)).max(axis=(0, 2), initial=0.0)
            k_scale = (amax(key) / top).astype(np.float32)
            v_scale = (amax(value) / top).astype(np.float32)
            k_scale[k_scale == 0] = 1.0
            v_scale[v_scale == 0] = 1.0
        else:
            k_scale = np.full(Hkv, scale, np.float32)
            v_scale = np.full(Hkv, scale, np.float32)
    shape = (num_pages, Hkv, P, D) if layout == "HND" else (num_pages, P, Hkv, D)
    if kv_dtype == "f16":
        kc = np.full(shape, np.uint16(F16_NAN_BITS)).view(np.float16)
    else:
        kc = np.full(shape, _poison_value(kv_dtype), np.uint8)
    vc = kc.copy()
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return WriteCase(key=t(key), value=t(value), slot_mapping=t(slots.astype(np.int32)),
                     k_cache=t(kc), v_cache=t(vc), k_scale=t(k_scale), v_scale=t(v_scale),
                     kv_dtype=kv_dtype, kv_layout=layout)


def visible_pairs(case: Case) -> int:
    """(query row, key) pairs one call scores: for every new token, the keys
    it can see, times the query heads. The flop count of a call is
    4 * head_dim * visible_pairs (2 D for q.k, 2 D for p.v)."""
    W = case.window
    total = 0
    for L, Q in zip(case.seq_lens_host.tolist(), case.q_lens_host.tolist()):
        for i in range(Q):
            p = L - Q + i
            if p < 0:
                continue
            lo = max(0, p - W + 1) if W > 0 else 0
            total += p - lo + 1
    return total * case.workload.num_q_heads
