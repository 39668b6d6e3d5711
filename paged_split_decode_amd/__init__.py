"""Paged split-K decode attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libpda.so`` (declared in
``include/pda.h``). The functions here only marshal torch tensors into
pointers and sizes; every step of the computation runs in the library's HIP
kernels, on the current torch stream. torch supplies device memory and
streams. There is no fallback: if the library is not built, every call raises.

Build the library with ``python -m paged_split_decode_amd.build``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "paged_decode_attention", "paged_decode_partials", "split_combine",
    "resolve_splits", "workspace_bytes", "attention_stages", "partials_bytes", "decode_dims",
    "load_library", "library_path", "KV_DTYPES", "PDA_MAX_ROWS", "PDA_MAX_SPLITS",
    "PdaError", "partials_views", "KERNELS", "paged_decode_attention_noalloc",
    "noalloc_scratch_bytes", "hbm_read_probe",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpda.so")

KV_DTYPES = {"f16": 0, "fp8_e4m3": 1, "int8": 2}
KERNELS = {"auto": 0, "vector": 1, "matrix": 2, "prefill": 3}
KV_LAYOUTS = {"NHD": 0, "HND": 1}
PDA_MAX_ROWS = 32
PDA_MAX_SPLITS = 256
STATUS = {0: "PDA_OK", -1: "PDA_ERR_NULL", -2: "PDA_ERR_SHAPE", -3: "PDA_ERR_ALIGN",
          -4: "PDA_ERR_UNSUPPORTED", -5: "PDA_ERR_WORKSPACE", -6: "PDA_ERR_DEVICE"}


class PdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class DecodeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_tokens", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
        "num_pages", "max_pages_per_seq", "max_q_len", "kv_dtype", "kernel", "kv_layout")]


class CacheDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "num_kv_heads", "head_dim", "page_size", "num_pages", "kv_dtype",
        "kv_layout")]


_lib: Optional[ctypes.CDLL] = None

_VP, _I32P = ctypes.c_void_p, ctypes.c_void_p
_DIMS = ctypes.POINTER(DecodeDims)

_SIGNATURES = {
    "pda_paged_decode_attention": (ctypes.c_int, [
        _VP, _VP, _VP, _I32P, _I32P, _I32P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
        _VP, _VP, _VP, _DIMS, _VP, ctypes.c_size_t, _VP]),
    "pda_attention_decode_stage": (ctypes.c_int, [
        _VP, _VP, _VP, _I32P, _I32P, _I32P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
        _VP, _VP, _VP, _DIMS, _VP, ctypes.c_size_t, _VP]),
    "pda_attention_combine_stage": (ctypes.c_int, [
        _VP, _DIMS, ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]),
    "pda_paged_decode_partials": (ctypes.c_int, [
        _VP, _VP, _VP, _I32P, _I32P, _I32P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
        _VP, _VP, _DIMS, _VP, ctypes.c_size_t, _VP]),
    "pda_split_combine": (ctypes.c_int, [
        _VP, _VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP]),
    "pda_decode_resolve_splits": (ctypes.c_int32, [_DIMS, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32]),
    "pda_decode_workspace_bytes": (ctypes.c_int64, [_DIMS, ctypes.c_int32, ctypes.c_int32]),
    "pda_decode_partials_bytes": (ctypes.c_int64, [_DIMS, ctypes.c_int32, ctypes.c_int32]),
    "pda_write_kv_cache": (ctypes.c_int, [
        _VP, _VP, _I32P, _VP, _VP, _VP, _VP, ctypes.POINTER(CacheDims), _VP]),
    "pda_paged_decode_attention_noalloc": (ctypes.c_int, [
        _VP, _VP, _VP, _I32P, _I32P, _I32P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
        _VP, _VP, _VP, _DIMS, _VP]),
    "pda_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "pda_hbm_read_probe": (ctypes.c_int, [_VP, ctypes.c_size_t, _VP, ctypes.c_int32, _VP]),
    "pda_last_error": (ctypes.c_char_p, []),
    "pda_version": (ctypes.c_char_p, []),
}


def library_path() -> str:
    """The library this process loads: libpda.so beside this file, or the
    build the environment variable PDA_LIBRARY names (read at the first
    load), such as the diagnostic timeline build."""
    return os.environ.get("PDA_LIBRARY") or _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libpda.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m paged_split_decode_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise PdaError(status, load_library().pda_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A call's own workspace, allocated on the stream its kernels run on.
    torch's caching allocator ties a freed block to the stream it was
    allocated on, so after this function's caller drops the tensor the block
    goes only to later work on that same stream, which runs after these
    kernels. (Allocated on another stream, it could be handed to new work
    there while the kernels still use it.)"""
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)),
                                           device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _kv_code(k_cache: torch.Tensor, kv_dtype: Optional[str]) -> int:
    if kv_dtype is None:
        kv_dtype = {torch.float16: "f16", torch.float8_e4m3fn: "fp8_e4m3",
                    torch.int8: "int8"}.get(k_cache.dtype)
        if kv_dtype is None:
            raise ValueError(f"kv_dtype needed for a {k_cache.dtype} cache")
    return KV_DTYPES[kv_dtype]


def decode_dims(q, k_cache, block_table, seq_lens, q_lens=None, max_q_len=None,
                kv_dtype=None, kernel="auto", kv_layout="NHD") -> DecodeDims:
    """Sizes of one call, read from tensor shapes. ``max_q_len`` defaults to
    1 without q_lens; with q_lens it must be given (reading q_lens would need
    a device synchronization). ``kv_layout``: "NHD" caches are
    [num_pages, P, Hkv, D], "HND" caches [num_pages, Hkv, P, D]."""
    T, Hq, D = q.shape
    if kv_layout == "HND":
        num_pages, Hkv, P, Dk = k_cache.shape
    else:
        num_pages, P, Hkv, Dk = k_cache.shape
    if q_lens is not None and max_q_len is None:
        raise ValueError("max_q_len is required when q_lens is given")
    return DecodeDims(batch=seq_lens.shape[0], num_tokens=T, num_q_heads=Hq,
                      num_kv_heads=Hkv, head_dim=D, page_size=P, num_pages=num_pages,
                      max_pages_per_seq=block_table.shape[1],
                      max_q_len=1 if q_lens is None else int(max_q_len),
                      kv_dtype=_kv_code(k_cache, kv_dtype), kernel=KERNELS[kernel],
                      kv_layout=KV_LAYOUTS[kv_layout])


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")


def resolve_splits(dims: DecodeDims, window: int = 0, num_splits: int = 0,
                   num_cus: int = 0) -> int:
    s = load_library().pda_decode_resolve_splits(ctypes.byref(dims), window, num_splits, num_cus)
    if s < 0:
        _check(s)
    return s


def workspace_bytes(dims: DecodeDims, window: int = 0, num_splits: int = 0) -> int:
    n = load_library().pda_decode_workspace_bytes(ctypes.byref(dims), window, num_splits)
    if n < 0:
        _check(int(n))
    return int(n)


def partials_bytes(dims: DecodeDims, window: int = 0, num_splits: int = 0) -> int:
    n = load_library().pda_decode_partials_bytes(ctypes.byref(dims), window, num_splits)
    if n < 0:
        _check(int(n))
    return int(n)


def paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale,
                           window, num_splits, out, k_scale=None, v_scale=None,
                           kv_dtype=None, max_q_len=None, workspace=None, stream=None,
                           kernel="auto", kv_layout="NHD"):
    """out[t, h] = softmax(scale q.K^T) V over each token's visible keys (see
    include/pda.h). Writes ``out`` (fp16 [T, Hq, D]) and returns None.
    ``kernel``: "auto", "vector" (v_dot2) or "matrix" (MFMA)."""
    lib = load_library()
    _contig(q, k_cache, v_cache, block_table, seq_lens, q_lens, out, k_scale, v_scale)
    dims = decode_dims(q, k_cache, block_table, seq_lens, q_lens, max_q_len, kv_dtype, kernel,
                       kv_layout)
    need = workspace_bytes(dims, window, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pda_paged_decode_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(q_lens), float(scale), int(window), int(num_splits), _ptr(out),
        _ptr(k_scale), _ptr(v_scale), ctypes.byref(dims), _ptr(workspace), ws_bytes,
        _stream(stream)))


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale,
                                   window, num_splits, out, k_scale=None, v_scale=None,
                                   kv_dtype=None, max_q_len=None, stream=None, kernel="auto",
                                   kv_layout="NHD"):
    """paged_decode_attention without a workspace: the library's per-device
    scratch array holds the split partials, so the call allocates nothing
    (see include/pda.h; calls that overlap on one device race)."""
    lib = load_library()
    _contig(q, k_cache, v_cache, block_table, seq_lens, q_lens, out, k_scale, v_scale)
    dims = decode_dims(q, k_cache, block_table, seq_lens, q_lens, max_q_len, kv_dtype, kernel,
                       kv_layout)
    _check(lib.pda_paged_decode_attention_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(q_lens), float(scale), int(window), int(num_splits), _ptr(out),
        _ptr(k_scale), _ptr(v_scale), ctypes.byref(dims), _stream(stream)))


def noalloc_scratch_bytes() -> int:
    return int(load_library().pda_noalloc_scratch_bytes())


def hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None):
    """One launch of the streaming-read probe over all of ``src`` (a
    contiguous device tensor); ``sink`` holds at least ``workgroups`` int32."""
    _contig(src, sink)
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink must hold one 32-bit word per workgroup")
    _check(load_library().pda_hbm_read_probe(_ptr(src), nbytes, _ptr(sink), int(workgroups),
                                             _stream(stream)))


def attention_stages(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale, window,
                     num_splits, out, k_scale=None, v_scale=None, kv_dtype=None,
                     max_q_len=None, workspace=None, stream=None, kernel="auto",
                     kv_layout="NHD", stage="both"):
    """paged_decode_attention as its two launches, run one at a time
    (``stage`` "decode", "combine" or "both"; a combine stage must follow a
    decode stage of the same call on the same ``workspace``). Returns the
    workspace used."""
    lib = load_library()
    _contig(q, k_cache, v_cache, block_table, seq_lens, q_lens, out, k_scale, v_scale)
    dims = decode_dims(q, k_cache, block_table, seq_lens, q_lens, max_q_len, kv_dtype, kernel,
                       kv_layout)
    need = workspace_bytes(dims, window, num_splits)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stage in ("decode", "both"):
        _check(lib.pda_attention_decode_stage(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
            _ptr(q_lens), float(scale), int(window), int(num_splits), _ptr(out),
            _ptr(k_scale), _ptr(v_scale), ctypes.byref(dims), _ptr(workspace), ws_bytes,
            _stream(stream)))
    if stage in ("combine", "both"):
        _check(lib.pda_attention_combine_stage(
            _ptr(out), ctypes.byref(dims), int(window), int(num_splits), _ptr(workspace),
            ws_bytes, _stream(stream)))
    return workspace


def paged_decode_partials(q, k_cache, v_cache, block_table, seq_lens, q_lens, scale,
                          window, num_splits, workspace, k_scale=None, v_scale=None,
                          kv_dtype=None, max_q_len=None, stream=None, kernel="auto",
                          kv_layout="NHD") -> int:
    """The decode stage alone: writes split partials into ``workspace`` (a
    float32 or uint8 tensor of at least partials_bytes(...) bytes). Returns
    the split count used."""
    lib = load_library()
    _contig(q, k_cache, v_cache, block_table, seq_lens, q_lens, workspace, k_scale, v_scale)
    dims = decode_dims(q, k_cache, block_table, seq_lens, q_lens, max_q_len, kv_dtype, kernel,
                       kv_layout)
    S = resolve_splits(dims, window, num_splits)
    _check(lib.pda_paged_decode_partials(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(q_lens), float(scale), int(window), S, _ptr(k_scale), _ptr(v_scale),
        ctypes.byref(dims), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return S


def split_combine(partial_o, partial_ml, out, num_splits: int, stream=None):
    """Merge split partials (float32 [T, Hq, S, D] and [T, Hq, S, 2]) into
    ``out`` (fp16 [T, Hq, D])."""
    lib = load_library()
    _contig(partial_o, partial_ml, out)
    T, Hq, D = out.shape
    _check(lib.pda_split_combine(_ptr(partial_o), _ptr(partial_ml), _ptr(out), T, Hq, D,
                                 int(num_splits), _stream(stream)))


def write_kv_cache(key, value, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None,
                   kv_dtype=None, stream=None, kv_layout="NHD"):
    """Store new tokens' rows key[t], value[t] (fp16 [T, Hkv, D]) at slot
    slot_mapping[t] (int32 [T]; page * P + position, negative: skipped) of
    the caches [num_pages, P, Hkv, D], quantizing to fp8-e4m3 / int8 codes
    with the per-KV-head fp32 scales for quantized caches (see
    include/pda.h). Writes the caches in place and returns None."""
    lib = load_library()
    _contig(key, value, slot_mapping, k_cache, v_cache, k_scale, v_scale)
    if slot_mapping.dtype != torch.int32:
        raise ValueError("slot_mapping must be int32")
    if key.dtype != torch.float16 or value.dtype != torch.float16:
        raise ValueError("key and value must be float16")
    T, Hkv, D = key.shape
    if tuple(value.shape) != (T, Hkv, D) or tuple(slot_mapping.shape) != (T,):
        raise ValueError("value must match key's shape and slot_mapping must be [T]")
    if kv_layout == "HND":
        num_pages, Hkv_c, P, D_c = k_cache.shape
    else:
        num_pages, P, Hkv_c, D_c = k_cache.shape
    if (Hkv_c, D_c) != (Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [num_pages, P, Hkv, D] (NHD) or "
                         "[num_pages, Hkv, P, D] (HND) matching key")
    dims = CacheDims(num_tokens=T, num_kv_heads=Hkv, head_dim=D, page_size=P,
                     num_pages=num_pages, kv_dtype=_kv_code(k_cache, kv_dtype),
                     kv_layout=KV_LAYOUTS[kv_layout])
    _check(lib.pda_write_kv_cache(_ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                  ctypes.byref(dims), _stream(stream)))


def partials_views(workspace: torch.Tensor, num_tokens: int, num_q_heads: int,
                   num_splits: int, head_dim: int):
    """(partial_o [T, Hq, S, D], partial_ml [T, Hq, S, 2]) float32 views of a
    workspace written by paged_decode_partials (layout of include/pda.h)."""
    f = workspace.view(torch.float32) if workspace.dtype != torch.float32 else workspace
    n_o = num_tokens * num_q_heads * num_splits * head_dim
    n_ml = num_tokens * num_q_heads * num_splits * 2
    po = f[:n_o].view(num_tokens, num_q_heads, num_splits, head_dim)
    pml = f[n_o:n_o + n_ml].view(num_tokens, num_q_heads, num_splits, 2)
    return po, pml
