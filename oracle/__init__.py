"""fp64 CPU oracle for paged split-K decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package; only the tests, the smoke check of ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may use it. It shares no code, tables or
constants with the HIP library: it is the plain definition of the operation,
written out in numpy float64 so that a reader can check it against the
pages by eye.
"""

from .attention import (  # noqa: F401
    decode_f16,
    decode_e4m3fn,
    decode_int8,
    dequantize,
    visible_range,
    as_nhd,
    paged_decode_attention,
    paged_decode_attention_split,
    split_combine,
)
from .kv_writer import (  # noqa: F401
    encode_e4m3fn,
    encode_int8,
    quantize,
    write_kv_cache,
)
