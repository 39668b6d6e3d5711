"""Per-item phase timeline of the long-query (prefill) kernel.

A diagnostic build of the library (-DPDA_PREFILL_TIMELINE=1) has wave 0 of
each work item (token block, KV head, sequence) read the 100 MHz clock at the
end of each phase of the item's start and end, and the shader clock over the
whole item, each reading waited for at once; it writes them over the first
values of the item's first output row, so its output is not the attention
result. This module builds that variant beside the library and reads it:

    python -m paged_split_decode_amd.timeline --build        (no GPU needed)
    python -m paged_split_decode_amd.timeline prefill_d128_b4_q2048 ...

For each named workload it prints the mean of each phase over the items with
at least one step (ns), the loop per step, the gap between an item's end and
the next item's start on the same CU, and the shader clock (cycles over the
item / its duration). Run from the repository root (the synthetic workloads
live in its `synth` package).
"""

from __future__ import annotations

import argparse
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
TL_DIR = os.path.join(PKG, "_timeline")
TL_LIB = os.path.join(TL_DIR, "libpda.so")
PHASES = ["setup and token offset", "Q and first steps' loads issued", "wait for step 0",
          "tail zeroing and first barrier", "step loop", "epilogue"]


def build() -> str:
    from paged_split_decode_amd import build as pda_build
    return pda_build.build(defines=("-DPDA_PREFILL_TIMELINE=1",), lib=TL_LIB,
                           build_dir=os.path.join(TL_DIR, "_build"), verbose=True)


def _waves(head_dim: int, max_q_len: int, key_capacity: int, group: int) -> int:
    # the host's choice of workgroup shape (prefill_waves in csrc/pda_kernels.h)
    if head_dim == 256:
        return 8
    return 8 if (4 * max_q_len <= key_capacity or group * max_q_len >= 512) else 4


def run(names, repeats: int = 3) -> None:
    if not os.path.exists(TL_LIB):
        raise SystemExit(f"{TL_LIB} is missing: python -m paged_split_decode_amd.timeline --build")
    os.environ["PDA_LIBRARY"] = TL_LIB
    import numpy as np
    import torch

    import paged_split_decode_amd as pda
    from synth import WORKLOADS, make_case

    assert pda.library_path() == TL_LIB
    for name in names:
        c = make_case(WORKLOADS[name], device="cuda")
        T, Hq, D = c.q.shape
        Hkv = c.workload.num_kv_heads
        G = Hq // Hkv
        ql = c.q_lens_host
        cap = int(c.block_table.shape[1]) * c.workload.page_size
        waves = _waves(D, int(ql.max()), cap, G)
        bq = 32 * (waves // 2 if D == 256 else waves) // G  # tokens per item
        out = torch.empty((T, Hq, D), dtype=torch.float16, device="cuda")
        for _ in range(repeats):
            pda.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.q_lens,
                                       c.scale, c.window, 1, out, k_scale=c.k_scale,
                                       v_scale=c.v_scale, kv_dtype=c.kv_dtype, max_q_len=int(ql.max()))
        torch.cuda.synchronize()
        u = out.view(torch.int32).reshape(T, Hq, D // 2).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        offs = np.concatenate([[0], np.cumsum(ql)[:-1]])
        rec = np.array([u[offs[b] + blk * bq, g * G, :11] for b in range(len(ql)) for g in range(Hkv)
                        for blk in range((int(ql[b]) + bq - 1) // bq)])
        t = rec[:, :7] - rec[:, 0].min()
        steps = rec[:, 8]
        cu = (rec[:, 10] & 0xF) * 4096 + (rec[:, 9] >> 8 & 0x3FFF)  # XCC, then SE / SH / CU of HW_ID
        gaps = []
        for k in np.unique(cu):
            o = np.where(cu == k)[0]
            o = o[np.argsort(t[o, 0])]
            gaps += [(t[o[i], 0] - t[o[i - 1], 6]) * 10 for i in range(1, len(o))]
        live = steps > 0
        d = np.diff(t[live], axis=1) * 10.0
        clock = rec[live, 7] / np.maximum((t[live, 6] - t[live, 0]) * 10.0, 1.0)
        print(f"{name}: {len(rec)} items, {waves} waves, {bq} tokens each, on {len(np.unique(cu))} CUs;"
              f" kernel span {t[:, 6].max() / 100:.1f} us")
        for i, ph in enumerate(PHASES):
            print(f"  {ph:34s} {d[:, i].mean():8.0f} ns")
        print(f"  {'step loop per step':34s} {(d[:, 4] / steps[live]).mean():8.0f} ns"
              f" ({steps[live].mean():.1f} steps per item)")
        if gaps:
            print(f"  {'gap to the next item on the CU':34s} {np.mean(gaps):8.0f} ns")
        print(f"  shader clock {clock.mean():.3f} GHz (items {clock.min():.3f} .. {clock.max():.3f})")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("workloads", nargs="*")
    ap.add_argument("--build", action="store_true", help="build the diagnostic library variant")
    ap.add_argument("--repeats", type=int, default=3)
    args = ap.parse_args(argv)
    if args.build:
        build()
    if args.workloads:
        run(args.workloads, args.repeats)


if __name__ == "__main__":
    main()
    sys.exit(0)
