"""Benchmark: paged split-K decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the whole hot path (pda_paged_decode_attention: decode
and split combine) over one batch of synthetic input already resident in HBM. The headline workload
is the fp16-KV D=128 case: 8 sequences of 4096 keys, 32 query heads over 8
KV heads, page size 16, seeded random page permutation, automatic splits.
Its KV pool (134 MB) fits in the 256 MiB Infinity Cache, so the timed loop
rotates over enough replicas of the inputs (>= 1 GiB in total) that every step
reads its KV from HBM.

Reported (one JSON line):
  value        algorithmic bytes (every visible K/V element once, q, out) per
               step / measured step time, GB/s
  roofline     the decode kernel alone: same bytes / its average launch
               duration (launches queued back to back on the launch stream,
               HIP events around them), against the 8 TB/s HBM peak;
               traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE +
               WRITE_SIZE counters (each scaled by what the counter reads for
               a plain 1 GiB copy) when a counter summary for the current
               kernel sources exists, else null
  cpu_baseline the fp64 oracle on this host's cores, on a bounded sample of
               the same workload
  cells        the same measurement for the D=256 and other workloads, each
               in a process of its own (its KV pool the first large
               allocation there, as in a serving process)
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "decode-attn achieved HBM GB/s (fraction of peak) + us/call, D=128 & D=256"
HEADLINE = "gqa4_d128_b8_l4096"
CELLS = [
    # the headline shape with a caller split count inside the 1..8 range its
    # configuration names for automatic splitting
    ("gqa4_d128_b8_l4096", dict(num_splits=8)),
    # the headline shape in the other cache layouts: HND ([page, head, slot,
    # dim]), 64-key pages, and an identity block table (pages in pool order)
    ("gqa4_d128_b8_l4096", dict(layout="HND")),
    ("gqa4_d128_b8_l4096", dict(page_size=64)),
    ("gqa4_d128_b8_l4096", dict(identity_table=True)),
    # D=256 batch sweep, without and with a 4096-key sliding window
    *[("gqa6_d256_l16384", dict(batch=b, window=win))
      for win in (0, 4096) for b in (1, 2, 3, 8, 32)],
    ("verify_q3_d128_b32", {}),
    # the same ragged batch with automatic splits (balanced per sequence)
    ("verify_q3_d128_b32", dict(num_splits=0)),
    ("quant_fp8_d256_b64_l32768", {}),
    ("quant_int8_d256_b64_l32768", {}),
]


# Sources the decode step is built from (kernels, their launch plan, combine),
# and those of the prefill kernel.
DECODE_SOURCES = ("pda_kernels.h", "pda_decode_impl.h", "pda_decode_mfma.h", "pda_decode_f16.hip",
                  "pda_decode_fp8.hip", "pda_decode_i8.hip", "pda_api.hip", "pda_combine.hip")
PREFILL_SOURCES = ("pda_kernels.h", "pda_decode_impl.h", "pda_decode_mfma.h",
                   "pda_prefill_mfma.h", "pda_prefill.hip", "pda_api.hip")


_TOKEN = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with whitespace collapsed (string
    literals kept), so that a comment edit does not count as a kernel change."""
    text = _TOKEN.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return " ".join(text.split())


def kernel_source_hash(kernel: str = "decode_mfma") -> str:
    """Hash of the HIP sources of a kernel (the decode step, or the prefill
    kernel when `kernel` starts with "prefill") and of the compiler flags they
    are built with: counter figures recorded for one hash do not describe a
    kernel built from different sources or flags."""
    from paged_split_decode_amd import build as pda_build

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_split_decode_amd", "csrc")
    for f in PREFILL_SOURCES if kernel.startswith("prefill") else DECODE_SOURCES:
        with open(os.path.join(csrc, f)) as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
        h.update(" ".join(pda_build.EXTRA.get(f, [])).encode())
    h.update(" ".join(a for a in pda_build.COMMON if not a.startswith("/")).encode())
    return h.hexdigest()[:16]


def workload_key(workload: str, over: dict) -> str:
    """Name of a workload with the command line's overrides (batch, window,
    split count), as profiles/ files are keyed."""
    tags = {"batch": "b", "window": "w", "num_splits": "s"}
    return workload + "".join(f"_{tags[k]}{v}" for k, v in sorted(over.items()) if k in tags)


def traffic_for(key: str):
    """HBM bytes per decode launch from a committed rocprofv3 counter summary
    of the current kernel sources (profiles/traffic_<key>.json), else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(rec.get("kernel", "decode_mfma")):
        return None
    return rec.get("hbm_bytes_per_launch")


class Runner:
    """Pre-marshalled C-ABI calls for one case (no per-step Python work
    beyond the ctypes call)."""

    def __init__(self, case, device, replicas: int, num_splits: int, kernel: str = "auto"):
        import torch

        import paged_split_decode_amd as pda

        self.pda = pda
        self.lib = pda.load_library()
        self.case = case
        c = case
        self.dims = pda.decode_dims(c.q, c.k_cache, c.block_table, c.seq_lens, c.q_lens,
                                    c.max_q_len, c.kv_dtype, kernel, c.kv_layout)
        # 0 stays 0 (automatic: split counts balanced per sequence where the
        # matrix kernel can); a caller's count is used as given.
        self.S = num_splits
        T, Hq, D = c.q.shape
        self.T, self.Hq, self.D = T, Hq, D
        self.out = torch.empty((T, Hq, D), dtype=torch.float16, device=device)
        nws = pda.workspace_bytes(self.dims, c.window, self.S)
        self.ws_all = torch.empty(max(nws, 16), dtype=torch.uint8, device=device)
        # Replicas of everything a step reads, so consecutive steps do not
        # hit in the Infinity Cache.
        self.reps = [(c.q, c.k_cache, c.v_cache)]
        for _ in range(replicas - 1):
            self.reps.append((c.q.clone(), c.k_cache.clone(), c.v_cache.clone()))
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = ctypes.c_void_p
        self.common = (P(c.block_table.data_ptr()), P(c.seq_lens.data_ptr()),
                       P(c.q_lens.data_ptr()), ctypes.c_float(c.scale),
                       ctypes.c_int32(c.window), ctypes.c_int32(self.S))
        self.scales = (None if c.k_scale is None else P(c.k_scale.data_ptr()),
                       None if c.v_scale is None else P(c.v_scale.data_ptr()))
        self.dims_ref = ctypes.byref(self.dims)
        self.wsa_ptr, self.wsa_bytes = P(self.ws_all.data_ptr()), self.ws_all.numel()
        self.out_ptr = P(self.out.data_ptr())
        self.rep_ptrs = [tuple(P(t.data_ptr()) for t in r) for r in self.reps]

    def step(self, i: int):
        """One full call of the hot path (pda_paged_decode_attention)."""
        q, k, v = self.rep_ptrs[i % len(self.rep_ptrs)]
        st = self.lib.pda_paged_decode_attention(
            q, k, v, *self.common, self.out_ptr, *self.scales, self.dims_ref, self.wsa_ptr,
            self.wsa_bytes, self.stream)
        if st != 0:
            raise RuntimeError(self.lib.pda_last_error().decode())

    def decode(self, i: int):
        """The dominant kernel alone: the decode stage of the same call (the
        step's first launch; its only one with one split)."""
        q, k, v = self.rep_ptrs[i % len(self.rep_ptrs)]
        st = self.lib.pda_attention_decode_stage(
            q, k, v, *self.common, self.out_ptr, *self.scales, self.dims_ref, self.wsa_ptr,
            self.wsa_bytes, self.stream)
        if st != 0:
            raise RuntimeError(self.lib.pda_last_error().decode())



SETTLE_MS = 20.0  # GPU time of untimed steps between the hold and a timed loop


def settle_steps(ms_per_step: float) -> int:
    """Untimed steps worth about SETTLE_MS of GPU time (5 to 400)."""
    return int(min(400, max(5, math.ceil(SETTLE_MS / max(ms_per_step, 1e-3)))))


def _hold_gpu():
    """Keep the GPU busy for a few ms so that the timed launches that follow
    are all queued before the first one runs (they then run back to back,
    as a captured graph would)."""
    import torch

    torch.cuda._sleep(50_000_000)


def measure(case, steps: int, warmup: int, num_splits: int, device, kernel: str = "auto"):
    """Time `steps` passes. Returns step time (device, launches queued ahead),
    eager step time (launches paced by the host), and the decode kernel's
    average launch duration from HIP events around each launch."""
    import torch

    from synth import algorithmic_bytes

    nbytes = algorithmic_bytes(case)
    pool = case.k_cache.numel() * case.k_cache.element_size() * 2
    replicas = max(1, min(16, math.ceil((1 << 30) / max(pool, 1))))
    r = Runner(case, device, replicas, num_splits, kernel)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # Every replica is read at least once before timing (first touches of
    # freshly allocated memory are not part of a step); the warmup also
    # gives an estimate of the step time.
    n_warm = max(warmup, replicas)
    t0.record()
    for i in range(n_warm):
        r.step(i)
    t1.record()
    torch.cuda.synchronize()
    settle = settle_steps(t0.elapsed_time(t1) / n_warm)

    def queued(fn):
        """`steps` calls queued back to back behind the hold, after `settle`
        untimed ones: the clocks drop while the GPU runs the hold's single
        wave and take tens of milliseconds of load to come back (the
        compute-bound prefill measured 10-15% slow without this; the decode
        did not change)."""
        _hold_gpu()
        for i in range(settle):
            fn(i)
        t0.record()
        for i in range(steps):
            fn(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    # Whole steps, queued ahead of the device.
    ms_step = queued(r.step)

    # The distribution over calls: the same queued steps with an event pair
    # around each call (the events add a little between calls, so the mean
    # above stays the figure of record).
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    _hold_gpu()
    for i in range(settle):
        r.step(i)
    for i, (a, b) in enumerate(pairs):
        a.record()
        r.step(i)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    pick = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]  # noqa: E731
    per_call = {"p10": round(pick(0.1), 2), "median": round(pick(0.5), 2),
                "p90": round(pick(0.9), 2), "calls": len(per)}

    # The same, paced by the host (no queue-ahead).
    t0.record()
    for i in range(steps):
        r.step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1) / steps

    # The decode kernel alone: `steps` launches queued back to back on the
    # launch stream, bracketed by two events.
    decode_ms = queued(r.decode)
    return dict(ms_per_step=ms_step, ms_eager=ms_eager, decode_ms=decode_ms, bytes=nbytes,
                splits=r.S if r.S >= 1 else "auto", replicas=replicas, settle=settle,
                per_call_us=per_call)


def cpu_baseline(case, budget_s: float = 12.0):
    """The fp64 oracle on this host, on whole (sequence, KV head) units of the
    same workload, repeated until about `budget_s` seconds of work."""
    import numpy as np

    import oracle
    from synth import algorithmic_bytes

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    h = case.host()
    nbytes = algorithmic_bytes(case)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_decode_attention(**h)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    np.asarray(0)
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the whole {case.workload.name} workload (all {len(h['seq_lens'])} "
                      f"sequences x {h['k_cache'].shape[2]} KV heads), {reps} pass(es) in "
                      f"{el:.1f} s"}


# Long-query (prefill kernel) cells: a fresh prefill and a chunked prefill.
PREFILL_CELLS = ["prefill_d128_b4_q2048", "chunked_d128_b8_l8192_q512", "prefill_d256_b4_q2048"]
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, AMD published


def prefill_record(name, case, m):
    from synth import visible_pairs

    flops = 4 * case.workload.head_dim * visible_pairs(case)
    us = m["ms_per_step"] * 1e3
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": name, "op": "prefill", "batch": case.workload.batch,
            "q_len": case.workload.q_len, "seq_len": case.workload.seq_len,
            "us_per_call": round(us, 2), "per_call_us": m["per_call_us"], "TFLOP_s": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)},
            "flops": flops, "GB_s": round(m["bytes"] / (us * 1e-6) / 1e9, 1),
            "algorithmic_bytes": m["bytes"]}


# Cache-writer cells: (tokens, KV heads, head dim, kv dtype): the new tokens of
# the fp8 long-context decode step, and prefill-sized writes.
WRITER_CELLS = [
    (64, 4, 256, "fp8_e4m3"),
    (32768, 8, 128, "f16"),
    (32768, 4, 256, "fp8_e4m3"),
    (32768, 4, 256, "int8"),
]


def measure_writer(T, Hkv, D, kv, steps, device):
    """One pda_write_kv_cache call per step over seeded rows (replicated past
    1 GiB so steps do not hit in the Infinity Cache). Bytes: the fp16 rows
    read, the cache rows written, the slots."""
    import torch

    import paged_split_decode_amd as pda
    from synth import make_write_case

    P = 16
    c = make_write_case(T, Hkv, D, P, num_pages=-(-T // P) + 1, kv_dtype=kv, seed=T + D,
                        skip_frac=0.0, device=device)
    e = 2 if kv == "f16" else 1
    nbytes = T * Hkv * D * (2 + e) * 2 + T * 4
    per = nbytes - T * 4
    reps = max(1, min(16, math.ceil((1 << 30) / per)))
    sets = [(c.key, c.value, c.k_cache, c.v_cache)]
    for _ in range(reps - 1):
        sets.append((c.key.clone(), c.value.clone(), c.k_cache.clone(), c.v_cache.clone()))

    def run(i):
        k, v, kc, vc = sets[i % reps]
        pda.write_kv_cache(k, v, c.slot_mapping, kc, vc, c.k_scale, c.v_scale, kv_dtype=kv)

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    n_warm = max(3, reps)
    t0.record()
    for i in range(n_warm):
        run(i)
    t1.record()
    torch.cuda.synchronize()
    settle = settle_steps(t0.elapsed_time(t1) / n_warm)
    _hold_gpu()
    for i in range(settle):
        run(i)
    t0.record()
    for i in range(steps):
        run(i)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"op": "write_kv_cache", "tokens": T, "num_kv_heads": Hkv, "head_dim": D,
            "kv_dtype": kv, "page_size": P, "us_per_call": round(us, 2), "GB_s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}


def cell_record(name, w, m):
    us = m["ms_per_step"] * 1e3
    gbs = m["bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    dec_gbs = m["bytes"] / (m["decode_ms"] * 1e-3) / 1e9
    return {"workload": name, "batch": w.batch, "window": w.window, "kv_dtype": w.kv_dtype,
            "head_dim": w.head_dim, "page_size": w.page_size, "kv_layout": w.layout,
            "identity_table": w.identity_table, "splits": m["splits"],
            "us_per_call": round(us, 2),
            "GB_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "eager_us_per_call": round(m["ms_eager"] * 1e3, 2), "per_call_us": m["per_call_us"],
            "decode_us": round(m["decode_ms"] * 1e3, 2), "decode_GB_s": round(dec_gbs, 1),
            "algorithmic_bytes": m["bytes"]}


def measure_cell(spec: str, steps: int, kernel: str, device):
    """One extra cell ("decode:i", "prefill:i" or "writer:i" of CELLS,
    PREFILL_CELLS, WRITER_CELLS)."""
    from synth import WORKLOADS, make_case

    kind, i = spec.split(":")
    i = int(i)
    n = max(50, steps // 2)  # at least 50 calls per cell (percentiles)
    if kind == "decode":
        name, over = CELLS[i]
        wc = WORKLOADS[name].with_(**over)
        return cell_record(name, wc, measure(make_case(wc, device=device), n, 10,
                                             wc.num_splits, device, kernel))
    if kind == "prefill":
        c = make_case(WORKLOADS[PREFILL_CELLS[i]], device=device)
        return prefill_record(PREFILL_CELLS[i], c, measure(c, n, 10, 1, device, kernel))
    T, Hkv, D, kv = WRITER_CELLS[i]
    return measure_writer(T, Hkv, D, kv, n, device)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    ap.add_argument("--window", type=int, default=None, help="override the sliding window")
    ap.add_argument("--splits", type=int, default=None, help="override num_splits (0: auto)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "vector", "matrix"],
                    help="decode kernel family")
    ap.add_argument("--reference-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for calibrating HBM byte counters)")
    ap.add_argument("--no-cells", action="store_true", help="skip the extra workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cell", default=None,
                    help="measure one extra cell (decode:i, prefill:i or writer:i) and print "
                         "its record; the full run measures each cell this way, in a process "
                         "of its own")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this operator runs on a single MI355X)", file=sys.stderr)
        return 2

    import torch

    from synth import WORKLOADS, make_case

    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.cell:
        print(json.dumps(measure_cell(args.cell, args.steps, args.kernel, device)), flush=True)
        return 0
    if args.reference_copy_mib > 0:
        src = torch.ones(args.reference_copy_mib << 20, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = WORKLOADS[args.workload]
    over = {k: v for k, v in (("batch", args.batch), ("window", args.window),
                              ("num_splits", args.splits)) if v is not None}
    if over:
        w = w.with_(**over)
    case = make_case(w, device=device)
    m = measure(case, args.steps, args.warmup, w.num_splits, device, args.kernel)
    gbs = m["bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    dec_gbs = m["bytes"] / (m["decode_ms"] * 1e-3) / 1e9
    traffic = traffic_for(workload_key(args.workload, over))
    rec = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "seq_len": w.seq_len,
                   "q_len": w.q_len, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "kv_dtype": w.kv_dtype, "num_splits": m["splits"],
                   "us_per_call": round(m["ms_per_step"] * 1e3, 2),
                   "eager_us_per_call": round(m["ms_eager"] * 1e3, 2),
                   "per_call_us": m["per_call_us"],
                   "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes": m["bytes"], "input_replicas": m["replicas"],
                   "settle_steps": m["settle"],
                   "kernel": args.kernel,
                   "accumulate": "fp32"},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "pda_decode_mfma_kernel" if args.kernel != "vector" else "pda_decode_kernel",
                     "decode_us": round(m["decode_ms"] * 1e3, 3),
                     "kernel_source_hash": kernel_source_hash()},
    }
    if not args.no_cells:
        # Each cell in a fresh process: a KV pool allocated after other large
        # buffers were freed measured up to 4.5% slower (D=256, 32 x 16384:
        # 369 against 354 us per decode), while a serving process allocates
        # its pool once.
        del case
        torch.cuda.empty_cache()
        for kind, n, key in (("decode", len(CELLS), "cells"), ("prefill", len(PREFILL_CELLS),
                                                            "prefill_cells"),
                             ("writer", len(WRITER_CELLS), "writer_cells")):
            rec[key] = []
            for i in range(n):
                r = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), "--cell",
                                    f"{kind}:{i}", "--steps", str(args.steps), "--kernel",
                                    args.kernel], capture_output=True, text=True, timeout=900)
                if r.returncode != 0:
                    raise RuntimeError(f"cell {kind}:{i} failed:\n{r.stderr[-2000:]}")
                rec[key].append(json.loads(r.stdout.strip().splitlines()[-1]))
                print(json.dumps({f"{kind}_cell": rec[key][-1]}), file=sys.stderr, flush=True)
        case = make_case(w, device=device)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(case)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
