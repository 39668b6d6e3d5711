"""Benchmark: paged split-K decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the whole hot path (pda_paged_decode_attention: decode
and split combine) over one batch of synthetic input already resident in HBM.
The headline workload is the largest one: fp8-e4m3 KV with per-KV-head
scales, D=256, 16 query heads over 4 KV heads, 64 sequences of 32768 keys,
8 splits (4.3 GB of K+V per call). Beside it, with the same fields, go a
D=128 line (fp16 KV, 32/8 heads, 8 x 4096 keys, automatic splits) and a D=256
fp16 line (24/4 heads, 32 x 16384 keys), since the metric names both head
dimensions. Pools smaller than 1 GiB are replicated so that every timed step
reads its KV from HBM, not from the 256 MiB Infinity Cache.

Reported (one JSON line):
  value        algorithmic bytes (every visible K/V element once, q, out) per
               step / measured step time, GB/s
  roofline     the decode kernel alone: same bytes / its average launch
               duration (launches queued back to back on the launch stream,
               HIP events around them), against the 8 TB/s HBM peak and
               against the streaming-read rate measured on this device by the
               library's read probe; traffic = HBM bytes per launch from
               rocprofv3 FETCH_SIZE + WRITE_SIZE counters (each scaled by what
               the counter reads for a plain 1 GiB copy) when a counter
               summary for the current kernel sources exists, else null
  lines        the D=128 and D=256 fp16 workloads with the same fields
  cpu_baseline the fp64 oracle on this host's cores (one BLAS thread per
               worker thread, a pool over (sequence, KV head) units), per
               workload: the headline's sample is its `value`
  cells        the other workloads and variants (the tiny workload, the D=256
               batch sweep with and without a window, the ragged verify batch,
               int8 KV, layouts, the vector kernel), each measured in a
               process of its own (its KV pool the first large allocation
               there, as in a serving process)

`python bench.py --summarize DIR ...` turns rocprofv3 output (kernel trace
statistics and FETCH_SIZE / WRITE_SIZE counter runs) into the summaries kept
under profiles/.
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
HEADLINE = "quant_fp8_d256_b64_l32768"
# Lines reported with the headline's fields (roofline, traffic): the D=128
# and D=256 fp16 workloads.
LINES = [("gqa4_d128_b8_l4096", {}), ("gqa6_d256_l16384", dict(batch=32))]
CELLS = [
    # the tiny workload at its two split counts (latency-bound: us only)
    ("tiny_d128", dict(num_splits=1)),
    ("tiny_d128", dict(num_splits=3)),
    # the D=128 shape with a caller split count inside the 1..8 range its
    # configuration names for automatic splitting
    ("gqa4_d128_b8_l4096", dict(num_splits=8)),
    # the D=128 shape in the other cache layouts: HND ([page, head, slot,
    # dim]), 64-key pages, and an identity block table (pages in pool order)
    ("gqa4_d128_b8_l4096", dict(layout="HND")),
    ("gqa4_d128_b8_l4096", dict(page_size=64)),
    ("gqa4_d128_b8_l4096", dict(identity_table=True)),
    # D=256 batch sweep, without and with a 4096-key sliding window (B=32
    # without a window is a line)
    *[("gqa6_d256_l16384", dict(batch=b, window=win))
      for win in (0, 4096) for b in (1, 2, 3, 8, 32) if (b, win) != (32, 0)],
    ("verify_q3_d128_b32", {}),
    # the same ragged batch with automatic splits (balanced per sequence)
    ("verify_q3_d128_b32", dict(num_splits=0)),
    ("quant_int8_d256_b64_l32768", {}),
]
# The vector (v_dot2) kernel family on the four larger workloads.
VECTOR_CELLS = [
    ("gqa4_d128_b8_l4096", {}),
    ("gqa6_d256_l16384", dict(batch=32)),
    ("verify_q3_d128_b32", {}),
    ("quant_fp8_d256_b64_l32768", {}),
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


def workload_key(workload: str, over: dict, kernel: str = "auto") -> str:
    """Name of a workload with the command line's overrides (batch, window,
    split count) and, for the vector kernel family, that family, as profiles/
    files are keyed."""
    tags = {"batch": "b", "window": "w", "num_splits": "s", "page_size": "p"}
    key = workload + "".join(f"_{tags[k]}{v}" for k, v in sorted(over.items()) if k in tags)
    if over.get("layout", "NHD") != "NHD":
        key += "_" + over["layout"].lower()
    if over.get("identity_table"):
        key += "_identity"
    return key + ("_vector" if kernel == "vector" else "")


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
                         "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic_for(name)},
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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Worker threads for the oracle: the host's cores, at most 16 (the CPU
    share of one GPU on the boxes this runs on)."""
    return max(1, min(16, os.cpu_count() or 1))


def time_oracle_units(case, units, threads: int, repeats: int = 1) -> float:
    """Wall seconds for the fp64 oracle over the given (sequence, KV head)
    units of `case` (each gathered from the pool beforehand, outside the
    timed region), `threads` units at a time on a pool of host threads with
    one BLAS thread each; the median of `repeats` runs."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    import oracle
    from synth import unit_subcase

    subs = [unit_subcase(case, b, g) for b, g in units]
    times = []
    with threadpool_limits(limits=1):
        for _ in range(repeats):
            t0 = time.perf_counter()
            if threads == 1:
                for sub in subs:
                    oracle.paged_decode_attention(**sub)
            else:
                with ThreadPoolExecutor(max_workers=threads) as ex:
                    list(ex.map(lambda sub: oracle.paged_decode_attention(**sub), subs))
            times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2]


# Oracle timings per workload: (workload, overrides, units timed (None: all),
# repeats, also with one thread). Every workload is timed whole (all its
# (sequence, KV head) units); a sample would scale the time by units.
CPU_CONFIGS = [
    ("tiny_d128", {}, None, 5, True),
    ("gqa4_d128_b8_l4096", {}, None, 3, True),
    ("gqa6_d256_l16384", dict(batch=32), None, 1, False),
    ("gqa6_d256_l16384", dict(batch=32, window=4096), None, 1, False),
    ("verify_q3_d128_b32", {}, None, 1, False),
    ("quant_fp8_d256_b64_l32768", {}, None, 1, False),
    ("quant_int8_d256_b64_l32768", {}, None, 1, False),
]


def cpu_baseline(device, gpu_us: dict, headline_case=None):
    """The fp64 oracle timed on this host, per workload. Returns the record
    whose `value` is the headline workload's rate (algorithmic bytes of one
    call / the oracle's time for that call)."""
    import torch

    from synth import WORKLOADS, algorithmic_bytes, make_case

    threads = oracle_threads()
    per = []
    head = None
    for name, over, n_units, repeats, single in CPU_CONFIGS:
        w = WORKLOADS[name].with_(**over)
        if headline_case is not None and name == HEADLINE and not over:
            case = headline_case
        else:
            case = make_case(w, device=device)
        units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
        total = len(units)
        if n_units is not None and n_units < total:
            step = total / n_units
            units = [units[int(i * step)] for i in range(n_units)]
        wall = time_oracle_units(case, units, threads, repeats)
        us = wall * 1e6 * total / len(units)
        nbytes = algorithmic_bytes(case)
        key = workload_key(name, over)
        rec = {"workload": key, "units": total, "units_timed": len(units), "threads": threads,
               "wall_s": round(wall, 4), "us_per_call": round(us, 1),
               "GB_s": round(nbytes / (us * 1e-6) / 1e9, 4)}
        if key in gpu_us:
            rec["gpu_us_per_call"] = gpu_us[key]
            rec["gpu_speedup"] = round(us / gpu_us[key], 1)
        if single:
            w1 = time_oracle_units(case, units, 1, repeats)
            rec["single_thread_wall_s"] = round(w1, 4)
            rec["single_thread_us_per_call"] = round(w1 * 1e6 * total / len(units), 1)
        per.append(rec)
        print(json.dumps({"cpu_oracle": rec}), file=sys.stderr, flush=True)
        if name == HEADLINE and not over:
            head = rec
        if case is not headline_case:
            del case
            torch.cuda.empty_cache()
    return {"value": head["GB_s"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{head['units_timed']} of the {head['units']} (sequence, KV head) units of "
                      f"{HEADLINE} (one whole call), on {threads} host threads (one BLAS thread "
                      f"each): {head['wall_s']} s",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(), "per_workload": per}


def measure_probe(device, steps: int = 20):
    """The streaming-read rate of one launch of the library's read probe over
    a 4 GiB buffer (well past the on-package caches), for a few grid sizes;
    the best one is this device's measured read roof."""
    import torch

    import paged_split_decode_amd as pda

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf.fill_(1)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    best, rows = None, []
    for per_cu in (4, 8, 16, 32, 64):
        wg = n_cu * per_cu
        sink = torch.zeros(wg, dtype=torch.int32, device=device)
        for _ in range(3):
            pda.hbm_read_probe(buf, sink, wg)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        _hold_gpu()
        t0.record()
        for _ in range(steps):
            pda.hbm_read_probe(buf, sink, wg)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / steps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        rows.append({"workgroups": wg, "us": round(us, 1), "GB_s": round(gbs, 1)})
        if best is None or gbs > best["GB_s"]:
            best = rows[-1]
    return {"probe": "pda_hbm_read_probe (16-byte non-temporal loads, grid-stride)",
            "bytes": nbytes, "GB_s": best["GB_s"], "workgroups": best["workgroups"],
            "frac_of_peak": round(best["GB_s"] / HBM_PEAK_GBS, 4), "sweep": rows}


def decode_record(name, over, w, m, kernel="auto", roof_gbs=None):
    """Fields of a measured decode workload: whole-call rate, and the decode
    kernel's own rate against the peak and the measured read roof."""
    us = m["ms_per_step"] * 1e3
    gbs = m["bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    dec_gbs = m["bytes"] / (m["decode_ms"] * 1e-3) / 1e9
    key = workload_key(name, over, kernel)
    rec = {"workload": key, "batch": w.batch, "window": w.window, "kv_dtype": w.kv_dtype,
           "head_dim": w.head_dim, "page_size": w.page_size, "kv_layout": w.layout,
           "identity_table": w.identity_table, "splits": m["splits"], "kernel": kernel,
           "us_per_call": round(us, 2), "GB_s": round(gbs, 1),
           "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
           "eager_us_per_call": round(m["ms_eager"] * 1e3, 2), "per_call_us": m["per_call_us"],
           "decode_us": round(m["decode_ms"] * 1e3, 2), "decode_GB_s": round(dec_gbs, 1),
           "algorithmic_bytes": m["bytes"]}
    if roof_gbs:
        rec["frac_of_measured_roof"] = round(gbs / roof_gbs, 4)
    return rec


def roofline_record(m, kernel, key, roof_gbs=None):
    dec_gbs = m["bytes"] / (m["decode_ms"] * 1e-3) / 1e9
    family = "decode_vector" if kernel == "vector" else "decode_mfma"
    rec = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(key),
           "kernel": "pda_decode_kernel" if kernel == "vector" else "pda_decode_mfma_kernel",
           "decode_us": round(m["decode_ms"] * 1e3, 3),
           "kernel_source_hash": kernel_source_hash(family)}
    if roof_gbs:
        rec["measured_roof_GB_s"] = roof_gbs
        rec["frac_of_measured_roof"] = round(dec_gbs / roof_gbs, 4)
    return rec


def measure_cell(spec: str, steps: int, kernel: str, device):
    """One workload measured on its own ("line:i", "decode:i", "vector:i",
    "prefill:i", "writer:i" or "probe:0")."""
    from synth import WORKLOADS, make_case

    kind, i = spec.split(":")
    i = int(i)
    n = max(50, steps // 2)  # at least 50 calls per cell (percentiles)
    if kind == "probe":
        return measure_probe(device)
    if kind in ("line", "decode", "vector"):
        name, over = {"line": LINES, "decode": CELLS, "vector": VECTOR_CELLS}[kind][i]
        kern = "vector" if kind == "vector" else kernel
        wc = WORKLOADS[name].with_(**over)
        m = measure(make_case(wc, device=device), n if kind != "line" else steps, 10,
                    wc.num_splits, device, kern)
        rec = decode_record(name, over, wc, m, kern)
        if kind in ("line", "vector"):
            rec["roofline"] = roofline_record(m, kern, rec["workload"])
        return rec
    if kind == "prefill":
        c = make_case(WORKLOADS[PREFILL_CELLS[i]], device=device)
        return prefill_record(PREFILL_CELLS[i], c, measure(c, n, 10, 1, device, kernel))
    T, Hkv, D, kv = WRITER_CELLS[i]
    return measure_writer(T, Hkv, D, kv, n, device)


def run_cell(spec: str, steps: int, kernel: str) -> dict:
    """measure_cell in a process of its own."""
    r = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), "--cell", spec,
                        "--steps", str(steps), "--kernel", kernel],
                       capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        raise RuntimeError(f"cell {spec} failed:\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def _with_roof(rec, roof):
    """Add the fractions of the measured read roof to a record."""
    if not roof:
        return rec
    rec["frac_of_measured_roof"] = round(rec["GB_s"] / roof, 4)
    if "roofline" in rec:
        rec["roofline"]["measured_roof_GB_s"] = roof
        rec["roofline"]["frac_of_measured_roof"] = round(rec["roofline"]["achieved"] / roof, 4)
    return rec


# ---------------------------------------------------------------------------
# rocprofv3 summaries (profiles/)
# ---------------------------------------------------------------------------


def _csv_rows(root: str, suffix: str):
    import csv

    rows = []
    for dirpath, _, files in os.walk(root):
        for fn in sorted(files):
            if fn.endswith(suffix):
                with open(os.path.join(dirpath, fn), newline="") as f:
                    rows.extend(csv.DictReader(f))
    return rows


def _kernel_family(name: str) -> str:
    if "pda_prefill_mfma_kernel" in name:
        return "prefill_mfma"
    if "pda_decode_mfma_kernel" in name:
        return "decode_mfma"
    if "pda_decode_kernel" in name:
        return "decode_vector"
    return ""


def summarize(run_dir: str, workload: str, over: dict, kernel: str, command: str,
              out_dir: str) -> str:
    """Write profiles/<family>_<key>.txt (and traffic_<key>.json when the
    FETCH_SIZE and WRITE_SIZE runs are there) from a directory holding the
    rocprofv3 output of `command`: trace/ (--kernel-trace --stats),
    FETCH_SIZE/, WRITE_SIZE/ (--pmc, with --reference-copy-mib 1024), and
    optionally one directory per further counter set."""
    from synth import WORKLOADS, workload_algorithmic_bytes, workload_visible_pairs

    w = WORKLOADS[workload].with_(**over)
    key = workload_key(workload, over, kernel)
    stats = _csv_rows(os.path.join(run_dir, "trace"), "kernel_stats.csv")
    mine = [r for r in stats if r.get("Name", "").find("pda::") >= 0]
    fam_rows = [r for r in mine if _kernel_family(r["Name"])]
    if not fam_rows:
        raise RuntimeError(f"no pda kernel in {run_dir}/trace")
    main_row = max(fam_rows, key=lambda r: float(r["TotalDurationNs"]))
    family = _kernel_family(main_row["Name"])
    avg_ns = float(main_row["AverageNs"])
    nbytes = workload_algorithmic_bytes(w)
    lines = [f"# {family} kernel, workload {key}", "",
             "Commands (run from the repository root on one MI355X, TMPDIR=/tmp; OUT = the",
             "output directory):",
             f"  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- {command}",
             f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/FETCH_SIZE -o run -- "
             f"{command} --steps 10 --warmup 2 --reference-copy-mib 1024",
             "  rocprofv3 --pmc WRITE_SIZE (same as above, -d OUT/WRITE_SIZE)",
             "  python bench.py --summarize OUT " + command.split("--no-cpu ", 1)[1], "",
             "Kernel trace (rocprofv3 --stats, rows of this library):",
             "  name | calls | average ns | min ns | max ns"]
    for r in sorted(mine, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"  {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{r['MinNs']} | {r['MaxNs']}")
    lines.append("")
    traffic = None
    if family == "prefill_mfma":
        flops = 4 * w.head_dim * workload_visible_pairs(w)
        tf = flops / (avg_ns * 1e-9) / 1e12
        lines.append(f"Algorithmic work per launch: {flops} flops (4 * D per visible (row, key))")
        lines.append(f"{family} kernel average duration: {avg_ns / 1e3:.2f} us -> {tf:.1f} TFLOP/s "
                     f"= {tf / 2500.0:.3f} of 2.5 PFLOP/s")
    else:
        gbs = nbytes / (avg_ns * 1e-9) / 1e9
        lines.append(f"Algorithmic bytes per launch (K+V visible keys once, q, out): {nbytes}")
        lines.append(f"{family} kernel average duration: {avg_ns / 1e3:.2f} us -> {gbs:.1f} GB/s "
                     f"= {gbs / HBM_PEAK_GBS:.3f} of 8 TB/s")
    # HBM counters
    fetch = _counter_means(os.path.join(run_dir, "FETCH_SIZE"), "FETCH_SIZE")
    write = _counter_means(os.path.join(run_dir, "WRITE_SIZE"), "WRITE_SIZE")
    if fetch and write and family in fetch[0] and family in write[0]:
        (fk, fref), (wk, wref) = (fetch[0][family], fetch[1]), (write[0][family], write[1])
        fscale = (1 << 30) / (fref * 1024.0)
        wscale = (1 << 30) / (wref * 1024.0)
        hbm = int(fk[0] * 1024 * fscale + wk[0] * 1024 * wscale)
        base = nbytes
        lines += ["", "HBM counters (rocprofv3 --pmc, KiB per dispatch, averaged over "
                      f"{fk[1]} dispatches of the kernel):",
                  f"  kernel FETCH_SIZE = {fk[0]:.1f} KiB, WRITE_SIZE = {wk[0]:.1f} KiB",
                  f"  reference plain copy of 1 GiB: FETCH_SIZE = {fref:.1f} KiB, "
                  f"WRITE_SIZE = {wref:.1f} KiB",
                  f"  calibration: bytes = FETCH_SIZE x 1024 x {fscale:.4f} + WRITE_SIZE x 1024 "
                  f"x {wscale:.4f}",
                  f"  HBM bytes per launch = {hbm} ({hbm / base:.4f} x algorithmic)"]
        traffic = {"workload": key, "kernel": family, "hbm_bytes_per_launch": hbm,
                   "algorithmic_bytes": base, "fetch_kib": round(fk[0], 1),
                   "write_kib": round(wk[0], 1), "fetch_scale": round(fscale, 4),
                   "write_scale": round(wscale, 4),
                   "kernel_source_hash": kernel_source_hash(family),
                   "source": f"{family}_{key}.txt"}
    # further counter sets: every directory other than the three above
    extra = []
    for d in sorted(os.listdir(run_dir)):
        if d in ("trace", "FETCH_SIZE", "WRITE_SIZE") or not os.path.isdir(os.path.join(run_dir, d)):
            continue
        means = _all_counter_means(os.path.join(run_dir, d), family)
        if means:
            extra.append(f"  {d}: " + ", ".join(f"{k} = {v:.4g}" for k, v in sorted(means.items())))
    if extra:
        lines += ["", "Other counters (rocprofv3 --pmc <set> with the first command's arguments "
                      "and --steps 10 --warmup 2; mean per dispatch of the kernel):"] + extra
    lines += ["", f"kernel_source_hash: {kernel_source_hash(family)}", ""]
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, f"{family}_{key}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    if traffic is not None:
        with open(os.path.join(out_dir, f"traffic_{key}.json"), "w") as f:
            json.dump(traffic, f, indent=1)
            f.write("\n")
    return path


def _counter_means(run_dir: str, counter: str):
    """({family: (mean KiB per dispatch, dispatches)}, reference copy value)
    from one --pmc run, or None. The reference copy is the largest value of
    the counter among the runtime's buffer-copy kernels (the 1 GiB copy that
    --reference-copy-mib runs is the largest of them)."""
    rows = _csv_rows(run_dir, "counter_collection.csv")
    if not rows:
        return None
    per, ref = {}, 0.0
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name, v = r.get("Kernel_Name", ""), float(r.get("Counter_Value", 0.0))
        fam = _kernel_family(name)
        if fam:
            per.setdefault(fam, []).append(v)
        elif "copyBuffer" in name:  # the runtime's device-to-device copy (torch copy_)
            ref = max(ref, v)
    if not per or ref <= 0:
        return None
    return {k: (sum(v) / len(v), len(v)) for k, v in per.items()}, ref


def _all_counter_means(run_dir: str, family: str) -> dict:
    rows = _csv_rows(run_dir, "counter_collection.csv")
    acc = {}
    for r in rows:
        if _kernel_family(r.get("Kernel_Name", "")) != family:
            continue
        acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


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
    ap.add_argument("--no-cells", action="store_true", help="skip the lines and extra cells")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cell", default=None,
                    help="measure one extra workload (line:i, decode:i, vector:i, prefill:i, "
                         "writer:i or probe:0) and print its record; the full run measures each "
                         "this way, in a process of its own")
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="write the profiles/ summary of the rocprofv3 output in DIR for the "
                         "workload given by --workload / --batch / --window / --splits / "
                         "--kernel (no GPU needed)")
    args = ap.parse_args(argv)
    over = {k: v for k, v in (("batch", args.batch), ("window", args.window),
                              ("num_splits", args.splits)) if v is not None}
    if args.summarize:
        cmd = "python -u bench.py --no-cells --no-cpu --workload " + args.workload + "".join(
            f" --{k.replace('num_splits', 'splits')} {v}" for k, v in sorted(over.items()))
        if args.kernel != "auto":
            cmd += f" --kernel {args.kernel}"
        cmd += f" --steps {args.steps} --warmup {args.warmup}"
        print(summarize(args.summarize, args.workload, over, args.kernel, cmd,
                        os.path.join(ROOT, "profiles")))
        return 0
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
    if over:
        w = w.with_(**over)
    case = make_case(w, device=device)
    m = measure(case, args.steps, args.warmup, w.num_splits, device, args.kernel)
    gbs = m["bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    key = workload_key(args.workload, over, args.kernel)
    rec = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": key, "batch": w.batch, "seq_len": w.seq_len,
                   "q_len": w.q_len, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "kv_dtype": w.kv_dtype, "window": w.window,
                   "num_splits": m["splits"],
                   "us_per_call": round(m["ms_per_step"] * 1e3, 2),
                   "eager_us_per_call": round(m["ms_eager"] * 1e3, 2),
                   "per_call_us": m["per_call_us"],
                   "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes": m["bytes"], "input_replicas": m["replicas"],
                   "settle_steps": m["settle"], "kernel": args.kernel,
                   "accumulate": "fp32"},
        "roofline": roofline_record(m, args.kernel, key),
    }
    gpu_us = {key: rec["config"]["us_per_call"]}
    if not args.no_cells:
        # Each workload in a fresh process: a KV pool allocated after other
        # large buffers were freed measured up to 4.5% slower (D=256, 32 x
        # 16384: 369 against 354 us per decode), while a serving process
        # allocates its pool once.
        del case
        torch.cuda.empty_cache()
        probe = run_cell("probe:0", args.steps, args.kernel)
        print(json.dumps({"probe": probe}), file=sys.stderr, flush=True)
        roof = probe["GB_s"]
        rec["hbm_read_roof"] = probe
        rec["config"]["frac_of_measured_roof"] = round(gbs / roof, 4)
        rec["roofline"]["measured_roof_GB_s"] = roof
        rec["roofline"]["frac_of_measured_roof"] = round(rec["roofline"]["achieved"] / roof, 4)
        for kind, n, field in (("line", len(LINES), "lines"), ("decode", len(CELLS), "cells"),
                               ("vector", len(VECTOR_CELLS), "vector_cells"),
                               ("prefill", len(PREFILL_CELLS), "prefill_cells"),
                               ("writer", len(WRITER_CELLS), "writer_cells")):
            rec[field] = []
            for i in range(n):
                r = run_cell(f"{kind}:{i}", args.steps, args.kernel)
                if kind in ("line", "decode", "vector"):
                    r = _with_roof(r, roof)
                    gpu_us[r["workload"]] = r["us_per_call"]
                rec[field].append(r)
                print(json.dumps({f"{kind}_cell": r}), file=sys.stderr, flush=True)
        case = None
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(device, gpu_us, case)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
