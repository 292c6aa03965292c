#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Headline step (``value``): one continuous-batching decode iteration of one
70B-shaped attention layer (128 sequences, 64 query / 8 KV heads, head dim
128, bf16, 16-token blocks, lognormal contexts of mean 1500):

  a1  host: libpa grows every sequence by one token (one block taken at each
      block boundary) and writes the new slots and context lengths into one
      pinned buffer (a ring of them, so this host work overlaps the previous
      steps' kernels); the block tables stay on the device;
  a2  one pa_stage_decode_append launch moves that buffer to the device,
      scatters the new tokens' K/V into their paged slots and enters each
      block a token opens in its sequence's device block table;
  a3  pa_decode: split-K paged attention (+ merge of multi-chunk contexts).

``value`` is the step's algorithmic HBM bytes (decode: every K/V byte of
every context once per KV head, Q, output, block-table entries and context
lengths; cache write: new K/V read and written) divided by the wall time of
the timed steps.  ``roofline`` is the decode kernel alone: the same
algorithmic decode bytes per launch over its mean duration from HIP events
on its own stream (libpa's pa_timing_* facility).

Secondary legs (skipped with --decode-only):
  ``decode_step_fused`` the same step as one pa_decode_step launch (a2 and
                 a3 in one kernel: the staging copy, the new tokens' K/V,
                 the table entries and the attention);
  ``mixed``      the chunked-prefill iteration: a 32768-token prompt as 64
                 causal 512-token slices, each iteration also decoding one
                 token for 127 sequences; tokens/s per layer over the 64
                 iterations with the slice's prefill on a second stream
                 beside the decode (``one_stream``: both on one stream), and
                 the prefill kernel's bf16 MFMA TFLOP/s on the algorithmic
                 causal flop count, timed in the one-stream pass;
  ``fp8_decode`` 64 sequences at context 8192 with an e4m3fn cache;
  ``fp8_prefill`` the 64 slices of the 32768-token prompt with an e4m3fn
                 cache: prefill kernel TFLOP/s;
  ``prefix_sharing`` 128 sequences behind one shared 1024-token prompt:
                 blocks held and decode kernel time: shared by naming the
                 owner, private, and found from the token ids (detected);
  ``prefix_trace`` 1000 iterations of requests behind 8 shared system
                 prompts, with and without their token ids: prefill tokens
                 computed, prompt tokens found shared, output tokens/s;
  ``preemption`` short prompts, long outputs, a small pool, running caps
                 32..256: preemptions, recomputed prefill, output tokens/s;
  ``block_size`` the decode-70b contexts with 8/16/32-token blocks: decode
                 kernel GB/s, and the trace's fragmentation per block size;
  ``trace``      1000 continuous-batching iterations (libpa scheduler +
                 kernels) with Poisson arrivals: tokens/s per layer and KV
                 fragmentation.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 5] [--no-cpu-baseline]
                       [--decode-only] [--step-launch separate|fused|fused-device]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
H_Q, H_KV, D, BLOCK = 64, 8, 128, 16
DECODE_EXTRA_STEPS = 4    # untimed steps after the timed ones (other kernels' timing)
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--overlap", action="store_true",
                    help="decode step: the append launch on a second stream")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--step-launch", choices=["fused", "fused-device", "separate"],
                    default="separate",
                    help="decode step as one pa_decode_step launch that also stages the "
                         "metadata (fused), as pa_stage + pa_decode_step reading it from the "
                         "device (fused-device), or as pa_stage_decode_append + pa_decode "
                         "(separate)")
    ap.add_argument("--stage-ahead", action="store_true",
                    help="decode step: stage the metadata on a side stream ahead of the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode step (no mixed chunked-prefill or fp8 legs)")
    ap.add_argument("--cpu-sample-seqs", type=int, default=32)
    ap.add_argument("--mixed-only", action="store_true",
                    help="only the mixed chunked-prefill leg (printed as one JSON line)")
    ap.add_argument("--pmc-prefill-summary", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="HBM traffic of the mixed leg's prefill slices from rocprofv3 runs")
    ap.add_argument("--trace-prefill-summary", metavar="TRACE_DIR",
                    help="no GPU work: the mixed leg's prefill roofline from a rocprofv3 "
                         "--kernel-trace run of bench.py --mixed-only")
    ap.add_argument("--sq-prefill-summary", nargs="+", metavar="PMC_DIR",
                    help="no GPU work: matrix-core / vector counters of the mixed leg's "
                         "prefill slices from rocprofv3 --pmc runs")
    ap.add_argument("--modes-only", action="store_true",
                    help="only the four-schedule serving comparison (printed as one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain streaming kernel of known size (HBM counter calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR",
                                                       "CAL_WRITE_DIR"),
                    help="no GPU work: turn rocprofv3 --pmc CSV runs into per-launch HBM bytes")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("pa_decode.hip", "pa_decode_body.h", "pa_device.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_cache_host_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def prefill_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("pa_prefill.hip", "pa_prefill_body.h", "pa_device.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_cache_host_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def decode_bytes(lens: np.ndarray) -> int:
    """Algorithmic HBM bytes of one decode launch (bf16)."""
    lens = lens.astype(np.int64)
    S = len(lens)
    kv = int(lens.sum()) * H_KV * D * 2 * 2
    qo = S * H_Q * D * (2 + 2)
    tables = int((-(-lens // BLOCK)).sum()) * 4 + 4 * S
    return kv + qo + tables


def cache_write_bytes(n_tok: int) -> int:
    return n_tok * H_KV * D * 2 * 2 * 2 + 4 * n_tok


def decode_pmc_from_profile(digest: str):
    """The committed PMC summary of the decode kernel, if it was taken on the
    current kernel source (else None)."""
    p = os.path.join(PROFILE_DIR, "decode_70b_128seq_pmc.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_digest") != digest:
        return None
    return d


def prefill_pmc_from_profile():
    """The committed PMC summary of the mixed leg's 64 prefill calls, if it
    was taken on the current prefill source (else None)."""
    try:
        d = json.load(open(os.path.join(PROFILE_DIR, "prefill_32k_slices_pmc.json")))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_digest") != prefill_source_digest():
        return None
    return d


def mixed_warmup_slices(warmup: int) -> int:
    """Prefill slices of the mixed leg's warm passes for --warmup W."""
    return min(64, max(warmup, 1) * 4)


def _host_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_workers() -> int:
    """Worker processes for the parallel oracle runs: the cores this
    process may use, at most 16 (one GPU's share of a box's cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


_ORACLE_JOB = {}


def _oracle_job(part):
    """One worker's share of an oracle call (set up in _ORACLE_JOB before the
    workers are forked), on one BLAS thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return _ORACLE_JOB["fn"](part)


def _time_oracle(fn, parts, seconds: float):
    """Mean wall time of fn over all parts in three configurations: one
    thread; one process with the BLAS default threads; the parts spread over
    worker processes of one BLAS thread each.  Returns {config: (seconds,
    cores)}.  Runs before the GPU is initialised (the workers are forked)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_info, threadpool_limits

    def run(call, budget):
        t0 = time.perf_counter()
        reps = 0
        while True:
            call()
            reps += 1
            if time.perf_counter() - t0 > budget:
                return (time.perf_counter() - t0) / reps, reps

    out = {}
    with threadpool_limits(limits=1):
        out["1 thread"] = run(lambda: [fn(p) for p in parts], seconds / 3)[0], 1
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    out[f"{blas} BLAS threads"] = run(lambda: [fn(p) for p in parts], seconds / 3)[0], blas
    n = min(_cpu_workers(), len(parts))
    _ORACLE_JOB["fn"] = fn
    with mp.get_context("fork").Pool(n) as pool:
        pool.map(_oracle_job, parts)           # workers started and warm
        out[f"{n} processes x 1 thread"] = \
            run(lambda: pool.map(_oracle_job, parts), seconds / 3)[0], n
    return out


def _best(configs: dict, work: float, scale: float):
    """(value, cores, config name, all) with value = work / time / scale."""
    allv = {k: round(work / t / scale, 3) for k, (t, _) in configs.items()}
    name = max(allv, key=allv.get)
    return allv[name], configs[name][1], name, allv


def cpu_baseline(n_seqs: int):
    """The oracle (numpy, fp64) on the first n_seqs sequences of the same
    workload: gather through the block tables + softmax attention, timed
    without data generation and cache construction, in its best
    configuration of the host's cores (one thread, BLAS threads, or the
    sequences spread over worker processes)."""
    import workloads
    from oracle import allocator as oa
    from oracle import attention as oat
    from oracle import cache as oc
    from oracle import codecs

    lengths, _, _ = workloads.decode_70b_layout()
    L = lengths[:n_seqs]
    rng = np.random.default_rng(12)
    nb = workloads.blocks_needed(L) + 8
    pool = oa.BlockPool(nb, BLOCK, rng.permutation(nb).tolist())
    kc, vc = oc.new_cache(nb, H_KV, BLOCK, D, "bf16")
    for s, l in enumerate(L.tolist()):
        pool.seq_create(s, l)
        k = workloads.normal_raw(rng, (l, H_KV, D), "bf16")
        v = workloads.normal_raw(rng, (l, H_KV, D), "bf16")
        oc.cache_write(kc, vc, k, v, pool.slots(s, 0, l), "bf16", "bf16")
    q = codecs.decode(workloads.normal_raw(rng, (len(L), H_Q, D), "bf16"), "bf16")
    tables, lens = pool.pack(range(len(L)), max(-(-int(l) // BLOCK) for l in L))
    tables = np.asarray(tables)
    lens = np.asarray(lens)
    sm = float(np.float32(1.0) / np.float32(math.sqrt(D)))
    parts = [np.arange(i, len(L), _cpu_workers()) for i in range(min(_cpu_workers(), len(L)))]

    def fn(idx):
        return oat.decode(q[idx], kc, vc, tables[idx], lens[idx], H_KV, sm, "bf16")

    configs = _time_oracle(fn, parts, 24.0)
    value, cores, name, allv = _best(configs, decode_bytes(lens), 1e9)
    return {"value": value, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "config": name, "all_configs_gb_s": allv,
            "sample": f"first {len(L)} of the 128 sequences ({int(L.sum())} context tokens), "
                      f"one decode launch's gather + fp64 attention, sequences split "
                      f"round-robin over workers; host {_host_model()}, "
                      f"{len(os.sched_getaffinity(0))} cores visible"}


CAL_BYTES = 1 << 30


def calibrate_copy():
    """A plain streaming kernel of known size for the HBM counter
    calibration: out = -in over 1 GiB of fp32 (reads 1 GiB, writes 1 GiB)."""
    import torch
    n = CAL_BYTES // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.empty(n, dtype=torch.float32, device="cuda")
    a.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "fp32 negation kernel", "bytes_read": CAL_BYTES,
                      "bytes_written": CAL_BYTES, "launches": 3}))


def _pmc_rows(d: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def _pmc_mean(rows, key: str) -> tuple[float, int]:
    vals = [v for name, v in rows if key in name]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel named *{key}*: "
                         f"{sorted(set(n for n, _ in rows))[:20]}")
    return sum(vals) / len(vals), len(vals)


def pmc_summary(fetch_dir: str, write_dir: str, cal_fetch_dir: str, cal_write_dir: str,
                warmup: int, steps: int):
    """HBM traffic of one decode launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (KiB per dispatch) of ``bench.py --decode-only --steps K --warmup W``,
    each scaled by what the same counter reads for the calibration kernel of
    known size, beside the algorithmic bytes of the same launches (launch i
    of that run attends contexts of the workload's lengths + i tokens)."""
    import workloads

    f_dec, n_f = _pmc_mean(_pmc_rows(fetch_dir, "FETCH_SIZE"), "decode_kernel<pa::BF16, 128, 16>")
    w_dec, n_w = _pmc_mean(_pmc_rows(write_dir, "WRITE_SIZE"), "decode_kernel<pa::BF16, 128, 16>")
    f_cal, _ = _pmc_mean(_pmc_rows(cal_fetch_dir, "FETCH_SIZE"), "neg")
    w_cal, _ = _pmc_mean(_pmc_rows(cal_write_dir, "WRITE_SIZE"), "neg")
    f_scale = CAL_BYTES / (f_cal * 1024.0)
    w_scale = CAL_BYTES / (w_cal * 1024.0)
    lengths, _, _ = workloads.decode_70b_layout()
    n_launch = warmup + steps + DECODE_EXTRA_STEPS
    if n_f != n_launch or n_w != n_launch:
        raise SystemExit(f"expected {n_launch} decode dispatches (--warmup {warmup} --steps "
                         f"{steps}), got {n_f} / {n_w}")
    alg = float(np.mean([decode_bytes(lengths + i) for i in range(n_launch)]))
    out = {
        "kernel": "decode_kernel<BF16,128,16>",
        "workload": f"decode-70b-shaped, 128 seqs: bench.py --decode-only --warmup {warmup} "
                    f"--steps {steps} (every decode launch of the run)",
        "kernel_source_digest": kernel_source_digest(),
        "fetch_kib_per_launch_raw": round(f_dec, 1), "fetch_dispatches": n_f,
        "write_kib_per_launch_raw": round(w_dec, 1), "write_dispatches": n_w,
        "calibration": {"kernel": "fp32 negation, 1 GiB in / 1 GiB out",
                        "fetch_kib_raw": round(f_cal, 1), "write_kib_raw": round(w_cal, 1),
                        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "hbm_read_bytes_per_launch": int(f_dec * 1024 * f_scale),
        "hbm_write_bytes_per_launch": int(w_dec * 1024 * w_scale),
        "algorithmic_bytes_per_launch": int(alg),
    }
    out["hbm_bytes_per_launch"] = out["hbm_read_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
    out["traffic_ratio"] = round(out["hbm_bytes_per_launch"] / alg, 4)
    print(json.dumps(out, indent=1))


def _pmc_seq(d: str, counter: str, key: str):
    """(dispatch id, value) of one counter for the dispatches of kernels named
    *key*, in dispatch order."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter and key in r["Kernel_Name"]:
                rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    rows.sort()
    return rows


def _window(prefill, merge, first: int, n: int):
    """Sum of the prefill dispatches [first, first + n) and of the merge
    dispatches that follow one of them (before the next prefill dispatch)."""
    ids = [i for i, _ in prefill]
    lo = ids[first]
    hi = ids[first + n] if first + n < len(ids) else float("inf")
    tot = sum(v for _, v in prefill[first:first + n])
    tot += sum(v for i, v in merge if lo < i < hi)
    return tot


def pmc_prefill_summary(fetch_dir: str, write_dir: str, cal_fetch_dir: str, cal_write_dir: str,
                        warmup: int):
    """HBM traffic of the mixed leg's 64 prefill calls (one-stream pass of
    ``bench.py --mixed-only --warmup W``: the prefill launches are, in order,
    the warm pass's slices, the 64 slices of the one-stream pass, then those
    of the two-stream passes), prefill kernel and merge kernel together,
    against their algorithmic bytes: the K/V of the prefix and the slice
    (read once), Q and the output."""
    key, mkey = "prefill_kernel<pa::BF16, 128, 16>", "prefill_merge_kernel<128>"
    f, w = _pmc_seq(fetch_dir, "FETCH_SIZE", key), _pmc_seq(write_dir, "WRITE_SIZE", key)
    fm, wm = _pmc_seq(fetch_dir, "FETCH_SIZE", mkey), _pmc_seq(write_dir, "WRITE_SIZE", mkey)
    first = mixed_warmup_slices(warmup)
    if len(f) < first + 64 or len(w) < first + 64:
        raise SystemExit(f"expected >= {first + 64} {key} dispatches, got {len(f)} / {len(w)}")
    f_cal, _ = _pmc_mean(_pmc_rows(cal_fetch_dir, "FETCH_SIZE"), "neg")
    w_cal, _ = _pmc_mean(_pmc_rows(cal_write_dir, "WRITE_SIZE"), "neg")
    f_scale = CAL_BYTES / (f_cal * 1024.0)
    w_scale = CAL_BYTES / (w_cal * 1024.0)
    C = 512
    alg_read = sum((C * c + C) * H_KV * D * 2 * 2 + C * H_Q * D * 2 for c in range(64))
    alg_write = 64 * C * H_Q * D * 2
    read = _window(f, fm, first, 64) * 1024 * f_scale
    write = _window(w, wm, first, 64) * 1024 * w_scale
    read_k = sum(v for _, v in f[first:first + 64]) * 1024 * f_scale
    write_k = sum(v for _, v in w[first:first + 64]) * 1024 * w_scale
    print(json.dumps({
        "kernel": "prefill_kernel<BF16,128,16> + prefill_merge_kernel<128>",
        "workload": f"mixed leg, 64 causal 512-token slices of a 32768-token prompt, one "
                    f"stream (bench.py --mixed-only --warmup {warmup}: prefill dispatches "
                    f"{first}..{first + 63} and the merges that follow them)",
        "calibration": {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "hbm_read_bytes": int(read), "algorithmic_read_bytes": alg_read,
        "read_ratio": round(read / alg_read, 3),
        "hbm_write_bytes": int(write), "algorithmic_write_bytes": alg_write,
        "write_ratio": round(write / alg_write, 3),
        "hbm_bytes": int(read + write),
        "prefill_kernel_only": {"hbm_read_bytes": int(read_k), "hbm_write_bytes": int(write_k)},
        "split_partials_note": "slices whose key range is split write partial states (fp16 "
                               "normalised outputs + fp32 (m, l)) that the merge kernel reads "
                               "back; the algorithmic count leaves them out",
        "kernel_source_digest": prefill_source_digest(),
    }, indent=1))


def _trace_rows(d: str):
    """(dispatch id, kernel name, duration ns) of a rocprofv3 --kernel-trace
    CSV run."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                         int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    return rows


def trace_prefill_summary(trace_dir: str, warmup: int):
    """The prefill roofline of the mixed leg recomputed from a rocprofv3
    --kernel-trace run of ``bench.py --mixed-only --warmup W``: durations of
    the one-stream pass's 64 prefill dispatches and of the merge dispatches
    that follow them, against the algorithmic causal flops."""
    rows = _trace_rows(trace_dir)
    pf = [(i, t) for i, n, t in rows if "prefill_kernel<pa::BF16, 128, 16>" in n]
    mg = [(i, t) for i, n, t in rows if "prefill_merge_kernel<128>" in n]
    first = mixed_warmup_slices(warmup)
    if len(pf) < first + 64:
        raise SystemExit(f"expected >= {first + 64} prefill dispatches, got {len(pf)}")
    t_pf = sum(t for _, t in pf[first:first + 64]) / 1e3
    t_all = _window(pf, mg, first, 64) / 1e3
    C = 512
    flops = 4 * D * H_Q * sum(C * (c * C) + C * (C + 1) // 2 for c in range(64))
    print(json.dumps({
        "workload": f"mixed leg, one-stream pass (bench.py --mixed-only --warmup {warmup}: "
                    f"prefill dispatches {first}..{first + 63} and their merges)",
        "prefill_kernel_us_total": round(t_pf, 1), "with_merge_us_total": round(t_all, 1),
        "algorithmic_flops": flops,
        "achieved_tflops": round(flops / t_all / 1e6, 1),
        "frac_of_bf16_peak": round(flops / t_all / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernel_only_tflops": round(flops / t_pf / 1e6, 1),
        "kernel_source_digest": prefill_source_digest(),
    }, indent=1))


def sq_prefill_summary(dirs, warmup: int):
    """Matrix-core and vector-unit counters of the mixed leg's 64 one-stream
    prefill dispatches (rocprofv3 --pmc runs of ``bench.py --mixed-only``,
    several counter passes), summed over the window.  SQ counters are
    aggregated over the 32 shader engines (8 XCDs x 4), GRBM_GUI_ACTIVE over
    the 8 XCDs; a busy fraction is per SIMD (256 CUs x 4 SIMDs)."""
    key = "prefill_kernel<pa::BF16, 128, 16>"
    first = mixed_warmup_slices(warmup)
    tot = {}
    import csv
    import glob
    for d in dirs:
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if key in r["Kernel_Name"]:
                    rows.setdefault(r["Counter_Name"], []).append(
                        (int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        for c, v in rows.items():
            v.sort()
            if len(v) < first + 64:
                raise SystemExit(f"{c}: {len(v)} dispatches")
            tot[c] = sum(x for _, x in v[first:first + 64])
    out = {"workload": f"mixed leg, one-stream pass, prefill dispatches {first}..{first + 63}",
           "counters": {k: tot[k] for k in sorted(tot)}, "kernel_source_digest":
           prefill_source_digest()}
    simds = 256 * 4
    if "GRBM_GUI_ACTIVE" in tot:
        cyc = tot["GRBM_GUI_ACTIVE"] / 8
        out["gpu_cycles"] = cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in tot:
            out["mfma_busy_frac"] = round(tot["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cyc, 4)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in tot and "SQ_VALU_MFMA_COEXEC_CYCLES" in tot:
        out["valu_coexec_share_of_mfma_busy"] = round(
            tot["SQ_VALU_MFMA_COEXEC_CYCLES"] / tot["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
    if "SQ_INSTS_MFMA" in tot and "SQ_INSTS_VALU" in tot:
        out["valu_insts_per_mfma"] = round((tot["SQ_INSTS_VALU"] - tot["SQ_INSTS_MFMA"]) /
                                           tot["SQ_INSTS_MFMA"], 3)
    if "SQ_INSTS_MFMA" in tot and "SQ_INSTS_VALU_TRANS_F32" in tot:
        out["exp_per_mfma"] = round(tot["SQ_INSTS_VALU_TRANS_F32"] / tot["SQ_INSTS_MFMA"], 3)
    if "SQ_INSTS_MFMA" in tot and "SQ_INSTS_LDS" in tot:
        out["lds_insts_per_mfma"] = round(tot["SQ_INSTS_LDS"] / tot["SQ_INSTS_MFMA"], 3)
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in tot and "SQ_INSTS_VALU_MFMA_MOPS_F16" in tot:
        C = 512
        flops = 4 * D * H_Q * sum(C * (c * C) + C * (C + 1) // 2 for c in range(64))
        # one MOP = 256 multiply-adds = 512 flops (a 32x32x16 MFMA counts 64)
        mops = tot["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + tot["SQ_INSTS_VALU_MFMA_MOPS_F16"]
        out["mfma_flops_counted"] = mops * 512
        out["mfma_flops_over_algorithmic"] = round(mops * 512 / flops, 4)
    print(json.dumps(out, indent=1))


def _fill_random(kv, slots: np.ndarray, gen, dev, chunk: int = 1 << 16):
    """Untimed set-up: write N(0,1) bf16 K/V for the given slots through
    pa_cache_write."""
    import torch
    for a in range(0, len(slots), chunk):
        n = min(chunk, len(slots) - a)
        kk = torch.randn((n, H_KV, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vv = torch.randn((n, H_KV, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        kv.write(kk, vv, torch.from_numpy(np.ascontiguousarray(slots[a:a + n], dtype=np.int32)).to(dev))


def _settle():
    """Before a timed loop: collect, then move every live object to the
    permanent generation, so that no full collection over the interpreter's
    (torch-sized) heap pauses the host thread inside the loop."""
    gc.collect()
    gc.freeze()


def _timings(pa, names):
    out = {}
    for name in names:
        st, cnt, mean_us, tot_us = pa.pa_timing_query(name)
        pa.check(st)
        out[name] = (cnt, mean_us, tot_us)
    return out


def decode_leg(args, dev, launch_mode: str | None = None):
    """The headline step: one decode iteration of the decode-70b layer
    (``launch_mode`` overrides --step-launch)."""
    import torch

    import workloads
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import PagedKV, decode_workspace, sm_scale_for

    K, W = args.steps, args.warmup
    lengths, num_blocks, free_order = workloads.decode_70b_layout()
    S = len(lengths)
    seqs = np.arange(S, dtype=np.int64)
    EXTRA, TIME_EVERY = DECODE_EXTRA_STEPS, 4
    max_ctx = int(lengths.max()) + W + K + EXTRA
    MB = -(-max_ctx // BLOCK)
    # the workload's pool (10% free) covers the growth of a default run; a
    # longer run appends fresh block ids behind the shuffled ones
    need = int(np.sum(-(-(lengths - 1 + W + K + EXTRA) // BLOCK)))
    if need > num_blocks:
        free_order = np.concatenate([free_order, np.arange(num_blocks, need, dtype=np.int32)])
        num_blocks = need

    # -- set-up (untimed): pool, contexts of L-1 tokens already cached
    kv = PagedKV(num_blocks, H_KV, D, "bf16", dev, free_order)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    fill_slots = []
    for s in range(S):
        pa.check(kv.create(s, int(lengths[s]) - 1))
        if lengths[s] > 1:
            fill_slots.append(kv.slots(s, 0, int(lengths[s]) - 1))
    _fill_random(kv, np.concatenate(fill_slots), gen, dev)
    R = 4
    k_ring = [torch.randn((S, H_KV, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    v_ring = [torch.randn((S, H_KV, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    q_ring = [torch.randn((S, H_Q, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    out = torch.empty((S, H_Q, D), dtype=torch.bfloat16, device=dev)
    ws = decode_workspace(S, H_Q, H_KV, D, max_ctx, dev)
    sm = sm_scale_for(D)

    # The batch's block tables live on the device: packed once at set-up,
    # then kept up to date by the launch that scatters each step's new
    # tokens (pa_stage_decode_append enters a token's block in its row when
    # the token opens one).  A ring of NBUF pinned host buffers, each with a
    # device twin, holds the steps' slots and context lengths; that same
    # launch carries a step's buffer (no copy engine, no cross-engine wait).
    # The host may refill a buffer once the launch that read it has run: one
    # event per GROUP steps tells it so (an event record costs the stream a
    # few microseconds, so not one per step).
    NBUF, GROUP = 8, 4
    n_meta = 2 * S
    st, tab0, lens_host = pa.pa_pack_batch(kv.pool, seqs, MB)
    pa.check(st)
    d_tab = torch.from_numpy(tab0).to(dev)
    lens_host = lens_host.copy()
    host_buf = [torch.empty(n_meta, dtype=torch.int32, pin_memory=True) for _ in range(NBUF)]
    dev_buf = [torch.empty(n_meta, dtype=torch.int32, device=dev) for _ in range(NBUF)]
    views = []
    for X in range(NBUF):
        h, d_ = host_buf[X].numpy(), dev_buf[X]
        views.append((h[:S].reshape(S, 1), h[S:2 * S], d_[S:2 * S]))
    compute = torch.cuda.Stream(device=dev)
    # With --overlap the append launch runs on a stream of its own, so that
    # step i+1's launch overlaps step i's decode: it writes only slots past
    # step i's contexts and table entries step i does not read (or rewrites
    # one with its own value), and the decode of step i+1 waits for it.
    aux = torch.cuda.Stream(device=dev) if getattr(args, "overlap", False) else compute
    # With --stage-ahead only the 1 KiB metadata copy runs on a side stream
    # (pa_stage, one work-group), and pa_decode_append on the compute stream
    # reads the staged slots and lengths from device memory.
    ahead = torch.cuda.Stream(device=dev) if getattr(args, "stage_ahead", False) else None
    # --step-launch fused: pa_decode_step stages the buffer, appends the new
    # tokens, enters their blocks and attends, all in one launch
    if launch_mode is None:
        launch_mode = getattr(args, "step_launch", "separate")
    fused = launch_mode in ("fused", "fused-device")
    if fused and (ahead is not None or aux is not compute):
        raise SystemExit("--step-launch fused runs on one stream (no --overlap / --stage-ahead)")
    kname = "decode_step" if fused else "decode"
    side = (["stage"] if launch_mode == "fused-device" else []) if fused else ["stage_cache_write"]
    ev_w = [torch.cuda.Event() for _ in range(2)]
    ev_group = [torch.cuda.Event() for _ in range(2)]
    for e in ev_group:
        e.record(compute)
    ctx_lens = []

    def step(i: int, timed: bool):
        X = i % NBUF
        g = i // GROUP
        h_slots, h_lens, d_lens = views[X]
        if i % GROUP == 0:
            # recorded after group g-2, whose steps last used this group's buffers
            ev_group[g % 2].synchronize()
        st, done, _ = pa.pa_batch_append(kv.pool, seqs, 1, h_slots)
        pa.check(st)
        np.add(lens_host, 1, out=lens_host)
        h_lens[:] = lens_host
        lens_np = lens_host
        r = i % R
        if fused:
            if launch_mode == "fused-device":
                pa.check(pa.pa_stage(compute, dev_buf[X], host_buf[X], 4 * n_meta))
            src = host_buf[X] if launch_mode == "fused" else None
            pa.check(pa.pa_decode_step(compute, dev_buf[X], src, 4 * n_meta, 0, 4 * S,
                                       k_ring[r], v_ring[r], out, q_ring[r], kv.k, kv.v, d_tab,
                                       num_blocks, H_KV, max_ctx, sm, 1.0, 1.0, ws))
        elif ahead is not None:
            # the buffer is staged on the side stream as soon as it is packed
            # (during an earlier step's decode); the compute stream then only
            # scatters the new tokens and enters their blocks
            pa.check(pa.pa_stage(ahead, dev_buf[X], host_buf[X], 4 * n_meta))
            ev_w[i % 2].record(ahead)
            compute.wait_event(ev_w[i % 2])
            pa.check(pa.pa_decode_append(compute, dev_buf[X][:S], d_lens, S, k_ring[r], v_ring[r],
                                         kv.k, kv.v, num_blocks, H_KV, D, d_tab, BLOCK))
        else:
            # one launch stages the buffer, scatters the new tokens (whose
            # slots lead the buffer) and enters the blocks they open
            pa.check(pa.pa_stage_decode_append(aux, dev_buf[X], host_buf[X], 4 * n_meta, 0,
                                               4 * S, S, k_ring[r], v_ring[r], kv.k, kv.v,
                                               num_blocks, H_KV, D, d_tab, BLOCK))
        if ahead is None and aux is not compute:
            ev_w[i % 2].record(aux)
            compute.wait_event(ev_w[i % 2])
        if not fused:
            pa.check(pa.pa_decode(compute, out, q_ring[r], kv.k, kv.v, d_tab, d_lens,
                                  num_blocks, H_KV, max_ctx, sm, 1.0, 1.0, ws))
        if timed:
            ctx_lens.append(lens_np.copy())
        if i % GROUP == GROUP - 1:
            ev_group[g % 2].record(compute)

    # Kernel timing: the library attaches a pair of HIP events to a selected
    # kernel's launch on the stream it launches on (here `compute`).  Each
    # timed launch costs the stream a few microseconds, so the timed steps
    # time every TIME_EVERY-th decode launch only; a few more steps time the
    # step's other kernels.  The warm-up steps already carry the timed
    # launches: the first launch with events attached pays a one-time set-up
    # (measured ~0.4 ms), which must not land in the timed window.
    pa.check(pa.pa_timing_enable([kname, "decode_merge"] + side, every=TIME_EVERY))
    # the collector is run and frozen before the warm-up steps, not right
    # before the timed ones: a full collection walks the whole heap and
    # leaves the host's caches cold for the first timed step (measured
    # ~0.25 ms of host time for that step alone)
    _settle()
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    pa.check(pa.pa_timing_enable([kname], every=TIME_EVERY))
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tm = _timings(pa, (kname,))
    assert tm[kname][0] == len(range(0, K, TIME_EVERY)), tm
    pa.check(pa.pa_timing_enable(["decode_merge"] + side))
    for i in range(EXTRA):
        step(W + K + i, False)
    torch.cuda.synchronize()
    tm.update(_timings(pa, ["decode_merge"] + side))
    pa.check(pa.pa_timing_enable(False))
    kv.close()

    dec_bytes = [decode_bytes(l) for l in ctx_lens]
    total_bytes = sum(dec_bytes) + K * cache_write_bytes(S)
    dec_avg_s = tm[kname][1] / 1e6
    # the fused kernel also moves the new tokens' K/V (the cache write's bytes)
    timed_bytes = float(np.mean(dec_bytes[::TIME_EVERY])) + (cache_write_bytes(S) if fused else 0)
    return {
        "value": total_bytes / wall / 1e9,
        "wall": wall,
        "mean_context": float(np.mean([l.mean() for l in ctx_lens])),
        "num_seqs": S, "num_blocks": num_blocks,
        "achieved": timed_bytes / dec_avg_s / 1e9,
        "timed_launches": tm[kname][0],
        "kernel_us": dec_avg_s * 1e6,
        "kernel": "decode_step_kernel<BF16,128>" if fused else "decode_kernel<BF16,128,16>",
        "fused": fused,
        "merge_us": tm["decode_merge"][1],
        "stage_cache_write_us": None if fused else tm["stage_cache_write"][1],
        "bytes_per_launch": int(sum(dec_bytes) / K) + (cache_write_bytes(S) if fused else 0),
    }


def mixed_leg(args, dev):
    """The chunked-prefill mixed batch: a 32768-token prompt as 64 causal
    512-token slices; every iteration also decodes one token for each of 127
    sequences.  One iteration = host append/pack + one pa_cache_write of the
    639 new tokens + pa_prefill_chunk of the slice + pa_decode of the 127
    sequences (on one stream, or the slice on a second stream), or, in the
    fused form, one pa_attend_varlen for both.  Reported as tokens/s per
    layer over the 64 iterations for each form, plus the prefill kernel's
    bf16 MFMA throughput."""
    import torch

    import workloads
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import (PagedKV, decode_workspace, prefill_workspace,
                                                sm_scale_for, varlen_buffers)

    P, C = 32768, 512
    iters = P // C
    dec_len, num_blocks, free_order = workloads.mixed_prefill_layout()
    S = len(dec_len)
    PROMPT = S  # sequence id of the prompt
    dec_seqs = np.arange(S, dtype=np.int64)
    max_dec = int(dec_len.max()) + iters
    MB = -(-max_dec // BLOCK)
    PB = P // BLOCK
    NT = C + S
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    sm = sm_scale_for(D)

    R = 2
    k_ring = [torch.randn((NT, H_KV, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    v_ring = [torch.randn((NT, H_KV, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    q_prompt = torch.randn((P, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    q_dec = [torch.randn((S, H_Q, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    out_p = torch.empty((C, H_Q, D), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((S, H_Q, D), dtype=torch.bfloat16, device=dev)
    ws_d = decode_workspace(S, H_Q, H_KV, D, max_dec, dev)
    ws_p = torch.empty(max(1, max(pa.pa_prefill_workspace_bytes(1, C, H_Q, H_KV, D, (c + 1) * C)
                                  for c in range(iters))), dtype=torch.uint8, device=dev)
    cu = torch.tensor([0, C], dtype=torch.int32, device=dev)

    # a ring of NBUF pinned buffers [slots NT | lens S | prompt 1 | tables S*MB],
    # each with a device twin, staged once per iteration on the compute
    # stream; one event per GROUP iterations frees them for refilling.  The
    # prompt word is the slice's start for pa_prefill_chunk and its context
    # length for pa_attend_varlen, whose seq_lens are then [lens | prompt].
    NBUF, GROUP = 8, 4
    n_meta = NT + S + 1 + S * MB
    host_buf = [torch.empty(n_meta, dtype=torch.int32, pin_memory=True) for _ in range(NBUF)]
    dev_buf = [torch.empty(n_meta, dtype=torch.int32, device=dev) for _ in range(NBUF)]
    views = []
    for X in range(NBUF):
        h, d_ = host_buf[X].numpy(), dev_buf[X]
        o1, o2, o3 = NT, NT + S, NT + S + 1
        views.append((h[:NT], h[o2:o3], h[o1:o2], h[o3:].reshape(S, MB),
                      d_[:NT], d_[o2:o3], d_[o1:o2], d_[o3:].view(S, MB), d_[o1:o3]))
    compute = torch.cuda.Stream(device=dev)
    # In the two-stream pass the prefill slice runs on a stream of its own
    # after the staging launch, beside the decode (the next iteration's
    # staging writes only slots neither kernel of this iteration reads), so
    # that each kernel's tail overlaps the other.  The one-stream pass
    # times the prefill kernel alone for its roofline.
    side_stream = torch.cuda.Stream(device=dev)
    ev_staged = [torch.cuda.Event() for _ in range(2)]
    ev_group = [torch.cuda.Event() for _ in range(2)]
    ev_group_side = [torch.cuda.Event() for _ in range(2)]

    # the fused form: one pa_attend_varlen per iteration over [127 decode rows;
    # the 512-row slice] (queries of both, the same values as the separate
    # forms use, laid out together once here)
    q_mix = torch.empty((iters, NT, H_Q, D), dtype=torch.bfloat16, device=dev)
    for c in range(iters):
        q_mix[c, :S] = q_dec[c % R]
        q_mix[c, S:] = q_prompt[c * C:(c + 1) * C]
    cu_mix = torch.tensor(list(range(S + 1)) + [S + C], dtype=torch.int32, device=dev)
    # two sets (output, counters + workspace): in the two-stream fused form
    # consecutive iterations run on alternate streams and may overlap
    out_mix = [torch.empty((NT, H_Q, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    bufs_mix = [varlen_buffers(S, 1, H_Q, H_KV, D, C, max_dec, P, dev) for _ in range(2)]

    def run_pass(timed: bool, n_iters: int, two_streams: bool, fused: bool = False):
        side = side_stream if two_streams else compute
        # fresh pool: decode contexts of L0-1 tokens cached, prompt blocks
        # allocated at admission (its K/V are written slice by slice)
        kv = PagedKV(num_blocks, H_KV, D, "bf16", dev, free_order)
        fill = []
        for s in range(S):
            pa.check(kv.create(s, int(dec_len[s]) - 1))
            fill.append(kv.slots(s, 0, int(dec_len[s]) - 1))
        _fill_random(kv, np.concatenate(fill), gen, dev)
        pa.check(kv.create(PROMPT, P))
        ptab, _ = kv.pack([PROMPT], PB)
        ptab_dev = torch.from_numpy(ptab).to(dev)
        torch.cuda.synchronize()
        for e in ev_group:
            e.record(compute)
        for e in ev_group_side:
            e.record(side)
        if timed:
            pa.check(pa.pa_timing_enable(["varlen"] if fused else ["prefill", "prefill_merge"]))
        _settle()
        t0 = time.perf_counter()
        for c in range(n_iters):
            X = c % NBUF
            h_sl, h_st, h_len, h_tab, d_sl, d_st, d_len, d_tab, d_seqlens = views[X]
            if c % GROUP == 0:
                ev_group[(c // GROUP) % 2].synchronize()
                ev_group_side[(c // GROUP) % 2].synchronize()
            pa.check(pa.pa_seq_slots(kv.pool, PROMPT, c * C, C, h_sl[:C])[0])
            st, _, _ = pa.pa_batch_append(kv.pool, dec_seqs, 1, h_sl[C:].reshape(S, 1))
            pa.check(st)
            st, _, _ = pa.pa_pack_batch(kv.pool, dec_seqs, MB, h_tab, h_len)
            pa.check(st)
            h_st[0] = (c + 1) * C if fused else c * C
            r = c % R
            # fused, two streams: iteration c stages and attends on stream c % 2
            # (iteration c+1 writes only its new tokens' slots, which iteration
            # c does not read, so the two may overlap)
            st_c = side if (fused and c % 2) else compute
            pa.check(pa.pa_stage_cache_write(st_c, dev_buf[X], host_buf[X], 4 * n_meta, 0, NT,
                                             k_ring[r], v_ring[r], kv.k, kv.v, num_blocks, H_KV,
                                             D, BLOCK))
            if fused:
                b2 = bufs_mix[c % 2]
                pa.check(pa.pa_attend_varlen(st_c, out_mix[c % 2], q_mix[c], cu_mix, d_seqlens, S,
                                             kv.k, kv.v, d_tab, ptab_dev, num_blocks, H_KV, C,
                                             max_dec, (c + 1) * C, sm, 1.0, 1.0, b2[0], b2[1]))
                if c % GROUP == GROUP - 1:
                    ev_group[(c // GROUP) % 2].record(compute)
                    ev_group_side[(c // GROUP) % 2].record(side)
                continue
            if side is not compute:
                ev_staged[c % 2].record(compute)
                side.wait_event(ev_staged[c % 2])
            pa.check(pa.pa_prefill_chunk(side, out_p, q_prompt[c * C:(c + 1) * C], cu,
                                         d_st, kv.k, kv.v, ptab_dev, num_blocks, H_KV, C,
                                         (c + 1) * C, sm, 1.0, 1.0, ws_p))
            pa.check(pa.pa_decode(compute, out_d, q_dec[r], kv.k, kv.v, d_tab,
                                  d_len, num_blocks, H_KV, max_dec, sm, 1.0, 1.0, ws_d))
            if c % GROUP == GROUP - 1:
                ev_group[(c // GROUP) % 2].record(compute)
                ev_group_side[(c // GROUP) % 2].record(side)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        tm = None
        if timed:
            tm = _timings(pa, ("varlen",) if fused else ("prefill", "prefill_merge"))
            pa.check(pa.pa_timing_enable(False))
        kv.close()
        return wall, tm

    # the warm pass carries timed launches too: the first launch with events
    # attached pays a one-time set-up, which must not land in a timed pass
    pa.check(pa.pa_timing_enable(["prefill", "prefill_merge"]))
    run_pass(False, mixed_warmup_slices(args.warmup), False)
    pa.check(pa.pa_timing_enable(False))
    wall1, tm = run_pass(True, iters, False)
    run_pass(False, mixed_warmup_slices(args.warmup), True)
    wall, _ = run_pass(False, iters, True)
    pa.check(pa.pa_timing_enable(["varlen"]))
    run_pass(False, mixed_warmup_slices(args.warmup), False, fused=True)
    pa.check(pa.pa_timing_enable(False))
    wall_f, tm_f = run_pass(True, iters, False, fused=True)
    run_pass(False, mixed_warmup_slices(args.warmup), True, fused=True)
    wall_f2, _ = run_pass(False, iters, True, fused=True)
    pairs = sum(C * (c * C) + C * (C + 1) // 2 for c in range(iters))
    flops = 4 * D * H_Q * pairs
    n_pf, mean_pf, tot_pf = tm["prefill"]
    assert n_pf == iters, tm
    tot_merge = tm["prefill_merge"][2]
    # a pa_prefill_chunk call is the prefill kernel plus, for slices whose
    # key range is split, the merge kernel: the roofline counts both
    achieved = flops / ((tot_pf + tot_merge) / 1e6) / 1e12
    achieved_kernel = flops / (tot_pf / 1e6) / 1e12
    pmc = prefill_pmc_from_profile()
    return {
        "tokens_per_s": iters * NT / wall,
        "ms_per_iteration": wall / iters * 1e3,
        "streams": "prefill beside decode (two streams)",
        "one_stream": {"tokens_per_s": iters * NT / wall1, "ms_per_iteration": wall1 / iters * 1e3},
        "fused": {"tokens_per_s": iters * NT / wall_f, "ms_per_iteration": wall_f / iters * 1e3,
                  "launch": "pa_attend_varlen: decode rows and the slice in one kernel",
                  "kernel_us_mean": round(tm_f["varlen"][1], 1),
                  "kernel_us_total": round(tm_f["varlen"][2], 1),
                  "two_streams": {"tokens_per_s": iters * NT / wall_f2,
                                  "ms_per_iteration": wall_f2 / iters * 1e3,
                                  "streams": "consecutive iterations on alternate streams"}},
        "iterations": iters,
        "tokens_per_iteration": NT,
        "prefill_roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                             "time": "prefill_kernel + prefill_merge_kernel of the 64 calls",
                             "traffic": None if pmc is None else pmc["hbm_bytes"],
                             "traffic_unit": "HBM bytes over the 64 calls (both kernels)",
                             "traffic_algorithmic_bytes": None if pmc is None else
                             pmc["algorithmic_read_bytes"] + pmc["algorithmic_write_bytes"],
                             "kernel": "prefill_kernel<BF16,128,16>",
                             "kernel_us_total": round(tot_pf, 1),
                             "merge_us_total": round(tot_merge, 1),
                             "kernel_only": {"achieved": round(achieved_kernel, 1),
                                             "frac": round(achieved_kernel /
                                                           MFMA_BF16_PEAK_TFLOPS, 4)},
                             "algorithmic_flops": flops},
        "prefill_merge_us_total": round(tm["prefill_merge"][2], 1),
    }


def fp8_leg(args, dev):
    """Long-context fp8 decode: 64 sequences at context 8192, e4m3fn K/V with
    per-tensor scales, bf16 Q; kernel time of pa_decode over `steps` launches."""
    import torch

    import workloads
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import PagedKV, decode_workspace, sm_scale_for

    S, L = 64, 8192
    _, lengths, num_blocks, free_order = workloads.decode_layout(
        4, lambda rng: np.full(S, L, dtype=np.int64), lambda Ls: workloads.blocks_needed(Ls))
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    # amax/448 of an N(0,1) source of this size: the scale is a plain input here
    kv = PagedKV(num_blocks, H_KV, D, "fp8", dev, free_order, 4.9 / 448.0, 4.9 / 448.0)
    fill = []
    for s in range(S):
        pa.check(kv.create(s, L))
        fill.append(kv.slots(s, 0, L))
    _fill_random(kv, np.concatenate(fill), gen, dev)
    tables, lens = kv.pack(list(range(S)), L // BLOCK)
    t_d = torch.from_numpy(tables).to(dev)
    l_d = torch.from_numpy(lens).to(dev)
    q = torch.randn((S, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((S, H_Q, D), dtype=torch.bfloat16, device=dev)
    ws = decode_workspace(S, H_Q, H_KV, D, L, dev)
    sm = sm_scale_for(D)
    for _ in range(args.warmup):
        kv.decode(out, q, t_d, l_d, L, sm, ws)
    torch.cuda.synchronize()
    pa.check(pa.pa_timing_enable(True))
    for _ in range(args.steps):
        kv.decode(out, q, t_d, l_d, L, sm, ws)
    torch.cuda.synchronize()
    tm = _timings(pa, ("decode", "decode_merge"))
    pa.check(pa.pa_timing_enable(False))
    kv.close()
    nbytes = S * L * H_KV * D * 2 * 1 + S * H_Q * D * 4 + S * (L // BLOCK) * 4 + 4 * S
    k_us = tm["decode"][1]
    return {"workload": "fp8 decode: 64 seqs x ctx 8192, 64/8 heads, d128, e4m3fn KV, bf16 Q",
            "bound": "hbm", "achieved": round(nbytes / (k_us / 1e6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(nbytes / (k_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": "decode_kernel<FP8,128,16>", "kernel_us": round(k_us, 2),
            "merge_us": round(tm["decode_merge"][1], 2), "algorithmic_bytes_per_launch": nbytes}


def block_size_leg(args, dev):
    """Block-size sweep (ARTICLE 4.1: small blocks cost table and kernel
    overhead, large ones allocation waste): the decode-70b contexts decoded
    from caches of 8-, 16- and 32-token blocks (pool = 1.1 x the blocks
    needed, shuffled), kernel GB/s on the same algorithmic bytes; and the
    continuous-batching trace's internal fragmentation with each block size
    (host-only scheduler runs)."""
    import torch

    import workloads
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import decode_workspace, sm_scale_for

    lengths, _, _ = workloads.decode_70b_layout()
    S = len(lengths)
    max_ctx = int(lengths.max())
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    q = torch.randn((S, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((S, H_Q, D), dtype=torch.bfloat16, device=dev)
    ws = decode_workspace(S, H_Q, H_KV, D, max_ctx, dev)
    sm = sm_scale_for(D)
    res = {}
    for bs in (8, 16, 32):
        need = int(sum(-(-int(L) // bs) for L in lengths))
        nb = -(-11 * need // 10)
        order = np.random.default_rng(6 + bs).permutation(nb).astype(np.int32)
        st, pool = pa.pa_pool_create(nb, bs, order)
        pa.check(st)
        for s_, L in enumerate(lengths.tolist()):
            pa.check(pa.pa_seq_create(pool, s_, int(L)))
        mb = -(-max_ctx // bs)
        st, tables, lens = pa.pa_pack_batch(pool, np.arange(S), mb)
        pa.check(st)
        pa.pa_pool_destroy(pool)
        # cache contents are random: the kernel's traffic does not depend on them
        k = torch.randn((nb, H_KV, D // 8, bs, 8), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((nb, H_KV, D, bs), generator=gen, device=dev).to(torch.bfloat16)
        t_d = torch.from_numpy(tables).to(dev)
        l_d = torch.from_numpy(lens).to(dev)
        for _ in range(args.warmup):
            pa.check(pa.pa_decode(None, out, q, k, v, t_d, l_d, nb, H_KV, max_ctx, sm, ws=ws,
                                  bs=bs))
        torch.cuda.synchronize()
        pa.check(pa.pa_timing_enable(["decode"]))
        for _ in range(max(args.steps // 4, 5)):
            pa.check(pa.pa_decode(None, out, q, k, v, t_d, l_d, nb, H_KV, max_ctx, sm, ws=ws,
                                  bs=bs))
        torch.cuda.synchronize()
        tm = _timings(pa, ("decode",))
        pa.check(pa.pa_timing_enable(False))
        del k, v
        torch.cuda.empty_cache()
        nbytes = int(lens.astype(np.int64).sum()) * H_KV * D * 2 * 2 + S * H_Q * D * 4 + \
            int((-(-lens.astype(np.int64) // bs)).sum()) * 4 + 4 * S
        k_us = tm["decode"][1]
        res[str(bs)] = {"kernel_us": round(k_us, 2),
                        "achieved_GBps": round(nbytes / (k_us / 1e6) / 1e9, 1),
                        "frac": round(nbytes / (k_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                        "blocks_held": need}
    # chunked prefill from caches of each block size: slices 15, 31, 47 and 63
    # of the 32768-token prompt (512 positions each, against their prefix)
    from paged_kv_cache_host_amd.engine import prefill_workspace
    P, C, picks = 32768, 512, (15, 31, 47, 63)
    qp = torch.randn((C, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    op = torch.empty((C, H_Q, D), dtype=torch.bfloat16, device=dev)
    wsp = prefill_workspace(1, C, H_Q, H_KV, D, P, dev)
    cu = torch.tensor([0, C], dtype=torch.int32, device=dev)
    for bs in (8, 16, 32):
        nb = P // bs + 64
        order = np.random.default_rng(60 + bs).permutation(nb).astype(np.int32)
        st, pool = pa.pa_pool_create(nb, bs, order)
        pa.check(st)
        pa.check(pa.pa_seq_create(pool, 0, P))
        st, tables, _ = pa.pa_pack_batch(pool, [0], P // bs)
        pa.check(st)
        pa.pa_pool_destroy(pool)
        k = torch.randn((nb, H_KV, D // 8, bs, 8), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((nb, H_KV, D, bs), generator=gen, device=dev).to(torch.bfloat16)
        t_d = torch.from_numpy(tables).to(dev)
        starts = {c: torch.tensor([c * C], dtype=torch.int32, device=dev) for c in picks}

        def call(c):
            pa.check(pa.pa_prefill_chunk(None, op, qp, cu, starts[c], k, v, t_d, nb, H_KV, C,
                                         (c + 1) * C, sm, ws=wsp, bs=bs))
        for _ in range(3):
            for c in picks:
                call(c)
        torch.cuda.synchronize()
        pa.check(pa.pa_timing_enable(["prefill", "prefill_merge"]))
        reps = 5
        for _ in range(reps):
            for c in picks:
                call(c)
        torch.cuda.synchronize()
        tm = _timings(pa, ("prefill", "prefill_merge"))
        pa.check(pa.pa_timing_enable(False))
        del k, v
        torch.cuda.empty_cache()
        flops = reps * sum(4.0 * D * H_Q * (C * c * C + C * (C + 1) / 2) for c in picks)
        kern = tm["prefill"][2]
        whole = kern + tm["prefill_merge"][2]
        res[str(bs)]["prefill_slices_15_31_47_63"] = {
            "kernel_us_per_pass": round(kern / reps, 1),
            "with_merge_us_per_pass": round(whole / reps, 1),
            "TFLOPs_kernel": round(flops / (kern / 1e6) / 1e12, 1),
            "frac_bf16_peak_with_merge": round(flops / (whole / 1e6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # fragmentation of the continuous-batching trace per block size
    w = workloads.trace()
    for bs in (8, 16, 32):
        nb = w.num_blocks * BLOCK // bs
        st, pool = pa.pa_pool_create(nb, bs, None)
        pa.check(st)
        st, sch = pa.pa_sched_create(pool, w.max_running, w.prefill_budget, bs)
        pa.check(st)
        b = pa.SchedBatch(w.max_running, w.prefill_budget)
        waste = []
        for it in range(w.iters):
            for sid, p_, o in w.arrivals[it]:
                pa.check(pa.pa_sched_add(sch, sid, p_, o))
            pa.check(pa.pa_sched_step(sch, b))
            st, acc = pa.pa_sched_stats(sch)
            pa.check(st)
            held = acc["blocks_held"] * bs
            if held:
                waste.append(1.0 - acc["tokens_held"] / held)
        pa.pa_sched_destroy(sch)
        pa.pa_pool_destroy(pool)
        res[str(bs)]["trace_internal_waste_mean"] = round(float(np.mean(waste)), 5)
        res[str(bs)]["trace_internal_waste_max"] = round(float(np.max(waste)), 5)
    return {"workload": "decode-70b contexts (128 seqs, 64/8 heads, d128, bf16) with 8/16/32-token "
                        "blocks; slices 15/31/47/63 of the 32768-token prompt (512 positions, "
                        "64/8 heads, d128, bf16) prefilled from the same block sizes; trace "
                        "fragmentation with the same block sizes",
            "by_block_size": res}


def fp8_prefill_leg(args, dev):
    """The chunked-prefill prompt with an fp8 cache: a 32768-token prompt
    (bf16 source K/V stored as e4m3fn with per-tensor scales, bf16 Q) attended
    as 64 causal 512-token slices; prefill kernel time over the slices and
    its MFMA throughput on the same algorithmic flop count as the bf16 leg."""
    import torch

    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import PagedKV, prefill_workspace, sm_scale_for

    P, C = 32768, 512
    iters = P // C
    nb = P // BLOCK
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    order = np.random.default_rng(6).permutation(nb).astype(np.int32)
    kv = PagedKV(nb, H_KV, D, "fp8", dev, order, 4.9 / 448.0, 4.9 / 448.0)
    pa.check(kv.create(0, P))
    _fill_random(kv, kv.slots(0, 0, P), gen, dev)
    tables, _ = kv.pack([0], nb)
    t_d = torch.from_numpy(tables).to(dev)
    q = torch.randn((P, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((C, H_Q, D), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, C], dtype=torch.int32, device=dev)
    starts = [torch.tensor([c * C], dtype=torch.int32, device=dev) for c in range(iters)]
    ws = prefill_workspace(1, C, H_Q, H_KV, D, P, dev)
    sm = sm_scale_for(D)
    for c in range(0, iters, 8):   # warm-up
        kv.prefill(out, q[c * C:(c + 1) * C], cu, starts[c], t_d, C, (c + 1) * C, sm, ws)
    torch.cuda.synchronize()
    pa.check(pa.pa_timing_enable(["prefill", "prefill_merge"]))
    for c in range(iters):
        kv.prefill(out, q[c * C:(c + 1) * C], cu, starts[c], t_d, C, (c + 1) * C, sm, ws)
    torch.cuda.synchronize()
    tm = _timings(pa, ("prefill", "prefill_merge"))
    pa.check(pa.pa_timing_enable(False))
    kv.close()
    assert tm["prefill"][0] == iters, tm
    pairs = sum(C * (c * C) + C * (C + 1) // 2 for c in range(iters))
    flops = 4 * D * H_Q * pairs
    achieved = flops / (tm["prefill"][2] / 1e6) / 1e12
    return {"workload": "fp8 prefill: 32768-token prompt as 64 causal 512-token slices, 64/8 heads, "
                        "d128, e4m3fn KV, bf16 Q",
            "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "peak_note": "the e4m3fn K/V are widened to bf16 / fp16 for the matrix cores, "
                         "so the contraction runs at the dense bf16 peak",
            "kernel": "prefill_kernel<FP8,128,16>",
            "kernel_us_total": round(tm["prefill"][2], 1),
            "prefill_merge_us_total": round(tm["prefill_merge"][2], 1),
            "algorithmic_flops": flops}


def prefix_leg(args, dev):
    """Prefix sharing (ARTICLE 4.3): 128 sequences that start with the same
    1024-token system prompt, followed by their own lognormal contexts
    (decode-70b lengths).  The same decode batch runs over three pools: one
    where every sequence holds the prompt's 64 blocks through pa_seq_share,
    one where each holds a private copy, and one where the prompt's owner
    registers its computed blocks by content and every other sequence is
    created from its token ids alone (pa_seq_create_prefix finds the 64
    blocks).  Reports the blocks held and the decode kernel time of each on
    the same algorithmic bytes."""
    import torch

    import workloads
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import PagedKV, decode_workspace, sm_scale_for

    PFX = 1024
    own, _, _ = workloads.decode_70b_layout()
    S = len(own)
    lens = PFX + own
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    sm = sm_scale_for(D)
    q = torch.randn((S, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((S, H_Q, D), dtype=torch.bfloat16, device=dev)
    res = {}
    # token ids (detected pool): one prompt, then each sequence's own ids,
    # drawn apart from the prompt's so that only the prompt's blocks match
    ids_rng = np.random.default_rng(11)
    prompt_ids = ids_rng.integers(0, 32000, PFX).astype(np.int32)
    own_ids = [ids_rng.integers(32000, 64000, int(n)).astype(np.int32) for n in own]
    for mode in ("shared", "private", "detected"):
        nb = int(np.sum(-(-lens // BLOCK))) + PFX // BLOCK + 8
        order = np.random.default_rng(7).permutation(nb).astype(np.int32)
        kv = PagedKV(nb, H_KV, D, "bf16", dev, order)
        if mode == "detected":
            st, _ = pa.pa_seq_create_prefix(kv.pool, S, prompt_ids)     # the prompt's owner
            pa.check(st)
            _fill_random(kv, kv.slots(S, 0, PFX), gen, dev)
            torch.cuda.synchronize()                           # its K/V are in the cache
            pa.check(pa.pa_seq_register_prefix(kv.pool, S, prompt_ids))
            fill, found = [], []
            for s in range(S):
                st, shared = pa.pa_seq_create_prefix(
                    kv.pool, s, np.concatenate([prompt_ids, own_ids[s]]))
                pa.check(st)
                found.append(shared)
                fill.append(kv.slots(s, shared, int(lens[s]) - shared))
            _fill_random(kv, np.concatenate(fill), gen, dev)
            if min(found) != PFX or max(found) != PFX:
                raise RuntimeError(f"prefix detection found {min(found)}..{max(found)} of "
                                   f"the {PFX} prompt tokens")
            registered = pa.pa_pool_num_registered(kv.pool)
        elif mode == "shared":
            pa.check(kv.create(S, PFX))                       # the prompt's owner
            _fill_random(kv, kv.slots(S, 0, PFX), gen, dev)
            fill = []
            for s in range(S):
                st, shared = pa.pa_seq_share(kv.pool, s, S, PFX, int(lens[s]))
                pa.check(st)
                fill.append(kv.slots(s, shared, int(lens[s]) - shared))
            _fill_random(kv, np.concatenate(fill), gen, dev)
        else:
            fill = []
            for s in range(S):
                pa.check(kv.create(s, int(lens[s])))
                fill.append(kv.slots(s, 0, int(lens[s])))
            _fill_random(kv, np.concatenate(fill), gen, dev)
        held = nb - pa.pa_pool_num_free(kv.pool)
        tables, lns = kv.pack(list(range(S)))
        t_d = torch.from_numpy(tables).to(dev)
        l_d = torch.from_numpy(lns).to(dev)
        mc = int(lns.max())
        ws = decode_workspace(S, H_Q, H_KV, D, mc, dev)
        for _ in range(args.warmup):
            kv.decode(out, q, t_d, l_d, mc, sm, ws)
        torch.cuda.synchronize()
        pa.check(pa.pa_timing_enable(["decode"]))
        for _ in range(args.steps):
            kv.decode(out, q, t_d, l_d, mc, sm, ws)
        torch.cuda.synchronize()
        tm = _timings(pa, ("decode",))
        pa.check(pa.pa_timing_enable(False))
        kv.close()
        nbytes = decode_bytes(lns)
        us = tm["decode"][1]
        res[mode] = {"blocks_held": int(held), "kernel_us": round(us, 2),
                     "achieved_GBps": round(nbytes / (us / 1e6) / 1e9, 1)}
    res["workload"] = ("prefix sharing: 128 seqs = 1024-token shared system prompt + decode-70b "
                       "lengths, 64/8 heads, d128, bf16; decode kernel on algorithmic bytes")
    res["algorithmic_bytes_per_launch"] = int(nbytes)
    res["blocks_saved"] = res["private"]["blocks_held"] - res["shared"]["blocks_held"]
    res["detected"]["registered_blocks"] = int(registered)
    res["detected"]["prompt_tokens_found_per_sequence"] = PFX
    return res


def prefix_trace_leg(args, dev):
    """Prefix caching in the serving loop: 1000 iterations of requests behind
    one of 8 shared system prompts (512-2048 tokens) plus their own tokens,
    run twice over the same arrivals: requests queued with their prompt's
    token ids (the scheduler shares the prompt blocks earlier requests
    computed and prefills after them) and without.  Reports prefill tokens
    computed, prompt tokens found shared, output tokens and their rate."""
    import torch

    import workloads
    from paged_kv_cache_host_amd.iteration import LayerIterations

    arrivals, num_blocks = workloads.prefix_trace()
    iters, R, B = len(arrivals), 256, 512
    max_ctx = max(p + o for row in arrivals for _, p, o, _ in row)
    ring_n = 8 * (R + B)
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    k_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    v_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    q_ring = torch.randn((ring_n, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    pos = [0]

    def provider(seqs, positions):
        n = len(seqs)
        a = pos[0] if pos[0] + n <= ring_n else 0
        pos[0] = a + n
        return k_ring[a:a + n], v_ring[a:a + n], q_ring[a:a + n]

    res = {}
    for mode in ("cached", "uncached"):
        run = LayerIterations(num_blocks, H_Q, H_KV, D, dev, provider, R, B, max_context=max_ctx,
                              provider_syncs=False)
        torch.cuda.synchronize()
        _settle()
        t0 = time.perf_counter()
        for it in range(iters):
            for sid, p_, o, ids in arrivals[it]:
                run.add(sid, p_, o, ids=ids if mode == "cached" else None)
            run.step()
        run.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        res[mode] = {"ms_per_iteration": round(wall / iters * 1e3, 4),
                     "prefill_tokens": run.totals["prefill_tokens"],
                     "prompt_tokens_found_shared": int(run.acc["prefix_hit_tokens"]),
                     "output_tokens": run.totals["decode_tokens"],
                     "output_tokens_per_s": round(run.totals["decode_tokens"] / wall, 1),
                     "finished": run.totals["finished"],
                     "preemptions": run.totals["preempted"]}
        run.close()
        del run
        torch.cuda.empty_cache()
    # the host side alone (ARTICLE 4.3 / 5: weigh what match detection adds
    # to the scheduler): the C scheduler over the same arrivals, no kernels,
    # with and without the token ids; best of three passes each
    from paged_kv_cache_host_amd import _pa as pa
    host = {}
    for mode in ("cached", "uncached"):
        best = None
        for _ in range(3):
            st_, pool = pa.pa_pool_create(num_blocks, BLOCK, None)
            pa.check(st_)
            st_, sch = pa.pa_sched_create(pool, R, B, BLOCK)
            pa.check(st_)
            b = pa.SchedBatch(R, B)
            t0 = time.perf_counter()
            for it in range(iters):
                for sid, p_, o, ids in arrivals[it]:
                    if mode == "cached":
                        pa.check(pa.pa_sched_add_prompt(sch, sid, o, ids))
                    else:
                        pa.check(pa.pa_sched_add(sch, sid, p_, o))
                pa.check(pa.pa_sched_step(sch, b))
            dt = time.perf_counter() - t0
            pa.pa_sched_destroy(sch)
            pa.pa_pool_destroy(pool)
            best = dt if best is None else min(best, dt)
        host[mode] = round(best / iters * 1e6, 2)
    # prefix retention (pool option, off by default): the scheduler's
    # decisions alone over the same trace and over arrivals 10x sparser, where
    # a system prompt often has no running holder when the next request comes
    ret = {}
    for lam in (0.5, 0.05):
        arr = arrivals if lam == 0.5 else workloads.prefix_trace(lam=lam)[0]
        row = {}
        for retain in (False, True):
            st_, pool = pa.pa_pool_create(num_blocks, BLOCK, None)
            pa.check(st_)
            pa.check(pa.pa_pool_set_prefix_retention(pool, retain))
            st_, sch = pa.pa_sched_create(pool, R, B, BLOCK)
            pa.check(st_)
            b = pa.SchedBatch(R, B)
            pf = 0
            for it in range(iters):
                for sid, p_, o, ids in arr[it]:
                    pa.check(pa.pa_sched_add_prompt(sch, sid, o, ids))
                pa.check(pa.pa_sched_step(sch, b))
                pf += b.n_prefill_tokens
            st_, acc = pa.pa_sched_stats(sch)
            pa.check(st_)
            row["retained" if retain else "not_retained"] = {
                "prompt_tokens_found_shared": int(acc["prefix_hit_tokens"]),
                "prefill_tokens": int(pf), "finished": int(acc["finished"])}
            pa.pa_sched_destroy(sch)
            pa.pa_pool_destroy(pool)
        ret[f"poisson_{lam}"] = row
    res["retention"] = {**ret, "note": ("scheduler decisions only (host), with the token ids; "
                                        "retained = freed registered blocks stay findable "
                                        "until the free list needs them")}
    res["host_us_per_iteration"] = {**host, "note": (
        "C scheduler alone (requests queued + pa_sched_step, through the ctypes binding), "
        "no kernels; cached = with the prompts' token ids (lookups at admission, "
        "registration of computed blocks)")}
    res["workload"] = (f"prefix trace: {iters} iterations, Poisson(0.5) arrivals, prompts = one of 8 "
                       "system prompts (512-2048 tokens) + lognormal own tokens (median 256, "
                       "sigma 1, cap 8192), geometric outputs (mean 256), <=256 running, "
                       "512-token prefill budget, 64/8 heads, d128, bf16, one layer")
    return res


def preemption_leg(args, dev):
    """ARTICLE 4.2: frequent preemption wastes work on recomputation, and the
    pages advise a reasonable cap on concurrent sequences.  1000 iterations
    of short prompts (lognormal median 200, cap 4096) with long outputs
    (geometric, mean 800) on a 2048-block pool, so that admitted sequences
    outgrow the pool, at running caps of 32, 64, 128 and 256: preemptions,
    prefill tokens (recomputation included), output tokens, their rate and
    the iteration time, kernels included."""
    import torch

    import workloads
    from paged_kv_cache_host_amd.iteration import LayerIterations

    w = workloads.trace(seed=5, iters=1000, lam=0.5, prompt_median=200, prompt_cap=4096,
                        out_mean=800, num_blocks=2048)
    B = 512
    max_ctx = max(p + o for row in w.arrivals for _, p, o in row)
    ring_n = 8 * (256 + B)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    k_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    v_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    q_ring = torch.randn((ring_n, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    pos = [0]

    def provider(seqs, positions):
        n = len(seqs)
        a = pos[0] if pos[0] + n <= ring_n else 0
        pos[0] = a + n
        return k_ring[a:a + n], v_ring[a:a + n], q_ring[a:a + n]

    res = {}
    # untimed warm-up: the first iterations of a fresh driver carry one-time
    # set-up (library kernels' first launches, allocator caches)
    run = LayerIterations(w.num_blocks, H_Q, H_KV, D, dev, provider, 64, B,
                          max_context=max_ctx, provider_syncs=False)
    for it in range(100):
        for sid, p_, o in w.arrivals[it]:
            run.add(sid, p_, o)
        run.step()
    run.synchronize()
    run.close()
    del run
    for R in (32, 64, 128, 256):
        run = LayerIterations(w.num_blocks, H_Q, H_KV, D, dev, provider, R, B,
                              max_context=max_ctx, provider_syncs=False)
        torch.cuda.synchronize()
        _settle()
        t0 = time.perf_counter()
        for it in range(w.iters):
            for sid, p_, o in w.arrivals[it]:
                run.add(sid, p_, o)
            run.step()
        run.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        res[f"max_running_{R}"] = {
            "preemptions": run.totals["preempted"], "prefill_tokens": run.totals["prefill_tokens"],
            "output_tokens": run.totals["decode_tokens"], "finished": run.totals["finished"],
            "ms_per_iteration": round(wall / w.iters * 1e3, 4),
            "output_tokens_per_s": round(run.totals["decode_tokens"] / wall, 1)}
        run.close()
        del run
        torch.cuda.empty_cache()
    res["workload"] = ("preemption: 1000 iterations, Poisson(0.5) arrivals, lognormal prompts "
                       "(median 200, sigma 1, cap 4096), geometric outputs (mean 800), pool 2048 "
                       "blocks, 512-token prefill budget, 64/8 heads, d128, bf16, one layer")
    return res


def trace_leg(args, dev):
    """The continuous-batching trace: Poisson arrivals, lognormal prompts,
    geometric outputs, 256 running, 512-token prefill budget, 1000
    iterations of scheduling + cache write + decode/prefill attention for one
    layer.  Reports tokens/s per layer, KV fragmentation and the requests'
    time to first token and inter-token gaps (iteration clock x measured
    iteration time)."""
    import torch

    import workloads
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.iteration import LatencyLog, LayerIterations

    w = workloads.trace()
    max_ctx = max(p + o for row in w.arrivals for _, p, o in row)
    # Host-only dry run of the same scheduler: the highest block id the trace
    # touches (the FIFO pool hands out low ids first), and every request's
    # token times on the iteration clock (the scheduler is deterministic, so
    # the timed run makes the same decisions).
    st, pool = pa.pa_pool_create(w.num_blocks, BLOCK, None)
    pa.check(st)
    st, sch = pa.pa_sched_create(pool, w.max_running, w.prefill_budget, BLOCK)
    pa.check(st)
    b = pa.SchedBatch(w.max_running, w.prefill_budget)
    top = 0
    lat = LatencyLog()
    for it in range(w.iters):
        for sid, p_, o in w.arrivals[it]:
            pa.check(pa.pa_sched_add(sch, sid, p_, o))
            lat.add(it, sid, o)
        pa.check(pa.pa_sched_step(sch, b))
        lat.step(it, b.decode()[0], b.prefill()[0], b.emits())
        if b.n_decode:
            top = max(top, int(b.decode()[2].max()) // BLOCK)
        if b.n_prefill_tokens:
            top = max(top, int(b.slots().max()) // BLOCK)
    pa.pa_sched_destroy(sch)
    pa.pa_pool_destroy(pool)
    used_blocks = top + 1

    torch.cuda.empty_cache()
    ring_n = 8 * (w.max_running + w.prefill_budget)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    k_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    v_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    q_ring = torch.randn((ring_n, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)
    pos = [0]

    def provider(seqs, positions):
        n = len(seqs)
        a = pos[0]
        if a + n > ring_n:
            a = 0
        pos[0] = a + n
        return k_ring[a:a + n], v_ring[a:a + n], q_ring[a:a + n]

    cache_note = "whole pool backed on the device"
    try:
        run = LayerIterations(w.num_blocks, H_Q, H_KV, D, dev, provider, w.max_running,
                              w.prefill_budget, max_context=max_ctx, provider_syncs=False)
    except torch.OutOfMemoryError:
        torch.cuda.empty_cache()
        cache_note = (f"device cache backs the {used_blocks} lowest block ids, the only ones "
                      f"the trace hands out (the host pool has all {w.num_blocks})")
        run = LayerIterations(w.num_blocks, H_Q, H_KV, D, dev, provider, w.max_running,
                              w.prefill_budget, max_context=max_ctx, cache_blocks=used_blocks,
                              provider_syncs=False)
    torch.cuda.synchronize()
    _settle()
    t0 = time.perf_counter()
    n_tok = 0
    for it in range(w.iters):
        for sid, p_, o in w.arrivals[it]:
            run.add(sid, p_, o)
        n_tok += run.step()
    run.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    waste = np.array(run.waste)
    unw = np.array(run.unwritten)
    out = {"workload": f"trace: {w.iters} iterations, Poisson(0.5) arrivals, lognormal prompts "
                       "(median 1000, sigma 1, cap 32768), geometric outputs (mean 256), "
                       "<=256 running, 512-token prefill budget, 64/8 heads, d128, bf16",
           "tokens_per_s": n_tok / wall, "ms_per_iteration": wall / w.iters * 1e3,
           "decode_tokens": run.totals["decode_tokens"],
           "prefill_tokens": run.totals["prefill_tokens"],
           "finished": run.totals["finished"], "preemptions": run.totals["preempted"],
           "latency": lat.summary(wall / w.iters * 1e3),
           "pool_blocks": w.num_blocks, "cache_blocks": run.cache_blocks,
           "cache_note": cache_note,
           "fragmentation": {"internal_waste_mean": float(np.nanmean(waste)),
                             "internal_waste_max": float(np.nanmax(waste)),
                             "reserved_unwritten_mean": float(np.nanmean(unw)),
                             "definition": "1 - tokens the held blocks are allocated for / "
                                           "(16 x blocks held), over running sequences, per "
                                           "iteration; reserved-but-unwritten prompt slots "
                                           "reported separately"}}
    run.close()
    return out


def modes_leg(args, dev):
    """The four schedules of the LESSON's simulator ("Use It": one request at
    a time, padded static batches, continuous batching with whole-prompt
    prefill, continuous batching with 512-token chunks) serving the same
    timed requests on one layer through the paged kernels, on a live clock:
    requests join when their arrival time has passed, every iteration's end
    is timed by an event.  Reports per schedule output tokens/s, mean and
    P99 time to first token, P50/P99/max inter-token latency and goodput
    (output tokens of the requests whose TTFT and every inter-token gap met
    the targets: one layer's 1/80 share of 1 s and 50 ms)."""
    import torch

    import workloads
    from paged_kv_cache_host_amd.iteration import LayerIterations, serve

    reqs = workloads.timed_requests()
    R, CAP = 64, 8192
    budgets = {"naive": CAP, "static": 8 * CAP, "continuous": CAP, "chunked": 512}
    ttft_slo, itl_slo = 1000.0 / 80, 50.0 / 80
    max_ctx = max(r[2] for r in reqs) + max(r[3] for r in reqs)
    num_blocks = 16384
    ring_n = R + max(budgets.values())
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    k_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    v_ring = torch.randn((ring_n, H_KV, D), generator=gen, device=dev).to(torch.bfloat16)
    q_ring = torch.randn((ring_n, H_Q, D), generator=gen, device=dev).to(torch.bfloat16)

    def provider(seqs, positions):
        n = len(seqs)
        return k_ring[:n], v_ring[:n], q_ring[:n]

    out = {"workload": (f"{len(reqs)} requests, Poisson arrivals at 2 per ms, lognormal prompts "
                        "(median 512, sigma 1.2, cap 8192), geometric outputs (mean 64, cap 512), "
                        f"<= {R} running, pool {num_blocks} blocks, 64/8 heads, d128, bf16, one "
                        "layer; live clock"),
           "prefill_budget": budgets,
           "slo_ms": {"ttft": ttft_slo, "itl": itl_slo}, "modes": {}}
    for mode in ("naive", "static", "continuous", "chunked"):
        run = LayerIterations(num_blocks, H_Q, H_KV, D, dev, provider, R, budgets[mode],
                              max_context=max_ctx, provider_syncs=False, mode=mode)
        torch.cuda.synchronize()
        r = serve(run, reqs, ttft_slo, itl_slo)
        run.close()
        del run
        torch.cuda.empty_cache()
        out["modes"][mode] = {
            "output_tokens_per_s": round(r["output_tokens_per_s"], 1),
            "goodput_tokens_per_s": round(r["goodput_tokens_per_s"], 1),
            "slo_met_requests": r["slo_met_requests"],
            "ttft_ms": {k: round(r["ttft"][k], 3) for k in ("mean_ms", "p99_ms")},
            "itl_ms": {k: round(r["itl"][k], 4) for k in ("p50_ms", "p99_ms", "max_ms")},
            "iterations": r["iterations"], "wall_s": round(r["wall_s"], 4),
            "preemptions": r["preemptions"], "prefill_tokens": r["prefill_tokens"],
            "output_tokens": r["output_tokens"]}
        print(f"modes leg: {mode} done ({r['iterations']} iterations)", file=sys.stderr,
              flush=True)
    return out


def cpu_prefill_baseline():
    """The oracle on one 512-token slice at prefix 512 (gather + fp64 causal
    attention of all 64 heads), as GFLOP/s on the algorithmic count, in its
    best configuration of the host's cores (the KV heads' groups spread over
    worker processes, or threads)."""
    from oracle import allocator as oa
    from oracle import attention as oat
    from oracle import cache as oc
    from oracle import codecs
    import workloads

    rng = np.random.default_rng(13)
    P0, C = 512, 512
    n = P0 + C
    nb = n // BLOCK + 4
    pool = oa.BlockPool(nb, BLOCK, rng.permutation(nb).tolist())
    pool.seq_create(0, n)
    kc, vc = oc.new_cache(nb, H_KV, BLOCK, D, "bf16")
    oc.cache_write(kc, vc, workloads.normal_raw(rng, (n, H_KV, D), "bf16"),
                   workloads.normal_raw(rng, (n, H_KV, D), "bf16"), pool.slots(0, 0, n),
                   "bf16", "bf16")
    q = codecs.decode(workloads.normal_raw(rng, (C, H_Q, D), "bf16"), "bf16")
    sm = float(np.float32(1.0) / np.float32(math.sqrt(D)))
    G = H_Q // H_KV
    table = pool.block_table(0)

    def fn(kvh):
        # the oracle on one KV head and its query heads
        return oat.prefill_chunk(q[:, kvh * G:(kvh + 1) * G], P0, kc[:, kvh:kvh + 1],
                                 vc[:, kvh:kvh + 1], table, 1, sm, "bf16")

    configs = _time_oracle(fn, list(range(H_KV)), 24.0)
    flops = 4 * D * H_Q * (C * P0 + C * (C + 1) // 2)
    value, cores, name, allv = _best(configs, flops, 1e9)
    return {"value": value, "unit": "GFLOP/s", "cores": int(cores), "kind": "oracle",
            "config": name, "all_configs_gflop_s": allv,
            "sample": "one 512-token slice at prefix 512, all 64 heads (8 KV-head groups)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the paged-attention path shards by sequence or KV head with no exchange, so "
              "multi-GPU figures are not produced here.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.warmup, args.steps)
        return
    if args.pmc_prefill_summary:
        pmc_prefill_summary(*args.pmc_prefill_summary, args.warmup)
        return
    if args.trace_prefill_summary:
        trace_prefill_summary(args.trace_prefill_summary, args.warmup)
        return
    if args.sq_prefill_summary:
        sq_prefill_summary(args.sq_prefill_summary, args.warmup)
        return

    # The CPU baselines run first: their worker processes are forked, which
    # must happen before this process initialises the GPU.
    cpu = cpu_pf = None
    if not args.no_cpu_baseline and not (args.modes_only or args.mixed_only):
        cpu = cpu_baseline(args.cpu_sample_seqs)
        if not args.decode_only:
            cpu_pf = cpu_prefill_baseline()

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup
    if args.modes_only:
        print(json.dumps({"schedules": modes_leg(args, dev)}), flush=True)
        return
    if args.mixed_only:
        print(json.dumps({"mixed": mixed_leg(args, dev)}), flush=True)
        return

    d = decode_leg(args, dev)
    digest = kernel_source_digest()
    dpmc = decode_pmc_from_profile(digest)
    result = {
        "metric": "paged-attn decode HBM GB/s (% peak); mixed decode+prefill tokens/s per layer",
        "value": round(d["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(d["wall"] / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode-70b-shaped: 128 seqs, 64/8 heads, d128, bf16 KV, "
                               "block 16, lognormal ctx mean 1500 (one layer, one decode "
                               "iteration per step incl. host append + cache write)",
                   "num_seqs": d["num_seqs"], "mean_context": round(d["mean_context"], 1),
                   "num_blocks": d["num_blocks"]},
        "roofline": {"bound": "hbm", "achieved": round(d["achieved"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(d["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": None if dpmc is None else dpmc["hbm_bytes_per_launch"],
                     "traffic_algorithmic_bytes": None if dpmc is None else
                     dpmc["algorithmic_bytes_per_launch"],
                     "traffic_note": "counter bytes and algorithmic bytes per launch of the "
                                     "profiled run (its contexts differ slightly from this run's)",
                     "kernel": d["kernel"],
                     "kernel_us": round(d["kernel_us"], 2),
                     "other_kernels_us": {"decode_merge_kernel": round(d["merge_us"], 2)} |
                     ({} if d["fused"] else {"stage_cache_write_kernel":
                                             round(d["stage_cache_write_us"], 2)}),
                     "algorithmic_bytes_per_launch": d["bytes_per_launch"],
                     "kernel_source_digest": digest},
    }
    if not args.decode_only:
        # the same step as one pa_decode_step launch (metadata staged, new
        # tokens appended, blocks entered and attention, in one kernel)
        alt = "fused" if not d["fused"] else "separate"
        f = decode_leg(args, dev, alt)
        result["decode_step_" + alt] = {
            "launch": ("pa_decode_step (staging, append, table entries and attention in one "
                       "kernel)" if alt == "fused" else "pa_stage_decode_append + pa_decode"),
            "value": round(f["value"], 2), "unit": "GB/s",
            "ms_per_step": round(f["wall"] / K * 1e3, 4),
            "kernel": f["kernel"], "kernel_us": round(f["kernel_us"], 2),
            "achieved": round(f["achieved"], 2),
            "frac": round(f["achieved"] / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": f["bytes_per_launch"]}
        m = mixed_leg(args, dev)
        m["workload"] = ("mixed chunked prefill: 32768-token prompt as 64 causal 512-token "
                         "slices + 127 decodes per iteration, 64/8 heads, d128, bf16")
        result["mixed"] = m
        result["fp8_decode"] = fp8_leg(args, dev)
        result["fp8_prefill"] = fp8_prefill_leg(args, dev)
        result["prefix_sharing"] = prefix_leg(args, dev)
        result["prefix_trace"] = prefix_trace_leg(args, dev)
        result["preemption"] = preemption_leg(args, dev)
        result["block_size"] = block_size_leg(args, dev)
        result["trace"] = trace_leg(args, dev)
        result["schedules"] = modes_leg(args, dev)
    result["cpu_baseline"] = cpu
    if "mixed" in result and cpu_pf is not None:
        result["mixed"]["cpu_baseline"] = cpu_pf
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
