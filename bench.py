#!/usr/bin/env python3
"""Benchmark of one decode step of paged attention on one MI355X.

A step is the whole hot path for one layer: reshape_and_cache appends the new
token of every sequence, paged_attention_decode attends each sequence's query
over its paged K/V, and (when a partition size is set) the partition reduce
merges split-K partials.  Inputs are seeded synthetic data with the shapes of
the workload (workloads.py), resident in HBM before timing starts.  Several
copies of the KV pool ("layers") are rotated so that consecutive steps never
find their K/V in the 256 MB last-level cache.

Prints ONE JSON line on stdout; progress goes to stderr.

  metric  achieved HBM bandwidth of the step (algorithmic bytes / step time)
          and decode tokens/s/layer
  roofline  the decode kernel alone, timed with HIP events on the stream it
          runs on, against the MI355X HBM peak of 8 TB/s
  cpu_baseline  the CPU oracle on this host, on a bounded sample of the same
          workload
  max_abs_err_vs_oracle  the oracle's sampled rows against the device output
          of the last step, with the tolerance of the cache type
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "paged decode attention: achieved HBM TB/s (% of peak) + decode tokens/s/layer"
PEAK_GBPS = 8000.0
E = workloads.ELEM_BYTES


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def chunk_floor(cache_dtype: str, bs: int, D: int) -> int:
    """Floor on the balanced split's later chunks: two rounds of the decode's
    tile ring (10 tiles for fp8, else 6, or 8 at D = 64; half with 8-token
    blocks)."""
    pair = bs == 8
    if E[cache_dtype] == 1:
        depth = 5 if pair else 10
    else:
        depth = 4 if pair else (8 if D == 64 else 6)
    return 2 * depth


def balanced_split(lens: np.ndarray, Hkv: int, nW: int, floor: int, tile_tokens=None):
    """The balanced split's pieces, replayed on the host: the streams
    (sequence, KV head) of 16-token tiles laid end to end and cut into chunks
    by the guided schedule (nW chunks of max(1, 4A/5) tiles, nW of
    max(A/7, F), then max(A/16, F), A = T / nW, F = max(floor, 4)), each cut
    inside a stream moved to the nearer end of that stream when it lies
    within an eighth of the smaller neighbouring chunk (a quarter after the
    first nW chunks).  tile_tokens: each
    sequence's tile (mixed block sizes: 8 for 8-token blocks), default 16.
    Returns (number of streams spread over several chunks, partial entries
    they write per query head)."""
    tt = 16 if tile_tokens is None else np.asarray(tile_tokens, np.int64)
    nt = -(-np.maximum(lens.astype(np.int64), 0) // tt)
    T = int(nt.sum()) * Hkv
    if T == 0:
        return 0, 0
    A = T // nW
    F = max(floor, 4)
    C1, C2, C3 = max(1, A * 4 // 5), max(F, A // 7), max(F, A // 16)
    if nW * C1 >= T:
        chunks = -(-T // C1)
    elif nW * (C1 + C2) >= T:
        chunks = nW + -(-(T - nW * C1) // C2)
    else:
        chunks = 2 * nW + -(-(T - nW * (C1 + C2)) // C3)
    c = np.arange(chunks + 1, dtype=np.int64)
    plain = np.where(c <= nW, c * C1,
                     np.where(c <= 2 * nW, nW * C1 + (c - nW) * C2,
                              nW * (C1 + C2) + (c - 2 * nW) * C3))
    plain = np.minimum(plain, T)
    g0 = (np.repeat(np.cumsum(nt) - nt, Hkv) * Hkv
          + np.tile(np.arange(Hkv), lens.size) * np.repeat(nt, Hkv))
    g1 = g0 + np.repeat(nt, Hkv)
    live = g1 > g0
    # move the inner cuts
    lo_s, hi_s = g0[live], g1[live]
    b = plain[1:-1]
    d = np.minimum(b - plain[:-2], plain[2:] - b) // np.where(c[1:-1] <= nW, 8, 4)
    k = np.searchsorted(lo_s, b, side="right") - 1
    r = b - lo_s[k]
    up = hi_s[k] - b
    moved = np.where(r <= d, b - r, np.where(up <= d, b + up, b))
    starts = np.concatenate([plain[:1], moved, plain[-1:]])
    c0 = np.searchsorted(starts, g0, side="right") - 1
    c1 = np.searchsorted(starts, np.maximum(g1 - 1, 0), side="right") - 1
    split = live & (c1 > c0)
    return int(split.sum()), int((c1 - c0 + 1)[split].sum())


def decode_bytes(c, P: int, nW: int = 0, tile_tokens=None, floor_bs=None) -> dict:
    """Algorithmic bytes one decode launch (and its reduce) must move: each KV
    head's rows once per group, Q in, O out, the table entries used, the
    lengths, and for split-K the partials written once and read once."""
    L = c.seq_lens.astype(np.int64)
    kv = int(L.sum()) * c.Hkv * c.D * E[c.cache_dtype] * 2
    row = c.Hq * c.D * E[c.q_dtype]                  # one sequence's Q (or O)
    table = 4 * int((-(-L // c.bs)).sum()) + 4 * c.S
    n_multi, partials = 0, 0
    if P > 0:
        nparts = -(-L // P)
        multi = nparts > 1
        n_multi = int(multi.sum())
        partials = int(nparts[multi].sum()) * c.Hq * (c.D + 2) * 4
    elif P < 0:
        # a split (sequence, KV head) stream writes one entry per piece for each
        # query head of its group; its G output rows come from the reduce
        split_streams, entries = balanced_split(
            L, c.Hkv, nW, chunk_floor(c.cache_dtype, floor_bs or c.bs, c.D), tile_tokens)
        n_multi = split_streams / c.Hkv          # in units of whole sequences
        partials = entries * c.G * (c.D + 2) * 4
    # decode: K/V, Q, O of sequences it finishes, table, lengths, partials out
    dec = kv + c.S * row + (c.S - n_multi) * row + table + partials
    # reduce: partials in, O of the split sequences, lengths
    red = partials + int(n_multi * row) + 4 * c.S if P != 0 else 0
    dec = int(dec)
    T = c.slot_mapping.size
    append = T * c.Hkv * c.D * (E[c.src_dtype] + E[c.cache_dtype]) * 2 + 8 * T
    return {"kv": kv, "decode_kernel": dec, "reduce_kernel": red,
            "append": append, "step": dec + red + append}


# Source file each profiled kernel is compiled from.
KERNEL_SOURCE = {"decode_balanced_kernel": "decode_balanced.hip",
                 "decode_mfma_kernel": "decode_mfma.hip",
                 "reduce_group_kernel": "reduce.hip"}
# kernels of one call whose counters a workload's record sums: the decode
# kernel alone, except verification, whose call is the balanced kernel and
# its grouped reduce
CALL_KERNELS = {"spec-verify": ("decode_balanced_kernel", "reduce_group_kernel")}


def decode_kernel_name(P: int) -> str:
    """The kernel a decode call of split P runs for 16-bit and fp8 caches."""
    return "decode_balanced_kernel" if P < 0 else "decode_mfma_kernel"


def traffic_key(args, bs: int) -> str:
    """Name of a workload's counter record: the workload, the block size of
    the shared-prefix workload, and the partition size when one is forced."""
    key = args.workload
    if args.workload == "shared-prefix-fp8":
        key += "-bs%d" % bs
    if args.partition is not None:
        key += "-P%d" % args.partition
    return key


def kernel_sources(top: str) -> list:
    """`top` and every csrc header it includes (quoted includes, recursively)."""
    csrc = os.path.join(ROOT, "paged_kv_cache_361_amd", "csrc")
    seen, todo = [], [top]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.append(name)
        with open(os.path.join(csrc, name)) as f:
            for line in f:
                m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
                if m and os.path.exists(os.path.join(csrc, m.group(1))):
                    todo.append(m.group(1))
    return sorted(seen)


def kernel_source_hash(kernel: str = "decode_balanced_kernel") -> str:
    """Hash of the sources the kernel is built from: counters taken from an
    older version of them no longer describe it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_361_amd", "csrc")
    for name in kernel_sources(KERNEL_SOURCE[kernel]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, launch_bytes: float):
    """HBM bytes per decode launch from committed PMC summaries, if they were
    taken from the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (ValueError, AttributeError):
        return None
    if not rec:
        return None
    kernels = rec.get("kernels") or [rec.get("kernel")]
    if any(k not in KERNEL_SOURCE for k in kernels):
        return None
    if rec.get("kernel_source_hash") != kernels_source_hash(kernels):
        return None
    return rec.get("hbm_bytes_per_launch")


def kernels_source_hash(kernels) -> str:
    """kernel_source_hash of one kernel, or of the sources of several."""
    if len(kernels) == 1:
        return kernel_source_hash(kernels[0])
    h = hashlib.sha256()
    for k in kernels:
        h.update(kernel_source_hash(k).encode())
    return h.hexdigest()[:16]


def _counter_means(path: str, kernel: str):
    """Mean counter value (KiB) per dispatch of `kernel`, and the value read
    for the calibration copy: the last device copy dispatched before the
    kernel's first dispatch (bench.py makes it after the pools' uploads and
    copies, which can be larger)."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    vals, calib = [], None
    for row in rows:
        name, v = row["Kernel_Name"], float(row["Counter_Value"])
        if kernel + "<" in name:
            vals.append(v)
        elif "copyBuffer" in name and not vals:
            calib = v
    if not vals or calib is None:
        raise SystemExit("%s: no %s dispatch, or no copy before it" % (path, kernel))
    return sum(vals) / len(vals), calib, len(vals)


def record_traffic(args) -> int:
    """Writes HBM bytes per launch of the workload's decode kernel (balanced
    or fixed partitions, as the run used) from two counter runs.  Each
    counter is scaled by what it reads for the plain device copy of
    --copy-calib-mib MiB (that many bytes fetched and written)."""
    if not args.copy_calib_mib:
        raise SystemExit("--record-traffic needs the --copy-calib-mib the runs used")
    known_kib = args.copy_calib_mib * 1024.0
    if args.workload in CALL_KERNELS:
        kernels = list(CALL_KERNELS[args.workload])
    else:
        P = DEFAULT_PARTITION[args.workload] if args.partition is None else args.partition
        kernels = [decode_kernel_name(P)]
    fetch = write = 0.0
    for k in kernels:
        f, fcopy, n = _counter_means(args.record_traffic[0], k)
        w, wcopy, _ = _counter_means(args.record_traffic[1], k)
        fetch, write = fetch + f, write + w
    fs, wsc = known_kib / fcopy, known_kib / wcopy
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    key = traffic_key(args, args.bs)
    rec = {"kernel": kernels[0]} if len(kernels) == 1 else {"kernels": kernels}
    rec.update({
        "kernel_source_hash": kernels_source_hash(kernels),
        "hbm_bytes_per_launch": int(round((fetch * fs + write * wsc) * 1024)),
        "fetch_size_kib": round(fetch, 1), "fetch_scale": round(fs, 4),
        "write_size_kib": round(write, 1), "write_scale": round(wsc, 4),
        "dispatches": n,
    })
    data[key] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(data[key]))
    return 0


def unique_kv_bytes(c) -> int:
    """K+V bytes of the distinct pool slots the tables reach: where sequences
    share prefix blocks, the bytes one launch could fetch from HBM at least."""
    L = c.seq_lens.astype(np.int64)
    slots = [c.block_tables[s, np.arange(L[s]) // c.bs].astype(np.int64) * c.bs
             + np.arange(L[s]) % c.bs for s in range(c.S) if L[s] > 0]
    n = np.unique(np.concatenate(slots)).size if slots else 0
    return int(n) * c.Hkv * c.D * E[c.cache_dtype] * 2


def host_append(c) -> None:
    """The step's cache writes, applied to the host pool by the oracle, so
    that the oracle sees what the device pool holds after a step."""
    import oracle
    if c.slot_mapping.size:
        oracle.reshape_and_cache(c.new_key, c.new_value, c.k_cache, c.v_cache, c.slot_mapping,
                                 src_dtype=c.src_dtype, cache_dtype=c.cache_dtype,
                                 k_scale=c.k_scale, v_scale=c.v_scale)


# Output tolerance against the oracle: 5e-3 for 16-bit (and fp32) caches,
# 3e-2 for fp8 caches (the oracle dequantises the same codes).
TOL = {"f32": 5e-3, "f16": 5e-3, "bf16": 5e-3, "fp8": 3e-2}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpus() -> dict:
    """Logical CPUs of the host and those this process may run on."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 0
    return {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count() or 0,
            "usable_cpus": usable}


def cpu_baseline(c, gpu_out=None, budget_s: float = 20.0):
    """The CPU oracle (as it stands) on the first sequences of the workload:
    a probe on a few sequences sizes a sample of about `budget_s`.  With
    `gpu_out` (the device output as float64 [S, Hq, D]) the sampled rows are
    also compared with it; returns (baseline, comparison or None)."""
    import oracle
    threads = oracle.max_threads()
    kw = dict(q_dtype=c.q_dtype, cache_dtype=c.cache_dtype, scale=c.scale,
              k_scale=c.k_scale, v_scale=c.v_scale, threads=threads)
    last = {}

    def run(n):
        sub_rows = np.arange(n * c.Hq, dtype=np.int32)
        t0 = time.perf_counter()
        r = oracle.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                rows=sub_rows, **kw)
        t = time.perf_counter() - t0
        last["n"], last["ref"] = n, r
        return t

    n = min(8, c.S)
    t = run(n)
    tok = int(c.seq_lens[:n].sum())
    if t < budget_s / 4 and n < c.S:
        per_tok = t / max(tok, 1)
        target = budget_s / per_tok
        cum = np.cumsum(c.seq_lens.astype(np.int64))
        n = int(min(c.S, max(n, np.searchsorted(cum, target) + 1)))
        t = run(n)
        tok = int(c.seq_lens[:n].sum())
    reps = 1
    if t < budget_s / 2:              # the whole workload is quick: repeat it
        reps = int(min(50, max(1, math.ceil(budget_s / 2 / t))))
        t = sum(run(n) for _ in range(reps)) / reps
    def sample_bytes(n):
        sub = c.copy()
        sub.S = n
        sub.seq_lens = c.seq_lens[:n]
        sub.slot_mapping = c.slot_mapping[:0]
        return decode_bytes(sub, 0)["decode_kernel"]

    nbytes = sample_bytes(n)
    base = {"value": round(nbytes / t / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle",
            "tokens_per_s_per_layer": round(n / t, 2),
            "seconds": round(t, 3),
            "sample": "decode of the first %d of %d sequences (%d tokens, all %d query "
                      "heads), gather + fp64 softmax attention, OpenMP over rows; mean "
                      "of %d run(s)" % (n, c.S, tok, c.Hq, reps)}
    base.update(host_cpus())
    # The same oracle on one thread, on the first sequences up to about a
    # quarter of the budget (a probe on the first sequence sizes it).
    kw1 = dict(kw, threads=1)

    def run1(n1):
        t0 = time.perf_counter()
        oracle.paged_decode(c.query, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                            rows=np.arange(n1 * c.Hq, dtype=np.int32), **kw1)
        return time.perf_counter() - t0

    n1 = 1
    t1 = run1(n1)
    if t1 < budget_s / 8 and n1 < c.S:
        per_tok = t1 / max(int(c.seq_lens[0]), 1)
        cum = np.cumsum(c.seq_lens.astype(np.int64))
        n1 = int(min(c.S, max(1, np.searchsorted(cum, budget_s / 4 / per_tok) + 1)))
        t1 = run1(n1)
    reps1 = 1
    if t1 < budget_s / 8:             # the whole workload is quick: repeat it
        reps1 = int(min(50, max(1, math.ceil(budget_s / 8 / max(t1, 1e-6)))))
        t1 = sum(run1(n1) for _ in range(reps1)) / reps1
    base["single_thread"] = {
        "value": round(sample_bytes(n1) / t1 / 1e12, 6), "unit": "TB/s", "cores": 1,
        "tokens_per_s_per_layer": round(n1 / t1, 2), "seconds": round(t1, 3),
        "sample": "decode of the first %d sequences (%d tokens, all %d query heads), "
                  "one thread; mean of %d run(s)" % (n1, int(c.seq_lens[:n1].sum()), c.Hq,
                                                      reps1)}
    cmp = None
    if gpu_out is not None:
        m = last["n"]
        err = float(np.max(np.abs(gpu_out[:m] - last["ref"][:m]))) if m else 0.0
        tol = TOL[c.cache_dtype]
        cmp = {"max_abs_err": err, "tol": tol, "within_tol": bool(err <= tol),
               "rows": m * c.Hq, "of_rows": c.S * c.Hq,
               "sample": "the oracle's rows above against the output of the last step"}
    return base, cmp


# Split used when --partition is not given: the fastest measured on MI355X
# for each workload (the balanced split for the batch workloads; for the
# shared-prefix fp8 workload, whose run is short, fixed 512-token partitions).
DEFAULT_PARTITION = {"tiny-f32": 0, "llama2-13b-mha": -1, "llama3-8b-gqa": -1,
                     "long-context-gqa": -1, "shared-prefix-fp8": 512}


def make_workload(args):
    if args.workload == "shared-prefix-fp8":
        c = workloads.shared_prefix_fp8(bs=args.bs)
    else:
        c = workloads.WORKLOADS[args.workload]()
    P = DEFAULT_PARTITION[args.workload] if args.partition is None else args.partition
    return c, P


WORKLOAD_NAMES = {
    "tiny-f32": "tiny fp32 paged decode: 4 seqs, L {7,16,33,100}, 4/4 heads, D 64, bs 16",
    "llama2-13b-mha": "Llama-2-13B-shaped MHA decode layer, fp16: 64 seqs, L~U[512,2048], 40/40 heads, "
       "D 128, bs 16, +1 appended token/seq",
    "llama3-8b-gqa": "Llama-3-8B-shaped GQA decode layer, bf16: 256 seqs, L~lognormal(median 1024, "
       "sigma 1, cap 4096), 32 q / 8 kv heads, D 128, bs 16, +1 appended token/seq",
    "long-context-gqa": "long-context GQA decode, bf16, split-K: 8 seqs, L {32,48,64,64,96,96,128,128}K, "
       "64 q / 8 kv heads, D 128, bs 32, partitions of 512",
    "shared-prefix-fp8": "shared-prefix decode with fp8-e4m3 KV: 128 seqs, 1024-token shared prefix + "
       "tails U[16,512], 32 q / 8 kv heads, D 128",
}


MULTI_WORKLOADS = {
    "spec-verify": ("speculative verification on the Llama-3-8B GQA decode shape, bf16: "
                    "256 seqs, L~lognormal(median 1024, sigma 1, cap 4096), 4 drafted "
                    "tokens/seq checked in one pass, 32 q / 8 kv heads, D 128, bs 16"),
    "chunked-prefill": ("chunked prefill on the Llama-3-8B GQA shape, bf16: 8 seqs with "
                        "512..3072 cached tokens + a 512-token prompt chunk each, causal "
                        "within the chunk, 32 q / 8 kv heads, D 128, bs 16"),
}
PEAK_BF16_TFLOPS = 2500.0


# Split-K partition size of the multi-query workloads: short drafts over long
# contexts split like decode; 512-token prefill chunks already give one
# wavefront per 16 / G tokens and need no split.
MULTI_PARTITION = {"spec-verify": -1, "chunked-prefill": 0}


def multi_cost(mc):
    """Algorithmic bytes (K/V of each (sequence, KV head) once, Q in, O out,
    table entries, lengths, query offsets) and flops (QK and PV, 2 per
    multiply-add) of one multi-query call."""
    c = mc.case
    L = c.seq_lens.astype(np.int64)
    Qn = np.diff(mc.query_start.astype(np.int64))
    kv = int(L.sum()) * c.Hkv * c.D * E[c.cache_dtype] * 2
    qo = int(Qn.sum()) * c.Hq * c.D * E[c.q_dtype] * 2
    table = 4 * int((-(-L // c.bs)).sum()) + 4 * c.S + 4 * (c.S + 1)
    seen = 0
    for s in range(c.S):              # tokens seen by each query token: its position + 1
        first = int(L[s] - Qn[s]) + 1
        seen += int(Qn[s]) * first + int(Qn[s]) * (int(Qn[s]) - 1) // 2
    flops = 4 * seen * c.Hq * c.D
    return kv + qo + table, flops


def settle_clocks(fn, seconds: float = 0.3) -> None:
    """Untimed calls of fn until `seconds` of wall time have passed: the
    GPU's clocks ramp up over the first tens of milliseconds of work, and a
    short warmup would leave the first timed calls at a lower clock."""
    import torch
    t = time.perf_counter()
    while time.perf_counter() - t < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def bench_multi(args) -> int:
    import torch
    import paged_kv_cache_361_amd as pkv
    torch.cuda.set_device(0)
    log("generating workload %s ..." % args.workload)
    mc = workloads.spec_verify() if args.workload == "spec-verify" else workloads.chunked_prefill()
    c = mc.case

    def dev(a, d):
        if d == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    query = dev(mc.query, c.q_dtype)
    qs = torch.from_numpy(mc.query_start).cuda()
    tables = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(c.seq_lens).cuda()
    k0, v0 = dev(c.k_cache, c.cache_dtype), dev(c.v_cache, c.cache_dtype)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(1, args.layers) - 1)]
    out = torch.empty_like(query)
    stream = torch.cuda.current_stream()
    P = MULTI_PARTITION[args.workload] if args.partition is None else args.partition
    ws = pkv.allocate_multi_workspace(c.S, mc.max_query_len, c.Hq, c.D, c.max_seq_len, P)
    if args.copy_calib_mib:                # a copy of known size, for HBM counter scaling
        a = torch.empty(args.copy_calib_mib << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def call(i):
        kc, vc = layers[i % len(layers)]
        pkv.paged_attention_multi(out, query, kc, vc, tables, lens, qs, scale=c.scale,
                                  max_seq_len=c.max_seq_len, max_query_len=mc.max_query_len,
                                  partition_size=P, workspace=ws)

    W, K = args.warmup, args.steps
    for i in range(W):
        call(i)
    torch.cuda.synchronize()
    settle_clocks(lambda: call(0))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        evs[i][0].record(stream)
        call(W + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    call_s = float(np.mean(ms)) / 1e3
    nbytes, flops = multi_cost(mc)
    total_q = int(mc.query_start[-1])
    if args.workload == "spec-verify":
        metric = "paged multi-query attention: achieved HBM TB/s (% of peak) + query tokens/s/layer"
        value, unit = nbytes / call_s / 1e12, "TB/s"
        traffic = (traffic_from_profiles(traffic_key(args, c.bs), nbytes)
                   if args.partition is None else None)
        roof = {"bound": "hbm", "kernel": "paged_attention_multi",
                "achieved": round(nbytes / call_s / 1e9, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(nbytes / call_s / 1e9 / PEAK_GBPS, 4), "traffic": traffic}
    else:
        metric = "paged multi-query attention: achieved TFLOP/s (% of bf16 MFMA peak) + query tokens/s/layer"
        value, unit = flops / call_s / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "kernel": "paged_attention_multi",
                "achieved": round(flops / call_s / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / call_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": None}
    res = {
        "metric": metric, "value": round(value, 4), "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(t_total / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": c.q_dtype, "data": "synthetic",
        "config": {"workload": MULTI_WORKLOADS[args.workload], "seqs": c.S,
                   "tokens": int(c.seq_lens.sum()), "query_tokens": total_q,
                   "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.D, "block_size": c.bs,
                   "kv_pools_rotated": len(layers), "partition_size": P},
        "call_us": round(call_s * 1e6, 2),
        "query_tokens_per_s_per_layer": round(total_q / call_s, 1),
        "bytes_per_call": nbytes, "flops_per_call": flops,
        "roofline": roof,
    }
    if args.cpu_baseline == "on":
        import oracle
        log("timing the CPU oracle ...")
        threads = oracle.max_threads()
        kc, vc = c.k_cache, c.v_cache
        n = 1
        while True:               # query tokens of the first sequence(s), about 10-20 s
            rows = np.arange(n * c.Hq, dtype=np.int32)
            t = time.perf_counter()
            ref = oracle.paged_multi(mc.query, kc, vc, c.block_tables, c.seq_lens,
                                     mc.query_start, q_dtype=c.q_dtype,
                                     cache_dtype=c.cache_dtype, scale=c.scale, rows=rows,
                                     threads=threads)
            t = time.perf_counter() - t
            if t > 5.0 or n >= total_q:
                break
            n = min(total_q, max(n + 1, int(n * min(8.0, 10.0 / max(t, 1e-3)))))
        res["cpu_baseline"] = {
            "value": round(n / t, 2), "unit": "query tokens/s", "cores": threads,
            "kind": "oracle", "seconds": round(t, 3),
            "sample": "the first %d of %d query tokens, all %d query heads, gather + fp64 "
                      "softmax attention, OpenMP over rows" % (n, total_q, c.Hq)}
        res["cpu_baseline"].update(host_cpus())
        gpu = out[:n].float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(gpu - ref[:n])))
        tol = TOL[c.cache_dtype]
        res["max_abs_err_vs_oracle"] = {
            "max_abs_err": err, "tol": tol, "within_tol": bool(err <= tol),
            "rows": n * c.Hq, "of_rows": total_q * c.Hq,
            "sample": "the oracle's rows above against the output of the last call"}
    print(json.dumps(res), flush=True)
    return 0


HOST_LINK_PEAK_GBPS = 64.0      # PCIe 5.0 x16, one direction, nominal


def bench_swap(args) -> int:
    """Swapping ("vLLM 推理引擎源码级拆解" §3.2): 2048 blocks of the Llama-3-8B
    GQA pool (16 tokens x 8 KV heads x 128, bf16: 32 KiB per block per pool)
    out to a pinned host pool and back, with pkv_copy_blocks (the GPU reads
    and writes host memory directly).  Bound by the host link."""
    import torch
    import paged_kv_cache_361_amd as pkv
    torch.cuda.set_device(0)
    n, bs, Hkv, D = 2048, 16, 8, 128
    NB = 4 * n
    k = torch.randn(NB, bs, Hkv, D, device="cuda").to(torch.bfloat16)
    v = torch.randn_like(k)
    hk = torch.empty((n, bs, Hkv, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    rng = np.random.default_rng(8)
    dev_blocks = rng.permutation(NB)[:n].astype(np.int32)
    out_pairs = torch.from_numpy(np.stack([dev_blocks, np.arange(n, dtype=np.int32)], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(n, dtype=np.int32), dev_blocks], 1)).cuda()
    nbytes = n * bs * Hkv * D * 2 * 2            # K and V blocks moved one way
    stream = torch.cuda.current_stream()
    res_ms = {}
    for name, fn in (("out", lambda: pkv.swap_blocks(hk, hv, k, v, out_pairs)),
                     ("in", lambda: pkv.swap_blocks(k, v, hk, hv, in_pairs))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        res_ms[name] = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    gbps = {k_: nbytes / (ms / 1e3) / 1e9 for k_, ms in res_ms.items()}
    res = {
        "metric": "block swap GPU <-> pinned host: achieved host-link GB/s per direction",
        "value": round(min(gbps.values()), 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res_ms["out"] + res_ms["in"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap 2048 random blocks of the Llama-3-8B GQA pool "
                               "(bs 16, 8 kv heads, D 128, bf16) out to pinned host memory "
                               "and back", "blocks": n, "bytes_per_direction": nbytes},
        "swap_out_gbps": round(gbps["out"], 2), "swap_in_gbps": round(gbps["in"], 2),
        "roofline": {"bound": "host link", "kernel": "copy_blocks",
                     "achieved": round(min(gbps.values()), 2), "peak": HOST_LINK_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(min(gbps.values()) / HOST_LINK_PEAK_GBPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_mixed(args) -> int:
    """Decode over a pool of 8-token pages whose sequences have 8-, 16- or
    32-token blocks (picked by length), with the append, split and reduce of
    a decode step, timed like the main bench."""
    import torch
    import paged_kv_cache_361_amd as pkv
    torch.cuda.set_device(0)
    log("generating workload %s ..." % args.workload)
    mc = workloads.mixed_block_sizes()
    c = mc.case
    P = -1 if args.partition is None else args.partition      # the balanced split

    def dev(a, d):
        if d == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    query = dev(c.query, c.q_dtype)
    tables = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(c.seq_lens).cuda()
    sbs = torch.from_numpy(mc.seq_bs).cuda()
    new_k, new_v = dev(c.new_key, c.src_dtype), dev(c.new_value, c.src_dtype)
    slots = torch.from_numpy(c.slot_mapping).cuda()
    k0, v0 = dev(c.k_cache, c.cache_dtype), dev(c.v_cache, c.cache_dtype)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(1, args.layers) - 1)]
    out = torch.empty_like(query)
    ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P) if P else None
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        kc, vc = layers[i % len(layers)]
        pkv.reshape_and_cache(new_k, new_v, kc, vc, slots)
        if ev:
            ev[0].record(stream)
        pkv.paged_attention_decode_mixed(out, query, kc, vc, tables, lens, sbs, scale=c.scale,
                                         max_seq_len=c.max_seq_len, partition_size=P,
                                         workspace=ws)
        if ev:
            ev[1].record(stream)
        if P:
            pkv.paged_attention_reduce(out, ws, lens, num_kv_heads=c.Hkv,
                                       max_seq_len=c.max_seq_len, partition_size=P)
        if ev:
            ev[2].record(stream)

    W, K = args.warmup, args.steps
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    settle_clocks(lambda: step(0))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    dec_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    red_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    nW = int(ws[:16].cpu().numpy().view(np.int32)[1]) if P < 0 else 0
    # the balanced walk takes 8-token tiles for 8-token blocks and the ring
    # of 16-token blocks
    b = decode_bytes(c, P, nW, tile_tokens=np.where(mc.seq_bs == 8, 8, 16), floor_bs=16)
    L = c.seq_lens.astype(np.int64)
    # table entries: one per block of each sequence's own size, plus the sizes
    table_fix = 4 * int((-(-L // mc.seq_bs.astype(np.int64))).sum()) + 4 * c.S \
        - 4 * int((-(-L // c.bs)).sum())
    dec_bytes = b["decode_kernel"] + table_fix
    call_s = float(np.mean(dec_ms + red_ms)) / 1e3
    dec_s = float(np.mean(dec_ms)) / 1e3
    counts = {int(k): int((mc.seq_bs == k).sum()) for k in (8, 16, 32)}
    res = {
        "metric": "paged decode attention, mixed block sizes: achieved HBM TB/s (% of peak) "
                  "+ decode tokens/s/layer",
        "value": round((dec_bytes + b["reduce_kernel"]) / call_s / 1e12, 4), "unit": "TB/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(t_total / K * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c.q_dtype,
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped GQA decode layer, bf16, block size per "
                               "sequence by length (<128: 8, <2048: 16, else 32 tokens) over "
                               "8-token pages: 256 seqs, L~lognormal(median 1024, sigma 1, "
                               "cap 4096), 32 q / 8 kv heads, D 128",
                   "seqs": c.S, "tokens": int(L.sum()), "sequences_by_block_size": counts,
                   "partition_size": P, "kv_pools_rotated": len(layers)},
        "decode_us": round(dec_s * 1e6, 2), "reduce_us": round(float(np.mean(red_ms)) * 1e3, 2),
        "tokens_per_s_per_layer": round(c.S / call_s, 1),
        "bytes_per_call": {"decode_kernel": dec_bytes, "reduce_kernel": b["reduce_kernel"]},
        "roofline": {"bound": "hbm", "kernel": "paged_attention_decode_mixed",
                     "achieved": round(dec_bytes / dec_s / 1e9, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dec_bytes / dec_s / 1e9 / PEAK_GBPS, 4),
                     "traffic": None},
    }
    if args.cpu_baseline == "on":
        import oracle
        log("timing the CPU oracle ...")
        host_append(c)
        threads = oracle.max_threads()

        def run(n):
            t = time.perf_counter()
            r = oracle.paged_decode_mixed(c.query, c.k_cache, c.v_cache, c.block_tables,
                                          c.seq_lens, mc.seq_bs, q_dtype=c.q_dtype,
                                          cache_dtype=c.cache_dtype, scale=c.scale,
                                          rows=np.arange(n * c.Hq, dtype=np.int32),
                                          threads=threads)
            return time.perf_counter() - t, r

        n = min(8, c.S)
        t, ref = run(n)
        if t < 5.0 and n < c.S:           # size the sample to about 20 s
            per_tok = t / max(int(c.seq_lens[:n].sum()), 1)
            cum = np.cumsum(c.seq_lens.astype(np.int64))
            n = int(min(c.S, max(n, np.searchsorted(cum, 20.0 / per_tok) + 1)))
            t, ref = run(n)
        sub = c.copy()
        sub.S, sub.seq_lens, sub.slot_mapping = n, c.seq_lens[:n], c.slot_mapping[:0]
        nbytes = decode_bytes(sub, 0)["decode_kernel"]
        res["cpu_baseline"] = {
            "value": round(nbytes / t / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle", "tokens_per_s_per_layer": round(n / t, 2), "seconds": round(t, 3),
            "sample": "decode of the first %d of %d sequences (%d tokens, all %d query heads), "
                      "gather by each sequence's block size + fp64 softmax attention, OpenMP "
                      "over rows" % (n, c.S, int(c.seq_lens[:n].sum()), c.Hq)}
        res["cpu_baseline"].update(host_cpus())
        gpu = out[:n].float().cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(gpu - ref[:n])))
        tol = TOL[c.cache_dtype]
        res["max_abs_err_vs_oracle"] = {
            "max_abs_err": err, "tol": tol, "within_tol": bool(err <= tol), "rows": n * c.Hq,
            "of_rows": c.S * c.Hq,
            "sample": "the oracle's rows above against the output of the last step"}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3-8b-gqa",
                    choices=list(workloads.WORKLOADS) + list(MULTI_WORKLOADS) +
                    ["swap", "mixed-bs"])
    ap.add_argument("--bs", type=int, default=16, help="block size of shared-prefix-fp8")
    ap.add_argument("--algo", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition", type=int, default=None,
                    help="split-K partition size: 0 one pass, P > 0 fixed partitions, "
                         "-1 the balanced split (default: per workload, DEFAULT_PARTITION)")
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct KV pools rotated across steps")
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--graphs", default="on", choices=["on", "off"],
                    help="time the steps as HIP graph replays (per-kernel times stay eager)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter scaling)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE "
                         "and a WRITE_SIZE run (each with --copy-calib-mib) into the "
                         "workload's entry of profiles/decode_traffic.json")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step "
              "in this library (each GPU owns its sequences' blocks); run with --gpus 1.",
              file=sys.stderr)
        return 2

    if args.workload in MULTI_WORKLOADS:
        return bench_multi(args)
    if args.workload == "swap":
        return bench_swap(args)
    if args.workload == "mixed-bs":
        return bench_mixed(args)

    import torch
    import paged_kv_cache_361_amd as pkv

    torch.cuda.set_device(0)
    log("generating workload %s ..." % args.workload)
    t0 = time.perf_counter()
    c, P = make_workload(args)
    log("generated in %.1fs: %d seqs, %d tokens, pool %d blocks" %
        (time.perf_counter() - t0, c.S, int(c.seq_lens.sum()), c.NB))

    def dev(a, d):
        if d == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    query = dev(c.query, c.q_dtype)
    tables = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(c.seq_lens).cuda()
    new_k = dev(c.new_key, c.src_dtype)
    new_v = dev(c.new_value, c.src_dtype)
    slots = torch.from_numpy(c.slot_mapping).cuda()
    k0, v0 = dev(c.k_cache, c.cache_dtype), dev(c.v_cache, c.cache_dtype)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(1, args.layers) - 1)]
    out = torch.empty(c.S, c.Hq, c.D, dtype=TD[c.q_dtype], device="cuda")
    ws = pkv.allocate_workspace(c.S, c.Hq, c.Hkv, c.D, c.max_seq_len, P)
    stream = torch.cuda.current_stream()

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step(i, ev=None):
        kc, vc = layers[i % len(layers)]
        if c.slot_mapping.size:
            if ev: ev[0].record(stream)
            pkv.reshape_and_cache(new_k, new_v, kc, vc, slots, k_scale=c.k_scale,
                                  v_scale=c.v_scale)
        if ev: ev[1].record(stream)
        pkv.paged_attention_decode(out, query, kc, vc, tables, lens, scale=c.scale,
                                   max_seq_len=c.max_seq_len, k_scale=c.k_scale,
                                   v_scale=c.v_scale, partition_size=P, workspace=ws,
                                   algo=args.algo)
        if ev: ev[2].record(stream)
        if P != 0:
            pkv.paged_attention_reduce(out, ws, lens, num_kv_heads=c.Hkv,
                                       max_seq_len=c.max_seq_len, partition_size=P)
        if ev: ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)

    K = args.steps
    # per-kernel durations: HIP events on the stream the kernels run on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t_eager = time.perf_counter() - t_start
    log("eager: %d steps in %.3fs" % (K, t_eager))

    # The timed steps: each KV pool's step (append, decode, reduce) captured
    # once in a HIP graph and replayed, as a serving loop runs it; the
    # calls hold no memset and the balanced counter is handed back by the
    # reduce, so replays are exact (checked below against an eager step).
    mode, graph_check = "eager", None
    t_total = t_eager
    if args.graphs == "on":
        try:
            graphs = []
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for li in range(len(layers)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        step(li)
                    graphs.append(g)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            for i in range(args.warmup):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for i in range(K):
                graphs[(args.warmup + i) % len(graphs)].replay()
            torch.cuda.synchronize()
            t_total = time.perf_counter() - t_start
            mode = "hip-graph"
            # a replay against an eager step on the same pool
            graphs[0].replay()
            torch.cuda.synchronize()
            replayed = out.clone()
            step(0)
            torch.cuda.synchronize()
            graph_check = bool(torch.equal(replayed.view(torch.uint8), out.view(torch.uint8)))
            log("graph replays: %d steps in %.3fs (check %s)" % (K, t_total, graph_check))
        except Exception as e:                      # report, and keep the eager timing
            log("graph capture failed (%s); timing eager steps" % e)
            mode, t_total = "eager (graph capture failed)", t_eager

    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    red_ms = np.array([e[2].elapsed_time(e[3]) for e in evs]) if P != 0 else np.zeros(K)
    app_ms = (np.array([e[0].elapsed_time(e[1]) for e in evs]) if c.slot_mapping.size
              else np.zeros(K))
    nW = 0
    if P < 0:     # the grid size the library chose, from the workspace header
        nW = int(ws[:16].cpu().numpy().view(np.int32)[1])
    nb = decode_bytes(c, P, nW)
    step_s = t_total / K
    attn_s = float(np.mean(dec_ms + red_ms)) / 1e3
    dec_s = float(np.mean(dec_ms)) / 1e3
    value = nb["step"] / step_s / 1e12
    achieved = nb["decode_kernel"] / dec_s / 1e9
    wl = WORKLOAD_NAMES[args.workload]
    if args.workload == "shared-prefix-fp8":
        wl += ", bs %d" % c.bs
    traffic = traffic_from_profiles(traffic_key(args, c.bs), nb["decode_kernel"])
    res = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "f32": "f32"}[c.q_dtype]
                 + ("/fp8-kv" if c.cache_dtype == "fp8" else ""),
        "data": "synthetic",
        "config": {"workload": wl, "seqs": c.S, "tokens": int(c.seq_lens.sum()),
                   "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": c.D, "block_size": c.bs,
                   "partition_size": P if P >= 0 else "balanced", "algo": args.algo,
                   "kv_pools_rotated": len(layers)},
        "pct_of_peak": round(100 * value * 1e3 / PEAK_GBPS, 2),
        "tokens_per_s_per_layer": round(c.S / attn_s, 1),
        "tokens_per_s_per_layer_with_append": round(c.S / step_s, 1),
        "decode_us": round(dec_s * 1e6, 2),
        "decode_us_p10_p90": [round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                              round(float(np.percentile(dec_ms, 90)) * 1e3, 2)],
        "reduce_us": round(float(np.mean(red_ms)) * 1e3, 2),
        "balanced_grid_waves": nW if P < 0 else None,
        "append_us": round(float(np.mean(app_ms)) * 1e3, 2),
        "step_mode": mode,
        "graph_replay_exact": graph_check,
        "eager_ms_per_step": round(t_eager / K * 1e3, 4),
        "bytes_per_step": nb,
        "roofline": {"bound": "hbm", "kernel": "paged_attention_decode",
                     "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic},
    }
    kv_u = unique_kv_bytes(c)
    if kv_u != nb["kv"]:
        # shared prefix blocks: a launch need fetch each distinct slot once
        res["kv_unique_bytes"] = kv_u
        res["decode_TBps_on_unique_kv"] = round(kv_u / dec_s / 1e12, 4)
    if args.cpu_baseline == "on":
        log("timing the CPU oracle ...")
        host_append(c)
        gpu = out.float().cpu().numpy().astype(np.float64)
        res["cpu_baseline"], res["max_abs_err_vs_oracle"] = cpu_baseline(c, gpu)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
