#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

A step is one pass of the whole hot path over one batch: the host-built slot
mapping is already resident (fixed device buffer), the scatter writes the
step's new K/V through it, and paged decode attention reads every sequence's
context through its block table.  Inputs are seeded synthetic data resident
in HBM before timing starts.

Default workload: Llama-3-8B-shaped decode layer (64 sequences, 32 query /
8 KV heads, head_dim 128, block 16, context lengths U[512, 4096], block tables
from a shuffled free list over a pool of 1.25x the blocks needed, bf16).

The pool holds ``--layers`` layers (default 4) and step i runs on layer
i mod LAYERS, as a model's decode step runs its layers one after another: no
call re-reads KV that the previous call left in L2 or the 256 MB MALL.  The
same call repeated on one layer (``same_layer``) and with the caches flushed
before it (``cold``) are reported beside it.

The K timed steps are replays of one captured HIP graph holding the step's
launches (how a serving loop submits its decode step), in two forms: scatter
+ attention, and, where every sequence writes one token at position L_i - 1,
those writes folded into the attention call (paged_attention_decode_append;
other writes such as a prefill chunk still go through reshape_and_cache).
Both leave bitwise the same pool and output (checked in the run); both times
are reported and the faster is the headline.  ``--no-fuse`` keeps the two
calls, ``--eager`` times eager launches instead.  The attention call's own duration, from events
around each of K eager calls, gives the roofline figure.

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention achieved HBM GB/s (% of peak) + decode tokens/sec/layer"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCES = ["paged_kv_cache_num_amd/csrc/decode.hip", "paged_kv_cache_num_amd/csrc/decode_mfma.hip",
                  "paged_kv_cache_num_amd/csrc/device_common.hpp", "paged_kv_cache_num_amd/csrc/split.hpp",
                  "paged_kv_cache_num_amd/csrc/fp8.hpp", "paged_kv_cache_num_amd/csrc/table_index.hpp",
                  "paged_kv_cache_num_amd/csrc/fp8_rows.hpp"]

WORKLOADS = {
    "C1": "tiny fp32 paged decode: 4 sequences, lengths {17,33,100,200}, 8 query / 2 KV heads, head_dim 64, block 16, 64-block pool",
    "C2": "Llama-3-8B-shaped decode layer: 64 sequences, 32 query / 8 KV heads, head_dim 128, block 16, lengths U[512,4096], shuffled free-list tables, pool 1.25x, bf16",
    "C3": "70B-class GQA decode layer: 256 sequences, 64 query / 8 KV heads, head_dim 128, block 16, lognormal lengths (median 1024, sigma 1, clip [16,8192]), permuted blocks, plus a 2048-token prefill-chunk scatter, bf16",
    "C4": "prefix-sharing decode: 128 sequences sharing 128 blocks (2048-token prefix) plus private suffixes U[64,512], 32 query / 8 KV heads, head_dim 128, bf16",
    "C5": "long-context split decode: 8 sequences, lengths U[32768,131072], 32 query / 8 KV heads, head_dim 128, partitions of 512 tokens, fragmented pool, bf16",
    "C3TP8": "one GPU's share of the 70B-class GQA decode layer under tensor parallelism over KV heads at TP 8: the same 256 sequences, lengths and 2048-token prefill chunk, 8 query / 1 KV head, head_dim 128, block 16, bf16",
}
# 0 = balanced split across the GPU; C5 names 512-token partitions explicitly
DEFAULT_PARTITION = {"C1": 0, "C2": 0, "C3": 0, "C4": 0, "C5": 512, "C3TP8": 0}


def kernel_sha() -> str:
    """sha256 of the decode sources' code: comments and blank space removed, so a
    comment edit does not invalidate the recorded traffic while any code change does."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def algorithmic_bytes(wl, fp8: bool = False):
    """Bytes the step must move at minimum.

    attention: every distinct (physical block, token) K and V row once, plus q
    in and the output out, plus the table entries and lengths read;
    scatter: new K/V rows read and written, plus the slot mapping.
    Split-partition partial states are not counted.
    FP8 pools: rows are one byte per element plus, per distinct block, its K
    and V scales (8 bytes per KV head); the scatter reads bf16 rows, writes
    codes and reads each written row's two scales.
    """
    import numpy as np
    B, Hkv, D, e = wl.block_size, wl.num_kv_heads, wl.head_dim, wl.elem_bytes
    e_pool = 1 if fp8 else e
    row = 2 * Hkv * D * e_pool                 # K and V of one token, all KV heads
    used = {}
    for i, L in enumerate(wl.context_lens):
        L = int(L)
        nb = -(-L // B)
        for b in range(nb):
            phys = int(wl.block_tables[i, b])
            tokens = min(B, L - b * B)
            used[phys] = max(used.get(phys, 0), tokens)
    kv_unique = sum(used.values()) * row + (len(used) * 8 * Hkv if fp8 else 0)
    kv_logical = int(np.sum(wl.context_lens)) * row
    nblk = int(sum(-(-int(L) // B) for L in wl.context_lens))
    qo = 2 * wl.num_seqs * wl.num_q_heads * D * e
    attn = kv_unique + qo + 4 * nblk + 4 * wl.num_seqs
    T = wl.num_write_tokens
    if fp8:
        scatter = T * 2 * Hkv * D * (e + 1) + 8 * T + 8 * Hkv * T
    else:
        scatter = 2 * T * row + 8 * T
    return dict(attn=attn, attn_logical=kv_logical + qo + 4 * nblk + 4 * wl.num_seqs, scatter=scatter,
                kv_unique=kv_unique, kv_logical=kv_logical, blocks=nblk)


def traffic_key(config: str, partition: int, block_size: int = 16, kv_dtype: str = "bf16") -> str:
    return (f"{config}/p{partition}" + ("" if block_size == 16 else f"/B{block_size}")
            + ("" if kv_dtype == "bf16" else f"/{kv_dtype}"))


def traffic_for(config: str, partition: int, block_size: int = 16, kv_dtype: str = "bf16"):
    """HBM bytes per decode launch from committed counter runs, or None if stale/absent."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(traffic_key(config, partition, block_size, kv_dtype))
    if not entry or entry.get("kernel_source_sha256") != kernel_sha():
        return None
    return entry.get("traffic_bytes_per_launch")


ATTN_KERNEL_MARKERS = ("decode_bf16_streamk_kernel", "streamk_fixup_kernel", "decode_bf16_mfma_kernel",
                       "decode_partitions_kernel", "decode_kernel", "reduce_kernel")


def record_traffic(fetch_csv: str, write_csv: str, copy_mib: int, config: str, partition: int,
                   command: str, block_size: int = 16, kv_dtype: str = "bf16") -> dict:
    """HBM bytes per attention call from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE).

    Each counter is scaled by what it reads for the copy probe of copy_mib MiB
    (known to read and write exactly that many bytes), then the kernels of one
    attention call (decode + merge) are summed, averaged over dispatches.
    """
    import csv
    import statistics

    def per_kernel(path, counter):
        out = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return out

    known = float(copy_mib << 20)
    res = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        k = per_kernel(path, counter)
        copy = [v for name, vs in k.items() if "copy_kernel" in name for v in vs]
        if not copy:
            raise SystemExit(f"no copy-probe dispatch in {path}")
        factor = known / (statistics.median(copy) * 1024.0)
        attn = {name: statistics.mean(vs) for name, vs in k.items()
                if "kvp::" in name and any(m in name for m in ATTN_KERNEL_MARKERS)}
        res[counter] = {"factor": round(factor, 4),
                        "kib_per_dispatch": {n.replace("(anonymous namespace)::", "").split("(")[0][-60:]: round(v, 1)
                                             for n, v in attn.items()},
                        "bytes_per_call": sum(attn.values()) * 1024.0 * factor}
    entry = {"traffic_bytes_per_launch": round(res["FETCH_SIZE"]["bytes_per_call"] + res["WRITE_SIZE"]["bytes_per_call"]),
             "fetch_bytes_per_launch": round(res["FETCH_SIZE"]["bytes_per_call"]),
             "write_bytes_per_launch": round(res["WRITE_SIZE"]["bytes_per_call"]),
             "fetch_factor": res["FETCH_SIZE"]["factor"], "write_factor": res["WRITE_SIZE"]["factor"],
             "fetch_kib_per_dispatch": res["FETCH_SIZE"]["kib_per_dispatch"],
             "write_kib_per_dispatch": res["WRITE_SIZE"]["kib_per_dispatch"],
             "kernel_source_sha256": kernel_sha(), "command": command}
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[traffic_key(config, partition, block_size, kv_dtype)] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    return entry


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    k = (len(xs) - 1) * q
    lo, hi = int(math.floor(k)), int(math.ceil(k))
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


CPU_SAMPLE_SECONDS = 10.0   # the oracle's sample: repeated until about this much CPU work is timed


def cpu_baseline(wl, bytes_total, nbytes=None):
    """The oracle's whole step (oracle.run_step's three calls: slot mapping,
    scatter, fp64 attention), repeated for about CPU_SAMPLE_SECONDS; the
    write path (slot mapping + scatter) and the attention are also timed
    apart.  The oracle's scatter returns new copies of the pools, so its
    time includes copying them."""
    import oracle
    threads = oracle.default_threads()
    scale = 1.0 / math.sqrt(wl.head_dim)
    reps, total, t_write, t_attn = 0, 0.0, 0.0, 0.0
    while total < CPU_SAMPLE_SECONDS and reps < 1000:
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(wl.all_tables(), wl.block_size, wl.num_blocks, wl.write_seq, wl.write_start,
                                    wl.write_count)
        kp, vp = oracle.scatter(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, slots)
        t1 = time.perf_counter()
        oracle.paged_attention(wl.q, kp, vp, wl.dtype, wl.block_tables, wl.context_lens, scale, threads)
        t2 = time.perf_counter()
        t_write += t1 - t0
        t_attn += t2 - t1
        total += t2 - t0
        reps += 1
        del kp, vp
    dt = total / reps
    res = {"value": round(bytes_total / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds": round(dt, 4), "repeats": reps, "seconds_total": round(total, 2),
           "sample": f"the whole {wl.name} step (all {wl.num_seqs} sequences): slot mapping, scatter and fp64 "
                     f"attention, run {reps} times (mean per step)",
           "tokens_per_s_per_layer": round(wl.num_seqs / dt, 3),
           "write_path_seconds": round(t_write / reps, 5), "attention_seconds": round(t_attn / reps, 5)}
    if nbytes is not None:
        res["write_path_gbps"] = round(nbytes["scatter"] / (t_write / reps) / 1e9, 4)
        res["attention_gbps"] = round(nbytes["attn"] / (t_attn / reps) / 1e9, 4)
        res["write_path_note"] = ("slot mapping and scatter; the oracle's scatter copies both pools first "
                                  "(it returns new arrays), which dominates its time")
    return res


def cpu_baseline_fp8(wl, state, nseq: int = 16):
    """The FP8 oracle (oracle/fp8.py: scatter with block scales, fp64 attention
    over the dequantized pool) on the first ``nseq`` sequences of the batch,
    their blocks gathered into a pool of their own first (outside the timing)."""
    import dataclasses

    import numpy as np

    import oracle
    import oracle.fp8 as ofp8
    B = wl.block_size
    S = min(nseq, wl.num_seqs)
    lens = wl.context_lens[:S]
    rows = [wl.block_tables[i, :-(-int(L) // B)] for i, L in enumerate(lens)]
    blocks = np.unique(np.concatenate(rows)) if rows else np.zeros(0, dtype=np.int32)
    where = {int(b): j for j, b in enumerate(blocks)}
    tables = np.zeros((S, max(1, max(len(r) for r in rows))), dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = [where[int(b)] for b in r]
    sub_state = tuple(a[blocks] for a in state)
    # the sample's decode writes: one row per sequence at L - 1
    keep = [k for k in range(len(wl.write_seq)) if wl.write_seq[k] < S and wl.write_count[k] == 1]
    row0 = np.concatenate([[0], np.cumsum(wl.write_count)])
    tok = np.array([row0[k] for k in keep], dtype=np.int64)
    sub = dataclasses.replace(wl, context_lens=lens, block_tables=tables, extra_tables=tables[:0],
                              write_seq=wl.write_seq[keep], write_start=wl.write_start[keep],
                              write_count=wl.write_count[keep], q=wl.q[:S], k_new=wl.k_new[tok],
                              v_new=wl.v_new[tok], k_pool=wl.k_pool[blocks], v_pool=wl.v_pool[blocks],
                              num_blocks=int(blocks.size))
    scale = 1.0 / math.sqrt(wl.head_dim)
    from threadpoolctl import threadpool_limits
    reps, total = 0, 0.0
    with threadpool_limits(1):      # numpy's BLAS on one thread: the figure is per core
        while total < CPU_SAMPLE_SECONDS and reps < 1000:
            t0 = time.perf_counter()
            slots = oracle.slot_mapping(sub.block_tables, B, sub.num_blocks, sub.write_seq, sub.write_start,
                                        sub.write_count)
            kc, vc, ks, vs = ofp8.scatter(*sub_state, sub.k_new, sub.v_new, slots, B)
            ofp8.paged_attention(sub.q, kc, vc, ks, vs, sub.block_tables, sub.context_lens, scale)
            total += time.perf_counter() - t0
            reps += 1
    dt = total / reps
    nb = algorithmic_bytes(sub, fp8=True)
    return {"value": round((nb["attn"] + nb["scatter"]) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 3), "repeats": reps, "seconds_total": round(total, 2),
            "sample": f"the first {S} of {wl.num_seqs} sequences of the {wl.name} step with their blocks: "
                      f"FP8 slot mapping, scatter with block scales and fp64 attention (numpy), run {reps} "
                      "times (mean per step)",
            "tokens_per_s_per_layer": round(S / dt, 3)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C2", choices=sorted(WORKLOADS))
    ap.add_argument("--partition", type=int, default=None, help="tokens per partition (0 = single pass)")
    ap.add_argument("--variant", default="spec")
    ap.add_argument("--block-size", type=int, default=None,
                    help="tokens per block (default: the workload's 16); bf16 and FP8 pools with head_dim 128 take 8..128")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="pool storage: the workload's bf16, or E4M3 codes with per-(block, KV head) scales "
                         "(q, new rows and outputs stay bf16)")
    ap.add_argument("--layers", type=int, default=4,
                    help="layers in the pool; step i reads and writes layer i mod LAYERS, as a model's layers "
                         "follow each other, so no call finds its own KV left in the caches by the previous one "
                         "(1: every step on the same layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-flushed timing pass")
    ap.add_argument("--no-identity", action="store_true",
                    help="skip timing the same batch with contiguous (identity-like) block tables")
    ap.add_argument("--no-copy-blocks", action="store_true", help="skip timing copy-on-write block copies")
    ap.add_argument("--no-shared", action="store_true",
                    help="batches with a shared prompt: time only the plain call, not paged_attention_decode_shared")
    ap.add_argument("--no-swap", action="store_true", help="skip timing swap of the batch's blocks to host and back")
    ap.add_argument("--table-walk-probe", type=int, default=0, metavar="N",
                    help="also run the table-walk probe N times in each workgroup ordering (for counter runs)")
    ap.add_argument("--no-fuse", action="store_true",
                    help="time the step as scatter + attention only (no paged_attention_decode_append form)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step from eager launches only (default: replays of a captured HIP graph)")
    ap.add_argument("--probe-copy-mib", type=int, default=0,
                    help="also run the copy probe once on buffers of this size (counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a run made with "
                         "--probe-copy-mib into the traffic record used by the roofline line, and exit")
    ap.add_argument("--record-command", default="", help="command line stored with --record-traffic")
    ap.add_argument("--attn-only", action="store_true",
                    help="run only the headline attention call (warmup + steps, layer after layer; the "
                         "shared-prefix call for a batch with a shared prompt) and exit: the run that "
                         "hardware counters are collected over for --record-traffic")
    args = ap.parse_args(argv)

    if args.record_traffic:
        part = DEFAULT_PARTITION[args.config] if args.partition is None else args.partition
        entry = record_traffic(args.record_traffic[0], args.record_traffic[1], args.probe_copy_mib or 1024,
                               args.config, part, args.record_command, args.block_size or 16, args.kv_dtype)
        print(json.dumps(entry))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the hot path on one GPU only; --gpus must be 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import kvgen
    from paged_kv_cache_num_amd import DecodeStep, probe_copy, probe_read

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    part = DEFAULT_PARTITION[args.config] if args.partition is None else args.partition

    print(f"bench: generating {args.config} ({args.variant})", file=sys.stderr, flush=True)
    wl = kvgen.make_workload(args.config, variant=args.variant, block_size=args.block_size)
    fp8 = args.kv_dtype == "fp8"
    if fp8 and (wl.dtype != "bf16" or wl.head_dim != 128):
        print("bench.py: FP8 pools are built for bf16 workloads with head_dim 128", file=sys.stderr)
        return 2

    def fp8_state(w):
        # codes and block scales drawn directly; the largest code stands for about 3 sigma of the
        # workload's values (N(0, 1/128) for the spec variant)
        sigma = 1.0 / math.sqrt(w.head_dim) if args.variant == "spec" else 1.0
        return kvgen.fp8_pool_state(w, seed=w.info.get("seed") or 0, largest=3.0 * sigma) if fp8 else None

    nbytes = algorithmic_bytes(wl, fp8=fp8)
    state = fp8_state(wl)
    NL = max(1, args.layers)
    step = DecodeStep.from_workload(wl, partition_size=part, fp8_pool=state, num_layers=NL)
    torch.cuda.synchronize()

    # achievable HBM read rate on this machine: a plain 16-byte-load read of 2 GiB (larger than the caches)
    big = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    sink = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    read_us = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        probe_read(big, sink)
        e1.record()
        e1.synchronize()
        read_us.append(e0.elapsed_time(e1) * 1e3)
    read_gbps = big.numel() / (min(read_us[1:]) * 1e-6) / 1e9
    print(f"bench: read probe 2 GiB: {read_gbps:.0f} GB/s", file=sys.stderr, flush=True)

    if args.probe_copy_mib:
        n = args.probe_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe_copy(dst, src)      # first touch
        e0.record()
        probe_copy(dst, src)
        e1.record()
        torch.cuda.synchronize()
        copy_us = e0.elapsed_time(e1) * 1e3
        print(f"bench: copy probe {args.probe_copy_mib} MiB: {copy_us:.1f} us, "
              f"{2 * n / copy_us / 1e3:.1f} GB/s (read+write)", file=sys.stderr, flush=True)
        del src, dst

    sb = int(wl.info.get("shared_prefix_blocks") or 0)
    shared_ok = bool(sb) and not fp8 and part == 0 and wl.dtype == "bf16" and not args.no_shared
    if args.attn_only:
        call = DecodeStep.from_workload(wl, partition_size=0, shared_blocks=sb, num_layers=NL) if shared_ok else step
        n = args.warmup + args.steps
        for i in range(n):
            call.layer = i % NL
            call.attend()
        torch.cuda.synchronize()
        print(f"bench: {n} {'shared-prefix' if shared_ok else 'plain'} attention calls", file=sys.stderr, flush=True)
        return 0

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step.layer = i % NL
        step.run()
    torch.cuda.synchronize()

    # timed region: K whole steps, step i on layer i mod NL, events on the stream the kernels run on
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step.layer = i % NL
        a, b, c = ev[i]
        a.record()
        step.scatter()
        b.record()
        step.attend()
        c.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    scatter_us = [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in range(K)]
    attn_us = [ev[i][1].elapsed_time(ev[i][2]) * 1e3 for i in range(K)]
    print(f"bench: timed {K} steps, {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    attn_mean = sum(attn_us) / K
    achieved = nbytes["attn"] / (attn_mean * 1e-6) / 1e9
    step_bytes = nbytes["attn"] + nbytes["scatter"]
    eager_ms_per_step = ms_per_step

    # The same K steps replayed from one captured HIP graph (how a serving loop
    # submits its decode step), in two forms: scatter + attention, and the
    # decode appends folded into the attention call (paged_attention_decode_append;
    # writes that are not decode appends, such as a prefill chunk, still go
    # through reshape_and_cache first).  The headline is the fused form when the
    # batch allows it.
    launch = "eager"
    graph_ms = {}
    graph_gpu_us = {}
    if not args.eager:
        forms = [False] + ([True] if step.can_fuse and not args.no_fuse else [])
        for fused in forms:
            graphs = []
            for li in range(NL):        # one captured step per layer, replayed in layer order
                step.layer = li
                graphs.append(step.capture(fused=fused))
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(K):
                graphs[i % NL].replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            graph_ms[fused] = (t1 - t0) * 1e3 / K
            # the same replays one at a time between events on the stream: the GPU's own time for one
            # replayed step, without the host's submission of the next one
            g_us = []
            for i in range(min(K, 50)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                graphs[i % NL].replay()
                b.record()
                b.synchronize()
                g_us.append(a.elapsed_time(b) * 1e3)
            graph_gpu_us[fused] = percentile(g_us, 0.5)
            del graphs
            print(f"bench: timed {K} graph replays ({'fused append' if fused else 'scatter + attention'}), "
                  f"{graph_ms[fused] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        # both forms leave bitwise the same pool and output (checked below); the
        # headline is the faster one on this batch
        fused_on = True in graph_ms and graph_ms[True] < graph_ms[False]
        ms_per_step = graph_ms[fused_on]
        fused_name = ("fused append + other rows (paged_attention_decode_step)" if step.num_other_tokens
                      else "fused append (paged_attention_decode_append)")
        launch = f"hip_graph, {fused_name}" if fused_on else "hip_graph, scatter + attention"
        # the fused form must leave the same pool and output as the two-call form
        step.layer = 0
        step.run()
        torch.cuda.synchronize()
        ref_out = step.out.clone()
        if True in graph_ms:
            step.run_fused()
            torch.cuda.synchronize()
            assert torch.equal(step.out.view(torch.int16) if step.out.dtype == torch.bfloat16 else step.out,
                               ref_out.view(torch.int16) if ref_out.dtype == torch.bfloat16 else ref_out), \
                "fused step output differs from scatter + attention"

    # A batch whose sequences share a prompt (the prefix-sharing workload: its
    # block manager knows the 128 shared blocks): the same step with
    # paged_attention_decode_shared, checked against the plain call's output
    # and timed the same ways; the faster form is the headline.
    shared = None
    head_step = step
    roofline_kernel = "paged_attention_decode"
    if shared_ok:
        sstep = DecodeStep.from_workload(wl, partition_size=0, shared_blocks=sb, num_layers=NL)
        for i in range(args.warmup):
            sstep.layer = i % NL
            sstep.run()
        step.layer = sstep.layer = 0
        step.run()
        sstep.run()
        torch.cuda.synchronize()
        diff = float((sstep.out.float() - step.out.float()).abs().max())
        assert diff <= 2e-2, f"shared-prefix call differs from the plain call by {diff}"
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            sstep.layer = i % NL
            sstep.scatter()
            sev[i][0].record()
            sstep.attend()
            sev[i][1].record()
        torch.cuda.synchronize()
        sh_us = [a.elapsed_time(b) * 1e3 for a, b in sev]
        sh_mean = sum(sh_us) / K
        sh_graph_ms = None
        if not args.eager:
            graphs = []
            for li in range(NL):
                sstep.layer = li
                graphs.append(sstep.capture())
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(K):
                graphs[i % NL].replay()
            torch.cuda.synchronize()
            sh_graph_ms = (time.perf_counter() - t0) * 1e3 / K
            del graphs
        shared = {"shared_blocks": sb, "attn_us_mean": round(sh_mean, 2),
                  "attn_us_p50": round(percentile(sh_us, 0.5), 2),
                  "achieved_gbps": round(nbytes["attn"] / (sh_mean * 1e-6) / 1e9, 1),
                  "frac": round(nbytes["attn"] / (sh_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                  "graph_ms_per_step": round(sh_graph_ms, 5) if sh_graph_ms is not None else None,
                  "plain_attn_us_mean": round(attn_mean, 2), "plain_ms_per_step": round(ms_per_step, 5),
                  "max_abs_diff_vs_plain": diff}
        print(f"bench: shared-prefix call {sh_mean:.1f} us (plain {attn_mean:.1f} us)", file=sys.stderr, flush=True)
        faster = sh_graph_ms < ms_per_step if sh_graph_ms is not None else sh_mean < attn_mean
        if faster:
            if sh_graph_ms is not None:
                ms_per_step = sh_graph_ms
                launch = "hip_graph, scatter + shared-prefix attention"
            attn_us, attn_mean = sh_us, sh_mean
            achieved = nbytes["attn"] / (attn_mean * 1e-6) / 1e9
            head_step = sstep
            roofline_kernel = "paged_attention_decode_shared"
        else:
            del sstep
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the same attention call K times on one layer, back to back: what part of
    # each call the caches (L2, 256 MB MALL) serve when it re-reads the KV the
    # previous call read (reported beside the layer-rotating figure)
    same_layer = None
    if NL > 1:
        head_step.layer = 0
        sl_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            sl_ev[i][0].record()
            head_step.attend()
            sl_ev[i][1].record()
        torch.cuda.synchronize()
        sl_us = [a.elapsed_time(b) * 1e3 for a, b in sl_ev]
        sl_mean = sum(sl_us) / K
        same_layer = {"attn_us_mean": round(sl_mean, 2), "attn_us_p50": round(percentile(sl_us, 0.5), 2),
                      "achieved_gbps": round(nbytes["attn"] / (sl_mean * 1e-6) / 1e9, 1),
                      "frac": round(nbytes["attn"] / (sl_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}

    cold = None
    if not args.no_cold:
        # evict L2 and the 256 MB MALL before every attention call by reading 2 GiB (outside its
        # events); a read leaves no dirty lines whose write-back would be charged to the kernel
        cold_us = []
        head_step.layer = 0
        for _ in range(min(K, 30)):
            probe_read(big, sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            head_step.attend()
            b.record()
            b.synchronize()
            cold_us.append(a.elapsed_time(b) * 1e3)
        cm = sum(cold_us) / len(cold_us)
        cold = {"attn_us_mean": round(cm, 2), "attn_us_p50": round(percentile(cold_us, 0.5), 2),
                "achieved_gbps": round(nbytes["attn"] / (cm * 1e-6) / 1e9, 1),
                "frac": round(nbytes["attn"] / (cm * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    del big

    # The same batch with every sequence's blocks laid out back to back
    # (identity-like tables, the dense layout of a contiguous cache): the
    # ratio is what the indirection costs.
    identity = None
    if not args.no_identity:
        dense_wl = kvgen.privatize_blocks(wl, contiguous=True)
        dense = DecodeStep.from_workload(dense_wl, partition_size=part, fp8_pool=fp8_state(dense_wl), num_layers=NL)
        for i in range(args.warmup):
            dense.layer = i % NL
            dense.attend()
        torch.cuda.synchronize()
        dense_us = []
        for i in range(K):
            dense.layer = i % NL
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dense.attend()
            b.record()
            b.synchronize()
            dense_us.append(a.elapsed_time(b) * 1e3)
        # the paged calls timed the same way (one call per synchronisation)
        paged_us = []
        for i in range(K):
            step.layer = i % NL
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step.attend()
            b.record()
            b.synchronize()
            paged_us.append(a.elapsed_time(b) * 1e3)
        dp, dd = percentile(paged_us, 0.5), percentile(dense_us, 0.5)
        identity = {"paged_attn_us_p50": round(dp, 2), "identity_attn_us_p50": round(dd, 2),
                    "paged_over_identity": round(dp / dd, 4)}
        del dense
        torch.cuda.synchronize()

    # Copy-on-write block copies (kv_copy_blocks) on a pool of the same block
    # shape: 512 disjoint (src, dst) pairs, bytes = read + write of K and V.
    copy = None
    if not args.no_copy_blocks:
        from paged_kv_cache_num_amd import KVPool
        npairs = 512
        cpool = KVPool.allocate(num_layers=1, num_blocks=2 * npairs, block_size=wl.block_size,
                                num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
                                dtype="fp8" if fp8 else (torch.float32 if wl.dtype == "f32" else torch.bfloat16),
                                device="cuda")
        cpool.k.fill_(1)
        cpool.v.fill_(2)
        perm = torch.randperm(2 * npairs, generator=torch.Generator().manual_seed(0)).to(torch.int32)
        pairs = perm.view(npairs, 2).contiguous().cuda()
        cus = []
        for i in range(args.warmup + K):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            cpool.copy_blocks(pairs)
            b.record()
            b.synchronize()
            if i >= args.warmup:
                cus.append(a.elapsed_time(b) * 1e3)
        block_bytes = wl.num_kv_heads * wl.block_size * wl.head_dim * (1 if fp8 else (4 if wl.dtype == "f32" else 2))
        if fp8:
            block_bytes += 4 * wl.num_kv_heads          # the block's scale per KV head
        moved = npairs * 2 * block_bytes * 2
        cp50 = percentile(cus, 0.5)
        copy = {"pairs": npairs, "bytes_moved": moved, "us_p50": round(cp50, 2),
                "gbps": round(moved / (cp50 * 1e-6) / 1e9, 1)}
        del cpool, pairs
        torch.cuda.synchronize()

    # Swap (kv_swap_out / kv_swap_in): every block the batch's tables name, out
    # to pinned host memory and back into the same blocks; bytes = the pool
    # bytes of those blocks each way.  Reference: one DMA copy of the same
    # byte count between a contiguous device buffer and pinned host memory.
    swap = None
    if not args.no_swap:
        nb = [-(-int(L) // wl.block_size) for L in wl.context_lens]
        blist = np.unique(np.concatenate([wl.block_tables[i, :n] for i, n in enumerate(nb)])).astype(np.int32)
        blocks_dev = torch.from_numpy(blist).cuda()
        nbytes_swap = step.pool.swap_bytes(blist.size)
        host = torch.empty(nbytes_swap, dtype=torch.uint8).pin_memory()
        dev = torch.empty(nbytes_swap, dtype=torch.uint8, device="cuda")
        times = {"out": [], "in": [], "dma_d2h": [], "dma_h2d": []}
        for i in range(3 + 10):
            for key, fn in (("out", lambda: step.pool.swap_out(blocks_dev, host)),
                            ("in", lambda: step.pool.swap_in(blocks_dev, host)),
                            ("dma_d2h", lambda: host.copy_(dev, non_blocking=True)),
                            ("dma_h2d", lambda: dev.copy_(host, non_blocking=True))):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                b.synchronize()
                if i >= 3:
                    times[key].append(a.elapsed_time(b) * 1e3)
        swap = {"blocks": int(blist.size), "bytes_each_way": nbytes_swap}
        for key, us in times.items():
            p50 = percentile(us, 0.5)
            swap[f"{key}_us_p50"] = round(p50, 1)
            swap[f"{key}_gbps"] = round(nbytes_swap / (p50 * 1e-6) / 1e9, 2)
        print(f"bench: swap {nbytes_swap / 2**20:.0f} MiB: out {swap['out_gbps']} GB/s, in {swap['in_gbps']} GB/s "
              f"(DMA {swap['dma_d2h_gbps']} / {swap['dma_h2d_gbps']})", file=sys.stderr, flush=True)
        del host, dev, blocks_dev
        torch.cuda.synchronize()

    table_walk = None
    if args.table_walk_probe:
        from paged_kv_cache_num_amd import probe_table_walk
        tsink = torch.empty(1 << 14, dtype=torch.uint8, device="cuda")
        table_walk = {}
        for grouped in (False, True):
            us = []
            for _ in range(args.table_walk_probe):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                probe_table_walk(step.block_tables, step.context_lens, wl.num_kv_heads, step.max_context_len,
                                 tsink, xcd_grouped=grouped)
                b.record()
                b.synchronize()
                us.append(a.elapsed_time(b) * 1e3)
            table_walk["xcd_grouped_us_p50" if grouped else "default_us_p50"] = round(percentile(us, 0.5), 2)

    traffic = traffic_for(args.config, part, wl.block_size, args.kv_dtype)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "launch": launch,
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "graph_two_call_ms_per_step": round(graph_ms[False], 5) if False in graph_ms else None,
        "graph_fused_ms_per_step": round(graph_ms[True], 5) if True in graph_ms else None,
        "graph_step_gpu_us_p50": {("fused" if f else "two_call"): round(v, 2) for f, v in graph_gpu_us.items()},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config, "variant": args.variant,
                   "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "partition_size": part,
                   "context_tokens": int(np.sum(wl.context_lens)), "scatter_tokens": wl.num_write_tokens,
                   "kv_dtype": "fp8_e4m3 codes + fp32 scale per (block, KV head)" if fp8 else wl.dtype,
                   "layers": NL, "seed": wl.info.get("seed")},
        "tokens_per_s_per_layer": round(wl.num_seqs / (ms_per_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "kernel": roofline_kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes["attn"],
                     "launch_us_mean": round(attn_mean, 2), "launch_us_p10": round(percentile(attn_us, 0.1), 2),
                     "launch_us_p50": round(percentile(attn_us, 0.5), 2),
                     "launch_us_p90": round(percentile(attn_us, 0.9), 2)},
        "scatter_us_mean": round(sum(scatter_us) / K, 2),
        "read_probe_gbps": round(read_gbps, 1),
        "frac_of_read_probe": round(achieved / read_gbps, 4),
        "step_bytes": step_bytes,
        "cold": cold,
        "same_layer": same_layer,
        "pool_utilization": round(float(wl.info.get("utilization") or 0.0), 4),
        "blocks_per_seq_mean": round(nbytes["blocks"] / max(1, wl.num_seqs), 2),
        "internal_waste_tokens": int(nbytes["blocks"] * wl.block_size - int(np.sum(wl.context_lens))),
        "identity_tables": identity,
        "shared_prefix": shared,
        "table_walk_probe": table_walk,
        "copy_blocks": copy,
        "swap": swap,
    }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_fp8(wl, state) if fp8 else cpu_baseline(wl, step_bytes, nbytes)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
