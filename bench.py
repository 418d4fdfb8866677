#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X.

A step is one decode step of the whole hot path for every sequence of the
batch: the host allocator appends one token per sequence into a pinned slot
stage, then one fused decode step runs on the device: a prologue kernel
extends the device block tables and lengths, plans the attention's work and
writes the new tokens' K/V into their slots (reading the slots from the stage
in place), and paged decode attention (main and merge kernels) reads every
sequence's K/V through its table.  --unfused makes the separate calls instead
(slot copy, append, scatter, plan, main, merge), with the same results.
The default workload is the Llama-3-70B-class layer: 256 sequences,
log-normal lengths (median 3000, clipped to [16, 32768]), 64 q / 8 KV heads,
head_dim 128, bf16 KV, 16-token blocks scattered through the pool, 3072-token
partitions.  All inputs are the seeded synthetic workload, resident in HBM
before the timed region.  Order of work: the batch is built, the streaming-read
probe runs (unless --no-read-ceiling), then the W warm-up steps and, with no
host work in between, the K timed steps.

Prints one JSON line: value = algorithmic KV-read GB/s over whole steps
(K + V bytes of every valid token plus block-table bytes), with seqs/s, the
decode kernel's roofline (HIP events on the kernel's stream), the decode
kernel's per-launch median / p10 / p90 over separately collected launches
after the timed region and the same over launches that each follow a 1 GiB
write and over launches that each follow a 1 GiB read (either evicts L2 and
the 256 MB Infinity Cache; --no-flush leaves these out), the device,
engine clock and ROCm version, and the fp64 CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config 3] [--block-size 16]
                    [--placement random|identity] [--kv-dtype native|fp8] [--no-cpu-baseline] [--sweep]

--kv-dtype fp8 runs the same workload on a quantised cache (FP8 E4M3 codes, per-tensor scales;
q and outputs keep the workload's type): bytes then count one byte per cached element.
--layout flat stores every sequence in a flat span (one contiguous virtual range, physical memory
mapped on demand) and decodes without a block table; no table bytes are counted.  --sweep covers
long_context over block sizes for random and identity placement and for flat spans.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + seqs/s, 1×MI355X"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--block-size", type=int, default=None)
    p.add_argument("--placement", default="random", choices=["random", "identity"])
    p.add_argument("--partition-size", type=int, default=None, help="default: the workload's own")
    p.add_argument("--seed", type=int, default=None,
                   help="another draw of the workload's distributions (default: the config's own seed)")
    p.add_argument("--copied-prefix", action="store_true", help="config 4: private prefix copies")
    p.add_argument("--kv-dtype", default="native", choices=["native", "fp8"],
                   help="fp8: the cache stores FP8 E4M3 codes (per-tensor scales)")
    p.add_argument("--layout", default="paged", choices=["paged", "flat"],
                   help="flat: per-sequence flat spans, decode reads no block table")
    p.add_argument("--chunk-bytes", type=int, default=0, help="flat spans: physical chunk size (0 = 2 MiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--sweep", action="store_true", help="config-5 block-size x placement sweep (decode only)")
    p.add_argument("--decode-only", action="store_true", help="time the decode call alone (no append/scatter)")
    p.add_argument("--reps", type=int, default=20,
                   help="separately collected launches for the decode kernel's median / p10 / p90")
    p.add_argument("--load-policy", default="auto", choices=["auto", "streamed", "cached", "prefix"],
                   help="how decode reads the pools (auto: the runtime's rule)")
    p.add_argument("--flush", dest="flush", action="store_true", default=True,
                   help="also time --reps launches after a 1 GiB write and --reps after a 1 GiB read "
                        "(each evicts L2 and MALL; the default)")
    p.add_argument("--no-flush", dest="flush", action="store_false",
                   help="leave out the cache-evicted launches")
    p.add_argument("--unfused", action="store_true",
                   help="paged steps as separate calls (slot copy, append_slots, scatter, decode) instead of "
                        "one decode_step")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    p.add_argument("--copy-blocks", action="store_true",
                   help="time the copy-on-write block copy kernel alone (4096 random block pairs)")
    p.add_argument("--swap", action="store_true",
                   help="time block moves between the pool and pinned host swap space (4096 blocks each way)")
    p.add_argument("--shared-prefix-tokens", type=int, default=None,
                   help="with --load-policy prefix: the prefix read cacheable (default: the batch's shared prefix)")
    p.add_argument("--math", default="mfma", choices=["mfma", "vector"],
                   help="with --decode-only: vector = the per-token vector path (16-bit KV, one head per KV head)")
    p.add_argument("--read-ceiling", action="store_true",
                   help="run only the streaming-read probe over its full sweep (one JSON line)")
    p.add_argument("--no-read-ceiling", action="store_true",
                   help="leave the short streaming-read probe out of the bench line")
    p.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                   help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of this bench and of "
                        "--copy-calibration into the traffic record (CPU only; writes --pmc-out)")
    p.add_argument("--pmc-out", default=None, help="default: the workload's traffic record under profiles/")
    p.add_argument("--pmc-command", default="", help="the command lines that produced the CSVs (recorded)")
    return p.parse_args()


# ------------------------------------------------------------------------------------- setup
def build_batch(w, fill="randn", extra_tokens=0, layout="paged", chunk_bytes=0):
    """The workload's prompts written through the library (allocator + scatter kernel).  layout
    "flat": each row's logical K/V goes into its own flat span (a shared prompt is copied per row:
    spans are never shared)."""
    import torch

    import workloads as wl
    from paged_kv_cache_53_amd.runtime import DecodeBatch, FlatDecodeBatch, FlatKVCache, PagedKVCache
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    if layout == "flat":
        if w.kv_format != "native":
            raise SystemExit("flat spans hold 16-bit KV")
        cache = FlatKVCache(w.num_seqs, w.max_seq_len + extra_tokens, w.block_size, w.n_kv_heads, w.head_dim, dt,
                            device="cuda", chunk_bytes=chunk_bytes)
        for r in range(w.num_seqs):
            # the prompt (L - 1 tokens): the first decode step appends the row's last token
            k, v = wl.kv_rows(w, int(w.batch[r]), 0, int(w.seq_lens[r]) - 1, device="cuda")
            cache.append(int(w.batch[r]), k, v)
            del k, v
        batch = FlatDecodeBatch(cache, w.batch.tolist(), w.n_q_heads, w.max_seq_len + extra_tokens,
                                partition_size=w.partition_size, scale=w.scale)
        return cache, batch
    if w.kv_format == "fp8":
        cache = PagedKVCache(w.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, torch.float8_e4m3fn,
                             device="cuda", free_order=w.free_order.tolist(), fill=fill, k_scale=w.k_scale,
                             v_scale=w.v_scale)
    else:
        cache = PagedKVCache(w.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, dt, device="cuda",
                             free_order=w.free_order.tolist(), fill=fill)
    for op in w.prompt_ops:
        if op["op"] == "alloc":
            k, v = wl.kv_rows(w, op["seq"], op["pos"], op["n"], device="cuda")
            cache.append(op["seq"], k, v)
            del k, v
        elif op["op"] == "fork":
            cache.fork(op["parent"], op["child"], op["n"])
        else:
            cache.free(op["seq"])
    batch = DecodeBatch(cache, w.batch.tolist(), w.n_q_heads, w.max_seq_len + extra_tokens,
                        partition_size=w.partition_size, scale=w.scale)
    return cache, batch


def host_duplicate_tokens(w):
    """duplicate_tokens of the workload's prompt batch, from its allocator operations replayed on a host
    allocator alone (no device memory: the counter summaries are made on the CPU)."""
    from paged_kv_cache_53_amd import Allocator
    alloc = Allocator(w.num_blocks, w.block_size, w.free_order.tolist())
    for op in w.prompt_ops:
        if op["op"] == "alloc":
            alloc.alloc(op["seq"], op["n"])
        elif op["op"] == "fork":
            alloc.fork(op["parent"], op["child"], op["n"])
        else:
            alloc.free(op["seq"])
    stride = -(-(int(w.seq_lens.max()) + 64) // w.block_size)
    tables, _ = alloc.fill_block_tables(w.batch.tolist(), stride, pad=0)
    return duplicate_tokens(tables, w.seq_lens - 1, w.block_size)


def kv_bytes(w, lens, table=True):
    """Algorithmic bytes one decode reads: K+V of every valid token, plus the block-table entries
    (none for flat spans)."""
    import numpy as np
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * 2 * w.n_kv_heads * w.head_dim * w.kv_esize
    tb = int(((lens + w.block_size - 1) // w.block_size).sum()) * 4 if table else 0
    return kv, tb


def load_description(batch):
    """How the decode batch reads the pools (the runtime's load policy in effect)."""
    args = batch._load_args()
    if args.get("shared_prefix_tokens"):
        return f"first {args['shared_prefix_tokens']} tokens of each row cacheable, the rest streamed"
    return "cached" if args.get("shared_kv") else "streamed"


def duplicate_tokens(tables, lens, block_size):
    """Tokens the rows of a batch read from blocks that another row of the batch also reads, beyond the
    first reading: every physical block's valid tokens count once towards the unique bytes HBM must
    supply (a shared prompt is stored once), and the rest are re-reads.  tables: [S, >= ceil(L/B)] block
    ids, lens: [S] lengths."""
    seen = {}
    total = 0
    for s in range(len(lens)):
        L = int(lens[s])
        for i in range(-(-L // block_size)):
            b = int(tables[s][i])
            v = min(block_size, L - i * block_size)
            seen[b] = max(seen.get(b, 0), v)
            total += v
    return total - sum(seen.values())


# ------------------------------------------------------------------------------------- GPU timing
def percentiles_us(ms_values):
    """median, p10 and p90 (and the extremes) of per-launch times given in ms, in us."""
    import numpy as np
    a = np.asarray(ms_values, dtype=np.float64) * 1e3
    return {"launches": int(a.size), "median": round(float(np.median(a)), 2),
            "p10": round(float(np.percentile(a, 10)), 2), "p90": round(float(np.percentile(a, 90)), 2),
            "min": round(float(a.min()), 2), "max": round(float(a.max()), 2)}


def time_steps(w, steps, warmup, decode_only=False, layout="paged", chunk_bytes=0, fused=True, reps=20,
               flush=False, load_policy="auto", math="mfma", shared_prefix_tokens=None, before_warmup=None):
    """Times `steps` decode steps of workload w after `warmup` untimed ones.  before_warmup: GPU work run
    once the batch is resident, right before the warm-up steps (the bench line's streaming-read probe).
    Nothing the host computes runs between the warm-up and the timed steps: an idle GPU that resumes
    work shows a clock transient for several milliseconds (decode launches 3 to 11 after resuming took
    800-870 us instead of about 750 on the Llama-70B-class batch), which a gap there would put into the
    timed region."""
    import numpy as np
    import torch

    import paged_kv_cache_53_amd as pkv
    import workloads as wl
    diag = min(10, steps)   # untimed pass that times every kernel of the step
    extra = steps + warmup + diag + reps * (3 if flush else 1) + 1
    cache, batch = build_batch(w, extra_tokens=extra, layout=layout, chunk_bytes=chunk_bytes)
    if load_policy != "auto":
        batch.load_policy = load_policy
    if shared_prefix_tokens is not None:
        batch.shared_prefix = shared_prefix_tokens
    if math == "vector":
        if not decode_only or layout != "paged":
            raise SystemExit("--math vector times the paged decode call alone (--decode-only)")
        batch.vector = True
    q = wl.q_values(w, device="cuda").contiguous()
    kn, vn = wl.new_token_kv(w, device="cuda")
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    log(f"workload ready: {w.describe()}")

    def one():
        if decode_only:
            batch.decode_only(q, out)
        elif layout == "paged":
            batch.step(q, kn, vn, out, fused=fused)
        else:
            batch.step(q, kn, vn, out)

    dup = 0
    if layout == "paged":
        tables0, lens_now = cache.allocator.fill_block_tables(batch.seq_ids, batch.stride, pad=0)
        dup = duplicate_tokens(tables0, lens_now, w.block_size)   # appends go to private blocks: constant
    extra_gpu = before_warmup() if before_warmup is not None else None
    for _ in range(warmup):
        one()
    # timed region: only the decode kernel carries an event pair (each pair costs the stream a few us)
    pkv.timing_select(["decode"])
    pkv.timing_enable(True)
    torch.cuda.synchronize()
    lens0 = batch.host_lens.copy()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    decode_timed = pkv.timing_collect()["decode"]
    # breakdown of every kernel of the step, from a short pass after the timed region
    pkv.timing_select(None)
    pkv.timing_enable(True)
    for _ in range(diag):
        one()
    torch.cuda.synchronize()
    kernels = pkv.timing_collect()
    # per-launch distribution of the decode kernel: one step at a time, each collected on its own
    # (untimed for `value`); with flush, each step follows a 1 GiB write that evicts L2 and MALL
    pkv.timing_select(["decode"])
    warm = []
    for _ in range(reps):
        one()
        torch.cuda.synchronize()
        n, ms = pkv.timing_collect()["decode"]
        warm.append(ms / n)
    cold = {}
    if flush:
        # after_write: each launch follows a 1 GiB write (L2 and MALL then hold the scratch's dirty
        # lines); after_read: each follows a 1 GiB read (clean lines, as when other layers' KV was
        # read in between)
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        for mode in ("after_write", "after_read"):
            scratch.fill_(1)
            scratch.view(torch.float32).amax()
            torch.cuda.synchronize()
            vals = []
            for i in range(reps):
                pkv.timing_enable(False)
                if mode == "after_write":
                    scratch.fill_((i + 2) & 0xFF)
                else:
                    scratch.view(torch.float32).amax()
                torch.cuda.synchronize()
                pkv.timing_enable(True)
                one()
                torch.cuda.synchronize()
                n, ms = pkv.timing_collect()["decode"]
                vals.append(ms / n)
            cold[mode] = percentiles_us(vals)
        del scratch
    pkv.timing_select(None)
    pkv.timing_enable(False)
    total_s = t1 - t0
    # bytes: during step i every row attends over lens0 + i + 1 tokens (the appended one included)
    kvb = tb = 0
    for i in range(steps):
        lens = lens0 if decode_only else lens0 + i + 1
        a, b = kv_bytes(w, lens, table=layout != "flat")
        kvb += a
        tb += b
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    per_token = 2 * w.n_kv_heads * w.head_dim * w.kv_esize
    return {"total_s": total_s, "kv_bytes": kvb, "table_bytes": tb, "kernels": kernels, "steps": steps,
            "kv_bytes_unique": kvb - dup * per_token * steps, "duplicate_tokens": dup,
            "lens0": lens0, "decode_timed": decode_timed, "diag_steps": diag,
            "decode_loads": load_description(batch) if layout == "paged" else "streamed",
            "decode_launch_us": percentiles_us(warm) if warm else None,
            "decode_launch_us_cold": cold or None, "before_warmup": extra_gpu}


def _read_text(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def gpu_env():
    """The device, its engine clock levels (sysfs, when readable) and the ROCm / HIP versions."""
    import torch
    p = torch.cuda.get_device_properties(0)
    env = {"device": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
           "rocm": _read_text("/opt/rocm/.info/version"), "torch_hip": torch.version.hip}
    pci = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    env["sclk_mhz"] = parse_dpm_sclk(_read_text(f"/sys/bus/pci/devices/{pci}/pp_dpm_sclk"))
    return env


def parse_dpm_sclk(txt):
    """{current, max} engine clock in MHz from the text of a pp_dpm_sclk file (one level a line,
    "<index>: <n>Mhz", the active level marked with "*"), or None."""
    if not txt:
        return None
    levels, cur = [], None
    for ln in txt.splitlines():
        parts = ln.replace(":", " ").split()
        mhz = [int(x[:-3]) for x in parts if x.lower().endswith("mhz") and x[:-3].isdigit()]
        if mhz:
            levels.append(mhz[0])
            if ln.rstrip().endswith("*"):
                cur = mhz[0]
    if not levels:
        return None
    return {"current": cur, "max": max(levels), "source": "pp_dpm_sclk after the timed region"}


def cpu_model():
    txt = _read_text("/proc/cpuinfo") or ""
    for ln in txt.splitlines():
        if ln.startswith("model name"):
            return ln.split(":", 1)[1].strip()
    return None


# Sources whose change invalidates measured HBM counters of the decode kernel.
KERNEL_SOURCES = ("paged_kv_cache_53_amd/csrc/decode.hip", "paged_kv_cache_53_amd/csrc/api.hip",
                  "paged_kv_cache_53_amd/csrc/pkv_internal.h")
DECODE_KERNEL_PREFIX = "_ZN3pkv12_GLOBAL__N_113decode_kernel"


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def workload_key(w):
    return {"workload": w.name, "variant": w.variant, "block_size": w.block_size,
            "partition_size": w.partition_size, "placement": w.placement}


def traffic_record_path(w):
    suffix = "_fp8" if w.kv_format == "fp8" else ""
    return os.path.join(ROOT, "profiles", f"decode_traffic_{w.name}{suffix}.json")


def measured_traffic(w):
    """HBM bytes per decode launch from the committed counter record, or None when the record
    was taken on other kernel sources or another workload."""
    path = traffic_record_path(w)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256() or rec.get("workload") != workload_key(w):
        return None
    return rec


def roofline(res, w=None, math="mfma"):
    n_dec, ms_dec = res.get("decode_timed", (0, 0.0))
    if not n_dec:
        return None
    # unique bytes: a block read by several rows of the batch counts once (the shared prompt of a
    # swarm is stored once); without sharing they equal the logical bytes
    per_launch = (res["kv_bytes_unique"] + res["table_bytes"]) / res["steps"]
    logical = (res["kv_bytes"] + res["table_bytes"]) / res["steps"]
    avg_s = ms_dec / n_dec / 1e3
    achieved = per_launch / avg_s / 1e9
    rec = measured_traffic(w) if w is not None else None
    out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBPS, 4),
           # measured HBM bytes per launch: the counters' bytes-per-algorithmic-byte ratio of this
           # kernel on this workload, times this run's algorithmic bytes per launch
           "traffic": int(rec["traffic_over_algorithmic"] * per_launch) if rec else None,
           "kernel": kernel_label(w, math),
           "bytes_per_launch": int(per_launch), "avg_launch_us": round(avg_s * 1e6, 2)}
    if w is not None:
        # beside the algorithmic bytes, not counted in them: q, the output and the lengths (each once per
        # row); and the attention's own flops, sum over rows of L * Hq * 4 * D
        e = 4 if w.dtype == "f32" else 2
        out["aux_bytes_per_launch"] = int(w.num_seqs * (2 * w.n_q_heads * w.head_dim * e + 4))
        tokens = res["kv_bytes"] / res["steps"] / (2 * w.n_kv_heads * w.head_dim * w.kv_esize)
        out["flop_per_launch"] = int(tokens * w.n_q_heads * 4 * w.head_dim)
    if logical != per_launch:
        out["achieved_logical"] = round(logical / avg_s / 1e9, 1)
        out["bytes_per_launch_logical"] = int(logical)
    if rec:
        out["traffic_detail"] = {"fetch_bytes": int(rec["fetch_over_algorithmic"] * per_launch),
                                 "write_bytes": int(rec["write_over_algorithmic"] * per_launch),
                                 "source": os.path.relpath(traffic_record_path(w), ROOT)}
    return out


def kernel_label(w, math="mfma"):
    """Which decode kernel the roofline covers."""
    if w is not None and w.dtype == "f32":
        return "decode_kernel (persistent paged decode, fp32 KV on the vector path)"
    if math == "vector":
        return "decode_kernel (persistent paged decode, 16-bit KV on the per-token vector path)"
    kv = "FP8 E4M3 KV widened in registers" if w is not None and w.kv_format == "fp8" else "16-bit KV"
    return f"decode_kernel (persistent paged decode on MFMA, {kv})"


def read_ceiling(full=False):
    """The streaming-read ceiling: pkv_read_probe over a 4 GiB buffer (read once per launch, nothing
    computed), timed with HIP events on the launch stream, over a sweep of waves per CU, loads per batch,
    contiguous or scattered 4 KiB chunks, with and without the non-temporal hint.  Returns the best rate
    and the sweep."""
    import torch

    import paged_kv_cache_53_amd as pkv
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    waves = (2, 4, 6, 8, 12, 16) if full else (4, 8)
    loads = (4, 8, 16) if full else (8, 16)
    modes = (0, 1, 2, 3) if full else (1, 3)
    rows = []
    for wpc in waves:
        for nl in loads:
            for mode in modes:
                nbytes = pkv.read_probe(buf, wpc, nl, bool(mode & 1), bool(mode & 2), sink=sink)   # warm-up
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                reps = 5
                ev[0].record()
                for _ in range(reps):
                    pkv.read_probe(buf, wpc, nl, bool(mode & 1), bool(mode & 2), sink=sink)
                ev[1].record()
                torch.cuda.synchronize()
                us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
                rows.append({"waves_per_cu": wpc, "loads_per_batch": nl, "nontemporal": bool(mode & 1),
                             "chunks": "scattered 4 KiB" if mode & 2 else "contiguous",
                             "gbps": round(nbytes / (us * 1e-6) / 1e9, 1), "us": round(us, 1)})
    del buf
    best = max(rows, key=lambda r: r["gbps"])
    return {"best_gbps": best["gbps"], "best": best, "sweep": rows if full else None,
            "note": "pkv_read_probe: 4 GiB read once per launch by single-wave workgroups, 16 B per lane per "
                    "load, two batches in flight per wave, no computation; mean of 5 launches per point"}


# ------------------------------------------------------------------------------------- counters
def _pmc_rows(path, counter):
    import csv
    with open(path, newline="") as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    return rows


def pmc_summary(args):
    """Calibrated HBM traffic of the decode kernel from FETCH_SIZE / WRITE_SIZE counter CSVs.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch; each is scaled by what it reads for a
    plain copy of known size (the 1 GiB copy kernel of --copy-calibration reads and writes 1 GiB).
    """
    import statistics
    fetch_csv, write_csv, cal_fetch_csv, cal_write_csv = args.pmc_summary
    copy_kib = (1 << 30) / 1024.0

    def copy_reading(path, counter):
        rows = [r for r in _pmc_rows(path, counter) if "copyBuffer" in r["Kernel_Name"]]
        if not rows:
            raise SystemExit(f"no copy kernel rows for {counter} in {path}")
        return statistics.median(float(r["Counter_Value"]) for r in rows)

    def decode_readings(path, counter):
        rows = [r for r in _pmc_rows(path, counter) if r["Kernel_Name"].startswith(DECODE_KERNEL_PREFIX)]
        if not rows:
            raise SystemExit(f"no decode kernel rows for {counter} in {path}")
        return [float(r["Counter_Value"]) for r in rows], rows[0]["Kernel_Name"]

    f_scale = copy_kib / copy_reading(cal_fetch_csv, "FETCH_SIZE")
    w_scale = copy_kib / copy_reading(cal_write_csv, "WRITE_SIZE")
    f_vals, kname = decode_readings(fetch_csv, "FETCH_SIZE")
    w_vals, _ = decode_readings(write_csv, "WRITE_SIZE")
    import numpy as np

    import workloads as wl
    w = make_workload(args)
    # decode dispatch j of the profiled bench run attends over the prompt (L - 1 tokens) plus the
    # j + 1 tokens appended so far; a --decode-only run appends nothing
    prompt = w.seq_lens.astype(np.int64) - 1
    # unique bytes, as the bench line's roofline counts them: a block several rows read counts once
    # (appended tokens go to private blocks, so the duplicates stay those of the prompt)
    dup_bytes = host_duplicate_tokens(w) * 2 * w.n_kv_heads * w.head_dim * w.kv_esize

    def algo(j):
        kvb, tb = kv_bytes(w, prompt if args.decode_only else prompt + j + 1)
        return kvb - dup_bytes + tb

    f_ratio = statistics.median(v * f_scale * 1024 / algo(j) for j, v in enumerate(f_vals))
    w_ratio = statistics.median(v * w_scale * 1024 / algo(j) for j, v in enumerate(w_vals))
    a_last = algo(len(f_vals) - 1)
    rec = {
        "kernel": kname, "workload": workload_key(w), "kernel_sources_sha256": kernel_sources_sha256(),
        "profiled_run": {"steps": args.steps, "warmup": args.warmup, "decode_only": bool(args.decode_only),
                         "decode_launches": {"fetch": len(f_vals), "write": len(w_vals)}},
        "raw_kib_per_launch_median": {"FETCH_SIZE": statistics.median(f_vals),
                                      "WRITE_SIZE": statistics.median(w_vals)},
        "calibration": {"copy_bytes": 1 << 30, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "fetch_over_algorithmic": round(f_ratio, 5), "write_over_algorithmic": round(w_ratio, 5),
        "traffic_over_algorithmic": round(f_ratio + w_ratio, 5),
        "duplicate_bytes_per_launch": int(dup_bytes),
        "last_launch": {"algorithmic_bytes": int(a_last), "fetch_bytes": int(f_vals[-1] * f_scale * 1024),
                        "write_bytes": int(w_vals[-1] * w_scale * 1024)},
        "command": args.pmc_command,
    }
    out_path = args.pmc_out or traffic_record_path(w)
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)


# ------------------------------------------------------------------------------------- CPU oracle
def cpu_baseline(w, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload's rows."""
    import numpy as np

    import workloads as wl
    from oracle import attention as O
    from oracle import scatter as SC
    from oracle.allocator import BlockAllocatorModel
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        used = max([i.get("num_threads", 1) for i in info] or [1])
        return _oracle_sample(w, budget_s, cores, used)


def _oracle_sample(w, budget_s, cores, used):
    import numpy as np

    import workloads as wl
    from oracle import attention as O
    from oracle import scatter as SC
    from oracle.allocator import BlockAllocatorModel
    fp8 = w.kv_format == "fp8"
    st = np.uint8 if fp8 else {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[w.dtype]
    order = np.random.default_rng([w.seed, 99]).permutation(w.num_seqs)
    done, kvb, tb, spent = [], 0, 0, 0.0
    for r in order.tolist():
        if spent >= budget_s:
            break
        seq = int(w.batch[r])
        L = int(w.seq_lens[r])
        # untimed: this row's pool built through the oracle's own allocator and scatter
        nb = -(-L // w.block_size)
        a = BlockAllocatorModel(nb, w.block_size, np.random.default_rng([w.seed, 98, r]).permutation(nb))
        kp, vp = SC.empty_pools(a.num_blocks, w.n_kv_heads, w.head_dim, w.block_size, st, 0)
        slots, _ = a.alloc(seq, L)
        K, V = wl.logical_kv(w, r)
        if fp8:
            kf = O.to_f64(wl.storage_to_numpy(K), w.dtype).astype(np.float32)
            vf = O.to_f64(wl.storage_to_numpy(V), w.dtype).astype(np.float32)
            SC.reshape_and_cache_fp8(kf, vf, np.array(slots), kp, vp, w.k_scale, w.v_scale)
        else:
            SC.reshape_and_cache(wl.storage_to_numpy(K), wl.storage_to_numpy(V), np.array(slots), kp, vp)
        q = wl.storage_to_numpy(wl.q_values(w))[r:r + 1]
        table = np.array([a.block_table(seq)])
        t0 = time.perf_counter()
        if fp8:
            O.paged_attention_decode_fp8(q, w.dtype, kp, vp, w.k_scale, w.v_scale, table, np.array([L]), w.scale)
        else:
            O.paged_attention_decode(q, kp, vp, table, np.array([L]), w.scale, w.dtype)
        spent += time.perf_counter() - t0
        done.append(r)
        x, y = kv_bytes(w, [L])
        kvb += x
        tb += y
    return {"value": round((kvb + tb) / spent / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle", "seqs_per_s": round(len(done) / spent, 3), "cpu_model": cpu_model(),
            "sample": f"{len(done)} of {w.num_seqs} rows of {w.name} (seeded order), "
                      f"{int(sum(int(w.seq_lens[r]) for r in done))} tokens, {spent:.1f} s of fp64 numpy "
                      f"(gather through the block table{' + dequantisation' if fp8 else ''} + attention), "
                      f"host cores available {cores}"}


# ------------------------------------------------------------------------------------- main
def step_description(args):
    if args.decode_only:
        return "decode_only"
    if args.layout == "flat":
        return "host append + span mapping + stage + append_slots + scatter + decode"
    if args.unfused:
        return "host append + slot copy + append_slots + scatter + decode (plan, attention, merge)"
    return "host append + decode_step (prologue: append_slots + plan + scatter; attention; merge)"


def make_workload(args):
    import workloads as wl
    w = wl.build(args.config, block_size=args.block_size, placement=args.placement,
                 copied_prefix=args.copied_prefix, partition_size=args.partition_size, seed=args.seed)
    return wl.quantised(w) if args.kv_dtype == "fp8" else w


def main():
    args = parse()
    if args.pmc_summary:
        return pmc_summary(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by sequence "
              "or KV head with no exchange, and this benchmark measures one GPU's share", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.sweep:
        return sweep(args)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 5}), flush=True)
        return

    if args.read_ceiling:
        rc = read_ceiling(full=True)
        print(json.dumps({"metric": "streaming HBM read GB/s (probe, no computation), 1×MI355X",
                          "value": rc["best_gbps"], "unit": "GB/s", "peak": HBM_PEAK_GBPS,
                          "frac": round(rc["best_gbps"] / HBM_PEAK_GBPS, 4), **rc, "env": gpu_env()}), flush=True)
        return
    if args.copy_blocks:
        return bench_copy_blocks(args)
    if args.swap:
        return bench_swap(args)

    w = make_workload(args)

    def probe():
        # the streaming-read probe runs right before the warm-up steps: about 30 ms of full-bandwidth
        # reads, after which the engine clock has settled under load
        log("streaming-read probe ...")
        return read_ceiling(full=False)

    res = time_steps(w, args.steps, args.warmup, decode_only=args.decode_only, layout=args.layout,
                     chunk_bytes=args.chunk_bytes, fused=not args.unfused, reps=args.reps, flush=args.flush,
                     load_policy=args.load_policy, math=args.math, shared_prefix_tokens=args.shared_prefix_tokens,
                     before_warmup=None if args.no_read_ceiling else probe)
    total_s = res["total_s"]
    gbps = (res["kv_bytes_unique"] + res["table_bytes"]) / total_s / 1e9
    gbps_logical = (res["kv_bytes"] + res["table_bytes"]) / total_s / 1e9
    seqs_s = w.num_seqs * args.steps / total_s
    kern = {k: {"launches": n, "avg_us": round(ms / n * 1e3, 2)} for k, (n, ms) in res["kernels"].items()}
    kern["_note"] = f"every kernel timed over {res['diag_steps']} untimed steps after the timed region"
    line = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_s / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "seqs": w.num_seqs, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "partition_size": w.partition_size,
                   "placement": w.placement, "total_tokens_at_start": int(res["lens0"].sum()),
                   "kv_dtype": "fp8_e4m3 (per-tensor scales)" if w.kv_format == "fp8" else w.dtype,
                   "layout": "paged" if args.layout == "paged" else
                   f"flat spans ({args.chunk_bytes or 2 << 20}-byte chunks, no block table)",
                   "seed": w.seed, "step": step_description(args)},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "seqs_per_s": round(seqs_s, 1),
        "kernels": kern,
        "roofline": roofline(res, w, args.math),
        "decode_loads": res["decode_loads"],
        "decode_math": args.math,
        "decode_launch_us": res["decode_launch_us"],
        "env": gpu_env(),
    }
    if res["decode_launch_us_cold"] is not None:
        line["decode_launch_us_cold"] = dict(res["decode_launch_us_cold"])
        line["decode_launch_us_cold"]["note"] = ("each launch follows a 1 GiB write (after_write) or a 1 GiB "
                                                 "read (after_read) that evicts L2 and the 256 MB Infinity Cache")
    if res["duplicate_tokens"]:
        # rows share blocks: value and pct_hbm_peak count each block once (unique bytes); the rate over
        # every row's own reading of its tokens is the logical one
        line["value_logical"] = round(gbps_logical, 2)
        line["bytes_note"] = (f"{res['duplicate_tokens']} tokens per step are read by more than one row; value, "
                              "pct_hbm_peak and roofline count each physical block once (unique bytes)")
    if not args.no_read_ceiling:
        rc = res["before_warmup"]
        line["measured_read_gbps"] = rc["best_gbps"]
        line["read_ceiling"] = {k: rc[k] for k in ("best", "note")}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def bench_copy_blocks(args):
    """Copy-on-write block copies on the workload's pool shape: 4096 (src, dst) pairs per call over a
    pool of 8192 blocks, random placement; bytes = every copied block read once and written once."""
    import numpy as np
    import torch

    import paged_kv_cache_53_amd as pkv
    import workloads as wl
    w = wl.build(args.config, block_size=args.block_size)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    n_pairs, N = 4096, 8192
    kp = torch.empty(pkv.key_pool_shape(N, w.n_kv_heads, w.head_dim, w.block_size, dt), dtype=dt, device="cuda")
    vp = torch.empty(pkv.value_pool_shape(N, w.n_kv_heads, w.head_dim, w.block_size), dtype=dt, device="cuda")
    perm = np.random.default_rng([w.seed, 7]).permutation(N)
    pairs = torch.from_numpy(np.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], 1).astype(np.int32)).cuda()
    for _ in range(args.warmup):
        pkv.copy_blocks(pairs, kp, vp)
    pkv.timing_select(["copy_blocks"])
    pkv.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pkv.copy_blocks(pairs, kp, vp)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n, ms = pkv.timing_collect()["copy_blocks"]
    pkv.timing_enable(False)
    pkv.timing_select(None)
    block_bytes = w.n_kv_heads * w.head_dim * w.block_size * w.esize
    moved = n_pairs * 2 * block_bytes * 2          # both pools, read + write
    us = ms / n * 1e3
    achieved = moved / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "copy-on-write block copies, GB/s moved (read + write)", "value": round(achieved, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} pool shape, {n_pairs} block pairs per call", "block_size": w.block_size,
                   "block_bytes_per_pool": block_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "copy_blocks_kernel",
                     "bytes_per_launch": moved, "avg_launch_us": round(us, 2)}}), flush=True)


def bench_swap(args):
    """Swap traffic on the workload's pool shape: 4096 random blocks from an 8192-block device pool to
    pinned host slots and back per call.  Bytes = blocks x block bytes x 2 pools, each way.  Beside
    it, a plain pinned-to-device copy of the same bytes (one contiguous buffer) gives the host link's
    practical rate."""
    import numpy as np
    import torch

    import paged_kv_cache_53_amd as pkv
    import workloads as wl
    w = wl.build(args.config, block_size=args.block_size)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    n, N, H = 4096, 8192, 4096
    kp = torch.empty(pkv.key_pool_shape(N, w.n_kv_heads, w.head_dim, w.block_size, dt), dtype=dt, device="cuda")
    vp = torch.empty(pkv.value_pool_shape(N, w.n_kv_heads, w.head_dim, w.block_size), dtype=dt, device="cuda")
    kh = torch.empty(pkv.key_pool_shape(H, w.n_kv_heads, w.head_dim, w.block_size, dt), dtype=dt, pin_memory=True)
    vh = torch.empty(pkv.value_pool_shape(H, w.n_kv_heads, w.head_dim, w.block_size), dtype=dt, pin_memory=True)
    rng = np.random.default_rng([w.seed, 8])
    dev, host = rng.permutation(N)[:n], rng.permutation(H)[:n]
    out_pairs = torch.from_numpy(np.stack([dev, host], 1).astype(np.int32)).cuda()
    in_pairs = torch.from_numpy(np.stack([host, rng.permutation(N)[:n]], 1).astype(np.int32)).cuda()
    block_bytes = w.n_kv_heads * w.head_dim * w.block_size * w.esize
    moved = n * block_bytes * 2
    res = {}
    for name, fn in (("to_host", lambda: pkv.swap_blocks(out_pairs, kp, vp, kh, vh)),
                     ("to_device", lambda: pkv.swap_blocks(in_pairs, kh, vh, kp, vp))):
        for _ in range(args.warmup):
            fn()
        pkv.timing_select(["swap_blocks"])
        pkv.timing_enable(True)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        k, ms = pkv.timing_collect()["swap_blocks"]
        pkv.timing_enable(False)
        pkv.timing_select(None)
        us = ms / k * 1e3
        res[name] = {"avg_us": round(us, 1), "GBps": round(moved / (us * 1e-6) / 1e9, 2)}
    flat_h = torch.empty(moved // 2, dtype=torch.uint8, pin_memory=True)
    flat_d = torch.empty(moved // 2, dtype=torch.uint8, device="cuda")
    plain = {}
    for name, (dst, src) in (("to_host", (flat_h, flat_d)), ("to_device", (flat_d, flat_h))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        plain[name] = {"avg_us": round(us, 1), "GBps": round(moved / 2 / (us * 1e-6) / 1e9, 2)}
    print(json.dumps({
        "metric": "swap block moves between the pool and pinned host memory, GB/s each way",
        "value": res["to_host"]["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} pool shape, {n} blocks per call, 8192-block pool, {H} host slots",
                   "block_bytes_per_pool": block_bytes, "bytes_per_call": moved},
        "swap_kernel": res, "plain_contiguous_copy_same_bytes": plain}), flush=True)


def sweep(args):
    """long_context decode over block sizes: paged with random and identity placement, and flat spans
    (no block table) with 2 MiB and 256 KiB chunks, at the launch's partition size; and paged with random
    placement in 512-token partitions (128 per row, the split the workload states).  The paged-over-flat
    ratio is the cost of reading through a block table."""
    import torch

    import workloads as wl
    rows = []
    for B in (8, 16, 32):
        per = {}
        for layout, placement, chunk, part in (("paged", "random", 0, args.partition_size),
                                               ("paged", "identity", 0, args.partition_size),
                                               ("flat", "random", 0, args.partition_size),
                                               ("flat", "random", 256 << 10, args.partition_size),
                                               ("paged", "random", 0, 512)):
            w = wl.build(5, block_size=B, placement=placement, partition_size=part)
            key = placement if layout == "paged" else f"flat_{(chunk or 2 << 20) >> 10}KiB"
            if part == 512 and args.partition_size != 512:
                key = "random_P512"
            try:
                # (the short read probe before each point's warm-up settles the clock, as for the bench line)
                res = time_steps(w, args.steps, args.warmup, decode_only=True, layout=layout, chunk_bytes=chunk,
                                 reps=0, flush=False, before_warmup=lambda: read_ceiling(full=False))
            except RuntimeError as e:      # a span pool that cannot map this many chunks
                per[key] = {"error": str(e)}
                log(f"B={B} {key}: {e}")
                torch.cuda.empty_cache()
                continue
            rf = roofline(res)
            per[key] = {"decode_GBps": rf["achieved"], "pct_hbm": round(100 * rf["frac"], 2),
                        "decode_us": rf["avg_launch_us"],
                        "seqs_per_s": round(w.num_seqs / (res["total_s"] / res["steps"]), 1),
                        "call_us": round(res["total_s"] / res["steps"] * 1e6, 2)}
            log(f"B={B} {key}: {per[key]}")
            torch.cuda.empty_cache()
        def ratio(a, b):
            if "decode_us" in per.get(a, {}) and "decode_us" in per.get(b, {}):
                return round(per[a]["decode_us"] / per[b]["decode_us"], 4)
            return None
        rows.append({"block_size": B, **per, "random_over_identity": ratio("random", "identity"),
                     "random_over_flat": ratio("random", "flat_2048KiB"),
                     "P512_over_P": ratio("random_P512", "random")})
    P = args.partition_size or wl.build(5, small=True).partition_size
    print(json.dumps({"sweep": f"long_context 8 x 65536, bf16, 64q/8kv heads, P={P} (random_P512: P=512); "
                               "decode us (lower is better); GB/s count K+V plus table bytes (none for flat)",
                      "rows": rows}), flush=True)


if __name__ == "__main__":
    main()
