#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X.

A step is one decode step of the whole hot path for every sequence of the
batch: the host allocator appends one token per sequence, the new slots are
staged to the device, the append kernel extends the device block tables,
the scatter kernel writes the new tokens' K/V, and paged decode attention
(plan, main, merge kernels) reads every sequence's K/V through its table.
The default workload is the Llama-3-70B-class layer: 256 sequences,
log-normal lengths (median 3000, clipped to [16, 32768]), 64 q / 8 KV heads,
head_dim 128, bf16 KV, 16-token blocks scattered through the pool, 512-token
partitions.  All inputs are the seeded synthetic workload, resident in HBM
before the timed region.

Prints one JSON line: value = algorithmic KV-read GB/s over whole steps
(K + V bytes of every valid token plus block-table bytes), with seqs/s, the
decode kernel's roofline (HIP events on the kernel's stream), and the fp64
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config 3] [--block-size 16]
                    [--placement random|identity] [--no-cpu-baseline] [--sweep]
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
    p.add_argument("--copied-prefix", action="store_true", help="config 4: private prefix copies")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--sweep", action="store_true", help="config-5 block-size x placement sweep (decode only)")
    p.add_argument("--decode-only", action="store_true", help="time the decode call alone (no append/scatter)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    return p.parse_args()


# ------------------------------------------------------------------------------------- setup
def build_batch(w, fill="randn", extra_tokens=0):
    """The workload's prompts written through the library (allocator + scatter kernel)."""
    import torch

    import workloads as wl
    from paged_kv_cache_53_amd.runtime import DecodeBatch, PagedKVCache
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
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


def kv_bytes(w, lens):
    """Algorithmic bytes one decode reads: K+V of every valid token, plus the block-table entries."""
    import numpy as np
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * 2 * w.n_kv_heads * w.head_dim * w.esize
    table = int(((lens + w.block_size - 1) // w.block_size).sum()) * 4
    return kv, table


# ------------------------------------------------------------------------------------- GPU timing
def time_steps(w, steps, warmup, decode_only=False):
    import numpy as np
    import torch

    import paged_kv_cache_53_amd as pkv
    import workloads as wl
    cache, batch = build_batch(w, extra_tokens=steps + warmup + 1)
    q = wl.q_values(w, device="cuda").contiguous()
    kn, vn = wl.new_token_kv(w, device="cuda")
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    log(f"workload ready: {w.describe()}")

    def one():
        if decode_only:
            batch.decode_only(q, out)
        else:
            batch.step(q, kn, vn, out)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    lens0 = batch.host_lens.copy() if decode_only else batch.host_lens.copy()
    pkv.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernels = pkv.timing_collect()
    pkv.timing_enable(False)
    total_s = t1 - t0
    # bytes: during step i every row attends over lens0 + i + 1 tokens (the appended one included)
    kvb = tb = 0
    for i in range(steps):
        lens = lens0 if decode_only else lens0 + i + 1
        a, b = kv_bytes(w, lens)
        kvb += a
        tb += b
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    return {"total_s": total_s, "kv_bytes": kvb, "table_bytes": tb, "kernels": kernels, "steps": steps,
            "lens0": lens0}


def roofline(res):
    n_dec, ms_dec = res["kernels"].get("decode", (0, 0.0))
    if not n_dec:
        return None
    per_launch = (res["kv_bytes"] + res["table_bytes"]) / res["steps"]
    avg_s = ms_dec / n_dec / 1e3
    achieved = per_launch / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
            "kernel": "decode_kernel (persistent paged decode, MFMA policy for 16-bit KV with G >= 3)",
            "bytes_per_launch": int(per_launch), "avg_launch_us": round(avg_s * 1e6, 2)}


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
    st = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[w.dtype]
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
        SC.reshape_and_cache(wl.storage_to_numpy(K), wl.storage_to_numpy(V), np.array(slots), kp, vp)
        q = wl.storage_to_numpy(wl.q_values(w))[r:r + 1]
        table = np.array([a.block_table(seq)])
        t0 = time.perf_counter()
        O.paged_attention_decode(q, kp, vp, table, np.array([L]), w.scale, w.dtype)
        spent += time.perf_counter() - t0
        done.append(r)
        x, y = kv_bytes(w, [L])
        kvb += x
        tb += y
    return {"value": round((kvb + tb) / spent / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle", "seqs_per_s": round(len(done) / spent, 3),
            "sample": f"{len(done)} of {w.num_seqs} rows of {w.name} (seeded order), "
                      f"{int(sum(int(w.seq_lens[r]) for r in done))} tokens, {spent:.1f} s of fp64 numpy "
                      f"(gather through the block table + attention), host cores available {cores}"}


# ------------------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by sequence "
              "or KV head with no exchange, but this build measures the one-GPU share", file=sys.stderr)
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

    w = wl.build(args.config, block_size=args.block_size, placement=args.placement,
                 copied_prefix=args.copied_prefix, partition_size=args.partition_size)
    res = time_steps(w, args.steps, args.warmup, decode_only=args.decode_only)
    total_s = res["total_s"]
    gbps = (res["kv_bytes"] + res["table_bytes"]) / total_s / 1e9
    seqs_s = w.num_seqs * args.steps / total_s
    kern = {k: {"launches": n, "avg_us": round(ms / n * 1e3, 2)} for k, (n, ms) in res["kernels"].items()}
    line = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_s / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "seqs": w.num_seqs, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "partition_size": w.partition_size,
                   "placement": w.placement, "total_tokens_at_start": int(res["lens0"].sum()),
                   "seed": w.seed, "step": "decode_only" if args.decode_only else
                   "host append + stage + append_slots + scatter + decode"},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "seqs_per_s": round(seqs_s, 1),
        "kernels": kern,
        "roofline": roofline(res),
    }
    if args.config == 4:
        # unique bytes: the shared prompt is stored (and mostly fetched from HBM) once
        prefix = 4000
        uniq_tokens = prefix + int(sum(int(L) - prefix for L in res["lens0"]))
        line["unique_kv_bytes_per_step"] = uniq_tokens * 2 * w.n_kv_heads * w.head_dim * w.esize
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def sweep(args):
    import workloads as wl
    rows = []
    for B in (8, 16, 32):
        per = {}
        for placement in ("random", "identity"):
            w = wl.build(5, block_size=B, placement=placement, partition_size=args.partition_size or 512)
            res = time_steps(w, args.steps, args.warmup, decode_only=True)
            rf = roofline(res)
            n, ms = res["kernels"]["decode"]
            per[placement] = {"decode_GBps": rf["achieved"], "pct_hbm": round(100 * rf["frac"], 2),
                              "decode_us": rf["avg_launch_us"],
                              "seqs_per_s": round(w.num_seqs / (res["total_s"] / res["steps"]), 1),
                              "call_us": round(res["total_s"] / res["steps"] * 1e6, 2)}
            log(f"B={B} {placement}: {per[placement]}")
        rows.append({"block_size": B, **per,
                     "random_over_identity": round(per["random"]["decode_GBps"] / per["identity"]["decode_GBps"], 4)})
    print(json.dumps({"sweep": "long_context 8 x 65536, bf16, 64q/8kv heads, P=512", "rows": rows}), flush=True)


if __name__ == "__main__":
    main()
