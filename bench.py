#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X: KV append + paged decode attention.

One step = one pass of the whole hot path over the workload's batch: the
append of one new token per sequence and decode attention over every
context.  By default the step is ``paged_attention_decode_append`` (split
pass, then the log-sum-exp merge that also adds and stores the new token);
``--step separate`` times ``paged_kv_write`` followed by the two launches of
``paged_attention_decode`` instead, and each run reports the other form's
time per step too.  Inputs are
seeded synthetic data resident in HBM before timing starts.  The K/V pool is
replicated into several copies that the steps rotate through, so a step never
finds its blocks in L2 / the 256 MB Infinity Cache from the step before.

Prints one JSON line (stdout).  Headline: KV bytes read per second over the
whole step (2 * Hkv * D * 2 bytes per context token), with the split
pass's own rate against HBM peak in "roofline", and the fp64 CPU oracle timed
on a bounded sample of the same workload in "cpu_baseline".
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "paged decode KV-read HBM GB/s (% of peak) + seq-tokens/s, Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0
WORKLOADS = ("llama8b", "long", "prefix", "short_bs8", "short_bs16", "short_bs32", "tiny")
ROOT = os.path.dirname(os.path.abspath(__file__))
SPLIT_KERNEL = "decode_split_kernel"
PREFILL_KERNEL = "prefill_kernel"
PREFILL_TAG = "llama8b_chunks"
# op -> (dominant kernel, its source file)
KERNELS = {"decode": (SPLIT_KERNEL, "pa_decode.hip"), "prefill": (PREFILL_KERNEL, "pa_prefill.hip")}
COPY_BYTES = 512 << 20   # plain device copy used to calibrate the byte counters


def kernel_source_hash(op: str = "decode") -> str:
    import hashlib
    src = os.path.join(ROOT, "pagedattention_kv_cache_paged_amd", "csrc", KERNELS[op][1])
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# Tensor scales of the E4M3 cache for N(0, 1) data: codes stay inside +-448.
FP8_K_SCALE, FP8_V_SCALE = 0.02, 0.02


def kv_bytes_per_token(w, fp8: bool) -> int:
    """K plus V bytes of one context token over all KV heads."""
    return 2 * w.num_kv_heads * w.head_dim * (1 if fp8 else 2)


def counters_path(tag: str, op: str = "decode") -> str:
    return os.path.join(ROOT, "profiles", f"{KERNELS[op][0]}_{tag}_counters.txt")


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, fp8: bool,
                       op: str = "decode") -> dict:
    """Per-launch HBM bytes of the op's dominant kernel (the decode split
    pass, or the prefill kernel) from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads
    for the plain COPY_BYTES device copy of the same run."""
    kernel = KERNELS[op][0]
    import csv
    import glob

    def per_dispatch(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        split, copy = [], []
        for fn in files:
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"]) * 1024.0
                if kernel in r["Kernel_Name"]:
                    split.append(v)
                elif "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= (1 << 16):
                    copy.append(v)
        if not split or not copy:
            raise SystemExit(f"{counter}: found {len(split)} {kernel} and {len(copy)} copy "
                             f"dispatches")
        return float(np.mean(split)), float(np.mean(copy))

    f_split, f_copy = per_dispatch(fetch_dir, "FETCH_SIZE")
    w_split, w_copy = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    opts = ("--op prefill" if op == "prefill" else f"--workload {workload}") + \
        (" --kv-dtype fp8" if fp8 else "")
    return {
        "kernel": kernel, "workload": workload + ("_fp8" if fp8 else ""),
        "source_sha256": kernel_source_hash(op),
        "fetch_bytes_raw": f_split, "write_bytes_raw": w_split,
        "copy_bytes": COPY_BYTES, "copy_fetch_raw": f_copy, "copy_write_raw": w_copy,
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "fetch_bytes": f_split * f_scale, "write_bytes": w_split * w_scale,
        "traffic_bytes": f_split * f_scale + w_split * w_scale,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o cnt -- "
            f"python3 bench.py {opts} --steps 10 --warmup 2 --no-cpu-baseline "
            f"--copy-calibration",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o cnt -- "
            f"python3 bench.py {opts} --steps 10 --warmup 2 --no-cpu-baseline "
            f"--copy-calibration",
            f"python3 bench.py --summarize-counters {fetch_dir} {write_dir} {opts}",
        ],
    }


def recorded_traffic(tag: str, op: str = "decode"):
    """Counter-measured bytes per launch of the op's dominant kernel, if
    recorded for this workload and for the kernel source as it is now; else
    None."""
    try:
        with open(counters_path(tag, op)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != tag or rec.get("source_sha256") != kernel_source_hash(op):
        return None
    return rec.get("traffic_bytes")


def copy_calibration(torch, dev):
    """Three plain COPY_BYTES device copies: what FETCH_SIZE and WRITE_SIZE
    read for them scales the kernel's own counts to bytes."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def make_workload(name, placement="random"):
    from pagedattention_kv_cache_paged_amd import workloads as W
    if name.startswith("short_bs"):
        return W.short(int(name[len("short_bs"):]))
    if name == "llama8b":
        return W.llama8b(placement=placement)
    return W.NAMED[name]()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds: float, fp8: bool = False):
    """The fp64 oracle on the first n sequences, all heads; n grows until
    about `seconds` of single-thread work.  The same rows are then run again
    shared out over a pool of host threads (the C oracle runs outside
    Python's lock), one GPU's share of the host: at most 16 threads, fewer
    if there are fewer rows.  Rates in KV GB/s of the same accounting as the
    GPU figure; the pooled run is the headline figure."""
    import oracle
    kc, vc = w.nan_caches_fp8() if fp8 else w.nan_caches()
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        if fp8:
            oracle.kv_write_fp8(k, v, s, kc, vc, w.block_size, w.dtype, FP8_K_SCALE,
                                FP8_V_SCALE)
        else:
            oracle.kv_write(k, v, s, kc, vc, w.block_size)

    def run(rows, threads):
        if fp8:
            oracle.decode_fp8_rows(rows, w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                   w.block_size, w.dtype, FP8_K_SCALE, FP8_V_SCALE,
                                   threads=threads)
        else:
            oracle.decode_rows(rows, w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                               w.block_size, w.dtype, threads=threads)

    done_tokens, t_total, n = 0, 0.0, 0
    while n < w.num_seqs and t_total < seconds:
        rows = np.array([(n, h) for h in range(w.num_heads)], dtype=np.int32)
        t0 = time.perf_counter()
        run(rows, 1)
        t_total += time.perf_counter() - t0
        done_tokens += int(w.context_lens[n])
        n += 1
    rows = oracle.all_rows(n, w.num_heads)
    threads = min(oracle.host_threads(), rows.shape[0])
    t0 = time.perf_counter()
    run(rows, threads)
    t_pool = time.perf_counter() - t0
    kvb = done_tokens * kv_bytes_per_token(w, fp8)
    sample = (f"first {n} of {w.num_seqs} sequences, all {w.num_heads} query heads "
              f"({done_tokens} context tokens), fp64 C oracle")
    return {"value": round(kvb / t_pool / 1e9, 6), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{sample}, (sequence, head) rows shared out over {threads} threads, "
                      f"{t_pool:.2f} s",
            "seq_tokens_per_s": round(done_tokens / t_pool, 1), "cpu": cpu_model(),
            "host_cpus": os.cpu_count(), "cpus_usable": len(os.sched_getaffinity(0)),
            "single_thread": {"value": round(kvb / t_total / 1e9, 6), "unit": "GB/s",
                              "cores": 1, "seq_tokens_per_s": round(done_tokens / t_total, 1),
                              "sample": f"{sample}, single thread, {t_total:.1f} s"}}


COPY_KERNEL = "copy_blocks_kernel"


def bench_copy_blocks(args, torch, B, W, dev, lib):
    """Copy-on-write at the prefix-sharing shape: 128 sequences forked from a
    1000-token prompt (bs 16, so the prompt's last block holds 8 tokens and is
    shared) each copy that block before their first append: 128 (src, dst)
    pairs, one source, distinct destinations; 8 KV heads, head_dim 128, bf16.
    Bytes per pair: K + V runs of H_kv * bs * D * 2 B, read and written.
    A second figure copies 4096 distinct random pairs (a swap-sized batch)."""
    hkv, d, bs, nforks = 8, 128, 16, 128
    run = hkv * bs * d * 2
    nb = 8192
    g = np.random.default_rng(31)
    ids = g.permutation(nb)
    shared = int(ids[0])
    cow_pairs = np.stack([np.full(nforks, shared), ids[1:1 + nforks]], axis=1).astype(np.int64)
    big_pairs = np.stack([ids[:4096], ids[4096:8192]], axis=1).astype(np.int64)
    kc = torch.randint(-30000, 30000, (nb, hkv, bs, d), dtype=torch.int16, device=dev)
    vc = torch.randint(-30000, 30000, (nb, hkv, bs // 4, d, 4), dtype=torch.int16, device=dev)
    sp = torch.cuda.current_stream().cuda_stream
    stream = torch.cuda.current_stream()

    def timed(pairs_np, K):
        pairs = torch.from_numpy(pairs_np).to(dev)
        n = pairs.shape[0]

        def launch():
            rc = lib.paged_copy_blocks(kc.data_ptr(), vc.data_ptr(), pairs.data_ptr(), n, hkv,
                                       d, bs, nb, 2, sp)
            assert rc == 0, rc
        for _ in range(args.warmup):
            launch()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K * 1e3  # us

    K = args.steps
    t_cow = timed(cow_pairs, K)
    t_big = timed(big_pairs, K)
    cow_bytes = nforks * 2 * run * 2          # K and V runs, read + written
    big_bytes = big_pairs.shape[0] * 2 * run * 2
    gbs = cow_bytes / (t_cow * 1e-6) / 1e9
    big_gbs = big_bytes / (t_big * 1e-6) / 1e9
    result = {
        "metric": "copy-on-write block copy GB/s (read + written), prefix-sharing shape",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(t_cow * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefix CoW: {nforks} forks copy one shared partly-filled "
                               f"block; {hkv} kv heads, head_dim {d}, block {bs}, bf16",
                   "pairs": nforks, "bytes_per_pair": 2 * run * 2},
        "roofline": {"kernel": COPY_KERNEL, "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(t_cow, 3), "traffic": None,
                     "bytes_per_launch": cow_bytes},
        "batch_4096_pairs": {"us": round(t_big, 3), "GB/s": round(big_gbs, 2),
                             "frac": round(big_gbs / HBM_PEAK_GBS, 4),
                             "bytes_per_launch": big_bytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        hk = kc[:].cpu().numpy().view(np.uint16)
        hv = vc[:].cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.copy_blocks(cow_pairs, hk, hv, bs)
            reps += 1
        t_cpu = (time.perf_counter() - t0) / reps
        result["cpu_baseline"] = {"value": round(cow_bytes / t_cpu / 1e9, 6), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"the same {nforks} pairs, {reps} repetitions, "
                                            f"the oracle's byte copy, single thread"}
    print(json.dumps(result), flush=True)


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def bench_swap_blocks(args, torch, B, dev, lib):
    """Preemption-sized swap at the Llama-3-8B head shape (8 KV heads,
    head_dim 128, block 16, bf16: 32 KiB per block per cache): 1024 random
    device blocks out to a pinned host pool, then back into other device
    blocks.  Bytes per block: K + V runs (64 KiB) crossing the host link."""
    hkv, d, bs, n = 8, 128, 16, 1024
    run = hkv * bs * d * 2
    nd = 8192
    g = np.random.default_rng(41)
    ids = g.permutation(nd)
    out_pairs = torch.from_numpy(np.stack([ids[:n], np.arange(n)], 1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), ids[n:2 * n]], 1).astype(np.int64)).to(dev)
    kc = torch.randint(-30000, 30000, (nd, hkv, bs, d), dtype=torch.int16, device=dev)
    vc = torch.randint(-30000, 30000, (nd, hkv, bs // 4, d, 4), dtype=torch.int16, device=dev)
    hk = torch.empty((n, hkv, bs, d), dtype=torch.int16).pin_memory()
    hv = torch.empty((n, hkv, bs // 4, d, 4), dtype=torch.int16).pin_memory()
    sp = torch.cuda.current_stream().cuda_stream
    stream = torch.cuda.current_stream()

    def swap(pairs, dk, dv, dn, sk, sv, sn):
        rc = lib.paged_swap_blocks(dk.data_ptr(), dv.data_ptr(), dn, sk.data_ptr(),
                                   sv.data_ptr(), sn, pairs.data_ptr(), n, hkv, d, bs, 2, sp)
        assert rc == 0, rc

    def timed(fn, K):
        for _ in range(min(args.warmup, 3)):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K * 1e3

    K = max(1, min(args.steps, 20))
    t_out = timed(lambda: swap(out_pairs, hk, hv, n, kc, vc, nd), K)
    t_in = timed(lambda: swap(in_pairs, kc, vc, nd, hk, hv, n), K)
    nbytes = n * 2 * run
    gb_out, gb_in = nbytes / (t_out * 1e-6) / 1e9, nbytes / (t_in * 1e-6) / 1e9
    result = {
        "metric": "KV block swap GB/s over the host link (out and in), Llama-3-8B head shape",
        "value": round(nbytes * 2 / ((t_out + t_in) * 1e-6) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": min(args.warmup, 3),
        "ms_per_step": round((t_out + t_in) * 1e-3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"swap {n} blocks out to pinned host memory and back into "
                               f"other device blocks; {hkv} kv heads, head_dim {d}, block "
                               f"{bs}, bf16", "blocks": n, "bytes_per_block": 2 * run},
        "swap_out": {"us": round(t_out, 2), "GB/s": round(gb_out, 2)},
        "swap_in": {"us": round(t_in, 2), "GB/s": round(gb_in, 2)},
        "roofline": {"kernel": COPY_KERNEL, "bound": "host link",
                     "achieved": round(max(gb_out, gb_in), 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(max(gb_out, gb_in) / HOST_LINK_PEAK_GBS, 4),
                     "avg_launch_us": round(min(t_out, t_in), 3), "traffic": None,
                     "bytes_per_launch": nbytes},
    }
    print(json.dumps(result), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 MFMA, MI355X


def bench_prefill(args, torch, B, W, dev, lib, fp8=False):
    """Chunked prefill at the Llama-3-8B shape: 8 sequences, each with 1536
    cached tokens and a 512-token chunk (32 q / 8 kv heads, head_dim 128,
    block 16, bf16, random block placement; with fp8, E4M3 caches and bf16
    q / out).  Algorithmic flops: for each chunk row at position p and each
    query head, 2*D*(p+1) for q K^T and the same for P V."""
    nseq, cached, chunk = 8, 1536, 512
    w = W.build("prefill", [cached + chunk] * nseq, num_heads=32, num_kv_heads=8,
                head_dim=128, block_size=16, dtype=W.BF16, seed=61)
    tdt = torch.bfloat16

    def dev_bits(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    ks, vs = w.cache_shapes()
    kc = torch.zeros(ks, dtype=torch.uint8 if fp8 else tdt, device=dev)
    vc = torch.zeros(vs, dtype=torch.uint8 if fp8 else tdt, device=dev)
    for which in ("hist", "new"):
        k, v, sl = w.write_batch(which)
        if fp8:
            B.paged_kv_write_fp8(dev_bits(k), dev_bits(v), torch.from_numpy(sl).to(dev), kc, vc,
                                 FP8_K_SCALE, FP8_V_SCALE)
        else:
            B.paged_kv_write(dev_bits(k), dev_bits(v), torch.from_numpy(sl).to(dev), kc, vc)
    qs_np = (np.arange(nseq + 1) * chunk).astype(np.int32)
    g = np.random.default_rng(62)
    q_bits = W.normal_bits(g, (nseq * chunk, 32, 128), W.BF16)
    q = dev_bits(q_bits)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    qs = torch.from_numpy(qs_np).to(dev)
    sp = torch.cuda.current_stream().cuda_stream
    stream = torch.cuda.current_stream()

    def launch():
        if fp8:
            rc = lib.paged_attention_prefill_fp8(
                out.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(),
                cl.data_ptr(), qs.data_ptr(), w.scale, FP8_K_SCALE, FP8_V_SCALE, 16, 8, nseq,
                32, 128, w.max_blocks_per_seq, w.num_blocks, 1, chunk, sp)
        else:
            rc = lib.paged_attention_prefill(out.data_ptr(), q.data_ptr(), kc.data_ptr(),
                                             vc.data_ptr(), bt.data_ptr(), cl.data_ptr(),
                                             qs.data_ptr(), w.scale, 16, 8, nseq, 32, 128,
                                             w.max_blocks_per_seq, w.num_blocks, 1, chunk, sp)
        assert rc == 0, rc
    # untimed warm-up long enough (~50 ms of launches) for the clocks to settle
    nwarm = max(args.warmup, 300)
    for _ in range(nwarm):
        launch()
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        launch()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / K * 1e3
    if args.copy_calibration:
        copy_calibration(torch, dev)
    positions = np.arange(cached, cached + chunk, dtype=np.float64)
    flops = nseq * 32 * float(np.sum(4.0 * 128 * (positions + 1)))
    tflops = flops / (us * 1e-6) / 1e12
    result = {
        "metric": "paged chunked-prefill attention TFLOP/s (% of MFMA peak), Llama-3-8B shape",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": nwarm, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"chunked prefill: {nseq} sequences x {chunk}-token chunk after "
                               f"{cached} cached tokens; 32 q / 8 kv heads, head_dim 128, "
                               f"block 16, bf16" + (", E4M3 KV cache" if fp8 else ""),
                   "rows": nseq * chunk, "kv_dtype": "e4m3" if fp8 else "bf16",
                   "context_tokens": nseq * (cached + chunk)},
        "tokens_per_s": round(nseq * chunk / (us * 1e-6), 1),
        "roofline": {"kernel": PREFILL_KERNEL, "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "avg_launch_us": round(us, 3),
                     "traffic": recorded_traffic(PREFILL_TAG + ("_fp8" if fp8 else ""),
                                                 "prefill"),
                     "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        import oracle
        okc, ovc = w.nan_caches_fp8() if fp8 else w.nan_caches()
        for which in ("hist", "new"):
            k, v, sl = w.write_batch(which)
            if fp8:
                oracle.kv_write_fp8(k, v, sl, okc, ovc, 16, W.BF16, FP8_K_SCALE, FP8_V_SCALE)
            else:
                oracle.kv_write(k, v, sl, okc, ovc, 16)
        done, fl, t_total = 0, 0.0, 0.0
        while done < chunk and t_total < min(args.cpu_seconds, 15.0):
            p = cached + done   # rows of sequence 0, one at a time
            t0 = time.perf_counter()
            one = (q_bits[done:done + 1], okc, ovc, w.block_tables[:1],
                   np.array([p + 1], np.int32), np.array([0, 1], np.int32), w.scale, 16, W.BF16)
            if fp8:
                oracle.prefill_fp8(*one, FP8_K_SCALE, FP8_V_SCALE)
            else:
                oracle.prefill(*one)
            t_total += time.perf_counter() - t0
            fl += 32 * 4.0 * 128 * (p + 1)
            done += 1
        result["cpu_baseline"] = {"value": round(fl / t_total / 1e12, 9), "unit": "TFLOP/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"the first {done} chunk rows of sequence 0, all 32 "
                                            f"heads, fp64 C oracle, single thread, "
                                            f"{t_total:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b", choices=WORKLOADS)
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library default)")
    ap.add_argument("--copies", type=int, default=0, help="pool copies rotated (0 = enough for >1 GB)")
    ap.add_argument("--placement", default="random", choices=("random", "identity"),
                    help="physical block placement of the llama8b workload")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", default="decode",
                    choices=("decode", "copy_blocks", "swap_blocks", "prefill"),
                    help="decode: the decode step (default); copy_blocks: the copy-on-write "
                         "block copy of 128 forks of a shared prompt (prefix-sharing shape); "
                         "swap_blocks: swap 1024 blocks out to pinned host memory and back; "
                         "prefill: 512-token chunks after 1536 cached tokens, 8 sequences")
    ap.add_argument("--step", default="fused", choices=("fused", "separate"),
                    help="fused: paged_attention_decode_append (two launches); separate: "
                         "paged_kv_write + paged_attention_decode (three launches)")
    ap.add_argument("--kv-dtype", default="native", choices=("native", "fp8"),
                    help="KV cache element type: the workload's 16-bit type, or E4M3 codes")
    ap.add_argument("--no-shared-path", action="store_true",
                    help="prefix workload: decode without telling the library about the "
                         "shared prefix (every sequence streams it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (byte-counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the dominant kernel's per-launch HBM bytes (decode split pass or "
                         "prefill kernel) from two rocprofv3 --pmc runs to profiles/ and exit")
    args = ap.parse_args()

    fp8 = args.kv_dtype == "fp8"
    cop = "prefill" if args.op == "prefill" else "decode"
    base = PREFILL_TAG if cop == "prefill" else args.workload
    tag = base + ("_fp8" if fp8 else "")
    if args.summarize_counters:
        if args.op not in ("decode", "prefill"):
            raise SystemExit("--summarize-counters covers --op decode and --op prefill")
        rec = summarize_counters(*args.summarize_counters, base, fp8, cop)
        os.makedirs(os.path.dirname(counters_path(tag, cop)), exist_ok=True)
        with open(counters_path(tag, cop), "w") as f:
            f.write(json.dumps(rec, indent=1) + "\n")
        print(json.dumps(rec))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU path only: the library has no multi-GPU "
              "code (the decode shards by sequence or KV head with no exchange); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from pagedattention_kv_cache_paged_amd import binding as B
    from pagedattention_kv_cache_paged_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = B.load()
    if args.op == "copy_blocks":
        return bench_copy_blocks(args, torch, B, W, dev, lib)
    if args.op == "swap_blocks":
        return bench_swap_blocks(args, torch, B, dev, lib)
    if args.op == "prefill":
        return bench_prefill(args, torch, B, W, dev, lib, fp8)
    w = make_workload(args.workload, args.placement)
    tdt = {W.F16: torch.float16, W.BF16: torch.bfloat16}[w.dtype]

    def dev_bits(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    ks, vs = w.cache_shapes()
    pool_bytes = 2 * int(np.prod(ks)) * (1 if fp8 else 2)
    copies = args.copies or max(4, math.ceil(1.1e9 / pool_bytes))
    nan_i16 = int(np.array([W.NAN_BITS[w.dtype]], np.uint16).view(np.int16)[0])
    hk, hv, hs = w.write_batch("hist")
    nk, nv, ns = w.write_batch("new")
    hk, hv, hs = dev_bits(hk), dev_bits(hv), torch.from_numpy(hs).to(dev)
    nk, nv, ns = dev_bits(nk), dev_bits(nv), torch.from_numpy(ns).to(dev)
    caches = []
    for _ in range(copies):
        if fp8:
            kc = torch.full(ks, W.FP8_NAN, dtype=torch.uint8, device=dev)
            vc = torch.full(vs, W.FP8_NAN, dtype=torch.uint8, device=dev)
            if hs.numel():
                B.paged_kv_write_fp8(hk, hv, hs, kc, vc, FP8_K_SCALE, FP8_V_SCALE)
        else:
            kc = torch.full(ks, nan_i16, dtype=torch.int16, device=dev).view(tdt)
            vc = torch.full(vs, nan_i16, dtype=torch.int16, device=dev).view(tdt)
            if hs.numel():
                B.paged_kv_write(hk, hv, hs, kc, vc)
        caches.append((kc, vc))
    del hk, hv, hs
    q = dev_bits(w.q)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    pt = args.partition
    # shared prefix: the leading table entries every sequence holds by reference
    sb = 0 if args.no_shared_path else w.shared_tokens // w.block_size
    waves = B.split_waves(w.num_seqs, w.num_kv_heads, w.max_blocks_per_seq, w.block_size, pt)
    ws_need = B.workspace_bytes_shared(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                       w.max_blocks_per_seq, w.block_size, sb, pt)
    ws = torch.empty(max(ws_need, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # Pre-marshalled C calls: the host stays well ahead of the GPU.
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    dtc = {W.F16: 0, W.BF16: 1}[w.dtype]
    T = w.num_seqs

    def write(i):
        kc, vc = caches[i % copies]
        if fp8:
            rc = lib.paged_kv_write_fp8(nk.data_ptr(), nv.data_ptr(), ns.data_ptr(),
                                        kc.data_ptr(), vc.data_ptr(), T, w.num_kv_heads,
                                        w.head_dim, w.block_size, w.num_blocks, dtc,
                                        FP8_K_SCALE, FP8_V_SCALE, sp)
        else:
            rc = lib.paged_kv_write(nk.data_ptr(), nv.data_ptr(), ns.data_ptr(), kc.data_ptr(),
                                    vc.data_ptr(), T, w.num_kv_heads, w.head_dim,
                                    w.block_size, w.num_blocks, dtc, sp)
        assert rc == 0, rc

    def decode(i, stages):
        kc, vc = caches[i % copies]
        if sb:
            rc = lib.paged_attention_decode_shared(
                out.data_ptr(), q.data_ptr(), None, None, kc.data_ptr(), vc.data_ptr(),
                bt.data_ptr(), cl.data_ptr(), w.scale, FP8_K_SCALE, FP8_V_SCALE, w.block_size,
                w.num_kv_heads, w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq,
                w.num_blocks, dtc, 1 if fp8 else 0, sb, pt, ws.data_ptr(), ws.numel(), stages,
                sp)
        elif fp8:
            rc = lib.paged_attention_decode_fp8(
                out.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(),
                cl.data_ptr(), w.scale, FP8_K_SCALE, FP8_V_SCALE, w.block_size,
                w.num_kv_heads, w.num_seqs, w.num_heads, w.head_dim, w.max_blocks_per_seq,
                w.num_blocks, dtc, pt, ws.data_ptr(), ws.numel(), stages, sp)
        else:
            rc = lib.paged_attention_decode_stages(
                out.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(),
                cl.data_ptr(), w.scale, w.block_size, w.num_kv_heads, w.num_seqs,
                w.num_heads, w.head_dim, w.max_blocks_per_seq, w.num_blocks, dtc, pt,
                ws.data_ptr(), ws.numel(), stages, sp)
        assert rc == 0, rc

    def fused(i, stages=3):
        kc, vc = caches[i % copies]
        if sb:
            rc = lib.paged_attention_decode_shared(
                out.data_ptr(), q.data_ptr(), nk.data_ptr(), nv.data_ptr(), kc.data_ptr(),
                vc.data_ptr(), bt.data_ptr(), cl.data_ptr(), w.scale, FP8_K_SCALE, FP8_V_SCALE,
                w.block_size, w.num_kv_heads, w.num_seqs, w.num_heads, w.head_dim,
                w.max_blocks_per_seq, w.num_blocks, dtc, 1 if fp8 else 0, sb, pt,
                ws.data_ptr(), ws.numel(), stages, sp)
            assert rc == 0, rc
            return
        rc = lib.paged_attention_decode_append_stages(
            out.data_ptr(), q.data_ptr(), nk.data_ptr(), nv.data_ptr(), kc.data_ptr(),
            vc.data_ptr(), bt.data_ptr(), cl.data_ptr(), w.scale, FP8_K_SCALE, FP8_V_SCALE,
            w.block_size, w.num_kv_heads, w.num_seqs, w.num_heads, w.head_dim,
            w.max_blocks_per_seq, w.num_blocks, dtc, 1 if fp8 else 0, pt, ws.data_ptr(),
            ws.numel(), stages, sp)
        assert rc == 0, rc

    def separate(i):
        write(i)
        decode(i, 1)
        decode(i, 2)

    steps = {"fused": fused, "separate": separate}
    step = steps[args.step]
    for i in range(args.warmup):
        for f in steps.values():
            f(i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, nothing else on the stream.
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / K

    # The other form of the step, timed the same way (informative).
    other = "separate" if args.step == "fused" else "fused"
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0.record(stream)
    for i in range(K):
        steps[other](i)
    o1.record(stream)
    torch.cuda.synchronize()
    ms_other = o0.elapsed_time(o1) / K

    def back_to_back(fn):
        """Average duration of K back-to-back calls of fn(i) on the launch
        stream, bracketed by two events (no event overhead between them)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e3   # us

    # Roofline of the dominant kernel: the split pass of the step timed above
    # (the fused step's variant, which also stores the new tokens), alone.
    t_split = back_to_back(lambda i: fused(i, 1))
    # The plain decode's split pass, and the decode alone (split + merge, no
    # append: attention over the block tables).
    t_split_plain = back_to_back(lambda i: decode(i, 1))
    t_decode = back_to_back(lambda i: decode(i, 3))

    # Per-launch breakdown (informative): the same K steps again with events
    # between the launches, which adds the events' own overhead.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        write(i)
        e[1].record(stream)
        decode(i, 1)
        e[2].record(stream)
        decode(i, 2)
        e[3].record(stream)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch, dev)
    t_write = np.mean([e[0].elapsed_time(e[1]) for e in ev]) * 1e3   # us
    t_part = np.mean([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    t_merge = np.mean([e[2].elapsed_time(e[3]) for e in ev]) * 1e3
    p_part = np.percentile([e[1].elapsed_time(e[2]) * 1e3 for e in ev], [10, 50, 90])

    # KV bytes the step must bring from HBM: every distinct block once.  With
    # shared prefix blocks the logical bytes (each sequence's whole context)
    # exceed them and are reported beside, since repeat reads of a shared
    # block can be served by the caches.
    logical_bytes = w.logical_tokens * kv_bytes_per_token(w, fp8)
    kv_bytes = w.unique_tokens * kv_bytes_per_token(w, fp8)
    gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (t_split * 1e-6) / 1e9
    dec_gbs = kv_bytes / (t_decode * 1e-6) / 1e9
    # cache slots the sequences hold (whole blocks) against tokens stored
    slots_held = sum(-(-int(L) // w.block_size) * w.block_size for L in w.context_lens)
    if w.shared_tokens:
        slots_held -= (w.num_seqs - 1) * w.shared_tokens
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {W.F16: "f16", W.BF16: "bf16"}[w.dtype],
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: batch {w.num_seqs}, {w.num_heads} q / {w.num_kv_heads} kv "
                        f"heads, head_dim {w.head_dim}, block {w.block_size}, "
                        f"{w.logical_tokens} context tokens"
                        + (", E4M3 KV cache" if fp8 else ""),
            "batch": w.num_seqs, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size,
            "kv_dtype": "e4m3" if fp8 else w.dtype,
            "context_tokens": w.logical_tokens, "partition_tokens": pt,
            "waves_per_kv_head": waves,
            "pool_copies": copies, "pool_mb_per_copy": round(pool_bytes / 2**20, 1),
            "placement": args.placement if args.workload == "llama8b" else "random",
            "shared_blocks": sb,
        },
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "step": args.step,
        f"ms_per_step_{other}": round(ms_other, 5),
        "seq_tokens_per_s": round(w.logical_tokens / (ms_step * 1e-3), 1),
        "new_tokens_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "split_us_back_to_back": round(t_split, 3),
        "split_plain_us_back_to_back": round(t_split_plain, 3),
        "t_decode": {"us": round(t_decode, 3), "GB/s": round(dec_gbs, 2),
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "seq_tokens_per_s": round(w.logical_tokens / (t_decode * 1e-6), 1),
                     "what": "split pass + merge pass back to back, no append (the append "
                             "is timed separately in kernel_us_event_bracketed.kv_write)"},
        "cache_tokens_per_slot": round(w.unique_tokens / slots_held, 4),
        "kernel_us_event_bracketed": {
            "kv_write": round(t_write, 3), "decode_split": round(t_part, 3),
            "decode_merge": round(t_merge, 3),
            "decode_split_p10_p50_p90": [round(x, 3) for x in p_part]},
        "host_wall_ms_per_step": round(t_wall * 1e3 / K, 5),
        "roofline": {
            "kernel": "decode_split_kernel (fused-append variant)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(t_split, 3),
            "traffic": recorded_traffic(tag),
            "bytes_per_launch": kv_bytes,
        },
    }
    if logical_bytes != kv_bytes:
        result["logical_kv_gbs"] = round(logical_bytes / (ms_step * 1e-3) / 1e9, 2)
        result["logical_bytes_per_launch"] = logical_bytes
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, fp8)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
