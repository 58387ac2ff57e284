#!/usr/bin/env python3
"""Benchmark of the paged-KV decode hot path on one MI355X.

One step = one pass of the hot path over one synthetic batch:
  kv_append of the batch's current tokens (one per sequence), then
  paged_decode_attn over every sequence's cached keys (split-KV partitions
  plus the log-sum-exp merge).
Default workload: Llama-3.1-8B-shaped single-layer decode, batch 64,
32 query / 8 KV heads, head_dim 128, context ~ U[512, 4096], 16-token
blocks, shuffled pool of used blocks + 10 % (about 0.65 GB of bf16 K/V, more
than the 256 MB Infinity Cache, so the pool is read from HBM every step).

Prints ONE JSON line.  `value` = KV bytes the decode must read
(sum_i ctx_i * 2 * Hkv * D * 2) / wall time per step, in GB/s, over K steps
timed with nothing recorded between them; seq-steps/s and the split into
kernels go in extra keys.  The per-call durations behind `roofline` come
from a second pass of K steps with HIP events around each call on the
library's stream (events between kernels lengthen the steps they sit in).
Inputs are resident in HBM before the timed region starts.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, published


def attention_flops(w):
    """Exact causal FLOPs: 2 D for q.k and 2 D for p.v per visible (query, key)
    pair and query head."""
    pairs = 0
    for c, lq in zip(w.context_lens, w.q_lens):
        # rows at positions c - lq .. c - 1 see c - lq + 1 .. c keys
        pairs += lq * (c - lq) + lq * (lq + 1) // 2
    return 4 * w.head_dim * w.num_q_heads * pairs


def hbm_traffic(workload_name):
    """HBM bytes per call (read + written) of the attention kernels, from the
    rocprofv3 byte counters recorded in profiles/hbm_traffic.json, scaled by
    the same counters' reading for a plain device copy; None when the
    recorded kernel sources differ from the ones in this tree."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        wl = rec["workloads"][workload_name]
        for src, digest in wl["sources_sha256"].items():
            with open(os.path.join(ROOT, src), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        cal = rec["calibration"]
        fs = cal["copy_bytes_read"] / (cal["fetch_kib"] * 1024.0)
        ws = cal["copy_bytes_written"] / (cal["write_kib"] * 1024.0)
        return round(sum(k["fetch_kib"] * 1024.0 * fs + k["write_kib"] * 1024.0 * ws
                         for k in wl["kernels"].values()))
    except (OSError, KeyError, ValueError):
        return None


# What each recorded workload's traffic covers: the kernels whose counters are
# summed per call, the sources they are built from (a change to any of them
# voids the record), and the bench.py arguments the counters are taken on.
_DECODE_SRC = ["paged_kv_cache_98_amd/csrc/decode.hip", "paged_kv_cache_98_amd/csrc/decode_core.h",
               "paged_kv_cache_98_amd/csrc/pkv_device.h"]
_PREFILL_SRC = ["paged_kv_cache_98_amd/csrc/prefill.hip", "paged_kv_cache_98_amd/csrc/decode_core.h",
                "paged_kv_cache_98_amd/csrc/pkv_device.h"]
_DECODE_K = ["decode_streamk_kernel", "decode_merge_kernel"]
TRAFFIC_SPEC = {
    "llama8b_decode_b64": {"kernels": _DECODE_K, "sources": _DECODE_SRC, "args": ""},
    "long_context_decode_b8": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                               "args": "--workload long_context_decode"},
    "llama70b_decode_b256_bs16": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                                  "args": "--workload llama70b_decode_bs16"},
    "llama70b_decode_b256_bs32": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                                  "args": "--workload llama70b_decode_bs32"},
    "mixed_prefill_c4x512_d0": {"kernels": ["prefill_mfma_kernel"], "sources": _PREFILL_SRC,
                                "args": "--workload prefill_chunks"},
    "mixed_prefill_c4x512_d128": {"kernels": ["mixed_kernel", "decode_merge_kernel"],
                                  "sources": _PREFILL_SRC + ["paged_kv_cache_98_amd/csrc/decode.hip"],
                                  "args": "--workload mixed_prefill"},
    "llama8b_decode_b64_fp8": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                               "args": "--workload llama8b_decode_fp8"},
    "llama70b_decode_b256_bs16_fp8": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                                      "args": "--workload llama70b_decode_bs16_fp8"},
    # the verify batches (6 rows, or 16-node trees, at 4 query heads per KV
    # head) take the rows path: the decode kernels
    "spec_verify_b64_q6": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                           "args": "--workload spec_verify"},
    "spec_verify_b8_q6": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                          "args": "--workload spec_verify_long"},
    "spec_tree_b64_n16": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                          "args": "--workload spec_verify_tree"},
    "spec_verify_b64_q6_fp8": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                               "args": "--workload spec_verify_fp8"},
    "mixed_prefill_c4x512_d0_fp8": {"kernels": ["prefill_mfma_kernel"], "sources": _PREFILL_SRC,
                                    "args": "--workload prefill_chunks_fp8"},
    # FP8 pools with per-(block, KV head) scales
    "llama8b_decode_b64_fp8_per_block": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                                         "args": "--workload llama8b_decode_fp8_per_block"},
    "spec_verify_b64_q6_fp8_per_block": {"kernels": _DECODE_K, "sources": _DECODE_SRC,
                                         "args": "--workload spec_verify_fp8_per_block"},
    "mixed_prefill_c4x512_d0_fp8_per_block": {"kernels": ["prefill_mfma_kernel"],
                                              "sources": _PREFILL_SRC,
                                              "args": "--workload prefill_chunks_fp8_per_block"},
    "cow_copy_4096x32k": {"kernels": ["copy_blocks_kernel"],
                          "sources": ["paged_kv_cache_98_amd/csrc/kv_append.hip"],
                          "args": "--workload cow_copy"},
}


def _pmc_per_dispatch(run_dir, kernel_substrings):
    """Mean per-dispatch counter value (KiB) of each matching kernel in a
    rocprofv3 --pmc CSV output directory."""
    import collections
    import csv
    import glob
    import re
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if not any(k in name for k in kernel_substrings):
                    continue
                m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
                per[m.group(1) if m else name][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(d.values()) / len(d) for k, d in per.items() if d}


def record_traffic(workload, fetch_dir, write_dir):
    """Write workload's entry of profiles/hbm_traffic.json from a FETCH_SIZE and
    a WRITE_SIZE run (``calibration`` takes the plain-copy runs instead)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    if workload == "calibration":
        fetch = _pmc_per_dispatch(fetch_dir, ["__amd_rocclr_copyBuffer"])
        write = _pmc_per_dispatch(write_dir, ["__amd_rocclr_copyBuffer"])
        (fk,), (wk,) = fetch.values(), write.values()
        rec["calibration"].update({"fetch_kib": round(fk, 1), "write_kib": round(wk, 1)})
    else:
        spec = TRAFFIC_SPEC[workload]
        fetch = _pmc_per_dispatch(fetch_dir, spec["kernels"])
        write = _pmc_per_dispatch(write_dir, spec["kernels"])
        if not fetch or set(fetch) != set(write):
            raise SystemExit(f"counter runs disagree on kernels: {sorted(fetch)} vs {sorted(write)}")
        digests = {}
        for src in spec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                digests[src] = hashlib.sha256(f.read()).hexdigest()
        rec["workloads"][workload] = {
            "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> "
                       "-o p -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline "
                       + spec["args"],
            "sources_sha256": digests,
            "kernels": {k: {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1)}
                        for k in sorted(fetch)},
        }
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["workloads"].get(workload, rec["calibration"]), indent=1))


# the kernels one paged_decode_attn call launches
DECODE_KERNEL = "paged_decode_attn (stream-K decode + merge kernels)"


def decode_kv_bytes(w):
    return sum(c for c, lq in zip(w.context_lens, w.q_lens) if lq == 1) * w.kv_token_bytes()


COPY_WORKLOAD = "cow_copy_4096x32k"


def bench_copy_blocks(args):
    """copy_blocks on its own: 4096 (source, destination) pairs of
    Llama-3.1-8B-shaped blocks (16 tokens x 8 KV heads x 128 x bf16 = 32 KiB
    of K and as much of V) in a 16384-block pool (0.5 GiB per pool, so the
    copies stream from HBM), destinations distinct and never a source.  Bytes
    per pair: K and V blocks each read once and written once = 128 KiB.
    Also times the native block manager on the host: one decode step of 256
    beams (64 prompts x 4 beams, forked after a 1000-token prompt) = one
    batched append of a token per beam (returning slots and copies) and the
    block table of all beams, both through the Python binding; and the
    prefix cache: 64 prompts sharing an 800-token system prompt, each
    allocated with its block lookups (microseconds per prompt)."""
    import numpy as np
    import torch
    from paged_kv_cache_98_amd import binding as pkv

    nb, bs, hkv, d, npairs = 16384, 16, 8, 128, 4096
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(2024)
    k = torch.randn((nb, bs, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((nb, bs, hkv, d), generator=g, device=dev).to(torch.bfloat16)
    rng = np.random.default_rng(2025)
    perm = rng.permutation(nb)
    pairs_np = np.stack([rng.choice(perm[npairs:], size=npairs), perm[:npairs]], 1).astype(np.int64)
    pairs = torch.from_numpy(pairs_np).to(dev)
    stream = torch.cuda.current_stream()
    block_bytes = bs * hkv * d * 2
    bytes_per_call = npairs * 4 * block_bytes
    for _ in range(args.warmup):
        pkv.copy_blocks(k, v, pairs, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pkv.copy_blocks(k, v, pairs, stream=stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        pkv.copy_blocks(k, v, pairs, stream=stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    call_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    achieved = bytes_per_call / (call_ms * 1e-3) / 1e9

    # host manager: 64 prompts x 4 beams, 6 decode steps timed
    with pkv.BlockManager(64 * 4 * 80, bs) as bm:
        beams = []
        for p in range(64):
            bm.allocate(p * 10, 1000)
            for j in range(1, 5):
                bm.fork(p * 10, p * 10 + j)
                beams.append(p * 10 + j)
            bm.free(p * 10)
        host_us = []
        beams = torch.tensor(beams, dtype=torch.int64)
        ones = torch.ones(len(beams), dtype=torch.int64)
        for _ in range(6):
            t1 = time.perf_counter()
            bm.append_batch(beams, ones)
            bm.block_table(beams, 80)
            host_us.append((time.perf_counter() - t1) * 1e6)
    # prefix cache: 64 prompts = one 800-token system prompt + a private tail
    # ~ U[64, 2048] (the mixed batch's shape), allocated with lookups
    gp = torch.Generator().manual_seed(2026)
    system = torch.randint(0, 32000, (800,), generator=gp, dtype=torch.int32)
    tails = torch.randint(64, 2049, (64,), generator=gp).tolist()
    prompts = [torch.cat([system, torch.randint(0, 32000, (t,), generator=gp, dtype=torch.int32)])
               for t in tails]
    with pkv.BlockManager(16384, bs) as bm:
        t1 = time.perf_counter()
        cached = [bm.allocate_cached(i, p) for i, p in enumerate(prompts)]
        pc_us = (time.perf_counter() - t1) * 1e6 / len(prompts)
    prompt_tokens = sum(p.numel() for p in prompts)
    print(f"[bench] prefix cache: {pc_us:.1f} us per prompt (64 prompts), "
          f"{sum(cached)} of {prompt_tokens} prompt tokens cached", file=sys.stderr, flush=True)
    # radix-tree sharing: the same tails after a 1000-token shared prefix,
    # which does not end on a block edge (62 blocks + 8 tokens)
    system2 = torch.randint(0, 32000, (1000,), generator=gp, dtype=torch.int32)
    prompts2 = [torch.cat([system2, p[800:]]) for p in prompts]
    with pkv.BlockManager(16384, bs) as bm:
        t1 = time.perf_counter()
        radix = [bm.allocate_radix(i, p) for i, p in enumerate(prompts2)]
        rx_us = (time.perf_counter() - t1) * 1e6 / len(prompts2)
    with pkv.BlockManager(16384, bs) as bm:
        chain2 = [bm.allocate_cached(i, p) for i, p in enumerate(prompts2)]
    rx_tokens = sum(p.numel() for p in prompts2)
    print(f"[bench] radix prefix sharing: {rx_us:.1f} us per prompt (64 prompts), "
          f"{sum(r[0] for r in radix)} of {rx_tokens} prompt tokens cached "
          f"({sum(chain2)} by whole blocks)", file=sys.stderr, flush=True)
    print(f"[bench] copy_blocks {call_ms * 1e3:.1f} us per call of {npairs} pairs: "
          f"{achieved:.0f} GB/s | host manager {statistics.median(host_us):.0f} us per "
          f"256-beam step", file=sys.stderr, flush=True)
    rec = {
        "metric": "copy_blocks (copy-on-write block copies): HBM GB/s",
        "value": round(bytes_per_call / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": COPY_WORKLOAD, "num_pairs": npairs, "num_blocks": nb,
                   "block_size": bs, "num_kv_heads": hkv, "head_dim": d},
        "kernels_us": {"copy_blocks": round(call_ms * 1e3, 2)},
        "host_block_manager_us_per_256_beam_step": round(statistics.median(host_us), 1),
        "host_prefix_cache": {"us_per_prompt": round(pc_us, 1), "prompts": len(prompts),
                              "prompt_tokens": prompt_tokens, "cached_tokens": sum(cached)},
        "host_radix_prefix": {"us_per_prompt": round(rx_us, 1), "prompts": len(prompts2),
                              "prompt_tokens": rx_tokens,
                              "cached_tokens": sum(r[0] for r in radix),
                              "block_cache_cached_tokens": sum(chain2),
                              "copies": sum(r[1] is not None for r in radix)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": hbm_traffic(COPY_WORKLOAD),
                     "kernel": "copy_blocks", "algorithmic_bytes_per_launch": bytes_per_call},
    }
    if not args.no_cpu_baseline:
        from oracle.blocks import copy_blocks as oracle_copy_blocks
        sample = 512
        kc = k[:nb // 4].view(torch.int16).cpu().numpy()
        vc = v[:nb // 4].view(torch.int16).cpu().numpy()
        sp = pairs_np[(pairs_np < nb // 4).all(1)][:sample]
        t2 = time.perf_counter()
        oracle_copy_blocks(kc, vc, sp.tolist())
        dt = time.perf_counter() - t2
        rec["cpu_baseline"] = {
            "value": round(len(sp) * 4 * block_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(sp)} pairs of the same mapping inside a {nb // 4}-block host copy "
                      f"of the pools (numpy, one thread): {dt * 1e3:.1f} ms including its "
                      f"copy of both pools"}
    print(json.dumps(rec), flush=True)


def workload_by_name(name):
    from paged_kv_cache_98_amd import workloads as W
    table = {
        "llama8b_decode": lambda: W.llama8b_decode(),
        "long_context_decode": lambda: W.long_context_decode(),
        "llama70b_decode_bs16": lambda: W.llama70b_decode(block_size=16),
        "llama70b_decode_bs32": lambda: W.llama70b_decode(block_size=32),
        "tiny_decode": lambda: W.tiny_decode(),
        # the 8B- and 70B-shaped batches over an FP8 (E4M3) cache
        "llama8b_decode_fp8": lambda: W.llama8b_decode(),
        "llama70b_decode_bs16_fp8": lambda: W.llama70b_decode(block_size=16),
        # chunked prefill: the 4 x 512-query chunks alone, then with the 128
        # decodes riding along in the same call
        "prefill_chunks": lambda: W.mixed_prefill(num_decodes=0),
        # speculative-decoding verification: 6 causal query rows per sequence
        "spec_verify": lambda: W.spec_verify(),
        "spec_verify_long": lambda: W.spec_verify(batch=8, lo=32768, hi=131072, seed=1007),
        # token-tree verification: 16-node candidate trees per sequence
        "spec_verify_tree": lambda: W.spec_verify_tree(),
        "mixed_prefill": lambda: W.mixed_prefill(),
        # the chunk and verify batches over an FP8 (E4M3) cache
        "prefill_chunks_fp8": lambda: W.mixed_prefill(num_decodes=0),
        "mixed_prefill_fp8": lambda: W.mixed_prefill(),
        "spec_verify_fp8": lambda: W.spec_verify(),
        # the same over FP8 pools with one scale per (block, KV head)
        "llama8b_decode_fp8_per_block": lambda: W.llama8b_decode(),
        "prefill_chunks_fp8_per_block": lambda: W.mixed_prefill(num_decodes=0),
        "mixed_prefill_fp8_per_block": lambda: W.mixed_prefill(),
        "spec_verify_fp8_per_block": lambda: W.spec_verify(),
    }
    if name not in table:
        raise SystemExit(f"unknown workload {name}; choose from {sorted(table)}")
    return table[name]()


def cpu_baseline(batch, w, min_seconds=10.0):
    """The fp64 oracle, as it stands, on the same batch (host copies),
    repeated over the whole batch for at least min_seconds; the rate is the
    mean over all repetitions."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    q = batch.q.cpu()
    kc, vc = batch.k_cache.cpu(), batch.v_cache.cpu()
    bt, cl = batch.block_table.cpu(), batch.context_lens.cpu()
    reps, total = 0, 0.0
    while reps < 2 or total < min_seconds:
        t0 = time.perf_counter()
        oracle.paged_attention(q, kc, vc, bt, cl, w.scale, num_threads=threads)
        total += time.perf_counter() - t0
        reps += 1
    t = total / reps
    kv_bytes = sum(w.context_lens) * w.kv_token_bytes()
    return {"value": round(kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole {w.name} batch ({w.num_seqs} seqs, sum ctx {sum(w.context_lens)}), "
                      f"fp64 C + OpenMP, {reps} repetitions in {total:.1f} s: {t:.3f} s per "
                      f"batch on average ({w.num_seqs / t:.2f} seq-steps/s)"}


def cpu_baseline_1t(batch, w, seqs=8, min_seconds=5.0):
    """The same fp64 oracle on ONE host thread, on the first `seqs` sequences
    of the batch (host copies of their blocks), repeated for at least
    min_seconds; the rate is the mean over the repetitions."""
    import oracle
    bt = batch.block_table.cpu()[:seqs]
    cl = batch.context_lens.cpu()[:seqs]
    q = batch.q.cpu()[:seqs]
    kc, vc = batch.k_cache.cpu(), batch.v_cache.cpu()
    reps, total = 0, 0.0
    while reps < 2 or total < min_seconds:
        t0 = time.perf_counter()
        oracle.paged_attention(q, kc, vc, bt, cl, w.scale, num_threads=1)
        total += time.perf_counter() - t0
        reps += 1
    t = total / reps
    kv_bytes = int(cl.sum()) * w.kv_token_bytes()
    return {"value": round(kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {seqs} sequences of the {w.name} batch (sum ctx {int(cl.sum())}), "
                      f"fp64 C, one thread, {reps} repetitions in {total:.1f} s: {t:.3f} s each "
                      f"on average ({seqs / t:.2f} seq-steps/s)"}


def hbm_ceiling(dev):
    """The practical streaming ceiling next to the 8 TB/s spec, measured with
    this library's own copy kernel: pkv_copy_blocks moving 8192 distinct
    32 KiB blocks of each pool (K and V: 512 MiB read and 512 MiB written
    per call), median of 10 event-timed calls, bytes read + written per
    second.  (torch's stock device copy and sum reach only 4.6 and 4.0 TB/s
    on this GPU, below the decode kernel, so they make no ceiling.)"""
    import torch
    from paged_kv_cache_98_amd import binding as pkv
    nb, bs, hkv, d, npairs = 16384, 16, 8, 128, 8192
    k = torch.zeros((nb, bs, hkv, d), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(npairs), torch.arange(npairs) + npairs], 1).to(
        torch.int64).to(dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        pkv.copy_blocks(k, v, pairs, stream=stream)
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pkv.copy_blocks(k, v, pairs, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    moved = 2 * 2 * npairs * bs * hkv * d * 2
    del k, v
    torch.cuda.empty_cache()
    return {"unit": "GB/s", "copy_read_write": round(moved / statistics.median(ts) / 1e9, 1),
            "what": "pkv_copy_blocks over 8192 distinct 32 KiB blocks of each pool (1 GiB read + "
                    "written per call), median of 10 event-timed calls"}


def cpu_baseline_fp8(batch, w, seqs=8, min_seconds=10.0, scales=None):
    """The fp64 FP8-cache oracle (numpy, one process), as it stands, on the
    first `seqs` sequences of the batch (host copies of their blocks),
    repeated for at least min_seconds; the rate is the mean.  scales: the
    (k, v) per-(block, head) tables of per-block pools, else None."""
    import numpy as np
    import torch
    from oracle import fp8
    from paged_kv_cache_98_amd import workloads as W
    bt = batch.block_table.cpu()
    ctx = list(w.context_lens)[:seqs]
    need = [-(-c // w.block_size) for c in ctx]
    ids = torch.cat([bt[i, :need[i]] for i in range(seqs)]).to(torch.int64)
    kc = batch.k_cache.index_select(0, ids.to(batch.k_cache.device)).cpu().numpy()
    vc = batch.v_cache.index_select(0, ids.to(batch.v_cache.device)).cpu().numpy()
    table = np.full((seqs, max(need)), -1, dtype=np.int32)
    base = 0
    for i in range(seqs):
        table[i, :need[i]] = np.arange(base, base + need[i])
        base += need[i]
    q = batch.q[:seqs].cpu().view(torch.int16).numpy().view(np.uint16)
    ks = vs = W.FP8_SCALE
    if scales is not None:
        idd = ids.to(scales[0].device)
        ks, vs = (t.index_select(0, idd).cpu().numpy() for t in scales)
    reps, total = 0, 0.0
    while reps < 2 or total < min_seconds:
        t0 = time.perf_counter()
        fp8.paged_decode_fp8(q, kc, vc, ks, vs, table, np.array(ctx, np.int32), w.scale)
        total += time.perf_counter() - t0
        reps += 1
    t = total / reps
    kv_bytes = sum(ctx) * w.kv_token_bytes() // 2
    return {"value": round(kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {seqs} sequences of the batch (sum ctx {sum(ctx)}), fp64 numpy, "
                      f"{reps} repetitions in {total:.1f} s: {t:.3f} s each on average "
                      f"({seqs / t:.2f} seq-steps/s)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="no benchmark: record WORKLOAD's HBM bytes (or 'calibration') in "
                         "profiles/hbm_traffic.json from rocprofv3 FETCH_SIZE / WRITE_SIZE runs")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (decode shards by sequence or KV head with no exchange, see the "
              "design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_98_amd import binding as pkv
    from paged_kv_cache_98_amd import workloads as W

    if args.copy_calibration:
        # A plain copy of known size: 1 GiB read + 1 GiB written per dispatch.
        # Profiled with the FETCH_SIZE / WRITE_SIZE counters it gives the
        # factor that turns those counters into bytes.
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": src.numel() * 2}), flush=True)
        return

    if args.workload in ("cow_copy", COPY_WORKLOAD):
        bench_copy_blocks(args)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workload_by_name(args.workload)
    kv_pb = args.workload.endswith("_fp8_per_block")
    kv_fp8 = kv_pb or args.workload.endswith("_fp8")
    wname = w.name + ("_fp8_per_block" if kv_pb else ("_fp8" if kv_fp8 else ""))
    print(f"[bench] workload {w.describe()}"
          f"{' FP8 KV, per-(block, head) scales' if kv_pb else (' FP8 KV' if kv_fp8 else '')}",
          file=sys.stderr, flush=True)
    b = W.materialize(w, device=dev, poison=False)
    ksc = vsc = None
    if kv_pb:
        # E4M3 codes with a scale per (block, KV head), from each block's
        # absolute maximum after a per-block magnitude spread
        b.k_cache, b.v_cache, ksc, vsc = W.fp8_block_pools(b, seed=1)
        torch.cuda.empty_cache()
    elif kv_fp8:
        # E4M3 code pools made by torch's float8 cast; the bf16 pools go
        b.k_cache, b.v_cache = W.fp8_pools(b)
        torch.cuda.empty_cache()
    ws_bytes = (pkv.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                           w.max_context_len) if w.is_decode else
                pkv.prefill_workspace_bytes(w.num_seqs, w.total_q, w.max_q_len, w.num_q_heads,
                                            w.num_kv_heads, w.max_context_len))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    if not w.is_decode:
        out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    is_tree = args.workload == "spec_verify_tree"
    tree_mask = W.tree_masks(w).to(dev) if is_tree else None

    def attend():
        if kv_pb and w.is_decode:
            pkv.paged_decode_attn_fp8_per_block(b.q, b.k_cache, b.v_cache, ksc, vsc,
                                                b.block_table, b.context_lens, w.scale,
                                                max_context_len=w.max_context_len, out=out,
                                                workspace=ws, stream=stream)
        elif kv_pb:
            pkv.paged_prefill_attn_fp8_per_block(b.q, b.cu_q_lens, b.k_cache, b.v_cache, ksc, vsc,
                                                 b.block_table, b.context_lens, w.scale,
                                                 max_context_len=w.max_context_len,
                                                 max_q_len=w.max_q_len, causal=True, out=out,
                                                 workspace=ws if ws_bytes else None,
                                                 stream=stream)
        elif kv_fp8 and w.is_decode:
            pkv.paged_decode_attn_fp8(b.q, b.k_cache, b.v_cache, W.FP8_SCALE, W.FP8_SCALE,
                                      b.block_table, b.context_lens, w.scale,
                                      max_context_len=w.max_context_len, out=out, workspace=ws,
                                      stream=stream)
        elif kv_fp8:
            pkv.paged_prefill_attn_fp8(b.q, b.cu_q_lens, b.k_cache, b.v_cache, W.FP8_SCALE,
                                       W.FP8_SCALE, b.block_table, b.context_lens, w.scale,
                                       max_context_len=w.max_context_len, max_q_len=w.max_q_len,
                                       causal=True, out=out,
                                       workspace=ws if ws_bytes else None, stream=stream)
        elif w.is_decode:
            pkv.paged_decode_attn(b.q, b.k_cache, b.v_cache, b.block_table, b.context_lens,
                                  w.scale, max_context_len=w.max_context_len, out=out,
                                  workspace=ws, stream=stream)
        else:
            pkv.paged_prefill_attn(b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table,
                                   b.context_lens, w.scale, max_context_len=w.max_context_len,
                                   max_q_len=w.max_q_len, causal=True, out=out,
                                   workspace=ws if ws_bytes else None, stream=stream,
                                   tree_mask=tree_mask)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if kv_pb:
            pkv.kv_append_fp8_per_block(b.k_new, b.v_new, b.slot_mapping, b.k_cache, b.v_cache,
                                        ksc, vsc, stream=stream)
        elif kv_fp8:
            pkv.kv_append_fp8(b.k_new, b.v_new, b.slot_mapping, b.k_cache, b.v_cache,
                              W.FP8_SCALE, W.FP8_SCALE, stream=stream)
        else:
            pkv.kv_append(b.k_new, b.v_new, b.slot_mapping, b.k_cache, b.v_cache, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        attend()
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by device synchronisation.  No
    # event is recorded between steps here: on this stack an event record
    # between kernels lengthens a 125 us step by about 5 us.
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for _ in range(args.steps):
        step()
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = region[0].elapsed_time(region[1]) / args.steps

    # the same K steps again with events around each kernel call, on the
    # stream the library launches on, for the per-call durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()

    append_ms = [e[0].elapsed_time(e[1]) for e in evs]
    decode_ms = [e[1].elapsed_time(e[2]) for e in evs]
    # bytes a decode must read: one byte per value in an FP8 cache
    kv_bytes = sum(w.context_lens) * w.kv_token_bytes() // (2 if kv_fp8 else 1)
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg = statistics.mean(decode_ms)
    achieved = kv_bytes / (dec_avg * 1e-3) / 1e9
    print(f"[bench] step {ms_per_step * 1e3:.1f} us (GPU {gpu_ms_per_step * 1e3:.1f} us) | decode avg {dec_avg * 1e3:.1f} us "
          f"(median {statistics.median(decode_ms) * 1e3:.1f}, p10 "
          f"{sorted(decode_ms)[len(decode_ms) // 10] * 1e3:.1f}, p90 "
          f"{sorted(decode_ms)[(9 * len(decode_ms)) // 10] * 1e3:.1f}) | append avg "
          f"{statistics.mean(append_ms) * 1e3:.1f} us | decode KV {achieved:.0f} GB/s",
          file=sys.stderr, flush=True)

    if not w.is_decode and w.max_q_len <= 16:
        # a verify batch reads every key once per KV head for a handful of
        # query rows: bandwidth-bound like a decode
        flops = attention_flops(w)
        print(f"[bench] verify attn {dec_avg * 1e3:.1f} us: KV {achieved:.0f} GB/s, "
              f"{flops / (dec_avg * 1e-3) / 1e12:.1f} TFLOP/s", file=sys.stderr, flush=True)
        rec = {
            "metric": ("paged token-tree verify attn (a candidate tree per sequence, each node "
                       "seeing its path): achieved KV HBM GB/s + verified tokens/s" if is_tree
                       else "paged verify attn (few causal query rows per sequence): achieved "
                            "KV HBM GB/s + verified tokens/s"),
            "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8-e4m3 KV, bf16 q" if kv_fp8 else "bf16",
            "data": "synthetic",
            "config": {"workload": wname, **{k: v for k, v in w.describe().items()
                                             if k != "workload"}},
            "tokens_per_s": round(w.total_q / (ms_per_step * 1e-3), 1),
            "kernels_us": {"kv_append": round(statistics.mean(append_ms) * 1e3, 2),
                           "paged_prefill_attn": round(dec_avg * 1e3, 2)},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": hbm_traffic(w.name),
                         "kernel": ("paged_prefill_attn_tree (few-row chunks, tree masks)"
                                    if is_tree else "paged_prefill_attn (few-row chunks)"),
                         "algorithmic_bytes_per_launch": kv_bytes},
        }
        print(json.dumps(rec), flush=True)
        return

    if not w.is_decode:
        flops = attention_flops(w)
        tflops = flops / (dec_avg * 1e-3) / 1e12
        dkv = decode_kv_bytes(w)
        print(f"[bench] prefill attn {dec_avg * 1e3:.1f} us: {tflops:.1f} TFLOP/s "
              f"({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of MFMA peak), decode rows "
              f"{dkv / (dec_avg * 1e-3) / 1e9:.0f} GB/s of KV", file=sys.stderr, flush=True)
        rec = {
            "metric": "paged prefill attn: MFMA TFLOP/s (exact causal FLOPs) + decode-row KV GB/s",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8-e4m3 KV, bf16 q" if kv_fp8 else "bf16",
            "data": "synthetic",
            "config": {"workload": wname, **{k: v for k, v in w.describe().items()
                                             if k != "workload"}},
            "kernels_us": {"kv_append": round(statistics.mean(append_ms) * 1e3, 2),
                           "paged_prefill_attn": round(dec_avg * 1e3, 2)},
            "decode_rows_kv_gbs": round(dkv / (dec_avg * 1e-3) / 1e9, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": hbm_traffic(w.name),
                         "kernel": "paged_prefill_attn (MFMA chunk kernel)",
                         "algorithmic_flops_per_launch": flops},
        }
        print(json.dumps(rec), flush=True)
        return

    rec = {
        "metric": ("paged decode attn over an FP8 (E4M3) KV cache: achieved KV HBM GB/s + "
                   "seq-steps/s" if kv_fp8 else
                   "paged decode attn: achieved KV HBM GB/s (% of MI355X peak) + seq-steps/s"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 KV, bf16 q" if kv_fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wname, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "sum_context": sum(w.context_lens),
                   "max_context": w.max_context_len, "num_blocks": w.num_blocks,
                   "seed": w.seed},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "gpu_ms_per_step": round(gpu_ms_per_step, 5),
        "kernels_us": {"kv_append": round(statistics.mean(append_ms) * 1e3, 2),
                       "paged_decode_attn": round(dec_avg * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": hbm_traffic(wname),
                     "kernel": DECODE_KERNEL,
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "timing": "mean HIP-event duration of the decode call over K calls of a "
                               "second pass, events on the library's stream around each call"},
        "value_timing": "wall clock over K un-evented steps (kv_append + paged_decode_attn), "
                        "bracketed by device synchronisation",
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = (cpu_baseline_fp8(b, w, scales=(ksc, vsc) if kv_pb else None)
                               if kv_fp8 else cpu_baseline(b, w))
        if not kv_fp8:
            rec["cpu_baseline_1t"] = cpu_baseline_1t(b, w)
        rec["hbm_ceiling"] = hbm_ceiling(dev)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
