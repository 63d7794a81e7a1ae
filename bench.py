#!/usr/bin/env python3
"""Decode-step benchmark for paged KV-cache attention on one MI355X.

One step = the cache write of each sequence's new token plus paged decode
attention over every sequence's context. By default (--kernel pstep) both are
one call, pa_decode_partitioned_step, which stores each new token's K/V in its
slot and attends to it from registers (--kernel step: the same fused step on
the balanced schedule, pa_decode_step); the other kernels (balanced,
partitioned, single, cascade on a shared-prefix workload) run after a
separate pa_reshape_and_cache call. The default workload is the Llama-8B-shaped GQA
batch: 64 sequences, 32 query / 8 KV heads, head size 128, bf16 KV, context
lengths min(4096, 100 + floor(Exp(mean 400))), 16-token blocks scattered
through a pool twice the size needed. Inputs are synthetic (seeded N(0, 1)
values) and already resident in HBM when timing starts.

The KV working set of one step (~131 MB) fits in the 256 MB Infinity Cache, so
consecutive steps rotate over R independent replicas of the batch (same
lengths, different block placement and values; R * 131 MB >> 256 MB).

Before the W counted warm-up steps, untimed steps run for 0.25 s of wall time
(reported as `settle_steps` / `settle_ms`): the GPU idles during the host-side
set-up and its clocks ramp up under load, so a timed region of a few
milliseconds would otherwise measure the ramp rather than the kernels.

Printed: one JSON line on stdout. `value` is KV-read GB/s of whole steps
(cache write + attention, launch gaps included, wall clock between two
synchronisations); `roofline` is the attention call alone, timed with HIP
events on the launch stream around a run of back-to-back calls (also after a
1 GiB write that evicts the caches: `attention_ms_cold_p50`); `stream_read` is
the rate of the library's plain streaming-read kernel over 2 GiB, the
achievable ceiling next to the nominal 8 TB/s; `cpu_baseline` is the fp64
oracle on the host cores (and on one thread) over a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention KV-read GB/s (% of HBM peak) and seq-steps/sec at 1 GPU"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_456_amd", "csrc", f)
               for f in ("pa_decode.hip", "pa_decode_balanced.hip", "pa_decode_core.h", "pa_device.h",
                         "pa_api.cpp", "pa_internal.h", "pa_cascade_tile.h", "pa_tile.h")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


SETTLE_S = 0.25   # untimed GPU work before the counted warm-up: the clocks ramp up under load


def settle_clocks(fn) -> dict:
    """Runs fn() back to back for SETTLE_S seconds of wall time (synchronising every 64 calls),
    so that the GPU's clocks have ramped up before the counted warm-up and the timed region:
    after the host-side set-up the GPU idles and a timed region of a few milliseconds would
    otherwise start at a low clock (measured on the headline batch: 5 warm-up and 20 timed
    steps gave 50.7 us per step, against 37.6 us once settled). Returns the count and time."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(64):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return {"settle_steps": n, "settle_ms": round((time.perf_counter() - t0) * 1e3, 1)}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str, partition_size: int):
    """HBM bytes per attention call from a committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except ValueError:
        return None
    key = f"{workload}/{kernel}/{partition_size}"
    ent = rec.get("entries", {}).get(key)
    if not ent or ent.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_call")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--op", choices=("decode", "copy_blocks", "swap", "prefill"), default="decode",
                    help="decode: the decode step (default); copy_blocks: pa_copy_blocks alone; "
                         "swap: pa_swap_blocks out to pinned host pools and back; "
                         "prefill: pa_prefill, a chunk of query tokens per sequence")
    ap.add_argument("--prefill-chunk", type=int, default=512,
                    help="--op prefill: query tokens per sequence (its last min(L, chunk) tokens)")
    ap.add_argument("--workload", default="llama8b_gqa_bf16")
    ap.add_argument("--kernel", choices=("step", "pstep", "balanced", "partitioned", "single", "cascade"),
                    default="pstep",
                    help="pstep: pa_decode_partitioned_step, the cache write and the partitioned "
                         "attention in one call (default); step: pa_decode_step, the same on the "
                         "work-balanced schedule; balanced: pa_reshape_and_cache then "
                         "pa_decode_balanced; partitioned / single: pa_reshape_and_cache then "
                         "pa_decode_partitioned / pa_decode; cascade: pa_decode_cascade over the "
                         "prefix every table shares (shared-prefix workloads only)")
    ap.add_argument("--partition-size", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--stream-read-mib", type=int, default=2048,
                    help="buffer read by the streaming-read calibration kernel (0 = skip)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="attention calls timed after a 1 GiB write evicts the caches (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU oracle baseline (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device-to-device copy of MIB MiB three times (a "
                         "kernel of known traffic that scales the HBM byte counters of a profile)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_456_amd as pa
    from paged_kv_cache_456_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load()
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 copies of {n} bytes")
        del src, dst
    if args.op == "copy_blocks":
        return bench_copy_blocks(args, dev)
    if args.op == "prefill":
        return bench_prefill(args, dev)
    if args.op == "swap":
        return bench_swap(args, dev)
    stream_read = stream_read_rate(dev, args.stream_read_mib << 20) if args.stream_read_mib > 0 else None
    spec = wl.SPECS[args.workload]
    psize = args.partition_size or spec.partition_size

    # Replicas of the batch: same lengths, independent placement and values.
    nb = None
    if spec.pool.startswith("hbm"):
        # A pool sized to a share of HBM: one replica (its KV is far beyond the
        # Infinity Cache anyway), capped by the memory that is actually free.
        args.replicas = 1
        free, _ = torch.cuda.mem_get_info()
        per_block = 2 * spec.num_kv_heads * wl.BLOCK_SIZE * spec.head_size * \
            torch.tensor([], dtype=spec.dtype).element_size()
        want = float(spec.pool.split(":")[1]) * wl.HBM_BYTES
        nb = int(min(want, 0.85 * free) // per_block)
    base = wl.make_workload(args.workload, device=dev, num_blocks=nb, poison=nb is None)
    lengths = base.context_lens.tolist()
    reps = [base] + [wl.make_workload(args.workload, device=dev, lengths=lengths, seed_offset=r)
                     for r in range(1, args.replicas)]
    S, Hq, D = base.query.shape
    Hkv = spec.num_kv_heads
    kv_bytes = base.kv_bytes()
    mcl = base.max_context_len
    npb = 0
    unique_bytes = kv_bytes
    if args.kernel == "cascade":
        if base.shared_blocks is None:
            print(f"--kernel cascade needs a shared-prefix workload, not {args.workload}",
                  file=sys.stderr)
            return 2
        # Every table starts with the same npb blocks: the prefix is read once per
        # step, each suffix once.
        npb = len(base.shared_blocks)
        prefix_tokens = npb * wl.BLOCK_SIZE
        tok = prefix_tokens + int((base.context_lens.astype(np.int64) - prefix_tokens).sum())
        unique_bytes = tok * Hkv * D * torch.tensor([], dtype=spec.dtype).element_size() * 2
    inputs = []
    for w in reps:
        inputs.append(dict(
            w=w, bt=torch.from_numpy(w.block_tables).to(dev), cl=torch.from_numpy(w.context_lens).to(dev),
            slots=torch.from_numpy(w.slot_mapping).to(dev),
            out=torch.empty((S, Hq, D), dtype=torch.float32, device=dev),
            ws=pa.cascade_workspace(S, Hq, D, mcl, psize, npb, device=dev) if npb
            else pa.balanced_workspace(Hq, Hkv, D, device=dev) if args.kernel in ("step", "balanced")
            else pa.decode_workspace(S, Hq, D, mcl, psize, device=dev)))
        per = spec.new_tokens_per_seq
        last = torch.arange(S, device=dev) * per + (per - 1)
        early = torch.ones(S * per, dtype=torch.bool, device=dev)
        early[last] = False
        inputs[-1].update(
            new_key=w.key[last].contiguous(), new_value=w.value[last].contiguous(),
            early_key=w.key[early].contiguous(), early_value=w.value[early].contiguous(),
            early_slots=inputs[-1]["slots"][early].contiguous())
    torch.cuda.synchronize()
    log(f"[bench] {args.workload}: S={S} Hq={Hq} Hkv={Hkv} D={D} sum(L)={int(base.context_lens.sum())} "
        f"KV bytes/step={kv_bytes / 1e6:.1f} MB, replicas={args.replicas}, kernel={args.kernel}, P={psize}")

    def attention(x):
        w = x["w"]
        if args.kernel == "step":
            pa.pa_decode_step(x["out"], w.query, x["new_key"], x["new_value"], w.key_cache,
                              w.value_cache, x["bt"], x["cl"], w.scale, x["ws"])
        elif args.kernel == "pstep":
            pa.pa_decode_partitioned_step(x["out"], w.query, x["new_key"], x["new_value"],
                                          w.key_cache, w.value_cache, x["bt"], x["cl"], w.scale,
                                          mcl, psize, x["ws"])
        elif args.kernel == "balanced":
            pa.pa_decode_balanced(x["out"], w.query, w.key_cache, w.value_cache, x["bt"], x["cl"],
                                  w.scale, x["ws"])
        elif args.kernel == "single":
            pa.pa_decode(x["out"], w.query, w.key_cache, w.value_cache, x["bt"], x["cl"], w.scale)
        elif args.kernel == "cascade":
            pa.pa_decode_cascade(x["out"], w.query, w.key_cache, w.value_cache, x["bt"], x["cl"],
                                 w.scale, npb, mcl, psize, x["ws"])
        else:
            pa.pa_decode_partitioned(x["out"], w.query, w.key_cache, w.value_cache, x["bt"], x["cl"],
                                     w.scale, mcl, psize, x["ws"])

    def step(i):
        x = inputs[i % len(inputs)]
        w = x["w"]
        if args.kernel not in ("step", "pstep"):
            pa.pa_reshape_and_cache(w.key, w.value, w.key_cache, w.value_cache, x["slots"])
        elif x["early_slots"].numel():
            # several new tokens per sequence: all but the last go through the cache write
            pa.pa_reshape_and_cache(x["early_key"], x["early_value"], w.key_cache, w.value_cache,
                                    x["early_slots"])
        attention(x)

    settle = settle_clocks(step)
    log(f"[bench] clocks settled: {settle['settle_steps']} untimed steps in {settle['settle_ms']} ms")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # Timed region: exactly K steps between two synchronisations, nothing else
    # on the stream (event records would add their own gaps).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {elapsed * 1e3:.2f} ms")

    # Duration of the attention call alone: the same K calls again, back to
    # back on the stream they run on, between two HIP events (an event pair
    # per call would add its own gap to every call). A short GPU-side wait
    # ahead of the first event keeps the GPU busy while the host enqueues the
    # first calls, so the host's launch latency stays outside the timed span.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(100_000)              # ~40 us at the GPU clock
    e0.record()
    for i in range(args.steps):
        attention(inputs[i % len(inputs)])
    e1.record()
    torch.cuda.synchronize()
    call_ms = np.array([e0.elapsed_time(e1) / args.steps])

    cold_ms = None
    if args.cold_calls > 0:
        # Each call after a 1 GiB write that pushes the batch out of L2 and the
        # Infinity Cache; only the attention call is timed.
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.cold_calls)]
        for i, (a, b) in enumerate(cevs):
            scratch.fill_(i & 0xFF)
            a.record()
            attention(inputs[i % len(inputs)])
            b.record()
        torch.cuda.synchronize()
        cold_ms = float(np.median([a.elapsed_time(b) for a, b in cevs]))
        del scratch
        log(f"[bench] cold calls: median {cold_ms * 1e3:.2f} us over {args.cold_calls}")

    ms_per_step = elapsed * 1e3 / args.steps
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    attn_ms = float(np.mean(call_ms))
    # Algorithmic bytes of the attention call: the KV it must read (for the
    # cascade, the shared prefix once and every suffix once).
    achieved = unique_bytes / (attn_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload, args.kernel, psize)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        **settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_size": D, "block_size": 16, "sum_context_len": int(base.context_lens.sum()),
            "max_context_len": mcl, "kv_bytes_per_step": kv_bytes,
            "kernel": {"single": "pa_decode", "partitioned": "pa_decode_partitioned",
                       "cascade": "pa_decode_cascade", "balanced": "pa_decode_balanced",
                       "step": "pa_decode_step",
                       "pstep": "pa_decode_partitioned_step"}[args.kernel],
            "partition_size": psize if args.kernel in ("partitioned", "cascade", "pstep") else None,
            "unique_kv_bytes_per_step": unique_bytes,
            "prefix_blocks": npb or None,
            "replicas": args.replicas, "pool_blocks": base.num_blocks,
            "step": f"{'pa_decode_step' if args.kernel == 'step' else 'pa_decode_partitioned_step'} "
                    "(cache write fused into the attention call)"
                    if args.kernel in ("step", "pstep") else "pa_reshape_and_cache + attention",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(S / (ms_per_step * 1e-3), 1),
        "attention_ms_per_call": round(attn_ms, 5),
        "attention_ms_p50": round(float(np.median(call_ms)), 5),
        "attention_ms_min": round(float(np.min(call_ms)), 5),
        "attention_ms_cold_p50": round(cold_ms, 5) if cold_ms is not None else None,
        "stream_read": stream_read,
        "pct_of_stream_read": round(100.0 * achieved / stream_read["gbs"], 2) if stream_read else None,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": {"step": "attention call: paged_decode_balanced_kernel (cache write "
                               "fused) + balanced_reduce_kernel",
                       "pstep": "attention call: paged_decode_persistent_kernel (cache write "
                                "fused) + lse_reduce_kernel",
                       "balanced": "attention call: paged_decode_balanced_kernel + "
                                   "balanced_reduce_kernel",
                       "single": "paged_decode_kernel",
                       "partitioned": "attention call: paged_decode_persistent_kernel + "
                                      "lse_reduce_kernel",
                       "cascade": "attention call: cascade_prefix_kernel + "
                                  "paged_decode_persistent_kernel + lse_reduce_kernel"}[args.kernel],
            "timing": "HIP events on the launch stream around the timed number of attention "
                      "calls issued back to back (no cache write between them), divided by that "
                      "number",
        },
        "cpu_baseline": None,
    }

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(base, kv_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def bench_copy_blocks(args, dev) -> int:
    """pa_copy_blocks on the Llama-8B pool shapes (8 KV heads, D = 128, bf16: 32 KB per block
    per pool): 2048 pairs per call (128 MB read + 128 MB written), four rotating mappings
    over a 16384-block pool; and the copy-on-write of one block per sequence of the
    prefix-shared batch (128 pairs), which is launch-bound. Synthetic data."""
    import numpy as np
    import torch

    import paged_kv_cache_456_amd as pa

    Hkv, D, NB, npairs = 8, 128, 16384, 2048
    block_bytes = Hkv * 16 * D * 2
    kc = torch.empty((NB, Hkv, 16, D), dtype=torch.bfloat16, device=dev).normal_()
    vc = torch.empty_like(kc).normal_()
    rng = np.random.default_rng(5)
    maps = []
    for _ in range(4):
        perm = rng.permutation(NB)
        maps.append(torch.from_numpy(np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1)).to(dev))
    small = torch.from_numpy(np.stack([np.arange(128), 8192 + np.arange(128)], 1)).to(dev)

    def timed(mapping_of, steps):
        for i in range(args.warmup):
            pa.pa_copy_blocks(kc, vc, mapping_of(i))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            pa.pa_copy_blocks(kc, vc, mapping_of(i))
        e1.record()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps, e0.elapsed_time(e1) * 1e-3 / steps

    wall, dev_s = timed(lambda i: maps[i % 4], args.steps)
    _, small_s = timed(lambda i: small, args.steps)
    moved = 2 * 2 * npairs * block_bytes            # both pools, read + write
    gbs = moved / dev_s / 1e9
    print(json.dumps({
        "metric": "copy-on-write block copy GB/s (bytes read + written)", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "copy_blocks", "num_pairs": npairs, "num_kv_heads": Hkv,
                   "head_size": D, "block_bytes_per_pool": block_bytes, "pool_blocks": NB},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "copy_blocks_kernel",
                     "timing": "HIP events around the timed calls, mean per call"},
        "cow_128_pairs_us": round(small_s * 1e6, 3),
        "cpu_baseline": None,
    }), flush=True)
    return 0


PCIE5_X16_GBS = 64.0     # the GPU's host link, PCIe 5.0 x16, nominal per direction


def bench_swap(args, dev) -> int:
    """pa_swap_blocks on the Llama-8B pool shapes (8 KV heads, D = 128, bf16: 32 KB per block
    per pool): 1024 scattered blocks of a 16384-block GPU pool swapped out to pinned host
    pools (64 MB over the host link per call), then back into other GPU blocks. Synthetic
    data. The bound is the host link, not HBM."""
    import numpy as np
    import torch

    import paged_kv_cache_456_amd as pa

    Hkv, D, NB, HNB, npairs = 8, 128, 16384, 2048, 1024
    block_bytes = Hkv * 16 * D * 2
    kc = torch.empty((NB, Hkv, 16, D), dtype=torch.bfloat16, device=dev).normal_()
    vc = torch.empty_like(kc).normal_()
    hk = torch.zeros((HNB, Hkv, 16, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    rng = np.random.default_rng(6)
    outs, ins = [], []
    for _ in range(4):
        dblk = rng.permutation(NB)[:npairs]
        hblk = rng.permutation(HNB)[:npairs]
        outs.append(torch.from_numpy(np.stack([dblk, hblk], 1)).to(dev))
        ins.append(torch.from_numpy(np.stack([hblk, rng.permutation(NB)[:npairs]], 1)).to(dev))

    def timed(fn, steps):
        for i in range(min(args.warmup, 10)):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / steps

    steps = min(args.steps, 50)
    t_out = timed(lambda i: pa.pa_swap_blocks(kc, vc, hk, hv, outs[i % 4]), steps)
    t_in = timed(lambda i: pa.pa_swap_blocks(hk, hv, kc, vc, ins[i % 4]), steps)
    moved = 2 * npairs * block_bytes                  # both pools, one direction
    gbs_out, gbs_in = moved / t_out / 1e9, moved / t_in / 1e9
    log(f"[bench] swap {npairs} blocks ({moved / 1e6:.1f} MB): out {t_out * 1e6:.1f} us "
        f"({gbs_out:.1f} GB/s), in {t_in * 1e6:.1f} us ({gbs_in:.1f} GB/s)")
    print(json.dumps({
        "metric": "block swap GB/s between GPU pools and pinned host pools (bytes moved, mean "
                  "of the two directions)",
        "value": round((gbs_out + gbs_in) / 2, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": min(args.warmup, 10), "ms_per_step": round((t_out + t_in) * 1e3 / 2, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swap_blocks", "num_pairs": npairs, "num_kv_heads": Hkv,
                   "head_size": D, "block_bytes_per_pool": block_bytes, "pool_blocks": NB,
                   "host_pool_blocks": HNB},
        "swap_out_gbs": round(gbs_out, 2), "swap_in_gbs": round(gbs_in, 2),
        "roofline": {"bound": "host link", "achieved": round((gbs_out + gbs_in) / 2, 2),
                     "peak": PCIE5_X16_GBS, "unit": "GB/s",
                     "frac": round((gbs_out + gbs_in) / 2 / PCIE5_X16_GBS, 4), "traffic": None,
                     "kernel": "swap_blocks_kernel",
                     "timing": "HIP events around the timed calls, mean per call"},
        "cpu_baseline": None,
    }), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(args, dev) -> int:
    """pa_prefill on the Llama-8B-shaped batch (64 sequences, 32/8 heads, D = 128, bf16,
    the headline context lengths): each sequence brings its last min(L, chunk) tokens as
    query rows (a chunked-prefill step), attending causally over its paged context.
    Algorithmic work = 4 D Hq sum over rows of (position + 1) flops (Q K^T and P V, causal);
    the bound is bf16 MFMA. Synthetic data, inputs resident in HBM."""
    import numpy as np
    import torch

    import paged_kv_cache_456_amd as pa
    from paged_kv_cache_456_amd import workloads as wl

    w = wl.make_workload(args.workload, device=dev)
    S, Hq, D = w.query.shape
    if w.query.dtype != torch.bfloat16:
        print("--op prefill needs a bf16 workload", file=sys.stderr)
        return 2
    L = w.context_lens.astype(np.int64)
    ql = np.minimum(L, args.prefill_chunk)
    q, qs = wl.prefill_queries(w, ql.tolist())
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    pa.pa_reshape_and_cache(w.key, w.value, w.key_cache, w.value_cache,
                            torch.from_numpy(w.slot_mapping).to(dev))
    qs_d = torch.from_numpy(qs).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    mq = int(ql.max())
    visible = int((ql * (L - ql) + ql * (ql + 1) // 2).sum())     # sum over rows of pos + 1
    flops = 4 * D * Hq * visible

    ws = torch.empty(pa.pa_prefill_workspace_size(S, Hq, w.key_cache.shape[1], mq), dtype=torch.uint8,
                     device=dev)

    def call():
        pa.pa_prefill(out, q, w.key_cache, w.value_cache, bt, cl, qs_d, w.scale, mq, ws)

    settle = settle_clocks(lambda i: call())
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    dev_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    tflops = flops / dev_s / 1e12
    log(f"[bench] prefill: {int(ql.sum())} query tokens over {S} sequences, {flops / 1e9:.2f} GFLOP "
        f"per call, {dev_s * 1e6:.1f} us per call")
    print(json.dumps({
        "metric": "multi-token query attention TFLOP/s (causal, algorithmic)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, **settle, "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload} prefill chunk {args.prefill_chunk}",
                   "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": int(w.key_cache.shape[1]),
                   "head_size": D, "query_tokens": int(ql.sum()), "sum_context_len": int(L.sum()),
                   "flops_per_call": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "prefill_kernel",
                     "timing": "HIP events around the timed calls, mean per call"},
        "cpu_baseline": None,
    }), flush=True)
    return 0


def stream_read_rate(dev, nbytes: int) -> dict:
    """The HBM read rate of pa_stream_read (the decode kernels' nontemporal 16-byte
    loads, nothing else) over an `nbytes` buffer, best over four grid sizes, each the
    mean of 10 launches timed with HIP events on the launch stream."""
    import torch

    import paged_kv_cache_456_amd as pa

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(7)
    best = None
    for wgs in (4 * cus, 8 * cus, 16 * cus, 32 * cus):
        sink = torch.empty(64 * wgs, dtype=torch.uint8, device=dev)
        for _ in range(2):
            pa.pa_stream_read(buf, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            pa.pa_stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"[bench] stream read {nbytes >> 20} MiB, {wgs} workgroups: {us:.1f} us = {gbs:.0f} GB/s")
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "bytes": nbytes, "workgroups": wgs, "us_per_launch": round(us, 2),
                    "kernel": "stream_read_kernel (pa_stream_read)"}
    del buf, sink
    torch.cuda.empty_cache()
    return best


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, kv_bytes: int, seconds: float):
    """The fp64 oracle (cache write + decode of the whole batch) on the host cores,
    repeated for about `seconds` of wall clock. Host copies are made first."""
    import numpy as np
    import torch

    import oracle

    B = w.block_size
    L = w.context_lens.astype(np.int64)
    nblk = -(-L // B)
    blocks = np.unique(np.concatenate([w.block_tables[s, :nblk[s]] for s in range(w.num_seqs)]))
    remap = np.full(w.num_blocks, -1, np.int64)
    remap[blocks] = np.arange(len(blocks))
    tables = np.full_like(w.block_tables, -1)
    for s in range(w.num_seqs):
        tables[s, :nblk[s]] = remap[w.block_tables[s, :nblk[s]]]
    slots = np.where(w.slot_mapping >= 0, remap[np.maximum(w.slot_mapping, 0) // B] * B + w.slot_mapping % B, -1)
    t_copy = time.perf_counter()
    ids = torch.from_numpy(blocks).to(w.key_cache.device)
    kc = w.key_cache.index_select(0, ids).cpu()
    vc = w.value_cache.index_select(0, ids).cpu()
    key, value, q = w.key.cpu(), w.value.cpu(), w.query.cpu()
    t_copy = time.perf_counter() - t_copy
    bits = (lambda t: t.view(torch.int16)) if kc.element_size() == 2 else (lambda t: t.view(torch.int32))
    kb, vb = bits(kc).numpy(), bits(vc).numpy()
    kn, vn = bits(key).numpy(), bits(value).numpy()
    threads = oracle.max_threads()
    log(f"[bench] cpu oracle: {len(blocks)} blocks copied to host in {t_copy:.2f} s, {threads} threads")
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.reshape_and_cache(kn, vn, kb, vb, slots, block_size=B)
        oracle.decode(q, kc, vc, tables, w.context_lens, w.scale)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"[bench] cpu oracle: {n} steps in {el:.2f} s")
    # The same steps on one thread, for a fifth of the time (last: the thread
    # count set here stays for the process).
    n1 = 0
    t1 = time.perf_counter()
    while True:
        oracle.reshape_and_cache(kn, vn, kb, vb, slots, block_size=B)
        oracle.decode(q, kc, vc, tables, w.context_lens, w.scale, num_threads=1)
        n1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 5:
            break
    log(f"[bench] cpu oracle, 1 thread: {n1} steps in {el1:.2f} s")
    return {
        "value": round(kv_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "seq_steps_per_s": round(w.num_seqs * n / el, 2),
        "value_1_thread": round(kv_bytes * n1 / el1 / 1e9, 4),
        "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
        "sample": f"{n} full decode steps of the same batch ({w.num_seqs} sequences, cache write + "
                  f"attention, fp64, inputs in host memory), {el:.1f} s wall; device-to-host copy "
                  f"{t_copy:.2f} s not included",
    }


if __name__ == "__main__":
    sys.exit(main())
