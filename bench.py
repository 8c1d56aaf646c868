#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.  Default workload: batch 32, 32k context, 32 q / 8 kv heads,
INT2 per-channel cache (`--workload` runs any workload of `synth.WORKLOADS` the same way).

One step = append one token per sequence (rotate/clip/quantize write, with group demotion when a
128-token group completes) + one decode attention (query rotation, split-K partials over the quantized
pages and the bf16 band, merge + un-rotation).  Inputs are resident in HBM before timing.

Prints ONE JSON line.  `value` is KV GB/s of the whole step: the decode's algorithmic bytes (codes,
scales/zeros, bf16 band, query, output) per step / step time.  `roofline` is for the split-K decode
kernel alone, timed with HIP events around its launches inside the timed steps, on the stream it runs
on.  `cpu_baseline` times the CPU oracle's read side on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_int2_batch32_32k_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # measured on MI355X: the first ~70 decode steps of a run take about 10% longer while the GPU settles
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="batch32_32k")
    ap.add_argument("--impl", default="auto", choices=["auto", "f32", "mfma"])
    ap.add_argument("--scheme", default=None, choices=["int2_channel", "int2_token", "int4_channel"],
                    help="INT2 workloads: quantize per channel over 128-token groups (the workloads' statement), "
                         "per token over its 128 channels, or per channel with 4-bit codes")
    ap.add_argument("--key-only", action="store_true", help="rotate K only; V quantized in its own frame")
    ap.add_argument("--hadamard-block", type=int, default=0, choices=[0, 16, 32, 64, 128],
                    help="block order of the randomized Hadamard (workloads with that rotation; 0 = 128)")
    ap.add_argument("--split", type=int, default=0, help="quantized tokens per decode work-group (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=8, help="read-leg repetitions per unit in the CPU baseline")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the second line of the default run: the ragged-length batch (8k..32k) of the same "
                         "throughput workload")
    ap.add_argument("--write-bench", action="store_true",
                    help="time the fused rotate-quantize write of one prefill chunk per sequence instead of the "
                         "decode step (the INT4 workload's 8192-token chunk x 8 kv heads; for INT2 workloads a "
                         "chunk of --write-tokens tokens); prints its own JSON line")
    ap.add_argument("--write-tokens", type=int, default=8192)
    ap.add_argument("--prefill-bench", action="store_true",
                    help="time prefill attention of the last --prefill-chunk tokens of every sequence over the "
                         "quantized history (any workload and scheme); prints its own JSON line")
    ap.add_argument("--prefill-chunk", type=int, default=4096)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy kernel) 5 times: the known-size "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for name in ("kvq_decode.hip", "kvq_internal.h"):
        with open(os.path.join(ROOT, "decode_attention_15_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload, variant=""):
    """HBM bytes per launch of the split-K decode kernel measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    scaled by a known-size copy), from the committed summary; None unless that measurement was taken on
    this workload with the kernel source as it is now."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha() or kv.get("workload") != workload:
        return None
    if kv.get("variant", "") != variant:  # scheme / rotation overrides of the workload
        return None
    return int(float(kv["bytes_per_launch"]))


GROUPED = {"int2_channel": 0, "int2_token": 2, "int4_channel": 3}  # grouped schemes and their kvq_scheme


def decode_bytes(wl, lens, S0, W):
    """Algorithmic bytes one decode step reads/writes.  INT2: codes + bf16 scale/zero of every group
    (72 B per token and kv head) and bf16 band tokens (512 B); per-channel INT4 the same with 4-bit
    codes (136 B per token); INT4 per token: codes + bf16 scale/zero of every token (136 B per token
    and kv head).  Plus the query (bf16) and the output (fp32)."""
    kv = 0
    for T in lens:
        if wl.scheme in GROUPED:
            ng = max(0, (T - S0 - W) // 128)
            per_tok = 136 if wl.scheme == "int4_channel" else 72
            kv += wl.n_kv_heads * (ng * 128 * per_tok + (T - 128 * ng) * 512)
        else:
            kv += wl.n_kv_heads * T * 136
    qo = len(lens) * wl.n_q_heads * 128 * (2 + 4)
    return kv, qo


def _cpu_unit(task):
    """One (sequence, kv head) unit of the oracle on one BLAS thread: the write leg (rotate, clip, quantize and
    pack every group of the unit's T tokens; the band tokens as bf16) and the read leg (dequantize, x^.R^T,
    fp64 softmax attention of the unit's GQ query heads), repeated `reps` times.  Runs in a worker process."""
    wl_name, changes, b, h, T, reps = task
    import numpy as np
    import oracle as O
    import synth
    from threadpoolctl import threadpool_limits
    wl = synth.scaled(synth.WORKLOADS[wl_name], **changes)
    grouped = wl.scheme in GROUPED
    with threadpool_limits(limits=1):
        k = synth.kv_tokens(wl, b, 0, T, "k")[:, h].copy()
        v = synth.kv_tokens(wl, b, 0, T, "v")[:, h].copy()
        q = synth.queries(wl, 10 ** 6)[b, h * wl.gq:(h + 1) * wl.gq]
        if grouped:
            rk = O.oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
            rv = None if wl.key_only else O.oscar_rotation(synth.rotation_gaussian(wl, "v")).astype(np.float32)
            axis = {"int2_channel": "channel", "int2_token": "token", "int4_channel": "channel4"}[wl.scheme]
            t0 = time.perf_counter()
            st = O.int2_state(k, v, T, wl.n_sink, wl.n_recent, wl.clip_k, wl.clip_v, rk, rv, axis=axis)
            t_write = time.perf_counter() - t0
            t0 = time.perf_counter()
            for _ in range(reps):
                Kh, Vh = O.int2_keys_values(st, rk, rv)
                O.attend(O.query_values(q), Kh, Vh)
            t_read = time.perf_counter() - t0
        else:
            sk = synth.sign_vector(wl, "k")
            sv = None if wl.key_only else synth.sign_vector(wl, "v")
            t0 = time.perf_counter()
            st = O.int4_state(k, v, T, sk, sv, block=wl.hadamard_block)
            t_write = time.perf_counter() - t0
            t0 = time.perf_counter()
            for _ in range(reps):
                Kh, Vh = O.int4_keys_values(st, sk, sv, wl.hadamard_block)
                O.attend(O.query_values(q), Kh, Vh)
            t_read = time.perf_counter() - t0
    kv_b, qo_b = decode_bytes(wl, [T], wl.n_sink, wl.n_recent)
    read_bytes = kv_b // wl.n_kv_heads + qo_b // wl.n_kv_heads
    write_bytes = T * 2 * 128 * 2 + kv_b // wl.n_kv_heads  # bf16 K, V in; packed pages and band out
    return t_write, t_read, reps, write_bytes, read_bytes


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, args):
    """The CPU oracle on the same workload and the host's cores, before the GPU is touched: (seq, kv head)
    units of the decode at the workload's context length, each on one BLAS thread, first one unit alone (one
    thread), then one unit per core in a pool of spawned worker processes (all cores the process may run on,
    at most 16).  The write leg (rotate, clip, quantize every group of the unit's context) and the read leg
    (dequantize, inverse-rotate, fp64 attention of its GQ heads, `reps` times) are timed separately.  `value`
    is the read leg on all cores in the decode's algorithmic bytes per second (the GPU's metric)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import numpy as np
    import synth
    T = int(synth.seq_lens(wl).max())
    base = synth.WORKLOADS[wl.name]
    changes = {k_: getattr(wl, k_) for k_ in ("scheme", "key_only", "hadamard_block") if getattr(wl, k_) != getattr(base, k_)}
    cores = min(16, len(os.sched_getaffinity(0)))
    reps = max(1, int(args.cpu_reps))
    units = [(n % wl.batch, (3 * n + 1) % wl.n_kv_heads) for n in range(cores)]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=1, mp_context=ctx) as ex:
        one = ex.submit(_cpu_unit, (wl.name, changes, units[0][0], units[0][1], T, reps)).result()
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        tw0 = time.perf_counter()
        res = list(ex.map(_cpu_unit, [(wl.name, changes, b, h, T, reps) for b, h in units]))
        wall = time.perf_counter() - tw0
    tw, tr, rp, wb, rb = zip(*res)
    # all cores: every unit's legs run concurrently; each leg's aggregate rate is its bytes over the slowest
    # worker's time for that leg
    write_all = sum(wb) / max(tw) / 1e9
    read_all = sum(rb) * reps / max(tr) / 1e9
    write_one = one[3] / one[0] / 1e9
    read_one = one[4] * reps / one[1] / 1e9
    unit_read_s = max(tr) / reps
    steps = cores / unit_read_s / (wl.batch * wl.n_kv_heads)  # decode steps/s of the whole batch on all cores
    return {
        "value": round(read_all, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu": cpu_model(),
        "read_gbps": {"all_cores": round(read_all, 4), "one_thread": round(read_one, 4)},
        "write_gbps": {"all_cores": round(write_all, 4), "one_thread": round(write_one, 4)},
        "decode_steps_per_s_all_cores": round(steps, 3),
        "sample": (f"{cores} (seq, kv head) units of {wl.name} at T={T} (of {wl.batch * wl.n_kv_heads} per step), "
                   f"one per core in spawned processes, one BLAS thread each, plus one unit alone; write leg = "
                   f"rotate/clip/quantize all {max(0, (T - wl.n_sink - wl.n_recent) // 128)} groups of the unit, "
                   f"read leg = dequantize, x^.R^T and fp64 attention of {wl.gq} q heads x {reps}; "
                   f"{time.perf_counter() - t0:.1f} s wall in total"),
    }


def calibrate_copy():
    """A plain device copy of 1 GiB, five times: rocprofv3 reads FETCH_SIZE / WRITE_SIZE of these
    dispatches to scale the counters (each dispatch reads and writes exactly 2^30 bytes)."""
    import torch
    torch.cuda.set_device(0)
    src = torch.empty(2 ** 30, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": 2 ** 30, "dispatches": 5}), flush=True)


def write_bench(args, K, synth, np, torch):
    """Fused rotate-quantize write of one prefill chunk per sequence (written at position 0 of an empty
    cache each time): HIP events around each write call on its stream, K warmup + K timed calls."""
    wl = synth.WORKLOADS[args.workload]
    if args.scheme and wl.scheme != "int4_token":
        wl = synth.scaled(wl, scheme=args.scheme)
    if args.key_only:
        wl = synth.scaled(wl, key_only=True)
    if args.hadamard_block and wl.rotation == "saw":
        wl = synth.scaled(wl, hadamard_block=args.hadamard_block)
    n = int(wl.extra.get("prefill_chunk", args.write_tokens))
    B = 1
    dev = "cuda"
    torch.cuda.set_device(0)
    int2 = wl.scheme in GROUPED
    if int2:
        scheme = GROUPED[wl.scheme]
        cfg = K.make_config(wl.n_kv_heads, wl.n_q_heads, scheme, K.ROT_DENSE, wl.n_sink, wl.n_recent, wl.clip_k,
                            wl.clip_v, 0, 0, wl.key_only)
        rk = K.build_oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
        rv = K.build_oscar_rotation(synth.rotation_gaussian(wl, "v")).astype(np.float32)
    else:
        cfg = K.make_config(wl.n_kv_heads, wl.n_q_heads, K.INT4_TOKEN, K.ROT_HADAMARD, 0, 0, 1.0, 1.0, 0, 0,
                            wl.key_only, wl.hadamard_block)
        rk = synth.sign_vector(wl, "k").astype(np.float32)
        rv = synth.sign_vector(wl, "v").astype(np.float32)
    mp = K.pages_for_len(cfg, n)
    n_pool = B * max(1, mp)
    pt = K.build_page_table(B, max(1, mp), n_pool, seed=wl.seed)
    cache = K.allocate_cache(cfg, B, torch.from_numpy(pt), torch.from_numpy(rk),
                             None if wl.key_only else torch.from_numpy(rv), n_pages=n_pool, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    k = (torch.randn((n, wl.n_kv_heads, 128), generator=gen, device=dev)).to(torch.bfloat16)
    v = (torch.randn((n, wl.n_kv_heads, 128), generator=gen, device=dev)).to(torch.bfloat16)
    cu = torch.tensor([0, n], dtype=torch.int32, device=dev)
    times = []
    for i in range(args.warmup + args.steps):
        cache.seq_lens.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        K.kv_rotate_quant_write(cache, k, v, cu, n, max_len=n)
        e1.record()
        e1.synchronize()
        if i >= args.warmup:
            times.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(times)[len(times) // 2]
    in_bytes = 2 * n * wl.n_kv_heads * 128 * 2
    if int2:
        ng = max(0, (n - wl.n_sink - wl.n_recent) // 128)
        out_bytes = wl.n_kv_heads * (ng * 128 * 72 + (n - 128 * ng) * 512)
    else:
        out_bytes = wl.n_kv_heads * n * 136
    gbps = (in_bytes + out_bytes) / t / 1e9
    log(f"[write] {wl.name}: {n} tokens x {wl.n_kv_heads} kv heads, median {t * 1e6:.1f} us, {gbps:.0f} GB/s")
    print(json.dumps({
        "metric": "fused rotate-quantize KV write GB/s (bf16 in + packed pages out)", "value": round(gbps, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "us_per_write": round(t * 1e6, 2),
        "higher_is_better": True, "dtype": "bf16 in, fp64 rotation", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": n, "n_kv_heads": wl.n_kv_heads, "scheme": wl.scheme,
                   "rotation": wl.rotation, "hadamard_block": wl.hadamard_block if wl.rotation == "saw" else None,
                   "key_only": wl.key_only},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": in_bytes + out_bytes},
    }), flush=True)


def prefill_bench(args, K, synth, np, torch):
    """Prefill attention of each sequence's last chunk over its quantized history (the cache written in
    chunks as in chunked prefill): HIP events around kv_prefill_attn (query rotation + attention kernel)."""
    wl = workload_of(args, synth)
    dev = "cuda"
    torch.cuda.set_device(0)
    B, n_kv, n_q = wl.batch, wl.n_kv_heads, wl.n_q_heads
    lens = synth.seq_lens(wl).astype(np.int64)
    n = int(args.prefill_chunk)
    cfg, rk, rv = config_of(wl, K, synth, np, 0, K.DECODE_AUTO)
    max_pages = K.pages_for_len(cfg, int(lens.max()))
    n_pool = B * max_pages
    pt = K.build_page_table(B, max_pages, n_pool, seed=0 if wl.identity_pages else wl.seed)
    cache = K.allocate_cache(cfg, B, torch.from_numpy(pt), torch.from_numpy(rk),
                             None if wl.key_only else torch.from_numpy(rv), n_pages=n_pool, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    done = np.zeros(B, dtype=np.int64)
    while True:  # the cache in chunks of n tokens per sequence, as chunked prefill writes it
        cnt = np.minimum(lens - done, n)
        if cnt.sum() == 0:
            break
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)).to(dev)
        k = torch.randn((int(cnt.sum()), n_kv, 128), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((int(cnt.sum()), n_kv, 128), generator=gen, device=dev).to(torch.bfloat16)
        K.kv_rotate_quant_write(cache, k, v, cu, int(cnt.max()), max_len=int(lens.max()))
        done += cnt
    chunk = np.minimum(lens, n)
    total = int(chunk.sum())
    q = torch.randn((total, n_q, 128), generator=gen, device=dev).to(torch.bfloat16)
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)).to(dev)
    out = torch.empty((total, n_q, 128), dtype=torch.float32, device=dev)
    ws = K.prefill_workspace_for(cfg, total, dev)
    torch.cuda.synchronize()
    times = []
    for i in range(args.warmup + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        K.kv_prefill_attn(cache, q, cu_q, int(chunk.max()), out, ws)
        e1.record()
        e1.synchronize()
        if i >= args.warmup:
            times.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(times)[len(times) // 2]
    # algorithmic work: every (query head, visible token) pair costs 128 MACs for the logit and 128 for the
    # value sum; visible tokens of the query at position p are p + 1
    pairs = 0
    for b in range(B):
        T, c = int(lens[b]), int(chunk[b])
        pairs += n_q * (c * (T - c) + c * (c + 1) // 2)
    ops = pairs * 2 * 2 * 128
    tops = ops / t / 1e12
    log(f"[prefill] {wl.name}: chunk {n} over {int(lens.max())}, median {t * 1e3:.3f} ms, {tops:.1f} TOP/s algorithmic")
    print(json.dumps({
        "metric": "prefill attention over the quantized history, algorithmic TOP/s", "value": round(tops, 2),
        "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_call": round(t * 1e3, 4),
        "higher_is_better": True, "dtype": "int8 limbs (24-bit fixed point) + bf16 band", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "ctx": int(lens.max()), "chunk": n, "n_q_heads": n_q,
                   "n_kv_heads": n_kv, "scheme": wl.scheme, "key_only": wl.key_only,
                   "hadamard_block": wl.hadamard_block if wl.rotation == "saw" else None},
        "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": 5000.0, "unit": "TOP/s",
                     "frac": round(tops / 5000.0, 5), "traffic": None,
                     "note": "int8 peak; each algorithmic MAC is three int8 MACs (limbs) here"},
    }), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this decode path runs on one GPU; runs on several GPUs are not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import synth

    if args.write_bench or args.prefill_bench:
        import torch
        import decode_attention_15_amd as K
    if args.write_bench:
        write_bench(args, K, synth, np, torch)
        return
    if args.prefill_bench:
        prefill_bench(args, K, synth, np, torch)
        return
    wl = workload_of(args, synth)
    # the CPU baseline runs first, in spawned processes, before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args)
    if cpu:
        log(f"[bench] CPU baseline: {cpu['value']} GB/s on {cpu['cores']} cores ({cpu['cpu']})")
    import torch
    import decode_attention_15_amd as K

    torch.cuda.set_device(0)
    res = measure_decode(wl, args, K, synth, np, torch)
    result = {
        "metric": "INT2 decode-attn KV GB/s (% of HBM peak); decode steps/s at BS=32, 32k ctx",
        "value": res["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 (matrix cores: 2/4-bit codes x 3-limb fixed-point operands) + f32 softmax",
        "data": "synthetic",
        "config": res["config"],
        "steps_per_s": res["steps_per_s"],
        "roofline": res["roofline"],
        "decode_kernels_us": res["decode_kernels_us"],
        "read_probe": res["read_probe"],
        "timed_window": res["timed_window"],
    }
    if args.workload == "batch32_32k" and not args.no_ragged and not (args.scheme or args.key_only or args.split):
        # the throughput workload as written: context lengths drawn from 8k..32k
        rg = measure_decode(synth.WORKLOADS["batch32_8k_32k"], args, K, synth, np, torch)
        result["ragged_8k_32k"] = {k_: rg[k_] for k_ in ("value", "ms_per_step", "steps_per_s", "timed_window")}
        result["ragged_8k_32k"]["roofline_frac"] = rg["roofline"]["frac"]
        result["ragged_8k_32k"]["splitk_us"] = rg["roofline"]["kernel_us"]
        result["ragged_8k_32k"]["ctx_range"] = rg["config"]["ctx_range"]
    if cpu:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def workload_of(args, synth):
    wl = synth.WORKLOADS[args.workload]
    if args.scheme and wl.scheme != "int4_token":
        wl = synth.scaled(wl, scheme=args.scheme)
    if args.key_only:
        wl = synth.scaled(wl, key_only=True)
    if args.hadamard_block and wl.rotation == "saw":
        wl = synth.scaled(wl, hadamard_block=args.hadamard_block)
    return wl


def config_of(wl, K, synth, np, split, impl):
    """The library config of a workload and its rotation inputs (dense R from the library's builder for the
    grouped schemes, sign vectors for the randomized Hadamard)."""
    if wl.scheme in GROUPED:
        cfg = K.make_config(wl.n_kv_heads, wl.n_q_heads, GROUPED[wl.scheme], K.ROT_DENSE, wl.n_sink, wl.n_recent,
                            wl.clip_k, wl.clip_v, split, impl, wl.key_only)
        rk = K.build_oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
        rv = K.build_oscar_rotation(synth.rotation_gaussian(wl, "v")).astype(np.float32)
    else:
        cfg = K.make_config(wl.n_kv_heads, wl.n_q_heads, K.INT4_TOKEN, K.ROT_HADAMARD, 0, 0, 1.0, 1.0, split, impl,
                            wl.key_only, wl.hadamard_block)
        rk = synth.sign_vector(wl, "k").astype(np.float32)
        rv = synth.sign_vector(wl, "v").astype(np.float32)
    return cfg, rk, rv


def measure_decode(wl, args, K, synth, np, torch):
    """Decode steps of one workload: a cache written to the lengths before the measured steps, then W warm-up
    steps, a 128-step window and the K timed steps, each step one append of a token per sequence followed by
    one decode attention.  Returns the step time, the split-K kernel's roofline and the kernels' times."""
    grouped = wl.scheme in GROUPED
    dev = "cuda"
    B, n_kv, n_q = wl.batch, wl.n_kv_heads, wl.n_q_heads
    # Any 128 consecutive appends complete exactly one group per sequence (grouped schemes), so the mean step
    # of a 128-step window carries the demotions at their steady rate: it is timed right before the K timed
    # steps, and if the timed window (which, with every length equal, may hold no demotion at all) runs faster
    # per step, the difference is added to it.
    DEM = 128 if grouped else 0
    n_steps = args.warmup + DEM + args.steps
    lens_end = synth.seq_lens(wl).astype(np.int64)          # lengths after the last timed step
    lens_start = lens_end - n_steps
    T_end = int(lens_end.max())
    impl = {"auto": K.DECODE_AUTO, "f32": K.DECODE_F32, "mfma": K.DECODE_MFMA}[args.impl]
    split = args.split if args.split else (wl.split_tokens if wl.name == "long_b4_131k" else 0)
    cfg, rk, rv = config_of(wl, K, synth, np, split, impl)
    max_pages = K.pages_for_len(cfg, T_end)
    n_pool = B * max_pages
    pt = K.build_page_table(B, max_pages, n_pool, seed=0 if wl.identity_pages else wl.seed)
    cache = K.allocate_cache(cfg, B, torch.from_numpy(pt), torch.from_numpy(rk),
                             None if wl.key_only else torch.from_numpy(rv), n_pages=n_pool, device=dev)
    log(f"[bench] {wl.name}: B={B} T={int(lens_start.min())}..{T_end} heads {n_q}/{n_kv}; "
        f"pages {n_pool} x {K.page_bytes(cfg)} B")

    # prefill with the workload's recipe (N(0,1) x channel gains, bf16), generated on the device, in
    # chunks of at most 8192 tokens per sequence (the prefill chunk of the INT4 workload)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    gk = torch.from_numpy(synth.channel_gain(wl, "k")).to(dev)
    gv = torch.from_numpy(synth.channel_gain(wl, "v")).to(dev)

    def draw(n, gain):
        x = torch.randn((n, n_kv, 128), generator=gen, device=dev, dtype=torch.float32)
        return (x * gain[None]).to(torch.bfloat16)

    t0 = time.perf_counter()
    per_call = 4
    chunk = 8192 if not grouped else int(lens_start.max())
    for b0 in range(0, B, per_call):
        sel = slice(b0, min(B, b0 + per_call))
        done = np.zeros(B, dtype=np.int64)
        while True:
            counts = np.zeros(B, dtype=np.int64)
            counts[sel] = np.minimum(lens_start[sel] - done[sel], chunk)
            if counts.sum() == 0:
                break
            cu = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
            k = draw(int(counts.sum()), gk)
            v = draw(int(counts.sum()), gv)
            K.kv_rotate_quant_write(cache, k, v, cu, int(counts.max()), max_len=T_end)
            done += counts
            del k, v
    torch.cuda.synchronize()
    log(f"[bench] prefill written in {time.perf_counter() - t0:.1f} s")

    ks = [draw(B, gk) for _ in range(n_steps)]
    vs = [draw(B, gv) for _ in range(n_steps)]
    qs = [torch.randn((B, n_q, 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(n_steps)]
    cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
    out = torch.empty((B, n_q, 128), dtype=torch.float32, device=dev)
    ws = K.workspace_for(cfg, B, T_end, dev)

    # one step = the append write, then the decode (query prep with the bf16 band, split-K partials of the
    # quantized chunks, merge).  Most timed steps make one kv_decode_attn call; every SAMPLE-th makes one
    # kv_decode_attn_timed call, whose split-K dispatch itself records two HIP events at the kernel's start
    # and end (on the call's stream: torch's current stream, which the binding passes to the library), so the
    # interval is the kernel's own whatever the host does.  Warm-up steps launch the three kernels one by one
    # with events around each, for the query-prep and merge times.
    SAMPLE = 10
    names = ("qprep", "splitk", "merge")
    stages = (K.STAGE_QPREP, K.STAGE_SPLITK, K.STAGE_MERGE)

    def write(i):
        K.kv_rotate_quant_write(cache, ks[i], vs[i], cu1, 1, max_len=T_end)

    def staged_step(i, ev, which):
        write(i)
        for n, st in enumerate(stages):
            if n in which:
                ev[n][0].record()
            K.kv_decode_attn_stages(cache, qs[i], out, T_end, ws, st)
            if n in which:
                ev[n][1].record()

    def step(i):
        write(i)
        K.kv_decode_attn(cache, qs[i], out, T_end, ws)

    def timed_step(i, ev):
        write(i)
        K.kv_decode_attn_timed(cache, qs[i], out, T_end, ws, ev[0], ev[1])

    def pairs(n):
        return [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in stages]
                for _ in range(n)]

    wevs = pairs(args.warmup)
    for i in range(args.warmup):
        staged_step(i, wevs[i], (0, 1, 2))
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    # the 128-step window (every sequence completes one group in it)
    dem_ms = None
    if DEM:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, args.warmup + DEM):
            step(i)
        torch.cuda.synchronize()
        dem_ms = (time.perf_counter() - t0) * 1e3 / DEM
    first = args.warmup + DEM
    sampled = [n for n in range(args.steps) if n % SAMPLE == 0]
    evs = pairs(args.steps)
    lens_before = cache.seq_lens.cpu().numpy().astype(np.int64)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n, i in enumerate(range(first, n_steps)):
        if n % SAMPLE == 0:
            timed_step(i, evs[n][1])
        else:
            step(i)
    host_ms = (time.perf_counter() - t0) * 1e3 / args.steps  # the host's enqueue time per step
    torch.cuda.synchronize()
    ms_timed = (time.perf_counter() - t0) * 1e3 / args.steps
    assert np.array_equal(cache.seq_lens.cpu().numpy().astype(np.int64), lens_end)
    # demotions (a sequence's append completing a group) inside the timed window
    n_dem = 0
    if grouped:
        for s_ in range(1, args.steps + 1):
            r = lens_before + s_ - wl.n_sink - wl.n_recent
            n_dem += int(((r > 0) & (r % 128 == 0)).sum())
    ms_step = max(ms_timed, dem_ms) if dem_ms is not None else ms_timed
    log(f"[bench] {args.steps} timed steps: {ms_timed:.4f} ms/step ({n_dem} demotions; host enqueue "
        f"{host_ms:.4f} ms/step); 128-step window "
        f"{dem_ms if dem_ms is None else round(dem_ms, 4)} ms/step")

    # algorithmic bytes of each timed step (lengths after that step's append)
    kv_sum = qo_sum = 0
    for s_ in range(1, args.steps + 1):
        kv_b, qo_b = decode_bytes(wl, lens_before + s_, wl.n_sink, wl.n_recent)
        kv_sum += kv_b
        qo_sum += qo_b
    step_bytes = (kv_sum + qo_sum) / args.steps

    # the split-K kernel inside the timed steps: its launches' average duration, and the bytes it reads: the
    # codes and scales/zeros of every quantized token and the bf16 band tokens (the KV bytes of the step);
    # query prep and merge: median over the warm-up steps (the first launches carry one-time costs)
    stage_us = {n: round(1e3 * float(np.median([ev[k_][0].elapsed_time(ev[k_][1]) for ev in wevs])), 2)
                for k_, n in enumerate(names) if n != "splitk" and wevs}
    kern_ms = sum(evs[n][1][0].elapsed_time(evs[n][1][1]) for n in sampled) / len(sampled)
    stage_us["splitk"] = round(kern_ms * 1e3, 2)
    kern_bytes = int(round(kv_sum / args.steps))
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    log(f"[bench] split-K kernel {kern_ms * 1e3:.1f} us, {achieved:.0f} GB/s; kernels {stage_us}")

    # the read pattern's ceiling: the library's read probe reads the same quantized head blocks as the split-K
    # kernel (same walks, work-groups and page order, no band, no arithmetic), timed the same way
    probe = None
    shape = K.decode_shape(cfg, B, T_end)
    if grouped and shape["matrix_cores"]:
        xo = torch.empty((B, n_kv, shape["max_chunks"] if shape["balanced"] else shape["walks"]), dtype=torch.int32,
                         device=dev)
        K.read_probe(cache, xo, T_end)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in pev:
            e0.record()
            K.read_probe(cache, xo, T_end)
            e1.record()
        torch.cuda.synchronize()
        p_ms = sum(e0.elapsed_time(e1) for e0, e1 in pev) / len(pev)
        hb = K.page_bytes(cfg) // n_kv
        q_bytes = sum(max(0, (int(t) - wl.n_sink - wl.n_recent) // 128) * 2 * hb * n_kv for t in lens_end)
        probe = {"kernel_us": round(p_ms * 1e3, 2), "bytes_per_launch": int(q_bytes),
                 "achieved": round(q_bytes / (p_ms * 1e-3) / 1e9, 1),
                 "frac": round(q_bytes / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "launches_timed": len(pev)}
        log(f"[bench] read probe {probe}")

    variant = ("" if wl.scheme == synth.WORKLOADS[wl.name].scheme else wl.scheme) + \
        (" key-only" if wl.key_only else "") + \
        (f" hadamard-{wl.hadamard_block}" if wl.rotation == "saw" and wl.hadamard_block != 128 else "")
    traffic = read_traffic(wl.name, variant.strip())
    kernel = {"int2_channel": "split-K decode, INT2 per-channel pages + bf16 band",
              "int2_token": "split-K decode, INT2 per-token pages + bf16 band",
              "int4_channel": "split-K decode, INT4 per-channel pages + bf16 band",
              "int4_token": "split-K decode, INT4 per-token pages"}
    return {
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2),
        "ms_per_step": round(ms_step, 5),
        "steps_per_s": round(1000.0 / ms_step, 2),
        "config": {"workload": wl.name, "batch": B, "ctx": T_end,
                   "ctx_range": [int(lens_end.min()), int(lens_end.max())], "n_q_heads": n_q, "n_kv_heads": n_kv,
                   "head_dim": 128,
                   "scheme": ({"int2_channel": "int2 per-channel, 128-token groups, bf16 scale/zero",
                               "int2_token": "int2 per-token over 128 channels, bf16 scale/zero",
                               "int4_channel": "int4 per-channel, 128-token groups, bf16 scale/zero",
                               "int4_token": "int4 per-token, bf16 scale/zero, randomized Hadamard"}
                              [wl.scheme] + (", key-only rotation" if wl.key_only else "") +
                              (f", Hadamard block {wl.hadamard_block}" if wl.rotation == "saw" else "")),
                   "sink_recent": [wl.n_sink, wl.n_recent], "page_tokens": 64, "split_tokens": split,
                   "decode_impl": args.impl,
                   "step": ("append 1 token/seq (write) + decode attention; group demotion counted at its steady "
                            "rate: ms_per_step = max(timed window, 128-step window), every sequence completing one "
                            "128-token group in the 128-step window" if grouped else
                            "append 1 token/seq (write) + decode attention")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": kernel[wl.scheme], "kernel_us": round(kern_ms * 1e3, 2),
                     "kernel_launches_timed": len(sampled), "bytes_per_launch": kern_bytes},
        "decode_kernels_us": stage_us,
        "read_probe": probe,
        "timed_window": {"ms_per_step": round(ms_timed, 5), "demotions": n_dem,
                         "window128_ms_per_step": None if dem_ms is None else round(dem_ms, 5)},
    }


if __name__ == "__main__":
    main()
