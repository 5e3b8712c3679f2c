#!/usr/bin/env python3
"""Decode-step benchmark: paged KV append + split-KV decode attention + merge.

One "step" is one pass of the whole hot path over one batch: the new token's
K/V appended, then decode attention and the LSE merge, through the C ABI's
``pkv_paged_decode_step`` (the append runs inside the decode kernel), on
synthetic inputs already resident in HBM.  The same step as two calls
(``pkv_kv_append`` then ``pkv_paged_decode_attention``) is timed alongside.  The default workload is
the Llama-3-8B-shaped layer (batch 64, 32 query / 8 KV heads, head dim 128,
bf16, 16-token blocks, context lengths uniform in [512, 4096]); ``--config``
picks another named workload.  Inputs are rotated over enough copies to span
more than the 256 MB last-level cache, so the timed steps read HBM.

Prints one JSON line.  ``value`` is the step's algorithmic bytes (K/V rows of
every attended token, the appended rows, q, out, block-table entries and
lengths) divided by the measured step time, in GB/s.  ``roofline`` reports the
decode kernel alone, timed live with HIP events on the launch stream through
``pkv_paged_decode_partials`` (the same kernel and grid without the merge), or,
for the balanced split (partition size -1, the default of the batch-64, mix and
fp8 workloads), ``pkv_paged_decode_partials_planned`` on a schedule made
beforehand, against the 8 TB/s HBM peak.
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the same
workload.  ``attainable`` is the read rate measured live by
``pkv_stream_read`` (a kernel that only reads a 2 GiB buffer) and the
roofline kernel's rate as a fraction of it: the practical ceiling, below the
data-sheet peak.
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

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="host seconds of timed oracle steps per CPU row (all cores, one core)")
    ap.add_argument("--new-tokens", type=int, default=0,
                    help="time the multi-token path instead: every sequence of the workload "
                         "brings this many new tokens (append + shifted-causal attention)")
    ap.add_argument("--quant-append", choices=["fixed", "running"], default=None,
                    help="with an e4m3 workload: the step appends bf16 rows through "
                         "pkv_kv_append_quant (scale policy fixed or running amax), then attends")
    ap.add_argument("--copy-blocks", type=int, default=0,
                    help="time pkv_copy_blocks alone: this many copy-on-write block copies "
                         "of the workload's pools (bf16 Llama-3-8B blocks: 32 KiB each of K and V)")
    ap.add_argument("--mla", default=None,
                    help="time absorbed MLA decode on a named latent-cache workload instead "
                         "(deepseek_mla_b64, deepseek_lite_mla_b8)")
    ap.add_argument("--vector-decode", action="store_true",
                    help="load libpkv_vector.so: every decode on the vector kernel (the "
                         "baseline the matrix-core kernel is measured against)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only time a plain device-to-device copy of this many MiB (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(mib, reps):
    """A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
    WRITE_SIZE per dispatch, divided by ``mib`` MiB, give the counters' scale."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_mib": mib, "us_per_copy": round(ms * 1e3, 2),
                      "copy_gbps_read_plus_write": round(2 * mib * 2 ** 20 / (ms * 1e-3) / 1e9, 1)}))


def main():
    args = parse()
    if args.vector_decode:
        os.environ["PKV_LIB"] = os.path.join(ROOT, "paged_kv_cache_25_amd", "libpkv_vector.so")
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only: the decode path "
                          "shards by sequence or KV head with no exchange, so N GPUs run N "
                          "independent copies of this benchmark; --gpus must be 1"}))
        sys.exit(2)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, max(1, args.steps))
        return
    if args.new_tokens:
        main_multi(args)
        return
    if args.quant_append:
        main_quant(args)
        return
    if args.copy_blocks:
        main_copy_blocks(args)
        return
    if args.mla:
        main_mla(args)
        return

    import torch

    from paged_kv_cache_25_amd import ops, traffic
    from workloads import named_config

    lib = ops.load()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")

    t0 = time.time()
    inp = named_config(args.config, seed=args.seed)
    P = inp.partition_size if args.partition_size is None else args.partition_size
    print(f"[bench] workload {inp.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    TD = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}

    def to_dev(arr, dt):
        if dt is None:
            return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
        if dt == "fp8_e4m3":
            return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)

    base = dict(q=to_dev(inp.q, inp.q_dtype), k_pool=to_dev(inp.k_pool, inp.kv_dtype),
                v_pool=to_dev(inp.v_pool, inp.kv_dtype), k_new=to_dev(inp.k_new, inp.kv_dtype),
                v_new=to_dev(inp.v_new, inp.kv_dtype), tables=to_dev(inp.block_tables, None),
                lens=to_dev(inp.context_lens, None),
                k_scales=None if inp.k_scales is None else to_dev(inp.k_scales, None),
                v_scales=None if inp.v_scales is None else to_dev(inp.v_scales, None))
    footprint = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    n_copies = max(1, math.ceil(1.5 * 2 ** 30 / footprint)) if footprint < 1.5 * 2 ** 30 else 1
    if footprint * n_copies > 0.5 * torch.cuda.get_device_properties(0).total_memory:
        n_copies = 1
    copies = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                       for _ in range(n_copies - 1)]

    B, Hq, Hkv, D = inp.num_seqs, inp.num_q_heads, inp.num_kv_heads, inp.head_dim
    NB, MB = inp.num_blocks, inp.block_tables.shape[1]
    mcl = inp.max_context_len
    qcode, kvcode = ops.dtype_code(base["q"].dtype), ops.dtype_code(base["k_pool"].dtype)
    ws_bytes = ops.workspace_bytes(B, Hq, D, mcl, P)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p

    def ptr(t):
        return None if t is None else V(t.data_ptr())

    balanced = P == ops.PKV_PARTITION_BALANCED
    slots = lib.pkv_decode_plan_slots(B, Hq, Hkv, D, qcode, kvcode) if balanced else 0
    calls = []
    for c in copies:
        c["out"] = torch.empty(B, Hq, D, dtype=c["q"].dtype, device=dev)
        c["ws"] = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        app = (ptr(c["k_pool"]), ptr(c["v_pool"]), ptr(c["k_new"]), ptr(c["v_new"]),
               ptr(c["tables"]), ptr(c["lens"]), B, Hkv, D, 16, NB, MB, kvcode, sp)
        att = (ptr(c["out"]), ptr(c["q"]), ptr(c["k_pool"]), ptr(c["v_pool"]),
               ptr(c["k_scales"]), ptr(c["v_scales"]), ptr(c["tables"]), ptr(c["lens"]), B, Hq,
               Hkv, D, 16, NB, MB, mcl, ctypes.c_float(inp.softmax_scale), P, ptr(c["ws"]),
               ctypes.c_size_t(c["ws"].numel()), qcode, kvcode, sp)
        if balanced:
            # the decode kernel alone on a schedule made beforehand (the plan
            # kernel and the merge are in the attention call and the step)
            c["plan"] = ops.decode_plan(c["lens"], slots, MB)
            c["parts"] = torch.empty(slots * Hq * (D + 1) * 4 + 512, dtype=torch.uint8, device=dev)
            lse_off = ((slots * Hq * D * 4 + 255) // 256) * 256
            prt = (V(c["parts"].data_ptr()), V(c["parts"].data_ptr() + lse_off), ptr(c["plan"]),
                   ctypes.c_size_t(c["plan"].numel()), slots, ptr(c["q"]), ptr(c["k_pool"]),
                   ptr(c["v_pool"]), ptr(c["k_scales"]), ptr(c["v_scales"]), ptr(c["tables"]),
                   ptr(c["lens"]), B, Hq, Hkv, D, 16, NB, MB, ctypes.c_float(inp.softmax_scale),
                   qcode, kvcode, sp)
            maxp = slots
        else:
            maxp = max(1, -(-mcl // P)) if P else 1
            c["parts"] = torch.empty(max(ops.workspace_bytes(B, Hq, D, mcl, P),
                                         B * Hq * maxp * (D + 1) * 4 + 256), dtype=torch.uint8,
                                     device=dev)
            lse_off = ((B * Hq * maxp * D * 4 + 255) // 256) * 256
            # the decode kernel alone, same grid and work, partials into its own buffer
            prt = (V(c["parts"].data_ptr()), V(c["parts"].data_ptr() + lse_off), maxp, ptr(c["q"]),
                   ptr(c["k_pool"]), ptr(c["v_pool"]), ptr(c["k_scales"]), ptr(c["v_scales"]),
                   ptr(c["tables"]), ptr(c["lens"]), B, Hq, Hkv, D, 16, NB, MB,
                   ctypes.c_float(inp.softmax_scale), P, qcode, kvcode, sp)
        stp = (ptr(c["out"]), ptr(c["q"]), ptr(c["k_pool"]), ptr(c["v_pool"]), ptr(c["k_new"]),
               ptr(c["v_new"]), ptr(c["k_scales"]), ptr(c["v_scales"]), ptr(c["tables"]),
               ptr(c["lens"]), B, Hq, Hkv, D, 16, NB, MB, mcl, ctypes.c_float(inp.softmax_scale),
               P, ptr(c["ws"]), ctypes.c_size_t(c["ws"].numel()), qcode, kvcode, sp)
        calls.append((app, att, prt, maxp > 1, stp))

    f_app, f_att = lib.pkv_kv_append, lib.pkv_paged_decode_attention
    f_prt = lib.pkv_paged_decode_partials_planned if balanced else lib.pkv_paged_decode_partials
    f_stp = lib.pkv_paged_decode_step

    def step(i):
        # one decode step: append + attention (+ merge), the append fused into the decode kernel
        if f_stp(*calls[i % n_copies][4]) != 0:
            raise RuntimeError("libpkv call failed")

    def step_two_calls(i):
        app, att = calls[i % n_copies][0], calls[i % n_copies][1]
        if f_app(*app) != 0 or f_att(*att) != 0:
            raise RuntimeError("libpkv call failed")

    print(f"[bench] {n_copies} input copies of {footprint / 1e6:.1f} MB; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- whole steps ----------------------------------------------------------
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    step_ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {args.steps} steps: {step_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    repeats = step_repeats(step, args.steps, stream)

    # ---- per kernel: the decode kernel alone (partials call), the merge as the
    # ---- attention call minus the decode kernel, the append alone ---------------
    def timed(fn, reps):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def att_only(i):
        if f_att(*calls[i % n_copies][1]) != 0:
            raise RuntimeError("attention call failed")

    def decode_only(i):
        if f_prt(*calls[i % n_copies][2]) != 0:
            raise RuntimeError("partials call failed")

    def append_only(i):
        if f_app(*calls[i % n_copies][0]) != 0:
            raise RuntimeError("append call failed")

    reps = args.kernel_reps
    two_call_ms = timed(step_two_calls, reps)
    att_ms = timed(att_only, reps)
    decode_ms = timed(decode_only, reps)
    append_ms = timed(append_only, reps)
    merge_ms = max(att_ms - decode_ms, 0.0) if calls[0][3] else 0.0

    # ---- accounting ---------------------------------------------------------------
    tr = traffic.attention_call_traffic(inp.context_lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                        head_dim=D, q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    ap = traffic.append_traffic(B, num_kv_heads=Hkv, head_dim=D, kv_dtype=inp.kv_dtype)
    step_bytes = tr["total_bytes"] + ap["bytes"]
    value = step_bytes / (step_ms * 1e-3) / 1e9
    # the decode kernel's own algorithmic reads: K/V rows (and e4m3 scales)
    roof_bytes = tr["kv_bytes"] + tr["scale_bytes"]
    kernel_gbps = roof_bytes / (decode_ms * 1e-3) / 1e9

    mfma = (inp.q_dtype == "bf16" and inp.kv_dtype == "bf16" and Hq // Hkv >= 2
            and not args.vector_decode)
    kernel_name = "paged_decode_mfma_kernel" if mfma else "paged_decode_kernel"
    traffic_bytes = measured_traffic(inp.name, P, kernel_name) if args.seed is None else None
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_budget_s)

    result = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) and decode tokens/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{inp.kv_dtype} kv, {inp.q_dtype} q, f32 accumulate",
        "data": "synthetic (seeded N(0,1) K/V/q, random block placement)",
        "config": {"workload": inp.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "block_size": 16, "partition_size": P,
                   "context_tokens": int(inp.context_lens.sum()), "max_context": mcl,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_steps_per_s": round(1e3 / step_ms, 1),
        "tokens_per_s": round(B * 1e3 / step_ms, 1),
        "kernel_us": {"append": round(append_ms * 1e3, 2), "decode": round(decode_ms * 1e3, 2),
                      ("plan_and_merge" if balanced else "merge"): round(merge_ms * 1e3, 2),
                      "attention_call": round(att_ms * 1e3, 2),
                      "step_as_two_calls": round(two_call_ms * 1e3, 2)},
        "roofline": {"kernel": f"{kernel_name}<{D}>",
                     "bound": "hbm",
                     "achieved": round(kernel_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_bytes,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "algorithmic_bytes_per_launch": roof_bytes},
        "step_repeats": repeats,
        "cpu_baseline": cpu,
        "attainable": attainable_entry(ops, stream, kernel_gbps),
        "input_copies": n_copies,
    }
    print(json.dumps(result), flush=True)


def step_repeats(step, steps, stream, n=5):
    """The timing protocol's repeats: after the timed region, ``n`` more runs
    of ``steps`` steps each, timed with HIP events on ``stream``; their median
    and best ms per step (the pages report the fastest of several runs)."""
    import torch
    per = []
    for r in range(n):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            step(i)
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / steps)
    return {"runs": n, "steps_each": steps, "median_ms_per_step": round(float(np.median(per)), 5),
            "best_ms_per_step": round(min(per), 5), "worst_ms_per_step": round(max(per), 5)}


def to_device(arr, dt, dev):
    import torch
    if dt is None:
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    if dt == "fp8_e4m3":
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def rotated_copies(base):
    """The inputs plus enough clones to span well over the last-level cache."""
    import torch
    footprint = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    n = max(1, math.ceil(1.5 * 2 ** 30 / footprint)) if footprint < 1.5 * 2 ** 30 else 1
    if footprint * n > 0.5 * torch.cuda.get_device_properties(0).total_memory:
        n = 1
    return [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                     for _ in range(n - 1)], footprint


def event_timer(stream):
    """ms per call of fn(i) over reps calls, with HIP events on ``stream``."""
    import torch

    def timed(fn, reps):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    return timed


STREAM_READ_BYTES = 2 * 2 ** 30
STREAM_READ_GRIDS = (1024, 2048, 4096, 8192, 16384)


def attainable_read(ops, stream, reps=20):
    """The measured read ceiling: pkv_stream_read over a 2 GiB buffer (8x the
    last-level cache), the best of a few grid sizes, timed with HIP events on
    ``stream``; returns (GB/s, workgroups)."""
    import torch
    buf = torch.arange(STREAM_READ_BYTES // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(int(ops.load().pkv_stream_read_out_words(max(STREAM_READ_GRIDS))),
                      dtype=torch.int32, device="cuda")
    timed = event_timer(stream)
    best = (0.0, 0)
    for g in STREAM_READ_GRIDS:
        run = lambda i, g=g: ops.stream_read(buf, g, out=out, stream=stream)
        for i in range(3):
            run(i)
        ms = min(timed(run, reps) for _ in range(2))
        best = max(best, (STREAM_READ_BYTES / (ms * 1e-3) / 1e9, g))
    del buf, out
    torch.cuda.empty_cache()
    return best


GATHER_WORKGROUPS = 6144          # two rounds of the 3,072 resident decode waves
GATHER_PER_WORKGROUP = 26         # about one decode workgroup's blocks on the batch-64 layer


def attainable_gather(ops, stream, reps=20):
    """The read ceiling of the decode kernels' access pattern: pkv_gather_read
    over 6,144 x 26 distinct 4 KiB chunks (654 MB) scattered at random over a
    2 GiB buffer, timed with HIP events on ``stream``; returns GB/s."""
    import torch
    n_chunks = STREAM_READ_BYTES // 4096
    buf = torch.arange(STREAM_READ_BYTES // 4, dtype=torch.int32, device="cuda")
    perm = np.random.default_rng(11).permutation(n_chunks)[:GATHER_WORKGROUPS * GATHER_PER_WORKGROUP]
    ids = torch.from_numpy(perm.astype(np.int32)).cuda()
    out = torch.empty(64 * GATHER_WORKGROUPS, dtype=torch.int32, device="cuda")
    run = lambda i: ops.gather_read(buf, ids, GATHER_PER_WORKGROUP, out=out, stream=stream)
    for i in range(3):
        run(i)
    timed = event_timer(stream)
    ms = min(timed(run, reps) for _ in range(2))
    del buf, ids, out
    torch.cuda.empty_cache()
    return len(perm) * 4096 / (ms * 1e-3) / 1e9


def attainable_entry(ops, stream, kernel_gbps):
    """The ``attainable`` object of the JSON line: the read ceilings (one
    large buffer in order; scattered 4 KiB chunks, the decode kernels' own
    unit) and the roofline kernel's rate as a fraction of each."""
    gbps, grid = attainable_read(ops, stream)
    print(f"[bench] stream read: {gbps:.1f} GB/s ({grid} workgroups)", file=sys.stderr, flush=True)
    gather = attainable_gather(ops, stream)
    print(f"[bench] gather read of 4 KiB chunks: {gather:.1f} GB/s", file=sys.stderr, flush=True)
    return {"kernel": "stream_read_kernel", "bytes": STREAM_READ_BYTES, "workgroups": grid,
            "read_gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "roofline_kernel_frac_of_attainable": round(kernel_gbps / gbps, 4),
            "gather_kernel": "gather_read_kernel",
            "gather_bytes": GATHER_WORKGROUPS * GATHER_PER_WORKGROUP * 4096,
            "gather_read_gbps": round(gather, 1),
            "roofline_kernel_frac_of_gather": round(kernel_gbps / gather, 4)}


def main_multi(args):
    """Several new tokens per sequence (chunked prefill, a verify pass): one
    step is pkv_kv_append_tokens then pkv_paged_multi_query_attention over the
    workload's sequences, each bringing ``--new-tokens`` tokens."""
    import torch

    from paged_kv_cache_25_amd import ops, traffic
    from workloads import named_config

    lib = ops.load()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    T = args.new_tokens
    t0 = time.time()
    from workloads.configs import CONFIG_NAMES
    inp = named_config(args.config, seed=args.seed, new_tokens=("const", T),
                       name=f"{CONFIG_NAMES[args.config]}_t{T}")
    P = inp.partition_size if args.partition_size is None else args.partition_size
    balanced = P == ops.PKV_PARTITION_BALANCED
    print(f"[bench] workload {inp.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    base = dict(q=to_device(inp.q, inp.q_dtype, dev),
                k_pool=to_device(inp.k_pool, inp.kv_dtype, dev),
                v_pool=to_device(inp.v_pool, inp.kv_dtype, dev),
                k_new=to_device(inp.k_new, inp.kv_dtype, dev),
                v_new=to_device(inp.v_new, inp.kv_dtype, dev),
                tables=to_device(inp.block_tables, None, dev),
                lens=to_device(inp.context_lens, None, dev),
                qsl=to_device(inp.query_start_loc.astype(np.int32), None, dev),
                k_scales=None if inp.k_scales is None else to_device(inp.k_scales, None, dev),
                v_scales=None if inp.v_scales is None else to_device(inp.v_scales, None, dev))
    copies, footprint = rotated_copies(base)
    n_copies = len(copies)

    B, Hq, Hkv, D = inp.num_seqs, inp.num_q_heads, inp.num_kv_heads, inp.head_dim
    NB, MB = inp.num_blocks, inp.block_tables.shape[1]
    R = inp.total_queries
    mcl, mq = inp.max_context_len, inp.max_new_tokens
    qcode, kvcode = ops.dtype_code(base["q"].dtype), ops.dtype_code(base["k_pool"].dtype)
    if balanced:
        ws_bytes = int(lib.pkv_multi_query_balanced_workspace_bytes(B, mq, Hq, Hkv, D, qcode,
                                                                    kvcode))
        slots = int(lib.pkv_multi_query_plan_slots(B, mq, Hq, Hkv, D, qcode, kvcode))
        maxp = 1
    else:
        ws_bytes = ops.multi_query_workspace_bytes(R, Hq, D, mcl, P)
        maxp = max(1, -(-mcl // P)) if P else 1
    lse_off = ((R * Hq * maxp * D * 4 + 255) // 256) * 256
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p

    def ptr(t):
        return None if t is None else V(t.data_ptr())

    calls = []
    for c in copies:
        c["out"] = torch.empty(R, Hq, D, dtype=c["q"].dtype, device=dev)
        c["ws"] = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        app = (ptr(c["k_pool"]), ptr(c["v_pool"]), ptr(c["k_new"]), ptr(c["v_new"]),
               ptr(c["tables"]), ptr(c["lens"]), ptr(c["qsl"]), B, R, Hkv, D, 16, NB, MB,
               kvcode, sp)
        att = (ptr(c["out"]), ptr(c["q"]), ptr(c["k_pool"]), ptr(c["v_pool"]),
               ptr(c["k_scales"]), ptr(c["v_scales"]), ptr(c["tables"]), ptr(c["lens"]),
               ptr(c["qsl"]), B, R, mq, Hq, Hkv, D, 16, NB, MB, mcl,
               ctypes.c_float(inp.softmax_scale), P, ptr(c["ws"]),
               ctypes.c_size_t(c["ws"].numel()), qcode, kvcode, sp)
        if balanced:
            # the decode kernel alone on the call's slots: chunk rows [R, max_q, Hq, D]
            rows = slots * mq * Hq
            b_lse = ((rows * D * 4 + 255) // 256) * 256
            c["parts"] = torch.empty(b_lse + rows * 4, dtype=torch.uint8, device=dev)
            c["plan"] = torch.empty(int(lib.pkv_decode_plan_bytes(B, slots)), dtype=torch.uint8,
                                    device=dev)
            prt = (V(c["parts"].data_ptr()), V(c["parts"].data_ptr() + b_lse), ptr(c["plan"]),
                   ctypes.c_size_t(c["plan"].numel()), slots, ptr(c["q"]), ptr(c["k_pool"]),
                   ptr(c["v_pool"]), ptr(c["k_scales"]), ptr(c["v_scales"]), ptr(c["tables"]),
                   ptr(c["lens"]), ptr(c["qsl"]), B, R, mq, Hq, Hkv, D, 16, NB, MB,
                   ctypes.c_float(inp.softmax_scale), qcode, kvcode, sp)
        else:
            # the decode kernel alone (same grid and work, partials for every row)
            c["parts"] = torch.empty(lse_off + R * Hq * maxp * 4, dtype=torch.uint8, device=dev)
            prt = (V(c["parts"].data_ptr()), V(c["parts"].data_ptr() + lse_off), maxp,
                   ptr(c["q"]), ptr(c["k_pool"]), ptr(c["v_pool"]), ptr(c["k_scales"]),
                   ptr(c["v_scales"]), ptr(c["tables"]), ptr(c["lens"]), ptr(c["qsl"]), B, R, mq,
                   Hq, Hkv, D, 16, NB, MB, ctypes.c_float(inp.softmax_scale), P, qcode, kvcode,
                   sp)
        calls.append((app, att, prt))

    f_app, f_att = lib.pkv_kv_append_tokens, lib.pkv_paged_multi_query_attention
    f_prt = (lib.pkv_paged_multi_query_partials_planned if balanced
             else lib.pkv_paged_multi_query_partials)

    def step(i):
        app, att, _ = calls[i % n_copies]
        if f_app(*app) != 0 or f_att(*att) != 0:
            raise RuntimeError("libpkv call failed")

    print(f"[bench] {n_copies} input copies of {footprint / 1e6:.1f} MB; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    timed = event_timer(stream)
    step_ms = timed(step, args.steps)
    print(f"[bench] {args.steps} steps: {step_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    def att_only(i):
        if f_att(*calls[i % n_copies][1]) != 0:
            raise RuntimeError("attention call failed")

    def decode_only(i):
        if f_prt(*calls[i % n_copies][2]) != 0:
            raise RuntimeError("partials call failed")

    def append_only(i):
        if f_app(*calls[i % n_copies][0]) != 0:
            raise RuntimeError("append call failed")

    reps = args.kernel_reps
    att_ms = timed(att_only, reps)
    # the decode kernel alone: the partials call (the balanced split's plans
    # its chunks inside the kernel, as the attention call does)
    decode_ms = timed(decode_only, reps)
    append_ms = timed(append_only, reps)
    merge_ms = max(att_ms - decode_ms, 0.0) if (maxp > 1 or balanced) else 0.0

    t_new = np.diff(inp.query_start_loc)
    tr = traffic.multi_query_traffic(inp.context_lens, t_new, num_q_heads=Hq, num_kv_heads=Hkv,
                                     head_dim=D, q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    ap = traffic.append_traffic(R, num_kv_heads=Hkv, head_dim=D, kv_dtype=inp.kv_dtype)
    step_bytes = tr["total_bytes"] + ap["bytes"] + 4 * (B + 1)
    value = step_bytes / (step_ms * 1e-3) / 1e9
    kernel_gbps = tr["kv_bytes"] / (decode_ms * 1e-3) / 1e9
    mfma = inp.q_dtype == "bf16" and inp.kv_dtype == "bf16" and (Hq // Hkv) * mq >= 2
    cpu = None if args.no_cpu_baseline else cpu_baseline_multi(inp, args.cpu_budget_s)
    # The decode kernel the library picks: the matrix cores in 16-column tiles
    # (two per wave past 16 columns per KV head), and at head dim 128 with
    # four or more tiles one LDS-staged workgroup per unit.
    columns = mq * (Hq // Hkv)
    tiles2 = mfma and columns > 16
    if mfma and tiles2 and D == 128 and -(-columns // 32) >= 2:
        kprefix, kname = "paged_decode_lds_kernel", "paged_decode_lds_kernel<2, 2>"
    elif mfma:
        kprefix, kname = "paged_decode_mfma_kernel", f"paged_decode_mfma_kernel<{D}>"
    else:
        kprefix, kname = "paged_decode_kernel", f"paged_decode_kernel<{D}>"
    result = {
        "metric": "paged multi-token attention achieved HBM GB/s (% of peak) and new tokens/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{inp.kv_dtype} kv, {inp.q_dtype} q, f32 accumulate",
        "data": "synthetic (seeded N(0,1) K/V/q, random block placement)",
        "config": {"workload": inp.name, "batch": B, "new_tokens_per_seq": T, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "block_size": 16, "partition_size": P,
                   "context_tokens": int(inp.context_lens.sum()), "max_context": mcl,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "steps_per_s": round(1e3 / step_ms, 1),
        "new_tokens_per_s": round(R * 1e3 / step_ms, 1),
        "kernel_us": {"append": round(append_ms * 1e3, 2), "decode": round(decode_ms * 1e3, 2),
                      "merge": round(merge_ms * 1e3, 2), "attention_call": round(att_ms * 1e3, 2)},
        "roofline": {"kernel": kname + " (several new tokens)",
                     "bound": "hbm", "achieved": round(kernel_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(inp.name, P, kprefix),
                     "traffic_unit": f"HBM bytes per launch of {kprefix} (rocprofv3 FETCH_SIZE + "
                                     "WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": tr["kv_bytes"],
                     "flops_per_launch": tr["flops"]},
        "cpu_baseline": cpu,
        "attainable": attainable_entry(ops, stream, kernel_gbps),
        "input_copies": n_copies,
    }
    print(json.dumps(result), flush=True)


def main_quant(args):
    """An e4m3 decode step whose new K/V rows arrive in bf16: one step is
    pkv_kv_append_quant (quantise with the block's scale, fixed or running
    amax) then pkv_paged_decode_attention."""
    import torch

    from paged_kv_cache_25_amd import ops, traffic
    from workloads import named_config

    lib = ops.load()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    cfg = 5 if args.config == 2 else args.config
    inp = named_config(cfg, seed=args.seed)
    if inp.kv_dtype != "fp8_e4m3":
        raise SystemExit("--quant-append needs an e4m3 workload (e.g. --config 5)")
    P = inp.partition_size if args.partition_size is None else args.partition_size
    mode = ops.PKV_SCALE_RUNNING_AMAX if args.quant_append == "running" else ops.PKV_SCALE_FIXED
    rng = np.random.default_rng(0)
    new = [torch.from_numpy(rng.standard_normal(inp.k_new.shape).astype(np.float32)).to(
        torch.bfloat16) for _ in range(2)]
    base = dict(q=to_device(inp.q, inp.q_dtype, dev),
                k_pool=to_device(inp.k_pool, inp.kv_dtype, dev),
                v_pool=to_device(inp.v_pool, inp.kv_dtype, dev),
                k_new=new[0].to(dev), v_new=new[1].to(dev),
                tables=to_device(inp.block_tables, None, dev),
                lens=to_device(inp.context_lens, None, dev),
                k_scales=to_device(inp.k_scales, None, dev),
                v_scales=to_device(inp.v_scales, None, dev))
    copies, footprint = rotated_copies(base)
    n_copies = len(copies)
    B, Hq, Hkv, D = inp.num_seqs, inp.num_q_heads, inp.num_kv_heads, inp.head_dim
    NB, MB, mcl = inp.num_blocks, inp.block_tables.shape[1], inp.max_context_len
    qcode = ops.dtype_code(base["q"].dtype)
    ws_bytes = ops.workspace_bytes(B, Hq, D, mcl, P)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p

    def ptr(t):
        return None if t is None else V(t.data_ptr())

    calls = []
    for c in copies:
        c["out"] = torch.empty(B, Hq, D, dtype=c["q"].dtype, device=dev)
        c["ws"] = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        qa = (ptr(c["k_pool"]), ptr(c["v_pool"]), ptr(c["k_scales"]), ptr(c["v_scales"]),
              ptr(c["k_new"]), ptr(c["v_new"]), ops.PKV_BF16, ptr(c["tables"]), ptr(c["lens"]),
              None, B, B, Hkv, D, 16, NB, MB, mode, sp)
        att = (ptr(c["out"]), ptr(c["q"]), ptr(c["k_pool"]), ptr(c["v_pool"]),
               ptr(c["k_scales"]), ptr(c["v_scales"]), ptr(c["tables"]), ptr(c["lens"]), B, Hq,
               Hkv, D, 16, NB, MB, mcl, ctypes.c_float(inp.softmax_scale), P, ptr(c["ws"]),
               ctypes.c_size_t(c["ws"].numel()), qcode, ops.PKV_FP8_E4M3, sp)
        calls.append((qa, att))
    f_q, f_att = lib.pkv_kv_append_quant, lib.pkv_paged_decode_attention

    def step(i):
        qa, att = calls[i % n_copies]
        if f_q(*qa) != 0 or f_att(*att) != 0:
            raise RuntimeError("libpkv call failed")

    def quant_only(i):
        if f_q(*calls[i % n_copies][0]) != 0:
            raise RuntimeError("quant append failed")

    def att_only(i):
        if f_att(*calls[i % n_copies][1]) != 0:
            raise RuntimeError("attention call failed")

    print(f"[bench] {inp.name} + quantise-on-append ({args.quant_append}): {n_copies} input "
          f"copies of {footprint / 1e6:.1f} MB; warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    timed = event_timer(stream)
    step_ms = timed(step, args.steps)
    quant_ms = timed(quant_only, args.kernel_reps)
    att_ms = timed(att_only, args.kernel_reps)
    tr = traffic.attention_call_traffic(inp.context_lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                        head_dim=D, q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    qb = traffic.quant_append_traffic(B, num_kv_heads=Hkv, head_dim=D, new_dtype="bf16")
    value = (tr["total_bytes"] + qb["bytes"]) / (step_ms * 1e-3) / 1e9
    result = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) and decode tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"fp8_e4m3 kv (quantised on append from bf16), {inp.q_dtype} q, f32 accumulate",
        "data": "synthetic (seeded N(0,1) K/V/q, random block placement)",
        "config": {"workload": f"{inp.name}_quant_{args.quant_append}", "batch": B,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "block_size": 16,
                   "partition_size": P, "context_tokens": int(inp.context_lens.sum()),
                   "scale_policy": args.quant_append, "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B * 1e3 / step_ms, 1),
        "kernel_us": {"quant_append": round(quant_ms * 1e3, 2),
                      "attention_call": round(att_ms * 1e3, 2)},
        "roofline": {"kernel": "kv_append_quant_kernel<bf16>", "bound": "hbm",
                     "achieved": round(qb["bytes"] / (quant_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(qb["bytes"] / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5),
                     "traffic": None, "algorithmic_bytes_per_launch": qb["bytes"],
                     "note": "launch-latency bound: a few hundred KB per launch"},
        "cpu_baseline": None,
        "input_copies": n_copies,
    }
    print(json.dumps(result), flush=True)


def main_copy_blocks(args):
    """pkv_copy_blocks on its own: ``--copy-blocks`` (src, dst) pairs over the
    workload's pools (distinct destinations, none a source), rotated over
    several pair lists so the sources come from HBM."""
    import torch

    from paged_kv_cache_25_amd import ops
    from workloads import named_config

    lib = ops.load()
    dev = torch.device("cuda:0")
    inp = named_config(args.config, seed=args.seed)
    NB, Hkv, D = inp.num_blocks, inp.num_kv_heads, inp.head_dim
    n = args.copy_blocks
    if 2 * n > NB:
        raise SystemExit(f"--copy-blocks {n}: the pool has {NB} blocks; at most {NB // 2}")
    kp = to_device(inp.k_pool, inp.kv_dtype, dev)
    vp = to_device(inp.v_pool, inp.kv_dtype, dev)
    ks = None if inp.k_scales is None else to_device(inp.k_scales, None, dev)
    vs = None if inp.v_scales is None else to_device(inp.v_scales, None, dev)
    rng = np.random.default_rng(0)
    lists = []
    for _ in range(4):
        ids = rng.permutation(NB)
        lists.append(torch.tensor(np.stack([ids[:n], ids[n:2 * n]], 1).astype(np.int32), device=dev))
    code = ops.dtype_code(kp.dtype)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    f = lib.pkv_copy_blocks

    def run(i):
        pr = lists[i % len(lists)]
        if f(V(kp.data_ptr()), V(vp.data_ptr()), None if ks is None else V(ks.data_ptr()),
             None if vs is None else V(vs.data_ptr()), V(pr.data_ptr()), n, NB, Hkv, D, 16, code,
             sp) != 0:
            raise RuntimeError("pkv_copy_blocks failed")

    for i in range(args.warmup):
        run(i)
    timed = event_timer(stream)
    ms = timed(run, args.steps)
    block = Hkv * 16 * D * {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[inp.kv_dtype]
    moved = n * 2 * block * 2 + (n * Hkv * 4 * 4 if ks is not None else 0)   # read + write
    gbps = moved / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "copy-on-write block copies achieved HBM GB/s (read + write)",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": inp.kv_dtype, "data": "synthetic",
        "config": {"workload": f"{inp.name}_copy_blocks_{n}", "pairs": n, "block_bytes": block,
                   "kv_heads": Hkv, "head_dim": D},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": moved},
        "cpu_baseline": None}), flush=True)


def main_mla(args):
    """Absorbed MLA decode: one step is pkv_mla_append (the new latent row)
    then pkv_mla_decode_attention over the paged latent cache.  The decode
    kernel alone is timed through pkv_mla_decode_partials."""
    import torch

    from paged_kv_cache_25_amd import ops, traffic
    from workloads.mla import named_mla

    lib = ops.load()
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = named_mla(args.mla)
    P = inp.partition_size if args.partition_size is None else args.partition_size
    print(f"[bench] workload {inp.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    base = dict(q=to_device(inp.q, inp.dtype, dev), pool=to_device(inp.latent_pool, inp.dtype, dev),
                new=to_device(inp.latent_new, inp.dtype, dev),
                tables=to_device(inp.block_tables, None, dev),
                lens=to_device(inp.context_lens, None, dev))
    copies, footprint = rotated_copies(base)
    n_copies = len(copies)
    B, H, dc, dr = inp.num_seqs, inp.num_heads, inp.kv_lora_rank, inp.rope_dim
    NB, MB, mcl = inp.num_blocks, inp.block_tables.shape[1], inp.max_context_len
    ws_bytes = int(lib.pkv_mla_workspace_bytes(B, H, dc, mcl, P))
    balanced = P == ops.PKV_PARTITION_BALANCED      # split + chunks + merge in one call
    maxp = 1 if balanced or not P else max(1, -(-mcl // P))
    lse_off = ((B * H * maxp * dc * 4 + 255) // 256) * 256
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p

    def ptr(t):
        return V(t.data_ptr())

    calls = []
    for c in copies:
        c["out"] = torch.empty(B, H, dc, dtype=torch.bfloat16, device=dev)
        c["ws"] = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        c["parts"] = torch.empty(lse_off + B * H * maxp * 4, dtype=torch.uint8, device=dev)
        app = (ptr(c["pool"]), ptr(c["new"]), ptr(c["tables"]), ptr(c["lens"]), B, dc + dr, 16, NB,
               MB, sp)
        att = (ptr(c["out"]), ptr(c["q"]), ptr(c["pool"]), ptr(c["tables"]), ptr(c["lens"]), B, H,
               dc, dr, 16, NB, MB, mcl, ctypes.c_float(inp.softmax_scale), P, ptr(c["ws"]),
               ctypes.c_size_t(c["ws"].numel()), sp)
        prt = (V(c["parts"].data_ptr()), V(c["parts"].data_ptr() + lse_off), maxp, ptr(c["q"]),
               ptr(c["pool"]), ptr(c["tables"]), ptr(c["lens"]), B, H, dc, dr, 16, NB, MB,
               ctypes.c_float(inp.softmax_scale), P, sp)
        calls.append((app, att, prt))
    f_app, f_att, f_prt = lib.pkv_mla_append, lib.pkv_mla_decode_attention, lib.pkv_mla_decode_partials

    def step(i):
        app, att, _ = calls[i % n_copies]
        if f_app(*app) != 0 or f_att(*att) != 0:
            raise RuntimeError("libpkv call failed")

    def att_only(i):
        if f_att(*calls[i % n_copies][1]) != 0:
            raise RuntimeError("attention call failed")

    def decode_only(i):
        if f_prt(*calls[i % n_copies][2]) != 0:
            raise RuntimeError("partials call failed")

    print(f"[bench] {n_copies} input copies of {footprint / 1e6:.1f} MB; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    timed = event_timer(stream)
    step_ms = timed(step, args.steps)
    att_ms = timed(att_only, args.kernel_reps)
    # The balanced split's kernels run inside one call: the roofline is then
    # taken over the whole call (chunks, each planning its own, and merge; a
    # plan kernel first for more than 256 sequences), a lower bound on the
    # chunk kernel's own rate (rocprofv3 gives the kernels apart).
    decode_ms = att_ms if balanced else timed(decode_only, args.kernel_reps)
    merge_ms = max(att_ms - decode_ms, 0.0) if maxp > 1 else 0.0
    tr = traffic.mla_attention_traffic(inp.context_lens, num_heads=H, kv_lora_rank=dc,
                                       rope_dim=dr)
    step_bytes = tr["total_bytes"] + 2 * B * (dc + dr) * 2
    value = step_bytes / (step_ms * 1e-3) / 1e9
    kernel_gbps = tr["kv_bytes"] / (decode_ms * 1e-3) / 1e9
    tflops = tr["flops"] / (decode_ms * 1e-3) / 1e12
    result = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) and decode tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 latent cache and queries, f32 accumulate",
        "data": "synthetic (seeded N(0,1) latents and absorbed queries, random block placement)",
        "config": {"workload": inp.name, "batch": B, "heads": H, "kv_lora_rank": dc,
                   "rope_dim": dr, "block_size": 16, "partition_size": P,
                   "context_tokens": int(inp.context_lens.sum()), "max_context": mcl,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B * 1e3 / step_ms, 1),
        "kernel_us": ({"attention_call": round(att_ms * 1e3, 2)} if balanced else
                      {"decode": round(decode_ms * 1e3, 2), "merge": round(merge_ms * 1e3, 2),
                       "attention_call": round(att_ms * 1e3, 2)}),
        "roofline": {"kernel": (("balanced_split_kernel + " if B > 256 else "")
                                + "mla_decode_kernel + merge_wide_kernel"
                                if balanced else "mla_decode_kernel"), "bound": "hbm",
                     "achieved": round(kernel_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(inp.name, P, "mla_decode_kernel"),
                     "traffic_unit": "HBM bytes per launch of mla_decode_kernel (rocprofv3 "
                                     "FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": tr["kv_bytes"],
                     "mfma": {"achieved_tflops": round(tflops, 1), "peak_tflops": 2500.0,
                              "frac": round(tflops / 2500.0, 4),
                              "flops_per_launch": tr["flops"]}},
        "cpu_baseline": None,
        "input_copies": n_copies,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_multi(inp, budget_s):
    """The float64 oracle on a bounded sample of the multi-token workload:
    append + attention for whole sequences in order, BLAS on one thread."""
    import oracle.paged_attention as pa
    from paged_kv_cache_25_amd import traffic
    from threadpoolctl import threadpool_limits
    qsl = inp.query_start_loc
    done, elapsed = [], 0.0
    with threadpool_limits(1):
        for k in range(-1, 1 << 30):      # k = -1 untimed; then around the batch until the budget
            if inp.num_seqs == 0:
                break
            b = max(k, 0) % inp.num_seqs
            q0, q1 = int(qsl[b]), int(qsl[b + 1])
            tab = inp.block_tables[b:b + 1]
            lens = inp.context_lens[b:b + 1]
            loc = np.array([0, q1 - q0])
            ids = tab[0][tab[0] >= 0]
            kp, vp = inp.k_pool[ids], inp.v_pool[ids]          # the sequence's own blocks
            local = np.arange(len(ids), dtype=np.int32)[None, :]
            t = time.perf_counter()
            kp, vp = pa.kv_append_tokens(kp, vp, inp.k_new[q0:q1], inp.v_new[q0:q1], local, lens,
                                         loc, inp.block_size, inplace=True)
            pa.multi_query_attention(inp.q[q0:q1], kp, vp, local, lens, loc,
                                     block_size=inp.block_size, softmax_scale=inp.softmax_scale,
                                     q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype,
                                     k_scales=None if inp.k_scales is None else inp.k_scales[ids],
                                     v_scales=None if inp.v_scales is None else inp.v_scales[ids])
            if k < 0:
                continue
            elapsed += time.perf_counter() - t
            done.append(b)
            if elapsed > budget_s:
                break
    t_new = np.diff(qsl)[done]
    tr = traffic.multi_query_traffic(inp.context_lens[done], t_new, num_q_heads=inp.num_q_heads,
                                     num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                                     q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    ap = traffic.append_traffic(int(t_new.sum()), num_kv_heads=inp.num_kv_heads,
                                head_dim=inp.head_dim, kv_dtype=inp.kv_dtype)
    return {"value": round((tr["total_bytes"] + ap["bytes"]) / elapsed / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} sequences taken in order from the {inp.num_seqs}-sequence batch "
                      f"({len(done) / max(inp.num_seqs, 1):.2f} passes, {tr['rows']} new tokens over "
                      f"{tr['tokens']} cached), append + attention, float64 NumPy, {elapsed:.1f} s",
            "new_tokens_per_s": round(int(t_new.sum()) / elapsed, 3)}


PROFILES = os.path.join(ROOT, "profiles")


def _traffic_fields(path):
    """The machine-readable 'key: value' lines of a profiles/*_traffic.txt summary."""
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip().replace("_", "").isalnum():
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    return fields


def sources_sha256(rels):
    import hashlib
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, partition_size, kernel):
    """HBM bytes per launch of ``kernel`` (a name prefix: paged_decode_mfma_kernel,
    paged_decode_kernel, mla_decode_kernel) on ``workload`` at ``partition_size``,
    from a committed rocprofv3 counter summary (profiles/*_traffic.txt, copy
    calibrated); None when no summary matches or the kernel's sources, listed
    in the summary, no longer hash to what was measured."""
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_traffic.txt"))):
        f = _traffic_fields(path)
        if (f.get("workload") != workload or f.get("kernel") != kernel
                or f.get("partition_size") != str(partition_size)):
            continue
        rels = [r.strip() for r in f.get("kernel_sources", "").split(",") if r.strip()]
        if rels and sources_sha256(rels) == f.get("kernel_source_sha256"):
            return int(f["traffic_bytes_per_launch"])
    return None


def host_description():
    """CPU model (/proc/cpuinfo), the cores this process may run on and the
    BLAS numpy calls (threadpoolctl)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')})"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return model, len(os.sched_getaffinity(0)), ", ".join(blas) or "none found"


def cpu_baseline(inp, budget_s):
    """The float64 oracle, as it stands, on the same workload: whole decode
    steps (append + attention for every sequence), BLAS on all the cores this
    process may use, then again on one core.  Each row runs one untimed step,
    then timed steps until about ``budget_s`` seconds (at least 3 when a step
    fits, the pages' own "fastest of several" convention); ``value`` is the
    best step's algorithmic bytes per second.  A workload whose one step
    takes longer than the budget is sampled by sequences instead."""
    import oracle.paged_attention as pa
    from threadpoolctl import threadpool_limits

    from paged_kv_cache_25_amd import traffic
    model, cores, blas = host_description()
    rows = {}
    for n in (cores, 1):
        with threadpool_limits(n):
            rows[n] = _cpu_steps(inp, budget_s, pa, traffic)
        rows[n]["cores"] = n
        if n == 1 == cores:
            break
    out = dict(rows[cores])
    out.update(kind="oracle", cpu_model=model, blas=blas)
    if cores != 1:
        out["single_core"] = {k: rows[1][k] for k in ("value", "cores", "sample",
                                                      "best_s_per_step", "median_s_per_step")}
    return out


def _one_step(inp, pa, kp, vp, seqs=None):
    """Seconds of one oracle append + attention over the batch (or ``seqs``)
    with the pools kp, vp."""
    sub = inp if seqs is None else inp.subset(seqs)
    t = time.perf_counter()
    kp, vp = pa.kv_append(kp, vp, sub.k_new, sub.v_new, sub.block_tables, sub.context_lens,
                          sub.block_size, inplace=True)
    pa.decode_attention(sub.q, kp, vp, sub.block_tables, sub.context_lens,
                        block_size=sub.block_size, softmax_scale=sub.softmax_scale,
                        q_dtype=sub.q_dtype, kv_dtype=sub.kv_dtype, k_scales=sub.k_scales,
                        v_scales=sub.v_scales)
    return time.perf_counter() - t


def _cpu_steps(inp, budget_s, pa, traffic):
    t_start = time.time()
    tr = traffic.attention_call_traffic(inp.context_lens, num_q_heads=inp.num_q_heads,
                                        num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                                        q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    ap = traffic.append_traffic(inp.num_seqs, num_kv_heads=inp.num_kv_heads,
                                head_dim=inp.head_dim, kv_dtype=inp.kv_dtype)
    step_bytes = tr["total_bytes"] + ap["bytes"]
    # the append writes into copies of the pools (made before the clock starts);
    # appending the same rows again leaves them unchanged
    kp, vp = inp.k_pool.copy(), inp.v_pool.copy()
    first = _one_step(inp, pa, kp, vp)                       # untimed: first touch, set-up
    if first <= budget_s:
        times = []
        while len(times) < 3 or sum(times) < budget_s:
            times.append(_one_step(inp, pa, kp, vp))
            if len(times) >= 3 and sum(times) + times[-1] > 2 * budget_s:
                break
        best, med = min(times), float(np.median(times))
        return {"value": round(step_bytes / best / 1e9, 4), "unit": "GB/s",
                "best_s_per_step": round(best, 4), "median_s_per_step": round(med, 4),
                "tokens_per_s": round(inp.num_seqs / best, 3),
                "sample": f"{len(times)} whole steps of the {inp.num_seqs}-sequence batch "
                          f"({tr['tokens']} attended tokens each), append + attention, "
                          f"float64 NumPy; best {best:.3f} s, median {med:.3f} s",
                "wall_s": round(time.time() - t_start, 1)}
    # one step exceeds the budget: sequences in order until the budget is spent
    done, elapsed = [], 0.0
    for k in range(1 << 30):
        b = k % inp.num_seqs
        elapsed += _one_step(inp, pa, kp, vp, seqs=[b])
        done.append(b)
        if elapsed > budget_s:
            break
    trs = traffic.attention_call_traffic(inp.context_lens[done], num_q_heads=inp.num_q_heads,
                                         num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                                         q_dtype=inp.q_dtype, kv_dtype=inp.kv_dtype)
    aps = traffic.append_traffic(len(done), num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                                 kv_dtype=inp.kv_dtype)
    per_step = elapsed * inp.num_seqs / len(done) if done else float("nan")
    return {"value": round((trs["total_bytes"] + aps["bytes"]) / elapsed / 1e9, 4), "unit": "GB/s",
            "best_s_per_step": None, "median_s_per_step": round(per_step, 3),
            "tokens_per_s": round(len(done) / elapsed, 3),
            "sample": f"one step takes {first:.1f} s, over the budget: {len(done)} sequences in "
                      f"order from the {inp.num_seqs}-sequence batch ({trs['tokens']} attended "
                      f"tokens), append + attention, float64 NumPy, {elapsed:.1f} s "
                      f"(median_s_per_step scaled to the whole batch)",
            "wall_s": round(time.time() - t_start, 1)}


if __name__ == "__main__":
    main()
