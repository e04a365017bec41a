#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Default workload: 70B-shaped decode, bf16, B=16, n_h=64, n_kv=8, d_h=128,
every context 8192 tokens, block 16, 80 layers, each layer its own pool of
8192 randomly permuted physical blocks (40 GiB of K+V in HBM).  One step is
the whole decode step of the path over the 80 layers: for each layer the new
token's K/V is written at position 8191 of every sequence (overwritten each
step) and the attention runs over the layer's cache, both in one
paged_decode_attention_append call (--separate-calls: reshape_and_cache,
then paged_decode_attention).  Inputs are seeded N(0,1) synthetic data
resident in HBM before timing starts.

Prints one JSON line:  KV GB/s (value), % of the 8 TB/s HBM peak, tokens/s,
token*heads/s, a roofline record of the dominant kernel (timed with HIP
events on the launch stream) and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn KV GB/s + % of MI355X HBM peak; tokens/s at 70B-shaped B=16 S=8K"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=80, help="layers of the 70B-shaped model (80)")
    ap.add_argument("--split-tokens", type=int, default=0, help="0 = library's automatic split")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--separate-calls", action="store_true",
                    help="step = reshape_and_cache + paged_decode_attention per layer (not the one-call append)")
    ap.add_argument("--kernel-reps", type=int, default=3,
                    help="passes over the layers when timing the attention kernel alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU budget of the oracle baseline sample")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the secondary workloads (8B-shaped layer, INT8 cache, MLA)")
    ap.add_argument("--only", choices=sorted(LEGS), default=None,
                    help="run one secondary workload alone and print its record (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of a known size: 1 GiB read, 1 GiB written per copy."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by sequence or by KV head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    cpu_pool = None
    if not args.no_cpu_baseline and not args.only:
        cpu_pool, cpu_cores = start_cpu_workers()

    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, structure, device_normal_
    from synth.workloads import decode_positions

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        print(json.dumps({"leg": args.only, **LEGS[args.only](dev)}), flush=True)
        return
    cfg = CONFIGS["llama70b"]
    L = args.layers
    B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d_k
    bs = cfg.block_size

    print(f"[bench] building {L} layers of {cfg.desc}", file=sys.stderr, flush=True)
    layers = []
    seq_ids, positions = decode_positions(np.full(B, 8192, dtype=np.int32))
    for l in range(L):
        s = structure(cfg, layer=l)
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16, device=dev)
        device_normal_(pool.k, cfg.seed * 1000 + 4 * l)
        device_normal_(pool.v, cfg.seed * 1000 + 4 * l + 1)
        q = device_normal_(torch.empty((B, n_h, d), dtype=torch.bfloat16, device=dev), cfg.seed * 1000 + 4 * l + 2)
        kv_new = device_normal_(torch.empty((2, B, n_kv, d), dtype=torch.bfloat16, device=dev),
                                cfg.seed * 1000 + 4 * l + 3)
        bt = torch.from_numpy(s.block_table).to(dev)
        ctx = torch.from_numpy(s.context_lens).to(dev)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq_ids).to(dev),
                                      torch.from_numpy(positions).to(dev), bs)
        out = torch.empty((B, n_h, d), dtype=torch.bfloat16, device=dev)
        layers.append(dict(pool=pool, q=q, k_new=kv_new[0], v_new=kv_new[1], bt=bt, ctx=ctx,
                           slots=slots, out=out, s=s))
    ws_bytes = 0
    calls_rc, calls_dec, calls_app = [], [], []
    workspace = None
    for ly in layers:
        desc = pk.make_desc(B=B, n_h=n_h, n_kv=n_kv, d_k=d, d_v=d, block_size=bs,
                            max_blocks_per_seq=ly["bt"].shape[1], max_context_len=8192,
                            q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, split_tokens=args.split_tokens)
        ws_bytes = pk.decode_workspace_size(desc)
        if workspace is None and ws_bytes:
            workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        calls_rc.append(pk.prepare_reshape_and_cache(ly["pool"], ly["k_new"], ly["v_new"], ly["slots"]))
        calls_app.append(pk.prepare_decode_append(ly["pool"], ly["q"], ly["k_new"], ly["v_new"], ly["bt"],
                                                  ly["ctx"], cfg.scale, ly["out"], max_context_len=8192,
                                                  split_tokens=args.split_tokens, workspace=workspace))
        calls_dec.append(pk.prepare_decode(ly["q"], ly["pool"].k, ly["pool"].v, ly["bt"], ly["ctx"],
                                           cfg.scale, ly["out"], max_context_len=8192,
                                           split_tokens=args.split_tokens, workspace=workspace))
    split = pk.decode_split_tokens(pk.make_desc(
        B=B, n_h=n_h, n_kv=n_kv, d_k=d, d_v=d, block_size=bs, max_blocks_per_seq=512,
        max_context_len=8192, q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, split_tokens=args.split_tokens))
    torch.cuda.synchronize()

    def step():
        if args.separate_calls:
            for rc, dec in zip(calls_rc, calls_dec):
                rc()
                dec()
        else:
            for app in calls_app:
                app()
    calls_attn = calls_dec if args.separate_calls else calls_app

    stream = torch.cuda.current_stream(dev)
    run = step
    if args.graph:
        g = torch.cuda.CUDAGraph()
        step()                                   # warm before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        run = g.replay

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f})",
          file=sys.stderr, flush=True)

    # ---- dominant kernel alone: attention launches over all layers, HIP events
    # on the launch stream; average duration per launch
    reps = args.kernel_reps
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(reps):
        for c in calls_attn:
            c()
    k1.record(stream)
    torch.cuda.synchronize()
    us_launch = 1e3 * k0.elapsed_time(k1) / (reps * L)

    kv_bytes_layer = B * 8192 * n_kv * d * 2 * 2            # K + V, bf16
    kv_bytes_step = kv_bytes_layer * L
    gbs = kv_bytes_step / (ms_step * 1e-3) / 1e9
    tokens_per_s = B / (ms_step * 1e-3)
    tok_heads = B * 8192 * n_h * L / (ms_step * 1e-3)
    achieved = kv_bytes_layer / (us_launch * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "70B-shaped paged decode attention, 80 layers",
                   "B": B, "n_h": n_h, "n_kv": n_kv, "d_h": d, "context": 8192, "block_size": bs,
                   "layers": L, "kv_bytes_per_step": kv_bytes_step, "split_tokens": split,
                   "graph": bool(args.graph),
                   "step": ("reshape_and_cache + paged_decode_attention" if args.separate_calls
                            else "paged_decode_attention_append"),
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "token_heads_per_s": float(f"{tok_heads:.4g}"),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": ("paged_decode_attention" if args.separate_calls else
                                "paged_decode_attention_append (the ring kernel writes the new rows)") +
                               ": decode_gqa_ring_kernel<128,8,4,2,MFMA,2 KV heads> + decode_reduce_kernel",
                     "avg_launch_us": round(us_launch, 2),
                     "bytes_per_launch": kv_bytes_layer},
    }

    if not args.headline_only:
        # The memory freed here stays in torch's cache for the later legs:
        # handed back to the driver, tens of GiB are cleared in the background
        # for up to a minute, and the device reads ~5-10 % slower meanwhile.
        del layers, calls_rc, calls_dec, calls_app, calls_attn
        result["secondary"] = []
        for name in ("llama8b", "int8", "mla", "window", "int4", "prefill", "blocks"):
            print(f"[bench] secondary: {name}", file=sys.stderr, flush=True)
            result["secondary"].append(LEGS[name](dev))
    ceiling = read_ceiling(dev)
    result["read_ceiling"] = ceiling
    result["pct_of_read_ceiling"] = round(100 * gbs / ceiling["gbs"], 2)
    result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["gbs"], 4)
    mfma = mfma_ceiling(dev)
    result["mfma_ceiling"] = mfma
    for leg in result.get("secondary", []):
        if "mfma_tflops" in leg:
            leg["pct_of_mfma_ceiling"] = round(100 * leg["mfma_tflops"] / mfma["tflops"], 2)
        if "tflops" in leg:
            leg["pct_of_mfma_ceiling"] = round(100 * leg["tflops"] / mfma["tflops"], 2)
    if cpu_pool is not None:
        try:
            result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, cpu_pool, cpu_cores)
            result["cpu_baseline"]["gpu_over_oracle"] = round(gbs / result["cpu_baseline"]["value"], 1)
        finally:
            cpu_pool.terminate()
            cpu_pool.join()
    print(json.dumps(result), flush=True)


def _time_calls(calls, cycles, warm=3, warm_s=0.1):
    """Average device time of one call, cycling through independent
    instances (so that repeated calls do not find their data in the
    256 MB last-level cache); HIP events on the launch stream.  The calls
    run for at least warm_s seconds first: after the idle set-up of a leg
    the device needs tens of milliseconds of load to reach its steady
    clock (the INT8 leg's first 4 ms ran ~10 % slower than later ones)."""
    import torch
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    n = 0
    while n < warm or time.perf_counter() - t0 < warm_s:
        for c in calls:
            c()
        torch.cuda.synchronize()
        n += 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(cycles):
        for c in calls:
            c()
    e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / (cycles * len(calls))


def bench_llama8b(dev, instances=16, cycles=20, shared_prefix_tokens=2048):
    """8B-shaped layer (B=32, n_h=32, n_kv=8, d=128, contexts U[512, 4096],
    2K system prompt shared by all sequences) with its block tables built by
    the library's block allocator from the prompts' token ids (the shared
    prompt's full blocks are found by prefix caching and shared), 16
    instances of identical structure and different contents cycled.  The
    calls pass the shared prefix's length as a hint (the prefix rows are
    then read once for all sequences); the same calls without it are timed
    too."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, device_normal_
    from synth.workloads import shared_prefix_prompts
    cfg = CONFIGS["llama8b"]
    prompts, num_blocks, order = shared_prefix_prompts(cfg, shared_prefix_tokens)
    table, ctx_np, cached = pk.BlockAllocator(num_blocks, cfg.block_size, order=order).allocate_batch(prompts)
    bt = torch.from_numpy(table).to(dev)
    ctx = torch.from_numpy(ctx_np).to(dev)
    max_ctx = int(ctx_np.max())
    total = int(ctx_np.sum())
    calls, calls_plain = [], []
    keep = []
    for i in range(instances):
        pool = pk.kv_pool_create(num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.bfloat16, device=dev)
        device_normal_(pool.storage.view(torch.bfloat16), cfg.seed * 100 + i)
        q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=torch.bfloat16, device=dev),
                           cfg.seed * 100 + 50 + i)
        out = torch.empty((cfg.B, cfg.n_h, cfg.d_v), dtype=torch.bfloat16, device=dev)
        calls.append(pk.prepare_decode(q, pool.k, pool.v, bt, ctx, cfg.scale, out, max_context_len=max_ctx,
                                       total_context_len=total, shared_prefix_tokens=shared_prefix_tokens))
        calls_plain.append(pk.prepare_decode(q, pool.k, pool.v, bt, ctx, cfg.scale, out, max_context_len=max_ctx,
                                             total_context_len=total))
        keep.append((pool, q, out))
    us = _time_calls(calls, cycles)
    us_plain = _time_calls(calls_plain, cycles)
    row = cfg.n_kv * cfg.d_k * 2 * 2                            # K + V bytes per token
    logical = total * row
    pos = np.concatenate([np.arange(c) for c in ctx_np])
    seq = np.repeat(np.arange(cfg.B), ctx_np)
    distinct_rows = np.unique(table[seq, pos // cfg.block_size].astype(np.int64) * cfg.block_size
                              + pos % cfg.block_size).size
    unique = int(distinct_rows) * row
    return {"workload": cfg.desc + ", tables from the block allocator", "instances": instances,
            "shared_prefix_hint": shared_prefix_tokens, "prefix_tokens_cached": int(sum(cached)),
            "us_per_call": round(us, 2), "us_per_call_without_hint": round(us_plain, 2),
            "kv_gbs_logical": round(logical / (us * 1e-6) / 1e9, 1),
            "kv_gbs_unique": round(unique / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak_logical": round(100 * logical / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "pct_hbm_peak_unique": round(100 * unique / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "token_heads_per_s": float(f"{total * cfg.n_h / (us * 1e-6):.4g}"),
            "logical_kv_bytes": logical, "unique_kv_bytes": unique,
            "note": "logical bytes count every sequence's view of the shared prefix; unique bytes count each "
                    "distinct cached row once; with the hint the prefix rows are read once for all sequences, "
                    "without it each sequence reads them (after the first mostly from cache)"}


def bench_int8(dev, instances=4, cycles=10):
    """INT8 cache, 70B-shaped heads (B=32, n_h=64, n_kv=8, d=128), contexts
    log-uniform in [50, 32768]; codes and scales written by reshape_and_cache
    from bf16 N(0,1) rows; 4 instances cycled."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, structure, device_normal_
    from synth.workloads import prefill_tokens
    cfg = CONFIGS["int8_70b"]
    s = structure(cfg)
    bt = torch.from_numpy(s.block_table).to(dev)
    ctx = torch.from_numpy(s.context_lens).to(dev)
    seq, pos = prefill_tokens(s.context_lens)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev),
                                  cfg.block_size)
    calls, keep = [], []
    for i in range(instances):
        pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.int8,
                                 device=dev)
        src = device_normal_(torch.empty((2, len(seq), cfg.n_kv, cfg.d_k), dtype=torch.bfloat16,
                                         device=dev), cfg.seed * 100 + i)
        pk.reshape_and_cache(pool, src[0], src[1], slots)
        del src
        q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=torch.bfloat16, device=dev),
                           cfg.seed * 100 + 50 + i)
        out = torch.empty((cfg.B, cfg.n_h, cfg.d_v), dtype=torch.bfloat16, device=dev)
        desc = pk.make_desc(B=cfg.B, n_h=cfg.n_h, n_kv=cfg.n_kv, d_k=cfg.d_k, d_v=cfg.d_v,
                            block_size=cfg.block_size, max_blocks_per_seq=s.max_blocks_per_seq,
                            max_context_len=s.max_context_len, q_dtype=pk.KVP_BF16,
                            kv_dtype=pk.KVP_INT8, total_context_len=int(s.context_lens.sum()))
        ws = pk.alloc_workspace(desc, dev)
        calls.append(lambda q=q, pool=pool, out=out, ws=ws: pk.paged_decode_attention_int8(
            q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx, cfg.scale, out,
            max_context_len=s.max_context_len, total_context_len=int(s.context_lens.sum()),
            workspace=ws))
        keep.append((pool, q, out, ws))
    torch.cuda.synchronize()
    us = _time_calls(calls, cycles)
    total = int(s.context_lens.sum())
    kv = total * cfg.n_kv * 2 * (cfg.d_k + 4)                  # codes + one fp32 scale, K and V
    return {"workload": cfg.desc, "instances": instances, "us_per_call": round(us, 2),
            "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "token_heads_per_s": float(f"{total * cfg.n_h / (us * 1e-6):.4g}"), "kv_bytes": kv}


def bench_mla(dev, instances=4, cycles=10):
    """Absorbed MLA (B=64, n_h=128, 576-wide latent rows, values = first
    512 columns, block 64, contexts U[1024, 8192]); 4 instances cycled."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, structure, device_normal_
    cfg = CONFIGS["mla"]
    s = structure(cfg)
    bt = torch.from_numpy(s.block_table).to(dev)
    ctx = torch.from_numpy(s.context_lens).to(dev)
    total = int(s.context_lens.sum())
    calls, keep = [], []
    for i in range(instances):
        pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, 1, cfg.d_k, cfg.d_v, torch.bfloat16,
                                 latent=True, device=dev)
        device_normal_(pool.k, cfg.seed * 100 + i)
        q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=torch.bfloat16, device=dev),
                           cfg.seed * 100 + 50 + i)
        out = torch.empty((cfg.B, cfg.n_h, cfg.d_v), dtype=torch.bfloat16, device=dev)
        desc = pk.make_desc(B=cfg.B, n_h=cfg.n_h, n_kv=1, d_k=cfg.d_k, d_v=cfg.d_v,
                            block_size=cfg.block_size, max_blocks_per_seq=s.max_blocks_per_seq,
                            max_context_len=s.max_context_len, q_dtype=pk.KVP_BF16,
                            kv_dtype=pk.KVP_BF16, total_context_len=total)
        ws = pk.alloc_workspace(desc, dev)
        calls.append(lambda q=q, pool=pool, out=out, ws=ws: pk.paged_decode_attention_mla(
            q, pool.k, bt, ctx, cfg.scale, cfg.d_v, out, max_context_len=s.max_context_len,
            total_context_len=total, workspace=ws))
        keep.append((pool, q, out, ws))
    torch.cuda.synchronize()
    us = _time_calls(calls, cycles)
    kv = total * cfg.d_k * 2
    flops = total * cfg.n_h * 2 * (cfg.d_k + cfg.d_v)
    return {"workload": cfg.desc, "instances": instances, "us_per_call": round(us, 2),
            "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "pct_mfma_bf16_peak": round(100 * flops / (us * 1e-6) / 2.5e15, 2),
            "token_heads_per_s": float(f"{total * cfg.n_h / (us * 1e-6):.4g}"), "kv_bytes": kv,
            "flops": flops}


def bench_window(dev, instances=4, cycles=10, window=4096):
    """Sliding-window decode on the 70B-shaped layer (B=16, n_h=64, n_kv=8,
    d=128, every context 8192): each sequence attends to its last 4096
    positions; 4 pools of identical structure cycled."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, structure, device_normal_
    cfg = CONFIGS["llama70b"]
    s = structure(cfg, layer=0)
    bt = torch.from_numpy(s.block_table).to(dev)
    ctx = torch.from_numpy(s.context_lens).to(dev)
    calls, keep = [], []
    for i in range(instances):
        pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.bfloat16,
                                 device=dev)
        device_normal_(pool.storage.view(torch.bfloat16), cfg.seed * 100 + 70 + i)
        q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=torch.bfloat16, device=dev),
                           cfg.seed * 100 + 80 + i)
        out = torch.empty((cfg.B, cfg.n_h, cfg.d_v), dtype=torch.bfloat16, device=dev)
        desc = pk.make_desc(B=cfg.B, n_h=cfg.n_h, n_kv=cfg.n_kv, d_k=cfg.d_k, d_v=cfg.d_v,
                            block_size=cfg.block_size, max_blocks_per_seq=s.max_blocks_per_seq,
                            max_context_len=8192, q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, window=window)
        ws = pk.alloc_workspace(desc, dev)
        calls.append(lambda q=q, pool=pool, out=out, ws=ws: pk.paged_decode_attention(
            q, pool.k, pool.v, bt, ctx, cfg.scale, out, max_context_len=8192, window=window, workspace=ws))
        keep.append((pool, q, out, ws))
    torch.cuda.synchronize()
    us = _time_calls(calls, cycles)
    tokens = int(np.minimum(s.context_lens, window).sum())
    kv = tokens * cfg.n_kv * cfg.d_k * 2 * 2
    return {"workload": f"bf16 B=16 n_h=64 n_kv=8 d=128 bs=16 S=8192, window {window}",
            "instances": instances, "us_per_call": round(us, 2),
            "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "token_heads_per_s": float(f"{tokens * cfg.n_h / (us * 1e-6):.4g}"), "kv_bytes": kv}


def bench_int4(dev, instances=4, cycles=10, n_sink=4):
    """INT4 cache with a 4-token unquantized sink, on the INT8 workload's
    shape (B=32, n_h=64, n_kv=8, d=128, contexts log-uniform in [50, 32768]):
    codes and scales written by reshape_and_cache from bf16 N(0,1) rows,
    sink rows bf16 N(0,1); 4 instances cycled."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, structure, device_normal_
    from synth.workloads import prefill_tokens
    cfg = CONFIGS["int8_70b"]
    s = structure(cfg)
    bt = torch.from_numpy(s.block_table).to(dev)
    ctx = torch.from_numpy(s.context_lens).to(dev)
    seq, pos = prefill_tokens(s.context_lens)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev),
                                  cfg.block_size)
    total = int(s.context_lens.sum())
    calls, keep = [], []
    for i in range(instances):
        pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, pk.INT4, device=dev)
        src = device_normal_(torch.empty((2, len(seq), cfg.n_kv, cfg.d_k), dtype=torch.bfloat16,
                                         device=dev), cfg.seed * 100 + 20 + i)
        pk.reshape_and_cache(pool, src[0], src[1], slots)
        del src
        sink = device_normal_(torch.empty((2, cfg.B, n_sink, cfg.n_kv, cfg.d_k), dtype=torch.bfloat16,
                                          device=dev), cfg.seed * 100 + 30 + i)
        q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=torch.bfloat16, device=dev),
                           cfg.seed * 100 + 40 + i)
        out = torch.empty((cfg.B, cfg.n_h, cfg.d_v), dtype=torch.bfloat16, device=dev)
        desc = pk.make_desc(B=cfg.B, n_h=cfg.n_h, n_kv=cfg.n_kv, d_k=cfg.d_k, d_v=cfg.d_v,
                            block_size=cfg.block_size, max_blocks_per_seq=s.max_blocks_per_seq,
                            max_context_len=s.max_context_len, q_dtype=pk.KVP_BF16,
                            kv_dtype=pk.KVP_INT4, total_context_len=total)
        ws = pk.alloc_workspace(desc, dev)
        calls.append(lambda q=q, pool=pool, out=out, ws=ws, sink=sink: pk.paged_decode_attention_int4(
            q, pool.k, pool.k_scale, pool.v, pool.v_scale, sink[0], sink[1], bt, ctx, cfg.scale, out,
            max_context_len=s.max_context_len, total_context_len=total, workspace=ws))
        keep.append((pool, sink, q, out, ws))
    torch.cuda.synchronize()
    us = _time_calls(calls, cycles)
    sink_tokens = int(np.minimum(s.context_lens, n_sink).sum())
    kv = (total - sink_tokens) * cfg.n_kv * 2 * (cfg.d_k // 2 + 4) + sink_tokens * cfg.n_kv * 2 * cfg.d_k * 2
    return {"workload": f"int4 KV + {n_sink}-token bf16 sink, B=32 n_h=64 n_kv=8 d=128 bs=16 "
                        "ctx log-U[50,32768]",
            "instances": instances, "us_per_call": round(us, 2),
            "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "token_heads_per_s": float(f"{total * cfg.n_h / (us * 1e-6):.4g}"), "kv_bytes": kv,
            "note": "kv bytes: codes (d/2 per row) + one fp32 scale per row, K and V; sink rows bf16"}


def bench_prefill(dev, instances=4, cycles=10):
    """Chunked prefill on 70B-shaped heads (n_h=64, n_kv=8, d=128, block 16):
    four 512-token chunks starting at positions 0, 1024, 4096 and 7680, each
    attending causally to its cache and itself; 4 instances cycled."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import device_normal_
    from synth.workloads import custom_structure
    starts, chunks, n_h, n_kv, d, bs = [0, 1024, 4096, 7680], [512] * 4, 64, 8, 128, 16
    ends = [a + c for a, c in zip(starts, chunks)]
    st = custom_structure(ends, bs, seed=31, pad_blocks=1)
    bt = torch.from_numpy(st.block_table).to(dev)
    sp = torch.tensor(starts, dtype=torch.int32, device=dev)
    cl = torch.tensor(chunks, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(d)
    calls, keep = [], []
    for i in range(instances):
        pool = pk.kv_pool_create(st.num_blocks, bs, n_kv, d, d, torch.bfloat16, device=dev)
        device_normal_(pool.storage.view(torch.bfloat16), 900 + i)
        q = device_normal_(torch.empty((4, 512, n_h, d), dtype=torch.bfloat16, device=dev), 910 + i)
        out = torch.empty_like(q)
        calls.append(lambda q=q, pool=pool, out=out: pk.paged_prefill_attention(
            q, pool.k, pool.v, bt, sp, cl, scale, out, max_context_len=max(ends)))
        keep.append((pool, q, out))
    torch.cuda.synchronize()
    us = _time_calls(calls, cycles)
    pairs = sum(sum(a + j + 1 for j in range(c)) for a, c in zip(starts, chunks))   # (query, key) pairs
    flops = pairs * n_h * 4 * d                                 # q.k and p.v, 2 flops per MAC
    kv = sum(ends) * n_kv * d * 2 * 2
    return {"workload": "chunked prefill bf16 n_h=64 n_kv=8 d=128 bs=16, chunks of 512 at 0/1024/4096/7680",
            "instances": instances, "us_per_call": round(us, 2),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "pct_mfma_bf16_peak": round(100 * flops / (us * 1e-6) / 2.5e15, 2),
            "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1), "flops": flops, "kv_bytes": kv,
            "note": "flops count every causal (query, key) pair of the chunks, 4*d per pair and head"}


def bench_blocks(dev, n_pairs=2048, n_swap=1024, cycles=10):
    """Block moves on a 70B-shaped layer pool (8192 blocks of 64 KiB, K and
    V): copy_blocks of 2048 (src, dst) pairs with distinct random blocks, and
    swap_out_blocks / swap_in_blocks of 1024 random blocks through pinned
    host memory."""
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import device_normal_
    nb, bs, n_kv, d = 8192, 16, 8, 128
    pool = pk.kv_pool_create(nb, bs, n_kv, d, d, torch.bfloat16, device=dev)
    device_normal_(pool.storage.view(torch.bfloat16), 77)
    bb = pk.kv_pool_block_bytes(pool)
    perm = np.random.default_rng(5).permutation(nb).astype(np.int32)
    pairs = torch.from_numpy(perm[:2 * n_pairs].reshape(2, n_pairs).T.copy()).to(dev)
    stream = torch.cuda.current_stream()

    def timed(fn, reps, warm_s=0.1):
        t0 = time.perf_counter()                    # to the steady clock first (see _time_calls)
        while True:
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / reps

    us_copy = timed(lambda: pk.copy_blocks(pool, pairs), cycles)
    blocks = torch.from_numpy(perm[:n_swap].copy()).to(dev)
    staging = torch.empty(n_swap * bb, dtype=torch.uint8, device=dev)
    host = torch.empty(n_swap * bb, dtype=torch.uint8, pin_memory=True)
    us_out = timed(lambda: pk.swap_out_blocks(pool, blocks, staging, host), cycles)
    us_in = timed(lambda: pk.swap_in_blocks(pool, blocks, staging, host), cycles)
    moved = n_pairs * bb
    sw = n_swap * bb
    return {"workload": f"block moves, 70B-shaped layer pool ({nb} blocks of {bb} bytes)",
            "copy_blocks_pairs": n_pairs, "copy_blocks_us": round(us_copy, 2),
            "copy_blocks_gbs": round(2 * moved / (us_copy * 1e-6) / 1e9, 1),
            "copy_blocks_pct_hbm_peak": round(100 * 2 * moved / (us_copy * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "swap_blocks": n_swap, "swap_out_us": round(us_out, 1), "swap_in_us": round(us_in, 1),
            "swap_out_gbs": round(sw / (us_out * 1e-6) / 1e9, 2),
            "swap_in_gbs": round(sw / (us_in * 1e-6) / 1e9, 2),
            "note": "copy GB/s counts bytes read + written; swap GB/s counts the host bytes "
                    "(gather/scatter through HBM staging + one PCIe copy)"}


def read_ceiling(dev, gib=4, reps=10):
    """A plain streaming read of a 4 GiB buffer (kvp_stream_read) at a few
    grid sizes: the HBM read rate this device reaches with the simplest
    kernel, against which the decode kernels' rates are put."""
    import torch
    import pagedattention_decode_paged_amd as pk
    buf = torch.ones(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    best, sweep = 0.0, {}
    for per_cu in (2, 4, 8, 16):
        wg = per_cu * cus
        pk.stream_read(buf, sink, wg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pk.stream_read(buf, sink, wg)
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = buf.numel() / (1e-3 * e0.elapsed_time(e1) / reps) / 1e9
        sweep[str(wg)] = round(gbs, 1)
        best = max(best, gbs)
    del buf
    return {"gbs": round(best, 1), "pct_hbm_peak": round(100 * best / HBM_PEAK_GBS, 2),
            "bytes": gib << 30, "gbs_by_workgroups": sweep,
            "kernel": "stream_read_kernel: 8 x 16-byte loads in flight per lane, grid-stride"}


def mfma_ceiling(dev, iterations=4096, reps=5):
    """The bf16 matrix-core rate this device reaches with back-to-back
    independent v_mfma_f32_16x16x32_bf16 on register operands
    (kvp_mfma_peak), at 4, 8 and 16 workgroups of four wavefronts per CU."""
    import torch
    import pagedattention_decode_paged_amd as pk
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    best, sweep = 0.0, {}
    for per_cu in (4, 8, 16):
        wg = per_cu * cus
        flops = pk.mfma_peak(sink, wg, iterations)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pk.mfma_peak(sink, wg, iterations)
        e1.record(stream)
        torch.cuda.synchronize()
        tf = flops / (1e-3 * e0.elapsed_time(e1) / reps) / 1e12
        sweep[str(wg)] = round(tf, 1)
        best = max(best, tf)
    return {"tflops": round(best, 1), "pct_of_dense_bf16_peak": round(100 * best / 2500.0, 2),
            "tflops_by_workgroups": sweep,
            "kernel": "mfma_peak_kernel: 8 independent v_mfma_f32_16x16x32_bf16 chains per wavefront"}


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record, if the kernel sources it was taken on are unchanged
    (else None: the counters describe a different kernel)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gqa_ring_70b_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() == rec["sources_sha256"]:
            return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def _cpu_cores():
    """Host cores the baseline may use: this process's CPU affinity, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:                                # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:                                   # pragma: no cover
        pass
    import oracle  # noqa: F401


def _cpu_worker(task):
    """Oracle calls on (sequence, KV head) units of one layer until the
    budget is spent: each unit is decode attention of the g query heads
    that share one KV head over the sequence's whole context."""
    import oracle
    d, items, budget = task
    k = np.load(os.path.join(d, "k.npy"), mmap_mode="r")
    v = np.load(os.path.join(d, "v.npy"), mmap_mode="r")
    q = np.load(os.path.join(d, "q.npy"))
    bt = np.load(os.path.join(d, "bt.npy"))
    ctx = np.load(os.path.join(d, "ctx.npy"))
    scale = float(np.load(os.path.join(d, "scale.npy")))
    g = q.shape[1] // k.shape[2]
    done, kv_bytes = 0, 0
    t0 = time.perf_counter()
    for b, h in items:
        if time.perf_counter() - t0 >= budget:
            break
        oracle.paged_decode_attention(q[b:b + 1, h * g:(h + 1) * g], k[:, :, h:h + 1], v[:, :, h:h + 1],
                                      bt[b:b + 1], ctx[b:b + 1], scale)
        done += 1
        kv_bytes += int(ctx[b]) * (k.shape[3] + v.shape[3]) * 2
    return done, kv_bytes, time.perf_counter() - t0


def start_cpu_workers():
    """The baseline's worker processes, started before this process touches
    the GPU (they only ever run the CPU oracle)."""
    import multiprocessing as mp
    cores = _cpu_cores()
    return mp.get_context("spawn").Pool(cores, initializer=_cpu_worker_init), cores


def cpu_baseline(budget_s, pool, cores):
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workload: layer 0 of the 70B-shaped step (its K/V drawn with the bench's
    seeds on the device, then held in host memory), split into its 128
    (sequence, KV head) units, dealt round-robin to one single-threaded
    process per core and cycled until the CPU budget is spent."""
    import shutil
    import tempfile
    import torch
    import pagedattention_decode_paged_amd as pk
    from synth import CONFIGS, structure, device_normal_
    cfg = CONFIGS["llama70b"]
    s = structure(cfg, layer=0)
    kvp = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.bfloat16)
    device_normal_(kvp.k, cfg.seed * 1000)
    device_normal_(kvp.v, cfg.seed * 1000 + 1)
    q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=torch.bfloat16, device="cuda"),
                       cfg.seed * 1000 + 2)
    need = 2 * s.num_blocks * cfg.block_size * cfg.n_kv * cfg.d_k * 2 + (64 << 20)
    base = None                                       # the default temp dir unless /dev/shm has the room
    try:
        if os.access("/dev/shm", os.W_OK) and shutil.disk_usage("/dev/shm").free > 2 * need:
            base = "/dev/shm"
    except OSError:                                   # pragma: no cover
        pass
    d = tempfile.mkdtemp(prefix="pkv_cpu_baseline_", dir=base)
    try:
        t_copy = time.perf_counter()
        for name, t in (("k", kvp.k), ("v", kvp.v), ("q", q)):
            np.save(os.path.join(d, f"{name}.npy"), t.cpu().view(torch.int16).numpy().view(np.uint16))
        t_copy = time.perf_counter() - t_copy
        del kvp, q
        np.save(os.path.join(d, "bt.npy"), s.block_table)
        np.save(os.path.join(d, "ctx.npy"), s.context_lens)
        np.save(os.path.join(d, "scale.npy"), np.float64(cfg.scale))
        units = [(b, h) for b in range(cfg.B) for h in range(cfg.n_kv)]
        cap = 64 * len(units)
        tasks = [(d, [units[i % len(units)] for i in range(w, cap, cores)], budget_s) for w in range(cores)]
        print(f"[bench] cpu baseline: {cores} processes, {budget_s:.0f} s", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        # bounded wait: a pool whose workers cannot start never finishes a map
        res = pool.map_async(_cpu_worker, tasks, chunksize=1).get(timeout=budget_s + 120)
        wall = time.perf_counter() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)
    done = sum(r[0] for r in res)
    kv_bytes = sum(r[1] for r in res)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:                                     # pragma: no cover
        pass
    tokens_equiv = kv_bytes / (cfg.n_kv * cfg.d_k * 2 * 2 * 8192 * 80)   # whole 80-layer decode steps of one sequence
    return {"value": round(kv_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"layer 0 of the 70B-shaped step: {done} (sequence, KV head) units of 8192 tokens x "
                      f"8 query heads ({len(units)} distinct, cycled) on {cores} single-threaded processes, "
                      f"{kv_bytes} KV bytes in {wall:.2f} s",
            "cpu_model": model, "host_copy_s": round(t_copy, 2),
            "tokens_per_s_equiv": round(tokens_equiv / wall, 6)}


LEGS = {"llama8b": bench_llama8b, "int8": bench_int8, "mla": bench_mla, "window": bench_window,
        "int4": bench_int4, "prefill": bench_prefill, "blocks": bench_blocks, "ceiling": read_ceiling,
        "mfma": mfma_ceiling}


if __name__ == "__main__":
    main()
