#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

A step is one decode step of one attention layer over a batch of sequences:
the C++ allocator appends one token per sequence (copy-on-write where blocks are
shared), the step's slot mapping / block tables go to the device, then
block_copy -> kv_append -> paged_attention_decode (+ partition merge) run on one
stream.  Inputs (cache contents, per-step q and new K/V) are resident in HBM
before the timed region starts.

Default workload: bf16 MHA decode, 64 sequences, context lengths U[128, 2048],
32 query / 32 KV heads, head_dim 128, 16-token blocks in a shuffled pool.
The first timed step attends over exactly those lengths; each later step one
token more.  --block-size 32 (64, ...) lays the same sequences out in a pool of
larger blocks, --head-dim 256 (or 64) gives them another head size (MHA, GQA and
long-context workloads).

Prints one JSON line: value = algorithmic HBM bytes of the whole step / step
time (GB/s), plus seq-tokens/s per layer, the main attention kernel's roofline
(bytes / its HIP-event-timed duration against 8 TB/s) and the fp64 oracle timed
on the host as a CPU baseline.
"""
import argparse
import gc
import json
import math
import os
import sys
import time

METRIC = "decode attention achieved HBM GB/s (% of peak) + seq-tokens/sec per layer"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FOREIGN = -1


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=55)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2", choices=["c2", "c3", "c4", "c5", "prefill"],
                    help="decode workloads c2..c5; 'prefill' times chunked prefill attention on c2's sequences")
    ap.add_argument("--chunk", type=int, default=512, help="prefill: chunk rows per sequence (at most its length)")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="split-context partition in tokens (0 = the workload's own)")
    ap.add_argument("--block-size", type=int, default=16,
                    help="decode c2/c3/c5: tokens per cache block (16; 32, 64, ... stream as 16-token tiles)")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="decode c2/c3/c5: head_dim other than the workload's 128 (64 or 256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size before the steps (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the paged decode path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.workload == "prefill":
        run_prefill(args)
        return
    BS = args.block_size
    if (BS != 16 or args.head_dim) and args.workload == "c4":
        sys.exit("bench.py: the sampling workload runs on 16-token blocks and head_dim 128 only")

    import numpy as np
    import torch

    import synth
    from paged_kv_cache_358_amd.engine import PagedDecodeLayer

    torch.cuda.init()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W, K = args.warmup, args.steps
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}

    def up(a, dtype):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(a)
        return t.to(dev)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------------ workload
    if args.workload == "c4":
        cfg = synth.C4
        part = args.partition_size or cfg.partition_size
        if W + K > cfg.steps:
            sys.exit(f"c4 runs at most {cfg.steps} decode steps")
        S, hq, hkv, D, dtype = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
        max_blocks = -(-(cfg.prefix_len + cfg.steps) // 16)
        layer = PagedDecodeLayer(cfg.pool_blocks(), hkv, D, hq, tdt[dtype], S, max_blocks,
                                 free_order=cfg.free_order(), partition_size=part, device=dev)
        for i in range(cfg.num_prompts):
            root = i * cfg.samples
            k, v = cfg.prefix_kv(i)
            layer.add(root)
            layer.prefill(root, up(k, dtype), up(v, dtype))
            for c in range(1, cfg.samples):
                layer.fork(root, root + c)
        step_inputs = []
        for st in range(1, W + K + 1):
            kn, vn = cfg.step_kv(st)
            step_inputs.append((up(cfg.step_q(st), dtype), up(kn, dtype), up(vn, dtype)))
        scale = cfg.softmax_scale
        kvbpt = cfg.kv_bytes_per_token()
        workload = {"workload": cfg.name, "prompts": cfg.num_prompts, "samples": cfg.samples,
                    "prefix_len": cfg.prefix_len, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D,
                    "block_size": 16, "partition_size": part,
                    "timed_steps": f"{W + 1}..{W + K}"}
        lens0 = None
    else:
        cfg = synth.CONFIGS[{"c2": "c2_mha_bf16", "c3": "c3_gqa_bf16", "c5": "c5_long_bf16"}[args.workload]]
        suffix = (f"_d{args.head_dim}" if args.head_dim else "") + (f"_b{BS}" if BS != 16 else "")
        if suffix:  # the same context lengths with another head size, or in a pool of larger blocks
            cfg = synth.scaled(cfg, name_suffix=suffix, block_size=BS, head_dim=args.head_dim or cfg.head_dim)
        part = args.partition_size or cfg.partition_size
        if W + K > cfg.pool_slack_tokens:
            sys.exit(f"{cfg.name}: warmup + steps must be <= {cfg.pool_slack_tokens}")
        S, hq, hkv, D, dtype = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
        lens0 = synth.context_lens(cfg)                # context at the first timed step
        plan = synth.pool_plan(cfg, lens0)
        prefill = np.maximum(lens0 - W - 1, 0)
        max_blocks = int(synth.blocks_for(lens0.max() + K, BS))
        layer = PagedDecodeLayer(plan.num_blocks, hkv, D, hq, tdt[dtype], S, max_blocks,
                                 free_order=plan.free_order, partition_size=part, device=dev, block_size=BS)
        if plan.preoccupy_blocks:
            layer.alloc.add(FOREIGN)
            layer.alloc.append(FOREIGN, plan.preoccupy_blocks * BS)
        for s in range(S):
            layer.add(s)
            if prefill[s]:
                k, v = synth.seq_kv(cfg, s, int(prefill[s]))
                layer.prefill(s, up(k, dtype), up(v, dtype))
        step_inputs = []
        for st in range(W + K):
            kn, vn = synth.new_tokens_kv(cfg.cfg_id, 1000 + st, S, hkv, D, dtype)
            step_inputs.append((up(synth.queries(cfg, step=1000 + st), dtype), up(kn, dtype), up(vn, dtype)))
        scale = cfg.softmax_scale
        kvbpt = cfg.kv_bytes_per_token()
        workload = {"workload": cfg.name, "num_seqs": S, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D,
                    "block_size": BS, "partition_size": part, "context_lens": cfg.lens,
                    "mean_context": float(lens0.mean()), "pool_blocks": plan.num_blocks}
    torch.cuda.synchronize()
    print(f"[bench] {workload['workload']}: workload resident on the GPU", file=sys.stderr, flush=True)
    seqs = np.arange(S, dtype=np.int64)
    eb = synth.ELEM_BYTES[dtype]
    out = torch.empty(S, hq, D, dtype=tdt[dtype], device=dev)

    for i in range(W):
        q, kn, vn = step_inputs[i]
        layer.decode_step(seqs, q, kn, vn, out, scale)
    torch.cuda.synchronize()

    events = []
    for _ in range(K):
        pair = tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
        for e in pair:
            e.record(layer.stream)  # torch creates events lazily; materialise before timing
        events.append(pair)
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ timed region
    # A collection of the interpreter's older generations can pause the host for tens of
    # milliseconds; collect now and keep everything allocated so far out of later passes.
    gc.collect()
    gc.freeze()
    shared = args.workload == "c4"  # forked samples share blocks: count each physical block once
    step_lens, step_pairs = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_groups, step_group_rows = [], []
    first_tables = None
    for i in range(K):
        q, kn, vn = step_inputs[W + i]
        step_pairs.append(layer.decode_step(seqs, q, kn, vn, out, scale, timing=events[i]))
        step_lens.append(layer.last_lens)
        step_groups.append(layer.last_groups)
        step_group_rows.append(layer.last_group_rows)
        if shared and i == 0:
            first_tables = layer.last_tables.copy()
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    print(f"[bench] {K} timed steps: {elapsed / K * 1e3:.3f} ms/step (host enqueue done after "
          f"{(t_enq - t0) / K * 1e3:.3f} ms/step)", file=sys.stderr, flush=True)

    # The events ride on the attention call's launch: start to end of the split kernel, which
    # merges split contexts itself (over groups of forked samples when they share blocks).
    main_ms = [a.elapsed_time(b) for a, b in events]
    block_bytes = hkv * D * BS * eb

    # Algorithmic bytes of one attention launch: K/V of every cached token (2 * H_kv * D * elem per
    # token), q and out, the block-table entries and context lengths read.  With shared blocks the
    # HBM-bound quantity counts each physical block once, at the most tokens any sequence uses of it.
    def attn_bytes(lens, tables=None):
        lens = np.asarray(lens, dtype=np.int64)
        fixed = S * hq * D * eb * 2 + int(synth.blocks_for(lens, BS).sum()) * 4 + S * 4
        if tables is None:
            return int(lens.sum() * kvbpt) + fixed
        used = {}
        for s_, n in enumerate(lens.tolist()):
            for b in range(-(-n // BS)):
                phys = int(tables[s_, b])
                used[phys] = max(used.get(phys, 0), min(BS, n - BS * b))
        return int(sum(used.values()) * kvbpt) + fixed

    # With groups, a group's k shared (full) blocks are one set of physical blocks and every other block
    # is held by one sequence: each member beyond the first re-reads B k tokens.  The first timed step
    # checks that against the count over its physical blocks.
    def group_bytes(lens, rows):
        if rows is None:
            return attn_bytes(lens)
        dup = int(sum((m - 1) * BS * k for _, m, k in rows.tolist()))
        return attn_bytes(lens) - dup * kvbpt

    logical = [attn_bytes(l) for l in step_lens]
    if shared:
        attn = [group_bytes(l, r) for l, r in zip(step_lens, step_group_rows)]
        exact = attn_bytes(step_lens[0], first_tables)
        if attn[0] != exact:
            sys.exit(f"bench: unique bytes from the groups ({attn[0]}) differ from the block count ({exact})")
    else:
        attn = logical
    append_b = S * hkv * D * eb * 2 * 2 + S * 4
    copy_b = [p * block_bytes * 2 * 2 for p in step_pairs]
    total_bytes = sum(attn) + K * append_b + sum(copy_b)
    value = total_bytes / elapsed / 1e9
    mean_main_s = float(np.mean(main_ms)) / 1e3
    achieved = float(np.mean(attn)) / mean_main_s / 1e9
    kernel = main_kernel_name(dtype, D, hq // hkv, S, BS)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, seeded context lengths and shuffled block pool)",
        "config": workload,
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "seq_tokens_per_s_per_layer": round(S / (elapsed / K), 1),
        "context_tokens_per_s_per_layer": round(float(np.mean([np.sum(l) for l in step_lens])) / (elapsed / K), 1),
        "attention_ms": {"main_kernel": round(float(np.mean(main_ms)), 4)},
        "shared_prefix_groups": int(max(step_groups)),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(kernel, workload["workload"], workload.get("timed_steps")),
                     "kernel": kernel, "bytes_per_launch": int(np.mean(attn))},
        "copy_on_write_blocks": int(sum(step_pairs)),
    }
    if shared:
        result["logical_attention_bytes_per_launch"] = int(np.mean(logical))
        result["effective_logical_gbs"] = round(float(np.mean(logical)) / mean_main_s / 1e9, 1)

    last_tables = layer.last_tables.copy()
    result["cache_ops"] = cache_ops_probe(layer, step_inputs[-1], last_tables, block_bytes)
    if not shared:
        result["decode_probes"] = decode_probes(layer, step_inputs[-1][0], out, scale, last_tables,
                                                step_lens[-1], part, attn[-1])

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, cfg, lens0, kvbpt)
    print(json.dumps(result), flush=True)


def cache_ops_probe(layer, step_input, tables, block_bytes, reps=20, max_pairs=448):
    """Bandwidth of block_copy and kv_append on their own, after the timed steps: `reps`
    back-to-back launches between two events.  Both write only blocks on the allocator's free
    list, so no live cache content changes.  block_copy copies up to 448 live blocks (the
    copy-on-write count of the first sampling step) into free ones; kv_append writes the last
    step's new K/V (one token per sequence) into free slots."""
    import numpy as np
    import torch
    from paged_kv_cache_358_amd import block_copy, kv_append

    free = layer.alloc.free_list()
    live = np.unique(np.asarray(tables)[np.asarray(tables) >= 0])
    out = {}
    n = min(max_pairs, len(free), len(live))
    if n > 0:
        pairs = torch.tensor(np.stack([live[:n], np.asarray(free[:n])], axis=1).astype(np.int32), device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(layer.stream):
            block_copy(layer.k_cache, layer.v_cache, pairs, stream=layer.stream)  # warm
            e0.record(layer.stream)
            for _ in range(reps):
                block_copy(layer.k_cache, layer.v_cache, pairs, stream=layer.stream)
            e1.record(layer.stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps / 1e3
        moved = n * block_bytes * 2 * 2  # K and V blocks, read and written
        out["block_copy"] = {"pairs": n, "us_per_launch": round(t * 1e6, 2), "bytes_per_launch": moved,
                             "achieved_gbs": round(moved / t / 1e9, 1),
                             "frac": round(moved / t / 1e9 / PEAK_HBM_GBS, 4)}
    _, k_new, v_new = step_input
    T = k_new.shape[0]
    B = layer.block_size
    if T > 0 and len(free) * B >= T:
        blocks = np.asarray(free[:(T + B - 1) // B], dtype=np.int64)
        slots = torch.tensor((np.repeat(blocks, B)[:T] * B + np.tile(np.arange(B), len(blocks))[:T]).astype(np.int32),
                             device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(layer.stream):
            kv_append(k_new, v_new, slots, layer.k_cache, layer.v_cache, stream=layer.stream)  # warm
            e0.record(layer.stream)
            for _ in range(reps):
                kv_append(k_new, v_new, slots, layer.k_cache, layer.v_cache, stream=layer.stream)
            e1.record(layer.stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps / 1e3
        moved = k_new.numel() * k_new.element_size() * 2 * 2 + T * 4  # K and V read and written, slots
        out["kv_append"] = {"tokens": T, "us_per_launch": round(t * 1e6, 2), "bytes_per_launch": int(moved),
                            "achieved_gbs": round(moved / t / 1e9, 1),
                            "frac": round(moved / t / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def decode_probes(layer, q, out, scale, tables, lens, part, nbytes, reps=20, flush_mib=1024):
    """The attention call alone, after the timed steps, on the last step's batch: with the
    step's (shuffled) block tables and with identity tables (each sequence's blocks contiguous
    in the pool, so the table lookup gathers nothing), each warm (launches back to back) and
    cold (a 1 GiB buffer written between launches evicts L2 and the 256 MiB last-level cache).
    The identity tables point at other blocks' data: only the timing is meaningful.  Last, a
    STREAM-style copy as a reference for the achievable HBM rate: block_copy of the pool's
    first half onto its second half (this overwrites cache contents; nothing reads them after)."""
    import numpy as np
    import torch
    from paged_kv_cache_358_amd import block_copy, paged_attention_decode

    S = len(lens)
    lens = np.asarray(lens, dtype=np.int64)
    nb = -(-lens // layer.block_size)
    num_blocks = layer.k_cache.shape[0]
    if int(nb.sum()) > num_blocks:
        return None
    ident = np.full_like(np.asarray(tables), -1)
    off = np.concatenate([[0], np.cumsum(nb)])
    for s_ in range(S):
        ident[s_, :nb[s_]] = np.arange(off[s_], off[s_ + 1])
    dev_lens = torch.from_numpy(lens.astype(np.int32)).cuda()
    flush = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    res = {}
    with torch.cuda.stream(layer.stream):
        for name, tb in (("shuffled", tables), ("identity", ident)):
            dev_t = torch.from_numpy(np.ascontiguousarray(tb, dtype=np.int32)).cuda()
            for mode in ("warm", "cold"):
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
                for a, b in ev:
                    a.record(layer.stream)
                    b.record(layer.stream)
                for i in range(reps + 1):
                    if mode == "cold":
                        flush.fill_(i & 0xFF)
                    e = ev[i - 1] if i else (None, None)          # launch 0 is a warm-up
                    paged_attention_decode(q, layer.k_cache, layer.v_cache, dev_t, dev_lens, scale, out,
                                           max_context_len=int(lens.max()), partition_size=part,
                                           workspace=layer.workspace, stream=layer.stream,
                                           start_event=e[0], stop_event=e[1])
                torch.cuda.synchronize()
                ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
                res[f"{name}_{mode}_ms"] = round(ms, 4)
                res[f"{name}_{mode}_gbs"] = round(nbytes / (ms / 1e3) / 1e9, 1)
    res["table_indirection_cost_cold"] = round(res["shuffled_cold_ms"] / res["identity_cold_ms"] - 1.0, 4)
    del flush
    half = num_blocks // 2
    pairs = torch.from_numpy(np.stack([np.arange(half), np.arange(half) + half], axis=1).astype(np.int32)).cuda()
    moved = 2 * half * layer.k_cache[0].numel() * layer.k_cache.element_size() * 2   # K and V, read and written
    with torch.cuda.stream(layer.stream):
        block_copy(layer.k_cache, layer.v_cache, pairs, stream=layer.stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(layer.stream)
        for _ in range(10):
            block_copy(layer.k_cache, layer.v_cache, pairs, stream=layer.stream)
        e1.record(layer.stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 10 / 1e3
    res["copy_probe_bytes"] = int(moved)
    res["copy_probe_gbs"] = round(moved / t / 1e9, 1)
    res["shuffled_cold_frac_of_copy_probe"] = round(res["shuffled_cold_gbs"] / res["copy_probe_gbs"], 4)
    return res


def run_prefill(args):
    """Chunked prefill attention on the MHA decode workload's sequences: the last
    min(chunk, n) tokens of each sequence are the chunk (their K/V already in the cache).
    Algorithmic work per query head and chunk row at position p: 2 D (p + 1) multiply-adds
    (scores and weighted sum), 4 D (p + 1) flops."""
    import numpy as np
    import torch

    import synth
    import paged_kv_cache_358_amd as pa

    W, K = args.warmup, args.steps
    dev = torch.device("cuda:0")
    cfg = synth.C2
    lens = synth.context_lens(cfg).astype(np.int64)
    chunks = np.minimum(lens, args.chunk)
    S, hq, hkv, D = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    plan = synth.pool_plan(cfg, lens)
    torch.manual_seed(cfg.cfg_id)
    k_cache, v_cache = pa.alloc_kv_cache(plan.num_blocks, hkv, D, torch.bfloat16, dev)
    k_cache.normal_()
    v_cache.normal_()
    alloc = pa.BlockAllocator(plan.num_blocks, 16, plan.free_order)
    for s_ in range(S):
        alloc.add(s_)
        alloc.append(s_, int(lens[s_]))
    max_blocks = int(synth.blocks_for(lens.max()))
    tables, lens_np = alloc.build_batch(list(range(S)), max_blocks)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    T = int(qs[-1])
    q = torch.randn(T, hq, D, device=dev).to(torch.bfloat16)
    out = torch.empty(T, hq, D, device=dev, dtype=torch.float32)
    bt, cl, qst = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (tables, lens_np, qs))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record()
        b.record()

    def launch(events=None):
        pa.paged_attention_prefill(q, k_cache, v_cache, bt, cl, qst, cfg.softmax_scale, out,
                                   max_query_len=int(chunks.max()),
                                   start_event=None if events is None else events[0],
                                   stop_event=None if events is None else events[1])

    for _ in range(W):
        launch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        launch(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    pos_sum = sum(int(n) * int(c) - int(c) * (int(c) - 1) // 2 for n, c in zip(lens, chunks))  # sum of p + 1
    flops = 4.0 * D * hq * pos_sum
    kv_bytes = int(lens.sum()) * cfg.kv_bytes_per_token() + 2 * T * hq * D * 2
    tflops = flops / kern_s / 1e12
    print(json.dumps({
        "metric": "prefill attention TFLOP/s (algorithmic)", "value": round(flops / (elapsed / K) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (torch-seeded N(0,1) q/K/V, seeded context lengths and shuffled block pool)",
        "config": {"workload": "c2_mha_bf16 chunked prefill", "num_seqs": S, "chunk": args.chunk,
                   "rows": T, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D, "block_size": 16},
        "kernel_ms": round(kern_s * 1e3, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_mfma_kernel", "flops_per_launch": flops},
        "kv_bytes_per_launch": kv_bytes, "kv_gbs_if_read_once": round(kv_bytes / kern_s / 1e9, 1),
    }), flush=True)


def main_kernel_name(dtype, head_dim, group, num_seqs, block_size=16):
    """The library's dominant kernel for this shape (its dispatch rule, restated)."""
    tiles = block_size in [16 << j for j in range(7)]
    if dtype == "f32" or group > 16:
        return "decode_generic_kernel"
    if head_dim == 256:
        return "decode_split_kernel" if block_size == 16 and num_seqs <= 2048 else "decode_generic_kernel"
    if head_dim not in (64, 128) or not tiles:
        return "decode_generic_kernel"
    if num_seqs <= 2048:
        return "decode_split_kernel"
    return "decode_mfma_kernel" if block_size == 16 else "decode_generic_kernel"


def kernel_code_hash(path):
    """sha256[:16] of a source file's code: comments and blank lines removed, so that edits to
    comments alone leave measurements taken on the file valid."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    lines = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
    return hashlib.sha256("\n".join(line for line in lines if line.strip()).encode()).hexdigest()[:16]


def measured_traffic(kernel, workload, steps=None):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
    profiles/hbm_traffic.txt, if they were taken on the current kernel code (and, for a record
    that names the decode steps it measured, on the steps timed here); else None."""
    root = os.path.dirname(os.path.abspath(__file__))
    src = os.path.join(root, "paged_kv_cache_358_amd", "csrc", "decode_attention.hip")
    table = os.path.join(root, "profiles", "hbm_traffic.txt")
    if not os.path.exists(table):
        return None
    sha = kernel_code_hash(src)
    for line in open(table):
        f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
        if f.get("kernel") == kernel and f.get("workload") == workload and f.get("code_sha256") == sha:
            if "steps" in f and f["steps"] != steps:
                continue
            return int(f["traffic_bytes"])
    return None


def cpu_baseline(args, cfg, lens0, kvbpt):
    """The fp64 oracle on a bounded sample of the same workload, one host thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle.attention import decode_attention_seq

    if lens0 is None:  # parallel sampling: every sample at its final context, prefix + appended tokens
        n_ctx = cfg.prefix_len + cfg.steps
        steps = [cfg.step_kv(t) for t in range(1, cfg.steps + 1)]

        def draw(s):
            pk, pv = cfg.prefix_kv(s // cfg.samples)
            return (np.concatenate([pk, np.stack([k[s] for k, _ in steps])]),
                    np.concatenate([pv, np.stack([v[s] for _, v in steps])]))
        lens = [n_ctx] * cfg.num_seqs
    else:
        draw = lambda s: synth.seq_kv(cfg, s, int(lens0[s]))
        lens = lens0.tolist()
    q = synth.queries(cfg) if lens0 is not None else cfg.step_q(cfg.steps)
    order = np.random.default_rng(0).permutation(len(lens))
    # One pass over the sequences; each is drawn once and the oracle is re-run on it until its
    # share of the time budget is used (at least once), so memory stays one sequence deep.
    share = args.cpu_seconds / len(order)
    spent, done, ctx_tokens = 0.0, 0, 0
    with threadpool_limits(limits=1):
        for i, s in enumerate(order):
            k, v = draw(int(s))
            k64, v64 = synth.decode_f64(k, cfg.dtype), synth.decode_f64(v, cfg.dtype)
            q64 = synth.decode_f64(q[s], cfg.dtype)
            mine = 0.0
            while mine < share or mine == 0.0:
                t = time.perf_counter()
                decode_attention_seq(q64, k64, v64, cfg.softmax_scale)
                mine += time.perf_counter() - t
                done += 1
                ctx_tokens += int(lens[s])
            spent += mine
            if i % 16 == 15 or i == len(order) - 1:
                print(f"[bench] cpu baseline: {i + 1}/{len(order)} sequences, {spent:.1f} s", file=sys.stderr,
                      flush=True)
    gbs = ctx_tokens * kvbpt / spent / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seq_tokens_per_s_per_layer": round(done / spent, 2),
            "sample": f"fp64 oracle, {done} sequence evaluations over all {len(lens)} sequences of the "
                      f"workload (each drawn once and evaluated until it had {share:.2f} s; all "
                      f"{cfg.num_q_heads} query heads; {ctx_tokens} context tokens in total), {spent:.1f} s "
                      f"on 1 host thread; inputs decoded to float64 beforehand"}


if __name__ == "__main__":
    main()
