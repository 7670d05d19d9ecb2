#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

A step is one decode step of one attention layer over a batch of sequences: the
C++ allocator appends one token per sequence (copy-on-write where blocks are
shared), the step's slot mapping / block tables go to the device, then
block_copy -> kv_append -> paged_attention_decode run on one stream.  Inputs
(cache contents, per-step q and new K/V) are resident in HBM before the timed
region starts.

By default every workload runs in turn, each with --warmup untimed and --steps
timed steps, and one JSON line reports them all:
  c1  tiny fp32 MHA decode, contexts {1, 15, 16, 33}, 4 heads, head_dim 64 (launch-bound: microseconds)
  c2  bf16 MHA decode, 64 sequences, contexts U[128, 2048], 32/32 heads, head_dim 128
  c3  bf16 GQA decode, 256 sequences, log-normal contexts (median 1024, clipped to [16, 8192]),
      64/8 heads, 30% of the pool held by another sequence
  c4  parallel sampling: 64 prompts x 8 samples on a shared 1000-token prefix, 32/8 heads,
      copy-on-write at the first appended token (bytes counted once per physical block)
  c5  long context: 4 sequences of 131072 tokens, 64/8 heads, 512-token partitions
The headline (top-level value, config, roofline, cpu_baseline) is c5, the
largest single-GPU workload; the others sit under "configs".  --workload picks
one of them alone (or "prefill": chunked prefill attention on c2's sequences).

value = algorithmic HBM bytes of the whole step / step time (GB/s).  roofline =
the main attention kernel's algorithmic bytes / its HIP-event-timed duration
against 8 TB/s.  cpu_baseline = the fp64 oracle on a bounded sample of the same
workload, on the host's cores.
"""
import argparse
import gc
import json
import os
import sys
import time

METRIC = "decode attention achieved HBM GB/s (% of peak) + seq-tokens/sec per layer"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FOREIGN = -1
WORKLOADS = {"c1": "c1_tiny_f32", "c2": "c2_mha_bf16", "c3": "c3_gqa_bf16", "c4": "c4_cow_sampling_bf16",
             "c5": "c5_long_bf16"}
HEADLINE = "c5"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=["all", "c1", "c2", "c3", "c4", "c5", "prefill"],
                    help="all decode workloads (default), one of them, or chunked prefill on c2's sequences")
    ap.add_argument("--dtype", default="", choices=["", "bf16", "f16", "f32"],
                    help="type of the c2/c3/c4/c5 caches (default: the workload's bf16); f32 runs the VALU kernel")
    ap.add_argument("--chunk", type=int, default=512, help="prefill: chunk rows per sequence (at most its length)")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="split-context partition in tokens (0 = the workload's own)")
    ap.add_argument("--block-size", type=int, default=16,
                    help="decode c2/c3/c4/c5 and prefill: tokens per cache block (16; 8, 32, 64, ...)")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="decode c2/c3/c4/c5 and prefill: head_dim other than the workload's 128 (64, 96 or 256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time budget of the headline CPU baseline (the other workloads get a third)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size before the steps (counter calibration)")
    return ap.parse_args()


def host_threads():
    """Host cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.workload == "prefill" and (args.head_dim not in (0, 64, 96, 128, 256) or
                                       (args.block_size != 8 and (args.block_size < 16 or
                                                                  args.block_size & (args.block_size - 1)))):
        sys.exit("prefill bench: head_dim 64, 96, 128 or 256 and blocks of 8 or 16 << j tokens (the MFMA kernel)")
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the paged decode path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    if args.dtype and "c1" in names and args.workload == "all":
        names.remove("c1")  # the tiny workload is fp32 by definition

    import torch
    from concurrent.futures import ThreadPoolExecutor

    torch.cuda.init()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "prefill":
        run_prefill(args)
        return

    blocks = {}
    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        for w in names:
            blocks[w] = run_decode(args, w, dev, pool)
            gc.collect()
            torch.cuda.empty_cache()
    head_key = HEADLINE if HEADLINE in blocks else names[0]
    head = blocks[head_key]
    result = {k: head[k] for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                                   "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config")}
    for k, v in head.items():
        if k not in result and k not in ("cpu_oracle", "metric"):
            result[k] = v
    if not args.no_cpu_baseline and "cpu_oracle" in head:
        result["cpu_baseline"] = head["cpu_oracle"]
    if len(blocks) > 1:
        result["configs"] = {blocks[w]["config"]["workload"]: config_summary(blocks[w]) for w in names}
    print(json.dumps(result), flush=True)


def config_summary(b):
    """The per-workload record inside the headline line."""
    keys = ("ms_per_step", "value", "unit", "pct_of_peak_hbm", "seq_tokens_per_s_per_layer",
            "context_tokens_per_s_per_layer", "dtype", "steps", "warmup", "kernel", "kernel_us", "roofline",
            "copy_on_write_blocks", "shared_prefix_groups", "logical_attention_bytes_per_launch",
            "effective_logical_gbs", "cache_ops", "decode_probes", "cpu_oracle", "cpu_oracle_1_thread", "note")
    out = {"config": b["config"]}
    out.update({k: b[k] for k in keys if k in b})
    return out


# ---------------------------------------------------------------------------------------- workloads
def _up(a, dtype, dev):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(a)
    return t.to(dev)


def _draw_heads(pool, fn, heads):
    """K and V [n, H_kv, D] of one sequence, its KV heads drawn in parallel (each head has its own seed
    stream, so the values do not depend on the split)."""
    import numpy as np
    parts = list(pool.map(lambda h: fn([h]), heads))
    return (np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1))


def run_decode(args, w, dev, pool):
    import numpy as np
    import torch

    import synth
    import paged_kv_cache_358_amd as pa
    from paged_kv_cache_358_amd.engine import PagedDecodeLayer

    W, K = args.warmup, args.steps
    BS = args.block_size
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    t_setup = time.perf_counter()

    if w == "c4":
        cfg = synth.C4
        kw, name = {}, cfg.name
        if args.dtype:
            kw["dtype"] = args.dtype
            name = name.replace("bf16", args.dtype)
        if args.head_dim:
            kw["head_dim"] = args.head_dim
            name += f"_d{args.head_dim}"
        if BS != 16:
            kw["block_size"] = BS
            name += f"_b{BS}"
        if kw:  # the same prompts and steps with another 16-bit type, head size or block size
            import dataclasses
            cfg = dataclasses.replace(cfg, name=name, **kw)
        part = args.partition_size or cfg.partition_size
        if W + K > cfg.steps:
            sys.exit(f"c4 runs at most {cfg.steps} decode steps")
        S, hq, hkv, D, dtype = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
        max_blocks = -(-(cfg.prefix_len + cfg.steps) // BS)
        layer = PagedDecodeLayer(cfg.pool_blocks(), hkv, D, hq, tdt[dtype], S, max_blocks,
                                 free_order=cfg.free_order(), partition_size=part, device=dev, block_size=BS)
        heads = list(range(hkv))
        for i in range(cfg.num_prompts):
            root = i * cfg.samples
            k, v = _draw_heads(pool, lambda hs: cfg.prefix_kv(i, hs), heads)
            layer.add(root)
            layer.prefill(root, _up(k, dtype, dev), _up(v, dtype, dev))
            for c in range(1, cfg.samples):
                layer.fork(root, root + c)
        steps = list(range(1, W + K + 1))
        drawn = list(pool.map(lambda st: (cfg.step_q(st), *cfg.step_kv(st)), steps))
        step_inputs = [tuple(_up(x, dtype, dev) for x in d) for d in drawn]
        scale = cfg.softmax_scale
        kvbpt = cfg.kv_bytes_per_token()
        workload = {"workload": cfg.name, "prompts": cfg.num_prompts, "samples": cfg.samples,
                    "prefix_len": cfg.prefix_len, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D,
                    "block_size": BS, "partition_size": part, "timed_steps": f"{W + 1}..{W + K}"}
        lens0 = None
    else:
        cfg = synth.CONFIGS[WORKLOADS[w]]
        kw = {}
        suffix = ""
        if args.head_dim and w != "c1":
            kw["head_dim"] = args.head_dim
            suffix += f"_d{args.head_dim}"
        if BS != 16 and w != "c1":
            kw["block_size"] = BS
            suffix += f"_b{BS}"
        if args.dtype and w != "c1" and args.dtype != cfg.dtype:
            kw["dtype"] = args.dtype
        if kw:  # the same context lengths with another head size, block size or 16-bit type
            import dataclasses
            name = cfg.name + suffix
            if "dtype" in kw:
                name = name.replace("_" + cfg.dtype, "_" + args.dtype)
            cfg = dataclasses.replace(cfg, name=name, **kw)
        BS = cfg.block_size
        part = args.partition_size or cfg.partition_size
        S, hq, hkv, D, dtype = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.dtype
        lens0 = synth.context_lens(cfg)                # context at the first timed step
        plan = synth.pool_plan(cfg, lens0)
        need = int(synth.blocks_for(lens0 + K, BS).sum()) + plan.preoccupy_blocks
        if need > plan.num_blocks:
            sys.exit(f"{cfg.name}: {K} steps need {need} blocks, the pool holds {plan.num_blocks}")
        prefill = np.maximum(lens0 - W - 1, 0)
        max_blocks = int(synth.blocks_for(lens0.max() + K, BS))
        layer = PagedDecodeLayer(plan.num_blocks, hkv, D, hq, tdt[dtype], S, max_blocks,
                                 free_order=plan.free_order, partition_size=part, device=dev, block_size=BS)
        if plan.preoccupy_blocks:
            layer.alloc.add(FOREIGN)
            layer.alloc.append(FOREIGN, plan.preoccupy_blocks * BS)
        heads = list(range(hkv))
        for s in range(S):
            layer.add(s)
            if prefill[s]:
                k, v = _draw_heads(pool, lambda hs: synth.seq_kv(cfg, s, int(prefill[s]), hs), heads)
                layer.prefill(s, _up(k, dtype, dev), _up(v, dtype, dev))
        drawn = list(pool.map(lambda st: (synth.queries(cfg, step=1000 + st),
                                          *synth.new_tokens_kv(cfg.cfg_id, 1000 + st, S, hkv, D, dtype)),
                              range(W + K)))
        step_inputs = [tuple(_up(x, dtype, dev) for x in d) for d in drawn]
        scale = cfg.softmax_scale
        kvbpt = cfg.kv_bytes_per_token()
        workload = {"workload": cfg.name, "num_seqs": S, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D,
                    "block_size": BS, "partition_size": part, "context_lens": cfg.lens,
                    "mean_context": float(lens0.mean()), "pool_blocks": plan.num_blocks}
    del drawn
    torch.cuda.synchronize()
    print(f"[bench] {workload['workload']}: workload resident on the GPU "
          f"({time.perf_counter() - t_setup:.1f} s)", file=sys.stderr, flush=True)
    seqs = np.arange(S, dtype=np.int64)
    eb = synth.ELEM_BYTES[dtype]
    out = torch.empty(S, hq, D, dtype=tdt[dtype], device=dev)
    kernel = pa.paged_attention_decode_kernel(step_inputs[0][0], layer.k_cache, layer.v_cache,
                                              torch.empty(S, max_blocks, dtype=torch.int32, device=dev), out,
                                              max_blocks * BS, part)

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
    shared = w == "c4"  # forked samples share blocks: count each physical block once
    step_lens, step_pairs = [], []
    step_groups, step_group_rows = [], []
    first_tables = None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
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
    gc.unfreeze()
    elapsed = t1 - t0
    print(f"[bench] {workload['workload']}: {K} timed steps, {elapsed / K * 1e3:.3f} ms/step (host enqueue done "
          f"after {(t_enq - t0) / K * 1e3:.3f} ms/step)", file=sys.stderr, flush=True)

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
    launch_bytes = float(np.mean(attn))
    achieved = launch_bytes / mean_main_s / 1e9

    block = {
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
        "kernel": kernel,
        "kernel_us": round(mean_main_s * 1e6, 2),
        "attention_ms": {"main_kernel": round(float(np.mean(main_ms)), 4)},
        "shared_prefix_groups": int(max(step_groups)),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(kernel, workload["workload"], workload.get("timed_steps")),
                     "kernel": kernel, "bytes_per_launch": int(launch_bytes)},
        "copy_on_write_blocks": int(sum(step_pairs)),
    }
    if w == "c1":
        block["note"] = ("launch-bound: the step moves about 0.15 MB, 20 ns at peak; its figures are "
                         "microseconds, not a fraction of the HBM roofline")
    if shared:
        block["logical_attention_bytes_per_launch"] = int(np.mean(logical))
        block["effective_logical_gbs"] = round(float(np.mean(logical)) / mean_main_s / 1e9, 1)

    last_tables = layer.last_tables.copy()
    block["cache_ops"] = cache_ops_probe(layer, step_inputs[-1], last_tables, block_bytes)
    if not shared and w != "c1":
        block["decode_probes"] = decode_probes(layer, step_inputs[-1][0], out, scale, last_tables,
                                               step_lens[-1], part, attn[-1])
    del layer, step_inputs, out
    gc.collect()
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        budget = args.cpu_seconds if w == HEADLINE else args.cpu_seconds / 3
        block["cpu_oracle"] = cpu_oracle(cfg, lens0, kvbpt, budget, host_threads(), pool)
        if w == "c2":
            block["cpu_oracle_1_thread"] = cpu_oracle(cfg, lens0, kvbpt, args.cpu_seconds / 3, 1, pool)
    return block


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
    BS = args.block_size
    if BS != 16 or args.head_dim:  # the same contexts laid out in other blocks, or with another head size
        import dataclasses
        cfg = dataclasses.replace(cfg, block_size=BS, head_dim=args.head_dim or cfg.head_dim)
    lens = synth.context_lens(cfg).astype(np.int64)
    chunks = np.minimum(lens, args.chunk)
    S, hq, hkv, D = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    plan = synth.pool_plan(cfg, lens)
    torch.manual_seed(cfg.cfg_id)
    k_cache, v_cache = pa.alloc_kv_cache(plan.num_blocks, hkv, D, torch.bfloat16, dev, block_size=BS)
    k_cache.normal_()
    v_cache.normal_()
    alloc = pa.BlockAllocator(plan.num_blocks, BS, plan.free_order)
    for s_ in range(S):
        alloc.add(s_)
        alloc.append(s_, int(lens[s_]))
    max_blocks = int(synth.blocks_for(lens.max(), BS))
    tables, lens_np = alloc.build_batch(list(range(S)), max_blocks)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    T = int(qs[-1])
    q = torch.randn(T, hq, D, device=dev).to(torch.bfloat16)
    out = torch.empty(T, hq, D, device=dev, dtype=torch.float32)
    bt, cl, qst = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (tables, lens_np, qs))
    order = torch.from_numpy(pa.prefill_order(lens_np, qs)).to(dev)  # heaviest sequences first
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record()
        b.record()

    def launch(events=None):
        pa.paged_attention_prefill(q, k_cache, v_cache, bt, cl, qst, cfg.softmax_scale, out,
                                   max_query_len=int(chunks.max()), seq_order=order,
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
                   "rows": T, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": D, "block_size": BS},
        "kernel_ms": round(kern_s * 1e3, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_tiled_kernel", "flops_per_launch": flops},
        "kv_bytes_per_launch": kv_bytes, "kv_gbs_if_read_once": round(kv_bytes / kern_s / 1e9, 1),
    }), flush=True)


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


def cpu_oracle(cfg, lens0, kvbpt, budget_s, threads, pool):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload with `threads` BLAS
    threads.  Sequences are drawn one at a time in a seeded order (each drawn once, its inputs decoded
    to float64 beforehand, outside the timing) and the oracle is run on each for its share of the
    budget.  A long-context sequence is sampled by two of its KV heads (and their query heads) and
    scaled to the whole sequence.  Reports the oracle's K/V GB/s and sequences per second (one decode
    step of one layer)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle.attention import decode_attention_seq

    hkv = cfg.num_kv_heads
    if lens0 is None:  # parallel sampling: every sample at its final context, prefix + appended tokens
        n_ctx = cfg.prefix_len + cfg.steps
        step_kv = list(pool.map(cfg.step_kv, range(1, cfg.steps + 1)))

        def draw(s, heads):
            pk, pv = cfg.prefix_kv(s // cfg.samples, heads)
            return (np.concatenate([pk, np.stack([k[s][heads] for k, _ in step_kv])]),
                    np.concatenate([pv, np.stack([v[s][heads] for _, v in step_kv])]))
        lens = [n_ctx] * cfg.num_seqs
        q = cfg.step_q(cfg.steps)
    else:
        def draw(s, heads):
            return _draw_heads(pool, lambda hs: synth.seq_kv(cfg, s, int(lens0[s]), hs), heads)
        lens = lens0.tolist()
        q = synth.queries(cfg)
    long_ctx = max(lens) > 65536
    # at most 8 sequences (2 of a long-context workload), in a seeded order
    order = np.random.default_rng(0).permutation(len(lens))[:2 if long_ctx else 8]
    heads = list(range(2)) if long_ctx else list(range(hkv))   # KV heads drawn per sequence
    g = cfg.num_q_heads // hkv
    per = budget_s / len(order)
    spent, done, ctx_tokens = 0.0, 0.0, 0
    t_all = time.perf_counter()
    with threadpool_limits(limits=threads):
        for i, s in enumerate(order):
            k, v = draw(int(s), heads)
            k64, v64 = synth.decode_f64(k, cfg.dtype), synth.decode_f64(v, cfg.dtype)
            q64 = synth.decode_f64(q[s], cfg.dtype)[heads[0] * g:(heads[-1] + 1) * g]
            mine = 0.0
            while mine < per or mine == 0.0:
                t = time.perf_counter()
                decode_attention_seq(q64, k64, v64, cfg.softmax_scale)
                mine += time.perf_counter() - t
                done += len(heads) / hkv
                ctx_tokens += int(lens[s]) * len(heads) / hkv
            spent += mine
            if spent >= budget_s or time.perf_counter() - t_all > 3 * budget_s + 30:
                break
    gbs = ctx_tokens * kvbpt / spent / 1e9
    what = (f"{len(heads)} of {hkv} KV heads ({len(heads) * g} query heads) of {i + 1} sequence(s) of "
            f"{max(lens)} tokens, scaled to whole sequences" if long_ctx else
            f"{i + 1} of {len(lens)} sequences (seeded choice), all {cfg.num_q_heads} query heads")
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seq_tokens_per_s_per_layer": round(done / spent, 3),
            "sample": f"fp64 oracle on {what}: {done:.2f} sequence evaluations, {ctx_tokens:.0f} context "
                      f"tokens in {spent:.1f} s with {threads} BLAS thread(s); inputs drawn and decoded to "
                      f"float64 outside the timing"}


if __name__ == "__main__":
    main()
