"""Benchmark: one decode step of a Llama-3-8B-shaped batch through the paged KV path.

A step is the whole hot path for one new token of every sequence:
  host:   allocate_slots for each sequence (kv_pool_append_batch), the dense block
          tables (kv_pool_build_tables) into pinned buffers, then their copy to HBM, and
          the step's decode order from the host lengths (paged_attention_decode_plan, used
          by every layer's single-pass launch; --no-plan: the kernel ranks the lengths);
  device: for each of the 32 layers, the new tokens' K/V written into that layer's pool
          and paged_attention_decode over the whole context, in one fused launch
          (paged_attention_decode_append; --unfused: reshape_and_cache then
          paged_attention_decode), and the partition reduce when partitioned.
Every layer has its own K/V pool (about 313 MB, more than the 256 MB Infinity Cache),
so each layer's context streams from HBM. Inputs are synthetic (seeded draws of the
8B-shaped workload) and resident in HBM before timing starts.

Python's garbage collector is frozen and disabled from the warm-up to the end of the
kernel-timing pass (a full collection takes about 40 ms and would otherwise land in one step).

Printed: one JSON line. `value` is KV GB/s over the whole step (algorithmic KV bytes
read by the decode kernels / step time), timed with no per-launch instrumentation;
`roofline` is the decode kernel alone, from a second pass of the same number of steps in
which the library binds HIP start/stop events to each of its kernel launches
(pkv_timer_*: the events carry the kernel's own begin/end timestamps); `cpu_baseline`
is the CPU oracle on a bounded sample.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--config llama8b]
                       [--partition P] [--no-cpu-baseline]
       python bench.py --config churn   (continuous batching; 50 timed steps after 10)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the sources that define the decode kernels: HBM counters taken for other sources are stale
DECODE_SOURCES = ("decode.hip", "decode_kernels.hpp", "tile.hpp", "device.hpp")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; churn: 50)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 5; churn: 10)")
    ap.add_argument("--config", default="llama8b")
    ap.add_argument("--partition", default=None,
                    help="auto (balanced split), 0 (single pass) or a multiple of 16; "
                         "default: the workload's setting")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="separate reshape_and_cache and paged_attention_decode launches")
    ap.add_argument("--no-kernel-timer", action="store_true",
                    help="skip the kernel-timing pass (no roofline figure)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-plan", action="store_true",
                    help="no host-side decode plan: the single-pass kernel ranks the lengths "
                         "itself at every launch")
    ap.add_argument("--block-size", type=int, default=None, choices=(8, 16, 32),
                    help="tokens per KV block (default: the workload's, 16)")
    ap.add_argument("--copy-blocks", type=int, default=0, metavar="N",
                    help="only time copy_blocks (copy-on-write of N forked sequences' partly "
                         "filled blocks, every layer of the workload) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB buffer 8 times (a plain copy of known size, to "
                         "scale the HBM byte counters) and exit")
    args = ap.parse_args()
    churn = args.config == "churn"
    if args.steps is None:
        args.steps = 50 if churn else 20
    if args.warmup is None:
        args.warmup = 10 if churn else 5
    return args


def decode_source_sha256() -> str:
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_28_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                   for f in DECODE_SOURCES)).hexdigest()


def measured_traffic(workload: str, partition_size: int, fused: bool, block_size: int):
    """HBM bytes per decode launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE runs recorded in
    profiles/ (scaled by the copy calibration), or None if those counters were taken for
    another workload/mode/block size or for kernel sources other than the ones built now."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if partition_size != 0 or not fused or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("mode") != "single pass, fused append" or rec.get("block_size") != block_size:
        return None
    if decode_source_sha256() != rec.get("source_sha256"):
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def calibrate_copy():
    """A plain device copy of known size: 8 copies of 1 GiB (read 1 GiB, write 1 GiB each)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": {"bytes_read_per_copy": n, "bytes_written_per_copy": n,
                                         "copies": 8}}), flush=True)


def bench_copy_blocks(args):
    """copy_blocks on the workload's layer pools: N (src, dst) pairs with distinct blocks,
    K and V of every layer, timed with the library's kernel timer."""
    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    import workloads
    w = workloads.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    lens = workloads.draw_seq_lens(w)
    nb = workloads.pool_blocks_for(lens)
    n = args.copy_blocks
    caches = [pkv.alloc_caches(nb, w.num_kv_heads, w.head_dim, w.cache_dtype, dev, fill=1)
              for _ in range(w.layers)]
    pick = np.random.default_rng(w.seed).permutation(nb)[:2 * n].astype(np.int32)
    pairs = torch.from_numpy(pick.reshape(2, n).T.copy()).to(dev)
    ks, vs = [c[0] for c in caches], [c[1] for c in caches]
    for _ in range(args.warmup):
        pkv.copy_blocks(ks, vs, pairs)
    torch.cuda.synchronize()
    pkv.timer_enable(True)
    for _ in range(args.steps):
        pkv.copy_blocks(ks, vs, pairs)
    torch.cuda.synchronize()
    ms, launches = pkv.timer_read(pkv.PKV_TIMER_COPY_BLOCKS)
    pkv.timer_enable(False)
    block_bytes = ks[0][0].numel() * ks[0].element_size()
    moved = 2 * 2 * w.layers * n * block_bytes          # K and V, read and written
    per_call_us = ms * 1e3 / args.steps
    print(json.dumps({"copy_blocks": {
        "workload": w.name, "pairs": n, "layers": w.layers, "block_bytes": block_bytes,
        "launches_per_call": launches // args.steps, "us_per_call": round(per_call_us, 3),
        "bytes_per_call": moved, "GB/s": round(moved / (per_call_us * 1e-6) / 1e9, 1),
        "frac_of_peak": round(moved / (per_call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}),
          flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak


def bench_prefill(args):
    """Chunked prefill (workloads with prefill_tokens): per step, one chunk of the long
    prompt (its K/V written, then paged_attention_prefill) and one fused decode token for
    each user, in every layer. A pass is all chunks of the prompt; one untimed pass, one
    timed pass, one pass with the library's kernel timer, each on a fresh pool."""
    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    import workloads
    w = workloads.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    L, U, Hq, Hkv, d = w.layers, w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    tdt = pkv.torch_dtype(w.dtype)
    C = -(-w.prefill_tokens // w.prefill_chunks)
    chunks = [(c0, min(w.prefill_tokens, c0 + C)) for c0 in range(0, w.prefill_tokens, C)]
    ulens = workloads.draw_seq_lens(w)
    nsteps = len(chunks)
    nb = workloads.pool_blocks_for(list(ulens) + [w.prefill_tokens], growth_tokens=nsteps)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    caches = []
    for _ in range(L):
        kc, vc = pkv.alloc_caches(nb, Hkv, d, tdt, dev)
        kc.normal_(generator=g)
        vc.normal_(generator=g)
        caches.append((kc, vc))
    qp = [torch.randn((C, Hq, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    kp = [torch.randn((C, Hkv, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    vp = [torch.randn((C, Hkv, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    qu = [torch.randn((U, Hq, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    ku = [torch.randn((U, Hkv, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    vu = [torch.randn((U, Hkv, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    outp = torch.empty((C, Hq, d), device=dev, dtype=tdt)
    outu = torch.empty((U, Hq, d), device=dev, dtype=tdt)
    mbp = -(-w.prefill_tokens // 16)
    mbu = int(-(-(int(ulens.max()) + nsteps) // 16))
    order = workloads.draw_free_order(nb, workloads.rng(w.seed, 1))

    def run_pass():
        pool = pkv.kv_pool_create(nb, L, Hkv, d, w.dtype, free_order=order)
        uid = np.arange(1, U + 1, dtype=np.int64)
        for u in range(U):
            pool.add_seq(int(uid[u]))
            pool.append(int(uid[u]), int(ulens[u]) - 1)
        pool.add_seq(0)
        for c0, c1 in chunks:
            ps = torch.from_numpy(pool.append(0, c1 - c0)).to(dev)
            tp, lp = pool.build_tables([0], mbp)
            us = torch.from_numpy(pool.append_batch(uid)).to(dev)
            tu, lu = pool.build_tables(uid, mbu)
            tp, lp, tu, lu = (torch.from_numpy(x).to(dev) for x in (tp, lp, tu, lu))
            qs = torch.tensor([0, c1 - c0], dtype=torch.int32, device=dev)
            for l in range(L):
                kc, vc = caches[l]
                pkv.reshape_and_cache(kp[l][:c1 - c0], vp[l][:c1 - c0], kc, vc, ps)
                pkv.paged_attention_prefill(outp[:c1 - c0], qp[l][:c1 - c0], qs, kc, vc, tp, lp,
                                            w.scale, c1 - c0)
                pkv.paged_attention_decode_append(outu, qu[l], ku[l], vu[l], us, kc, vc, tu, lu,
                                                  w.scale)
        pool.close()

    run_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_pass()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pkv.timer_enable(True)
    run_pass()
    torch.cuda.synchronize()
    pre_ms, pre_n = pkv.timer_read(pkv.PKV_TIMER_PREFILL)
    dec_ms, dec_n = pkv.timer_read(pkv.PKV_TIMER_DECODE)
    cw_ms, cw_n = pkv.timer_read(pkv.PKV_TIMER_CACHE_WRITE)
    pkv.timer_enable(False)
    # causal attention of the whole prompt: query at position p attends to p + 1 keys;
    # 2 flops per multiply-add in Q K^T and in P V, every query head, every layer
    pairs = sum((c1 * (c1 + 1) - c0 * (c0 + 1)) // 2 for c0, c1 in chunks)
    flops = 4 * d * Hq * pairs * L
    tflops = flops / (pre_ms * 1e-3) / 1e12
    result = {
        "metric": "chunked prefill: paged_attention_prefill MFMA TFLOP/s (causal attention of "
                  "the prompt) + step time with the users' decode",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": nsteps,
        "warmup": 1, "ms_per_step": round(elapsed / nsteps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded draws)",
        "config": {"workload": w.name, "layers": L, "prompt_tokens": w.prefill_tokens,
                   "chunks": nsteps, "chunk_tokens": C, "decode_users": U,
                   "user_seq_len_range": [w.len_lo, w.len_hi], "num_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "block_size": 16},
        "prefill_kernel_us_avg": round(pre_ms * 1e3 / pre_n, 2),
        "prefill_tokens_per_s_per_layer": round(w.prefill_tokens / (pre_ms * 1e-3 / L), 1),
        "decode_kernel_us_avg": round(dec_ms * 1e3 / dec_n, 3) if dec_n else None,
        "cache_write_kernel_us_avg": round(cw_ms * 1e3 / cw_n, 3) if cw_n else None,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_attention_prefill",
                     "alg_flops_per_pass": flops},
    }
    print(json.dumps(result), flush=True)


def bench_churn(args):
    """Continuous-batching churn: the 8B shape on a ~200 GB pool, 256 live sequences with log-uniform prompts in [16, 32768], 20% of them
    aliasing a 1,024-token system prompt written once. A step retires 5% of the live
    sequences (their blocks back to the free queue), admits as many (pool allocation of
    their prompts, and in every layer the prompts' K/V written with reshape_and_cache),
    appends one token to every live sequence and decodes it in every layer (balanced split:
    the new rows' cache write, the decode and the reduce). Timed: K steps after W warm-up
    steps with no instrumentation, then K more steps under the library's kernel timer."""
    import gc

    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    import workloads
    w = workloads.WORKLOADS["churn"]
    dev = torch.device("cuda:0")
    L, B, Hq, Hkv, d = w.layers, w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    e = w.elem_bytes
    tdt = pkv.torch_dtype(w.dtype)
    P = pkv.PKV_PARTITION_AUTO
    nb = workloads.churn_pool_blocks(w)
    order = workloads.draw_free_order(nb, workloads.rng(w.seed, 1))
    pool = pkv.kv_pool_create(nb, L, Hkv, d, w.dtype, free_order=order)
    total_steps = args.warmup + 2 * args.steps
    max_blocks = -(-(w.prefix_tokens + w.prompt_hi + total_steps + 1) // 16)
    maxp = pkv.max_partitions_for(max_blocks, P)
    caches = [pkv.alloc_caches(nb, Hkv, d, w.dtype, dev) for _ in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    SRC = 1 << 17   # prompt rows are slices of one random buffer (values do not set the time)
    src_k = torch.randn((SRC, Hkv, d), generator=g, device=dev, dtype=tdt)
    src_v = torch.randn((SRC, Hkv, d), generator=g, device=dev, dtype=tdt)
    q = [torch.randn((B, Hq, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    k_new = torch.randn((B, Hkv, d), generator=g, device=dev, dtype=tdt)
    v_new = torch.randn((B, Hkv, d), generator=g, device=dev, dtype=tdt)
    out = torch.empty((B, Hq, d), device=dev, dtype=tdt)
    parts = pkv.alloc_partials(B, Hq, d, maxp, dev)

    def write_prompts(slots, timed_cw=None):
        """The prompt rows of every layer; slots: int32 host array."""
        if len(slots) == 0:
            return
        for c0 in range(0, len(slots), SRC):
            sl = torch.from_numpy(np.ascontiguousarray(slots[c0:c0 + SRC])).to(dev)
            n = sl.numel()
            for layer in range(L):
                kc, vc = caches[layer]
                if timed_cw is not None:
                    timed_cw[1] += pkv.timer_read(pkv.PKV_TIMER_CACHE_WRITE)[0]
                pkv.reshape_and_cache(src_k[:n], src_v[:n], kc, vc, sl)
                if timed_cw is not None:
                    timed_cw[0] += pkv.timer_read(pkv.PKV_TIMER_CACHE_WRITE)[0]

    # the shared system prompt (sequence -1) and the initial batch
    PREFIX = -1
    pool.add_seq(PREFIX)
    init_slots = [pool.append(PREFIX, w.prefix_tokens)]
    live, sharer, next_id = [], {}, 0
    for is_sharer, n in workloads.draw_churn_initial(w, workloads.rng(w.seed, 5, 0)):
        pool.add_seq(next_id)
        if is_sharer:
            pool.share_prefix(next_id, PREFIX, w.prefix_tokens)
        init_slots.append(pool.append(next_id, n))
        live.append(next_id)
        sharer[next_id] = is_sharer
        next_id += 1
    write_prompts(np.concatenate(init_slots))
    torch.cuda.synchronize()
    print(f"churn: pool of {nb} blocks, {len(live)} sequences written", file=sys.stderr, flush=True)

    h_tab = torch.empty((B, max_blocks), dtype=torch.int32, pin_memory=True)
    h_len = torch.empty(B, dtype=torch.int32, pin_memory=True)
    stats = {"prompt_tokens": 0, "kv_logical": 0, "kv_unique": 0}
    prefix_bytes = w.prefix_tokens * Hkv * d * 2 * e

    def step(s, timed_cw=None):
        nonlocal next_id
        retire, admits = workloads.draw_churn_step(w, workloads.rng(w.seed, 6, 0, s), live)
        for pos in sorted(retire, reverse=True):
            sid = live.pop(pos)
            pool.free_seq(sid)
            sharer.pop(sid)
        pslots = []
        for is_sharer, n in admits:
            pool.add_seq(next_id)
            if is_sharer:
                pool.share_prefix(next_id, PREFIX, w.prefix_tokens)
            pslots.append(pool.append(next_id, n))
            live.append(next_id)
            sharer[next_id] = is_sharer
            next_id += 1
        pslots = np.concatenate(pslots) if pslots else np.zeros(0, np.int32)
        stats["prompt_tokens"] += len(pslots)
        dslots = torch.from_numpy(pool.append_batch(live)).to(dev)
        pool.build_tables(live, max_blocks, h_tab.numpy(), h_len.numpy())
        lens = h_len.numpy().astype(np.int64)
        n_share = sum(1 for sid in live if sharer[sid])
        kv = int(lens.sum()) * Hkv * d * 2 * e
        stats["kv_logical"] += kv * L
        stats["kv_unique"] += (kv - max(0, n_share - 1) * prefix_bytes) * L
        d_tab = h_tab.to(dev, non_blocking=True)
        d_len = h_len.to(dev, non_blocking=True)
        write_prompts(pslots, timed_cw)
        for layer in range(L):
            kc, vc = caches[layer]
            if timed_cw is not None:
                timed_cw[1] += pkv.timer_read(pkv.PKV_TIMER_CACHE_WRITE)[0]
            pkv.decode(out, q[layer], kc, vc, d_tab, d_len, w.scale, P, parts,
                       append=(k_new, v_new, dslots))
        torch.cuda.synchronize()   # the pinned table buffer is reused by the next step

    gc.collect()
    gc.freeze()
    gc.disable()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    print("churn: warm-up done", file=sys.stderr, flush=True)
    stats = {k: 0 for k in stats}
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed = dict(stats)
    print("churn: timed steps done", file=sys.stderr, flush=True)
    # kernel-timing pass: prompt writes timed alone (cw[0]), the new rows' writes (cw[1])
    stats = {k: 0 for k in stats}
    cw = [0.0, 0.0]
    pkv.timer_enable(True)
    for s in range(args.steps):
        step(args.warmup + args.steps + s, cw)
    torch.cuda.synchronize()
    cw[1] += pkv.timer_read(pkv.PKV_TIMER_CACHE_WRITE)[0]
    dec_ms, dec_n = pkv.timer_read(pkv.PKV_TIMER_DECODE)
    red_ms, red_n = pkv.timer_read(pkv.PKV_TIMER_REDUCE)
    pkv.timer_enable(False)
    gc.enable()
    attn_s = (dec_ms + red_ms) * 1e-3
    pt = stats["prompt_tokens"]
    prompt_bytes = pt * Hkv * d * 2 * e * L          # written (the rows are read as much)
    result = {
        "metric": "paged decode attention: achieved KV HBM GB/s (% of peak) + decode tokens/s/layer",
        "value": round(timed["kv_logical"] / elapsed / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded churn events, prompt lengths and prefix sharing)",
        "config": {"workload": "churn", "layers": L, "batch": B, "num_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "block_size": 16,
                   "pool_blocks": nb, "pool_gb": round(nb * w.block_bytes_per_layer * L / 1e9, 1),
                   "prefix_tokens": w.prefix_tokens, "share_frac": w.share_frac,
                   "retire_frac": w.retire_frac, "prompt_range": [w.prompt_lo, w.prompt_hi],
                   "partition_size": "auto"},
        "step_kv_gb_s_note": "value = logical KV bytes read by the decode over whole steps "
                             "(retire + admit + prompt writes + 32 layers of decode) / step time",
        "attention_kv_logical_gb_s": round(stats["kv_logical"] / attn_s / 1e9, 1),
        "attention_kv_unique_gb_s": round(stats["kv_unique"] / attn_s / 1e9, 1),
        "attention_pct_of_peak": round(100 * stats["kv_logical"] / attn_s / 1e9 / HBM_PEAK_GBS, 2),
        "decode_kernel_us": round(dec_ms * 1e3 / dec_n, 2) if dec_n else None,
        "reduce_kernel_us": round(red_ms * 1e3 / red_n, 2) if red_n else None,
        "new_rows_cache_write_us": round(cw[1] * 1e3 / dec_n, 2) if dec_n else None,
        "prompt_tokens_per_step": round(pt / args.steps, 1),
        "prompt_write_us_per_layer": round(cw[0] * 1e3 / (args.steps * L), 2),
        "prompt_write_gb_s": round(2 * prompt_bytes / (cw[0] * 1e-3) / 1e9, 1) if cw[0] else None,
        "decode_tok_s_per_layer": round(B * args.steps * L / (attn_s + cw[1] * 1e-3), 1),
        "kernel_timing": "library timer (HIP events bound to each launch) in a second pass of "
                         "K steps; the prompt writes are read back one by one",
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    pool.close()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (run with --gpus 1): every path here is timed "
              "on one GPU's share of the work", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.copy_blocks:
        bench_copy_blocks(args)
        return
    import workloads as _wl
    if args.config == "churn":
        bench_churn(args)
        return
    if _wl.WORKLOADS[args.config].prefill_tokens:
        bench_prefill(args)
        return
    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.config]
    if args.partition is None:
        P = w.partition_size
    else:
        P = pkv.PKV_PARTITION_AUTO if args.partition == "auto" else int(args.partition)
    L, B, Hq, Hkv, d = w.layers, w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    bs = args.block_size or w.block_size
    e = w.elem_bytes                 # q, out and new-row inputs
    ekv = w.cache_elem_bytes         # cache elements (1 for an FP8 cache)
    fp8 = w.cache_dtype == "fp8"
    tdt = pkv.torch_dtype(w.dtype)

    # ---------------------------------------------------------------- setup
    lens0 = workloads.draw_seq_lens(w)                 # context at the first step
    total_steps = args.warmup + 2 * args.steps        # timed steps + kernel-timing pass
    nb = workloads.pool_blocks_for(lens0, growth_tokens=total_steps, block_size=bs)
    order = workloads.draw_free_order(nb, workloads.rng(w.seed, 1))
    pool = pkv.kv_pool_create(nb, L, Hkv, d, w.cache_dtype, free_order=order, block_size=bs)
    ids = np.arange(B, dtype=np.int64)
    for b in range(B):
        pool.add_seq(int(b))
        pool.append(int(b), int(lens0[b]) - 1)        # the cached prompt
    max_blocks = int(-(-(int(lens0.max()) + total_steps) // bs))
    maxp = pkv.max_partitions_for(max_blocks, P, bs) if P != 0 else 0

    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    caches = []
    for _ in range(L):
        kc, vc = pkv.alloc_caches(nb, Hkv, d, w.cache_dtype, dev, block_size=bs)
        if fp8:   # codes of N(0,1) draws under the workload's scales
            for t, sc in ((kc, w.k_scale), (vc, w.v_scale)):
                x = torch.randn(t.shape, generator=g, device=dev).div_(sc).clamp_(-448, 448)
                t.copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
                del x
        else:
            kc.normal_(generator=g)
            vc.normal_(generator=g)
        caches.append((kc, vc))
    q = [torch.randn((B, Hq, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    k_new = [torch.randn((B, Hkv, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    v_new = [torch.randn((B, Hkv, d), generator=g, device=dev, dtype=tdt) for _ in range(L)]
    out = [torch.empty((B, Hq, d), device=dev, dtype=tdt) for _ in range(L)]
    parts = pkv.alloc_partials(B, Hq, d, maxp, dev) if P != 0 else None

    # double-buffered pinned metadata; an event guards each buffer's reuse
    h_tab = [torch.empty((B, max_blocks), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    h_len = [torch.empty(B, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    h_slot = [torch.empty(B, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    copied = [torch.cuda.Event() for _ in range(2)]
    d_tab = torch.empty((B, max_blocks), dtype=torch.int32, device=dev)
    d_len = torch.empty(B, dtype=torch.int32, device=dev)
    d_slot = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    kv_bytes_steps = []

    def step(s: int):
        k = s & 1
        copied[k].synchronize()                       # H2D of two steps ago has finished
        pool.append_batch(ids, out=h_slot[k].numpy())
        pool.build_tables(ids, max_blocks, h_tab[k].numpy(), h_len[k].numpy())
        # the step's schedule, once for all layers (the single pass uses it)
        order = None if args.no_plan else pkv.paged_attention_decode_plan(h_len[k].numpy(), Hkv)
        kv_bytes_steps.append(int(h_len[k].numpy().astype(np.int64).sum()) * Hkv * d * 2 * ekv * L)
        d_slot.copy_(h_slot[k], non_blocking=True)
        d_tab.copy_(h_tab[k], non_blocking=True)
        d_len.copy_(h_len[k], non_blocking=True)
        copied[k].record(stream)
        po, pm, ps = parts if P != 0 else (None, None, None)
        for layer in range(L):
            kc, vc = caches[layer]
            if fp8 and args.unfused:
                pkv.reshape_and_cache_fp8(k_new[layer], v_new[layer], kc, vc, d_slot, w.k_scale,
                                          w.v_scale)
                pkv.paged_attention_decode_fp8(out[layer], q[layer], kc, vc, d_tab, d_len, w.scale,
                                               w.k_scale, w.v_scale, P, po, pm, ps, maxp,
                                               seq_order=order)
            elif fp8:
                pkv.paged_attention_decode_append_fp8(out[layer], q[layer], k_new[layer],
                                                      v_new[layer], d_slot, kc, vc, d_tab, d_len,
                                                      w.scale, w.k_scale, w.v_scale, P, po, pm,
                                                      ps, maxp, seq_order=order)
            elif args.unfused:
                pkv.reshape_and_cache(k_new[layer], v_new[layer], kc, vc, d_slot)
                pkv.paged_attention_decode(out[layer], q[layer], kc, vc, d_tab, d_len, w.scale,
                                           P, po, pm, ps, maxp, seq_order=order)
            else:
                pkv.paged_attention_decode_append(out[layer], q[layer], k_new[layer],
                                                  v_new[layer], d_slot, kc, vc, d_tab, d_len,
                                                  w.scale, P, po, pm, ps, maxp, seq_order=order)
            if P != 0:
                pkv.paged_attention_reduce(out[layer], po, pm, ps, d_len, P, Hkv, max_blocks, bs)

    # Python's cyclic collector stays off from the warm-up to the end of the kernel-timing
    # pass: a full collection of the interpreter's heap (torch's objects) takes about 40 ms
    # and would land in whichever step crosses its allocation threshold.
    import gc
    gc.collect()
    gc.freeze()
    gc.disable()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    kv_bytes_steps.clear()
    lens_steps = []
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s)
        lens_steps.append(h_len[(args.warmup + s) & 1].numpy().copy())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    kv_total = sum(kv_bytes_steps)                # KV bytes of the timed steps only

    # kernel-timing pass: the same steps again (the contexts keep growing), every launch
    # carrying its own start/stop events
    kernel_us = {"decode": None, "reduce": None, "cache_write": None}
    timing_lens = []
    step_pct = None
    if not args.no_kernel_timer:
        pkv.timer_enable(True)
        base = args.warmup + args.steps
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        marks[0].record(stream)
        for s in range(args.steps):
            step(base + s)
            marks[s + 1].record(stream)
            timing_lens.append(h_len[(base + s) & 1].numpy().copy())
        torch.cuda.synchronize()
        per_step = np.sort([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
        step_pct = {f"p{p}": round(float(np.percentile(per_step, p)), 4) for p in (10, 50, 90)}
        for name, entry in (("decode", pkv.PKV_TIMER_DECODE), ("reduce", pkv.PKV_TIMER_REDUCE),
                            ("cache_write", pkv.PKV_TIMER_CACHE_WRITE)):
            ms, n = pkv.timer_read(entry)
            kernel_us[name] = round(ms / n * 1e3, 3) if n else None
        pkv.timer_enable(False)
    gc.enable()
    dec_avg_s = kernel_us["decode"] / 1e6 if kernel_us["decode"] else float("nan")
    # algorithmic bytes of one decode launch: KV once per (seq, KV head), q, out, table rows;
    # fused, also the new rows read from the inputs and written to the pool
    new_rows = 0 if args.unfused else 2 * (B * Hkv * d * (e + ekv)) + 4 * B
    alg = []
    for ln in timing_lens:
        ln = ln.astype(np.int64)
        alg.append(int(ln.sum()) * Hkv * d * 2 * ekv + 2 * B * Hq * d * e +
                   int((-(-ln // bs)).sum()) * 4 + 4 * B + new_rows)
    alg_per_launch = sum(alg) / len(alg) if alg else float("nan")
    achieved = alg_per_launch / dec_avg_s / 1e9
    value = kv_total / elapsed / 1e9
    result = {
        "metric": "paged decode attention: achieved KV HBM GB/s (% of peak) + decode tokens/s/layer",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded draws of the workload's shapes and length mix)",
        "config": {"workload": f"{w.name}-decode", "layers": L, "batch": B, "num_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "block_size": bs,
                   "kv_cache_dtype": ("fp8 e4m3, k_scale %g, v_scale %g" % (w.k_scale, w.v_scale)
                                      if fp8 else w.dtype),
                   "seq_len_range": [w.len_lo, w.len_hi],
                   "partition_size": "auto" if P == pkv.PKV_PARTITION_AUTO else P,
                   "cache_write": ("separate launch" if args.unfused else
                                   "paged_attention_decode_append: separate launch in the balanced split"
                                   if P == pkv.PKV_PARTITION_AUTO else "fused into the decode launch"),
                   "decode_plan": ("in-kernel ranking" if args.no_plan or P != 0 else
                                   "host plan once per step (paged_attention_decode_plan)"),
                   "pool_blocks": nb,
                   "pool_gb_per_layer": round(nb * w.block_bytes_per_layer * bs / w.block_size / 1e9, 3),
                   "block_table_bytes": B * max_blocks * 4},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tok_s_per_layer": round(B * L * args.steps / elapsed, 1),
        "step_ms_percentiles": step_pct,
        "decode_kernel_us": kernel_us["decode"],
        "reduce_kernel_us": kernel_us["reduce"],
        "cache_write_kernel_us": kernel_us["cache_write"],
        "kernel_timing": "HIP start/stop events bound to each kernel launch (library timer), "
                         "averaged over every launch of the timed steps; step percentiles "
                         "from events between the steps of that same instrumented pass",
        "cache_state": f"{L} distinct per-layer pools cycled; warm-up {args.warmup} steps excluded",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1) if alg else None,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4) if alg else None, "traffic": None,
                     "kernel": ("paged_attention_decode" if args.unfused
                                else "paged_attention_decode_append (fused cache write + decode)")
                               + ("_fp8" if fp8 else ""),
                     "alg_bytes_per_launch": int(alg_per_launch) if alg else None},
        "cpu_baseline": None,
    }
    result["roofline"]["traffic"] = measured_traffic(w.name, P, not args.unfused, bs)
    ceiling = stream_ceiling()
    result["stream_ceiling"] = ceiling
    if alg:
        result["roofline"]["frac_of_ceiling"] = round(achieved / ceiling["GB/s"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, caches[0], q[0], d_tab, d_len, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def stream_ceiling():
    """What this GPU streams in practice, measured beside the roofline's spec peak: a plain
    device-to-device copy of 1 GiB (read + write bytes) and a read-only pass (fp32 sum of
    1 GiB), each the median of 10 runs bracketed by events, rotating over buffers so no
    run finds its input in cache. The decode kernel is read-dominated, so its fraction is
    taken against the higher of the two."""
    import torch
    n = 1 << 30
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(4)]
    for t in bufs:
        t.fill_(1)

    def median(fn):
        times = []
        for i in range(12):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(i)
            b.record()
            b.synchronize()
            if i >= 2:
                times.append(a.elapsed_time(b) / 1e3)
        return sorted(times)[len(times) // 2]

    t_copy = median(lambda i: bufs[(2 * i + 1) % 4].copy_(bufs[(2 * i) % 4]))
    t_read = median(lambda i: bufs[i % 4].view(torch.float32).sum())
    del bufs
    torch.cuda.empty_cache()
    copy_gbs, read_gbs = 2 * n / t_copy / 1e9, n / t_read / 1e9
    best = max(copy_gbs, read_gbs)
    return {"copy_1GiB_GB/s": round(copy_gbs, 1), "read_1GiB_GB/s": round(read_gbs, 1),
            "GB/s": round(best, 1), "frac_of_peak": round(best / HBM_PEAK_GBS, 4)}


def cpu_baseline(w, cache0, q0, d_tab, d_len, budget_s: float):
    """The CPU oracle (fp64, as it stands) on a bounded sample of the same workload:
    layer 0 of the batch, decoded repeatedly for about budget_s seconds of wall time on
    all host threads. Reported as KV GB/s and tokens/s/layer of that sample."""
    import numpy as np

    import oracle

    kc, vc = cache0
    kc_h, vc_h = oracle.raw(kc), oracle.raw(vc)
    q_h = oracle.raw(q0)
    tab = d_tab.cpu().numpy()
    lens = d_len.cpu().numpy()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    kv_per_pass = (int(lens.astype(np.int64).sum()) * w.num_kv_heads * w.head_dim * 2 *
                   w.cache_elem_bytes)
    passes, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        oracle.decode(q_h, kc_h, vc_h, tab, lens, w.scale, w.dtype, nthreads=cores,
                      kv_dtype=w.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        t += time.perf_counter() - t0
        passes += 1
    return {"value": round(kv_per_pass * passes / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "tok_s_per_layer": round(len(lens) * passes / t, 2),
            "seconds": round(t, 2),
            "sample": f"layer 0 of the step, all {len(lens)} sequences "
                      f"({int(lens.sum())} context tokens), decoded {passes}x by the fp64 "
                      f"oracle on {cores} threads"}


if __name__ == "__main__":
    main()
