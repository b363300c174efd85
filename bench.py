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
    ap.add_argument("--no-70b", action="store_true",
                    help="llama8b: skip the second object (the 70B batch, balanced split)")
    ap.add_argument("--print-launch-bytes", action="store_true",
                    help="add the algorithmic bytes of every decode launch to the line (for "
                         "pairing with HBM counters of the same run)")
    ap.add_argument("--traffic-summary", nargs=5, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR", "BENCH_LOG"),
                    help="only pair rocprofv3 HBM counters with the launches' algorithmic "
                         "bytes and write profiles/decode_<workload>_traffic.json")
    ap.add_argument("--cache-write-sweep", action="store_true",
                    help="only time reshape_and_cache / reshape_and_cache_fp8 over token counts "
                         "and slot patterns (8B shape) and exit")
    ap.add_argument("--rates", action="store_true",
                    help="only measure the unit rates (LDS reads, exponentials, FMAs, bf16 "
                         "16x16x32 products, products mixed with exponentials or FMAs) at 1, 2, "
                         "4 and 8 waves per SIMD and exit")
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


def measured_traffic(workload: str, partition_size: int, fused: bool, block_size: int, args,
                     alg_per_launch):
    """HBM bytes per decode launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
    profiles/decode_<workload>_traffic.json (copy-calibrated, averaged over the kernel-timing
    pass's dispatches of a run of this same command), or None unless that record was taken
    for the kernel sources built now, in this launch mode, with this many steps, and over
    launches whose algorithmic bytes equal this run's (the same dispatches)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if partition_size != 0 or not fused or not os.path.exists(path) or alg_per_launch is None:
        return None
    rec = json.load(open(path))
    if rec.get("mode") != "single pass, fused append" or rec.get("block_size") != block_size:
        return None
    if decode_source_sha256() != rec.get("source_sha256"):
        return None
    tp = rec.get("timing_pass") or {}
    if (rec.get("steps"), rec.get("warmup")) != (args.steps, args.warmup) or \
            tp.get("alg_bytes_per_launch") != alg_per_launch:
        return None
    return {"bytes_per_launch": int(tp["fetch_bytes_per_launch"] + tp["write_bytes_per_launch"]),
            "record": {"file": os.path.relpath(path, ROOT),
                       "fetch_bytes_per_launch": tp["fetch_bytes_per_launch"],
                       "write_bytes_per_launch": tp["write_bytes_per_launch"],
                       "fetch_over_alg": round(tp["fetch_bytes_per_launch"] / alg_per_launch, 4),
                       "dispatches": tp["dispatches"]}}


def _counter_rows(d: str):
    """(dispatch id, kernel name, counter, value) rows of a rocprofv3 --pmc CSV directory."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                             float(r["Counter_Value"])))
    rows.sort()
    return rows


def traffic_summary(spec):
    """Pair the HBM counters of a decode run with the algorithmic bytes of the same
    dispatches. spec: FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR BENCH_LOG: the
    rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE directories of `bench.py ... --no-cpu-baseline
    --no-70b --print-launch-bytes`, those of `bench.py --calibrate-copy`, and the bench's
    JSON line from the FETCH_SIZE run. Writes profiles/decode_<workload>_traffic.json and
    prints the figures."""
    import numpy as np
    fetch_d, write_d, cal_f, cal_w, log = spec
    line = [ln for ln in open(log) if ln.startswith("{") and '"launch_alg_bytes"' in ln][-1]
    bench = json.loads(line)
    alg = np.asarray(bench["launch_alg_bytes"], dtype=np.float64)

    def per_dispatch(d, counter, match):
        vals = {}
        for did, name, cn, v in _counter_rows(d):
            if cn == counter and match(name):
                vals[did] = vals.get(did, 0.0) + v
        return np.asarray([vals[k] for k in sorted(vals)])

    def scale(d, counter):   # bytes per KiB of the counter, from 1 GiB copies
        v = per_dispatch(d, counter, lambda n: "copyBuffer" in n)
        big = v[v > 0.9 * v.max()]
        return (1 << 30) / (float(np.median(big)) * 1024)

    is_decode = lambda n: "pkv::decode_" in n   # noqa: E731
    fs, ws = scale(cal_f, "FETCH_SIZE"), scale(cal_w, "WRITE_SIZE")
    f = per_dispatch(fetch_d, "FETCH_SIZE", is_decode) * 1024 * fs
    wr = per_dispatch(write_d, "WRITE_SIZE", is_decode) * 1024 * ws
    if "fp8_accuracy" in bench and len(f) == len(wr) > len(alg):
        # the FP8 run's accuracy check decodes after the timed passes: not in the record
        f, wr = f[:len(alg)], wr[:len(alg)]
    if not (len(f) == len(wr) == len(alg)):
        raise SystemExit(f"dispatch counts differ: fetch {len(f)}, write {len(wr)}, "
                         f"launches {len(alg)}")
    cfg = bench["config"]
    n_t = bench["steps"] * cfg["layers"]
    sl = slice(len(alg) - n_t, len(alg))
    rec = {
        "kernel": bench["roofline"]["kernel"], "mode": "single pass, fused append",
        "workload": cfg["workload"].replace("-decode", ""), "block_size": cfg["block_size"],
        "source_sha256": decode_source_sha256(), "steps": bench["steps"],
        "warmup": bench["warmup"], "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
        "timing_pass": {"dispatches": n_t,
                        "fetch_bytes_per_launch": int(f[sl].mean()),
                        "write_bytes_per_launch": int(wr[sl].mean()),
                        "alg_bytes_per_launch": int(alg[sl].mean())},
        "all_dispatches": {"dispatches": len(alg), "fetch_over_alg": round(float(f.sum() / alg.sum()), 4),
                           "write_bytes_per_launch": int(wr.mean())},
    }
    out = os.path.join(ROOT, "profiles", f"decode_{rec['workload']}_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def bench_rates():
    """Unit rates of the device's SIMDs (pkv_measure_rate), library timer, median of 5
    launches of each kind at 1, 2, 4 and 8 waves per SIMD. Counts per launch: LDS bytes =
    waves x 64 lanes x iters x 8 x 16; exponentials or FMAs = lanes x iters x 8 (16 FMAs in
    the mixed kind); products = waves x iters x 4 (16,384 flops each). "overlap" is the mixed
    kind's time over the sum of its two parts' times (0.5 = fully hidden, 1 = none)."""
    import torch

    import paged_kv_cache_28_amd as pkv
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4096
    sink = torch.zeros(cus * 8 * 4, dtype=torch.int32, device=dev)

    def timed(kind, wps):
        pkv.measure_rate(kind, wps, iters, sink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            pkv.timer_enable(True)
            pkv.measure_rate(kind, wps, iters, sink)
            ms, n = pkv.timer_read(pkv.PKV_TIMER_MEASURE)
            pkv.timer_enable(False)
            ts.append(ms / n)
        return sorted(ts)[2]

    rows = []
    for wps in (1, 2, 4, 8):
        waves = cus * 4 * wps
        t = {k: timed(k, wps) for k in pkv.RATE_KINDS}
        lanes = waves * 64
        rows.append({
            "waves_per_simd": wps, "ms": {k: round(v, 4) for k, v in t.items()},
            "lds_TB/s": round(waves * 64 * iters * 8 * 16 / t["lds_read"] / 1e9, 1),
            "exp_per_s": float(f"{lanes * iters * 8 / t['exp'] * 1e3:.4g}"),
            "fma_per_s": float(f"{lanes * iters * 8 / t['fma'] * 1e3:.4g}"),
            "mfma_TFLOP/s": round(waves * iters * 4 * 16384 / t["mfma"] / 1e9, 1),
            "mfma_16x16x16_TFLOP/s": round(waves * iters * 4 * 8192 / t["mfma_16x16x16"] / 1e9, 1),
            "overlap_mfma_exp": round(t["mfma_exp"] / (t["mfma"] + t["exp"]), 3),
            "overlap_mfma_16fma": round(t["mfma_fma"] / (t["mfma"] + 2 * t["fma"]), 3),
        })
    print(json.dumps({"rates": rows, "cus": cus, "iters": iters,
                      "kernel": "pkv_measure_rate (library timer, median of 5)"}), flush=True)


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


def bench_cache_write_sweep(args):
    """reshape_and_cache (and its FP8 form) on the 8B shape (8 KV heads, d 128, bf16 rows) for
    prompt-sized and decode-sized token counts, with consecutive slots (a prompt or chunk in
    consecutive blocks), a prompt's slots in blocks placed at random (as the pool hands them
    out after churn), and scattered ones (one token each of many sequences), timed with the
    library's kernel timer (median of 20 launches over a pool larger than the Infinity
    Cache)."""
    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    dev = torch.device("cuda:0")
    Hkv, d = 8, 128
    nb = 70000                                        # 4.6 GB per cache pair in bf16
    rows = {}
    for cache in ("bf16", "fp8"):
        kc, vc = pkv.alloc_caches(nb, Hkv, d, cache, dev, fill=0)
        for T in (64, 256, 1024, 4096, 16384, 65536):
            src = torch.randn((T, Hkv, d), device=dev).to(torch.bfloat16)
            gen = np.random.default_rng(T)
            for pattern in ("consecutive", "blocks", "scattered"):
                if pattern == "consecutive":
                    start = int(gen.integers(0, nb * 16 - T))
                    slots = np.arange(start, start + T, dtype=np.int32)
                elif pattern == "blocks":   # a prompt's slots: whole blocks, placed at random
                    blk = gen.permutation(nb)[:-(-T // 16)]
                    slots = (blk[:, None] * 16 + np.arange(16)).ravel()[:T].astype(np.int32)
                else:
                    slots = (gen.permutation(nb)[:T] * 16 + gen.integers(0, 16, T)).astype(np.int32)
                sl = torch.from_numpy(slots).to(dev)

                def call():
                    if cache == "fp8":
                        pkv.reshape_and_cache_fp8(src, src, kc, vc, sl, 0.015, 0.0125)
                    else:
                        pkv.reshape_and_cache(src, src, kc, vc, sl)
                call()
                torch.cuda.synchronize()
                pkv.timer_enable(True)
                times = []
                for _ in range(20):
                    call()
                    ms, n = pkv.timer_read(pkv.PKV_TIMER_CACHE_WRITE)
                    times.append(ms * 1e3 / max(n, 1))
                pkv.timer_enable(False)
                us = float(np.median(times))
                moved = T * Hkv * d * (2 + (1 if cache == "fp8" else 2)) * 2   # read + write
                rows[f"{cache}/{pattern}/{T}"] = {"us": round(us, 2),
                                                  "GB/s": round(moved / (us * 1e-6) / 1e9, 1)}
        del kc, vc
        torch.cuda.empty_cache()
    print(json.dumps({"cache_write_sweep": rows, "shape": "8 KV heads, head_dim 128, bf16 rows",
                      "timing": "library kernel timer, median of 20 launches",
                      "bytes": "rows read + cache bytes written"}), flush=True)


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
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.rates:
        bench_rates()
        return
    if args.cache_write_sweep:
        bench_cache_write_sweep(args)
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
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = _wl.WORKLOADS[args.config]
    result, ceiling = bench_decode(args, w, primary=True)
    # The other decode configuration the target names: the 70B batch in its own launch mode
    # (balanced split, its own 80 layer pools), timed the same way in the same run.
    if (args.config == "llama8b" and not args.no_70b and args.partition is None and
            args.block_size is None and not args.unfused and not args.no_plan):
        r70, _ = bench_decode(args, _wl.WORKLOADS["llama70b"], primary=False, ceiling=ceiling)
        result["llama70b"] = r70
    print(json.dumps(result), flush=True)


def bench_decode(args, w, primary: bool, ceiling=None):
    """The decode step of workload w: K timed steps after W warm-up steps with no
    instrumentation, then K more under the library's kernel timer. Returns the bench line
    (primary) or its compact form for a second configuration, and the measured ceilings."""
    import gc

    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    if args.partition is None or not primary:
        P = w.partition_size
    else:
        P = pkv.PKV_PARTITION_AUTO if args.partition == "auto" else int(args.partition)
    L, B, Hq, Hkv, d = w.layers, w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    bs = (args.block_size if primary else None) or w.block_size
    e = w.elem_bytes                 # q, out and new-row inputs
    ekv = w.cache_elem_bytes         # cache elements (1 for an FP8 cache)
    fp8 = w.cache_dtype == "fp8"
    tdt = pkv.torch_dtype(w.dtype)
    unfused = args.unfused and primary
    no_plan = args.no_plan and primary

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
    step_lens = []      # every step's lengths, in launch order (for per-launch bytes)

    def step(s: int):
        k = s & 1
        copied[k].synchronize()                       # H2D of two steps ago has finished
        pool.append_batch(ids, out=h_slot[k].numpy())
        pool.build_tables(ids, max_blocks, h_tab[k].numpy(), h_len[k].numpy())
        # the step's schedule, once for all layers (the single pass uses it)
        order = None if no_plan else pkv.paged_attention_decode_plan(h_len[k].numpy(), Hkv)
        kv_bytes_steps.append(int(h_len[k].numpy().astype(np.int64).sum()) * Hkv * d * 2 * ekv * L)
        step_lens.append(h_len[k].numpy().copy())
        d_slot.copy_(h_slot[k], non_blocking=True)
        d_tab.copy_(h_tab[k], non_blocking=True)
        d_len.copy_(h_len[k], non_blocking=True)
        copied[k].record(stream)
        po, pm, ps = parts if P != 0 else (None, None, None)
        for layer in range(L):
            kc, vc = caches[layer]
            if fp8 and unfused:
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
            elif unfused:
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
    gc.collect()
    gc.freeze()
    gc.disable()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    kv_bytes_steps.clear()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s)
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
    attn_s = dec_avg_s + (kernel_us["reduce"] or 0.0) / 1e6

    # algorithmic bytes of one decode launch: KV once per (seq, KV head), q, out, table rows;
    # fused, also the new rows read from the inputs and written to the pool
    fused_write = not unfused and P != pkv.PKV_PARTITION_AUTO
    new_rows = 2 * (B * Hkv * d * (e + ekv)) + 4 * B if fused_write else 0

    def alg_bytes(ln):
        ln = ln.astype(np.int64)
        return (int(ln.sum()) * Hkv * d * 2 * ekv + 2 * B * Hq * d * e +
                int((-(-ln // bs)).sum()) * 4 + 4 * B + new_rows)

    alg = [alg_bytes(ln) for ln in timing_lens]
    alg_per_launch = sum(alg) / len(alg) if alg else float("nan")
    kv_per_launch = (sum(int(ln.astype(np.int64).sum()) for ln in timing_lens) * Hkv * d * 2 * ekv
                     / len(timing_lens)) if timing_lens else float("nan")
    achieved = alg_per_launch / dec_avg_s / 1e9
    value = kv_total / elapsed / 1e9

    # ceilings: a contiguous read, and the same tile set gathered through the tables of the
    # kernel-timing pass's last step (no arithmetic), each from HIP kernels of the library
    if ceiling is None:
        ceiling = read_ceiling(dev, int(alg_per_launch) if alg else 1 << 28)
    gather = gather_ceiling(caches, d_tab, d_len, timing_lens[-1] if timing_lens else None,
                            Hkv, P, no_plan, alg_bytes, kv_bytes=lambda ln: int(
                                ln.astype(np.int64).sum()) * Hkv * d * 2 * ekv)

    cfg = {"workload": f"{w.name}-decode", "layers": L, "batch": B, "num_heads": Hq,
           "num_kv_heads": Hkv, "head_dim": d, "block_size": bs,
           "kv_cache_dtype": ("fp8 e4m3, k_scale %g, v_scale %g" % (w.k_scale, w.v_scale)
                              if fp8 else w.dtype),
           "seq_len_range": ([w.len_lo, w.len_hi] if not w.long_frac else
                             {"short": [w.len_lo, w.len_hi], "long": [w.long_lo, w.long_hi],
                              "long_frac": w.long_frac}),
           "partition_size": "auto" if P == pkv.PKV_PARTITION_AUTO else P,
           "cache_write": ("separate launch" if unfused else
                           "paged_attention_decode_append: separate launch in the balanced split"
                           if P == pkv.PKV_PARTITION_AUTO else "fused into the decode launch"),
           "decode_plan": ("in-kernel ranking" if no_plan or P != 0 else
                           "host plan once per step (paged_attention_decode_plan)"),
           "pool_blocks": nb,
           "pool_gb_per_layer": round(nb * w.block_bytes_per_layer * bs / w.block_size / 1e9, 3),
           "block_table_bytes": B * max_blocks * 4}
    kernel_name = (("paged_attention_decode" if unfused or P == pkv.PKV_PARTITION_AUTO
                    else "paged_attention_decode_append (fused cache write + decode)")
                   + ("_fp8" if fp8 else "")
                   + (" (balanced split)" if P == pkv.PKV_PARTITION_AUTO else ""))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1) if alg else None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4) if alg else None, "traffic": None,
                "kernel": kernel_name,
                "alg_bytes_per_launch": int(alg_per_launch) if alg else None}
    if alg:
        # against the read of one launch's bytes (8B); a 1.9 GB launch against the 1 GiB read
        read_rate = ceiling["GB/s"] if primary else ceiling["GB/s_1GiB"]
        roofline["frac_of_read_ceiling"] = round(achieved / read_rate, 4)
        if gather:
            roofline["frac_of_gather_ceiling"] = round(
                (kv_per_launch / dec_avg_s / 1e9) / gather["GB/s"], 4)
    if not primary:
        res = {"workload": cfg["workload"], "config": cfg,
               "decode_kernel_us": kernel_us["decode"], "reduce_kernel_us": kernel_us["reduce"],
               "cache_write_kernel_us": kernel_us["cache_write"],
               "kv_bytes_per_layer": int(kv_per_launch),
               "attention_kv_gb_s": round(kv_per_launch / attn_s / 1e9, 1),
               "attention_pct_of_peak": round(100 * kv_per_launch / attn_s / 1e9 / HBM_PEAK_GBS, 2),
               "step_kv_gb_s": round(value, 1), "ms_per_step": round(elapsed / args.steps * 1e3, 4),
               "tok_s_per_layer": round(B * L * args.steps / elapsed, 1),
               "roofline": roofline, "gather_ceiling": gather}
        del caches, q, k_new, v_new, out, parts
        pool.close()
        torch.cuda.empty_cache()
        return res, ceiling

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
        "config": cfg,
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
        "roofline": roofline,
        "read_ceiling": ceiling,
        "gather_ceiling": gather,
        "cpu_baseline": None,
    }
    # HBM counters of the same launches: the rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
    # same command, recorded with the algorithmic bytes of the dispatches they averaged
    tr = measured_traffic(w.name, P, not unfused, bs, args, int(alg_per_launch) if alg else None)
    if tr:
        roofline["traffic"] = tr["bytes_per_launch"]
        roofline["traffic_record"] = tr["record"]
    if args.print_launch_bytes:
        # algorithmic bytes of every decode launch of this run, in launch order (warm-up,
        # timed, kernel-timing pass): what the traffic summary pairs the counters with
        result["launch_alg_bytes"] = [alg_bytes(ln) for ln in step_lens for _ in range(L)]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, caches[0], q[0], d_tab, d_len, args.cpu_seconds)
    del caches, q, k_new, v_new, out, parts
    if fp8:
        result["fp8_accuracy"] = fp8_accuracy(w, dev)
    pool.close()
    torch.cuda.empty_cache()
    return result, ceiling


def fp8_accuracy(w, dev):
    """What the FP8 cache costs in accuracy at several context lengths: one sequence of N(0, 1)
    K/V (the workload's scales), written to a bf16 cache and to an FP8 cache and decoded from
    each; the FP8 output's max |difference| from the bf16 output, absolute and over the
    largest output. The bf16 path itself is within about 4e-6 of the fp64 oracle over these
    outputs (relative), so the difference is the quantisation's error."""
    import numpy as np
    import torch

    import paged_kv_cache_28_amd as pkv
    Hq, Hkv, d = w.num_heads, w.num_kv_heads, w.head_dim
    tdt = pkv.torch_dtype(w.dtype)
    rows = []
    for n in (128, 2048, 32768):
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + n)
        k = torch.randn((n, Hkv, d), generator=g, device=dev).to(tdt)
        v = torch.randn((n, Hkv, d), generator=g, device=dev).to(tdt)
        q = torch.randn((1, Hq, d), generator=g, device=dev).to(tdt)
        nb = -(-n // 16)
        perm = torch.randperm(nb, generator=g, device=dev).to(torch.int32)
        slots = (perm.repeat_interleave(16)[:n] * 16 +
                 torch.arange(n, device=dev, dtype=torch.int32) % 16).to(torch.int32)
        tab, lens = perm[None, :].contiguous(), torch.tensor([n], dtype=torch.int32, device=dev)
        outs = {}
        for cache in ("bf16", "fp8"):
            kc, vc = pkv.alloc_caches(nb, Hkv, d, cache if cache == "fp8" else w.dtype, dev, fill=0)
            o = torch.empty((1, Hq, d), dtype=torch.float32, device=dev)
            if cache == "fp8":
                pkv.reshape_and_cache_fp8(k, v, kc, vc, slots, w.k_scale, w.v_scale)
                pkv.decode(o, q, kc, vc, tab, lens, w.scale, 0, kv_scales=(w.k_scale, w.v_scale))
            else:
                pkv.reshape_and_cache(k, v, kc, vc, slots)
                pkv.decode(o, q, kc, vc, tab, lens, w.scale, 0)
            outs[cache] = o.double()
        err = float((outs["fp8"] - outs["bf16"]).abs().max())
        top = float(outs["bf16"].abs().max())
        rows.append({"context": n, "max_abs_err": round(err, 6), "max_abs_out": round(top, 6),
                     "norm_err": round(err / top, 5)})
    return {"vs": "the bf16-cache decode of the same K/V", "kv": "N(0, 1)",
            "k_scale": w.k_scale, "v_scale": w.v_scale, "by_context": rows}


def _median_us(pkv, fn, runs: int):
    """Median kernel time (us) of fn() over `runs` launches under the library timer."""
    import numpy as np
    times = []
    pkv.timer_enable(True)
    for i in range(runs):
        fn(i)
        ms, n = pkv.timer_read(pkv.PKV_TIMER_MEASURE)
        times.append(ms * 1e3 / max(n, 1))
    pkv.timer_enable(False)
    return float(np.median(times))


def read_ceiling(dev, launch_bytes: int):
    """What this GPU streams with no indirection, from the library's contiguous-read kernel
    with non-temporal loads (as the decode's tile loads): 1 GiB at several launch shapes
    (the best median of 10 runs), and, at the best shape, a read of exactly one decode
    launch's bytes (the same ramp-up and tail per launch as the decode pays), beside the
    same two reads with plain loads. Buffers rotate so that no run finds its input in the
    256 MB Infinity Cache."""
    import torch

    import paged_kv_cache_28_amd as pkv
    n = 1 << 30
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(2)]
    for t in bufs:
        t.fill_(1)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    shapes = {}
    for wpc in (8, 16):
        for lif in (4, 8, 16):
            pkv.measure_read(bufs[0], sink, wpc, lif)            # warm
            us = _median_us(pkv, lambda i: pkv.measure_read(bufs[i % 2], sink, wpc, lif), 10)
            shapes[f"{wpc}w_{lif}l"] = round(n / (us * 1e-6) / 1e9, 1)
    best = max(shapes, key=shapes.get)
    wpc, lif = (int(x[:-1]) for x in best.split("_"))
    us = _median_us(pkv, lambda i: pkv.measure_read(bufs[i % 2], sink, wpc, lif, False), 10)
    plain_1g = round(n / (us * 1e-6) / 1e9, 1)
    del bufs
    m = (launch_bytes + 15) // 16 * 16
    small = [torch.ones(m, dtype=torch.uint8, device=dev) for _ in range(4)]
    same = {}
    for nt in (True, False):
        us = _median_us(pkv, lambda i: pkv.measure_read(small[i % 4], sink, wpc, lif, nt), 24)
        same[nt] = (round(us, 2), round(m / (us * 1e-6) / 1e9, 1))
    del small
    torch.cuda.empty_cache()
    return {"GB/s": same[True][1], "frac_of_peak": round(same[True][1] / HBM_PEAK_GBS, 4),
            "bytes": m, "us": same[True][0], "plain_loads_GB/s": same[False][1],
            "GB/s_1GiB": shapes[best], "plain_loads_GB/s_1GiB": plain_1g, "best_shape": best,
            "by_shape_GB/s_1GiB": shapes,
            "kernel": "pkv_measure_read: contiguous 16-byte non-temporal loads, no arithmetic; "
                      "GB/s is a read of one decode launch's bytes, GB/s_1GiB a 1 GiB read"}


def gather_ceiling(caches, d_tab, d_len, lens, Hkv, P, no_plan, alg_bytes, kv_bytes):
    """The same K/V tiles a decode launch of the last step reads, gathered through its
    block tables with no arithmetic (library kernels), cycling over the layers' pools as
    the decode does: in the single pass's decomposition (one workgroup per (sequence, KV
    head), the step's host plan) and perfectly balanced (equal runs of tiles per wave).
    The balanced rate over the read ceiling is the cost of the indirection itself."""
    import torch

    import paged_kv_cache_28_amd as pkv
    if lens is None:
        return None
    dev = d_tab.device
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    L = len(caches)
    order = None if no_plan else pkv.paged_attention_decode_plan(lens, Hkv)
    kvb = kv_bytes(lens)
    res = {"kv_bytes": kvb, "kernel": "pkv_measure_gather: K and V tiles through the block "
                                      "tables, two in flight per wave, no arithmetic, "
                                      "non-temporal loads (and plain ones for comparison)"}
    bs = int(caches[0][1].shape[3])
    modes = [("per_seq", False)] + ([("balanced", True)] if bs == 16 else [])
    for name, bal in modes:
        for nt, tag in ((True, ""), (False, "_plain_loads")):
            pkv.measure_gather(*caches[0], d_tab, d_len, sink, order, bal, nt)   # warm
            us = _median_us(pkv, lambda i: pkv.measure_gather(*caches[i % L], d_tab, d_len, sink,
                                                              order, bal, nt), 2 * L)
            res[f"{name}{tag}_us"] = round(us, 2)
            res[f"{name}{tag}_GB/s"] = round(kvb / (us * 1e-6) / 1e9, 1)
    best = max(res.get("per_seq_GB/s", 0), res.get("balanced_GB/s", 0))
    res["GB/s"] = best
    res["frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
    return res


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), so the baseline states where it ran."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


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
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "tok_s_per_layer": round(len(lens) * passes / t, 2),
            "seconds": round(t, 2),
            "sample": f"layer 0 of the step, all {len(lens)} sequences "
                      f"({int(lens.sum())} context tokens), decoded {passes}x by the fp64 "
                      f"oracle on {cores} threads"}


if __name__ == "__main__":
    main()
