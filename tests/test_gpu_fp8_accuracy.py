"""What an FP8 KV cache costs in accuracy, measured against the unquantised K/V.

The page on serving capacity ("Yerel LLM sistemlerinde backpressure ve ölçekleme", the
paragraph on KV cache quantisation) gives FP8 storage as the way to halve the bytes per
token and warns that it can lose accuracy on long contexts, so it should be measured on
one's own data first. The other FP8 tests compare the kernels with the oracle's attention
over the *dequantised* codes (the kernels are exact there); this one compares the FP8 path
with the fp64 oracle over the original bf16 K/V, i.e. it includes the quantisation error,
next to the same figures for a bf16 cache, at context lengths from 128 to 131,072 tokens:
  * the 8B shape: K/V ~ N(0, 1), q ~ N(0, 1), k_scale 0.015, v_scale 0.0125 (the
    llama8b_fp8 workload's scales);
  * the long-context shape: K/V ~ N(0, 0.5^2), scales halved (the same codes per standard
    deviation).
Reported per length: max|err| and max|err| / max|ref| over every output row, and the rms
error. The bars asserted are sanity bounds only (FP8 error above the bf16 cache's, and below a
quarter of the output scale: e4m3 keeps 3 mantissa bits, so single values are off by up to
6%); the figures themselves are the result, printed and written to
gpurun_out/fp8_accuracy.json when that folder exists.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_28_amd as pkv
import workloads

pytestmark = pytest.mark.gpu
W8 = workloads.WORKLOADS["llama8b_fp8"]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RESULTS = {}

# (shape name, workload, context lengths, K/V std, scale factor of the FP8 scales)
CASES = [("8b", W8, [128, 512, 2048, 8192, 32768], 1.0),
         ("long", dataclasses.replace(W8, kv_std=0.5), [32768, 131072], 0.5)]


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _one_length(w, n, std_mult, device, seed):
    """One sequence of n tokens (B = 1, all heads): bf16 K/V drawn on the host, written to a
    bf16 cache and to an FP8 cache through the library; both decoded; the oracle attends
    over the bf16 K/V themselves (no quantisation)."""
    Hq, Hkv, d, bs = w.num_heads, w.num_kv_heads, w.head_dim, 16
    ks, vs = w.k_scale * std_mult, w.v_scale * std_mult
    gen = workloads.rng(w.seed, 90, seed)
    k = workloads.draw_tokens(n, w, gen)
    v = workloads.draw_tokens(n, w, gen)
    q = workloads.draw_q(w, gen, batch=1)
    nb = -(-n // bs)
    perm = gen.permutation(nb).astype(np.int32)
    slots = (perm[np.arange(n) // bs] * bs + np.arange(n) % bs).astype(np.int32)
    tables = perm[None, :]
    lens = np.array([n], np.int32)
    dev = lambda x: torch.from_numpy(x).to(device)   # noqa: E731
    outs = {}
    for cache in ("bf16", "fp8"):
        kc, vc = pkv.alloc_caches(nb, Hkv, d, cache, device, fill=0)
        kd, vd = k.to(device), v.to(device)
        if cache == "fp8":
            pkv.reshape_and_cache_fp8(kd, vd, kc, vc, dev(slots), ks, vs)
        else:
            pkv.reshape_and_cache(kd, vd, kc, vc, dev(slots))
        out = torch.empty((1, Hq, d), dtype=torch.float32, device=device)
        pkv.decode(out, q.to(device), kc, vc, dev(tables), dev(lens), w.scale, 0,
                   kv_scales=(ks, vs) if cache == "fp8" else None)
        torch.cuda.synchronize()
        outs[cache] = out.cpu().double().numpy()[0]
        del kc, vc
    # the reference: every query head over the unquantised rows of its KV head
    qf = oracle.to_f64(q, w.dtype)[0]
    K, V = oracle.to_f64(k, w.dtype), oracle.to_f64(v, w.dtype)
    ref = np.stack([oracle.attend(qf[h], K[:, h // w.group], V[:, h // w.group], w.scale)[0]
                    for h in range(Hq)])
    top = float(np.abs(ref).max())
    row = {"n": n, "max_abs_ref": top}
    for cache, o in outs.items():
        err = np.abs(o - ref)
        row[cache] = {"max_err": float(err.max()), "norm_err": float(err.max() / top),
                      "rms_err": float(np.sqrt(np.mean(err ** 2)))}
    return row


@pytest.mark.parametrize("name,w,lengths,std_mult", CASES, ids=[c[0] for c in CASES])
def test_fp8_cache_accuracy_against_unquantised_kv(name, w, lengths, std_mult, device):
    rows = []
    for i, n in enumerate(lengths):
        r = _one_length(w, n, std_mult, device, seed=i)
        rows.append(r)
        RESULTS[name] = rows
        print(f"{name} n={n}: max|ref| {r['max_abs_ref']:.3e}; bf16 cache max|err| "
              f"{r['bf16']['max_err']:.2e} (norm {r['bf16']['norm_err']:.2e}); fp8 cache max|err| "
              f"{r['fp8']['max_err']:.2e} (norm {r['fp8']['norm_err']:.2e}, rms "
              f"{r['fp8']['rms_err']:.2e})", flush=True)
        assert r["bf16"]["max_err"] <= 2e-3 and r["bf16"]["norm_err"] <= 1e-3
        assert r["fp8"]["max_err"] > r["bf16"]["max_err"]
        assert r["fp8"]["norm_err"] < 0.25
    out_dir = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(out_dir):
        with open(os.path.join(out_dir, "fp8_accuracy.json"), "w") as fh:
            json.dump(RESULTS, fh, indent=1)
