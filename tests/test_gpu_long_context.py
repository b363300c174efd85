"""GPU parity at long contexts: the later block-id segments of the decode kernels, and
the prefill kernel over contexts of up to 30,000 keys.

Each wave of the decode kernels reads the block ids of its work one segment of 64 at a
time (one id per lane) and walks the segment before reading the next. A context reaches a
wave's second segment past:
  * 64 x 4 waves x 16 tokens = 4,096 tokens in the single-pass decode (and in a fixed
    partition longer than that);
  * 64 x 4 x 32 = 8,192 tokens in the whole-block decode at 32 tokens per block (FP8 and
    bf16 caches).
The lengths below put the newest token's tile in segment 1, 2 and 8 of the wave holding
it, so the fused append's substitution of the new row (decided per segment) runs there
too. The prefill kernel reads the ids of each 64-key stage as it stages it; its cases go
past 8,192 keys and include the 30,000-token document of the chunked-prefill workload at
its real chunk size ("vLLM Nedir? PagedAttention ile Production LLM Serving", section
"Chunked prefill"; "Yerel LLM sistemlerinde backpressure ve ölçekleme", section
"4. Prefill ve decode").

Bars as everywhere: fp32 output within 2e-3 of the fp64 oracle and max|err| / max|ref|
<= 1e-3; caches bit-exact.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gpu_batch
import oracle
import paged_batch
import paged_kv_cache_28_amd as pkv
import workloads
from test_gpu_parity import check_close

pytestmark = pytest.mark.gpu
AUTO = pkv.PKV_PARTITION_AUTO
W = workloads.WORKLOADS

# Newest tile jl = (n - 1) // 16 sits in wave jl % 4 at index (jl - wave) // 4 of its
# list, i.e. segment index // 64: 4097 -> 1, 8193 -> 2, 9001 -> 2, 34000 -> 8. 4096 fills
# exactly one segment per wave; the short rows share the launch with the long ones.
LONG = [4097, 9001, 34000, 4096, 8193, 300, 1, 0]
# 32-token blocks, whole blocks: newest block jb = (n - 1) // 32 in segment
# ((jb - jb % 4) // 4) // 64: 8193 -> 1, 9001 -> 1, 34000 -> 4, 8192 fills one segment.
LONG_BS32 = [8193, 9001, 34000, 8192, 700, 1]

SHAPE_8B = dataclasses.replace(W["llama8b"], num_blocks=0)
SHAPE_70B = dataclasses.replace(W["llama70b"], num_blocks=0)
SHAPE_FP8_BS32 = dataclasses.replace(W["llama8b_fp8"], num_blocks=0, block_size=32)
SHAPE_FP8 = dataclasses.replace(W["llama8b_fp8"], num_blocks=0)
SHAPE_8B_BS32 = dataclasses.replace(W["llama8b"], num_blocks=0, block_size=32)


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _oracle_decode(ob, w):
    kw = {}
    if w.cache_dtype == "fp8":
        kw = dict(kv_dtype="fp8", k_scale=w.k_scale, v_scale=w.v_scale)
    return oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype, **kw)


def _decode(gb, w, P, append=None, plan=False):
    B, Hq, d = gb.q.shape
    dev = gb.q.device
    out = gpu_batch.guarded_full((B, Hq, d), float("nan"), torch.float32, dev)
    parts = None
    if P != 0:
        maxp = pkv.max_partitions_for(gb.tables.shape[1], P, w.block_size)
        parts = gpu_batch.guarded_partials(B, Hq, d, maxp, dev)
    order = pkv.paged_attention_decode_plan(gb.lens, w.num_kv_heads) if plan else None
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, P, parts,
               append=append, kv_scales=gpu_batch.kv_scales(w), seq_order=order)
    gpu_batch.check_guards()   # outputs, partials and both caches: nothing written past them
    return out


# (shape, lengths, partition size, host plan): the single pass with and without the plan,
# fixed partitions of 8,192 and 16,384 tokens (two and four segments per wave inside one
# partition; the whole-block kernel takes 16,384 for two), fixed partitions of 512 and
# 1,024 tokens, where the table holds enough partitions (67 and 34 at 34,000 tokens) for
# one partition per wave (also over an FP8 cache), the balanced split, and the 70B shape
# (G = 8, fp16)
DECODE_CASES = [("8b", LONG, 0, True), ("8b", LONG, 0, False), ("8b", LONG, 8192, False),
                ("8b", LONG, 16384, False), ("8b", LONG, 512, False), ("8b", LONG, AUTO, False),
                ("70b", LONG, 0, True), ("70b", LONG, 8192, False), ("70b", LONG, 1024, False),
                ("fp8", LONG, 512, False),
                ("fp8-bs32", LONG_BS32, 0, True), ("fp8-bs32", LONG_BS32, 16384, False),
                ("8b-bs32", LONG_BS32, 0, True), ("8b-bs32", LONG_BS32, 16384, False)]
SHAPES = {"8b": SHAPE_8B, "70b": SHAPE_70B, "fp8": SHAPE_FP8, "fp8-bs32": SHAPE_FP8_BS32,
          "8b-bs32": SHAPE_8B_BS32}


def _ids(cases):
    return [f"{s}-{'auto' if P == AUTO else P}{'-plan' if plan else ''}" for s, _, P, plan in cases]


@pytest.fixture(scope="module")
def batches():
    """Oracle-side batches and their oracle outputs, built once per shape."""
    cache = {}

    def get(shape):
        if shape not in cache:
            w = SHAPES[shape]
            lens = LONG_BS32 if shape.endswith("bs32") else LONG
            ob = paged_batch.build(w, lens=lens, seed_stream=5)
            cache[shape] = (ob, _oracle_decode(ob, w))
        return cache[shape]
    return get


@pytest.mark.parametrize("shape,lens,P,plan", DECODE_CASES, ids=_ids(DECODE_CASES))
def test_long_decode_matches_oracle(shape, lens, P, plan, device, batches):
    w = SHAPES[shape]
    ob, ref = batches(shape)
    gb = gpu_batch.build(ob, device)
    out = _decode(gb, w, P, plan=plan)
    check_close(out.cpu().double().numpy(), ref, w.dtype, f"{shape} P={P} plan={plan}")


APPEND_CASES = [("8b", LONG, 0, True), ("8b", LONG, 0, False), ("8b", LONG, 8192, False), ("8b", LONG, 512, False),
                ("8b", LONG, AUTO, False), ("70b", LONG, AUTO, False), ("8b-bs32", LONG_BS32, AUTO, False),
                ("70b", LONG, 0, True), ("fp8-bs32", LONG_BS32, 0, True),
                ("fp8-bs32", LONG_BS32, 16384, False), ("8b-bs32", LONG_BS32, 0, True),
                ("8b-bs32", LONG_BS32, 16384, False)]


@pytest.mark.parametrize("shape,lens,P,plan", APPEND_CASES, ids=_ids(APPEND_CASES))
def test_long_fused_append_matches_oracle(shape, lens, P, plan, device, batches):
    """The new row is written by the wave that holds the newest tile, which here sits in a
    later segment of that wave's list; that wave then attends to the row from the inputs.
    Caches must equal the oracle's bit for bit afterwards."""
    w = SHAPES[shape]
    ob, ref = batches(shape)
    gb = gpu_batch.build(ob, device, write_new=False)
    append = (ob.new_k.to(device), ob.new_v.to(device), torch.from_numpy(gb.new_slots).to(device))
    out = _decode(gb, w, P, append=append, plan=plan)
    assert np.array_equal(oracle.raw(gb.k_cache), ob.k_cache), "k_cache"
    assert np.array_equal(oracle.raw(gb.v_cache), ob.v_cache), "v_cache"
    check_close(out.cpu().double().numpy(), ref, w.dtype, f"{shape} fused P={P} plan={plan}")


# ---------------------------------------------------------------------- prefill
def _prefill_rows(T, Hq, n_rows, seed):
    """Sampled (row, head) pairs: every head of the first and last rows, and one random
    row and head from each run of 8 consecutive rows (the query tile of 8 tokens at
    G = 4), so every workgroup of the launch is checked."""
    gen = np.random.default_rng(seed)
    rows = {(0, h) for h in range(Hq)} | {(T - 1, h) for h in range(Hq)}
    for t0 in range(0, T, 8):
        r = int(gen.integers(t0, min(T, t0 + 8)))
        rows.add((r, int(gen.integers(Hq))))
    extra = gen.integers(0, T, size=n_rows)
    rows |= {(int(r), int(gen.integers(Hq))) for r in extra}
    return sorted(rows)


PREFILL_CASES = [
    # (context, chunk): contexts past 8,192 keys; the 30,000-token document of the
    # chunked-prefill workload at chunks 3 and 8 of 8 (3,750 queries each)
    (9000, 600), (8193, 64), (11250, 3750), (30000, 3750)]


@pytest.mark.parametrize("n,L", PREFILL_CASES, ids=[f"n{n}-chunk{L}" for n, L in PREFILL_CASES])
def test_long_prefill_matches_oracle(n, L, device):
    w = SHAPE_8B
    ob = paged_batch.build(w, lens=[n], seed_stream=7)
    gb = gpu_batch.build(ob, device)
    q = workloads.draw_q(w, workloads.rng(w.seed, 62, n), batch=L)
    qs = np.array([0, L], np.int32)
    out = gpu_batch.guarded_full(tuple(q.shape), float("nan"), torch.float32, device)
    pkv.paged_attention_prefill(out, q.to(device), torch.from_numpy(qs).to(device), gb.k_cache,
                                gb.v_cache, gb.tables_d, gb.lens_d, w.scale, L)
    gpu_batch.check_guards()
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite output"
    if L * w.num_heads <= 2048:   # every row
        ref = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
        check_close(got, ref, w.dtype, f"prefill n={n} L={L}")
        return
    rows = _prefill_rows(L, w.num_heads, 64, seed=n)
    ref = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype,
                         rows=rows)
    sel = np.array([got[r, h] for r, h in rows])
    check_close(sel, ref, w.dtype, f"prefill n={n} L={L}, {len(rows)} sampled rows")
