"""GPU parity of paged_attention_prefill (causal multi-query attention for chunked
prefill) against the oracle on the same seeded inputs.

Bars as for decode: fp32 output max |err| <= 2e-3 and max|err| / max|ref| <= 1e-3 for
16-bit inputs; 16-bit output equal to the RNE cast of the kernel's fp32 result and within
the fp32 bar plus half an output ulp of the oracle. Cases: whole prompts, chunks that end
longer contexts, single-query rows mixed with chunks, chunks longer than their sequence
(zero rows), several shapes of GQA group and head size, and a prompt processed in chunks
over several calls against one call over the whole prompt ("vLLM Nedir? PagedAttention ile
Production LLM Serving", section "Chunked prefill"). The kernel's one-product form takes V in
fp16: bf16 V values at fp16's edges, beyond its range (the pass that redoes such workgroups
with split weights) and in slots past a sequence's end are checked too.
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
from test_gpu_parity import TOL, _ulp, check_close

pytestmark = pytest.mark.gpu
B8 = workloads.WORKLOADS["llama8b"]
SHAPES = {
    "bf16-d128-g4": dataclasses.replace(B8, num_blocks=0),
    "f16-d64-g8": dataclasses.replace(B8, dtype="f16", num_heads=16, num_kv_heads=2, head_dim=64,
                                      num_blocks=0),
    "bf16-d128-g16": dataclasses.replace(B8, num_heads=32, num_kv_heads=2, num_blocks=0),
    "bf16-d64-g1": dataclasses.replace(B8, num_heads=4, num_kv_heads=4, head_dim=64, num_blocks=0),
    # a group that does not divide a wave's 32 columns: 5 tokens of 6 heads, 2 idle columns
    "bf16-d128-g6": dataclasses.replace(B8, num_heads=24, num_kv_heads=4, num_blocks=0),
}
# (context length, chunk length) per sequence
CASES = {
    "whole": [(1, 1), (16, 16), (23, 23), (70, 70), (129, 129)],
    "chunks": [(40, 7), (97, 33), (300, 64), (513, 100), (1000, 17)],
    "mixed": [(700, 1), (64, 64), (250, 1), (431, 150), (33, 1), (2, 2)],
    "short": [(5, 8), (12, 12), (3, 30)],
}


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(w, spec, device, out_dtype=torch.float32, seed=0, scale=None):
    lens = [n for n, _ in spec]
    chunk = [L for _, L in spec]
    ob = paged_batch.build(w, lens=lens, seed_stream=seed)
    gb = gpu_batch.build(ob, device)
    q = workloads.draw_q(w, workloads.rng(w.seed, 60, seed), batch=int(sum(chunk)))
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    out = torch.full(tuple(q.shape), float("nan"), dtype=out_dtype, device=device)
    scale = w.scale if scale is None else scale
    pkv.paged_attention_prefill(out, q.to(device), torch.from_numpy(qs).to(device), gb.k_cache,
                                gb.v_cache, gb.tables_d, gb.lens_d, scale, max(chunk))
    torch.cuda.synchronize()
    ref = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, scale, w.dtype)
    return out, ref


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("name", list(SHAPES))
def test_prefill_matches_oracle(name, case, device):
    out, ref = _run(SHAPES[name], CASES[case], device)
    check_close(out.cpu().double().numpy(), ref, SHAPES[name].dtype, f"{name} {case}")


@pytest.mark.parametrize("name", ["bf16-d128-g4", "f16-d64-g8"])
def test_prefill_16bit_output(name, device):
    w = SHAPES[name]
    tdt = pkv.torch_dtype(w.dtype)
    out_lp, ref = _run(w, CASES["mixed"], device, out_dtype=tdt)
    out_32, _ = _run(w, CASES["mixed"], device)
    assert torch.equal(out_lp, out_32.to(tdt))
    got = out_lp.cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= TOL[w.dtype] + 0.5 * _ulp(got, w.dtype))


@pytest.mark.parametrize("factor", [-1.0, -0.5, 0.0])
def test_prefill_scale_sign_and_zero(factor, device):
    """A negative scale (the kernel flips the queries' signs and scales by |scale|) and a
    zero one (every visible key weighs the same) against the oracle."""
    w = SHAPES["bf16-d128-g4"]
    out, ref = _run(w, CASES["chunks"], device, scale=factor * w.scale)
    check_close(out.cpu().double().numpy(), ref, w.dtype, f"scale x {factor}")


def test_a_prompt_in_chunks_equals_one_pass(device):
    """The same 300-token prompt: written and attended in 64-token chunks over five calls,
    and in one call; every row within the bar of the oracle, and the two GPU results within
    fp32 summation-order differences of each other."""
    w = SHAPES["bf16-d128-g4"]
    n = 300
    ob = paged_batch.build(w, lens=[n])
    gb = gpu_batch.build(ob, device)
    q = workloads.draw_q(w, workloads.rng(w.seed, 61), batch=n).to(device)
    ref = oracle.prefill(q.cpu(), np.array([0, n], np.int32), ob.k_cache, ob.v_cache, ob.tables,
                         ob.lens, w.scale, w.dtype)
    one = torch.empty(q.shape, dtype=torch.float32, device=device)
    pkv.paged_attention_prefill(one, q, torch.tensor([0, n], dtype=torch.int32, device=device),
                                gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, n)
    parts = torch.empty_like(one)
    for c0 in range(0, n, 64):
        c1 = min(n, c0 + 64)
        qs = torch.tensor([0, c1 - c0], dtype=torch.int32, device=device)
        lens = torch.tensor([c1], dtype=torch.int32, device=device)   # the context so far
        pkv.paged_attention_prefill(parts[c0:c1], q[c0:c1], qs, gb.k_cache, gb.v_cache,
                                    gb.tables_d, lens, w.scale, c1 - c0)
    torch.cuda.synchronize()
    for got in (one, parts):
        check_close(got.cpu().double().numpy(), ref, w.dtype, "chunked prompt")
    assert ((one - parts).abs() <= 2e-5 + 1e-5 * one.abs()).all()


def test_prefill_rejects_bad_arguments(device):
    w = SHAPES["bf16-d128-g4"]
    kc, vc = pkv.alloc_caches(4, w.num_kv_heads, w.head_dim, w.dtype, device, fill=0.0)
    q = torch.zeros((3, w.num_heads, w.head_dim), dtype=torch.float32, device=device)
    qs = torch.tensor([0, 3], dtype=torch.int32, device=device)
    tab = torch.zeros((1, 1), dtype=torch.int32, device=device)
    ln = torch.tensor([3], dtype=torch.int32, device=device)
    kc32, vc32 = pkv.alloc_caches(4, w.num_kv_heads, w.head_dim, "f32", device, fill=0.0)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_prefill(q.clone(), q, qs, kc32, vc32, tab, ln, 0.1, 3)
    assert e.value.code == pkv.PKV_ENOTSUP                 # fp32 queries and caches
    with pytest.raises(ValueError, match="k_cache must be"):
        pkv.paged_attention_prefill(q.clone(), q, qs, kc, vc, tab, ln, 0.1, 3)   # f32 over bf16
    qb = q.bfloat16()
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_prefill(qb.half(), qb, qs, kc, vc, tab, ln, 0.1, 3)
    assert e.value.code == pkv.PKV_ENOTSUP                 # out type neither bf16 nor f32
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_prefill(q, qb, qs, kc, vc, tab, ln, float("nan"), 3)
    assert e.value.code == pkv.PKV_EINVAL


# ---- the one-product form: a bf16 cache's V is rounded to fp16 as it is staged, which is
# exact from 2^-17 to 65,280 in magnitude; a wave that meets |v| >= 65,536 (fp16 +-inf) is
# redone by the split-weight pass. Both are checked against the oracle here.

def _set_v(ob, gb, b, pos, dims, value):
    """V of sequence b at position pos, every KV head, the given dims, set to `value` (a
    bf16 number) in the oracle's cache and in the GPU's."""
    bs = ob.w.block_size
    blk, off = int(ob.tables[b][pos // bs]), pos % bs
    bits = int(torch.tensor([value], dtype=torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    for d in dims:
        ob.v_cache[blk, :, d, off] = bits
        gb.v_cache[blk, :, d, off] = value


def _run_edited(w, spec, edits, device, out_dtype=torch.float32, gpu_only=()):
    lens = [n for n, _ in spec]
    chunk = [L for _, L in spec]
    ob = paged_batch.build(w, lens=lens, seed_stream=5)
    gb = gpu_batch.build(ob, device)
    assert np.array_equal(gb.tables, ob.tables)
    for b, pos, dims, value in edits:
        _set_v(ob, gb, b, pos, dims, value)
    for b, pos, dims, value in gpu_only:      # slots past a sequence's end: never read
        bs = w.block_size
        gb.v_cache[int(ob.tables[b][pos // bs]), :, dims, pos % bs] = value
    q = workloads.draw_q(w, workloads.rng(w.seed, 62), batch=int(sum(chunk)))
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    out = torch.full(tuple(q.shape), float("nan"), dtype=out_dtype, device=device)
    pkv.paged_attention_prefill(out, q.to(device), torch.from_numpy(qs).to(device), gb.k_cache,
                                gb.v_cache, gb.tables_d, gb.lens_d, w.scale, max(chunk))
    torch.cuda.synchronize()
    ref = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    return out.cpu().double().numpy(), ref, qs


def _check_seq(got, ref, qs, b, dtype, what, normalised_only=False, half_ulp=False):
    g, r = got[qs[b]:qs[b + 1]], ref[qs[b]:qs[b + 1]]
    slack = 0.5 * _ulp(g, dtype) if half_ulp else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    if not normalised_only:
        assert np.all(err <= TOL[dtype] + slack), f"{what}: max|err| {err.max():.3e}"
    scale = np.abs(r).max()
    assert np.all(err <= 1e-3 * scale + slack), f"{what}: normalised {err.max() / scale:.3e}"


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name", ["bf16-d128-g4", "bf16-d128-g6"])
def test_prefill_v_beyond_fp16_range_is_redone(name, out_dtype, device):
    """V values of 65,536 and -98,304 (beyond fp16) in two sequences: their rows match the
    oracle within the normalised bar (the values make the outputs large), the other
    sequences' rows within the usual bars, in one call."""
    w = SHAPES[name]
    spec = CASES["chunks"]            # contexts 40, 97, 300, 513, 1000
    edits = [(2, 150, [5, 77], 65536.0), (4, 999, [127], -98304.0), (4, 3, [0], 131072.0)]
    got, ref, qs = _run_edited(w, spec, edits, device, out_dtype)
    half = out_dtype != torch.float32
    for b in range(len(spec)):
        _check_seq(got, ref, qs, b, w.dtype, f"{name} seq {b}", normalised_only=b in (2, 4),
                   half_ulp=half)


def test_prefill_v_at_fp16_edges(device):
    """V values that fp16 holds exactly (+-65,280, 2^-14, 2^-17) and ones it rounds
    (1.171875 * 2^-20, 3e-7: fp16 subnormals) take the one-product form; within the bars of
    the oracle."""
    w = SHAPES["bf16-d128-g4"]
    spec = CASES["chunks"]
    edits = [(1, 50, [3, 4], 65280.0), (1, 60, [3], -65280.0), (2, 10, [0, 1, 2], 2.0 ** -14),
             (2, 11, [9], 2.0 ** -17), (3, 400, [100], 1.171875 * 2.0 ** -20), (3, 401, [101], -3e-7)]
    got, ref, qs = _run_edited(w, spec, edits, device)
    for b in range(len(spec)):
        _check_seq(got, ref, qs, b, w.dtype, f"seq {b}", normalised_only=b == 1)


def test_prefill_ignores_huge_values_past_the_sequence(device):
    """Slots after a sequence's last token in its last block hold values beyond fp16 (never
    read by the oracle): the rows stay within the usual bars."""
    w = SHAPES["bf16-d128-g4"]
    spec = CASES["chunks"]            # 97 and 513 end inside a block
    gpu_only = [(1, 97, list(range(128)), 1e6), (1, 100, [7], -3e38), (3, 513, [0, 64], 2e5)]
    got, ref, qs = _run_edited(w, spec, [], device, gpu_only=gpu_only)
    for b in range(len(spec)):
        _check_seq(got, ref, qs, b, w.dtype, f"seq {b}")


@pytest.mark.parametrize("bs", [8, 32])
def test_prefill_v_beyond_fp16_range_at_other_block_sizes(bs, device):
    """The redo pass at 8 and 32 tokens per block (bf16 output): the marked waves' rows
    against the oracle within the normalised bar, the others within the usual bars."""
    w = dataclasses.replace(SHAPES["bf16-d128-g4"], block_size=bs)
    spec = CASES["chunks"]
    edits = [(2, 150, [5, 77], 65536.0), (4, 999, [127], -98304.0), (0, 39, [64], 70144.0)]
    got, ref, qs = _run_edited(w, spec, edits, device, torch.bfloat16)
    for b in range(len(spec)):
        _check_seq(got, ref, qs, b, w.dtype, f"bs {bs} seq {b}", normalised_only=b in (0, 2, 4),
                   half_ulp=True)


def test_prefill_v_beyond_fp16_range_group_of_16(device):
    """The redo pass with a GQA group of 16 (a wave's 32 columns are 2 tokens)."""
    w = SHAPES["bf16-d128-g16"]
    spec = CASES["mixed"]              # single-query rows beside chunks
    edits = [(0, 500, [1], 65536.0), (3, 200, [100, 101], -131072.0)]
    got, ref, qs = _run_edited(w, spec, edits, device)
    for b in range(len(spec)):
        _check_seq(got, ref, qs, b, w.dtype, f"g16 seq {b}", normalised_only=b in (0, 3))


def test_prefill_fp16_cache_extremes(device):
    """An fp16 cache goes through the one-product form directly (its V is fp16 already):
    V at +-65504 and at subnormals against the oracle."""
    w = SHAPES["f16-d64-g8"]
    spec = CASES["chunks"]
    got_edits = []
    for b, pos, dims, value in [(1, 50, [3], 65504.0), (1, 51, [4], -65504.0),
                                (3, 10, [0, 1], 2.0 ** -24), (3, 11, [2], -3 * 2.0 ** -24)]:
        got_edits.append((b, pos, dims, value))
    lens = [n for n, _ in spec]
    chunk = [L for _, L in spec]
    ob = paged_batch.build(w, lens=lens, seed_stream=5)
    gb = gpu_batch.build(ob, device)
    bs = w.block_size
    for b, pos, dims, value in got_edits:
        blk, off = int(ob.tables[b][pos // bs]), pos % bs
        bits = int(torch.tensor([value], dtype=torch.float16).view(torch.int16).item()) & 0xFFFF
        for d in dims:
            ob.v_cache[blk, :, d, off] = bits
            gb.v_cache[blk, :, d, off] = value
    q = workloads.draw_q(w, workloads.rng(w.seed, 63), batch=int(sum(chunk)))
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=device)
    pkv.paged_attention_prefill(out, q.to(device), torch.from_numpy(qs).to(device), gb.k_cache,
                                gb.v_cache, gb.tables_d, gb.lens_d, w.scale, max(chunk))
    torch.cuda.synchronize()
    ref = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    got = out.cpu().double().numpy()
    for b in range(len(spec)):
        _check_seq(got, ref, qs, b, w.dtype, f"f16 seq {b}", normalised_only=b == 1)
