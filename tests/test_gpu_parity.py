"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bars
  * slots, block tables, caches: bit-exact;
  * attention with fp32 output: max |err| <= 2e-3 for bf16/fp16 inputs, 1e-5 for fp32
    inputs, and max |err| / max |ref| <= 1e-3;
  * bf16/fp16 output: within one unit in the last place of the oracle rounded to it;
  * partition results: part_out within the same bars; part_max + log(part_sum) (the
    partition's log-sum-exp) within 2e-5 of the oracle's.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import gpu_batch
import oracle
import paged_batch
import workloads

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
AUTO = -1      # PKV_PARTITION_AUTO
TOL = {"f32": 1e-5, "bf16": 2e-3, "f16": 2e-3}


def _shape(name, **kw):
    base = W["tiny"] if name == "tiny" else W["llama8b"]
    return dataclasses.replace(base, num_blocks=0, **kw) if name != "tiny" else \
        dataclasses.replace(base, **kw)


SHAPES = {
    "tiny-f32": _shape("tiny"),
    "8b-bf16": _shape("8b"),
    "70b-f16": dataclasses.replace(W["llama70b"], num_blocks=0),
    "bf16-d64-g1": _shape("8b", num_heads=8, num_kv_heads=8, head_dim=64),
    "f16-d64-g16": _shape("8b", dtype="f16", num_heads=32, num_kv_heads=2, head_dim=64),
    "bf16-d128-g16": _shape("8b", num_heads=32, num_kv_heads=2),
    "f32-d128-g8": _shape("tiny", num_heads=16, num_kv_heads=2, head_dim=128, num_blocks=0),
}
RAGGED = [0, 1, 2, 15, 16, 17, 31, 33, 100, 255, 256, 257, 700]


def check_close(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = TOL[dtype]
    bad = np.argwhere(err > tol)
    assert err.max() <= tol, f"{what}: max|err| {err.max():.3e} > {tol} at {bad[:5].tolist()}"
    scale = np.abs(ref).max()
    if scale > 0:
        assert err.max() / scale <= 1e-3, f"{what}: normalised error {err.max() / scale:.3e}"


def _round_to(ref, dtype):
    t = torch.from_numpy(ref)
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float16).to(torch.float64).numpy()


def _ulp(x, dtype):
    mant = 7 if dtype == "bf16" else 10
    a = np.maximum(np.abs(x), 2.0 ** (-126 if dtype == "bf16" else -14))
    return 2.0 ** (np.floor(np.log2(a)) - mant)


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


# ------------------------------------------------------------------ cache write
@pytest.mark.parametrize("name", ["tiny-f32", "8b-bf16", "70b-f16"])
def test_slots_tables_and_caches_are_bit_exact(name, device):
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    assert np.array_equal(gb.prompt_slots, ob.prompt_slots)
    assert np.array_equal(gb.new_slots, ob.new_slots)
    assert np.array_equal(gb.tables, ob.tables) and np.array_equal(gb.lens, ob.lens)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(gb.k_cache).view(np.uint8), ob.k_cache.view(np.uint8))
    assert np.array_equal(oracle.raw(gb.v_cache).view(np.uint8), ob.v_cache.view(np.uint8))


def test_cache_write_with_token_stride_and_skipped_slots(device):
    """key/value as a strided slice of a fused buffer; negative slots write nothing."""
    w = SHAPES["8b-bf16"]
    gen = workloads.rng(91)
    T, nb = 40, 8
    fused = workloads.draw_tokens(T, dataclasses.replace(w, num_kv_heads=3 * w.num_kv_heads), gen)
    key, value = fused[:, :w.num_kv_heads], fused[:, w.num_kv_heads:2 * w.num_kv_heads]
    slots = np.random.default_rng(3).permutation(nb * 16)[:T].astype(np.int32)
    slots[::5] = -1
    import paged_kv_cache_28_amd as pkv
    kc, vc = pkv.alloc_caches(nb, w.num_kv_heads, w.head_dim, w.dtype, device, fill=0.0)
    fd = fused.to(device)
    pkv.reshape_and_cache(fd[:, :w.num_kv_heads], fd[:, w.num_kv_heads:2 * w.num_kv_heads], kc,
                          vc, torch.from_numpy(slots).to(device))
    okc, ovc = oracle.empty_caches(nb, w.num_kv_heads, w.head_dim, w.dtype, fill_nan=False)
    oracle.cache_write(key.contiguous(), value.contiguous(), okc, ovc, slots, w.dtype)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(kc), okc) and np.array_equal(oracle.raw(vc), ovc)


# The library picks between two kernels by size: a flat one (a thread per 16-byte group,
# decode steps) and a rows one (a wave per 16 tokens of a KV head, prompts and chunks)
# once ceil(T / 16) * Hkv reaches the device's compute units (256 on MI355X). The cases
# below sit on either side of that line for each element size and block size.
CW_CASES = [
    ("bf16", 16, 128, 8, 519),    # rows: 33 tiles x 8 heads
    ("f16", 8, 64, 8, 517),
    ("bf16", 32, 128, 8, 530),
    ("f32", 16, 128, 2, 2055),    # rows with 4-byte elements: 129 tiles x 2 heads
    ("f32", 32, 64, 4, 1030),
    ("f32", 8, 128, 1, 40),       # flat
    ("bf16", 16, 128, 8, 40),     # flat
]


@pytest.mark.parametrize("dtype,bs,d,hkv,T", CW_CASES)
@pytest.mark.parametrize("pattern", ["consecutive", "scattered"])
def test_cache_write_forms_are_bit_exact(dtype, bs, d, hkv, T, pattern, device):
    """Consecutive slots from a start inside a block (a prompt), or a random permutation;
    key/value are strided slices of a fused buffer; some slots are negative and one lies
    past the pool (both write nothing)."""
    import paged_kv_cache_28_amd as pkv
    w = dataclasses.replace(W["llama8b"], num_kv_heads=3 * hkv, head_dim=d, dtype=dtype,
                            block_size=bs)
    fused = workloads.draw_tokens(T, w, workloads.rng(92, T, bs))
    key, value = fused[:, :hkv], fused[:, hkv:2 * hkv]
    if pattern == "consecutive":
        start = 3 * bs + 5
        nb = (start + T) // bs + 2
        slots = (start + np.arange(T)).astype(np.int32)
    else:
        nb = 2 * T // bs + 2
        slots = np.random.default_rng(T + bs).permutation(nb * bs)[:T].astype(np.int32)
    slots[::37] = -1
    slots[min(11, T - 1)] = nb * bs + 3
    kc, vc = pkv.alloc_caches(nb, hkv, d, dtype, device, fill=0.0, block_size=bs)
    fd = fused.to(device)
    pkv.reshape_and_cache(fd[:, :hkv], fd[:, hkv:2 * hkv], kc, vc,
                          torch.from_numpy(slots).to(device))
    okc, ovc = oracle.empty_caches(nb, hkv, d, dtype, fill_nan=False, block_size=bs)
    oracle.cache_write(key.contiguous(), value.contiguous(), okc, ovc,
                       np.where(slots >= nb * bs, -1, slots), dtype)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(kc), okc) and np.array_equal(oracle.raw(vc), ovc)


# ------------------------------------------------------------------- decode
@pytest.mark.parametrize("name", list(SHAPES))
def test_single_pass_decode_matches_oracle(name, device):
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    out, _ = gpu_batch.run_decode(gb, w, 0)
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    got = out.cpu().double().numpy()
    check_close(got, ref, w.dtype, name)
    assert np.array_equal(got[0], np.zeros_like(got[0]))       # n = 0 -> zero row


@pytest.mark.parametrize("name", ["8b-bf16", "70b-f16", "tiny-f32", "f16-d64-g16", "bf16-d128-g16"])
@pytest.mark.parametrize("P", [16, 32, 256, 512])
def test_partitioned_decode_and_reduce_match_oracle(name, P, device):
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    out, (po, pm, ps) = gpu_batch.run_decode(gb, w, P)
    torch.cuda.synchronize()
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    check_close(out.cpu().double().numpy(), ref, w.dtype, f"{name} P={P}")
    maxp = po.shape[2]
    o, m, l = oracle.decode_partitions(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens,
                                       w.scale, w.dtype, P, maxp)
    B, Hq = len(ob.lens), w.num_heads
    po, pm, ps = (t.cpu().double().numpy() for t in (po, pm, ps))
    for b in range(B):
        npart = -(-int(ob.lens[b]) // P)
        if npart <= 1:
            continue                       # written straight to out
        rows = slice(b * Hq, (b + 1) * Hq)
        check_close(po[b, :, :npart], o[rows, :npart], w.dtype, f"part_out b={b}")
        # (part_max, part_sum) is a reference point and the sum of exponentials
        # relative to it: unique is their log-sum-exp, and the reference lies within
        # 8 ln 2 below the partition's largest logit.
        lse = pm[b, :, :npart] + np.log(ps[b, :, :npart])
        np.testing.assert_allclose(lse, m[rows, :npart] + np.log(l[rows, :npart]), rtol=0,
                                   atol=2e-5)
        assert np.all(pm[b, :, :npart] <= m[rows, :npart] + 1e-5)
        assert np.all(pm[b, :, :npart] >= m[rows, :npart] - 8 * math.log(2) - 1e-5)


@pytest.mark.parametrize("name", ["8b-bf16", "70b-f16"])
@pytest.mark.parametrize("P", [0, 64, AUTO])
def test_low_precision_output(name, P, device):
    """bf16/fp16 output: the same accumulation as the fp32 output, rounded to nearest even
    once at the end. So (a) it equals torch's RNE cast of our fp32 output bit for bit, and
    (b) it lies within the fp32 bar plus half an output ulp of the fp64 oracle."""
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    out_lp, _ = gpu_batch.run_decode(gb, w, P, out_dtype=gb.q.dtype)
    out_32, _ = gpu_batch.run_decode(gb, w, P, out_dtype=torch.float32)
    assert torch.equal(out_lp, out_32.to(gb.q.dtype))
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    got = out_lp.cpu().double().numpy()
    bound = TOL[w.dtype] + 0.5 * _ulp(got, w.dtype)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


@pytest.mark.parametrize("name", ["8b-bf16", "tiny-f32"])
@pytest.mark.parametrize("P", [0, 32, AUTO])
def test_block_relabelling_leaves_gpu_output_bits_unchanged(name, P, device):
    w = SHAPES[name]
    if P == AUTO and w.dtype == "f32":
        pytest.skip("the balanced split is built for fp16/bf16 only")
    ob = paged_batch.build(w, lens=[3, 16, 49, 120, 300])
    gb = gpu_batch.build(ob, device)
    base, _ = gpu_batch.run_decode(gb, w, P)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(ob.num_blocks)).to(device)
    kc = torch.empty_like(gb.k_cache)
    vc = torch.empty_like(gb.v_cache)
    kc[perm] = gb.k_cache
    vc[perm] = gb.v_cache
    tables = torch.where(gb.tables_d >= 0, perm[gb.tables_d.clamp(min=0).long()].int(),
                         gb.tables_d)
    gb2 = dataclasses.replace(gb, k_cache=kc, v_cache=vc, tables_d=tables.contiguous())
    got, _ = gpu_batch.run_decode(gb2, w, P)
    assert torch.equal(base, got)


def test_poisoned_slots_never_reach_the_result(device):
    """The same batch with every unwritten slot NaN and with every unwritten slot 0."""
    w = SHAPES["8b-bf16"]
    ob = paged_batch.build(w, lens=[1, 17, 30, 47, 129])
    a, _ = gpu_batch.run_decode(gpu_batch.build(ob, device, fill=float("nan")), w, 32)
    b, _ = gpu_batch.run_decode(gpu_batch.build(ob, device, fill=0.0), w, 32)
    assert torch.isfinite(a).all() and torch.equal(a, b)


def test_closed_forms_on_gpu(device):
    """One token -> its V row exactly; a zero query -> the mean of V."""
    w = SHAPES["8b-bf16"]
    ob = paged_batch.build(w, lens=[1, 1, 64, 200])
    ob.q[2:] = 0
    gb = gpu_batch.build(ob, device)
    out, _ = gpu_batch.run_decode(gb, w, 0)
    got = out.cpu().double().numpy()
    G = w.group
    for b in range(4):
        K, V = ob.logical_kv(b)
        for h in range(w.num_heads):
            if b < 2:
                assert np.array_equal(got[b, h], V[0, h // G])
            else:
                np.testing.assert_allclose(got[b, h], V[:, h // G].mean(axis=0), atol=1e-5)


@pytest.mark.parametrize("P", [256, AUTO])
def test_repeated_calls_are_deterministic(P, device):
    w = SHAPES["70b-f16"]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    a, _ = gpu_batch.run_decode(gb, w, P)
    b, _ = gpu_batch.run_decode(gb, w, P)
    assert torch.equal(a, b)


# ------------------------------------------------------------- balanced split
SPLIT_LENS = {
    "ragged": RAGGED,
    "one-long": [5000],
    "many-short": [1, 2, 3, 16, 17, 18, 31, 32, 33] * 7,
    "empty-mixed": [0, 0, 40, 0, 1, 0],
}


@pytest.mark.parametrize("name", ["8b-bf16", "70b-f16", "f16-d64-g16", "bf16-d64-g1", "bf16-d128-g16"])
@pytest.mark.parametrize("lens", list(SPLIT_LENS))
@pytest.mark.parametrize("maxp", [2, 5, None])
def test_balanced_split_matches_oracle(name, lens, maxp, device):
    """The balanced split over several length mixes and piece bounds; when pieces are
    few (maxp 2) every piece is long, when the bound is loose many pieces are short."""
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=SPLIT_LENS[lens])
    gb = gpu_batch.build(ob, device)
    out, _ = gpu_batch.run_decode(gb, w, AUTO, max_partitions=maxp)
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    got = out.cpu().double().numpy()
    check_close(got, ref, w.dtype, f"{name} {lens} maxp={maxp}")
    for b in np.flatnonzero(ob.lens == 0):
        assert np.array_equal(got[b], np.zeros_like(got[b]))


# ------------------------------------------------------------- batch sizes
@pytest.mark.parametrize("B,P", [(256, 0), (300, 0), (300, 64), (1024, AUTO)])
def test_many_sequences(B, P, device):
    """Batch sizes around the single pass's length-ordering limit (256 sequences) and
    the balanced split's maximum (1024), with short ragged lengths including empty ones."""
    w = SHAPES["8b-bf16"]
    lens = workloads.rng(77, B).integers(0, 160, size=B, endpoint=True)
    ob = paged_batch.build(w, lens=lens)
    gb = gpu_batch.build(ob, device)
    out, _ = gpu_batch.run_decode(gb, w, P)
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    got = out.cpu().double().numpy()
    check_close(got, ref, w.dtype, f"B={B} P={P}")
    for b in np.flatnonzero(ob.lens == 0):
        assert np.array_equal(got[b], np.zeros_like(got[b]))
