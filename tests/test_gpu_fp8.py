"""GPU parity of the FP8 (OCP e4m3) KV cache: the HIP path against the CPU oracle.

The page on serving capacity ("Yerel LLM sistemlerinde backpressure ve ölçekleme",
paragraph on KV cache quantisation) gives FP8 KV storage as the way to halve the bytes
per token. Bars:
  * cache codes: bit-exact. Both sides take the same binary32 quotient x / scale and
    round it to the nearest e4m3 value, ties to even, saturating at 448;
  * attention with fp32 output: the 16-bit bars (max |err| <= 2e-3, max|err| / max|ref|
    <= 1e-3) against the oracle's attention over the dequantised cache: the kernels widen
    the codes exactly, so quantisation itself is not part of the error;
  * 16-bit output: the fp32 result rounded once (torch's cast of it, bit for bit), within
    the fp32 bar plus half an output ulp of the oracle;
  * the fused append: caches and outputs bit-exact against the two calls it stands for
    (16-token blocks: the new row's codes go into the newest tile's registers).
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
from test_gpu_parity import RAGGED, TOL, _ulp, check_close

pytestmark = pytest.mark.gpu
AUTO = pkv.PKV_PARTITION_AUTO
W8 = workloads.WORKLOADS["llama8b_fp8"]

SHAPES = {
    "8b-bf16-fp8": dataclasses.replace(W8, num_blocks=0),
    # 32-token blocks: the whole-block kernel in the single pass and partitions of 64 tokens
    "8b-bf16-fp8-bs32": dataclasses.replace(W8, num_blocks=0, block_size=32),
    "f16-d64-g8-fp8": dataclasses.replace(W8, dtype="f16", num_heads=16, num_kv_heads=2,
                                          head_dim=64, k_scale=0.031, v_scale=0.0097),
    "bf16-d128-g16-fp8": dataclasses.replace(W8, num_heads=32, num_kv_heads=2, k_scale=0.02,
                                             v_scale=0.011),
}


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float16


# ------------------------------------------------------------------ cache write
def _special_rows(scale, dtype, hkv, d):
    """Rows holding every tie between neighbouring e4m3 magnitudes (times scale), values
    past the range, infinities, NaN, signed zeros and values below the smallest code."""
    mags = oracle.to_f64(np.arange(0x7F, dtype=np.uint8), "fp8")
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([mids, -mids, [449.0, 464.0, 1000.0, -3e4, np.inf, -np.inf, np.nan,
                                         0.0, -0.0, 2.0 ** -11, -(2.0 ** -12), 2.0 ** -10]])
    x = torch.from_numpy(vals * scale).to(_tdt(dtype))
    n = -(-x.numel() // (hkv * d))
    buf = torch.zeros(n * hkv * d, dtype=x.dtype)
    buf[:x.numel()] = x
    return buf.view(n, hkv, d)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [0.5, 0.0173, 3.0])
def test_fp8_cache_write_is_bit_exact(dtype, scale, device):
    """scale 0.5 keeps x / scale exact, so the ties reach the rounding as ties."""
    hkv, d, nb = 4, 128, 12
    w = dataclasses.replace(W8, dtype=dtype, num_kv_heads=hkv, head_dim=d)
    gen = workloads.rng(77, int(scale * 1000))
    T = 90
    key = workloads.draw_tokens(T, w, gen, std=2.5)
    value = workloads.draw_tokens(T, w, gen, std=2.5)
    sk = _special_rows(scale, dtype, hkv, d)
    key[:sk.shape[0]] = sk
    value[T - sk.shape[0]:] = sk
    # strided key/value: slices of a fused [T][3 * Hkv][d] buffer
    fused = torch.zeros((T, 3 * hkv, d), dtype=key.dtype)
    fused[:, :hkv], fused[:, 2 * hkv:] = key, value
    slots = np.random.default_rng(5).permutation(nb * 16)[:T].astype(np.int32)
    slots[::7] = -1
    kc, vc = pkv.alloc_caches(nb, hkv, d, "fp8", device, fill=0x5A)
    fd = fused.to(device)
    pkv.reshape_and_cache_fp8(fd[:, :hkv], fd[:, 2 * hkv:], kc, vc,
                              torch.from_numpy(slots).to(device), scale, scale * 1.5)
    okc, ovc = oracle.empty_caches(nb, hkv, d, "fp8", fill_nan=False)
    okc[:], ovc[:] = 0x5A, 0x5A
    oracle.cache_write(key, value, okc, ovc, slots, dtype, cache_dtype="fp8", k_scale=scale,
                       v_scale=scale * 1.5)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(kc), okc) and np.array_equal(oracle.raw(vc), ovc)


# Both forms of the FP8 write (flat: a thread per 4 dimensions; rows: a wave per 16 tokens
# of a KV head, taken once ceil(T / 16) * Hkv reaches the compute units, 256 on MI355X).
FP8_CW_CASES = [
    ("bf16", 16, 128, 8, 519),    # rows
    ("f16", 8, 64, 8, 517),       # rows
    ("bf16", 32, 128, 4, 1030),   # rows
    ("bf16", 16, 128, 8, 40),     # flat
]


@pytest.mark.parametrize("dtype,bs,d,hkv,T", FP8_CW_CASES)
@pytest.mark.parametrize("pattern", ["consecutive", "scattered"])
def test_fp8_cache_write_forms_are_bit_exact(dtype, bs, d, hkv, T, pattern, device):
    """Consecutive slots from a start inside a block, or a random permutation; the special
    rows (ties, range limits, NaN, zeros) at both ends; strided inputs; negative slots and
    one past the pool write nothing."""
    w = dataclasses.replace(W8, dtype=dtype, num_kv_heads=hkv, head_dim=d, block_size=bs)
    gen = workloads.rng(78, T, bs)
    key = workloads.draw_tokens(T, w, gen, std=2.5)
    value = workloads.draw_tokens(T, w, gen, std=2.5)
    ks, vs = 0.0173, 0.026
    sk = _special_rows(ks, dtype, hkv, d)
    key[:sk.shape[0]] = sk
    sv = _special_rows(vs, dtype, hkv, d)
    value[T - sv.shape[0]:] = sv
    fused = torch.zeros((T, 3 * hkv, d), dtype=key.dtype)
    fused[:, :hkv], fused[:, 2 * hkv:] = key, value
    if pattern == "consecutive":
        start = 3 * bs + 5
        nb = (start + T) // bs + 2
        slots = (start + np.arange(T)).astype(np.int32)
    else:
        nb = 2 * T // bs + 2
        slots = np.random.default_rng(T + bs).permutation(nb * bs)[:T].astype(np.int32)
    slots[::37] = -1
    slots[min(11, T - 1)] = nb * bs + 3
    kc, vc = pkv.alloc_caches(nb, hkv, d, "fp8", device, fill=0x5A, block_size=bs)
    fd = fused.to(device)
    pkv.reshape_and_cache_fp8(fd[:, :hkv], fd[:, 2 * hkv:], kc, vc,
                              torch.from_numpy(slots).to(device), ks, vs)
    okc, ovc = oracle.empty_caches(nb, hkv, d, "fp8", fill_nan=False, block_size=bs)
    okc[:], ovc[:] = 0x5A, 0x5A
    oracle.cache_write(key, value, okc, ovc, np.where(slots >= nb * bs, -1, slots), dtype,
                       cache_dtype="fp8", k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(kc), okc) and np.array_equal(oracle.raw(vc), ovc)


def test_fp8_pool_slots_tables_and_caches_are_bit_exact(device):
    w = SHAPES["8b-bf16-fp8"]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    assert np.array_equal(gb.prompt_slots, ob.prompt_slots)
    assert np.array_equal(gb.tables, ob.tables) and np.array_equal(gb.lens, ob.lens)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(gb.k_cache), ob.k_cache)
    assert np.array_equal(oracle.raw(gb.v_cache), ob.v_cache)


# ------------------------------------------------------------------ decode
def _oracle_decode(ob, w):
    return oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype,
                         kv_dtype="fp8", k_scale=w.k_scale, v_scale=w.v_scale)


@pytest.mark.parametrize("P", [0, 64, AUTO], ids=["single", "p64", "auto"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_fp8_decode_matches_oracle(name, P, device):
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    out, _ = gpu_batch.run_decode(gb, w, P)
    torch.cuda.synchronize()
    check_close(out.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype, f"{name} P={P}")


@pytest.mark.parametrize("P", [0, AUTO], ids=["single", "auto"])
def test_fp8_decode_16bit_output(P, device):
    """bf16 output: the fp32 result rounded to nearest even once, so it equals torch's
    cast of the fp32 output bit for bit and lies within the fp32 bar plus half an output
    ulp of the oracle."""
    w = SHAPES["8b-bf16-fp8"]
    ob = paged_batch.build(w, lens=RAGGED)
    gb = gpu_batch.build(ob, device)
    out_lp, _ = gpu_batch.run_decode(gb, w, P, out_dtype=torch.bfloat16)
    out_32, _ = gpu_batch.run_decode(gb, w, P, out_dtype=torch.float32)
    assert torch.equal(out_lp, out_32.to(torch.bfloat16))
    got = out_lp.cpu().double().numpy()
    err = np.abs(got - _oracle_decode(ob, w))
    assert np.all(err <= TOL["bf16"] + 0.5 * _ulp(got, "bf16")), err.max()


@pytest.mark.parametrize("P", [0, AUTO], ids=["single", "auto"])
def test_fp8_decode_of_every_finite_code(P, device):
    """Caches of uniformly drawn codes (every finite e4m3 value, NaN codes excluded):
    checks the kernels' widening of all 254 codes, including subnormals and +-448."""
    hq, hkv, d, B, n = 16, 4, 128, 6, 200
    gen = torch.Generator().manual_seed(2028)
    nb = B * 13 + 5
    codes = torch.randint(0, 254, (2, nb, hkv, d, 16), generator=gen, dtype=torch.int32)
    codes = torch.where(codes >= 0x7F, codes + 1, codes).to(torch.uint8)   # skip 0x7F, 0xFF
    kc = codes[0].reshape(nb, hkv, d // 16, 16, 16).contiguous()
    vc = codes[1].contiguous()
    assert set(torch.unique(kc).tolist()) | set(torch.unique(vc).tolist()) == \
        set(range(256)) - {0x7F, 0xFF}
    perm = np.random.default_rng(4).permutation(nb).astype(np.int32)
    lens = np.array([n, 1, 17, 96, 0, 150], np.int32)
    tables = np.full((B, 13), -1, np.int32)
    k = 0
    for b in range(B):
        m = -(-int(lens[b]) // 16)
        tables[b, :m] = perm[k:k + m]
        k += m
    q = (torch.randn((B, hq, d), generator=gen) * 0.5).to(torch.bfloat16)
    ks, vs, scale = 1.0 / 448, 0.37, 1.0 / np.sqrt(d)
    ref = oracle.decode(q, kc, vc, tables, lens, scale, "bf16", kv_dtype="fp8", k_scale=ks,
                        v_scale=vs)
    out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device=device)
    parts = None
    if P != 0:
        parts = pkv.alloc_partials(B, hq, d, pkv.max_partitions_for(13, P), device)
    pkv.decode(out, q.to(device), kc.to(device), vc.to(device), torch.from_numpy(tables).to(device),
               torch.from_numpy(lens).to(device), scale, P, parts, kv_scales=(ks, vs))
    torch.cuda.synchronize()
    # values span +-448 v_scale: the bars are taken relative to the largest one
    top = 448 * vs
    check_close(out.cpu().double().numpy() / top, ref / top, "bf16", f"every code P={P}")


# ------------------------------------------------------------------ fused append
def _run(gb, w, P, out_dtype, append):
    B, Hq, d = gb.q.shape
    dev = gb.q.device
    out = gpu_batch.guarded_full((B, Hq, d), float("nan"), out_dtype, dev)
    parts = None
    if P != 0:
        parts = gpu_batch.guarded_partials(B, Hq, d, pkv.max_partitions_for(gb.tables.shape[1], P,
                                                                            w.block_size), dev)
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, P, parts,
               append=append, kv_scales=(w.k_scale, w.v_scale))
    gpu_batch.check_guards()
    return out


@pytest.mark.parametrize("P", [0, 64, AUTO], ids=["single", "p64", "auto"])
@pytest.mark.parametrize("name", ["8b-bf16-fp8", "f16-d64-g8-fp8", "8b-bf16-fp8-bs32"])
def test_fp8_fused_append_equals_two_calls_and_oracle(name, P, device):
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    res = []
    for fused in (False, True):
        gb = gpu_batch.build(ob, device, write_new=False)
        nk, nv = ob.new_k.to(device), ob.new_v.to(device)
        slots = torch.from_numpy(gb.new_slots).to(device)
        if fused:
            out = _run(gb, w, P, torch.float32, (nk, nv, slots))
        else:
            pkv.reshape_and_cache_fp8(nk, nv, gb.k_cache, gb.v_cache, slots, w.k_scale, w.v_scale)
            out = _run(gb, w, P, torch.float32, None)
        res.append((out, gb.k_cache, gb.v_cache))
    (o2, k2, v2), (of, kf, vf) = res
    assert torch.equal(kf, k2) and torch.equal(vf, v2)
    assert np.array_equal(oracle.raw(kf), ob.k_cache) and np.array_equal(oracle.raw(vf), ob.v_cache)
    # the fused kernel quantises the new row to the same codes and puts them into the
    # newest tile's registers, so it sums what the two-call path reads back, in its order
    assert torch.isfinite(of).all()
    assert torch.equal(of.view(torch.int32), o2.view(torch.int32)), (of.double() - o2.double()).abs().max().item()
    check_close(of.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype, f"{name} fused P={P}")


# ------------------------------------------------------------------ argument checks
def test_fp8_entry_points_reject_bad_scales_and_types(device):
    w = SHAPES["8b-bf16-fp8"]
    kc, vc = pkv.alloc_caches(4, w.num_kv_heads, w.head_dim, "fp8", device, fill=0)
    key = torch.zeros((2, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=device)
    slots = torch.zeros(2, dtype=torch.int32, device=device)
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))):
        with pytest.raises(pkv.PkvError) as e:
            pkv.reshape_and_cache_fp8(key, key, kc, vc, slots, ks, vs)
        assert e.value.code == pkv.PKV_EINVAL
    with pytest.raises(pkv.PkvError) as e:
        pkv.reshape_and_cache_fp8(key.float(), key.float(), kc, vc, slots, 1.0, 1.0)
    assert e.value.code == pkv.PKV_ENOTSUP
    q = torch.zeros((2, w.num_heads, w.head_dim), dtype=torch.float32, device=device)
    out = torch.zeros_like(q)
    tab = torch.zeros((2, 1), dtype=torch.int32, device=device)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_fp8(out, q, kc, vc, tab, slots, 0.1, 1.0, 1.0)
    assert e.value.code == pkv.PKV_ENOTSUP
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_fp8(out, q.bfloat16(), kc, vc, tab, slots, 0.1, 0.0, 1.0)
    assert e.value.code == pkv.PKV_EINVAL
