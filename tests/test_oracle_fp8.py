"""Pins for the oracle's FP8 KV cache, each against something other than the oracle.

The page on serving capacity ("Yerel LLM sistemlerinde backpressure ve ölçekleme",
paragraph on KV cache quantisation) says that FP8 storage halves the bytes per token
and may cost accuracy on long contexts. Format and scaling are our reading: OCP e4m3
(bias 7, 3 mantissa bits, no infinities, largest finite 448), one scale per tensor for
K and one for V, quantisation of x / scale in binary32 to the nearest finite value with
ties to the even code (so larger magnitudes saturate).

* decoding: every one of the 256 codes against torch's float8_e4m3fn, plus the format's
  closed-form anchor values;
* encoding: the exhaustive round trip, every tie between neighbours, random values in
  range against torch's round-to-nearest-even conversion, saturation;
* quantisation: torch's binary32 division followed by its conversion;
* cache write and gather: numpy's indexing of the documented [d/16][16][16] layout;
* attention over an fp8 cache: torch scaled_dot_product_attention (fp64) on K/V that
  torch dequantises itself, and closed forms that separate the K and V scales.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")


def _torch_decode_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


# ------------------------------------------------------------------ decoding
def test_decode_of_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.to_f64(codes, "fp8")
    ref = _torch_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]   # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))   # -0 at 0x80


def test_decode_closed_forms():
    v = oracle.to_f64(np.array([0x38, 0x7E, 0x01, 0x07, 0x08, 0x40, 0xB8, 0x00, 0x80], np.uint8),
                      "fp8")
    assert v.tolist()[:7] == [1.0, 448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 2.0, -1.0]
    assert v[7] == 0.0 and not np.signbit(v[7]) and v[8] == 0.0 and np.signbit(v[8])


# ------------------------------------------------------------------ encoding
def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.fp8_encode(oracle.to_f64(codes, "fp8")), codes)


def test_ties_go_to_the_even_code_and_neighbours_to_the_nearest():
    mags = oracle.to_f64(np.arange(0x7F, dtype=np.uint8), "fp8")      # 0 .. 448 ascending
    assert np.all(np.diff(mags) > 0)
    for c in range(0x7E):
        lo, hi = mags[c], mags[c + 1]
        mid = (lo + hi) / 2                                            # exact in binary64
        even = c if c % 2 == 0 else c + 1
        got = oracle.fp8_encode(np.array([mid, np.nextafter(mid, 0), np.nextafter(mid, 1e9),
                                          -mid]))
        assert got.tolist() == [even, c, c + 1, 0x80 | even], (c, lo, hi)


def test_encode_matches_torch_in_range():
    gen = np.random.default_rng(8)
    x = np.concatenate([gen.standard_normal(20000) * s for s in (2.0 ** -8, 0.05, 1.0, 60.0)])
    x = np.concatenate([x, gen.uniform(-463.9, 463.9, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_encode(x.astype(np.float64)), ref)


def test_encode_saturates_and_keeps_nan():
    got = oracle.fp8_encode(np.array([464.0, 480.0, 1e30, np.inf, -500.0, -np.inf, np.nan,
                                      -np.nan]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF]


# ------------------------------------------------------------------ quantisation
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("scale", [1.0, 0.0125, 3.7])
def test_quantize_is_binary32_division_then_rounding(dtype, scale):
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    gen = torch.Generator().manual_seed(11)
    x = (torch.randn(30000, generator=gen) * 2.5).to(tdt)
    q32 = x.float() / torch.tensor(scale, dtype=torch.float32)      # IEEE binary32 division
    inr = q32.abs() < 464
    assert inr.float().mean() > 0.5
    ref = q32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.fp8_quantize(x, dtype, scale)
    assert np.array_equal(got[inr.numpy()], ref[inr.numpy()])
    big = ~inr.numpy()
    assert np.all(got[big] == np.where(q32.numpy()[big] > 0, 0x7E, 0xFE))


def test_fp8_halves_bytes_per_token():
    """The page's FP8 claim on the pages' two model shapes: half of the fp16 cost."""
    for L, hkv, d in ((80, 8, 128), (32, 8, 128)):
        assert 2 * oracle.bytes_per_token(L, hkv, d, 1) == oracle.bytes_per_token(L, hkv, d, 2)
    assert oracle.bytes_per_token(80, 8, 128, 1) == 163840       # 327,680 B / 2


# ------------------------------------------------------------------ cache write, gather
def _tokens(T, hkv, d, dtype, seed):
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn((T, hkv, d), generator=gen) * 1.5).to(tdt)


def test_fp8_cache_write_matches_numpy_scatter():
    hkv, d, nb = 2, 64, 6
    k, v = _tokens(20, hkv, d, "bf16", 1), _tokens(20, hkv, d, "bf16", 2)
    slots = np.array([5, 17, -1, 40, 41, 0, 95, -3, 16, 30] + list(range(60, 70)), np.int32)
    ks, vs = 0.0125, 0.02
    kc, vc = oracle.empty_caches(nb, hkv, d, "fp8")
    assert kc.shape == (nb, hkv, d // 16, 16, 16) and vc.shape == (nb, hkv, d, 16)
    assert kc.dtype == np.uint8 and np.all(kc == 0x7F)
    ref_k, ref_v = kc.copy(), vc.copy()
    kq = (k.float() / ks).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vq = (v.float() / vs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), 16)
        for i in range(d):
            ref_k[blk, :, i // 16, off, i % 16] = kq[t, :, i]
            ref_v[blk, :, i, off] = vq[t, :, i]
    oracle.cache_write(k, v, kc, vc, slots, "bf16", cache_dtype="fp8", k_scale=ks, v_scale=vs)
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)


def test_fp8_gather_dequantises_with_each_scale():
    hkv, d, nb = 2, 64, 4
    k, v = _tokens(33, hkv, d, "f16", 3), _tokens(33, hkv, d, "f16", 4)
    order = np.array([2, 0, 3], np.int32)                       # logical block -> physical
    slots = np.array([order[t // 16] * 16 + t % 16 for t in range(33)], np.int32)
    ks, vs = 0.5, 0.03125
    kc, vc = oracle.empty_caches(nb, hkv, d, "fp8")
    oracle.cache_write(k, v, kc, vc, slots, "f16", cache_dtype="fp8", k_scale=ks, v_scale=vs)
    for g in range(hkv):
        K, V = oracle.gather(kc, vc, order, 0, 33, g, hkv, d, "fp8", k_scale=ks, v_scale=vs)
        rk = (k[:, g].float() / ks).to(torch.float8_e4m3fn).double().numpy() * ks
        rv = (v[:, g].float() / vs).to(torch.float8_e4m3fn).double().numpy() * vs
        assert np.array_equal(K, rk) and np.array_equal(V, rv)


# ------------------------------------------------------------------ attention
def _fp8_batch(lens, hq, hkv, d, ks, vs, seed=5):
    """Paged fp8 caches filled through the oracle's cache write from bf16 draws, block
    tables from a seeded permutation. Returns q, caches, tables, lens, logical rows."""
    B = len(lens)
    mb = max(1, max(-(-n // 16) for n in lens))
    nb = sum(-(-n // 16) for n in lens) + 3
    perm = workloads.draw_free_order(nb, np.random.default_rng(seed))
    tables = np.full((B, mb), -1, np.int32)
    kc, vc = oracle.empty_caches(nb, hkv, d, "fp8")
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((B, hq, d), generator=gen).to(torch.bfloat16)
    rows, nxt = [], 0
    for b, n in enumerate(lens):
        nbk = -(-n // 16)
        tables[b, :nbk] = perm[nxt:nxt + nbk]
        nxt += nbk
        k = (torch.randn((n, hkv, d), generator=gen) * 1.3).to(torch.bfloat16)
        v = (torch.randn((n, hkv, d), generator=gen) * 1.3).to(torch.bfloat16)
        slots = np.array([tables[b, t // 16] * 16 + t % 16 for t in range(n)], np.int32)
        oracle.cache_write(k, v, kc, vc, slots, "bf16", cache_dtype="fp8", k_scale=ks, v_scale=vs)
        rows.append((k, v))
    return q, kc, vc, tables, np.array(lens, np.int32), rows


def test_fp8_decode_matches_torch_sdpa_on_torch_dequantised_kv():
    hq, hkv, d, ks, vs = 8, 2, 64, 0.0125, 0.02
    q, kc, vc, tables, lens, rows = _fp8_batch([1, 16, 17, 90], hq, hkv, d, ks, vs)
    out = oracle.decode(q, kc, vc, tables, lens, 0.125, "bf16", kv_dtype="fp8", k_scale=ks,
                        v_scale=vs)
    qf = q.double()
    for b, (k, v) in enumerate(rows):
        n = int(lens[b])
        K = (k.float() / ks).to(torch.float8_e4m3fn).double() * ks      # torch's own path
        V = (v.float() / vs).to(torch.float8_e4m3fn).double() * vs
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[b].view(1, hq, 1, d), K.permute(1, 0, 2).reshape(1, hkv, n, d),
            V.permute(1, 0, 2).reshape(1, hkv, n, d), scale=0.125,
            enable_gqa=True).view(hq, d).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-13)


def test_fp8_one_token_is_its_dequantised_value_row_whatever_k_scale():
    hq, hkv, d = 4, 1, 64
    outs = []
    for ks in (0.01, 0.3):
        q, kc, vc, tables, lens, rows = _fp8_batch([1], hq, hkv, d, ks, 0.02, seed=9)
        outs.append(oracle.decode(q, kc, vc, tables, lens, 0.125, "bf16", kv_dtype="fp8",
                                  k_scale=ks, v_scale=0.02))
        v = rows[0][1]
        rv = (v[0, 0].float() / 0.02).to(torch.float8_e4m3fn).double().numpy() * 0.02
        for h in range(hq):
            assert np.array_equal(outs[-1][0, h], rv)


def test_fp8_partitions_merge_to_single_pass():
    hq, hkv, d, ks, vs = 8, 2, 64, 0.0125, 0.02
    q, kc, vc, tables, lens, _ = _fp8_batch([40, 97, 5], hq, hkv, d, ks, vs, seed=13)
    full = oracle.decode(q, kc, vc, tables, lens, 0.125, "bf16", kv_dtype="fp8", k_scale=ks,
                         v_scale=vs)
    P, maxp = 32, 4
    o, m, l = oracle.decode_partitions(q, kc, vc, tables, lens, 0.125, "bf16", P, maxp,
                                       kv_dtype="fp8", k_scale=ks, v_scale=vs)
    nparts = np.repeat(-(-lens // P), hq)
    merged = oracle.merge(o, m, l, nparts).reshape(full.shape)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-14)
