"""Pins for the oracle's paging: cache write, gather, and paged decode.

* The cache layout is checked through numpy's own indexing of an array of the
  documented shape, not through the oracle's index formula.
* Paged decode equals attention over the contiguous logical K/V, bit for bit: the
  math is unchanged, only where K and V are read from changes ("vLLM ve Triton ile
  maliyet optimizasyonu", §03 Yöntem, closing paragraphs).
* Blocks need not be adjacent: relabelling the physical blocks (moving their data)
  leaves every output bit unchanged (same page, §03 steps 1-2; "vLLM Nedir? ...",
  section "PagedAttention").
* Bytes past a sequence's length, in its partly filled last block or in unused
  blocks, never reach the result (they are NaN here).
"""
import math

import numpy as np
import pytest

import oracle
import paged_batch
import workloads

TINY = workloads.WORKLOADS["tiny"]


def _w(**kw):
    import dataclasses
    return dataclasses.replace(TINY, **kw)


SHAPES = [
    _w(),                                                          # fp32, G=4, d=64
    _w(name="bf16", dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128, num_blocks=0),
    _w(name="f16", dtype="f16", num_heads=8, num_kv_heads=1, head_dim=64, num_blocks=0),
]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_cache_write_matches_numpy_scatter(w):
    ob = paged_batch.build(w, lens=[1, 16, 17, 40, 0, 33])
    x = 4 if w.dtype == "f32" else 8
    kc, vc = oracle.empty_caches(ob.num_blocks, w.num_kv_heads, w.head_dim, w.dtype)
    kv = kc.reshape(ob.num_blocks, w.num_kv_heads, w.head_dim // x, 16, x)
    vv = vc.reshape(ob.num_blocks, w.num_kv_heads, w.head_dim, 16)
    pk, pv = oracle.raw(ob.prompt_k), oracle.raw(ob.prompt_v)
    nk, nv = oracle.raw(ob.new_k), oracle.raw(ob.new_v)
    for rows_k, rows_v, slots in ((pk, pv, ob.prompt_slots), (nk, nv, ob.new_slots)):
        for t, s in enumerate(slots):
            if s < 0:
                continue
            blk, off = divmod(int(s), 16)
            for i in range(w.head_dim):
                kv[blk, :, i // x, off, i % x] = rows_k[t, :, i]
                vv[blk, :, i, off] = rows_v[t, :, i]
    assert np.array_equal(kc.view(np.uint8), ob.k_cache.view(np.uint8))
    assert np.array_equal(vc.view(np.uint8), ob.v_cache.view(np.uint8))


def test_cache_write_skips_negative_slots_and_rejects_out_of_pool():
    w = TINY
    kc, vc = oracle.empty_caches(8, w.num_kv_heads, w.head_dim, w.dtype, fill_nan=False)
    gen = workloads.rng(5)
    k = workloads.draw_tokens(3, w, gen)
    v = workloads.draw_tokens(3, w, gen)
    before_k, before_v = kc.copy(), vc.copy()
    oracle.cache_write(k, v, kc, vc, np.array([-1, -5, -1], np.int32), w.dtype)
    assert np.array_equal(kc, before_k) and np.array_equal(vc, before_v)
    with pytest.raises(ValueError):
        oracle.cache_write(k, v, kc, vc, np.array([0, 8 * 16, 3], np.int32), w.dtype)
    assert np.array_equal(kc, before_k) and np.array_equal(vc, before_v)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_gather_returns_the_logical_rows(w):
    ob = paged_batch.build(w, lens=[1, 15, 16, 17, 50])
    for b in range(len(ob.lens)):
        K, V = ob.logical_kv(b)
        for g in range(w.num_kv_heads):
            gk, gv = oracle.gather(ob.k_cache, ob.v_cache, ob.tables[b], 0, int(ob.lens[b]), g,
                                   w.num_kv_heads, w.head_dim, w.dtype)
            assert np.array_equal(gk, K[:, g]) and np.array_equal(gv, V[:, g])


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_paged_decode_equals_contiguous_attention_bitwise(w):
    ob = paged_batch.build(w, lens=[1, 2, 16, 17, 31, 64, 100, 0])
    out = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    qf = oracle.to_f64(ob.q, w.dtype)
    G = w.group
    for b in range(len(ob.lens)):
        K, V = ob.logical_kv(b)
        for h in range(w.num_heads):
            o, _, _ = oracle.attend(qf[b, h], K[:, h // G].copy(), V[:, h // G].copy(), w.scale)
            assert np.array_equal(out[b, h], o), (b, h)
    assert np.all(np.isfinite(out))
    assert np.array_equal(out[7], np.zeros_like(out[7]))   # n = 0 -> zero row


def test_paged_decode_matches_torch_sdpa_per_sequence():
    torch = pytest.importorskip("torch")
    w = _w(name="bf16", dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128, num_blocks=0)
    ob = paged_batch.build(w, lens=[5, 77, 200])
    out = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    qf = torch.from_numpy(oracle.to_f64(ob.q, w.dtype))
    for b in range(3):
        K, V = ob.logical_kv(b)
        n = int(ob.lens[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[b].view(1, w.num_heads, 1, w.head_dim),
            torch.from_numpy(K).permute(1, 0, 2).reshape(1, w.num_kv_heads, n, w.head_dim),
            torch.from_numpy(V).permute(1, 0, 2).reshape(1, w.num_kv_heads, n, w.head_dim),
            scale=w.scale, enable_gqa=True).view(w.num_heads, w.head_dim).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-13)


def _relabel(ob, perm):
    """Move physical block j to perm[j] (data and tables)."""
    kc = np.empty_like(ob.k_cache)
    vc = np.empty_like(ob.v_cache)
    kc[perm] = ob.k_cache
    vc[perm] = ob.v_cache
    tables = np.where(ob.tables >= 0, perm[np.maximum(ob.tables, 0)], -1).astype(np.int32)
    return kc, vc, tables


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_block_relabelling_leaves_output_bits_unchanged(w):
    ob = paged_batch.build(w, lens=[3, 16, 49, 120])
    base = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    for seed in range(3):
        perm = np.random.default_rng(seed).permutation(ob.num_blocks)
        kc, vc, tables = _relabel(ob, perm)
        got = oracle.decode(ob.q, kc, vc, tables, ob.lens, w.scale, w.dtype)
        assert np.array_equal(got, base)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_bytes_past_the_length_never_reach_the_result(w):
    """Same batch with the unwritten slots holding NaN and holding zeros."""
    ob = paged_batch.build(w, lens=[1, 17, 30, 47])
    assert np.isnan(oracle.to_f64(ob.k_cache, w.dtype)).any()    # poison is present
    nan_out = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    kc, vc = oracle.empty_caches(ob.num_blocks, w.num_kv_heads, w.head_dim, w.dtype,
                                 fill_nan=False)
    oracle.cache_write(ob.prompt_k, ob.prompt_v, kc, vc, ob.prompt_slots, w.dtype)
    oracle.cache_write(ob.new_k, ob.new_v, kc, vc, ob.new_slots, w.dtype)
    zero_out = oracle.decode(ob.q, kc, vc, ob.tables, ob.lens, w.scale, w.dtype)
    assert np.all(np.isfinite(nan_out)) and np.array_equal(nan_out, zero_out)


@pytest.mark.parametrize("P", [16, 32, 48, 4096])
def test_partitions_merge_to_single_pass(P):
    w = _w(name="bf16", dtype="bf16", num_heads=8, num_kv_heads=2, head_dim=128, num_blocks=0)
    ob = paged_batch.build(w, lens=[1, 16, 17, 100, 257, 0])
    maxp = -(-ob.max_blocks * 16 // P)
    o, m, l = oracle.decode_partitions(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens,
                                       w.scale, w.dtype, P, maxp)
    n_parts = np.repeat(-(-ob.lens.astype(np.int64) // P), w.num_heads)
    merged = oracle.merge(o, m, l, n_parts).reshape(len(ob.lens), w.num_heads, w.head_dim)
    single = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    np.testing.assert_allclose(merged, single, rtol=0, atol=1e-14)
    # dead partitions are (0, -inf, 0)
    for r in range(o.shape[0]):
        for p in range(int(n_parts[r]), maxp):
            assert m[r, p] == -math.inf and l[r, p] == 0 and not o[r, p].any()


def test_row_sampling_matches_full_decode():
    w = _w(name="bf16", dtype="bf16", num_heads=8, num_kv_heads=2, head_dim=128, num_blocks=0)
    ob = paged_batch.build(w, lens=[9, 70, 33])
    full = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    rows = [(2, 7), (0, 0), (1, 3)]
    got = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype,
                        rows=rows)
    for k, (b, h) in enumerate(rows):
        assert np.array_equal(got[k], full[b, h])
