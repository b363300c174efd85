"""GPU parity at block sizes 8 and 32 (the default 16 is covered everywhere else).

"vLLM ve Triton ile maliyet optimizasyonu" (the paragraph on the costs of PagedAttention)
names the block size as a tuning knob. The kernels keep their 16-token tile at 8 tokens per
block (two blocks per tile) and in the balanced split and partitions of 16-token multiples at
32 (half a block per tile); the single pass and partitions of whole 32-token blocks walk
whole blocks. Checked here, against the oracle on the same seeded inputs:
  * slots, block tables and caches bit-exact (16-bit and FP8 caches);
  * decode in the three launch modes (single pass, fixed partitions, including partitions
    of half a 32-token block, of whole blocks, balanced split), fused append, FP8 cache,
    chunked prefill, with the bars of the 16-token tests;
  * the same logical K/V packed at 8, 16 and 32 tokens per block: bit-identical outputs
    wherever the 16-token tiles are walked (only the addresses they are read from change),
    including a table width that leaves the last tile's second 8-token block outside the
    table row; the whole-block walk sums in 32-position steps and meets the oracle bars.
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
B8 = workloads.WORKLOADS["llama8b"]
SHAPES = {
    "bf16-d128-g4": dataclasses.replace(B8, num_blocks=0),
    "f16-d64-g8": dataclasses.replace(B8, dtype="f16", num_heads=16, num_kv_heads=2, head_dim=64,
                                      num_blocks=0),
    "bf16-d64-g1": dataclasses.replace(B8, num_heads=4, num_kv_heads=4, head_dim=64, num_blocks=0),
    "bf16-d128-g16": dataclasses.replace(B8, num_heads=32, num_kv_heads=2, num_blocks=0),
}
LENS = [0, 1, 2, 7, 8, 9, 15, 16, 17, 24, 31, 32, 33, 63, 100, 255, 257, 700]
SHORT = [1, 9, 17]          # at 8 tokens per block: a 3-entry table row


def _w(name, bs, **kw):
    return dataclasses.replace(SHAPES[name], block_size=bs, **kw)


def _fp8(w):
    return dataclasses.replace(w, kv_dtype="fp8", k_scale=0.02, v_scale=0.015)


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _oracle_decode(ob, w):
    return oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype,
                         **({"kv_dtype": "fp8", "k_scale": w.k_scale, "v_scale": w.v_scale}
                            if w.cache_dtype == "fp8" else {}))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [8, 32])
def test_slots_tables_and_caches_are_bit_exact(bs, kv, device):
    w = _w("bf16-d128-g4", bs)
    w = _fp8(w) if kv == "fp8" else w
    ob = paged_batch.build(w, lens=LENS)
    gb = gpu_batch.build(ob, device)
    assert tuple(gb.v_cache.shape)[3] == bs
    assert np.array_equal(gb.prompt_slots, ob.prompt_slots)
    assert np.array_equal(gb.new_slots, ob.new_slots)
    assert np.array_equal(gb.tables, ob.tables) and np.array_equal(gb.lens, ob.lens)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(gb.k_cache).view(np.uint8), ob.k_cache.view(np.uint8))
    assert np.array_equal(oracle.raw(gb.v_cache).view(np.uint8), ob.v_cache.view(np.uint8))


@pytest.mark.parametrize("P", [0, 16, 48, 64, AUTO], ids=["single", "p16", "p48", "p64", "auto"])
@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("bs", [8, 32])
def test_decode_matches_oracle(bs, name, P, device):
    w = _w(name, bs)
    for lens in (LENS, SHORT):
        ob = paged_batch.build(w, lens=lens)
        gb = gpu_batch.build(ob, device)
        out, _ = gpu_batch.run_decode(gb, w, P)
        torch.cuda.synchronize()
        check_close(out.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype,
                    f"bs {bs} {name} P {P} lens {lens[:3]}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [0, 16, AUTO], ids=["single", "p16", "auto"])
def test_bs8_decode_over_caches_past_2gib(P, kv, device):
    """At 8 tokens per block a 16-token tile spans two blocks, read through per-lane
    addresses. Here the batch's blocks are spread over caches of just over 2 GiB each (ids
    up to the top of the pool, so that tile offsets pass 31 bits and the two blocks of a
    tile can lie more than 2 GiB apart), and the decode is checked against the oracle on
    the compact pool."""
    w = _w("bf16-d128-g4", 8)
    w = _fp8(w) if kv == "fp8" else w
    ob = paged_batch.build(w, lens=[1, 9, 17, 300, 700])
    gb = gpu_batch.build(ob, device)
    per_block = int(np.prod(gb.k_cache.shape[1:])) * gb.k_cache.element_size()
    nb_big = (1 << 31) // per_block + 4099
    assert nb_big * per_block > (1 << 31)
    nb = gb.k_cache.shape[0]
    big_ids = (np.arange(nb, dtype=np.int64) * 104729 + 4098) % nb_big
    assert len(np.unique(big_ids)) == nb and big_ids.max() * per_block > (1 << 31)
    fill = 0x7F if kv == "fp8" else float("nan")
    kc, vc = pkv.alloc_caches(nb_big, w.num_kv_heads, w.head_dim, w.cache_dtype, device,
                              fill=fill, block_size=8)
    idx = torch.from_numpy(big_ids).to(device)
    kc.index_copy_(0, idx, gb.k_cache)
    vc.index_copy_(0, idx, gb.v_cache)
    tab = np.where(gb.tables >= 0, big_ids[np.maximum(gb.tables, 0)], -1).astype(np.int32)
    B, Hq, d = gb.q.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=device)
    parts = None
    if P != 0:
        maxp = pkv.max_partitions_for(tab.shape[1], P, 8)
        parts = pkv.alloc_partials(B, Hq, d, maxp, device)
    pkv.decode(out, gb.q, kc, vc, torch.from_numpy(tab).to(device), gb.lens_d, w.scale, P, parts,
               kv_scales=gpu_batch.kv_scales(w))
    torch.cuda.synchronize()
    check_close(out.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype,
                f"bs 8 caches past 2 GiB {kv} P {P}")
    del kc, vc
    torch.cuda.empty_cache()


# at 32 tokens per block, caches are walked in whole blocks (single pass, partitions of
# whole blocks) or 16-token tiles (partitions of 16 tokens): both paths are covered
@pytest.mark.parametrize("P", [0, 16, 32, AUTO], ids=["single", "p16", "p32", "auto"])
@pytest.mark.parametrize("bs", [8, 32])
def test_fp8_decode_matches_oracle(bs, P, device):
    w = _fp8(_w("bf16-d128-g4", bs))
    ob = paged_batch.build(w, lens=LENS)
    gb = gpu_batch.build(ob, device)
    out, _ = gpu_batch.run_decode(gb, w, P)
    torch.cuda.synchronize()
    check_close(out.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype, f"fp8 bs {bs} P {P}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [0, 16, 32, AUTO], ids=["single", "p16", "p32", "auto"])
@pytest.mark.parametrize("bs", [8, 32])
def test_fused_append_matches_oracle(bs, P, kv, device):
    """The decode step in one call: the new rows land bit-exactly where the oracle's cache
    write puts them, and the attention over them meets the oracle bar."""
    w = _w("f16-d64-g8", bs)
    w = _fp8(w) if kv == "fp8" else w
    ob = paged_batch.build(w, lens=LENS)
    gb = gpu_batch.build(ob, device, write_new=False)
    B, Hq, d = gb.q.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=device)
    parts = None
    if P != 0:
        maxp = pkv.max_partitions_for(gb.tables.shape[1], P, bs)
        parts = tuple(t.fill_(float("nan")) for t in pkv.alloc_partials(B, Hq, d, maxp, device))
    slots = torch.from_numpy(gb.new_slots).to(device)
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, P, parts,
               append=(ob.new_k.to(device), ob.new_v.to(device), slots),
               kv_scales=gpu_batch.kv_scales(w))
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(gb.k_cache).view(np.uint8), ob.k_cache.view(np.uint8))
    assert np.array_equal(oracle.raw(gb.v_cache).view(np.uint8), ob.v_cache.view(np.uint8))
    check_close(out.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype,
                f"append {kv} bs {bs} P {P}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("append", [False, True], ids=["decode", "append"])
@pytest.mark.parametrize("name", ["bf16-d128-g16", "bf16-d64-g1"])
def test_whole_blocks_at_group_size_extremes(name, append, kv, device):
    """The whole-block kernel (32 tokens per block, single pass) with the largest and the
    smallest GQA group, plain and with the fused append, over 16-bit and FP8 caches."""
    w = _w(name, 32)
    w = _fp8(w) if kv == "fp8" else w
    ob = paged_batch.build(w, lens=LENS)
    gb = gpu_batch.build(ob, device, write_new=not append)
    B, Hq, d = gb.q.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=device)
    app = None
    if append:
        app = (ob.new_k.to(device), ob.new_v.to(device), torch.from_numpy(gb.new_slots).to(device))
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, 0, None,
               append=app, kv_scales=gpu_batch.kv_scales(w))
    torch.cuda.synchronize()
    assert np.array_equal(oracle.raw(gb.k_cache).view(np.uint8), ob.k_cache.view(np.uint8))
    assert np.array_equal(oracle.raw(gb.v_cache).view(np.uint8), ob.v_cache.view(np.uint8))
    check_close(out.cpu().double().numpy(), _oracle_decode(ob, w), w.dtype, f"{name} {append}")


# (context length, chunk length) per sequence
PREFILL = [(1, 1), (9, 9), (40, 7), (97, 33), (300, 64), (513, 100), (5, 8), (70, 70)]


@pytest.mark.parametrize("name", ["bf16-d128-g4", "f16-d64-g8"])
@pytest.mark.parametrize("bs", [8, 32])
def test_prefill_matches_oracle(bs, name, device):
    w = _w(name, bs)
    lens = [n for n, _ in PREFILL]
    chunk = [L for _, L in PREFILL]
    ob = paged_batch.build(w, lens=lens)
    gb = gpu_batch.build(ob, device)
    q = workloads.draw_q(w, workloads.rng(w.seed, 62, bs), batch=int(sum(chunk)))
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=device)
    pkv.paged_attention_prefill(out, q.to(device), torch.from_numpy(qs).to(device), gb.k_cache,
                                gb.v_cache, gb.tables_d, gb.lens_d, w.scale, max(chunk))
    torch.cuda.synchronize()
    ref = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    check_close(out.cpu().double().numpy(), ref, w.dtype, f"prefill bs {bs} {name}")


# --------------------------------------------------- one context, three block sizes
def _repack(ob, w, bs, device, max_len):
    """The batch's logical rows written through the library's pool and cache write at
    bs tokens per block (its own random free-queue order); tables max_len / bs wide."""
    lens = [int(n) for n in ob.lens]
    nb = sum(-(-n // bs) for n in lens) + 5
    order = np.random.default_rng(1000 + bs).permutation(nb).astype(np.int32)
    pool = pkv.kv_pool_create(nb, 1, w.num_kv_heads, w.head_dim, w.cache_dtype, free_order=order,
                              block_size=bs)
    fill = 0x7F if w.cache_dtype == "fp8" else float("nan")
    kc, vc = pkv.alloc_caches(nb, w.num_kv_heads, w.head_dim, w.cache_dtype, device, fill=fill,
                              block_size=bs)
    off = 0
    for b, n in enumerate(lens):
        pool.add_seq(b)
        if n == 0:
            continue
        slots = torch.from_numpy(pool.append(b, n)).to(device)
        k = torch.cat([ob.prompt_k[off:off + n - 1], ob.new_k[b:b + 1]]).to(device)
        v = torch.cat([ob.prompt_v[off:off + n - 1], ob.new_v[b:b + 1]]).to(device)
        gpu_batch.write(w, k, v, kc, vc, slots)
        off += n - 1
    tables, tl = pool.build_tables(list(range(len(lens))), max_len // bs)
    return kc, vc, torch.from_numpy(tables).to(device), torch.from_numpy(tl).to(device)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [0, 32, AUTO], ids=["single", "p32", "auto"])
def test_decode_is_bit_identical_across_block_sizes(P, kv, device):
    w = _w("bf16-d128-g4", 16)
    w = _fp8(w) if kv == "fp8" else w
    ob = paged_batch.build(w, lens=LENS)
    max_len = -(-max(LENS) // 32) * 32
    outs = []
    for bs in (8, 16, 32):
        kc, vc, tab, tl = _repack(ob, w, bs, device, max_len)
        B, Hq, d = ob.q.shape
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=device)
        parts = None
        if P != 0:
            maxp = pkv.max_partitions_for(max_len // bs, P, bs)
            parts = pkv.alloc_partials(B, Hq, d, maxp, device)
        pkv.decode(out, ob.q.to(device), kc, vc, tab, tl, w.scale, P, parts,
                   kv_scales=gpu_batch.kv_scales(w))
        torch.cuda.synchronize()
        outs.append(out.cpu())
    ref = _oracle_decode(ob, w)
    check_close(outs[1].double().numpy(), ref, w.dtype, "bs 16")
    assert torch.equal(outs[0], outs[1])
    if P != AUTO:
        # at 32 tokens per block the single pass and partitions of whole blocks walk whole
        # blocks (32-position steps): the same values summed in another order, so they are
        # held to the oracle's bars instead
        check_close(outs[2].double().numpy(), ref, w.dtype, "bs 32")
    else:
        assert torch.equal(outs[2], outs[1])


def test_prefill_is_bit_identical_across_block_sizes(device):
    w = _w("bf16-d128-g4", 16)
    lens = [n for n, _ in PREFILL]
    chunk = [L for _, L in PREFILL]
    ob = paged_batch.build(w, lens=lens)
    max_len = -(-max(lens) // 32) * 32
    q = workloads.draw_q(w, workloads.rng(w.seed, 63), batch=int(sum(chunk))).to(device)
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)).to(device)
    outs = []
    for bs in (8, 16, 32):
        kc, vc, tab, tl = _repack(ob, w, bs, device, max_len)
        out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=device)
        pkv.paged_attention_prefill(out, q, qs, kc, vc, tab, tl, w.scale, max(chunk))
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert torch.isfinite(outs[1]).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[2], outs[1])


def test_fp32_inputs_need_sixteen_token_blocks(device):
    w = _w("bf16-d64-g1", 8, dtype="f32")
    kc, vc = pkv.alloc_caches(4, w.num_kv_heads, w.head_dim, "f32", device, fill=0.0,
                              block_size=8)
    q = torch.zeros((1, w.num_heads, w.head_dim), dtype=torch.float32, device=device)
    tab = torch.zeros((1, 2), dtype=torch.int32, device=device)
    ln = torch.tensor([3], dtype=torch.int32, device=device)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode(q.clone(), q, kc, vc, tab, ln, 0.1)
    assert e.value.code == pkv.PKV_ENOTSUP
