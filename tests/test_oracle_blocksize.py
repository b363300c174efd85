"""Pins for the oracle at block sizes 8 and 32 next to the default 16.

"vLLM ve Triton ile maliyet optimizasyonu" (the paragraph on the costs of PagedAttention)
calls the block size a tuning knob: small blocks add indirection and larger block tables,
large blocks bring back internal fragmentation in the last block. Pinned here:
  * the worked example of 17 tokens (2 blocks at 16, "vLLM Nedir? ...", section "Bir istek
    motorun içinde") and its closed forms at 8 and 32; the waste bound (fewer than one
    block per sequence, "at most 15 tokens" at 16: section "PagedAttention") for each size;
  * the cache layout at each size through numpy's indexing of the documented shape;
  * paged decode equals contiguous attention bit for bit, and the same logical K/V give
    bit-identical outputs whatever the block size (only where K/V are read from changes).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import paged_batch
import workloads

W = dataclasses.replace(workloads.WORKLOADS["llama8b"], num_heads=8, num_kv_heads=2,
                        head_dim=64, num_blocks=0)
SIZES = [8, 16, 32]


@pytest.mark.parametrize("bs,blocks", [(8, 3), (16, 2), (32, 1)])
def test_seventeen_tokens(bs, blocks):
    m = oracle.PoolModel(8, block_size=bs)
    m.add_seq(0)
    slots = m.append(0, 17)
    assert len(m.seq_blocks(0)) == blocks
    b = m.seq_blocks(0)
    assert slots == [b[t // bs] * bs + t % bs for t in range(17)]


@pytest.mark.parametrize("bs", SIZES)
def test_waste_is_less_than_one_block_and_tables_shrink_with_size(bs):
    gen = np.random.default_rng(bs)
    lens = gen.integers(1, 3000, size=200)
    m = oracle.PoolModel(int(sum(-(-lens // bs))), block_size=bs)
    for i, n in enumerate(lens):
        m.add_seq(i)
        m.append(i, int(n))
        nb = len(m.seq_blocks(i))
        assert nb == -(-int(n) // bs)                       # table entries
        assert 0 <= nb * bs - n <= bs - 1                  # the last block's leftover
    assert m.stats()["free"] == 0


@pytest.mark.parametrize("bs", [8, 32])
def test_cache_layout_matches_numpy_indexing(bs):
    w = dataclasses.replace(W, block_size=bs)
    ob = paged_batch.build(w, lens=[1, 9, 31, 33, 70])
    x = 8
    kc, vc = oracle.empty_caches(ob.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, block_size=bs)
    kv = kc.reshape(ob.num_blocks, w.num_kv_heads, w.head_dim // x, bs, x)
    vv = vc.reshape(ob.num_blocks, w.num_kv_heads, w.head_dim, bs)
    for rows_k, rows_v, slots in ((oracle.raw(ob.prompt_k), oracle.raw(ob.prompt_v), ob.prompt_slots),
                                  (oracle.raw(ob.new_k), oracle.raw(ob.new_v), ob.new_slots)):
        for t, s in enumerate(slots):
            if s < 0:
                continue
            blk, off = divmod(int(s), bs)
            for i in range(w.head_dim):
                kv[blk, :, i // x, off, i % x] = rows_k[t, :, i]
                vv[blk, :, i, off] = rows_v[t, :, i]
    assert np.array_equal(kc, ob.k_cache) and np.array_equal(vc, ob.v_cache)


def test_decode_is_the_same_at_every_block_size():
    """One batch's logical K/V, packed into pools of 8-, 16- and 32-token blocks (random
    free-queue order each): bit-identical decode outputs."""
    import torch
    lens = [1, 7, 8, 9, 16, 33, 100, 0]
    ob = paged_batch.build(W, lens=lens)
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    for bs in (8, 32):
        nb = sum(-(-n // bs) for n in lens) + 3
        m = oracle.PoolModel(nb, np.random.default_rng(bs).permutation(nb), block_size=bs)
        kc, vc = oracle.empty_caches(nb, W.num_kv_heads, W.head_dim, W.dtype, block_size=bs)
        off = 0
        for b, n in enumerate(lens):
            m.add_seq(b)
            if n == 0:
                continue
            slots = np.asarray(m.append(b, n), np.int32)
            k = torch.cat([ob.prompt_k[off:off + n - 1], ob.new_k[b:b + 1]])
            v = torch.cat([ob.prompt_v[off:off + n - 1], ob.new_v[b:b + 1]])
            oracle.cache_write(k, v, kc, vc, slots, W.dtype)
            off += n - 1
        tables, tl = m.tables(list(range(len(lens))), max(1, max(-(-n // bs) for n in lens)))
        out = oracle.decode(ob.q, kc, vc, tables, tl, W.scale, W.dtype)
        assert np.array_equal(out, ref), bs
