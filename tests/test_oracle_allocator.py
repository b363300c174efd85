"""Pins for the oracle's block-pool model and the KV bytes/token formula.

* the pages' worked examples (tests/golden/*.json, each entry cites its source),
* invariants the pages state: waste at most 15 tokens per sequence, no external
  fragmentation (every block is free or referenced), reference counts equal the
  number of tables holding the block, freed blocks return to the free queue,
* brute-force cross-checks of slots against the definition slot = block*16 + offset.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle.allocator import BLOCK_SIZE, PoolError, PoolModel, bytes_per_token

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- worked examples
def test_bytes_per_token_worked_examples():
    g = _load("kv_bytes_per_token.json")
    exact = {c["name"]: c for c in g["cases"]}
    c = exact["llama3-70b-fp16"]
    assert bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"]) == \
        c["bytes_per_token"]
    c = exact["gqa-32layer-bf16"]
    # the page says "about 128 KB"; the formula lands on exactly 128 KiB
    assert bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"]) == \
        c["bytes_per_token_approx"] == 128 * 1024


def test_context_size_examples():
    g = _load("kv_bytes_per_token.json")
    ex = {c["name"]: c for c in g["context_examples"]}
    per_tok = bytes_per_token(32, 8, 128, 2)
    assert ex["8k-context-one-request"]["tokens"] * per_tok == ex["8k-context-one-request"]["approx_bytes"]
    for name in ("70b-128k-with-gqa", "70b-128k-without-gqa"):
        c = ex[name]
        total = bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"]) * c["tokens"]
        assert total == c["approx_gb"] * 2 ** 30          # the pages' "GB" are GiB here
    # the 8x ratio the page attributes to GQA (64 attention heads vs 8 KV heads)
    assert bytes_per_token(80, 64, 128, 2) == 8 * bytes_per_token(80, 8, 128, 2)


def test_seventeen_tokens_take_two_blocks():
    g = _load("allocate_slots.json")
    for c in g["cases"]:
        pool = PoolModel(64, np.random.default_rng(0).permutation(64))
        pool.add_seq(0)
        if c["start_len"]:
            pool.append(0, c["start_len"])
        slots = pool.append(0, c["append"])
        blocks = pool.seq_blocks(0)
        assert len(blocks) == c["blocks_after"]
        assert slots == [blocks[p // 16] * 16 + p % 16 for p in range(c["append"])]
        assert pool.stats()["free"] == 64 - c["blocks_after"]


def test_blocks_are_taken_only_when_the_last_one_is_full():
    pool = PoolModel(10)
    pool.add_seq(7)
    seen = []
    for n in range(1, 50):
        pool.append(7, 1)
        seen.append(len(pool.seq_blocks(7)))
        assert seen[-1] == -(-n // 16)


def test_fifo_free_queue_order():
    order = [5, 3, 9, 0, 1, 2, 4, 6, 7, 8]
    pool = PoolModel(10, order)
    pool.add_seq(1)
    pool.append(1, 40)                  # 3 blocks: 5, 3, 9
    assert pool.seq_blocks(1) == [5, 3, 9]
    pool.add_seq(2)
    pool.append(2, 1)                   # block 0
    pool.free_seq(1)                    # 5, 3, 9 go to the back, in table order
    assert list(pool.free) == [1, 2, 4, 6, 7, 8, 5, 3, 9]
    pool.add_seq(3)
    pool.append(3, 16 * 9)
    assert pool.seq_blocks(3) == [1, 2, 4, 6, 7, 8, 5, 3, 9]


def test_exhaustion_is_atomic():
    pool = PoolModel(4)
    pool.add_seq(0)
    pool.append(0, 20)                  # 2 blocks
    before = (list(pool.free), pool.seq_blocks(0), pool.seq_len(0))
    with pytest.raises(PoolError) as e:
        pool.append(0, 64)              # needs 4 more, only 2 free
    assert e.value.code == "ENOMEM"
    assert (list(pool.free), pool.seq_blocks(0), pool.seq_len(0)) == before
    assert pool.stats()["alloc_failures"] == 1
    pool.append(0, 44)                  # exactly fills the pool
    assert pool.stats()["free"] == 0


def test_prefix_sharing_refcounts():
    pool = PoolModel(32)
    pool.add_seq(0)
    pool.append(0, 70)                  # 5 blocks
    pool.add_seq(1)
    pool.share_prefix(1, 0, 64)         # alias 4 full blocks
    pool.add_seq(2)
    pool.share_prefix(2, 0, 32)
    shared = pool.seq_blocks(0)
    assert pool.seq_blocks(1) == shared[:4] and pool.seq_len(1) == 64
    assert [pool.ref[b] for b in shared] == [3, 3, 2, 2, 1]
    pool.append(1, 1)                   # goes to a fresh block, not a shared one
    assert pool.seq_blocks(1)[4] not in shared
    pool.free_seq(0)
    assert [pool.ref[b] for b in shared] == [2, 2, 1, 1, 0]
    assert list(pool.free)[-1] == shared[4]
    with pytest.raises(PoolError):
        pool.add_seq(3)
        pool.share_prefix(3, 1, 20)     # not a multiple of 16


def test_error_codes():
    pool = PoolModel(4)
    with pytest.raises(PoolError) as e:
        pool.append(9, 1)
    assert e.value.code == "ENOENT"
    pool.add_seq(1)
    with pytest.raises(PoolError) as e:
        pool.add_seq(1)
    assert e.value.code == "EINVAL"
    with pytest.raises(PoolError):
        PoolModel(4, [0, 1, 1, 2])


# ------------------------------------------------------------ random invariants
def check_invariants(pool: PoolModel):
    refs = np.zeros(pool.num_blocks, dtype=np.int64)
    for sid, (blocks, length) in pool.seqs.items():
        assert len(blocks) == -(-length // BLOCK_SIZE)
        assert 0 <= len(blocks) * BLOCK_SIZE - length <= BLOCK_SIZE - 1   # waste <= 15
        for b in blocks:
            refs[b] += 1
    assert list(refs) == pool.ref                       # refcount = references
    free = list(pool.free)
    assert len(set(free)) == len(free)
    assert all(refs[b] == 0 for b in free)              # free blocks are unreferenced
    assert len(free) + int((refs > 0).sum()) == pool.num_blocks   # nothing lost


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["add", "append", "free", "share"]),
                          st.integers(0, 7), st.integers(0, 70)), max_size=80),
       st.integers(0, 2 ** 31 - 1))
def test_random_operation_sequences_keep_invariants(ops, seed):
    nb = 40
    pool = PoolModel(nb, np.random.default_rng(seed).permutation(nb))
    for op, sid, n in ops:
        try:
            if op == "add":
                pool.add_seq(sid)
            elif op == "append":
                slots = pool.append(sid, n)
                blocks, length = pool.seqs[sid]
                for k, s in enumerate(slots):
                    pos = length - n + k
                    assert s == blocks[pos // 16] * 16 + pos % 16
            elif op == "free":
                pool.free_seq(sid)
            else:
                src = (sid + 1) % 8
                if sid not in pool.seqs:
                    pool.add_seq(sid)
                if src in pool.seqs:
                    pool.share_prefix(sid, src, (pool.seq_len(src) // 16) * 16)
        except PoolError:
            pass
        check_invariants(pool)


def test_tables_are_padded_and_dense():
    pool = PoolModel(20, list(range(19, -1, -1)))
    for sid, n in ((4, 33), (9, 0), (2, 16)):
        pool.add_seq(sid)
        pool.append(sid, n)
    t, l = pool.tables([4, 9, 2], 5)
    assert t.dtype == np.int32 and t.shape == (3, 5)
    assert t.tolist() == [[19, 18, 17, -1, -1], [-1] * 5, [16, -1, -1, -1, -1]]
    assert l.tolist() == [33, 0, 16]
    with pytest.raises(PoolError):
        pool.tables([4], 2)
