"""Pins for the oracle pool model's prefix cache and copy-on-write.

Each scenario restates one thing the pages say ("vLLM Nedir? PagedAttention ile Production
LLM Serving", section "Prefix caching", and section "Bir istek motorun içinde", step 5;
"Yerel LLM sistemlerinde backpressure ve ölçekleme", section "4. Prefill ve decode";
"vLLM ve Triton ile maliyet optimizasyonu", §03, paragraph on sharing):
  * only full 16-token blocks are found again; the rest of a prompt is computed;
  * the match runs from the first token on: a changed first token finds nothing;
  * a salt in the first block's key keeps tenants apart;
  * blocks of a finished request stay findable until their memory is reused;
  * a shared block is copied only when one of its users writes to it.
Random operation sequences then check invariants that any mistake in sharing breaks:
no slot handed out for writing ever lies in a block another table references, and every
table that references a keyed block agrees with that block's content.
"""
import numpy as np
import pytest

from oracle import PoolError, PoolModel

BS = 16


def _prompt(n, start=1000):
    return list(range(start, start + n))


def test_only_full_blocks_of_a_repeated_prompt_are_found():
    m = PoolModel(64)
    a = _prompt(40)
    assert m.add_seq_prefix(1, a) == 0
    slots, cp = m.append_tokens(1, a)
    assert cp is None and len(slots) == 40
    ablocks = m.seq_blocks(1)
    b = a + _prompt(10, start=5000)
    assert m.add_seq_prefix(2, b) == 32          # blocks 0 and 1; block 2 is not full in seq 1
    assert m.seq_blocks(2) == ablocks[:2]
    assert m.ref[ablocks[0]] == 2 and m.ref[ablocks[1]] == 2 and m.ref[ablocks[2]] == 1
    slots, cp = m.append_tokens(2, b[32:])
    assert cp is None and len(slots) == 18
    assert all(s // BS not in ablocks for s in slots)   # the rest is computed into new blocks


def test_a_changed_first_token_finds_nothing():
    m = PoolModel(64)
    a = _prompt(64)
    m.add_seq_prefix(1, a)
    m.append_tokens(1, a)
    b = [7] + a[1:]
    assert m.add_seq_prefix(2, b) == 0


def test_salt_keeps_tenants_apart():
    m = PoolModel(64)
    a = _prompt(48)
    m.add_seq_prefix(1, a, salt=11)
    m.append_tokens(1, a)
    assert m.add_seq_prefix(2, a, salt=12) == 0
    assert m.add_seq_prefix(3, a, salt=11) == 32      # the last block ends at the last token


def test_the_last_prompt_token_is_always_left_to_compute():
    m = PoolModel(64)
    a = _prompt(32)
    m.add_seq_prefix(1, a)
    m.append_tokens(1, a)
    assert m.add_seq_prefix(2, a) == 16
    assert m.add_seq_prefix(3, a + [1]) == 32


def test_finished_blocks_stay_findable_until_reused():
    m = PoolModel(8)
    a = _prompt(33)
    m.add_seq_prefix(1, a)
    m.append_tokens(1, a)
    blocks = m.seq_blocks(1)
    m.free_seq(1)
    assert len(m.free) == 8
    assert m.add_seq_prefix(2, a) == 32                # found in the free queue
    assert m.seq_blocks(2) == blocks[:2] and len(m.free) == 6
    m.free_seq(2)
    # use every block once: the cached ones come last in the free queue and are evicted
    m.add_seq(3)
    m.append(3, 8 * BS)
    m.free_seq(3)
    assert m.stats()["cached"] == 0
    assert m.add_seq_prefix(4, a) == 0


def test_fork_shares_and_the_first_write_copies_the_partly_filled_block():
    m = PoolModel(16)
    a = _prompt(20)
    m.add_seq_prefix(1, a)
    m.append_tokens(1, a)
    p0, p1 = m.seq_blocks(1)
    m.fork(1, 2)
    assert m.ref[p0] == 2 and m.ref[p1] == 2
    slots, cp = m.append_tokens(2, [77])
    assert cp is not None and cp[0] == p1
    new = cp[1]
    assert m.seq_blocks(2) == [p0, new] and slots == [new * BS + 4]
    assert m.ref[p0] == 2 and m.ref[p1] == 1 and m.ref[new] == 1
    slots, cp = m.append_tokens(1, [88])               # p1 is no longer shared: no copy
    assert cp is None and slots == [p1 * BS + 4]


def test_fork_at_a_block_boundary_needs_no_copy():
    m = PoolModel(16)
    a = _prompt(32)
    m.add_seq_prefix(1, a)
    m.append_tokens(1, a)
    m.fork(1, 2)
    slots, cp = m.append_tokens(2, [5])
    assert cp is None and slots[0] // BS not in m.seq_blocks(1)


def test_a_refused_copy_on_write_changes_nothing():
    m = PoolModel(2)
    m.add_seq(1)
    m.append_tokens(1, _prompt(20))                    # both blocks in use
    m.fork(1, 2)
    before = (m.seq_blocks(1), m.seq_blocks(2), list(m.ref), list(m.free))
    with pytest.raises(PoolError) as e:
        m.append_tokens(2, [3])
    assert e.value.code == "ENOMEM"
    assert (m.seq_blocks(1), m.seq_blocks(2), list(m.ref), list(m.free)) == before
    with pytest.raises(PoolError) as e:                # no token ids: no copy-on-write
        m.append(2, 1)
    assert e.value.code == "EINVAL"


def test_a_step_where_all_sharers_write_copies_for_all_but_the_last():
    m = PoolModel(3)
    m.add_seq(1)
    m.append_tokens(1, _prompt(20))                    # blocks 0 and 1 in use, one free
    m.fork(1, 2)
    slots, copies = m.append_batch_tokens([1, 2], [5, 6])
    b0, b1 = m.seq_blocks(2)
    assert len(copies) == 1 and copies[0][0] == b1     # seq 1 copies, seq 2 keeps b1
    new = copies[0][1]
    assert m.seq_blocks(1) == [b0, new] and slots == [new * BS + 4, b1 * BS + 4]
    assert m.ref[b1] == 1 and m.ref[new] == 1 and len(m.free) == 0
    m.fork(2, 3)
    with pytest.raises(PoolError) as e:                # one copy needed, no free block
        m.append_batch_tokens([2, 3], [7, 8])
    assert e.value.code == "ENOMEM"


def _check_invariants(m, written):
    refs = [0] * m.num_blocks
    for sid, (blocks, n) in m.seqs.items():
        assert len(blocks) == -(-n // BS)
        for b in blocks:
            refs[b] += 1
    assert refs == m.ref
    assert sorted(m.free) == [b for b in range(m.num_blocks) if refs[b] == 0]
    assert len(set(m.free)) == len(m.free)
    for key, blk in m.cache.items():
        assert m.key_of[blk] == key
        salt, toks = key
        j = len(toks) // BS - 1
        for sid, (blocks, n) in m.seqs.items():
            if j < len(blocks) and blocks[j] == blk and m.tokens[sid] is not None:
                assert m.salt[sid] == salt and tuple(m.tokens[sid][:len(toks)]) == toks
    for sid, slots in written:                         # this step's writes: unshared blocks
        for s in slots:
            assert m.ref[s // BS] == 1 and s // BS in m.seqs[sid][0]


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_keep_sharing_sound(seed):
    gen = np.random.default_rng(seed)
    m = PoolModel(48, gen.permutation(48))
    prompts = [list(gen.integers(0, 3, size=int(gen.integers(1, 70)))) for _ in range(6)]
    live, nxt = [], 0
    for _ in range(400):
        op = gen.integers(0, 5)
        written = []
        try:
            if op == 0 or not live:                     # admit with a lookup
                p = prompts[int(gen.integers(len(prompts)))]
                salt = int(gen.integers(0, 2))
                n = m.add_seq_prefix(nxt, p, salt)
                live.append(nxt)
                nxt += 1
                try:
                    written.append((nxt - 1, m.append_tokens(nxt - 1, p[n:])[0]))
                except PoolError:
                    m.free_seq(nxt - 1)
                    live.remove(nxt - 1)
            elif op == 1:                               # decode one token
                sid = live[int(gen.integers(len(live)))]
                written.append((sid, m.append_tokens(sid, [int(gen.integers(0, 3))])[0]))
            elif op == 2 and len(live) > 0:             # fork
                sid = live[int(gen.integers(len(live)))]
                m.fork(sid, nxt)
                live.append(nxt)
                nxt += 1
            elif op == 3 and len(live) > 1:             # finish
                sid = live.pop(int(gen.integers(len(live))))
                m.free_seq(sid)
            else:                                       # several tokens at once
                sid = live[int(gen.integers(len(live)))]
                k = int(gen.integers(1, 20))
                written.append((sid, m.append_tokens(sid, list(gen.integers(0, 3, size=k)))[0]))
        except PoolError as e:
            assert e.code == "ENOMEM"
        _check_invariants(m, written)
    assert m.hits > 0
