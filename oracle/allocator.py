"""Reference model of the paged KV block pool (host side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Plain Python; shares nothing with
the library's C++ allocator, and the two are compared integer for integer.

What the pages fix, and how this model reads it:

* The cache is cut into fixed blocks of 16 tokens that need not be adjacent; each
  request keeps a block table from its logical blocks to physical ones
  ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem, steps 1-2;
  "vLLM Nedir? ...", section "PagedAttention").
* A new physical block is taken only when the request's last block is full
  (§03 step 3). Worked example: 17 new tokens at block size 16 need 2 blocks
  ("vLLM Nedir? ...", section "Bir istek motorun içinde", step 2 "Schedule").
* When a request finishes its blocks go back to a free queue (same section,
  step 5 "Postprocess"); when the pool is short a request is dropped and its
  blocks returned (step 2), so a failed allocation must leave nothing behind.
* Physical blocks may be shared by several requests with a reference count
  ("vLLM Nedir? ...", section "PagedAttention", last paragraph; §03 on sharing).

Readings where the pages are silent:
* The free queue is FIFO: allocation pops from the front, a freed block is pushed
  at the back, in the order of the freed request's table. The initial order is
  given by the caller (a random permutation scatters requests over the pool).
* slot = physical_block * 16 + offset_in_block.
* share_prefix aliases whole blocks only (the shared token count must be a multiple
  of 16), so a block shared that way is full and is never written again.

Prefix caching and copy-on-write ("vLLM Nedir? ...", section "Prefix caching": every
full 16-token block is keyed by the previous block's key, its own tokens and, for the
first block, a cache salt; a request that brings the same chain references the cached
physical block instead of recomputing it; only full blocks are keyed, so a prefix that
ends inside a block leaves its last tokens to compute; a salt in the first block keeps
tenants apart. Same page, step 5: a finished request's blocks go back to the free queue
unless the prefix cache still holds them. "Yerel LLM ...", section "4. Prefill ve
decode": the cache lives while memory allows and is evicted when room is needed.
"vLLM ve Triton ...", §03, paragraph on sharing: a shared block stays a single copy
until one of its users wants to change it, and is copied then, as copy-on-write.)
Readings, where the pages leave steps open:
* The key of block j is the exact content it stands for: (salt, the sequence's tokens
  0 .. 16(j+1) - 1). A chain of the previous block's key and this block's tokens is
  that same content. Here the key is held exactly.
* A block is registered when it becomes full in a sequence whose every token id is
  known (appended with append_tokens); the first block with a key keeps it (a later
  block with the same content stays unregistered).
* Freed blocks always go to the back of the free queue and keep their key: the free
  queue is the eviction order. A block popped for allocation loses its key. A hit on a
  block with no references takes it out of the free queue.
* Lookups stop at the first miss. They cover only blocks that end before the prompt's
  last token, so at least one prompt token is always left to compute (the step that
  yields the first output token needs one).
* fork(parent, child) shares every block of the parent, the partly filled last one
  included. Appending to a partly filled block that other tables also reference first
  moves this sequence to a fresh block: the call returns (old, new), and the caller
  copies the old block's rows into the new one on the device (copy_blocks) before
  writing the new tokens.
"""
from __future__ import annotations

from collections import deque

import numpy as np

BLOCK_SIZE = 16


class PoolError(Exception):
    """Raised with .code in {'EINVAL', 'ENOMEM', 'ENOENT'}."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class PoolModel:
    def __init__(self, num_blocks: int, free_order=None, block_size: int = BLOCK_SIZE):
        if num_blocks <= 0 or block_size <= 0:
            raise PoolError("EINVAL", "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError("EINVAL", "free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.seqs: dict[int, list] = {}   # seq_id -> [blocks, length]
        self.alloc_failures = 0
        # prefix cache: key -> block and block -> key, key = (salt, tuple(prefix tokens));
        # per sequence: its salt and token ids (None once a token id is unknown)
        self.cache: dict[tuple, int] = {}
        self.key_of: dict[int, tuple] = {}
        self.salt: dict[int, int] = {}
        self.tokens: dict[int, list | None] = {}
        self.hits = 0                     # blocks found in the prefix cache so far

    # -- sequences ------------------------------------------------------------
    def add_seq(self, sid: int, salt: int = 0) -> None:
        if sid in self.seqs:
            raise PoolError("EINVAL", f"sequence {sid} exists")
        self.seqs[sid] = [[], 0]
        self.salt[sid] = salt
        self.tokens[sid] = []

    def _pop_free(self) -> int:
        """Take the front of the free queue for a new use: it loses its cache key."""
        blk = self.free.popleft()
        key = self.key_of.pop(blk, None)
        if key is not None:
            del self.cache[key]
        return blk

    def add_seq_prefix(self, sid: int, prompt, salt: int = 0) -> int:
        """New sequence whose table starts with the cached blocks of its prompt's prefix.
        Returns the number of prompt tokens found (a multiple of 16); the caller appends
        the rest with append_tokens."""
        self.add_seq(sid, salt)
        prompt = [int(t) for t in prompt]
        blocks, n = [], 0
        while n + self.bs <= len(prompt) - 1:
            blk = self.cache.get((salt, tuple(prompt[:n + self.bs])))
            if blk is None:
                break
            if self.ref[blk] == 0:
                self.free.remove(blk)
            self.ref[blk] += 1
            blocks.append(blk)
            n += self.bs
        self.hits += len(blocks)
        self.seqs[sid] = [blocks, n]
        self.tokens[sid] = prompt[:n]
        return n

    def fork(self, parent: int, child: int) -> None:
        """child shares every block of parent (partly filled last block included)."""
        p = self._seq(parent)
        if child in self.seqs:
            raise PoolError("EINVAL", f"sequence {child} exists")
        for blk in p[0]:
            self.ref[blk] += 1
        self.seqs[child] = [list(p[0]), p[1]]
        self.salt[child] = self.salt[parent]
        toks = self.tokens[parent]
        self.tokens[child] = None if toks is None else list(toks)

    def _seq(self, sid: int):
        if sid not in self.seqs:
            raise PoolError("ENOENT", f"unknown sequence {sid}")
        return self.seqs[sid]

    def share_prefix(self, sid: int, src: int, n_tokens: int) -> None:
        """Alias the first n_tokens (a multiple of 16) of src's table into empty sid."""
        dst, s = self._seq(sid), self._seq(src)
        if dst[1] != 0 or n_tokens < 0 or n_tokens % self.bs or n_tokens > s[1]:
            raise PoolError("EINVAL", "bad prefix share")
        nb = n_tokens // self.bs
        for blk in s[0][:nb]:
            self.ref[blk] += 1
        dst[0] = list(s[0][:nb])
        dst[1] = n_tokens
        self.tokens[sid] = None            # shared without token ids: never keyed

    def _shared_tail(self, s) -> bool:
        blocks, length = s
        return length % self.bs != 0 and self.ref[blocks[-1]] > 1

    def _append(self, sid: int, n_tokens: int, token_ids):
        s = self._seq(sid)
        if n_tokens < 0:
            raise PoolError("EINVAL", "negative token count")
        blocks, length = s
        cow = n_tokens > 0 and self._shared_tail(s)
        need = -(-(length + n_tokens) // self.bs) - len(blocks) + int(cow)
        if need > len(self.free):
            self.alloc_failures += 1
            raise PoolError("ENOMEM", f"need {need} blocks, {len(self.free)} free")
        pair = None
        if cow:                      # copy-on-write of the shared, partly filled last block
            new = self._pop_free()
            self.ref[new] = 1
            old = blocks[-1]
            self.ref[old] -= 1       # others still reference it (ref was > 1)
            blocks[-1] = new
            pair = (old, new)
        while len(blocks) * self.bs < length + n_tokens:
            blk = self._pop_free()
            self.ref[blk] = 1
            blocks.append(blk)
        slots = [blocks[pos // self.bs] * self.bs + pos % self.bs
                 for pos in range(length, length + n_tokens)]
        s[1] = length + n_tokens
        toks = self.tokens[sid]
        if token_ids is None or toks is None:
            self.tokens[sid] = None
        else:
            toks.extend(int(t) for t in token_ids)
            for j in range(length // self.bs, s[1] // self.bs):   # blocks now full
                key = (self.salt[sid], tuple(toks[:(j + 1) * self.bs]))
                blk = blocks[j]
                if key not in self.cache and blk not in self.key_of:
                    self.cache[key] = blk
                    self.key_of[blk] = key
        return slots, pair

    def append(self, sid: int, n_tokens: int) -> list[int]:
        """Reserve slots for n_tokens new tokens whose ids are not given (the sequence's
        later blocks are never keyed); returns their slot ids. Raises ENOMEM (and
        changes nothing) when the free queue is too short. A shared, partly filled last
        block needs append_tokens (copy-on-write): EINVAL."""
        if n_tokens > 0 and self._shared_tail(self._seq(sid)):
            raise PoolError("EINVAL", "shared partly filled block: use append_tokens")
        return self._append(sid, n_tokens, None)[0]

    def append_tokens(self, sid: int, token_ids):
        """append for tokens with known ids: returns (slots, copy) where copy is
        (old_block, new_block) when the shared last block was copied, else None."""
        token_ids = [int(t) for t in token_ids]
        return self._append(sid, len(token_ids), token_ids)

    def append_batch_tokens(self, sids, token_ids):
        """The decode step with token ids: one token per distinct sequence, all or
        nothing. Returns (slots, copies) with the (old, new) copies in batch order."""
        sids = [int(x) for x in sids]
        if len(set(sids)) != len(sids):
            raise PoolError("EINVAL", "duplicate sequence")
        ref = list(self.ref)          # a dry run in batch order counts the blocks needed
        need = 0
        for sid in sids:
            blocks, length = self._seq(sid)
            if length % self.bs == 0:
                need += 1
            elif ref[blocks[-1]] > 1:
                ref[blocks[-1]] -= 1
                need += 1
        if need > len(self.free):
            self.alloc_failures += 1
            raise PoolError("ENOMEM", f"need {need} blocks, {len(self.free)} free")
        slots, copies = [], []
        for sid, t in zip(sids, token_ids):
            sl, cp = self.append_tokens(sid, [t])
            slots += sl
            if cp is not None:
                copies.append(cp)
        return slots, copies

    def free_seq(self, sid: int) -> None:
        blocks, _ = self._seq(sid)
        for blk in blocks:
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)      # keeps its key until popped again
        del self.seqs[sid]
        del self.salt[sid], self.tokens[sid]

    # -- views ------------------------------------------------------------------
    def seq_len(self, sid: int) -> int:
        return self._seq(sid)[1]

    def seq_blocks(self, sid: int) -> list[int]:
        return list(self._seq(sid)[0])

    def tables(self, sids, max_blocks: int):
        """Dense int32 [len(sids)][max_blocks] block tables padded with -1, and lengths."""
        out = np.full((len(sids), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for r, sid in enumerate(sids):
            blocks, length = self._seq(sid)
            if len(blocks) > max_blocks:
                raise PoolError("EINVAL", "table wider than max_blocks")
            out[r, :len(blocks)] = blocks
            lens[r] = length
        return out, lens

    def stats(self) -> dict:
        used = sum(1 for r in self.ref if r > 0)
        shared = sum(1 for r in self.ref if r > 1)
        return {"total": self.num_blocks, "free": len(self.free), "used": used,
                "shared": shared, "alloc_failures": self.alloc_failures,
                "num_seqs": len(self.seqs), "cached": len(self.cache),
                "prefix_hits": self.hits}


def bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """KV bytes per token: K and V (the 2), for every layer and KV head
    ("Yerel LLM ...", section "KV bütçesi"; "vLLM Nedir? ...", section
    "Asıl şişen şey ağırlık değil, KV cache")."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes
