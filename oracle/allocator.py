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
* Sharing aliases whole blocks only (the shared token count must be a multiple
  of 16), so a shared block is always full and is never written again.
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
    def __init__(self, num_blocks: int, free_order=None):
        if num_blocks <= 0:
            raise PoolError("EINVAL", "num_blocks must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError("EINVAL", "free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.seqs: dict[int, list] = {}   # seq_id -> [blocks, length]
        self.alloc_failures = 0

    # -- sequences ------------------------------------------------------------
    def add_seq(self, sid: int) -> None:
        if sid in self.seqs:
            raise PoolError("EINVAL", f"sequence {sid} exists")
        self.seqs[sid] = [[], 0]

    def _seq(self, sid: int):
        if sid not in self.seqs:
            raise PoolError("ENOENT", f"unknown sequence {sid}")
        return self.seqs[sid]

    def share_prefix(self, sid: int, src: int, n_tokens: int) -> None:
        """Alias the first n_tokens (a multiple of 16) of src's table into empty sid."""
        dst, s = self._seq(sid), self._seq(src)
        if dst[1] != 0 or n_tokens < 0 or n_tokens % BLOCK_SIZE or n_tokens > s[1]:
            raise PoolError("EINVAL", "bad prefix share")
        nb = n_tokens // BLOCK_SIZE
        for blk in s[0][:nb]:
            self.ref[blk] += 1
        dst[0] = list(s[0][:nb])
        dst[1] = n_tokens

    def append(self, sid: int, n_tokens: int) -> list[int]:
        """Reserve slots for n_tokens new tokens; returns their slot ids.
        Raises ENOMEM (and changes nothing) when the free queue is too short."""
        s = self._seq(sid)
        if n_tokens < 0:
            raise PoolError("EINVAL", "negative token count")
        blocks, length = s
        need = -(-(length + n_tokens) // BLOCK_SIZE) - len(blocks)
        if need > len(self.free):
            self.alloc_failures += 1
            raise PoolError("ENOMEM", f"need {need} blocks, {len(self.free)} free")
        for _ in range(need):
            blk = self.free.popleft()
            self.ref[blk] = 1
            blocks.append(blk)
        slots = []
        for pos in range(length, length + n_tokens):
            slots.append(blocks[pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE)
        s[1] = length + n_tokens
        return slots

    def free_seq(self, sid: int) -> None:
        blocks, _ = self._seq(sid)
        for blk in blocks:
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
        del self.seqs[sid]

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
                "num_seqs": len(self.seqs)}


def bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """KV bytes per token: K and V (the 2), for every layer and KV head
    ("Yerel LLM ...", section "KV bütçesi"; "vLLM Nedir? ...", section
    "Asıl şişen şey ağırlık değil, KV cache")."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes
