"""Builds one paged decode batch on the oracle side (host, numpy), from workload draws.

The flow mirrors a decode step: every sequence is admitted with its prompt
(n_b - 1 tokens) and then appends the one token being decoded, so its context
n_b counts that token. Slots come from the oracle's pool model and the host caches
are filled by the oracle's cache write; nothing here touches the HIP library.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import workloads


@dataclasses.dataclass
class OracleBatch:
    w: workloads.Workload
    lens: np.ndarray               # int32 [B]
    free_order: np.ndarray         # int32 [num_blocks]
    num_blocks: int
    q: object                      # torch [B][Hq][d] (CPU)
    prompt_k: object               # torch [T_prompt][Hkv][d]
    prompt_v: object
    new_k: object                  # torch [B][Hkv][d]
    new_v: object
    prompt_slots: np.ndarray       # int32 [T_prompt]
    new_slots: np.ndarray          # int32 [B]
    tables: np.ndarray             # int32 [B][max_blocks]
    max_blocks: int
    k_cache: np.ndarray            # raw storage, documented layout
    v_cache: np.ndarray
    pool: oracle.PoolModel

    def logical_kv(self, b: int):
        """fp64 logical K, V of sequence b: [n_b][Hkv][d] (prompt rows then the new row)."""
        off = int(np.sum(np.maximum(self.lens[:b] - 1, 0)))
        n = int(self.lens[b])
        dt = self.w.dtype
        if n == 0:
            z = np.zeros((0, self.w.num_kv_heads, self.w.head_dim))
            return z, z
        pk, pv = self._stored(self.prompt_k[off:off + n - 1], self.prompt_v[off:off + n - 1])
        nk, nv = self._stored(self.new_k[b:b + 1], self.new_v[b:b + 1])
        return np.concatenate([pk, nk]), np.concatenate([pv, nv])

    def _stored(self, k, v):
        """fp64 values of rows as the cache holds them (FP8: dequantised codes)."""
        w, dt = self.w, self.w.dtype
        if w.cache_dtype != "fp8":
            return oracle.to_f64(k, dt), oracle.to_f64(v, dt)
        return (oracle.to_f64(oracle.fp8_quantize(k, dt, w.k_scale), "fp8") * w.k_scale,
                oracle.to_f64(oracle.fp8_quantize(v, dt, w.v_scale), "fp8") * w.v_scale)


def build(w: workloads.Workload, lens=None, seed_stream: int = 0, num_blocks: int | None = None,
          max_blocks: int | None = None, layer: int = 0) -> OracleBatch:
    gen = workloads.rng(w.seed, 1000 + seed_stream, layer)
    lens = (workloads.draw_seq_lens(w, workloads.rng(w.seed, 0, seed_stream))
            if lens is None else np.asarray(lens, dtype=np.int64))
    B = len(lens)
    bs = w.block_size
    if num_blocks is None:
        num_blocks = w.num_blocks or workloads.pool_blocks_for(lens, block_size=bs)
    free_order = workloads.draw_free_order(num_blocks, gen)
    n_prompt = np.maximum(lens - 1, 0)
    prompt_k = workloads.draw_tokens(int(n_prompt.sum()), w, gen)
    prompt_v = workloads.draw_tokens(int(n_prompt.sum()), w, gen)
    new_k = workloads.draw_tokens(B, w, gen)
    new_v = workloads.draw_tokens(B, w, gen)
    q = workloads.draw_q(w, gen, batch=B)

    pool = oracle.PoolModel(num_blocks, free_order, block_size=bs)
    prompt_slots, new_slots = [], []
    for b in range(B):
        pool.add_seq(b)
        prompt_slots += pool.append(b, int(n_prompt[b]))
    for b in range(B):
        if lens[b] > 0:
            new_slots += pool.append(b, 1)
        else:
            new_slots.append(-1)       # an empty sequence writes nothing
    if max_blocks is None:
        max_blocks = max(1, int(max(-(-int(n) // bs) for n in lens)))
    tables, tl = pool.tables(list(range(B)), max_blocks)
    assert np.array_equal(tl, lens)

    kc, vc = oracle.empty_caches(num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype,
                                 block_size=bs)
    ps = np.asarray(prompt_slots, dtype=np.int32)
    ns = np.asarray(new_slots, dtype=np.int32)
    cw = dict(cache_dtype=w.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    if len(ps):
        oracle.cache_write(prompt_k, prompt_v, kc, vc, ps, w.dtype, **cw)
    oracle.cache_write(new_k, new_v, kc, vc, ns, w.dtype, **cw)
    return OracleBatch(w, lens.astype(np.int32), free_order, num_blocks, q, prompt_k, prompt_v,
                       new_k, new_v, ps, ns, tables, max_blocks, kc, vc, pool)
