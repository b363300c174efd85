"""Builds the HIP-side twin of an OracleBatch: the same workload draws go through the
library's own block pool and reshape_and_cache on the GPU. Only the random inputs are
shared with the oracle side; slots, tables and caches are produced independently and
compared by the tests."""
from __future__ import annotations

import dataclasses
import weakref

import numpy as np
import torch

import paged_kv_cache_28_amd as pkv


@dataclasses.dataclass
class GpuBatch:
    pool: pkv.KVPool
    prompt_slots: np.ndarray
    new_slots: np.ndarray
    tables: np.ndarray
    lens: np.ndarray
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    q: torch.Tensor
    tables_d: torch.Tensor
    lens_d: torch.Tensor


# ------------------------------------------------------------------ guard bands
# Output, partial and cache buffers are views into allocations with a guard band of 0xA5
# bytes after them; check_guards() asserts after a call that no kernel wrote past the end
# of what it was given. Buffers are tracked by weak reference, so a buffer the test has
# dropped is neither kept alive nor checked.
GUARD_BYTES = 16384
_GUARDED = []


def _guarded_view(shape, dtype, device, extra_bytes=GUARD_BYTES):
    esize = torch.empty(0, dtype=dtype).element_size()
    nbytes = int(np.prod(shape)) * esize
    raw = torch.empty(nbytes + extra_bytes, dtype=torch.uint8, device=device)
    raw[nbytes:].fill_(0xA5)
    view = raw[:nbytes].view(dtype).view(*shape)
    _GUARDED.append((weakref.ref(view), nbytes))
    return view


def guarded_full(shape, fill, dtype, device):
    """A tensor of `shape` filled with `fill`, followed in memory by a guard band."""
    t = _guarded_view(shape, dtype, device)
    t.fill_(fill)
    return t


def check_guards():
    """Every guard band behind a live guarded buffer is intact."""
    torch.cuda.synchronize()
    try:
        for ref, nbytes in _GUARDED:
            v = ref()
            if v is None:
                continue
            full = torch.empty(0, dtype=torch.uint8, device=v.device).set_(v.untyped_storage())
            assert bool((full[nbytes:] == 0xA5).all()), \
                f"a kernel wrote past the end of a {v.dtype} buffer of shape {tuple(v.shape)}"
    finally:
        _GUARDED[:] = [(r, n) for r, n in _GUARDED if r() is not None]


def guarded_caches(num_blocks, hkv, d, dtype, device, fill, block_size):
    """One layer's caches, each followed by a guard band one block long."""
    ks, vs = pkv.cache_shapes(num_blocks, hkv, d, dtype, block_size)
    td = pkv.torch_dtype(dtype)
    out = []
    for shape in (ks, vs):
        block = int(np.prod(shape[1:])) * torch.empty(0, dtype=td).element_size()
        t = _guarded_view(shape, td, device, extra_bytes=block)
        if fill is not None:
            t.fill_(fill)
        out.append(t)
    return tuple(out)


def write(w, key, value, kc, vc, slots):
    """The library's cache write for the workload's cache type."""
    if w.cache_dtype == "fp8":
        pkv.reshape_and_cache_fp8(key, value, kc, vc, slots, w.k_scale, w.v_scale)
    else:
        pkv.reshape_and_cache(key, value, kc, vc, slots)


def kv_scales(w):
    return (w.k_scale, w.v_scale) if w.cache_dtype == "fp8" else None


def build(ob, device="cuda", fill=float("nan"), write_new: bool = True) -> GpuBatch:
    """write_new=False leaves the new tokens' slots unwritten (for the fused append).
    An FP8 cache is filled with the NaN code 0x7F where fill is NaN."""
    w = ob.w
    B = len(ob.lens)
    pool = pkv.kv_pool_create(ob.num_blocks, 1, w.num_kv_heads, w.head_dim, w.cache_dtype,
                              free_order=ob.free_order, block_size=w.block_size)
    prompt = []
    for b in range(B):
        pool.add_seq(b)
        prompt.append(pool.append(b, max(int(ob.lens[b]) - 1, 0)))
    prompt_slots = np.concatenate(prompt) if prompt else np.zeros(0, np.int32)
    live = [b for b in range(B) if ob.lens[b] > 0]
    new = np.full(B, -1, dtype=np.int32)
    if live:
        new[live] = pool.append_batch(live)
    tables, lens = pool.build_tables(list(range(B)), ob.max_blocks)

    if w.cache_dtype == "fp8" and fill is not None and fill != fill:
        fill = 0x7F
    kc, vc = guarded_caches(ob.num_blocks, w.num_kv_heads, w.head_dim, w.cache_dtype, device,
                            fill, w.block_size)
    if len(prompt_slots):
        write(w, ob.prompt_k.to(device), ob.prompt_v.to(device), kc, vc,
              torch.from_numpy(prompt_slots).to(device))
    if write_new:
        write(w, ob.new_k.to(device), ob.new_v.to(device), kc, vc, torch.from_numpy(new).to(device))
    return GpuBatch(pool, prompt_slots, new, tables, lens, kc, vc, ob.q.to(device),
                    torch.from_numpy(tables).to(device), torch.from_numpy(lens).to(device))


def run_decode(gb: GpuBatch, w, partition_size=0, out_dtype=torch.float32, max_partitions=None):
    """One layer's attention (decode, and reduce when partitioned). Returns out and, when
    partitioned, the partial buffers."""
    B, Hq, d = gb.q.shape
    dev = gb.q.device
    out = guarded_full((B, Hq, d), float("nan"), out_dtype, dev)
    parts = None
    if partition_size != 0:
        maxp = max_partitions or pkv.max_partitions_for(gb.tables.shape[1], partition_size,
                                                        w.block_size)
        parts = guarded_partials(B, Hq, d, maxp, dev)
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale,
               partition_size, parts, kv_scales=kv_scales(w))
    check_guards()
    return out, parts


def guarded_partials(B, Hq, d, maxp, device):
    """NaN-filled partial buffers (part_out, part_max, part_sum), each guarded."""
    return (guarded_full((B, Hq, maxp, d), float("nan"), torch.float32, device),
            guarded_full((B, Hq, maxp), float("nan"), torch.float32, device),
            guarded_full((B, Hq, maxp), float("nan"), torch.float32, device))
