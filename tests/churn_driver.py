"""Continuous-batching churn on one layer: the seeded churn events of workloads.py go to
the library's block pool (and through reshape_and_cache into the GPU caches) and, in
lockstep, to the oracle's pool model. Every slot and table is compared as it is made.

A sequence is admitted with its own prompt; a sharer first points its table at the
cached 1,024-token system prompt (refcounted blocks, "vLLM Nedir? ...", section
"PagedAttention"; [3Y] §03 on sharing). Each step retires ~5% of the live sequences
(blocks back to the free queue), admits as many, and appends one decode token to every
live sequence. The logical K/V of every sequence is kept (on the GPU) for the oracle.
With device=None only the pool side runs (no K/V, no kernels): a CPU check of the event
stream at full size.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_cache_28_amd as pkv
import workloads

PREFIX_ID = -1


class Churn:
    def __init__(self, w: workloads.Workload, device, layer: int = 0, num_blocks: int | None = None):
        self.w, self.device, self.layer = w, device, layer
        nb = num_blocks or workloads.churn_pool_blocks(w)
        order = workloads.draw_free_order(nb, workloads.rng(w.seed, 1, layer))
        self.pool = pkv.kv_pool_create(nb, 1, w.num_kv_heads, w.head_dim, w.dtype, free_order=order)
        self.model = oracle.PoolModel(nb, order)
        self.num_blocks = nb
        self.kc = self.vc = None
        if device is not None:
            self.kc, self.vc = pkv.alloc_caches(nb, w.num_kv_heads, w.head_dim, w.dtype, device,
                                                fill=float("nan"))
        self.kv: dict[int, list] = {}
        self.sharer: dict[int, bool] = {}
        # the shared system prompt
        self._add(PREFIX_ID, False, w.prefix_tokens, stream=(4, layer, 10 ** 6))
        self.live: list[int] = []
        self.next_id = 0
        gen = workloads.rng(w.seed, 5, layer)
        for sharer, p in workloads.draw_churn_initial(w, gen):
            self.admit(sharer, p)
        self.steps = 0
        self.prompt_tokens_written = 0

    # -- both sides -------------------------------------------------------------------
    def _write(self, sid, slots, k, v):
        if self.device is None:
            return
        pkv.reshape_and_cache(k, v, self.kc, self.vc, torch.from_numpy(slots).to(self.device))
        self.kv.setdefault(sid, []).append((k, v))

    def _add(self, sid, sharer, n_own, stream):
        self.pool.add_seq(sid)
        self.model.add_seq(sid)
        self.sharer[sid] = sharer
        if sharer:
            self.pool.share_prefix(sid, PREFIX_ID, self.w.prefix_tokens)
            self.model.share_prefix(sid, PREFIX_ID, self.w.prefix_tokens)
            self.kv[sid] = list(self.kv.get(PREFIX_ID, []))
        slots = self.pool.append(sid, n_own)
        assert slots.tolist() == self.model.append(sid, n_own), f"slots of {sid}"
        if self.device is not None:
            k = workloads.draw_tokens_device(n_own, self.w, stream + (0,), self.device)
            v = workloads.draw_tokens_device(n_own, self.w, stream + (1,), self.device)
            self._write(sid, slots, k, v)

    def admit(self, sharer: bool, prompt: int):
        sid = self.next_id
        self.next_id += 1
        self._add(sid, sharer, prompt, stream=(4, self.layer, sid))
        self.live.append(sid)

    def retire(self, sid: int):
        self.pool.free_seq(sid)
        self.model.free_seq(sid)
        self.kv.pop(sid, None)
        self.live.remove(sid)

    def step(self):
        """One churn step: retire, admit, then one decode token for every live sequence."""
        gen = workloads.rng(self.w.seed, 6, self.layer, self.steps)
        retire, admits = workloads.draw_churn_step(self.w, gen, self.live)
        for pos in sorted(retire, reverse=True):
            self.retire(self.live[pos])
        for sharer, p in admits:
            self.admit(sharer, p)
            self.prompt_tokens_written += p
        slots = self.pool.append_batch(self.live)
        assert slots.tolist() == [self.model.append(s, 1)[0] for s in self.live], "decode slots"
        self.steps += 1
        if self.device is None:
            return
        st = (7, self.layer, self.steps - 1)
        k = workloads.draw_tokens_device(len(self.live), self.w, st + (0,), self.device)
        v = workloads.draw_tokens_device(len(self.live), self.w, st + (1,), self.device)
        pkv.reshape_and_cache(k, v, self.kc, self.vc, torch.from_numpy(slots).to(self.device))
        for i, s in enumerate(self.live):
            self.kv[s].append((k[i:i + 1], v[i:i + 1]))

    # -- views --------------------------------------------------------------------------
    def tables(self):
        lens = [self.model.seq_len(s) for s in self.live]
        mb = max(1, max(-(-n // 16) for n in lens))
        t, l = self.pool.build_tables(self.live, mb)
        mt, ml = self.model.tables(self.live, mb)
        assert np.array_equal(t, mt) and np.array_equal(l, ml), "tables"
        return t, l

    def check_pool_state(self):
        ps, ms = self.pool.stats(), self.model.stats()
        for key in ("free", "used", "shared", "alloc_failures", "num_seqs"):
            assert ps[key] == ms[key], (key, ps[key], ms[key])
        assert self.pool.free_queue() == list(self.model.free)

    def logical_kv(self, sid: int, g: int):
        k = torch.cat([c[0][:, g] for c in self.kv[sid]]).cpu()
        v = torch.cat([c[1][:, g] for c in self.kv[sid]]).cpu()
        return oracle.to_f64(k, self.w.dtype), oracle.to_f64(v, self.w.dtype)
