"""Prefix caching and copy-on-write on the GPU.

* copy_blocks: bit-exact against a copy of the same blocks in numpy, skipped pairs left
  alone, more layers than one launch carries.
* A serving scenario through the library's pool, in lockstep with the oracle's pool model:
  requests admitted with prefix lookups, forked (parallel samples), decoded one token per
  step with copy-on-write copies run by copy_blocks, finished and re-admitted. After every
  step each live sequence's attention output is compared with the oracle's attention over
  that sequence's own token history. K/V rows are a fixed function of (position, token id),
  so a reused block holds exactly the rows the sequence would have written itself
  ("vLLM Nedir? PagedAttention ile Production LLM Serving", section "Prefix caching":
  the KV of a matching prefix is referenced, not recomputed; "vLLM ve Triton ile maliyet
  optimizasyonu", §03, paragraph on sharing: copy-on-write).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_28_amd as pkv
import workloads
from test_gpu_parity import check_close

pytestmark = pytest.mark.gpu
AUTO = pkv.PKV_PARTITION_AUTO


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("dtype,layers", [("bf16", 3), ("fp8", 70)])
def test_copy_blocks_is_bit_exact(dtype, layers, device):
    hkv, d, nb = 2, 64, 24
    gen = np.random.default_rng(7)
    ks, vs = pkv.cache_shapes(nb, hkv, d, dtype)
    tdt = pkv.torch_dtype(dtype)
    host_k = [gen.integers(0, 256, size=int(np.prod(ks)) * (2 if dtype == "bf16" else 1),
                           dtype=np.uint8) for _ in range(layers)]
    host_v = [gen.integers(0, 256, size=int(np.prod(vs)) * (2 if dtype == "bf16" else 1),
                           dtype=np.uint8) for _ in range(layers)]
    kc = [torch.from_numpy(h).to(device).view(tdt).view(ks) for h in host_k]
    vc = [torch.from_numpy(h).to(device).view(tdt).view(vs) for h in host_v]
    # distinct destinations, none of them a source; (5, 5), (-1, 4) and (7, 30) are skipped
    pairs = np.array([[3, 9], [5, 5], [-1, 4], [7, 30], [11, 2], [12, 13], [0, 23]], np.int32)
    pkv.copy_blocks(kc, vc, torch.from_numpy(pairs).to(device))
    torch.cuda.synchronize()
    for l in range(layers):
        for host, dev_t in ((host_k[l], kc[l]), (host_v[l], vc[l])):
            ref = host.reshape(nb, -1).copy()
            for s, t in pairs:
                if 0 <= s < nb and 0 <= t < nb and s != t:
                    ref[t] = host.reshape(nb, -1)[s]
            got = dev_t.cpu().contiguous().view(torch.uint8).numpy().reshape(nb, -1)
            assert np.array_equal(got, ref), l


class Serving:
    """Library pool + GPU caches on one side, the oracle's pool model on the other."""

    def __init__(self, w, device, nb=72, seed=0):
        self.w, self.dev = w, device
        self.bs = bs = w.block_size
        nb = nb * 16 // bs
        self.gen = np.random.default_rng(seed)
        order = self.gen.permutation(nb).astype(np.int32)
        self.pool = pkv.kv_pool_create(nb, 1, w.num_kv_heads, w.head_dim, w.cache_dtype,
                                       free_order=order, block_size=bs)
        self.model = oracle.PoolModel(nb, order, block_size=bs)
        fill = 0x7F if w.cache_dtype == "fp8" else float("nan")
        self.kc, self.vc = pkv.alloc_caches(nb, w.num_kv_heads, w.head_dim, w.cache_dtype,
                                            device, fill=fill, block_size=bs)
        # K/V row of (position, token id): positions < 256, token ids < 4
        g = workloads.rng(w.seed, 40)
        self.emb_k = workloads.draw_tokens(256 * 4, w, g).view(256, 4, w.num_kv_heads, w.head_dim)
        self.emb_v = workloads.draw_tokens(256 * 4, w, g).view(256, 4, w.num_kv_heads, w.head_dim)
        self.tokens: dict[int, list] = {}
        self.next_id = 0
        self.copies = 0
        self.hit_tokens = 0

    def _rows(self, positions, toks):
        p = torch.as_tensor(positions)
        t = torch.as_tensor(toks)
        return self.emb_k[p, t], self.emb_v[p, t]

    def _write(self, sid, first_pos, toks, slots):
        if not len(toks):
            return
        k, v = self._rows(list(range(first_pos, first_pos + len(toks))), toks)
        k, v = k.to(self.dev), v.to(self.dev)
        sl = torch.from_numpy(np.asarray(slots, np.int32)).to(self.dev)
        w = self.w
        if w.cache_dtype == "fp8":
            pkv.reshape_and_cache_fp8(k, v, self.kc, self.vc, sl, w.k_scale, w.v_scale)
        else:
            pkv.reshape_and_cache(k, v, self.kc, self.vc, sl)

    def _copy(self, copies):
        if len(copies):
            self.copies += len(copies)
            pkv.copy_blocks([self.kc], [self.vc],
                            torch.from_numpy(np.asarray(copies, np.int32).reshape(-1, 2)).to(self.dev))

    def admit(self, prompt, salt=0):
        sid = self.next_id
        self.next_id += 1
        n = self.pool.add_seq_prefix(sid, prompt, salt)
        assert n == self.model.add_seq_prefix(sid, prompt, salt)
        self.hit_tokens += n
        slots, cp = self.pool.append_tokens(sid, prompt[n:])
        mslots, mcp = self.model.append_tokens(sid, prompt[n:])
        assert slots.tolist() == mslots and cp == mcp and cp is None
        self._write(sid, n, prompt[n:], slots)
        self.tokens[sid] = list(prompt)
        return sid

    def fork(self, sid):
        child = self.next_id
        self.next_id += 1
        self.pool.fork(sid, child)
        self.model.fork(sid, child)
        self.tokens[child] = list(self.tokens[sid])
        return child

    def finish(self, sid):
        self.pool.free_seq(sid)
        self.model.free_seq(sid)
        del self.tokens[sid]

    def step(self):
        """One decode token for every live sequence: copies first, then the new rows."""
        live = sorted(self.tokens)
        toks = [int(x) for x in self.gen.integers(0, 4, size=len(live))]
        slots, copies = self.pool.append_batch_tokens(live, toks)
        mslots, mcopies = self.model.append_batch_tokens(live, toks)
        assert slots.tolist() == mslots and [tuple(c) for c in copies.tolist()] == mcopies
        self._copy(copies)
        for i, sid in enumerate(live):
            self._write(sid, len(self.tokens[sid]), [toks[i]], [slots[i]])
            self.tokens[sid].append(toks[i])

    def check_decode(self, P, step):
        w = self.w
        live = sorted(self.tokens)
        lens = [len(self.tokens[s]) for s in live]
        mb = max(-(-n // self.bs) for n in lens)
        tables, tl = self.pool.build_tables(live, mb)
        mt, ml = self.model.tables(live, mb)
        assert np.array_equal(tables, mt) and np.array_equal(tl, ml)
        q = workloads.draw_q(w, workloads.rng(w.seed, 41, step), batch=len(live))
        out = torch.full((len(live), w.num_heads, w.head_dim), float("nan"), device=self.dev)
        parts = None
        if P != 0:
            parts = pkv.alloc_partials(len(live), w.num_heads, w.head_dim,
                                       pkv.max_partitions_for(mb, P, self.bs), self.dev)
        pkv.decode(out, q.to(self.dev), self.kc, self.vc, torch.from_numpy(tables).to(self.dev),
                   torch.from_numpy(tl).to(self.dev), w.scale, P, parts,
                   kv_scales=(w.k_scale, w.v_scale) if w.cache_dtype == "fp8" else None)
        torch.cuda.synchronize()
        qf = oracle.to_f64(q, w.dtype)
        ref = np.empty((len(live), w.num_heads, w.head_dim))
        for i, sid in enumerate(live):
            n = lens[i]
            k, v = self._rows(list(range(n)), self.tokens[sid])
            if w.cache_dtype == "fp8":
                K = oracle.to_f64(oracle.fp8_quantize(k, w.dtype, w.k_scale), "fp8") * w.k_scale
                V = oracle.to_f64(oracle.fp8_quantize(v, w.dtype, w.v_scale), "fp8") * w.v_scale
            else:
                K, V = oracle.to_f64(k, w.dtype), oracle.to_f64(v, w.dtype)
            for h in range(w.num_heads):
                g = h // w.group
                ref[i, h] = oracle.attend(qf[i, h], K[:, g].copy(), V[:, g].copy(), w.scale)[0]
        check_close(out.cpu().double().numpy(), ref, w.dtype, f"step {step}")


SHAPE = dataclasses.replace(workloads.WORKLOADS["llama8b"], num_heads=8, num_kv_heads=2,
                            head_dim=64, num_blocks=0)


@pytest.mark.parametrize("kv,P,bs", [("bf16", 0, 16), ("bf16", AUTO, 16), ("fp8", 0, 16),
                                     ("bf16", AUTO, 8), ("fp8", 32, 32)],
                         ids=["bf16-single", "bf16-auto", "fp8-single", "bf16-auto-bs8",
                              "fp8-p32-bs32"])
def test_decode_through_prefix_hits_forks_and_copies(kv, P, bs, device):
    w = dataclasses.replace(SHAPE, block_size=bs)
    if kv == "fp8":
        w = dataclasses.replace(w, kv_dtype="fp8", k_scale=0.02, v_scale=0.015)
    s = Serving(w, device)
    gen = s.gen
    # prompts several blocks long at every block size, so repeated prefixes cover full
    # blocks (at 32 tokens per block a 40-token prompt holds one)
    n0 = 40 if bs <= 16 else 100
    a = s.admit([int(x) for x in gen.integers(0, 4, size=n0)])
    s.admit(s.tokens[a][:n0 - 3] + [int(x) for x in gen.integers(0, 4, size=10)])
    first_hit = (n0 - 3) // bs * bs
    assert s.hit_tokens == first_hit             # the full blocks of the n0 - 3 shared tokens
    s.fork(a)                                    # shares A's last block (partly filled at 16, 32)
    for step in range(24):
        s.step()
        s.check_decode(P, step)
        r = gen.random()
        live = sorted(s.tokens)
        if r < 0.3:
            s.fork(live[int(gen.integers(len(live)))])
        elif r < 0.5 and len(live) > 2:
            s.finish(live[int(gen.integers(len(live)))])
        elif r < 0.8:                            # a request repeating a live one's prefix
            src = s.tokens[live[int(gen.integers(len(live)))]]
            cut = int(gen.integers(1, len(src) + 1))
            s.admit(src[:cut] + [int(x) for x in gen.integers(0, 4, size=int(gen.integers(1, 9)))])
    assert s.copies > 0
    assert s.hit_tokens > first_hit              # later requests found cached blocks too
    st, ms = s.pool.stats(), s.model.stats()
    assert st["prefix_hits"] == ms["prefix_hits"] and st["cached"] == ms["cached"]
