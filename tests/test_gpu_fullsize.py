"""Full-size parity: one layer of each workload at its real size, in the launch mode the
bench uses for it (the 8B single pass with the step's host plan) and in the balanced split,
and the 8B workload at 8 and 32 tokens per block, checked on sampled outputs; for the 8B
and 70B workloads also layers 1, the last and two seeded random ones in the bench's mode.

* slots and block tables: every one, bit-exact against the oracle's pool model;
* cache write: a random sample of tokens read back through the documented layout,
  bit-exact against the rows that were written (FP8 cache: against the oracle's codes of
  those rows);
* attention: sampled (sequence, head) rows against the oracle's textbook attention over
  the sequence's logical K/V (paged equals contiguous is pinned in the oracle tests),
  max |err| <= 2e-3 on fp32 output (inputs fp16/bf16) and max|err|/max|ref| <= 1e-3.

Inputs are drawn on the GPU by workloads.draw_*_device and copied to the host for the
oracle; nothing the oracle reads comes from the HIP path.
"""
import numpy as np
import pytest
import torch

import gpu_batch
import oracle
import paged_kv_cache_28_amd as pkv
import workloads

pytestmark = pytest.mark.gpu
W = workloads.WORKLOADS
AUTO = pkv.PKV_PARTITION_AUTO


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


class Layer:
    """One layer of a workload through the library, with its oracle-side twin state."""

    def __init__(self, w, device, layer=0, block_size=16):
        self.w = w
        self.bs = bs = block_size
        lens = workloads.draw_seq_lens(w).astype(np.int64)
        B, Hkv, d = len(lens), w.num_kv_heads, w.head_dim
        nb = workloads.pool_blocks_for(lens, block_size=bs)
        order = workloads.draw_free_order(nb, workloads.rng(w.seed, 1, layer))
        pool = pkv.kv_pool_create(nb, 1, Hkv, d, w.cache_dtype, free_order=order, block_size=bs)
        model = oracle.PoolModel(nb, order, block_size=bs)
        prompt = np.maximum(lens - 1, 0)
        ps_p, ps_m = [], []
        for b in range(B):
            pool.add_seq(b)
            model.add_seq(b)
            ps_p.append(pool.append(b, int(prompt[b])))
            ps_m += model.append(b, int(prompt[b]))
        self.prompt_slots = np.concatenate(ps_p).astype(np.int32)
        assert np.array_equal(self.prompt_slots, np.asarray(ps_m, np.int32)), "prompt slots"
        self.new_slots = pool.append_batch(list(range(B)))
        assert self.new_slots.tolist() == [model.append(b, 1)[0] for b in range(B)], "new slots"
        self.max_blocks = int(-(-lens.max() // bs))
        self.tables, self.lens = pool.build_tables(list(range(B)), self.max_blocks)
        mt, ml = model.tables(list(range(B)), self.max_blocks)
        assert np.array_equal(self.tables, mt) and np.array_equal(self.lens, ml), "tables"
        self.offsets = np.concatenate([[0], np.cumsum(prompt)])
        # inputs, on the device
        self.pk = workloads.draw_tokens_device(int(prompt.sum()), w, (2, layer, 0), device)
        self.pv = workloads.draw_tokens_device(int(prompt.sum()), w, (2, layer, 1), device)
        self.nk = workloads.draw_tokens_device(B, w, (2, layer, 2), device)
        self.nv = workloads.draw_tokens_device(B, w, (2, layer, 3), device)
        self.q = workloads.draw_q_device(w, (3, layer), device)
        self.fp8 = w.cache_dtype == "fp8"
        self.kc, self.vc = gpu_batch.guarded_caches(nb, Hkv, d, w.cache_dtype, device,
                                                    0x7F if self.fp8 else float("nan"), bs)
        for k, v, sl in ((self.pk, self.pv, self.prompt_slots), (self.nk, self.nv, self.new_slots)):
            sl = torch.from_numpy(sl).to(device)
            if self.fp8:
                pkv.reshape_and_cache_fp8(k, v, self.kc, self.vc, sl, w.k_scale, w.v_scale)
            else:
                pkv.reshape_and_cache(k, v, self.kc, self.vc, sl)
        self.tables_d = torch.from_numpy(self.tables).to(device)
        self.lens_d = torch.from_numpy(self.lens).to(device)
        self.num_blocks = nb
        self.device = device

    def decode(self, P, plan=False):
        w, dev = self.w, self.device
        B = len(self.lens)
        out = gpu_batch.guarded_full((B, w.num_heads, w.head_dim), float("nan"), torch.float32,
                                     dev)
        parts = None
        if P != 0:
            maxp = pkv.max_partitions_for(self.max_blocks, P, self.bs)
            parts = gpu_batch.guarded_partials(B, w.num_heads, w.head_dim, maxp, dev)
        order = pkv.paged_attention_decode_plan(self.lens, w.num_kv_heads) if plan else None
        pkv.decode(out, self.q, self.kc, self.vc, self.tables_d, self.lens_d, w.scale, P, parts,
                   kv_scales=(w.k_scale, w.v_scale) if self.fp8 else None, seq_order=order)
        gpu_batch.check_guards()
        return out

    def logical_kv(self, b, g):
        """fp64 logical K, V [n_b][d] of (sequence b, KV head g) from the drawn inputs."""
        lo, hi = int(self.offsets[b]), int(self.offsets[b + 1])
        k = torch.cat([self.pk[lo:hi, g], self.nk[b:b + 1, g]]).cpu()
        v = torch.cat([self.pv[lo:hi, g], self.nv[b:b + 1, g]]).cpu()
        w = self.w
        if self.fp8:   # the values the cache holds: the oracle's codes, dequantised
            return (oracle.to_f64(oracle.fp8_quantize(k, w.dtype, w.k_scale), "fp8") * w.k_scale,
                    oracle.to_f64(oracle.fp8_quantize(v, w.dtype, w.v_scale), "fp8") * w.v_scale)
        return oracle.to_f64(k, w.dtype), oracle.to_f64(v, w.dtype)

    def check_cache_sample(self, n=4096, seed=0):
        """Read a random sample of written tokens back through the documented layout."""
        w = self.w
        x = 16 // w.cache_elem_bytes if self.fp8 else (8 if w.elem_bytes == 2 else 4)
        gen = np.random.default_rng(seed)
        T = len(self.prompt_slots)
        pick = gen.choice(T, size=min(n, T), replace=False) if T else np.zeros(0, np.int64)
        bs = self.bs
        slots = torch.from_numpy(self.prompt_slots[pick].astype(np.int64)).to(self.device)
        blk, off = slots // bs, slots % bs
        kv = self.kc.view(self.num_blocks, w.num_kv_heads, w.head_dim // x, bs, x)
        got_k = kv[blk, :, :, off, :].reshape(len(pick), w.num_kv_heads, w.head_dim)
        got_v = self.vc[blk, :, :, off]
        idx = torch.from_numpy(pick).to(self.device)
        nslots = torch.from_numpy(self.new_slots.astype(np.int64)).to(self.device)
        got_nk = kv[nslots // bs, :, :, nslots % bs, :].reshape(-1, w.num_kv_heads, w.head_dim)
        got_nv = self.vc[nslots // bs, :, :, nslots % bs]
        if self.fp8:
            def codes(x, sc):
                return torch.from_numpy(oracle.fp8_quantize(x.cpu(), w.dtype, sc))
            assert torch.equal(got_k.cpu(), codes(self.pk[idx], w.k_scale))
            assert torch.equal(got_v.cpu(), codes(self.pv[idx], w.v_scale))
            assert torch.equal(got_nk.cpu(), codes(self.nk, w.k_scale))
            assert torch.equal(got_nv.cpu(), codes(self.nv, w.v_scale))
            return
        assert torch.equal(got_k.view(torch.int16), self.pk[idx].view(torch.int16))
        assert torch.equal(got_v.view(torch.int16), self.pv[idx].view(torch.int16))
        assert torch.equal(got_nk.view(torch.int16), self.nk.view(torch.int16))
        assert torch.equal(got_nv.view(torch.int16), self.nv.view(torch.int16))

    def sample_rows(self, n_random, seed=1):
        w = self.w
        gen = np.random.default_rng(seed)
        B = len(self.lens)
        longest, shortest = int(np.argmax(self.lens)), int(np.argmin(self.lens))
        rows = {(longest, h) for h in range(w.num_heads)}
        rows |= {(shortest, h) for h in range(0, w.num_heads, max(1, w.group // 2))}
        for _ in range(n_random):
            rows.add((int(gen.integers(B)), int(gen.integers(w.num_heads))))
        return sorted(rows)

    def check_rows(self, out, rows):
        w = self.w
        qf = oracle.to_f64(self.q.cpu(), w.dtype)
        got = out.cpu().double().numpy()
        errs, refs = [], []
        kv_key, K, V = None, None, None      # rows are sorted: reuse one (b, g) at a time
        for b, h in rows:
            g = h // w.group
            if kv_key != (b, g):
                kv_key = (b, g)
                K, V = self.logical_kv(b, g)
            ref, _, _ = oracle.attend(qf[b, h], K, V, w.scale)
            errs.append(np.abs(got[b, h] - ref).max())
            refs.append(np.abs(ref).max())
        err, scale = max(errs), max(refs)
        assert np.all(np.isfinite(got)), "non-finite output"
        assert err <= 2e-3, f"max|err| {err:.3e} over {len(rows)} sampled rows"
        assert err / scale <= 1e-3, f"normalised error {err / scale:.3e}"
        return err


# (workload, partition size, random rows, block size, host plan)
CASES = [("llama8b", 0, 0, 16, True), ("llama8b", 0, 0, 16, False), ("llama8b", AUTO, 0, 16, False),
         ("llama8b_fp8", 0, 48, 16, True), ("llama8b_fp8", AUTO, 48, 16, False),
         ("llama8b", 0, 0, 8, True), ("llama8b", AUTO, 0, 32, False),
         ("llama8b_fp8", 0, 48, 32, True),
         ("llama70b", 512, 96, 16, False), ("llama70b", AUTO, 96, 16, False),
         ("long", 512, 24, 16, False), ("long", AUTO, 24, 16, False)]


@pytest.mark.parametrize("name,P,n_random,bs,plan", CASES,
                         ids=[f"{n}-{'auto' if p == AUTO else p}-bs{bs}{'-plan' if pl else ''}"
                              for n, p, _, bs, pl in CASES])
def test_full_size_layer(name, P, n_random, bs, plan, device):
    w = W[name]
    layer = Layer(w, device, block_size=bs)
    layer.check_cache_sample()
    out = layer.decode(P, plan)
    if name == "llama8b":
        rows = [(b, h) for b in range(w.batch) for h in range(w.num_heads)]
    else:
        rows = layer.sample_rows(n_random)
    layer.check_rows(out, rows)


def _other_layers(name):
    """Layer 1, the last layer and two seeded random layers in between (layer 0 is above)."""
    L = W[name].layers
    extra = np.random.default_rng(28).choice(np.arange(2, L - 1), size=2, replace=False)
    return [1, L - 1] + sorted(int(x) for x in extra)


# the bench's launch mode of each multi-layer workload: 8B single pass with the host plan,
# 70B balanced split
LAYER_CASES = ([("llama8b", 0, 0, True, layer) for layer in _other_layers("llama8b")] +
               [("llama70b", AUTO, 48, False, layer) for layer in _other_layers("llama70b")])


@pytest.mark.parametrize("name,P,n_random,plan,layer", LAYER_CASES,
                         ids=[f"{n}-layer{layer}" for n, _, _, _, layer in LAYER_CASES])
def test_full_size_other_layers(name, P, n_random, plan, layer, device):
    """Each layer has its own pool order and its own K/V and query draws."""
    w = W[name]
    lay = Layer(w, device, layer=layer)
    lay.check_cache_sample(seed=layer)
    out = lay.decode(P, plan)
    if name == "llama8b":
        rows = [(b, h) for b in range(w.batch) for h in range(w.num_heads)]
    else:
        rows = lay.sample_rows(n_random, seed=layer)
    lay.check_rows(out, rows)
