"""The host-side decode plan (paged_attention_decode_plan, passed as seq_order) only
schedules: the single-pass decode gives bit-identical outputs, and the fused append
bit-identical caches, with the plan's order, with any other permutation and with none
(where the kernel ranks the lengths itself), for 16-bit and FP8 caches at every block
size."""
import dataclasses

import numpy as np
import pytest
import torch

import gpu_batch
import paged_batch
import paged_kv_cache_28_amd as pkv
import workloads
from test_gpu_parity import RAGGED

pytestmark = pytest.mark.gpu
B8 = workloads.WORKLOADS["llama8b"]


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(ob, w, device, order, append):
    gb = gpu_batch.build(ob, device, write_new=not append)
    B, Hq, d = gb.q.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=device)
    app = None
    if append:
        app = (ob.new_k.to(device), ob.new_v.to(device), torch.from_numpy(gb.new_slots).to(device))
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, 0, None,
               append=app, kv_scales=gpu_batch.kv_scales(w), seq_order=order)
    torch.cuda.synchronize()
    return out.cpu(), gb.k_cache.cpu(), gb.v_cache.cpu()


@pytest.mark.parametrize("append", [False, True], ids=["decode", "append"])
@pytest.mark.parametrize("kv,bs", [("bf16", 16), ("fp8", 16), ("bf16", 8), ("fp8", 32)])
def test_any_order_gives_identical_results(kv, bs, append, device):
    w = dataclasses.replace(B8, num_blocks=0, block_size=bs)
    if kv == "fp8":
        w = dataclasses.replace(w, kv_dtype="fp8", k_scale=0.02, v_scale=0.015)
    lens = RAGGED + [3, 900, 48, 1]
    ob = paged_batch.build(w, lens=lens)
    ref = _run(ob, w, device, None, append)
    plan = pkv.paged_attention_decode_plan(ob.lens, w.num_kv_heads)
    other = np.random.default_rng(4).permutation(len(lens)).astype(np.int32)
    for order in (plan, other):
        got = _run(ob, w, device, order, append)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert torch.isfinite(ref[0]).all()


def test_a_bad_order_is_rejected_before_launch(device):
    w = dataclasses.replace(B8, num_blocks=0)
    ob = paged_batch.build(w, lens=[5, 17, 40])
    gb = gpu_batch.build(ob, device)
    out = torch.empty(gb.q.shape, dtype=torch.float32, device=device)
    for bad in ([0, 0, 1], [0, 1, 3]):
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_attention_decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d,
                                       w.scale, seq_order=bad)
        assert e.value.code == pkv.PKV_EINVAL
