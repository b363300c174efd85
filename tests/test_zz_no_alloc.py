"""paged_attention_decode_noalloc: the partitioned decode and its reduce with the records in
the library's static per-device workspace, for callers that cannot allocate, against
paged_attention_decode + paged_attention_reduce with caller-owned buffers (the existing
entry points) on the same inputs, and against the fp64 oracle.

The call goes through the C ABI directly. Two calls in a row on one device, the second
with a smaller batch and shorter contexts, so the second reads a workspace the first
left filled: with the same partition count both paths run the same kernels on the same
plan and must agree bit for bit, and both meet the oracle bars (fp32 output within 2e-3,
max|err| / max|ref| <= 1e-3). Oversized requests are refused before any launch.
"""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import gpu_batch
import oracle
import paged_batch
import paged_kv_cache_28_amd as pkv
import workloads
from test_gpu_parity import check_close

pytestmark = pytest.mark.gpu
AUTO = pkv.PKV_PARTITION_AUTO
W8 = dataclasses.replace(workloads.WORKLOADS["llama8b"], num_blocks=0)

# first call, then a smaller second call on the same device
CALLS = [[3000, 700, 17, 0, 2048, 1, 4097, 513, 129, 64, 1999, 33],
         [40, 1, 300, 16, 5]]


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _noalloc(gb, w, P, out):
    B, Hq, d = gb.q.shape
    rc = pkv.lib().paged_attention_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(gb.q.data_ptr()), gb.q.stride(0),
        ctypes.c_void_p(gb.k_cache.data_ptr()), ctypes.c_void_p(gb.v_cache.data_ptr()),
        ctypes.c_void_p(gb.tables_d.data_ptr()), ctypes.c_void_p(gb.lens_d.data_ptr()), B, Hq,
        w.num_kv_heads, d, w.block_size, gb.tables.shape[1], gb.k_cache.shape[0], w.scale, P,
        pkv.dtype_code(gb.q.dtype), pkv.dtype_code(out.dtype),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("P", [512, 256, AUTO], ids=["p512", "p256", "auto"])
def test_noalloc_equals_caller_buffers(P, out_dtype, device):
    w = W8
    for i, lens in enumerate(CALLS):
        ob = paged_batch.build(w, lens=lens, seed_stream=30 + i)
        gb = gpu_batch.build(ob, device)
        B, Hq, d = gb.q.shape
        print(f"noalloc P={P} call {i}: B={B} max_len={max(lens)}", flush=True)
        got = gpu_batch.guarded_full((B, Hq, d), float("nan"), out_dtype, device)
        assert _noalloc(gb, w, P, got) == pkv.PKV_OK, pkv.lib().pkv_last_error()
        # the existing entry points with torch-allocated partials of the same count (the
        # natural bound fits the workspace at these sizes)
        ref_out = gpu_batch.guarded_full((B, Hq, d), float("nan"), out_dtype, device)
        maxp = pkv.max_partitions_for(gb.tables.shape[1], P)
        parts = gpu_batch.guarded_partials(B, Hq, d, maxp, device)
        pkv.decode(ref_out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, P,
                   parts)
        gpu_batch.check_guards()
        assert torch.equal(got.view(torch.uint8), ref_out.view(torch.uint8)), \
            (got.double() - ref_out.double()).abs().max().item()
        if out_dtype == torch.float32:
            ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
            check_close(got.cpu().double().numpy(), ref, w.dtype, f"noalloc P={P} call {i}")


def test_noalloc_single_pass_and_binding(device):
    """partition_size 0 (no workspace) through the Python binding equals the single pass."""
    w = W8
    ob = paged_batch.build(w, lens=CALLS[0], seed_stream=40)
    gb = gpu_batch.build(ob, device)
    a = torch.empty(gb.q.shape, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    pkv.paged_attention_decode_noalloc(a, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d,
                                       w.scale, 0)
    pkv.paged_attention_decode(b, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale)
    pkv.paged_attention_decode_noalloc(a, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d,
                                       w.scale, AUTO)
    torch.cuda.synchronize()
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    check_close(a.cpu().double().numpy(), ref, w.dtype, "noalloc auto via the binding")
    check_close(b.cpu().double().numpy(), ref, w.dtype, "single pass")


def test_noalloc_refuses_what_does_not_fit(device):
    """Fixed partitions whose records exceed the workspace: EINVAL, nothing launched (the
    output keeps its NaN fill). The 70B batch of 128 sequences x 64 heads at 512-token
    partitions over 34,000-token tables needs 67 records of 520 bytes per row, 285 MB."""
    ws = pkv.noalloc_workspace_bytes()
    assert ws == 64 << 20
    B, Hq, Hkv, d, mb = 128, 64, 8, 128, 2125
    kc, vc = pkv.alloc_caches(4, Hkv, d, "f16", device, fill=0.0)
    q = torch.zeros((B, Hq, d), dtype=torch.float16, device=device)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=device)
    tab = torch.full((B, mb), -1, dtype=torch.int32, device=device)
    lens = torch.zeros(B, dtype=torch.int32, device=device)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_decode_noalloc(out, q, kc, vc, tab, lens, 0.1, 512)
    assert e.value.code == pkv.PKV_EINVAL and "workspace" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # the balanced split lowers its record count to what fits instead
    pkv.paged_attention_decode_noalloc(out, q, kc, vc, tab, lens, 0.1, AUTO)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))   # every sequence is empty: zero rows
