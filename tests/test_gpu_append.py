"""paged_attention_decode_append, the decode step in one call, against the two calls it
stands for (reshape_and_cache of the new tokens, then paged_attention_decode) and
against the oracle. The caches must agree bit for bit. The fused kernel puts the new
token into row n-1 of the newest tile in its registers, the values the two-call path
reads back from the cache, so the sums run in the same order and the outputs agree bit
for bit too; both meet the oracle tolerance."""
import numpy as np
import pytest
import torch

import gpu_batch
import oracle
import paged_batch
import paged_kv_cache_28_amd as pkv
from test_gpu_parity import RAGGED, SHAPES, TOL, _ulp, check_close

pytestmark = pytest.mark.gpu
AUTO = pkv.PKV_PARTITION_AUTO


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def _same_output(a, b):
    """Outputs of the two paths: finite and bit-identical."""
    assert torch.isfinite(a).all() and torch.isfinite(b).all()
    assert torch.equal(_bits(a), _bits(b)), (a.double() - b.double()).abs().max().item()


def _run(gb, w, P, out_dtype, append, plan=False):
    B, Hq, d = gb.q.shape
    dev = gb.q.device
    out = gpu_batch.guarded_full((B, Hq, d), float("nan"), out_dtype, dev)
    parts = None
    if P != 0:
        maxp = pkv.max_partitions_for(gb.tables.shape[1], P)
        parts = gpu_batch.guarded_partials(B, Hq, d, maxp, dev)
    order = pkv.paged_attention_decode_plan(gb.lens, w.num_kv_heads) if plan else None
    pkv.decode(out, gb.q, gb.k_cache, gb.v_cache, gb.tables_d, gb.lens_d, w.scale, P, parts,
               append=append, seq_order=order)
    gpu_batch.check_guards()   # outputs, partials and both caches: nothing written past them
    return out


def _pair(ob, w, P, device, out_dtype=torch.float32, pre_written=(), plan=False):
    """(two-call result, fused result): outputs and both caches of each path.
    Sequences in pre_written already hold their new row and pass slot -1. plan: both
    paths take the step's host plan (paged_attention_decode_plan) as seq_order."""
    res = []
    for fused in (False, True):
        gb = gpu_batch.build(ob, device, write_new=False)
        nk, nv = ob.new_k.to(device), ob.new_v.to(device)
        slots = gb.new_slots.copy()
        if len(pre_written):
            idx = np.asarray(pre_written)
            pkv.reshape_and_cache(nk[idx], nv[idx], gb.k_cache, gb.v_cache,
                                  torch.from_numpy(slots[idx]).to(device))
            slots[idx] = -1
        slots_d = torch.from_numpy(slots).to(device)
        if fused:
            out = _run(gb, w, P, out_dtype, (nk, nv, slots_d), plan)
        else:
            pkv.reshape_and_cache(nk, nv, gb.k_cache, gb.v_cache, slots_d)
            out = _run(gb, w, P, out_dtype, None, plan)
        res.append((out, gb.k_cache, gb.v_cache))
    return res


CASES = [(name, P) for name in ("8b-bf16", "70b-f16", "f16-d64-g16", "bf16-d64-g1")
         for P in (0, 64, AUTO)] + [("tiny-f32", 0), ("tiny-f32", 64)]


@pytest.mark.parametrize("name,P", CASES)
def test_append_equals_write_then_decode(name, P, device):
    w = SHAPES[name]
    ob = paged_batch.build(w, lens=RAGGED)
    (oa, ka, va), (ob_, kb, vb) = _pair(ob, w, P, device)
    assert torch.equal(_bits(ka), _bits(kb)) and torch.equal(_bits(va), _bits(vb)), "caches"
    _same_output(oa, ob_)
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    check_close(ob_.cpu().double().numpy(), ref, w.dtype, f"{name} P={P}")


@pytest.mark.parametrize("P", [0, 256, AUTO])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_append_with_cached_rows_and_bf16_out(P, out_dtype, device):
    """Half of the sequences pass slot -1 (their newest row is already cached), and the
    output is also produced in the input type."""
    w = SHAPES["8b-bf16"]
    ob = paged_batch.build(w, lens=RAGGED)
    pre = [b for b in range(len(RAGGED)) if b % 2 and RAGGED[b] > 0]
    (oa, ka, va), (ob_, kb, vb) = _pair(ob, w, P, device, out_dtype, pre_written=pre)
    assert torch.equal(_bits(ka), _bits(kb)) and torch.equal(_bits(va), _bits(vb))
    _same_output(oa, ob_)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_append_full_size_8b(out_dtype, device):
    """The 8B workload at full size in the bench's launch mode: the fused append with the
    step's host plan. Caches bit-exact against the oracle's cache write and the two-call
    path; every one of the 2,048 output rows against the fp64 oracle (fp32 output: the
    2e-3 and 1e-3 bars; bf16 output, what the bench writes: the fp32 bar plus half an
    output ulp)."""
    w = SHAPES["8b-bf16"]
    ob = paged_batch.build(w)
    (oa, ka, va), (ob_, kb, vb) = _pair(ob, w, w.partition_size, device, out_dtype, plan=True)
    assert torch.equal(_bits(ka), _bits(kb)) and torch.equal(_bits(va), _bits(vb))
    assert np.array_equal(oracle.raw(kb), ob.k_cache) and np.array_equal(oracle.raw(vb), ob.v_cache)
    _same_output(oa, ob_)
    ref = oracle.decode(ob.q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, w.scale, w.dtype)
    got = ob_.cpu().double().numpy()
    assert got.shape[0] * got.shape[1] == 2048
    if out_dtype == torch.float32:
        check_close(got, ref, w.dtype, "8B fused + plan")
    else:
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - ref) <= TOL["bf16"] + 0.5 * _ulp(got, "bf16"))


def test_append_validation(device):
    w = SHAPES["8b-bf16"]
    ob = paged_batch.build(w, lens=[5, 17])
    gb = gpu_batch.build(ob, device, write_new=False)
    out = torch.empty(gb.q.shape, dtype=torch.float32, device=device)
    nk, nv = ob.new_k.to(device), ob.new_v.to(device)
    slots = torch.from_numpy(gb.new_slots).to(device)
    L = pkv.lib()
    args = [out.data_ptr(), None, None, None, gb.q.data_ptr(), gb.q.stride(0), nk.data_ptr(),
            nv.data_ptr(), nk.stride(0), nv.stride(0), slots.data_ptr(), gb.k_cache.data_ptr(),
            gb.v_cache.data_ptr(), gb.tables_d.data_ptr(), gb.lens_d.data_ptr(), 2, w.num_heads,
            w.num_kv_heads, w.head_dim, 16, gb.tables.shape[1], gb.k_cache.shape[0], w.scale, 0,
            0, pkv.PKV_BF16, pkv.PKV_F32, None, None]
    bad = list(args); bad[10] = None                      # no slot_mapping
    assert L.paged_attention_decode_append(*bad) == pkv.PKV_EINVAL
    bad = list(args); bad[8] = w.num_kv_heads * w.head_dim - 8   # key stride too short
    assert L.paged_attention_decode_append(*bad) == pkv.PKV_EINVAL
    bad = list(args); bad[6] = nk.data_ptr() + 2          # misaligned key
    assert L.paged_attention_decode_append(*bad) == pkv.PKV_EINVAL
    assert L.paged_attention_decode_append(*args) == pkv.PKV_OK
    torch.cuda.synchronize()
