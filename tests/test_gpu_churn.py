"""Churn workload on the GPU: the 8B shape with a ~200 GB-class pool (one layer of it,
95,367 blocks = 6.25 GB), 256 live sequences, 20% sharing a 1,024-token prefix,
log-uniform prompts in [16, 32768], ~5% retired and admitted per step.

Checked after several steps: every slot, table, reference count and the free-queue order
against the oracle's pool model; decode (balanced split, as the workload runs it, and
fixed 512-token partitions) on sampled rows, including rows of sharers, against the
oracle's attention over each sequence's logical K/V.
"""
import numpy as np
import pytest
import torch

import churn_driver
import oracle
import paged_kv_cache_28_amd as pkv
import workloads

pytestmark = pytest.mark.gpu
AUTO = pkv.PKV_PARTITION_AUTO


@pytest.fixture(scope="module")
def churn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = churn_driver.Churn(workloads.WORKLOADS["churn"], torch.device("cuda:0"))
    for _ in range(3):
        c.step()
    torch.cuda.synchronize()
    return c


def test_pool_state_matches_model_after_churn(churn):
    churn.check_pool_state()
    churn.tables()
    st = churn.pool.stats()
    assert st["num_seqs"] == 257                       # 256 live + the shared prefix
    assert st["shared"] == churn.w.prefix_tokens // 16  # the prefix blocks
    n_sharers = sum(churn.sharer[s] for s in churn.live)
    blocks = churn.pool.seq_blocks(churn_driver.PREFIX_ID)
    assert all(churn.pool.refcount(b) == 1 + n_sharers for b in blocks)


@pytest.mark.parametrize("P", [AUTO, 512])
def test_churn_decode_matches_oracle(churn, P):
    w = churn.w
    tables, lens = churn.tables()
    B = len(churn.live)
    dev = churn.device
    q = workloads.draw_q_device(w, (8, churn.steps), dev, batch=B)
    out = torch.full((B, w.num_heads, w.head_dim), float("nan"), dtype=torch.float32, device=dev)
    maxp = pkv.max_partitions_for(tables.shape[1], P)
    parts = pkv.alloc_partials(B, w.num_heads, w.head_dim, maxp, dev)
    pkv.decode(out, q, churn.kc, churn.vc, torch.from_numpy(tables).to(dev),
               torch.from_numpy(lens).to(dev), w.scale, P, parts)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    qf = oracle.to_f64(q.cpu(), w.dtype)
    gen = np.random.default_rng(3)
    sharers = [i for i, s in enumerate(churn.live) if churn.sharer[s]]
    rows = {(int(np.argmax(lens)), h) for h in range(0, w.num_heads, 3)}
    rows |= {(sharers[0], h) for h in range(w.num_heads)}
    rows |= {(int(gen.integers(B)), int(gen.integers(w.num_heads))) for _ in range(48)}
    err, scale = 0.0, 0.0
    for b, h in sorted(rows):
        K, V = churn.logical_kv(churn.live[b], h // w.group)
        assert K.shape[0] == lens[b]
        ref, _, _ = oracle.attend(qf[b, h], K, V, w.scale)
        err = max(err, float(np.abs(got[b, h] - ref).max()))
        scale = max(scale, float(np.abs(ref).max()))
    assert err <= 2e-3 and err / scale <= 1e-3, (err, scale)
