"""Pins for the oracle's multi-query (chunked prefill) attention.

The pages split a long prompt into chunks that are processed over several steps, the
chunk's K/V joining the cache before its queries attend ("vLLM Nedir? PagedAttention ile
Production LLM Serving", section "Chunked prefill"; "Yerel LLM sistemlerinde backpressure
ve ölçekleme", section "4. Prefill ve decode"). The attention of each query is the
ordinary causal attention of the prompt, whatever the chunking:
  * a whole prompt equals torch's scaled_dot_product_attention with is_causal (fp64, GQA);
  * a chunk that ends a longer context equals SDPA with the explicit causal mask of its
    rows (query i of an L-token chunk of an n-token context sees positions 0 .. n-L+i);
  * single-query rows are bit-identical to the decode oracle;
  * a chunk claiming more tokens than its sequence holds leaves zero rows.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import paged_batch
import workloads

torch = pytest.importorskip("torch")

W = dataclasses.replace(workloads.WORKLOADS["llama8b"], num_heads=8, num_kv_heads=2,
                        head_dim=64, num_blocks=0)


def _queries(lens_q, seed=3):
    gen = workloads.rng(W.seed, 50, seed)
    q = workloads.draw_q(W, gen, batch=int(sum(lens_q)))
    qs = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    return q, qs


def _sdpa(qf, K, V, mask):
    """fp64 SDPA of queries [L][Hq][d] over K/V [n][Hkv][d] with a boolean [L][n] mask."""
    L, n = mask.shape
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qf).permute(1, 0, 2).unsqueeze(0),
        torch.from_numpy(K).permute(1, 0, 2).unsqueeze(0),
        torch.from_numpy(V).permute(1, 0, 2).unsqueeze(0),
        attn_mask=torch.from_numpy(mask), scale=W.scale, enable_gqa=True)
    return out[0].permute(1, 0, 2).numpy()


def test_whole_prompts_match_causal_sdpa():
    lens = [1, 16, 23, 70]
    ob = paged_batch.build(W, lens=lens)
    q, qs = _queries(lens)
    got = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    qf = oracle.to_f64(q, W.dtype)
    for b, n in enumerate(lens):
        K, V = ob.logical_kv(b)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf[qs[b]:qs[b + 1]]).permute(1, 0, 2).unsqueeze(0),
            torch.from_numpy(K).permute(1, 0, 2).unsqueeze(0),
            torch.from_numpy(V).permute(1, 0, 2).unsqueeze(0),
            is_causal=True, scale=W.scale, enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[qs[b]:qs[b + 1]], ref, rtol=0, atol=1e-13)


def test_chunks_ending_a_longer_context_match_masked_sdpa():
    lens = [40, 97, 130]
    chunk = [7, 33, 16]
    ob = paged_batch.build(W, lens=lens)
    q, qs = _queries(chunk)
    got = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    qf = oracle.to_f64(q, W.dtype)
    for b, (n, L) in enumerate(zip(lens, chunk)):
        K, V = ob.logical_kv(b)
        mask = np.arange(n)[None, :] <= (n - L + np.arange(L))[:, None]
        ref = _sdpa(qf[qs[b]:qs[b + 1]], K, V, mask)
        np.testing.assert_allclose(got[qs[b]:qs[b + 1]], ref, rtol=0, atol=1e-13)


def test_single_query_rows_are_the_decode_oracle():
    lens = [1, 17, 64, 200]
    ob = paged_batch.build(W, lens=lens)
    q, qs = _queries([1] * len(lens))
    got = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    dec = oracle.decode(q, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    assert np.array_equal(got, dec)


def test_rows_before_the_first_position_are_zero():
    lens = [5]
    ob = paged_batch.build(W, lens=lens)
    q, qs = _queries([8])                       # 8 queries, only 5 positions
    got = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    assert np.all(got[:3] == 0) and np.all(np.abs(got[3:]).sum(axis=-1) > 0)
    K, V = ob.logical_kv(0)
    mask = np.arange(5)[None, :] <= np.arange(5)[:, None]
    ref = _sdpa(oracle.to_f64(q, W.dtype)[3:], K, V, mask)
    np.testing.assert_allclose(got[3:], ref, rtol=0, atol=1e-13)


def test_sampled_rows_match_full_output():
    lens = [50, 90]
    ob = paged_batch.build(W, lens=lens)
    q, qs = _queries([20, 31])
    full = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype)
    rows = [(0, 0), (19, 7), (20, 3), (50, 5)]
    some = oracle.prefill(q, qs, ob.k_cache, ob.v_cache, ob.tables, ob.lens, W.scale, W.dtype,
                          rows=rows)
    for k, (r, h) in enumerate(rows):
        assert np.array_equal(some[k], full[r, h])
