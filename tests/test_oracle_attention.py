"""Pins for the oracle's attention math, each against something other than the oracle.

* closed forms (one token; zero query; equal keys; one dominant logit),
* a library routine on the same data (torch scaled_dot_product_attention in fp64,
  with enable_gqa for the query-head -> KV-head grouping),
* exact brute force on tiny inputs (mpmath at 50 digits),
* the split-over-context identity, checked against scipy's logsumexp.

The attention being pinned is ordinary scaled dot-product attention; paging changes
only where K and V come from ("vLLM ve Triton ile maliyet optimizasyonu", §03 Yöntem,
closing paragraphs).
"""
import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ------------------------------------------------------------------ closed forms
def test_single_token_returns_its_value_row():
    q, K, V = _rand(16), _rand(1, 16), _rand(1, 16)
    o, m, l = oracle.attend(q, K, V, 0.25)
    assert np.array_equal(o, V[0])
    assert l == 1.0
    assert m == pytest.approx(0.25 * float(q @ K[0]), rel=1e-15)


def test_zero_query_is_mean_of_values():
    n, d = 37, 8
    K, V = _rand(n, d), _rand(n, d)
    o, m, l = oracle.attend(np.zeros(d), K, V, 0.5)
    assert m == 0.0 and l == float(n)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=0, atol=1e-15)


def test_equal_keys_is_mean_of_values():
    n, d = 23, 8
    k = _rand(d)
    K, V = np.tile(k, (n, 1)), _rand(n, d)
    o, _, _ = oracle.attend(_rand(d), K, V, 0.3)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=0, atol=1e-15)


def test_dominant_logit_selects_its_value_row():
    n, d = 19, 8
    K, V = _rand(n, d), _rand(n, d)
    q = np.zeros(d)
    q[0] = 1.0
    K[:, 0] = 0.0
    K[7, 0] = 1e4          # logit of token 7 is 1e4 above every other one
    o, m, l = oracle.attend(q, K, V, 1.0)
    assert np.array_equal(o, V[7])
    assert m == 1e4 and l == 1.0


def test_empty_context_is_zero():
    o, m, l = oracle.attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.array_equal(o, np.zeros(4)) and m == -math.inf and l == 0.0


def test_scale_enters_once_and_linearly():
    """Doubling q with half the scale gives the same logits (a scale applied twice,
    or to V, would break this)."""
    n, d = 30, 16
    q, K, V = _rand(d), _rand(n, d), _rand(n, d)
    a, ma, _ = oracle.attend(q, K, V, 0.125)
    b, mb, _ = oracle.attend(2 * q, K, V, 0.0625)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)
    assert ma == pytest.approx(mb, rel=1e-15)


# ------------------------------------------------------------ library special case
@pytest.mark.parametrize("n,d,G", [(1, 64, 4), (37, 64, 1), (300, 128, 4), (513, 128, 8)])
def test_matches_torch_sdpa_fp64(n, d, G):
    torch = pytest.importorskip("torch")
    Hkv = 2
    Hq = Hkv * G
    q = _rand(Hq, d)
    K, V = _rand(Hkv, n, d), _rand(Hkv, n, d)
    scale = 1.0 / math.sqrt(d)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).view(1, Hq, 1, d), torch.from_numpy(K).view(1, Hkv, n, d),
        torch.from_numpy(V).view(1, Hkv, n, d), scale=scale, enable_gqa=True)
    ref = ref.view(Hq, d).numpy()
    for h in range(Hq):
        o, _, _ = oracle.attend(q[h], K[h // G], V[h // G], scale)
        np.testing.assert_allclose(o, ref[h], rtol=0, atol=1e-13)


# ------------------------------------------------------------- exact brute force
def test_matches_high_precision_brute_force():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    for n in (1, 2, 3, 17, 40):
        d = 4
        q, K, V = _rand(d), _rand(n, d), _rand(n, d)
        scale = 0.7
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i]) * mpmath.mpf(K[t, i])
                                             for i in range(d)) for t in range(n)]
        z = mpmath.fsum(mpmath.exp(x) for x in s)
        exact = [mpmath.fsum(mpmath.exp(s[t]) / z * mpmath.mpf(V[t, i]) for t in range(n))
                 for i in range(d)]
        o, m, l = oracle.attend(q, K, V, scale)
        for i in range(d):
            assert abs(o[i] - float(exact[i])) <= 1e-14 * max(1.0, abs(float(exact[i])))
        assert abs(m + math.log(l) - float(mpmath.log(z))) < 1e-13


# --------------------------------------------------------------------- split-K
def test_partition_results_match_logsumexp_and_merge_to_single_pass():
    scipy_special = pytest.importorskip("scipy.special")
    n, d, P = 1000, 32, 128
    q, K, V = _rand(d), _rand(n, d), _rand(n, d)
    scale = 1.0 / math.sqrt(d)
    full, _, _ = oracle.attend(q, K, V, scale)
    np_ = -(-n // P)
    O = np.zeros((1, np_ + 2, d))
    M = np.full((1, np_ + 2), -np.inf)
    L = np.zeros((1, np_ + 2))
    for p in range(np_):
        sl = slice(p * P, min(n, (p + 1) * P))
        O[0, p], M[0, p], L[0, p] = oracle.attend(q, K[sl], V[sl], scale)
        logits = scale * (K[sl] @ q)
        assert M[0, p] == pytest.approx(logits.max(), rel=1e-14)
        assert M[0, p] + math.log(L[0, p]) == pytest.approx(scipy_special.logsumexp(logits),
                                                            rel=1e-13)
    merged = oracle.merge(O, M, L, [np_])[0]
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-14)
    # merging in another order gives the same answer
    perm = RNG.permutation(np_)
    merged2 = oracle.merge(O[:, list(perm) + [np_, np_ + 1]], M[:, list(perm) + [np_, np_ + 1]],
                           L[:, list(perm) + [np_, np_ + 1]], [np_])[0]
    np.testing.assert_allclose(merged2, full, rtol=0, atol=1e-14)


def test_merge_of_one_partition_is_identity():
    q, K, V = _rand(8), _rand(50, 8), _rand(50, 8)
    o, m, l = oracle.attend(q, K, V, 0.4)
    merged = oracle.merge(o.reshape(1, 1, 8), np.array([[m]]), np.array([[l]]), [1])[0]
    np.testing.assert_allclose(merged, o, rtol=1e-15, atol=0)


def test_merge_of_no_partition_is_zero():
    out = oracle.merge(np.ones((1, 3, 4)), np.zeros((1, 3)), np.ones((1, 3)), [0])
    assert np.array_equal(out, np.zeros((1, 4)))


# ------------------------------------------------------------ element conversion
def test_half_conversion_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.to_f64(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_conversion_matches_torch_for_every_bit_pattern():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
