"""Pins of the dropout oracle: the Philox4x32-10 generator and attention with dropout on P.

The generator is pinned by its published known-answer vectors; the attention by the p = 0
reduction to the undropped definition, central finite differences of the backward with the mask
held fixed, the keep rate, and unbiasedness over many seeds.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as att
from oracle import dropout as dr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(*words):
    return np.random.default_rng(np.random.SeedSequence(list(words)))


def _kat():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        return json.load(f)["vectors"]


@pytest.mark.parametrize("vec", _kat())
def test_philox_known_answers(vec):
    ctr = [int(x, 16) for x in vec["counter"]]
    key = [int(x, 16) for x in vec["key"]]
    out = [int(x, 16) for x in vec["output"]]
    assert list(dr.philox4x32_10(ctr, key)) == out
    words = dr.philox4x32_10_np(*[np.array([c]) for c in ctr], *key)
    assert [int(w[0]) for w in words] == out


def test_philox_vectorised_equals_scalar():
    r = _rng(91, 1)
    c = r.integers(0, 2**32, size=(4, 50), dtype=np.uint64)
    key = (0x12345678, 0x9ABCDEF0)
    words = dr.philox4x32_10_np(c[0], c[1], c[2], c[3], *key)
    for n in range(50):
        assert tuple(int(w[n]) for w in words) == dr.philox4x32_10([int(x[n]) for x in c], key)


def test_keep_mask_layout_and_rate():
    # key j of row i takes 16-bit field j % 8 of the generator at counter (j // 8, i, bh, 0):
    # fields 0..3 are the low halves of words 0..3, fields 4..7 their high halves
    seed = 0x0123456789ABCDEF
    keys = np.arange(24)
    thr = dr.threshold(0.5)
    assert thr == 2**15
    for p in (0.5, 0.3):
        m = dr.keep_mask(seed, p, 7, [3], keys)[0]
        t = dr.threshold(p)
        for j in keys:
            w = dr.philox4x32_10((j // 8, 3, 7, 0), (seed & 0xFFFFFFFF, seed >> 32))
            x = (w[j % 4] & 0xFFFF) if j % 8 < 4 else (w[j % 4] >> 16)
            assert x == dr.keep_field(w, j)
            assert bool(m[j]) == (x >= t)
    # one call's 128 bits decide 8 keys: keys 8g .. 8g + 7 share a counter, the next 8 do not
    w0 = dr.philox4x32_10((0, 3, 7, 0), (seed & 0xFFFFFFFF, seed >> 32))
    w1 = dr.philox4x32_10((1, 3, 7, 0), (seed & 0xFFFFFFFF, seed >> 32))
    assert [dr.keep_field(w0, j) for j in range(8)] != [dr.keep_field(w1, j) for j in range(8, 16)]
    # rate: binomial, 5 sigma
    for p in (0.1, 0.5, 0.9):
        mask = dr.keep_mask(1234, p, 0, np.arange(256), np.arange(4096))
        n = mask.size
        sigma = math.sqrt(n * p * (1 - p))
        assert abs(mask.sum() - n * (1 - p)) < 5 * sigma
    assert dr.keep_mask(99, 0.0, 3, np.arange(64), np.arange(300)).all()
    with pytest.raises(ValueError):
        dr.threshold(1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_the_definition(causal):
    r = _rng(91, 2, int(causal))
    q, k, v, do = (r.standard_normal((37, 8)) for _ in range(4))
    o, lse = dr.forward_slice(q, k, v, 0.3, causal, 0.0, 5, 0)
    o_ref, lse_ref = att.forward_slice(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)
    g = dr.backward_slice(q, k, v, do, 0.3, causal, 0.0, 5, 0)
    g_ref = att.backward_slice(q, k, v, do, 0.3, causal)
    for a, b in zip(g, g_ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_is_the_undropped_statistic(causal):
    r = _rng(91, 3)
    q, k, v = (r.standard_normal((20, 4)) for _ in range(3))
    _, lse = dr.forward_slice(q, k, v, 0.5, causal, 0.4, 77, 1)
    _, lse_ref = att.forward_slice(q, k, v, 0.5, causal)
    np.testing.assert_array_equal(lse, lse_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences_with_fixed_mask(causal):
    r = _rng(91, 4, int(causal))
    n, d, scale, p, seed, bh = 6, 3, 0.7, 0.35, 2024, 5
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))

    def loss(q_, k_, v_):
        o, _ = dr.forward_slice(q_, k_, v_, scale, causal, p, seed, bh)
        return float(np.sum(o * do))

    dq, dk, dv = dr.backward_slice(q, k, v, do, scale, causal, p, seed, bh)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros((n, d))
        for i in range(n):
            for j in range(d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][i, j] += h
                args_m[which][i, j] -= h
                num[i, j] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1e-12, np.max(np.abs(grad)))
        assert err < 1e-7, (which, err)


def test_dropout_is_unbiased_over_seeds():
    # E_mask[O] = O of the undropped softmax: mean over many seeds within 6 standard errors
    r = _rng(91, 5)
    q, k, v = (r.standard_normal((4, 8)) for _ in range(3))
    o_ref, _ = att.forward_slice(q, k, v, 0.4, False)
    outs = np.stack([dr.forward_slice(q, k, v, 0.4, False, 0.3, s, 0)[0] for s in range(400)])
    mean = outs.mean(axis=0)
    se = outs.std(axis=0, ddof=1) / math.sqrt(outs.shape[0])
    assert np.all(np.abs(mean - o_ref) <= 6 * se + 1e-12)
