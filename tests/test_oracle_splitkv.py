"""Pins of the split-KV oracle (per-range partials and their merge) and of the causal offset.

Nothing here retypes the oracle's arithmetic: the pins are page 3's worked example split in two,
closed forms of the merge, the unsplit definition it must reproduce, scipy's logsumexp/softmax
over explicitly listed key sets, and invariances (split order, empty splits, decode rows equal
to the last rows of the square causal problem).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import fattn_inputs as fi
from oracle import attention as att
from oracle import splitkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expr(s):
    if isinstance(s, (int, float)):
        return float(s)
    if isinstance(s, list):  # a fraction [numerator, denominator]
        return s[0] / s[1]
    return float(eval(s, {"__builtins__": {}}, {"exp": math.exp, "ln": math.log}))


def _rng(*words):
    return np.random.default_rng(np.random.SeedSequence(list(words)))


def _decode(B, H, nq, nk, d, seed):
    inp = fi.make_decode_inputs(B, H, nq, nk, d, "f32", seed)
    return (inp.q.astype(np.float64), inp.k.astype(np.float64), inp.v.astype(np.float64))


# --------------------------------------------------------------------------------------------
# Page 3's worked example as two one-key splits


def test_p3_example_as_two_partials():
    with open(os.path.join(GOLDEN, "p3_worked_example.json")) as f:
        g = json.load(f)
    s = [_expr(x) for x in g["scores"]]
    vals = [float(x) for x in g["values"]]
    q = np.array([[1.0]])
    k = np.array([[s[0]], [s[1]]])
    v = np.array([[vals[0]], [vals[1]]])
    o_p, lse_p = splitkv.partials_slice(q, k, v, 1.0, [(0, 1), (1, 2)])
    # a one-key split returns that key's value and its logit
    assert o_p[:, 0, 0] == pytest.approx(vals, abs=0)
    assert lse_p[:, 0] == pytest.approx(s, abs=1e-15)
    o, lse = splitkv.combine(o_p, lse_p)
    assert o[0, 0] == pytest.approx(_expr(g["output"]), abs=1e-13)  # 50/3
    assert lse[0] == pytest.approx(math.log(3.0), abs=1e-15)         # ln(e^0 + e^ln2)
    # and, the other way round, the naive average of the normalised partials is not the answer
    assert abs(o_p[:, 0, 0].sum() - g["wrong_sum_of_blockwise_normalised_outputs"]) < 1e-12


# --------------------------------------------------------------------------------------------
# Closed forms of the merge


def test_combine_single_partial_is_identity():
    r = _rng(61, 1)
    o = r.standard_normal((1, 5, 7))
    lse = r.standard_normal((1, 5)) * 30
    o2, lse2 = splitkv.combine(o, lse)
    assert np.array_equal(o2, o[0]) and np.array_equal(lse2, lse[0])


def test_combine_equal_lse_is_mean_plus_log_count():
    r = _rng(61, 2)
    S = 6
    o = r.standard_normal((S, 4, 3))
    lse = np.broadcast_to(r.standard_normal(4) * 5, (S, 4))
    o2, lse2 = splitkv.combine(o, lse)
    np.testing.assert_allclose(o2, o.mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[0] + math.log(S), rtol=0, atol=1e-14)


def test_combine_two_partials_closed_form():
    # weights e^{L1} : e^{L2}; checked with scipy's softmax and logsumexp
    r = _rng(61, 3)
    o = r.standard_normal((2, 8, 5))
    lse = r.standard_normal((2, 8)) * 4
    o2, lse2 = splitkv.combine(o, lse)
    w = scipy.special.softmax(lse, axis=0)
    np.testing.assert_allclose(o2, (w[..., None] * o).sum(axis=0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, scipy.special.logsumexp(lse, axis=0), rtol=0, atol=1e-13)


def test_combine_empty_partials_are_neutral_and_all_empty_is_empty():
    r = _rng(61, 4)
    o = r.standard_normal((3, 4, 2))
    lse = r.standard_normal((3, 4))
    o_e = np.concatenate([np.zeros((2, 4, 2)), o[:1], np.zeros((1, 4, 2)), o[1:]])
    lse_e = np.concatenate([np.full((2, 4), -np.inf), lse[:1], np.full((1, 4), -np.inf), lse[1:]])
    a, la = splitkv.combine(o, lse)
    b, lb = splitkv.combine(o_e, lse_e)
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lb, la, rtol=0, atol=1e-15)
    z, lz = splitkv.combine(np.zeros((3, 4, 2)), np.full((3, 4), -np.inf))
    assert np.all(z == 0) and np.all(lz == -np.inf)


def test_combine_is_order_independent_and_stable_at_large_lse():
    r = _rng(61, 5)
    S = 7
    o = r.standard_normal((S, 6, 4))
    lse = 500.0 + r.standard_normal((S, 6)) * 3  # every partial's exp-sum is ~e^500
    a, la = splitkv.combine(o, lse)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(la))
    perm = r.permutation(S)
    b, lb = splitkv.combine(o[perm], lse[perm])
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lb, la, rtol=0, atol=1e-12)
    # shifting every LSE by the same amount shifts the result and leaves O alone
    c, lc = splitkv.combine(o, lse - 500.0)
    np.testing.assert_allclose(c, a, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lc, la - 500.0, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------------
# The partition


@pytest.mark.parametrize("nk,S", [(1, 1), (63, 4), (64, 1), (65, 2), (1000, 3), (16384, 16), (100, 16),
                                  (16384, 7), (4097, 64)])
def test_split_ranges_partition(nk, S):
    rs = splitkv.split_ranges(nk, S)
    assert len(rs) == S
    covered = []
    for k0, k1 in rs:
        assert 0 <= k0 <= k1 <= nk
        assert k0 % splitkv.ALIGN == 0 or k0 == nk
        covered.extend(range(k0, k1))
    assert covered == list(range(nk))
    sizes = [k1 - k0 for k0, k1 in rs]
    # equal lengths, a multiple of the alignment, except the last non-empty one
    nonempty = [x for x in sizes if x]
    assert all(x == nonempty[0] for x in nonempty[:-1])
    assert nonempty[0] % splitkv.ALIGN == 0 or len(nonempty) == 1


# --------------------------------------------------------------------------------------------
# The causal offset (decode rows are the last rows of the square problem)


def test_causal_offset_brute_force_scipy():
    q, k, v = _decode(1, 1, 5, 11, 4, 62)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    off = 11 - 5
    o, lse = att.forward_slice(q, k, v, 0.7, causal=True, causal_offset=off)
    for i in range(5):
        vis = np.arange(0, i + off + 1)
        s = 0.7 * (k[vis] @ q[i])
        assert lse[i] == pytest.approx(scipy.special.logsumexp(s), abs=1e-13)
        np.testing.assert_allclose(o[i], scipy.special.softmax(s) @ v[vis], rtol=0, atol=1e-13)


def test_decode_rows_equal_last_rows_of_square_causal():
    r = _rng(61, 7)
    N, nq, d = 40, 6, 8
    q = r.standard_normal((N, d))
    k = r.standard_normal((N, d))
    v = r.standard_normal((N, d))
    o_full, lse_full = att.forward_slice(q, k, v, 0.5, causal=True)
    o_dec, lse_dec = att.forward_slice(q[N - nq:], k, v, 0.5, causal=True, causal_offset=N - nq)
    np.testing.assert_array_equal(o_dec, o_full[N - nq:])
    np.testing.assert_array_equal(lse_dec, lse_full[N - nq:])
    # one query at offset Nk - 1 sees every key: the same as no mask
    o1, l1 = att.forward_slice(q[-1:], k, v, 0.5, causal=True, causal_offset=N - 1)
    o2, l2 = att.forward_slice(q[-1:], k, v, 0.5, causal=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# --------------------------------------------------------------------------------------------
# Split partials merged == the unsplit definition


@pytest.mark.parametrize("nq,nk,S,causal", [
    (1, 300, 1, False), (1, 300, 2, False), (1, 300, 5, True), (3, 129, 3, True),
    (16, 1000, 7, True), (16, 1000, 16, False), (5, 70, 16, True), (33, 33, 2, True),
    (2, 64, 64, False)])
def test_split_merge_equals_definition(nq, nk, S, causal):
    q, k, v = _decode(1, 2, nq, nk, 16, 63)
    scale = 0.25
    o, lse, op, lp = splitkv.forward(q, k, v, scale, S, causal)
    o_ref, lse_ref = att.forward(q, k, v, scale, causal, causal_offset=nk - nq)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
    # each partial is the definition restricted to its key range (or empty)
    for s, (k0, k1) in enumerate(splitkv.split_ranges(nk, S)):
        for b, h in [(0, 0), (0, 1)]:
            for i in range(nq):
                hi = min(k1, i + (nk - nq) + 1) if causal else k1
                if hi <= k0:
                    assert lp[s, b, h, i] == -np.inf and np.all(op[s, b, h, i] == 0)
                    continue
                sc = scale * (k[b, h, k0:hi] @ q[b, h, i])
                assert lp[s, b, h, i] == pytest.approx(scipy.special.logsumexp(sc), abs=1e-12)
                np.testing.assert_allclose(op[s, b, h, i], scipy.special.softmax(sc) @ v[b, h, k0:hi],
                                           rtol=0, atol=1e-12)


def test_split_merge_stays_finite_under_plus_500_shift():
    # every logit +500 (page 1's stability example): partials' LSE move by exactly 500, O does not
    r = _rng(61, 8)
    nk, d = 200, 8
    q = r.standard_normal((1, 1, 2, d))
    k = r.standard_normal((1, 1, nk, d))
    v = r.standard_normal((1, 1, nk, d))
    q2 = q.copy()
    q2[..., 0] = 1.0
    k2 = k.copy()
    o_a, l_a, _, _ = splitkv.forward(q2, k2, v, 1.0, 4)
    k2[..., 0] += 500.0
    o_b, l_b, _, lp = splitkv.forward(q2, k2, v, 1.0, 4)
    assert np.all(np.isfinite(o_b)) and np.all(np.isfinite(l_b))
    np.testing.assert_allclose(o_b, o_a, rtol=0, atol=1e-11)
    np.testing.assert_allclose(l_b, l_a + 500.0, rtol=0, atol=1e-10)
