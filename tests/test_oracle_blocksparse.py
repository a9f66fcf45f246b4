"""Pins of the block-sparse oracle: reductions to dense attention on sub-problems, the page-3
merge of per-block partials, and scipy over explicitly listed key sets."""
import numpy as np
import pytest
import scipy.special

import fattn_inputs as fi
from oracle import attention as att
from oracle import blocksparse as bs
from oracle import splitkv


def _rng(*words):
    return np.random.default_rng(np.random.SeedSequence(list(words)))


def _qkv(n, d, *seed):
    r = _rng(*seed)
    return tuple(r.standard_normal((n, d)) for _ in range(3))


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_is_dense(causal):
    q, k, v = _qkv(300, 8, 101, int(causal))
    o, lse = bs.forward_slice(q, k, v, 0.3, np.ones((3, 3)), causal)
    o_ref, lse_ref = att.forward_slice(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)


def test_block_diagonal_is_independent_blocks():
    q, k, v = _qkv(300, 8, 102)
    o, lse = bs.forward_slice(q, k, v, 0.3, np.eye(3))
    for b in range(3):
        sl = slice(128 * b, min(300, 128 * b + 128))
        o_ref, lse_ref = att.forward_slice(q[sl], k[sl], v[sl], 0.3)
        np.testing.assert_allclose(o[sl], o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[sl], lse_ref, rtol=0, atol=1e-13)


def test_first_column_only_and_empty_rows():
    q, k, v = _qkv(260, 4, 103)
    m = np.zeros((3, 3))
    m[:2, 0] = 1  # rows of block 2 see nothing
    o, lse = bs.forward_slice(q, k, v, 0.5, m)
    o_ref, lse_ref = att.forward_slice(q[:256], k[:128], v[:128], 0.5)
    np.testing.assert_allclose(o[:256], o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:256], lse_ref, rtol=0, atol=1e-13)
    assert np.all(o[256:] == 0) and np.all(lse[256:] == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
def test_equals_merge_of_per_block_partials(causal):
    # page 3's merge of the allowed key blocks' partial results reproduces every row
    n = 384
    q, k, v = _qkv(n, 8, 104, int(causal))
    m = fi.block_mask(1, 1, 3, 0.5, 104)[0, 0]
    o, lse = bs.forward_slice(q, k, v, 0.4, m, causal)
    for i in range(0, n, 37):
        parts_o, parts_l = [], []
        for jb in range(3):
            keys = np.arange(128 * jb, 128 * jb + 128)
            if causal:
                keys = keys[keys <= i]
            if not m[i // 128, jb] or keys.size == 0:
                parts_o.append(np.zeros(8))
                parts_l.append(-np.inf)
                continue
            po, pl = att.forward_slice(q[i:i + 1], k[keys], v[keys], 0.4)
            parts_o.append(po[0])
            parts_l.append(pl[0])
        mo, ml = splitkv.combine(np.array(parts_o)[:, None, :], np.array(parts_l)[:, None])
        np.testing.assert_allclose(o[i], mo[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], ml[0], rtol=0, atol=1e-13)


def test_scipy_over_explicit_allowed_sets():
    n = 200
    q, k, v = _qkv(n, 6, 105)
    m = fi.block_mask(1, 1, 2, 0.5, 105)[0, 0]
    o, lse = bs.forward_slice(q, k, v, 0.6, m, causal=True)
    for i in (0, 5, 127, 128, 150, 199):
        keys = [j for j in range(n) if m[i // 128, j // 128] and j <= i]
        sc = 0.6 * (k[keys] @ q[i])
        assert lse[i] == pytest.approx(scipy.special.logsumexp(sc), abs=1e-12)
        np.testing.assert_allclose(o[i], scipy.special.softmax(sc) @ v[keys], rtol=0, atol=1e-12)


def test_block_mask_generator():
    m = fi.block_mask(2, 3, 5, 0.25, 9)
    assert m.shape == (2, 3, 5, 5) and m.dtype == np.uint8
    assert np.all(m[..., np.arange(5), np.arange(5)] == 1)
    assert np.array_equal(m, fi.block_mask(2, 3, 5, 0.25, 9))


# ---------------------------------------------------------------------------------------------
# Backward


def _loss(q, k, v, do, scale, m, causal, mb):
    o, _ = bs.forward_slice(q, k, v, scale, m, causal, mb)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    # mb = 2 on N = 7 gives a 4 x 4 block mask with a ragged last block; the mask zeroes a whole
    # block row (rows 4, 5 see nothing) and some off-diagonal blocks
    n, d, mb, scale = 7, 3, 2, 0.7
    r = _rng(201, int(causal))
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    m = np.array([[1, 0, 1, 0], [1, 1, 0, 1], [0, 0, 0, 0], [1, 0, 1, 1]], dtype=np.uint8)
    dq, dk, dv = bs.backward_slice(q, k, v, do, scale, m, causal, mb)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, scale, m, causal, mb)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, scale, m, causal, mb)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7 * max(1.0, np.max(np.abs(num))), err_msg=name)
    # the empty block row: no gradient flows through rows 4 and 5
    assert np.all(dq[4:6] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_all_ones_is_dense(causal):
    r = _rng(202, int(causal))
    q, k, v, do = (r.standard_normal((300, 8)) for _ in range(4))
    got = bs.backward_slice(q, k, v, do, 0.3, np.ones((3, 3)), causal)
    ref = att.backward_slice(q, k, v, do, 0.3, causal)
    for g, x in zip(got, ref):
        np.testing.assert_allclose(g, x, rtol=0, atol=1e-12)


def test_backward_block_diagonal_is_independent_blocks():
    r = _rng(203)
    q, k, v, do = (r.standard_normal((300, 8)) for _ in range(4))
    got = bs.backward_slice(q, k, v, do, 0.3, np.eye(3))
    for b in range(3):
        sl = slice(128 * b, min(300, 128 * b + 128))
        ref = att.backward_slice(q[sl], k[sl], v[sl], do[sl], 0.3)
        for g, x in zip(got, ref):
            np.testing.assert_allclose(g[sl], x, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    # sum_j dS_ij = 0 for every row with an allowed key, so sum_j dK_j = 0; dV sums dO over the
    # rows that see at least one key
    r = _rng(204, int(causal))
    q, k, v, do = (r.standard_normal((400, 8)) for _ in range(4))
    m = fi.block_mask(1, 1, 4, 0.4, 204, diagonal=False)[0, 0]
    m[2, :] = 0
    dq, dk, dv = bs.backward_slice(q, k, v, do, 0.25, m, causal)
    _, lse = bs.forward_slice(q, k, v, 0.25, m, causal)
    seen = np.isfinite(lse)
    assert not np.all(seen)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do[seen].sum(axis=0), rtol=0, atol=1e-11)
    assert np.all(dq[~seen] == 0)
