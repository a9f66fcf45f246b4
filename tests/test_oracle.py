"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these tests retypes the oracle's formulas: they use the pages' printed worked examples
(tests/golden), closed forms, invariances, independent library routines (scipy's softmax and
logsumexp, torch's CPU float64 attention and autograd) and central finite differences.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import fattn_inputs as fi
from oracle import attention as att
from oracle import tiled
from oracle import traffic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _expr(s):
    """Evaluate a fixture expression written with exp, ln, numbers and + - * / ( )."""
    if isinstance(s, (int, float)):
        return float(s)
    if isinstance(s, list):
        return s[0] / s[1]
    return float(eval(s, {"__builtins__": {}}, {"exp": math.exp, "ln": math.log}))


def _rng(*words):
    return np.random.default_rng(np.random.SeedSequence(list(words)))


# --------------------------------------------------------------------------------------------
# Worked example of page 3: scores [0, ln 2], values [10, 20]


def _p3_case():
    g = _golden("p3_worked_example.json")
    s = [_expr(x) for x in g["scores"]]
    # d = 1, scale = 1, a single query equal to 1 so that the logits are the keys themselves.
    q = np.array([[1.0]])
    k = np.array([[s[0]], [s[1]]])
    v = np.array([[float(g["values"][0])], [float(g["values"][1])]])
    return g, q, k, v


def test_p3_definition_gives_fifty_thirds():
    g, q, k, v = _p3_case()
    o, lse = att.forward_slice(q, k, v, 1.0)
    assert o[0, 0] == pytest.approx(_expr(g["output"]), abs=1e-13)
    # weights follow from the saved statistic: P = exp(S - LSE)
    w = np.exp(k[:, 0] - lse[0])
    assert w == pytest.approx([_expr(x) for x in g["full_softmax_weights"]], abs=1e-15)


def test_p3_blockwise_merge_trace():
    g, q, k, v = _p3_case()
    trace = []
    o, lse, visited = tiled.forward_slice(q, k, v, 1.0, Br=1, Bc=1, trace=trace)
    assert visited == 2
    _, _, m1, l1, u1 = trace[0]
    assert m1[0] == _expr(g["block_1"]["m"]) and l1[0] == g["block_1"]["l"] and u1[0, 0] == g["block_1"]["u"]
    _, _, m2, l2, u2 = trace[1]
    assert m2[0] == pytest.approx(_expr(g["merged"]["m_new"]), abs=1e-15)
    assert l2[0] == pytest.approx(_expr(g["merged"]["l_new"]), abs=1e-15)
    assert u2[0, 0] == pytest.approx(g["merged"]["u_new"], abs=1e-13)
    assert o[0, 0] == pytest.approx(_expr(g["merged_output"]), abs=1e-13)
    assert o[0, 0] == pytest.approx(_expr(g["output"]), abs=1e-13)
    # the standalone two-state merge on the block statistics the page prints
    b1, b2 = g["block_1"], g["block_2"]
    m, l, u = tiled.merge(np.array([_expr(b1["m"])]), np.array([b1["l"]]), np.array([[b1["u"]]]),
                          np.array([_expr(b2["m_b"])]), np.array([b2["l_b"]]), np.array([[b2["u_b"]]]))
    assert l[0] == pytest.approx(1.5, abs=1e-15) and u[0, 0] == pytest.approx(25.0, abs=1e-13)
    # the old block is rescaled by exp(m - m_new) = 1/2
    assert math.exp(_expr(b1["m"]) - m[0]) == pytest.approx(_expr(g["merged"]["old_block_factor"]), abs=1e-15)


def test_p3_wrong_blockwise_sum_gives_thirty():
    g, q, k, v = _p3_case()
    out = tiled.wrong_blockwise_sum(q, k, v, 1.0, Bc=1)
    assert out[0, 0] == pytest.approx(g["wrong_sum_of_blockwise_normalised_outputs"], abs=1e-13)
    assert abs(out[0, 0] - _expr(g["output"])) > 10


def test_p3_causal_rows():
    g, _, k, v = _p3_case()
    q = np.array([[1.0], [1.0]])
    o, lse = att.forward_slice(q, k, v, 1.0, causal=True)
    assert o[0, 0] == pytest.approx(g["values"][0], abs=1e-13)  # row 0 sees key 0 only
    assert lse[0] == pytest.approx(0.0, abs=1e-15)
    assert o[1, 0] == pytest.approx(_expr(g["output"]), abs=1e-13)
    assert lse[1] == pytest.approx(math.log(3.0), abs=1e-15)


# --------------------------------------------------------------------------------------------
# Incremental example of page 1: scores [1, 2, 3]


def test_p1_incremental_exp_sum():
    g = _golden("p1_online_softmax.json")
    scores = [float(x) for x in g["scores"]]
    q = np.array([[1.0]])
    k = np.array(scores)[:, None]
    v = np.eye(3)
    # first two scores as one block, then the third
    trace = []
    tiled.forward_slice(q, k[:2], v[:2], 1.0, Br=1, Bc=2, trace=trace)
    assert trace[-1][2][0] == g["after_first_two"]["m"]
    assert trace[-1][3][0] == pytest.approx(_expr(g["after_first_two"]["l"]), abs=1e-15)
    trace = []
    o, lse, _ = tiled.forward_slice(q, k, v, 1.0, Br=1, Bc=2, trace=trace)
    assert trace[-1][2][0] == g["after_third"]["m"]
    assert trace[-1][3][0] == pytest.approx(_expr(g["after_third"]["l"]), abs=1e-15)
    # element by element (block size 1) reaches the same state
    trace = []
    tiled.forward_slice(q, k, v, 1.0, Br=1, Bc=1, trace=trace)
    assert trace[1][3][0] == pytest.approx(_expr(g["after_first_two"]["l"]), abs=1e-15)
    assert trace[2][3][0] == pytest.approx(_expr(g["after_third"]["l"]), abs=1e-15)
    # and the normalised result is the textbook softmax of the row
    assert o[0] == pytest.approx(scipy.special.softmax(scores), abs=1e-15)
    assert lse[0] == pytest.approx(scipy.special.logsumexp(scores), abs=1e-15)
    o2, lse2 = att.forward_slice(q, k, v, 1.0)
    assert o2[0] == pytest.approx(scipy.special.softmax(scores), abs=1e-15)
    assert lse2[0] == pytest.approx(scipy.special.logsumexp(scores), abs=1e-15)


def test_p1_causal_rows_of_the_incremental_example():
    q = np.ones((3, 1))
    k = np.array([[1.0], [2.0], [3.0]])
    v = np.eye(3)
    o, lse = att.forward_slice(q, k, v, 1.0, causal=True)
    for i in range(3):
        ref = scipy.special.softmax(k[: i + 1, 0])
        assert o[i, : i + 1] == pytest.approx(ref, abs=1e-15)
        assert np.all(o[i, i + 1:] == 0.0)
        assert lse[i] == pytest.approx(scipy.special.logsumexp(k[: i + 1, 0]), abs=1e-15)


# --------------------------------------------------------------------------------------------
# Library cross-checks on random inputs


@pytest.mark.parametrize("N,d,causal", [(1, 4, False), (7, 3, True), (33, 16, False), (65, 8, True)])
def test_softmax_matches_scipy(N, d, causal):
    r = _rng(11, N, d)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    scale = 0.37
    o, lse = att.forward_slice(q, k, v, scale, causal)
    for i in range(N):
        keys = slice(0, i + 1) if causal else slice(0, N)
        logits = scale * (k[keys] @ q[i])
        w = scipy.special.softmax(logits)
        np.testing.assert_allclose(o[i], w @ v[keys], rtol=0, atol=1e-13)
        assert lse[i] == pytest.approx(scipy.special.logsumexp(logits), abs=1e-13)


def _torch_attention(q, k, v, scale, causal):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    return tq, tk, tv, o


@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_gradients_match_torch_cpu_float64(causal):
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 37, 16
    r = _rng(12, int(causal))
    q, k, v, do = (r.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 1 / math.sqrt(d)
    o, lse = att.forward(q, k, v, scale, causal)
    tq, tk, tv, to = _torch_attention(q, k, v, scale, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    to.backward(torch.tensor(do))
    dq, dk, dv = att.backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


# --------------------------------------------------------------------------------------------
# Closed forms


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("how", ["k_zero", "scale_zero"])
def test_uniform_attention_closed_form(causal, how):
    N, d = 50, 8
    r = _rng(13)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    scale = 0.5
    if how == "k_zero":
        k = np.zeros_like(k)
    else:
        scale = 0.0
    o, lse = att.forward_slice(q, k, v, scale, causal)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-14)
        assert lse[i] == pytest.approx(math.log(n), abs=1e-14)


def test_single_key_closed_form():
    r = _rng(14)
    q, k, v = (r.standard_normal((1, 5)) for _ in range(3))
    for causal in (False, True):
        o, lse = att.forward_slice(q, k, v, 0.3, causal)
        np.testing.assert_array_equal(o, v)
        assert lse[0] == pytest.approx(0.3 * float(np.dot(q[0], k[0])), abs=1e-15)
    dq, dk, dv = att.backward_slice(q, k, v, np.ones((1, 5)), 0.3)
    # one key: P = 1 regardless of the logit, so O = V and the logit gradients vanish
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv, np.ones((1, 5)), atol=1e-15)


# --------------------------------------------------------------------------------------------
# Invariances


def test_logit_shift_of_exactly_500():
    scale = 1 / 8.0
    base = fi.make_inputs((1, 2, 64, 64), "f16", 2, fi.VARIANT_SHIFT_EXACT, scale=scale)
    partner = fi.unshifted_partner(base, scale)
    o1, l1 = att.forward(base.q, base.k, base.v, scale)
    o0, l0 = att.forward(partner.q, partner.k, partner.v, scale)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-11)
    np.testing.assert_allclose(l1 - l0, 500.0, rtol=0, atol=1e-11)
    # the logits really are around +500
    s = scale * (base.q[0, 0].astype(np.float64) @ base.k[0, 0].astype(np.float64).T)
    assert s.min() > 450
    # the unshifted float32 softmax overflows to NaN there (page 2, stability check)
    bad = att.forward_unshifted_f32(base.q[0, 0], base.k[0, 0], base.v[0, 0], scale)
    assert np.isnan(bad).any()
    # while on the unshifted partner it is fine
    ok = att.forward_unshifted_f32(partner.q[0, 0], partner.k[0, 0], partner.v[0, 0], scale)
    assert np.all(np.isfinite(ok))


def test_literal_shift_variant_stays_finite():
    scale = 1 / 8.0
    inp = fi.make_inputs((1, 2, 64, 64), "f16", 2, fi.VARIANT_SHIFT_LITERAL, scale=scale)
    for causal in (False, True):
        o, lse = att.forward(inp.q, inp.k, inp.v, scale, causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        # each output row is a convex combination of value rows
        assert np.all(o <= inp.v.max(axis=2, keepdims=True) + 1e-12)
        assert np.all(o >= inp.v.min(axis=2, keepdims=True) - 1e-12)


def test_unshifted_softmax_overflow_needs_float32():
    x = np.array([[500.0, 501.0, 499.0]])
    assert np.isnan(att.softmax_unshifted_f32(x)).all()
    # the stable definition is finite and equals the textbook softmax
    q = np.array([[1.0]])
    o, lse = att.forward_slice(q, x.T, np.eye(3), 1.0)
    np.testing.assert_allclose(o[0], scipy.special.softmax(x[0]), atol=1e-15)


@pytest.mark.parametrize("i", [0, 5, 31, 62])
def test_causal_prefix_is_bitwise_independent_of_later_keys(i):
    N, d = 63, 8
    r = _rng(15)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    o, lse = att.forward_slice(q, k, v, 0.4, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] = r.standard_normal(k2[i + 1:].shape) * 7
    v2[i + 1:] = r.standard_normal(v2[i + 1:].shape) * 7
    o2, lse2 = att.forward_slice(q, k2, v2, 0.4, causal=True)
    np.testing.assert_array_equal(o2[: i + 1], o[: i + 1])
    np.testing.assert_array_equal(lse2[: i + 1], lse[: i + 1])
    if i + 1 < N:
        assert not np.array_equal(o2[i + 1:], o[i + 1:])


def test_key_permutation_invariance():
    N, d = 40, 6
    r = _rng(16)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    perm = r.permutation(N)
    o, lse = att.forward_slice(q, k, v, 0.7)
    o2, lse2 = att.forward_slice(q, k[perm], v[perm], 0.7)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)


# --------------------------------------------------------------------------------------------
# The tiled model against the definition


@pytest.mark.parametrize("N", [1, 2, 37, 100, 129])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_model_matches_definition_for_every_tile_size(N, causal):
    d = 8
    r = _rng(17, N)
    q, k, v = (r.standard_normal((N, d)) * 2 for _ in range(3))
    o_ref, lse_ref = att.forward_slice(q, k, v, 0.35, causal)
    for Br in (1, 2, 3, 5, 16, 64, 128):
        for Bc in (1, 2, 3, 5, 16, 64, 128):
            o, lse, visited = tiled.forward_slice(q, k, v, 0.35, Br, Bc, causal)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
            if causal:
                assert visited == tiled.causal_blocks_visited(N, Br, Bc)
            else:
                assert visited == math.ceil(N / Br) * math.ceil(N / Bc)


def test_causal_tile_skipping_halves_the_work():
    N, B = 4096, 128
    full = (N // B) ** 2
    visited = tiled.causal_blocks_visited(N, B, B)
    assert visited == (N // B) * (N // B + 1) // 2
    assert visited / full == pytest.approx(0.5, abs=0.02)


def test_tiled_model_block_with_only_masked_keys():
    # Br > Bc: the first query rows of a block see key blocks that are wholly masked for them.
    N, d = 12, 4
    r = _rng(18)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    o_ref, lse_ref = att.forward_slice(q, k, v, 1.0, True)
    o, lse, _ = tiled.forward_slice(q, k, v, 1.0, Br=8, Bc=2, causal=True)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-13)


# --------------------------------------------------------------------------------------------
# Gradients


def _loss(q, k, v, do, scale, causal, causal_offset=0):
    o, _ = att.forward_slice(q, k, v, scale, causal, causal_offset=causal_offset)
    return float(np.sum(do * o))


@pytest.mark.parametrize("N,d", [(1, 1), (3, 3), (5, 4), (7, 3), (7, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_finite_differences(N, d, causal):
    r = _rng(19, N, d, int(causal))
    scale = 0.8
    for h in range(2):  # two heads
        q, k, v, do = (r.standard_normal((N, d)) for _ in range(4))
        dq, dk, dv = att.backward_slice(q, k, v, do, scale, causal)
        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name], args_m[name] = xp, xm
                num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                            - _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * eps)
            den = max(1.0, float(np.max(np.abs(num))))
            assert float(np.max(np.abs(num - g))) / den < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_identities(causal):
    B, H, N, d = 1, 2, 45, 8
    r = _rng(20, int(causal))
    q, k, v, do = (r.standard_normal((B, H, N, d)) for _ in range(4))
    dq, dk, dv = att.backward(q, k, v, do, 0.5, causal)
    # each row of dS sums to 0, so the key gradients sum to 0 per head
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # each row of P sums to 1, so the value gradients sum to the output gradients
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


# --------------------------------------------------------------------------------------------
# Traffic model


def test_traffic_naive_quadratic_flash_linear():
    Ns = [128, 256, 512, 1024, 2048, 4096]
    rows = traffic.traffic_table(Ns, d=64)
    for a, b in zip(rows, rows[1:]):
        assert b["naive_nn_elements"] == 4 * a["naive_nn_elements"]
        assert b["flash_nn_touches"] == 0 and b["flash_nn_elements"] == 0
        assert b["flash_bytes"] == 2 * a["flash_bytes"]
    # growth exponent between the two largest lengths: quadratic for naive, linear for tiled
    slope_naive = math.log2(rows[-1]["naive_bytes"] / rows[-2]["naive_bytes"])
    slope_flash = math.log2(rows[-1]["flash_bytes"] / rows[-2]["flash_bytes"])
    assert slope_naive > 1.95 and slope_flash == pytest.approx(1.0, abs=1e-12)
    # page 1: one FP16 4096 x 4096 score table is about 32 MiB
    assert 4096 * 4096 * 2 == 32 * 2**20
    # without cache reuse the tiled design re-reads K and V once per query block
    assert traffic.tiled_bytes_with_rereads(4096, 128, 128) > traffic.memory_work(4096, 128)["flash_bytes"]


def test_print_traffic_table_runs(capsys):
    traffic.print_traffic_table()
    out = capsys.readouterr().out
    assert "4096" in out


# --------------------------------------------------------------------------------------------
# Inputs


def test_bf16_and_f16_rounding_match_torch_bit_for_bit():
    torch = pytest.importorskip("torch")
    r = _rng(21)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * s for s in (1, 1e-3, 300, 7e4)])
    x = np.concatenate([x, np.array([1.00390625, 1.01171875, -2.0039062, 0.0, -0.0,
                                     3.4028235e38, -3.4028235e38, 3.3e38, 1e-45, -1e-40], np.float32)])
    bv, bb = fi.round_bits(x, "bf16")
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bb, tb)
    np.testing.assert_array_equal(bv, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    xh = x[np.abs(x) < 6e4]
    _, hb = fi.round_bits(xh, "f16")
    th = torch.from_numpy(xh).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(hb, th)


def test_inputs_are_seeded_and_independent_per_tensor():
    a = fi.make_inputs((1, 2, 16, 8), "bf16", 3)
    b = fi.make_inputs((1, 2, 16, 8), "bf16", 3, with_do=True)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.v, b.v)
    c = fi.make_inputs((1, 2, 16, 8), "bf16", 4)
    assert not np.array_equal(a.q, c.q)
    assert b.do is not None and b.do.shape == (1, 2, 16, 8)


# --------------------------------------------------------------------------------------------
# K-outer loop order (page 2, FA-1 to FA-2 section): the ablation's model


@pytest.mark.parametrize("N,Br,Bc,causal", [(1, 1, 1, False), (37, 5, 3, True), (100, 16, 64, False),
                                            (129, 64, 16, True), (200, 32, 32, True), (64, 128, 64, False)])
def test_kouter_equals_qouter_bitwise_and_the_definition(N, Br, Bc, causal):
    r = _rng(71, N, Br, Bc, int(causal))
    q, k, v = (r.standard_normal((N, 8)) for _ in range(3))
    o1, l1, vis1 = tiled.forward_slice(q, k, v, 0.4, Br, Bc, causal)
    trace = []
    o2, l2, vis2 = tiled.forward_slice_kouter(q, k, v, 0.4, Br, Bc, causal, trace=trace)
    # every row merges the same blocks in the same order: identical float64 results
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(l2, l1)
    assert vis1 == vis2
    if causal:
        assert vis2 == tiled.causal_blocks_visited(N, Br, Bc)
    else:
        assert vis2 == math.ceil(N / Br) * math.ceil(N / Bc)
    # the visiting order is key-block major
    order = [(jb, ib) for ib, jb, *_ in trace]
    assert order == sorted(order)
    o_ref, l_ref = att.forward_slice(q, k, v, 0.4, causal)
    np.testing.assert_allclose(o2, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l_ref, rtol=0, atol=1e-12)


def test_kouter_worked_example_fifty_thirds():
    g, q, k, v = _p3_case()
    o, lse, visits = tiled.forward_slice_kouter(q, k, v, 1.0, Br=1, Bc=1)
    assert visits == 2
    assert o[0, 0] == pytest.approx(_expr(g["output"]), abs=1e-13)
    assert lse[0] == pytest.approx(math.log(3.0), abs=1e-15)


def test_loop_order_bytes_closed_forms():
    N, d, s = 4096, 128, 2
    for Br, Bc in ((128, 64), (256, 128), (64, 64)):
        # Q-outer, no cache: Q + O once, LSE once, K and V once per query block
        q_outer = traffic.loop_order_bytes(N, d, Br, Bc, "q_outer")
        assert q_outer == 2 * N * d * s + 4 * N + 2 * N * d * s * (N // Br)
        assert q_outer == traffic.tiled_bytes_with_rereads(N, d, Br, s)
        # K-outer: K, V once; Q once per key block; state (d + 2) floats per row read and written
        # on every visit but the first / last; O and LSE once
        nb = N // Bc
        k_outer = traffic.loop_order_bytes(N, d, Br, Bc, "k_outer")
        assert k_outer == 2 * N * d * s + nb * N * d * s + 2 * (nb - 1) * N * (d + 2) * 4 + N * d * s + 4 * N
    # the K-outer order moves more bytes whenever there is more than one key block
    assert traffic.loop_order_bytes(N, d, 128, 64, "k_outer") > 4 * traffic.loop_order_bytes(N, d, 128, 64, "q_outer")
    # causal: the visit counts fall to the lower triangle in both orders
    qc = traffic.loop_order_bytes(N, d, 128, 128, "q_outer", causal=True)
    nb = N // 128
    assert qc == 2 * N * d * s + 4 * N + 2 * 128 * d * s * (nb * (nb + 1) // 2)


# --------------------------------------------------------------------------------------------
# Whole-tensor wrappers and the causal traffic branch


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_forward_over_batch_and_heads_matches_the_definition(causal):
    # [B, H, N, d] with every (b, h) slice drawn differently (and scaled differently), so a
    # swapped or repeated batch/head index in the wrapper shows up as a large error
    B, H, N, d = 2, 3, 37, 8
    r = _rng(81, int(causal))
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            q[b, h] *= 1 + b + 2 * h
            v[b, h] += 10 * (b * H + h)
    o_ref, lse_ref = att.forward(q, k, v, 0.3, causal)
    o, lse = tiled.forward(q, k, v, 0.3, 16, 5, causal)
    assert o.shape == (B, H, N, d) and lse.shape == (B, H, N)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-11)
    # each output slice depends on its own input slice only: permuting the heads permutes them
    perm = [2, 0, 1]
    o_p, lse_p = tiled.forward(q[:, perm], k[:, perm], v[:, perm], 0.3, 16, 5, causal)
    np.testing.assert_array_equal(o_p, o[:, perm])
    np.testing.assert_array_equal(lse_p, lse[:, perm])


def test_tiled_bytes_with_rereads_causal_closed_form():
    s = 2
    # N a multiple of Br: query block i re-reads the K/V prefix of (i + 1) Br keys, so the K/V
    # reads sum to Br d s nb (nb + 1) (an arithmetic series), plus Q and O once and 4 B of LSE
    for N, d, Br in ((4096, 128, 128), (4096, 128, 256), (1024, 64, 64)):
        nb = N // Br
        got = traffic.tiled_bytes_with_rereads(N, d, Br, s, causal=True)
        assert got == 2 * N * d * s + 4 * N + Br * d * s * nb * (nb + 1)
        # about half the non-causal re-reads for many blocks
        full = traffic.tiled_bytes_with_rereads(N, d, Br, s)
        kv_c, kv_f = got - 2 * N * d * s - 4 * N, full - 2 * N * d * s - 4 * N
        assert kv_c / kv_f == pytest.approx((nb + 1) / (2 * nb), rel=1e-12)
    # ragged N: the last block's prefix is capped at N keys
    N, d, Br = 1000, 64, 128
    nb = math.ceil(N / Br)
    kv = sum(2 * min(N, (i + 1) * Br) * d * s for i in range(nb))
    assert kv == 2 * d * s * (128 * (nb - 1) * nb // 2 + N)
    assert traffic.tiled_bytes_with_rereads(N, d, Br, s, causal=True) == 2 * N * d * s + 4 * N + kv
    # when Bc divides Br, the causal Q-outer visits of the loop-order model read exactly the same
    # key prefix for every query block, so both models agree
    for N, Br, Bc in ((4096, 128, 64), (4096, 256, 128), (1000, 128, 64), (1000, 128, 32), (77, 16, 16)):
        assert traffic.tiled_bytes_with_rereads(N, 64, Br, s, causal=True) == \
            traffic.loop_order_bytes(N, 64, Br, Bc, "q_outer", causal=True, elem_bytes=s)
    # one query block: no re-reads at all, causal or not
    assert traffic.tiled_bytes_with_rereads(100, 64, 128, s, causal=True) == \
        traffic.tiled_bytes_with_rereads(100, 64, 128, s) == 4 * 100 * 64 * s + 4 * 100


def test_max_rel_floor_binds_only_below_it():
    from oracle import metrics as M
    r = np.zeros((2, 3, 4))
    r[0] = 2.0            # slice 0: exact values of magnitude 2
    x = r.copy()
    x[0, 0, 0] += 0.01    # slice 0 error 0.01 -> 0.005 relative, whatever the floor below 2
    x[1, 1, 1] = 1e-6     # slice 1: exact zero, rounding noise 1e-6
    assert M.max_rel(x[:1], r[:1]) == pytest.approx(0.005, rel=1e-12)
    assert M.max_rel(x[:1], r[:1], floor=1.0) == pytest.approx(0.005, rel=1e-12)
    # the zero slice alone: infinite without a floor, noise / floor with one
    assert M.max_rel(x[1:], r[1:]) == np.inf
    assert M.max_rel(x[1:], r[1:], floor=1e-3) == pytest.approx(1e-3, rel=1e-9)
    # both slices: the worse of the two
    assert M.max_rel(x, r, floor=1e-3) == pytest.approx(0.005, rel=1e-12)
    # identical zero slices are exact
    assert M.max_rel(r[1:], r[1:]) == 0.0
    # a floor above a slice's own scale replaces its denominator
    assert M.max_rel(x[:1], r[:1], floor=4.0) == pytest.approx(0.0025, rel=1e-12)


@pytest.mark.parametrize("Nq,Nk,offset", [(1, 5, 4), (3, 7, 4), (4, 4, 2), (5, 9, 6), (2, 6, 0)])
def test_gradients_with_a_causal_offset_match_finite_differences(Nq, Nk, offset):
    # queries are the last positions of a longer key sequence (query i sees keys j <= i + offset)
    r = _rng(24, Nq, Nk, offset)
    d, scale = 3, 0.7
    q, do = r.standard_normal((Nq, d)), r.standard_normal((Nq, d))
    k, v = r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    dq, dk, dv = att.backward_slice(q, k, v, do, scale, True, causal_offset=offset)
    assert dq.shape == (Nq, d) and dk.shape == dv.shape == (Nk, d)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = {"q": q, "k": k, "v": v}
            b = {"q": q, "k": k, "v": v}
            a[name], b[name] = x.copy(), x.copy()
            a[name][idx] += eps
            b[name][idx] -= eps
            num[idx] = (_loss(a["q"], a["k"], a["v"], do, scale, True, offset)
                        - _loss(b["q"], b["k"], b["v"], do, scale, True, offset)) / (2 * eps)
        den = max(1.0, float(np.max(np.abs(num))))
        assert float(np.max(np.abs(num - g))) / den < 1e-7, name
    # keys no query can see get no gradient
    hidden = np.arange(Nk) > Nq - 1 + offset
    assert np.all(dk[hidden] == 0) and np.all(dv[hidden] == 0)


def test_periodic_block_problem_equals_the_explicit_head():
    # the folding used by the 2 GiB backward test, on a head small enough to build explicitly:
    # 3 whole copies of a 64-row block plus a 5-row tail
    from tests.periodic import block_problem
    d, R, t, scale = 8, 3, 5, 0.6
    r = _rng(25)
    q, k, v, do = (r.standard_normal((64, d)) for _ in range(4))
    rep = lambda x: np.concatenate([np.tile(x, (R, 1)), x[:t]])
    dq, dk, dv = att.backward_slice(rep(q), rep(k), rep(v), rep(do), scale, True)
    for c in range(R + 1):
        nr = 64 if c < R else t
        got = block_problem(q, k, v, do, scale, c, nr)
        np.testing.assert_allclose(got[0], dq[64 * c: 64 * c + nr], rtol=0, atol=1e-11)
    # keys of block c collect their own block's part and one folded part per later block
    for c in range(R + 1):
        nr = 64 if c < R else t
        _, _, _, dk_own, dv_own = block_problem(q, k, v, do, scale, c, nr)
        ek, ev = dk_own.copy(), dv_own.copy()
        for b in range(c + 1, R + 1):
            _, dk_f, dv_f, _, _ = block_problem(q, k, v, do, scale, b, 64 if b < R else t)
            ek += dk_f[:nr]
            ev += dv_f[:nr]
        np.testing.assert_allclose(ek, dk[64 * c: 64 * c + nr], rtol=0, atol=1e-11)
        np.testing.assert_allclose(ev, dv[64 * c: 64 * c + nr], rtol=0, atol=1e-11)
