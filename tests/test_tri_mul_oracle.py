"""Pins of the FP64 triangle-multiplication oracle against values fixed by the mathematics:
a hand-computed 2 x 2 case, explicit loops, closed forms (one-hot and rank-one inputs), the
symmetry of the outgoing form with a = b, the relation between the two directions, and the
gradients by central differences and the bilinear adjoint identity.

Definition (kongchang.com article on fast_trimul, section "什么是三角乘法更新"; reading in
``oracle/tri_mul_oracle.py``): outgoing x[i,j,c] = sum_k a[i,k,c] b[j,k,c], incoming
x[i,j,c] = sum_k a[k,i,c] b[k,j,c].
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_computed_two_by_two():
    # one batch, one channel: a = [[1, 2], [3, 4]], b = [[5, 6], [7, 8]] (row = first pair index)
    a = np.array([[1.0, 2.0], [3.0, 4.0]]).reshape(1, 2, 2, 1)
    b = np.array([[5.0, 6.0], [7.0, 8.0]]).reshape(1, 2, 2, 1)
    out = oracle.tri_mul_forward64(a, b, "outgoing")[0, :, :, 0]
    inc = oracle.tri_mul_forward64(a, b, "incoming")[0, :, :, 0]
    # outgoing x[i,j] = a[i,0] b[j,0] + a[i,1] b[j,1]: [[1*5+2*6, 1*7+2*8], [3*5+4*6, 3*7+4*8]]
    assert np.array_equal(out, [[17.0, 23.0], [39.0, 53.0]])
    # incoming x[i,j] = a[0,i] b[0,j] + a[1,i] b[1,j]: [[1*5+3*7, 1*6+3*8], [2*5+4*7, 2*6+4*8]]
    assert np.array_equal(inc, [[26.0, 30.0], [38.0, 44.0]])


@pytest.mark.parametrize("direction", oracle.DIRECTIONS)
def test_matches_explicit_loops(direction):
    a, b = _rand((2, 5, 5, 3), 1), _rand((2, 5, 5, 3), 2)
    np.testing.assert_allclose(oracle.tri_mul_forward64(a, b, direction), oracle.tri_mul_loops64(a, b, direction),
                               rtol=1e-13, atol=1e-13)


def test_one_hot_reduction_index_selects_a_slice():
    N, C, k0 = 6, 4, 3
    a = _rand((1, N, N, C), 3)
    onehot = np.zeros((1, N, N, C))
    onehot[:, :, k0, :] = 1.0  # b[j,k,c] = [k == k0]
    x = oracle.tri_mul_forward64(a, onehot, "outgoing")
    assert np.array_equal(x, np.broadcast_to(a[:, :, k0:k0 + 1, :], x.shape))  # x[i,j,c] = a[i,k0,c]
    onehot_in = np.zeros((1, N, N, C))
    onehot_in[:, k0, :, :] = 1.0  # b[k,j,c] = [k == k0]
    x = oracle.tri_mul_forward64(a, onehot_in, "incoming")
    assert np.array_equal(x, np.broadcast_to(a[:, k0, :, None, :], x.shape))  # x[i,j,c] = a[k0,i,c]


def test_rank_one_closed_form():
    N, C = 7, 3
    rng = np.random.default_rng(4)
    u, v, w, g = rng.standard_normal(N), rng.standard_normal(N), rng.standard_normal(N), rng.standard_normal(C)
    a = np.einsum("i,k,c->ikc", u, w, g)[None]
    b = np.einsum("j,k->jk", v, w)[None, :, :, None] * np.ones(C)
    x = oracle.tri_mul_forward64(a, b, "outgoing")[0]
    np.testing.assert_allclose(x, np.einsum("i,j,c->ijc", u, v, g) * (w @ w), rtol=1e-12, atol=1e-12)


def test_outgoing_with_equal_operands_is_symmetric():
    a = _rand((2, 6, 6, 5), 5)
    x = oracle.tri_mul_forward64(a, a, "outgoing")
    np.testing.assert_allclose(x, x.transpose(0, 2, 1, 3), rtol=0, atol=1e-12)
    assert not np.allclose(oracle.tri_mul_forward64(a, a, "incoming"),
                           oracle.tri_mul_forward64(a, a, "outgoing"))


def test_incoming_is_outgoing_on_transposed_pairs():
    a, b = _rand((2, 6, 6, 4), 6), _rand((2, 6, 6, 4), 7)
    t = (0, 2, 1, 3)
    np.testing.assert_allclose(oracle.tri_mul_forward64(a, b, "incoming"),
                               oracle.tri_mul_forward64(a.transpose(t), b.transpose(t), "outgoing"),
                               rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("direction", oracle.DIRECTIONS)
def test_gradients_by_central_differences(direction):
    Bn, N, C = 1, 4, 2
    a, b, dx = _rand((Bn, N, N, C), 8), _rand((Bn, N, N, C), 9), _rand((Bn, N, N, C), 10)
    da, db = oracle.tri_mul_backward64(a, b, dx, direction)

    def loss(aa, bb):
        return float((oracle.tri_mul_loops64(aa, bb, direction) * dx).sum())

    eps = 1e-3
    for idx in np.ndindex(a.shape):
        e = np.zeros_like(a)
        e[idx] = eps
        # the loss is bilinear, so the central difference is exact up to rounding
        assert abs((loss(a + e, b) - loss(a - e, b)) / (2 * eps) - da[idx]) < 1e-9, ("da", idx)
        assert abs((loss(a, b + e) - loss(a, b - e)) / (2 * eps) - db[idx]) < 1e-9, ("db", idx)


@pytest.mark.parametrize("direction", oracle.DIRECTIONS)
def test_bilinear_adjoint_identity(direction):
    # x is linear in a and in b, so <dx, x> = <da, a> = <db, b>
    a, b, dx = _rand((2, 9, 9, 3), 11), _rand((2, 9, 9, 3), 12), _rand((2, 9, 9, 3), 13)
    x = oracle.tri_mul_forward64(a, b, direction)
    da, db = oracle.tri_mul_backward64(a, b, dx, direction)
    ref = float((dx * x).sum())
    assert abs(float((da * a).sum()) - ref) < 1e-9 * max(1.0, abs(ref))
    assert abs(float((db * b).sum()) - ref) < 1e-9 * max(1.0, abs(ref))


def test_gate_closed_forms():
    rng = np.random.default_rng(20)
    p = rng.standard_normal((1, 4, 4, 3))
    # sigmoid(0) = 1/2 exactly; sigmoid(+-40) is 1 and 0 to double precision
    assert np.array_equal(oracle.gate_forward64(np.zeros_like(p), p), p / 2)
    np.testing.assert_allclose(oracle.gate_forward64(np.full_like(p, 40.0), p), p, rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.gate_forward64(np.full_like(p, -40.0), p), 0 * p, rtol=0, atol=1e-16)
    # sigmoid(x) + sigmoid(-x) = 1
    g = rng.standard_normal(p.shape) * 3
    np.testing.assert_allclose(oracle.gate_forward64(g, p) + oracle.gate_forward64(-g, p), p, rtol=1e-14, atol=1e-14)
    # masked pair entries give zeros in every channel
    m = (rng.random((1, 4, 4)) > 0.5).astype(np.uint8)
    a = oracle.gate_forward64(g, p, m)
    assert np.all(a[m == 0] == 0) and np.array_equal(a[m == 1], oracle.gate_forward64(g, p)[m == 1])


def test_gate_gradients_by_central_differences():
    rng = np.random.default_rng(21)
    g, p, da = (rng.standard_normal((1, 3, 3, 2)) for _ in range(3))
    m = np.array([[[1, 0, 1], [1, 1, 0], [0, 1, 1]]], dtype=np.uint8)
    dg, dp = oracle.gate_backward64(g, p, da, m)

    def loss(gg, pp):
        return float((oracle.gate_forward64(gg, pp, m) * da).sum())

    eps = 1e-6
    for idx in np.ndindex(g.shape):
        e = np.zeros_like(g)
        e[idx] = eps
        assert abs((loss(g + e, p) - loss(g - e, p)) / (2 * eps) - dg[idx]) < 1e-7, ("dg", idx)
        assert abs((loss(g, p + e) - loss(g, p - e)) / (2 * eps) - dp[idx]) < 1e-7, ("dp", idx)
