"""Pins of the length-head oracle (oracle/length_head.py) against values the
mathematics fixes: textbook sigmoid/SiLU values, the clamp of k_hat at its
ends, invariants of the mean over positions, and central finite differences
for every gradient."""
import math

import numpy as np
import pytest
from scipy import special

from oracle import length_head as LH


def _params(rng, H, Hp, scale=0.05):
    W1 = rng.normal(0, scale, (Hp, H))
    b1 = rng.normal(0, 0.1, Hp)
    w2 = rng.normal(0, 0.3, Hp)
    b2 = float(rng.normal(0, 0.2))
    return W1, b1, w2, b2


def test_zero_projection_gives_sigmoid_of_bias():
    # W1 = 0, b1 = 0: SiLU(0) = 0, so the pooled vector is 0 and a_hat = sigmoid(b2).
    h = np.random.default_rng(0).normal(size=(3, 16, 8))
    W1, b1, w2 = np.zeros((4, 8)), np.zeros(4), np.ones(4)
    out = LH.forward(h, W1, b1, w2, 0.0, 1.0)
    assert np.all(out["a_hat"] == 0.5)
    assert np.all(out["k_hat"] == 8)                    # floor(0.5 * 16)
    out = LH.forward(h, W1, b1, w2, math.log(3.0), 1.0)
    assert np.allclose(out["a_hat"], 0.75, rtol=0, atol=1e-15)
    assert np.all(out["k_hat"] == 12)                   # floor(0.75 * 16)


@pytest.mark.parametrize("gamma,expect", [(0.1, 1), (0.124, 1), (0.125, 1), (0.25, 2), (1.0, 8), (1.99, 15),
                                          (2.0, 16), (3.0, 16)])
def test_k_hat_floor_and_clamp(gamma, expect):
    # a_hat = 0.5 exactly; k_hat = clamp(floor(gamma * 0.5 * 16), 1, 16).
    h = np.zeros((1, 16, 4))
    out = LH.forward(h, np.zeros((2, 4)), np.zeros(2), np.zeros(2), 0.0, gamma)
    assert int(out["k_hat"][0]) == expect


def test_single_position_is_sigmoid_of_silu():
    # H = H' = 1, W1 = 1, b1 = 0, w2 = 1, b2 = 0: a_hat = sigmoid(SiLU(x)), with
    # SiLU(x) = x * sigmoid(x) from the library's logistic function.
    x = np.linspace(-6, 6, 13)
    h = x.reshape(-1, 1, 1)
    out = LH.forward(h, np.ones((1, 1)), np.zeros(1), np.ones(1), 0.0, 1.0)
    silu = x * special.expit(x)
    assert np.allclose(out["hbar"][:, 0], silu, rtol=1e-14, atol=1e-15)
    assert np.allclose(out["a_hat"], special.expit(silu), rtol=1e-14, atol=1e-15)


def test_mean_over_positions_invariants():
    rng = np.random.default_rng(1)
    W1, b1, w2, b2 = _params(rng, 32, 8)
    h = rng.normal(size=(4, 16, 32))
    base = LH.forward(h, W1, b1, w2, b2, 1.0)
    # Order of the positions inside a block does not matter.
    perm = h[:, rng.permutation(16), :]
    assert np.allclose(LH.forward(perm, W1, b1, w2, b2, 1.0)["a_hat"], base["a_hat"], rtol=1e-13)
    # A block of k identical positions pools to that position alone.
    one = h[:, :1, :]
    rep = np.repeat(one, 16, axis=1)
    assert np.allclose(LH.forward(rep, W1, b1, w2, b2, 1.0)["a_hat"], LH.forward(one, W1, b1, w2, b2, 1.0)["a_hat"],
                       rtol=1e-13)
    # Requests are independent: each row of the batch alone gives the same value.
    for b in range(4):
        assert np.allclose(LH.forward(h[b:b + 1], W1, b1, w2, b2, 1.0)["a_hat"][0], base["a_hat"][b], rtol=1e-13)


def test_label_and_zero_loss_at_the_label():
    assert np.allclose(LH.label([16, 0, 3], [16, 5, 12]), [1.0, 0.0, 0.25])
    # a_hat = sigmoid(b2) = a* exactly (W1 = 0, b1 = 0): zero loss and zero gradients.
    a_star = 0.25
    b2 = math.log(a_star / (1 - a_star))
    h = np.random.default_rng(2).normal(size=(2, 16, 4))
    g = LH.loss_backward(h, np.zeros((3, 4)), np.zeros(3), np.ones(3), b2, [3, 3], [12, 12])
    assert np.allclose(g["loss"], 0.0, atol=1e-30)
    for key in ("dW1", "db1", "dw2"):
        assert np.allclose(g[key], 0.0, atol=1e-15)
    assert abs(g["db2"]) < 1e-15


def _total_loss(h, W1, b1, w2, b2, A, L):
    return float(LH.loss_backward(h, W1, b1, w2, b2, A, L)["loss"].sum())


def test_gradients_match_central_differences():
    rng = np.random.default_rng(3)
    B, k, H, Hp = 3, 16, 12, 6
    W1, b1, w2, b2 = _params(rng, H, Hp, scale=0.3)
    h = rng.normal(size=(B, k, H))
    A, L = np.array([2, 9, 0]), np.array([10, 12, 4])
    g = LH.loss_backward(h, W1, b1, w2, b2, A, L)
    eps = 1e-6

    def fd(arr, idx, fn):
        a0 = arr[idx]
        arr[idx] = a0 + eps
        up = fn()
        arr[idx] = a0 - eps
        dn = fn()
        arr[idx] = a0
        return (up - dn) / (2 * eps)

    f = lambda: _total_loss(h, W1, b1, w2, b2, A, L)
    for idx in [(0, 0), (2, 5), (5, 11), (3, 7)]:
        assert abs(fd(W1, idx, f) - g["dW1"][idx]) < 1e-8 + 1e-6 * abs(g["dW1"][idx])
    for n in range(Hp):
        assert abs(fd(b1, n, f) - g["db1"][n]) < 1e-8 + 1e-6 * abs(g["db1"][n])
        assert abs(fd(w2, n, f) - g["dw2"][n]) < 1e-8 + 1e-6 * abs(g["dw2"][n])
    bb = np.array([b2])
    fb = lambda: _total_loss(h, W1, b1, w2, bb[0], A, L)
    assert abs(fd(bb, 0, fb) - g["db2"]) < 1e-8 + 1e-6 * abs(g["db2"])


def test_bf16_conversion_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    vals = LH.bf16_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 3.140625 and vals[3] == 0.0
    assert np.signbit(vals[4]) and vals[5] == 3.3895313892515355e38
