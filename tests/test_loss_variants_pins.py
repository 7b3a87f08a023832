"""Pins of the loss-variants oracle (oracle/loss_variants.py): the worked toy
position printed on the AdaFlash review (EN) for the mixture, the DFlash
notes' printed position weight, closed forms of the two divergences, their
zeros at q = p, and central finite differences for every gradient."""
import json
import math
import os

import numpy as np
import pytest

from oracle import loss_variants as LV

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _logits(probs):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(probs, np.float64))


def test_mixture_matches_the_worked_example():
    g = json.load(open(os.path.join(GOLD, "opd_worked_example.json")))
    zp, zq = _logits(g["p"]), _logits(g["q"])
    # The page clips each term at delta; at delta = 10 nothing is clipped here.
    loss, _ = LV.variant_row(zp, zq, "mixture", 0, g["alpha"], 10.0)
    assert abs(loss - g["l_opd"]) < 2.5e-4
    t = LV.row_terms(zp, zq, np.inf)
    assert abs(t["ce"] - g["l_hard"]) < 5e-4 and abs(t["R"] - g["l_rkl"]) < 5e-4
    # Entry-wise clipping at a threshold between the printed terms: the two
    # largest positive terms (0.208, 0.092) are capped, the rest kept.
    R, _ = LV.variant_row(zp, zq, "rkl_clip", 0, 0.09)
    assert abs(R - (-0.206 + 0.09 + 0.09 + 0.080)) < 5e-4


def test_position_weight_printed_value():
    # DFlash notes, section 7.3: at block size 16 (lambda = 7) the last predicted
    # position (k = 15) has weight e^{-14/7} = e^{-2} ~ 0.135; the first has 1.
    zp = np.array([2.0, 0.0, -1.0])
    zq = np.array([0.5, 0.2, -0.3])
    ce, _ = LV.variant_row(zp, zq, "rkl", 0)  # any row
    l0, _ = LV.variant_row(zp, zq, "wce", 0, 7.0)
    l14, _ = LV.variant_row(zp, zq, "wce", 14, 7.0)
    t = LV.row_terms(zp, zq, np.inf)
    assert abs(l0 - t["ce"]) < 1e-15
    assert abs(l14 / t["ce"] - math.exp(-2.0)) < 1e-15
    assert abs(math.exp(-2.0) - 0.135) < 5e-4


def test_two_point_closed_forms():
    # Bernoulli distributions: KL(q||p) = a log(a/b) + (1-a) log((1-a)/(1-b)).
    a, b = 0.3, 0.6
    zq, zp = _logits([a, 1 - a]), _logits([b, 1 - b])
    rkl, _ = LV.variant_row(zp, zq, "rkl", 0)
    fkl, _ = LV.variant_row(zp, zq, "fkl", 0)
    assert abs(rkl - (a * math.log(a / b) + (1 - a) * math.log((1 - a) / (1 - b)))) < 1e-14
    assert abs(fkl - (b * math.log(b / a) + (1 - b) * math.log((1 - b) / (1 - a)))) < 1e-14


@pytest.mark.parametrize("variant", LV.VARIANTS)
def test_zero_divergence_at_equal_distributions(variant):
    z = np.random.default_rng(4).normal(size=12)
    loss, g = LV.variant_row(z, z, variant, 3, 0.8 if variant == "mixture" else 7.0, 0.01)
    if variant in ("rkl", "rkl_clip", "fkl"):
        assert abs(loss) < 1e-14 and np.max(np.abs(g)) < 1e-14
    else:  # the hard-label term remains: -log q(x*) and q - onehot
        assert loss > 0 and abs(np.sum(g)) < 1e-14


@pytest.mark.parametrize("variant,p1,p2", [("rkl", 0, 0), ("rkl_clip", 0.05, 0), ("mixture", 0.8, 0.05),
                                           ("fkl", 0, 0), ("wce", 7.0, 0)])
def test_gradients_match_central_differences(variant, p1, p2):
    rng = np.random.default_rng(5)
    V = 9
    zp = rng.normal(0, 1.5, V)
    zq = 0.7 * zp + rng.normal(0, 0.8, V)
    i = 4
    _, g = LV.variant_row(zp, zq, variant, i, p1, p2)
    eps = 1e-6
    for v in range(V):
        up, dn = zq.copy(), zq.copy()
        up[v] += eps
        dn[v] -= eps
        fd = (LV.variant_row(zp, up, variant, i, p1, p2)[0] - LV.variant_row(zp, dn, variant, i, p1, p2)[0]) / (2 * eps)
        assert abs(fd - g[v]) < 1e-7 + 1e-6 * abs(g[v]), (variant, v, fd, g[v])


def test_clip_set_changes_the_gradient():
    # An entry whose term exceeds c gets no gradient of its own and only the -S q share.
    zp = _logits([0.8, 0.15, 0.04, 0.01])
    zq = _logits([0.55, 0.30, 0.10, 0.05])
    _, g_all = LV.variant_row(zp, zq, "rkl_clip", 0, 10.0)
    _, g_cut = LV.variant_row(zp, zq, "rkl_clip", 0, 0.1)   # clips token B (term 0.208)
    assert g_all[1] != g_cut[1]
    q = np.array([0.55, 0.30, 0.10, 0.05])
    t = LV.row_terms(zp, zq, 0.1)
    # clipped entry: q_B (0 - S)
    f = q * (np.log(q) - np.log([0.8, 0.15, 0.04, 0.01]))
    S = np.sum(np.where(f <= 0.1, f + q, 0.0))
    assert abs(g_cut[1] - (-q[1] * S)) < 1e-12
    assert t["R"] < LV.row_terms(zp, zq, 10.0)["R"]


def test_batch_packs_rows_in_request_order():
    rng = np.random.default_rng(6)
    B, k, V = 3, 4, 7
    tgt = rng.normal(size=(B, k + 1, V))
    drf = rng.normal(size=(B, k, V))
    L = np.array([2, 4, 1])
    loss, grad = LV.batch(tgt, drf, L, "wce", 7.0)
    assert loss.shape == (7,) and grad.shape == (7, V)
    l, g = LV.variant_row(tgt[1, 3], drf[1, 3], "wce", 3, 7.0)
    assert loss[2 + 3] == l and np.array_equal(grad[5], g)
