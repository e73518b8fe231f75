"""Pins of the oracle's per-channel scaling pre-passes (page "LLM 量化方法原理与实现详解",
§4.2 AWQ and §4.3 SmoothQuant): closed forms of the scale formulas, the balance
SmoothQuant is built for, the equivalence of the scaled problem with the original
one (through X directly), and AWQ's search reducing to RTN at alpha = 0."""
import numpy as np
import pytest

import datagen


def test_scale_formulas_closed_form(oracle_mod):
    # AWQ: (mean|X| / mean|W|)^alpha
    s = oracle_mod.awq_scales([4.0, 1.0, 9.0, 2.0], [1.0, 1.0, 1.0, 0.0], 0.5)
    assert np.allclose(s, [2.0, 1.0, 3.0, 1.0], rtol=1e-6)  # the last column is all zero: s = 1
    assert np.array_equal(oracle_mod.awq_scales([4.0, 1.0], [1.0, 1.0], 0.0), np.ones(2, dtype=np.float32))
    # SmoothQuant: max|X|^a / max|W|^(1-a)
    s = oracle_mod.smooth_scales([16.0, 1.0], [4.0, 1.0], 0.5)
    assert np.allclose(s, [2.0, 1.0], rtol=1e-6)
    assert np.allclose(oracle_mod.smooth_scales([16.0, 1.0], [4.0, 1.0], 1.0), [16.0, 1.0], rtol=1e-6)
    assert np.allclose(oracle_mod.smooth_scales([16.0, 1.0], [4.0, 2.0], 0.0), [0.25, 0.5], rtol=1e-6)


def test_channel_and_weight_statistics(oracle_mod):
    X = np.array([[1.0, -3.0, 2.0], [0.0, 0.5, -0.5]], dtype=np.float32)  # 2 channels x 3 tokens
    mx, mn = oracle_mod.channel_stats(X)
    assert np.allclose(mx, [3.0, 0.5]) and np.allclose(mn, [2.0, 1.0 / 3.0])
    W = np.array([[1.0, -2.0], [-3.0, 0.0]], dtype=np.float32)  # 2 rows x 2 input columns
    wx, wn = oracle_mod.weight_stats(W)
    assert np.allclose(wx, [3.0, 2.0]) and np.allclose(wn, [2.0, 1.0])


@pytest.mark.parametrize("alpha", [0.25, 0.5, 0.75])
def test_smoothing_balances_the_ranges(oracle_mod, alpha):
    """After X' = X / s and W' = W s: max|X'_j| = (max|X_j| max|W_j|)^(1-a) and
    max|W'_j| = (max|X_j| max|W_j|)^a; at a = 0.5 both ranges meet at sqrt(max|X_j| max|W_j|)."""
    lay = datagen.make_layer("tiny")
    X, W = lay["X"], lay["W"]
    amax, _ = oracle_mod.channel_stats(X)
    wmax, _ = oracle_mod.weight_stats(W)
    s = oracle_mod.smooth_scales(amax, wmax, alpha).astype(np.float64)
    xs = np.abs(oracle_mod.widen(X) / s[:, None]).max(axis=1)
    ws = np.abs(W.astype(np.float64) * s[None, :]).max(axis=0)
    assert np.allclose(xs, (amax * wmax) ** (1 - alpha), rtol=1e-5)
    assert np.allclose(ws, (amax * wmax) ** alpha, rtol=1e-5)
    if alpha == 0.5:
        assert np.allclose(xs, ws, rtol=1e-5)


def test_scaled_problem_is_the_original_one(oracle_mod):
    """Quantizing W' = W diag(s) and undoing the scale: the loss through H' = S^-1 H S^-1 on W' equals
    ||(Q(W') S^-1 - W) X||^2 computed from X itself."""
    lay = datagen.make_layer("tiny")
    X, W = lay["X"], lay["W"]
    H = oracle_mod.hessian(X)
    _, amean = oracle_mod.channel_stats(X)
    _, wmean = oracle_mod.weight_stats(W)
    s = oracle_mod.awq_scales(amean, wmean, 0.5)
    Ws, Hs = oracle_mod.scale_layer(W, H, s)
    r = oracle_mod.rtn(Ws, 4, True, 32)
    Wq = oracle_mod.dequant(r["codes"], r["scales"], r["zeros"], 32)
    l_scaled = oracle_mod.layer_loss(Ws, Wq, Hs)
    l_direct = oracle_mod.layer_loss_from_x(W, Wq / s.astype(np.float64)[None, :], X)
    assert l_scaled == pytest.approx(l_direct, rel=1e-6)


def test_awq_search(oracle_mod):
    """alpha = 0 is plain RTN; on a layer with salient channels the search beats it (the pages' claim)."""
    lay = datagen.make_layer("tiny")
    X, W = lay["X"], lay["W"]
    H = oracle_mod.hessian(X)
    _, amean = oracle_mod.channel_stats(X)
    alphas, losses, best, s = oracle_mod.awq_search(W, H, amean, 4, True, 32)
    assert alphas[0] == 0.0 and len(alphas) == 20 and max(alphas) < 1.0
    r = oracle_mod.rtn(W, 4, True, 32)
    l_rtn = oracle_mod.layer_loss(W, oracle_mod.dequant(r["codes"], r["scales"], r["zeros"], 32), H)
    assert losses[0] == pytest.approx(l_rtn, rel=1e-12)
    assert losses[best] == losses.min() and best == int(np.argmin(losses))
    assert losses[best] < 0.5 * l_rtn
    _, wmean = oracle_mod.weight_stats(W)
    assert np.array_equal(s, oracle_mod.awq_scales(amean, wmean, alphas[best]))
