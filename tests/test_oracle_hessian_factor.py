"""Pins of the oracle's Hessian, ordering, damping and inverse factor."""
import numpy as np
import pytest

import datagen


def hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_bf16_widen_exact(oracle_mod):
    bits = np.array([[0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F]], dtype=np.uint16)
    v = oracle_mod.widen(bits)[0]
    assert list(v[:5]) == [1.0, -2.0, 1.0078125, 0.0, 0.0]
    assert v[5] == (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bf16


def test_hessian_orthogonal_rows_closed_form(oracle_mod):
    """Rows of a Hadamard matrix are orthogonal with squared norm n, so 2 X X^T = 2 n I exactly."""
    for n in (4, 16, 64):
        X = hadamard(n).astype(np.float32)
        H = oracle_mod.hessian(X, chunk=max(1, n // 4))
        assert np.array_equal(H, 2.0 * n * np.eye(n))


def test_hessian_is_objective_quadratic_form(oracle_mod):
    """Objective of page "LLM 量化方法原理与实现详解" §4.1: ||W X - W_hat X||^2 == 1/2 D H D^T.

    The left side is computed directly from X, so this pins the factor 2 and
    that X is stored one row per input channel.
    """
    rng = np.random.default_rng(3)
    X = rng.standard_normal((24, 300)).astype(np.float32)
    W = rng.standard_normal((5, 24))
    What = W + 0.1 * rng.standard_normal((5, 24))
    H = oracle_mod.hessian(X, chunk=64)
    a = oracle_mod.layer_loss(W, What, H)
    b = oracle_mod.layer_loss_from_x(W, What, X)
    assert a == pytest.approx(b, rel=1e-12)


def test_hessian_entries_and_bf16_path(oracle_mod):
    r = datagen.recipe("q_proj_7b", d_out=8, d_in=96, n_tok=1000)
    X = datagen.make_activations(r, 0)
    assert X.dtype == np.uint16
    H = oracle_mod.hessian(X, chunk=128)
    assert np.array_equal(H, H.T)
    ev = np.linalg.eigvalsh(H)
    assert ev.min() > -1e-9 * ev.max()
    rows = np.array([0, 5, 95, 17, 40])
    cols = np.array([0, 90, 95, 3, 40])
    ent = oracle_mod.hessian_entries(X, rows, cols)
    assert np.allclose(ent, H[rows, cols], rtol=1e-12, atol=1e-9)
    dg = oracle_mod.hessian_diag(X, chunk=300)
    assert np.allclose(dg, np.diag(H), rtol=1e-12)


def test_damping_mean_diag(oracle_mod):
    H = np.diag([1.0, 2.0, 3.0, 6.0]) + 0.5
    Hd = oracle_mod.damp(H, 0.1)
    lam = 0.1 * np.mean(np.diag(H))
    assert np.allclose(np.diag(Hd) - np.diag(H), lam)
    off = ~np.eye(4, dtype=bool)
    assert np.array_equal(Hd[off], H[off])


def test_act_order_perm_descending_stable(oracle_mod):
    key = np.array([1.0, 5.0, 3.0, 5.0, 0.5, 3.0, 5.0])
    perm = oracle_mod.act_order_perm(key)
    assert list(perm) == [1, 3, 6, 2, 5, 0, 4]


def _spd(d, seed, outliers=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((d, 4 * d))
    if outliers:
        X[rng.choice(d, max(1, d // 20), replace=False)] *= 20.0
    return 2.0 * X @ X.T


@pytest.mark.parametrize("d", [2, 7, 64, 200])
def test_inverse_factor_defining_property(oracle_mod, d):
    H = _spd(d, d)
    Hd = oracle_mod.damp(H, 0.01)
    U = oracle_mod.inv_chol_upper(Hd)
    assert np.array_equal(U, np.triu(U))
    assert (np.diag(U) > 0).all()
    R = U.T @ U @ Hd - np.eye(d)
    assert np.abs(R).max() < 1e-9


def test_obs_elimination_rows_match_factor(oracle_mod):
    """Row j of U is row j of H_F^-1 (F = columns not yet quantized) over sqrt of its diagonal."""
    Hd = oracle_mod.damp(_spd(96, 11), 0.01)
    U = oracle_mod.inv_chol_upper(Hd)
    V = oracle_mod.obs_rows(Hd)
    Vn = V / np.sqrt(np.diag(V))[:, None]
    assert np.allclose(np.triu(Vn), U, rtol=1e-9, atol=1e-12 * np.abs(U).max())


def test_obs_rows_are_rows_of_subset_inverses_tiny(oracle_mod):
    """Most literal reading of H_F^-1 (page "PTQ 权重量化：从 GPTQ 到 AWQ"): invert H_d on F directly, every j."""
    lay = datagen.make_layer("tiny")
    H = oracle_mod.hessian(lay["X"])
    Hd = oracle_mod.damp(H, 0.01)
    V = oracle_mod.obs_rows(Hd)
    d = Hd.shape[0]
    for j in range(d):
        row = np.linalg.inv(Hd[j:, j:])[0]
        assert np.allclose(V[j, j:], row, rtol=1e-8, atol=1e-14 * np.abs(row).max())
