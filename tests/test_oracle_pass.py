"""Pins of the oracle's GPTQ column pass: special cases, identities, brute force."""
import itertools

import numpy as np
import pytest

import datagen


def _layer(d_out, d_in, seed, n_tok=None, outliers=True):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    X = rng.standard_normal((d_in, n_tok or 4 * d_in)).astype(np.float32)
    if outliers:
        X[rng.choice(d_in, max(1, d_in // 16), replace=False)] *= 15.0
    return W, X


GRIDS = [(4, True, 32), (4, False, 32), (3, False, 0), (2, False, 16), (8, True, 64)]


@pytest.mark.parametrize("bits,sym,group", GRIDS)
def test_diagonal_hessian_reduces_to_rtn(oracle_mod, bits, sym, group):
    """With a diagonal H the factor U is diagonal, no error is fed forward and GPTQ is RTN exactly."""
    rng = np.random.default_rng(bits + group)
    W = (rng.standard_normal((12, 128)) * 0.02).astype(np.float32)
    for H in (np.eye(128), np.diag(rng.uniform(0.5, 3.0, 128))):
        g = oracle_mod.gptq(W, H, bits, sym, group, damp_rel=0.01)
        r = oracle_mod.rtn(W, bits, sym, group)
        assert np.array_equal(g["codes"], r["codes"])
        assert np.array_equal(g["scales"], r["scales"])
        assert np.array_equal(g["zeros"], r["zeros"])


def test_two_columns_closed_form(oracle_mod):
    """d_in = 2: after quantizing w0 the best real w1 is w1 - (H01/H11) (w0_hat - w0)."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        A = rng.standard_normal((2, 9))
        H = 2.0 * A @ A.T
        W = rng.standard_normal((6, 2)).astype(np.float32)
        g = oracle_mod.gptq(W, H, 3, False, 0, damp_rel=0.05)
        Hd = g["Hd"]
        w0hat = oracle_mod.dequant(g["codes"][:, :1], g["scales"], g["zeros"], 1)[:, 0]
        expect = W[:, 1].astype(np.float64) - Hd[0, 1] / Hd[1, 1] * (w0hat - W[:, 0])
        assert np.allclose(g["w_at_q"][:, 1], expect, rtol=1e-12, atol=1e-15)


def test_update_is_page_formula_with_explicit_subset_inverses(oracle_mod):
    """The page's update, with H_F^-1 inverted directly on the remaining set F at every step.

    Page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ section: after weight q is quantized
    the remaining weights move by -(w_q - quant(w_q)) / [H_F^-1]_qq * (H_F^-1)_{:,q}.
    Replaying that with the oracle's own dequantized values must reproduce the
    oracle's trajectory (its value of every weight when it was quantized).
    """
    W, X = _layer(3, 40, 1)
    H = oracle_mod.hessian(X)
    g = oracle_mod.gptq(W, H, 4, False, 8, damp_rel=0.01)
    Hd = g["Hd"]
    What = oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 8)
    d = W.shape[1]
    for r in range(W.shape[0]):
        w = W[r].astype(np.float64).copy()
        for q in range(d):
            assert w[q] == pytest.approx(g["w_at_q"][r, q], rel=1e-10, abs=1e-14)
            Finv = np.linalg.inv(Hd[q:, q:])
            w[q:] = w[q:] - (w[q] - What[r, q]) / Finv[0, 0] * Finv[:, 0]
            assert abs(w[q] - What[r, q]) < 1e-14  # the quantized weight itself lands on its grid value


@pytest.mark.parametrize("bits,sym,group", GRIDS)
def test_blocked_equals_unblocked(oracle_mod, bits, sym, group):
    """Lazy batch updates (page "量化经典" §二 step 4; page "PTQ 权重量化" GPTQ section) only reorder sums."""
    W, X = _layer(16, 128, 2)
    H = oracle_mod.hessian(X)
    ref = oracle_mod.gptq(W, H, bits, sym, group, damp_rel=0.01, block=0)
    for B in (1, 5, 8, 32, 48, 128):
        b = oracle_mod.gptq(W, H, bits, sym, group, damp_rel=0.01, block=B)
        assert np.array_equal(b["codes"], ref["codes"]), B
        assert np.allclose(b["w_at_q"], ref["w_at_q"], rtol=0, atol=1e-13)
        assert np.array_equal(b["scales"], ref["scales"])


def test_act_order_equivariance(oracle_mod):
    W, X = _layer(10, 96, 4)
    H = oracle_mod.hessian(X)
    a = oracle_mod.gptq(W, H, 4, True, 32, damp_rel=0.01, act_order=True)
    perm = a["perm"]
    assert list(perm) == list(np.argsort(-np.diag(H), kind="stable"))
    b = oracle_mod.gptq(W[:, perm], H[np.ix_(perm, perm)], 4, True, 32, damp_rel=0.01)
    assert np.array_equal(a["codes"][:, perm], b["codes"])
    assert np.array_equal(a["scales"], b["scales"])
    assert np.array_equal(a["g_idx"][perm], np.arange(96) // 32)


@pytest.mark.parametrize("act_order", [False, True])
def test_error_telescoping_identity(oracle_mod, act_order):
    """W - W_hat = E U row by row, so sum_j e_j^2 == D H_d D^T with D = W_hat - W (processing order)."""
    W, X = _layer(8, 64, 5)
    H = oracle_mod.hessian(X)
    g = oracle_mod.gptq(W, H, 3, False, 16, damp_rel=0.01, act_order=act_order)
    perm = g["perm"]
    What = oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 16, g["g_idx"])
    D = (What - W)[:, perm]
    lhs = np.sum(g["err"] ** 2, axis=1)
    rhs = np.einsum("ri,ij,rj->r", D, g["Hd"], D)
    assert np.allclose(lhs, rhs, rtol=1e-9)
    assert np.allclose(g["err"] @ g["U"], -D, rtol=1e-9, atol=1e-15)


def test_brute_force_lower_bound(oracle_mod):
    """On tiny rows the best of all code vectors (GPTQ's grid held fixed) is never worse than GPTQ."""
    rng = np.random.default_rng(9)
    d, bits = 6, 3
    codes_all = np.array(list(itertools.product(range(2 ** bits), repeat=d)), dtype=np.float64)
    worse = 0
    for t in range(12):
        A = rng.standard_normal((d, 20))
        A[t % d] *= 5.0
        H = 2.0 * A @ A.T
        W = rng.standard_normal((1, d)).astype(np.float32)
        g = oracle_mod.gptq(W, H, bits, False, 0, damp_rel=0.01)
        s, z = float(g["scales"][0, 0]), float(g["zeros"][0, 0])
        What = oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 0)
        l_gptq = oracle_mod.layer_loss(W, What, H)
        cand = ((codes_all.astype(np.float32) - np.float32(z)) * np.float32(s)).astype(np.float64)
        D = cand - W.astype(np.float64)
        l_all = 0.5 * np.einsum("ni,ij,nj->n", D, H, D)
        assert l_all.min() <= l_gptq * (1 + 1e-12)
        # the brute-force table contains GPTQ's own choice, at GPTQ's loss
        idx = int(np.dot(g["codes"][0].astype(np.int64), (2 ** bits) ** np.arange(d - 1, -1, -1)))
        assert l_all[idx] == pytest.approx(l_gptq, rel=1e-12)
        worse += l_gptq > l_all.min() * (1 + 1e-9)
    assert worse < 12  # greedy is sometimes optimal on such tiny rows


def test_hessian_scale_invariance(oracle_mod):
    W, X = _layer(12, 64, 6)
    H = oracle_mod.hessian(X)
    a = oracle_mod.gptq(W, H, 4, False, 16, damp_rel=0.01)
    b = oracle_mod.gptq(W, 4.0 * H, 4, False, 16, damp_rel=0.01)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["scales"], b["scales"])


def test_more_bits_lower_loss(oracle_mod):
    W, X = _layer(16, 64, 8)
    H = oracle_mod.hessian(X)
    losses = []
    for bits in range(2, 9):
        g = oracle_mod.gptq(W, H, bits, False, 16, damp_rel=0.01)
        What = oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 16)
        losses.append(oracle_mod.layer_loss(W, What, H))
    assert all(b < a for a, b in zip(losses, losses[1:]))
    assert losses[-1] < 1e-3 * losses[0]


def test_gptq_beats_rtn_tiny_config(oracle_mod):
    lay = datagen.make_layer("tiny")
    H = oracle_mod.hessian(lay["X"])
    g = oracle_mod.gptq(lay["W"], H, 4, True, 32, damp_rel=0.01)
    r = oracle_mod.rtn(lay["W"], 4, True, 32)
    lg = oracle_mod.layer_loss(lay["W"], oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 32), H)
    lr = oracle_mod.layer_loss(lay["W"], oracle_mod.dequant(r["codes"], r["scales"], r["zeros"], 32), H)
    lx = oracle_mod.layer_loss_from_x(lay["W"], oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 32), lay["X"])
    assert lg == pytest.approx(lx, rel=1e-10)
    assert lg < lr


@pytest.mark.parametrize("group,min_wins", [(0, 95), (16, 75)])
def test_gptq_beats_rtn_on_random_layers(oracle_mod, group, min_wins):
    """Empirical (not a theorem): over 100 random small layers GPTQ's loss is mostly below RTN's.

    With one grid per row GPTQ wins essentially always.  With small groups
    refitted from the updated weights a group's range can grow from the
    feedback it absorbs, so on 4x32 layers GPTQ loses to RTN now and then
    (about 1 in 6); the median loss ratio stays below 1.
    """
    wins, ratios = 0, []
    for seed in range(100):
        W, X = _layer(4, 32, 1000 + seed)
        H = oracle_mod.hessian(X)
        g = oracle_mod.gptq(W, H, 3, False, group, damp_rel=0.01)
        r = oracle_mod.rtn(W, 3, False, group)
        lg = oracle_mod.layer_loss(W, oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], group), H)
        lr = oracle_mod.layer_loss(W, oracle_mod.dequant(r["codes"], r["scales"], r["zeros"], group), H)
        wins += lg < lr
        ratios.append(lg / lr)
    assert wins >= min_wins
    assert np.median(ratios) < 0.95


def test_sampled_rows_equal_full(oracle_mod):
    """Rows are independent given U: quantizing a subset of rows reproduces those rows exactly."""
    W, X = _layer(20, 64, 10)
    H = oracle_mod.hessian(X)
    full = oracle_mod.gptq(W, H, 4, False, 32, damp_rel=0.01, act_order=True)
    rows = [3, 17, 0]
    part = oracle_mod.gptq(W, H, 4, False, 32, damp_rel=0.01, act_order=True, rows=rows)
    assert np.array_equal(part["codes"], full["codes"][rows])
    assert np.array_equal(part["scales"], full["scales"][rows])


def test_group_grid_fitted_from_weights_at_group_start(oracle_mod):
    """A group's grid is the RTN grid of its weights as they stand when its first column is reached.

    The weights of a group at that moment are rebuilt from the trajectory:
    w_k(start) = w_k(when quantized) + sum over group columns i < k of e_i U[i, k].
    """
    W, X = _layer(6, 96, 12)
    H = oracle_mod.hessian(X)
    for sym, bits in ((False, 3), (True, 4)):
        g = oracle_mod.gptq(W, H, bits, sym, 32, damp_rel=0.01)
        U, e, wq = g["U"], g["err"], g["w_at_q"]
        for gi in range(3):
            j0 = gi * 32
            cols = np.arange(j0, j0 + 32)
            start = wq[:, cols].copy()
            for k in range(1, 32):
                start[:, k] += e[:, j0:j0 + k] @ U[j0:j0 + k, j0 + k]
            ref = oracle_mod.rtn(start.astype(np.float32), bits, sym, 0)
            assert np.allclose(ref["scales"][:, 0], g["scales"][:, gi], rtol=1e-6)
            assert np.array_equal(ref["zeros"][:, 0], g["zeros"][:, gi])


def test_pass_uses_damped_hessian(oracle_mod):
    """The factor the pass uses inverts H + lambda I, lambda = damp_rel * mean(diag H).

    A rank-deficient H (fewer tokens than channels) has no inverse, so the
    damped matrix is the one whose telescoping identity must hold.
    """
    W, X = _layer(4, 48, 13, n_tok=24)
    H = oracle_mod.hessian(X)
    assert np.linalg.matrix_rank(H) < 48
    g = oracle_mod.gptq(W, H, 4, False, 16, damp_rel=0.05)
    Hd = H + 0.05 * np.mean(np.diag(H)) * np.eye(48)
    assert np.abs(g["U"].T @ g["U"] @ Hd - np.eye(48)).max() < 1e-8
    What = oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], 16)
    D = What - W
    assert np.allclose(np.sum(g["err"] ** 2, axis=1), np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)
