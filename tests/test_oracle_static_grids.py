"""Pins of the oracle's column pass on grids fixed before the pass.

Page "LLM 量化方法原理与实现详解", §2.3 (granularity): per-group grids and a
single grid for the whole tensor.  "static" fits every group of the original
W before the pass (groups stay in original column order under act-order);
"tensor" fits one grid on the whole original W.  The pins tie these variants
to results fixed by other means: the already pinned dynamic pass where the
two must agree, RTN where no error is fed forward, the two-column closed
form, and the telescoping identity of the updates.
"""
import numpy as np
import pytest


def _layer(d_out, d_in, seed, n_tok=None):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    X = rng.standard_normal((d_in, n_tok or 4 * d_in)).astype(np.float32)
    X[rng.choice(d_in, max(1, d_in // 16), replace=False)] *= 15.0
    return W, X


def _code_f32(x, s, z, bits, sym):
    """Stored code of fp32 values on one grid, written from §2.2's formulas with numpy fp32."""
    x = np.asarray(x, dtype=np.float32)
    s, z = np.float32(s), np.float32(z)
    if sym:
        qmax = np.float32(2 ** (bits - 1) - 1)
        return np.clip(np.rint(x / s), -qmax, qmax) + np.float32(2 ** (bits - 1))
    return np.clip(np.rint(x / s + z), np.float32(0), np.float32(2 ** bits - 1))


@pytest.mark.parametrize("act_order", [False, True])
@pytest.mark.parametrize("bits,sym", [(4, True), (3, False)])
def test_static_per_row_grid_equals_dynamic(oracle_mod, act_order, bits, sym):
    """One group per row: the dynamic grid is fitted at the first processed column, before any
    update, so it is the static grid; the two passes must agree exactly."""
    W, X = _layer(10, 96, 1)
    H = oracle_mod.hessian(X)
    for block in (0, 32):
        d = oracle_mod.gptq(W, H, bits, sym, 0, 0.01, act_order=act_order, block=block)
        s = oracle_mod.gptq(W, H, bits, sym, 0, 0.01, act_order=act_order, block=block, grid="static")
        assert np.array_equal(s["codes"], d["codes"])
        assert np.array_equal(s["scales"], d["scales"])
        assert np.array_equal(s["zeros"], d["zeros"])
        assert np.array_equal(s["w_at_q"], d["w_at_q"])


@pytest.mark.parametrize("bits,sym,group", [(4, True, 16), (3, False, 8), (2, False, 32)])
def test_static_groups_without_feedback_are_rtn(oracle_mod, bits, sym, group):
    """Diagonal H: no error is fed forward, so every weight is rounded on its own group's grid.

    Static groups keep original column order under act-order, so the result is
    RTN of W whatever the processing order.  The groups are given very
    different magnitudes: quantizing a column on another group's grid (for
    instance the group of its processing position) changes its code.  The
    dynamic variant, whose groups follow the processing order, must differ.
    """
    rng = np.random.default_rng(group + bits)
    d = 128
    W = (rng.standard_normal((12, d)) * 0.02).astype(np.float32)
    W *= np.repeat(rng.uniform(0.1, 10.0, d // group), group).astype(np.float32)[None, :]
    H = np.diag(rng.uniform(0.5, 3.0, d))
    r = oracle_mod.rtn(W, bits, sym, group)
    s = oracle_mod.gptq(W, H, bits, sym, group, 0.01, act_order=True, grid="static")
    assert not np.array_equal(s["perm"], np.arange(d))
    assert np.array_equal(s["codes"], r["codes"])
    assert np.array_equal(s["scales"], r["scales"])
    assert np.array_equal(s["zeros"], r["zeros"])
    assert np.array_equal(s["g_idx"], np.arange(d) // group)
    dyn = oracle_mod.gptq(W, H, bits, sym, group, 0.01, act_order=True)
    assert not np.array_equal(dyn["codes"], r["codes"])


def test_static_two_columns_closed_form(oracle_mod):
    """Two columns, one per group: column 0 is rounded on the grid of the original w0; the best real
    w1 is then w1 - (H01/H11) (w0_hat - w0), rounded on the grid fitted on the ORIGINAL w1."""
    rng = np.random.default_rng(3)
    for bits, sym in ((3, False), (4, True)):
        for _ in range(10):
            A = rng.standard_normal((2, 9))
            H = 2.0 * A @ A.T
            W = rng.standard_normal((6, 2)).astype(np.float32)
            g = oracle_mod.gptq(W, H, bits, sym, 1, damp_rel=0.05, grid="static")
            Hd = g["Hd"]
            ref = oracle_mod.rtn(W, bits, sym, 1)
            w0hat = (g["codes"][:, 0].astype(np.float32) - ref["zeros"][:, 0]) * ref["scales"][:, 0]
            w1 = W[:, 1].astype(np.float64) - Hd[0, 1] / Hd[1, 1] * (w0hat.astype(np.float64) - W[:, 0])
            assert np.allclose(g["w_at_q"][:, 1], w1, rtol=1e-12, atol=1e-15)
            for i in range(W.shape[0]):
                c1 = _code_f32(np.float32(g["w_at_q"][i, 1]), ref["scales"][i, 1], ref["zeros"][i, 1], bits, sym)
                assert g["codes"][i, 1] == int(c1)


@pytest.mark.parametrize("grid,group", [("static", 16), ("static", 0), ("tensor", 0)])
def test_fixed_grid_error_telescoping_identity(oracle_mod, grid, group):
    """W - W_hat = E U row by row (processing order), so sum_j e_j^2 == D H_d D^T with D = W_hat - W."""
    W, X = _layer(8, 64, 5)
    H = oracle_mod.hessian(X)
    g = oracle_mod.gptq(W, H, 3, False, group, 0.01, act_order=True, grid=grid)
    perm = g["perm"]
    What = oracle_mod.dequant(g["codes"], g["scales"], g["zeros"], group, g["g_idx"])
    D = (What - W)[:, perm]
    assert np.allclose(np.sum(g["err"] ** 2, axis=1), np.einsum("ri,ij,rj->r", D, g["Hd"], D), rtol=1e-9)
    assert np.allclose(g["err"] @ g["U"], -D, rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("grid,group", [("static", 32), ("tensor", 0)])
def test_fixed_grid_blocked_equals_unblocked(oracle_mod, grid, group):
    """Lazy batches only reorder the sums of the updates."""
    W, X = _layer(16, 128, 2)
    H = oracle_mod.hessian(X)
    ref = oracle_mod.gptq(W, H, 4, False, group, 0.01, act_order=True, block=0, grid=grid)
    for B in (1, 5, 8, 32, 48, 128):
        b = oracle_mod.gptq(W, H, 4, False, group, 0.01, act_order=True, block=B, grid=grid)
        assert np.array_equal(b["codes"], ref["codes"]), B
        assert np.allclose(b["w_at_q"], ref["w_at_q"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("bits,sym", [(4, True), (4, False), (8, True)])
def test_tensor_grid_is_per_row_grid_when_rows_share_their_range(oracle_mod, bits, sym):
    """Every row holds the matrix's largest and smallest value: each row's own grid is then the
    tensor's one grid, so per-tensor RTN and GPTQ equal their per-row forms; on a W whose rows differ
    in range the per-tensor scale is the largest per-row scale."""
    W, X = _layer(12, 64, 7)
    H = oracle_mod.hessian(X)
    Wshared = W.copy()
    Wshared[:, 5] = 0.5
    Wshared[:, 40] = -0.3
    for a, b in ((oracle_mod.rtn(Wshared, bits, sym, 0, grid="tensor"), oracle_mod.rtn(Wshared, bits, sym, 0)),
                 (oracle_mod.gptq(Wshared, H, bits, sym, 0, 0.01, act_order=True, grid="tensor"),
                  oracle_mod.gptq(Wshared, H, bits, sym, 0, 0.01, act_order=True))):
        assert np.array_equal(a["codes"], b["codes"])
        assert np.array_equal(a["scales"], b["scales"])
        assert np.array_equal(a["zeros"], b["zeros"])
    t = oracle_mod.rtn(W, bits, sym, 0, grid="tensor")
    rows = oracle_mod.rtn(W, bits, sym, 0)
    assert np.all(t["scales"] == t["scales"][0, 0])
    if sym:
        assert t["scales"][0, 0] == rows["scales"].max()
    else:
        assert t["scales"][0, 0] >= rows["scales"].max()


def test_tensor_grid_sampled_rows_use_whole_matrix(oracle_mod):
    """The per-tensor grid is fitted on the whole W, so a sample of rows reproduces the full result."""
    W, X = _layer(20, 64, 10)
    W[11, 3] = 0.9  # the matrix's largest weight sits outside the sample
    H = oracle_mod.hessian(X)
    full = oracle_mod.gptq(W, H, 4, True, 0, 0.01, act_order=True, grid="tensor")
    rows = [3, 17, 0]
    part = oracle_mod.gptq(W, H, 4, True, 0, 0.01, act_order=True, rows=rows, grid="tensor")
    assert np.array_equal(part["codes"], full["codes"][rows])
    assert np.array_equal(part["scales"], full["scales"][rows])
    assert part["scales"][0, 0] == np.float32(0.9) / np.float32(7)


def test_fixed_grid_configs_rejected(oracle_mod):
    W, X = _layer(4, 32, 11)
    H = oracle_mod.hessian(X)
    with pytest.raises(ValueError):
        oracle_mod.gptq(W, H, 4, True, 16, 0.01, grid="tensor")
    with pytest.raises(ValueError):
        oracle_mod.gptq(W, H, 4, True, 16, 0.01, grid="bogus")
    with pytest.raises(ValueError):
        oracle_mod.rtn(W, 4, True, 16, grid="tensor")
