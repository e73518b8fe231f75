"""Pins of the oracle's grids (RTN) against values the pages and arithmetic fix."""
import numpy as np
import pytest

from golden_io import load

pytestmark = []


def rtn1(oracle_mod, values, bits, sym):
    w = np.asarray(values, dtype=np.float32)[None, :]
    out = oracle_mod.rtn(w, bits, sym, 0)
    return out["codes"][0], float(out["scales"][0, 0]), float(out["zeros"][0, 0])


def test_worked_example_int4(oracle_mod):
    """Page "15. 大模型量化是什么？..." section "量化的核心": 0.7 on [-2.5, 2.5] -> level 2."""
    g = load("rtn_worked_example.txt")
    vals = [g["group_min"], g["value"], g["group_max"]]
    codes, s, z = rtn1(oracle_mod, vals, g["bits"], sym=False)
    assert abs(s - g["scale_approx"]) < g["print_tolerance"]
    assert int(codes[1]) - int(z) == g["level"]
    xhat = (float(codes[1]) - z) * s
    assert abs(xhat - g["dequant_approx"]) < g["print_tolerance"]
    assert abs(abs(g["value"] - xhat) - g["abs_error_approx"]) < g["print_tolerance"]
    # 16 levels: the range ends land on the first and last code.
    assert int(codes[0]) == 0 and int(codes[2]) == 2 ** g["bits"] - 1


def test_int8_ranges(oracle_mod):
    """Page "LLM 量化方法原理与实现详解" §2.2: INT8 symmetric clamps to +-127, asymmetric uses 0..255."""
    g = load("int8_ranges.txt")
    rng = np.random.default_rng(1)
    v = rng.standard_normal(256).astype(np.float32)
    codes, s, z = rtn1(oracle_mod, v, g["sym_bits"], sym=True)
    q = codes.astype(np.int64) - int(z)
    assert q.max() == g["sym_qmax"] or q.min() == -g["sym_qmax"]
    assert q.max() <= g["sym_qmax"] and q.min() >= -g["sym_qmax"]
    assert s == pytest.approx(np.abs(v).max() / g["sym_qmax"], rel=1e-7)
    codes, s, z = rtn1(oracle_mod, v, g["asym_bits"], sym=False)
    assert codes.min() == g["asym_qmin"] and codes.max() == g["asym_qmax"]


def test_asym_extremes_exact_grid(oracle_mod):
    # scale 0.5, zero 3 exactly: the group's min and max are grid points 0 and 15.
    codes, s, z = rtn1(oracle_mod, [-1.5, 6.0, 0.0, 2.25], 4, sym=False)
    assert s == 0.5 and z == 3.0
    assert list(codes) == [0, 15, 3, 8]  # 2.25/0.5 + 3 = 7.5 -> ties to even 8


def test_round_half_to_even(oracle_mod):
    # symmetric 4-bit: max|x| = 7 -> scale 1, zero 8.
    vals = [7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.49]
    codes, s, z = rtn1(oracle_mod, vals, 4, sym=True)
    assert s == 1.0 and z == 8.0
    assert list(codes.astype(int) - 8) == [7, 0, 2, 2, 0, -2, -2, 3]


def test_asym_rounds_after_adding_zero(oracle_mod):
    """The printed asymmetric code rounds x/scale + zero as one value.

    With x/s = 0.5 and an odd zero point the two orders differ:
    rint(0.5 + 1) = 2, but rint(0.5) + 1 = 1.
    """
    codes, s, z = rtn1(oracle_mod, [-1.0, 14.0, 0.5], 4, sym=False)
    assert s == 1.0 and z == 1.0
    assert int(codes[2]) == 2


def test_zero_and_single_signed_groups(oracle_mod):
    codes, s, z = rtn1(oracle_mod, [0.0] * 8, 4, sym=False)
    assert (s, z) == (1.0, 0.0) and not codes.any()
    codes, s, z = rtn1(oracle_mod, [0.0] * 8, 4, sym=True)
    assert (s, z) == (1.0, 8.0) and (codes == 8).all()
    # all-positive group: the grid still contains 0 (lo = 0), so zero = 0.
    v = np.array([0.25, 1.0, 3.0, 0.75], dtype=np.float32)
    codes, s, z = rtn1(oracle_mod, v, 4, sym=False)
    assert z == 0.0 and s == np.float32(3.0) / np.float32(15.0)
    assert int(codes[2]) == 15
    # all-negative group: hi = 0 maps to the top code
    codes, s, z = rtn1(oracle_mod, -v, 4, sym=False)
    assert z == 15.0 and int(codes[2]) == 0


@pytest.mark.parametrize("bits,sym", [(2, False), (3, False), (4, False), (8, False), (3, True), (4, True), (8, True)])
def test_rtn_half_step_bound(oracle_mod, bits, sym):
    """Every weight inside the grid's span is within half a step of its dequantized value."""
    rng = np.random.default_rng(bits * 10 + sym)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    out = oracle_mod.rtn(W, bits, sym, 64)
    What = oracle_mod.dequant(out["codes"], out["scales"], out["zeros"], 64)
    s = np.repeat(out["scales"], 64, axis=1).astype(np.float64)
    err = np.abs(W.astype(np.float64) - What)
    assert (err <= 0.5 * s * (1 + 1e-6) + 1e-12).all()
    lo = 1 if sym else 0
    assert out["codes"].min() >= lo and out["codes"].max() <= 2 ** bits - 1


def test_rtn_groups_are_independent(oracle_mod):
    """Per-group granularity (page "LLM 量化方法原理与实现详解" §2.3): a group's grid sees only its own columns."""
    rng = np.random.default_rng(5)
    W = rng.standard_normal((4, 128)).astype(np.float32)
    a = oracle_mod.rtn(W, 4, False, 32)
    W2 = W.copy()
    W2[:, 32:64] *= 100.0
    b = oracle_mod.rtn(W2, 4, False, 32)
    for gi in (0, 2, 3):
        sl = slice(gi * 32, gi * 32 + 32)
        assert np.array_equal(a["codes"][:, sl], b["codes"][:, sl])
        assert np.array_equal(a["scales"][:, gi], b["scales"][:, gi])
