"""Pins of the oracle's bf16 rounding and of the calibration forward Y = bf16(X W^T)."""
import numpy as np
import pytest
import torch


def test_bf16_round_hand_values(oracle_mod):
    """Bit patterns derived by hand from the format (sign, 8 exponent bits, 7 stored bits)."""
    one = 1.0
    cases = [
        (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (one + 2.0 ** -8, 0x3F80),                 # midpoint of 1 and 1 + 2^-7: ties to the even 1.0
        (one + 3 * 2.0 ** -8, 0x3F82),             # midpoint of 0x3F81 and 0x3F82: to the even 0x3F82
        (one + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above a midpoint: up
        (one + 2.0 ** -8 - 2.0 ** -30, 0x3F80),    # just below: down
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # half of it: tie to the even 0
        (1.5 * 2.0 ** -133, 0x0002),               # between subnormals 1 and 2: tie to the even 2
        (2.0 ** -126, 0x0080),                     # smallest normal
        ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
        ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # midpoint to 2^128: to even, which overflows
        (2.0 ** 128, 0x7F80), (-np.inf, 0xFF80),
    ]
    x = np.array([c[0] for c in cases])
    got = oracle_mod.bf16_round(x)
    assert [int(v) for v in got] == [c[1] for c in cases]
    assert int(oracle_mod.bf16_round(np.array([np.nan]))[0]) == 0x7FC0


def test_bf16_round_matches_library_on_fp32_values(oracle_mod):
    """For values that fp32 holds exactly, rounding from fp64 is torch's fp32 -> bf16 conversion."""
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle_mod.bf16_round(x.astype(np.float64)), ref)


def _bits(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_linear_forward_selects_weight_columns(oracle_mod):
    """Unit token vectors pick out one weight column each: Y[t][o] = W[o][k_t] exactly."""
    rng = np.random.default_rng(1)
    d_prev, d_out, n = 37, 11, 20
    W = _bits(rng.standard_normal((d_out, d_prev)))
    ks = rng.integers(0, d_prev, n)
    X = np.zeros((n, d_prev), dtype=np.uint16)
    X[np.arange(n), ks] = 0x3F80  # 1.0
    Y = oracle_mod.linear_forward(X, W)
    assert Y.shape == (n, d_out)
    assert np.array_equal(Y, W[:, ks].T)


def test_linear_forward_integer_sums(oracle_mod):
    """Small integers: the sums are exact integers, rounded to bf16 by the library's fp32 -> bf16."""
    rng = np.random.default_rng(2)
    n, d_prev, d_out = 50, 300, 23
    Xi = rng.integers(-4, 5, (n, d_prev))
    Wi = rng.integers(-4, 5, (d_out, d_prev))
    Y = oracle_mod.linear_forward(_bits(Xi), _bits(Wi))
    exact = Xi.astype(np.int64) @ Wi.T.astype(np.int64)  # |sum| <= 4800: exact in fp32
    assert np.array_equal(Y, _bits(exact))
    assert Y.shape == (n, d_out)


@pytest.mark.parametrize("seed", [3, 4])
def test_linear_forward_single_rounding(oracle_mod, seed):
    """Random values: Y is the fp64 sum rounded once; every entry is within half a bf16 step of it."""
    rng = np.random.default_rng(seed)
    X = _bits(rng.standard_normal((40, 64)))
    W = _bits(rng.standard_normal((24, 64)))
    exact = oracle_mod.widen(X) @ oracle_mod.widen(W).T
    Y = oracle_mod.widen(oracle_mod.linear_forward(X, W))
    half_step = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 9)
    assert np.all(np.abs(Y - exact) <= half_step)
