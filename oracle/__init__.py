"""fp64 CPU oracle of GPTQ layer quantization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the two
share no code: the oracle is numpy (fp64) plus the C column pass in
``gptq_oracle.c`` (fp64, OpenMP over rows).

Steps, in the pages' order:

1. ``hessian``: H = 2 X X^T, summed over all calibration tokens (page "LLM 量化
   方法原理与实现详解", §4.1 GPTQ, the Hessian line of the printed sketch).
2. ``act_order_perm``: optional column order by descending diag(H) (page
   "量化经典：LLM.int8 / GPTQ / AWQ", §二 "方法核心" step 2 orders columns by the
   Hessian; the descending direction is the one the workload definition fixes).
3. ``damp``: H_d = H + lambda I with lambda = damp_rel * mean(diag H) (not on the
   pages; the standard regulariser that makes H_d positive definite).
4. ``inv_chol_upper``: U = upper Cholesky factor of H_d^-1 (U^T U = H_d^-1).  The
   sketch on page "LLM 量化方法原理与实现详解" §4.1 inverts H "via Cholesky";
   this is the plain definition written with library primitives.  ``obs_rows``
   is the literal elimination sequence H_F^-1 of page "PTQ 权重量化：从 GPTQ 到
   AWQ" (GPTQ section) and pins U in the tests.
5. ``gptq``: the greedy column pass with error feedback (C, ``gptq_oracle.c``),
   unblocked by default, or with lazy batches of B columns; group grids fitted
   as the pass reaches them (dynamic), from the original W before the pass
   (static), or one grid for the whole matrix (tensor) -- page "LLM 量化方法原理
   与实现详解", §2.3 granularity.
6. ``layer_loss``: ||W X - W_hat X||_F^2 = 1/2 sum_r D_r H D_r^T with D = W_hat - W
   and the undamped H (page "LLM 量化方法原理与实现详解", §4.1 objective).
7. ``pack_codes`` / ``w4a16_matmul``: the codes as little-endian bit streams and
   the product of 16-bit activations with the dequantized 4-bit weights.
8. ``awq_search`` / ``smooth_scales`` / ``scale_layer``: the per-channel scaling
   pre-passes (page "LLM 量化方法原理与实现详解", §4.2 AWQ and §4.3 SmoothQuant)
   and the equivalent problem (W diag(s), diag(s)^-1 H diag(s)^-1) GPTQ then solves.

9. ``linear_forward``: the forward of the layer before, Y = bf16(X W^T), whose
   outputs are the calibration inputs step 1 sums over (page "量化经典", §二
   "方法核心" step 1: the calibration set runs through the model layer by layer;
   page "LLM 量化方法原理与实现详解", §3.1, the PTQ flow); ``bf16_round`` is
   the format's round-to-nearest-even.

Every function is pinned by ``tests/test_oracle_*.py`` (closed forms, special
cases, invariants, brute force and the pages' worked example).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        from . import build as _b
        path = _b.build(force=False)
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_rtn.argtypes = [i64, i64, vp, i32, i32, i64, vp, vp, vp]
        lib.oracle_rtn.restype = i32
        lib.oracle_gptq_pass.argtypes = [i64, i64, vp, i64, vp, i32, i32, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_gptq_pass.restype = i32
        lib.oracle_gptq_pass_fixed.argtypes = [i64, i64, vp, i64, vp, i32, i32, vp, i64, vp, vp, i64, vp, vp, vp]
        lib.oracle_gptq_pass_fixed.restype = i32
        lib.oracle_hessian_entries.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp]
        lib.oracle_hessian_entries.restype = i32
        _LIB = lib
    return _LIB


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def widen(X: np.ndarray) -> np.ndarray:
    """Exact fp64 values of X given as bf16 bit patterns (uint16) or fp32."""
    if X.dtype == np.uint16:
        return (X.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return X.astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp64 values rounded once to the format's 8
    significant bits, ties to even; subnormals on the 2^-133 grid; past the
    largest finite value, inf; NaN -> the quiet NaN 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a = m 2^e, m in [0.5, 1): the leading bit is 2^(e-1)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))  # spacing of 8-bit significands, the subnormal grid below 2^-126
    r = np.rint(a / q) * q  # round half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


# ----------------------------------------------------------------------------
# the layer before: calibration forward
# ----------------------------------------------------------------------------
def linear_forward(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Y[t][o] = bf16(sum_i X[t][i] W[o][i]): X [n][d_prev] and W [d_out][d_prev]
    as bf16 bit patterns; the products are exact in fp64, summed in fp64, and
    the sum rounded once to bf16.  Returns Y's bit patterns [n][d_out]."""
    return bf16_round(widen(X) @ widen(W).T)


# ----------------------------------------------------------------------------
# step 1: Hessian
# ----------------------------------------------------------------------------
def hessian(X: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """H = 2 X X^T in fp64 (full symmetric matrix), summed over token chunks."""
    d = X.shape[0]
    H = np.zeros((d, d), dtype=np.float64)
    for t0 in range(0, X.shape[1], chunk):
        xc = widen(X[:, t0:t0 + chunk])
        H += xc @ xc.T
    H *= 2.0
    return H


def hessian_entries(X: np.ndarray, rows, cols) -> np.ndarray:
    """Sampled entries H[i, j] = 2 sum_t X[i,t] X[j,t], each an fp64 dot product."""
    X = np.ascontiguousarray(X)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.zeros(rows.shape[0], dtype=np.float64)
    _lib().oracle_hessian_entries(_p(X), int(X.dtype == np.uint16), X.shape[0], X.shape[1], X.shape[1],
                                  rows.shape[0], _p(rows), _p(cols), _p(out))
    return out


def hessian_diag(X: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """diag(H) = 2 sum_t X[i,t]^2 in fp64."""
    out = np.zeros(X.shape[0], dtype=np.float64)
    for t0 in range(0, X.shape[1], chunk):
        xc = widen(X[:, t0:t0 + chunk])
        out += np.einsum("it,it->i", xc, xc)
    return 2.0 * out


# ----------------------------------------------------------------------------
# steps 2-4: order, damping, inverse factor
# ----------------------------------------------------------------------------
def act_order_perm(diag: np.ndarray) -> np.ndarray:
    """Columns by descending diag(H); equal keys keep the lower index first."""
    return np.argsort(-np.asarray(diag, dtype=np.float64), kind="stable").astype(np.int32)


def damp(H: np.ndarray, damp_rel: float) -> np.ndarray:
    Hd = np.array(H, dtype=np.float64, copy=True)
    lam = damp_rel * np.mean(np.diag(Hd))
    Hd[np.diag_indices_from(Hd)] += lam
    return Hd


def inv_chol_upper(Hd: np.ndarray) -> np.ndarray:
    """Upper U with U^T U = Hd^-1 (Cholesky factor of the inverse, transposed)."""
    L = np.linalg.cholesky(np.linalg.inv(Hd))
    return np.ascontiguousarray(L.T)


def obs_rows(Hd: np.ndarray) -> np.ndarray:
    """Literal OBS elimination: row j of V is row j of H_F^-1 on F = {j, ..., d-1}.

    Starting from H_d^-1, after column j is fixed the inverse Hessian of the
    remaining set is the Schur-complement downdate
    Hinv_F <- Hinv_F - Hinv_F[:, j] Hinv_F[j, :] / Hinv_F[j, j].
    O(d^3) Python-level work: use on small matrices only.
    """
    d = Hd.shape[0]
    Hinv = np.linalg.inv(Hd)
    V = np.zeros_like(Hinv)
    for j in range(d):
        V[j, j:] = Hinv[j, j:]
        col = Hinv[j + 1:, j].copy()
        row = Hinv[j, j + 1:].copy()
        Hinv[j + 1:, j + 1:] -= np.outer(col, row) / Hinv[j, j]
    return V


# ----------------------------------------------------------------------------
# step 5: the column pass
# ----------------------------------------------------------------------------
def gptq_pass(W: np.ndarray, U: np.ndarray, bits: int, sym: bool, group: int, block: int = 0):
    """Column pass on rows of W (processing order).  Returns a dict of arrays."""
    W64 = np.ascontiguousarray(W, dtype=np.float64)
    U64 = np.ascontiguousarray(U, dtype=np.float64)
    n, d = W64.shape
    g = group if group > 0 else d
    ng = d // g
    codes = np.zeros((n, d), dtype=np.uint8)
    scales = np.zeros((n, ng), dtype=np.float32)
    zeros = np.zeros((n, ng), dtype=np.float32)
    w_at_q = np.zeros((n, d), dtype=np.float64)
    err = np.zeros((n, d), dtype=np.float64)
    st = _lib().oracle_gptq_pass(n, d, _p(W64), d, _p(U64), bits, int(bool(sym)), group, block,
                                 _p(codes), _p(scales), _p(zeros), _p(w_at_q), _p(err))
    if st != 0:
        raise ValueError(f"oracle_gptq_pass failed ({st})")
    return dict(codes=codes, scales=scales, zeros=zeros, w_at_q=w_at_q, err=err)


def gptq_pass_fixed(W: np.ndarray, U: np.ndarray, bits: int, sym: bool, col_grid, gscales, gzeros,
                    block: int = 0):
    """Column pass on grids fixed beforehand: processing column j uses grid col_grid[j] of its row."""
    W64 = np.ascontiguousarray(W, dtype=np.float64)
    U64 = np.ascontiguousarray(U, dtype=np.float64)
    n, d = W64.shape
    cg = np.ascontiguousarray(col_grid, dtype=np.int64)
    gs = np.ascontiguousarray(gscales, dtype=np.float32)
    gz = np.ascontiguousarray(gzeros, dtype=np.float32)
    if cg.shape != (d,) or gs.shape != gz.shape or gs.shape[0] != n:
        raise ValueError("gptq_pass_fixed: shape mismatch")
    codes = np.zeros((n, d), dtype=np.uint8)
    w_at_q = np.zeros((n, d), dtype=np.float64)
    err = np.zeros((n, d), dtype=np.float64)
    st = _lib().oracle_gptq_pass_fixed(n, d, _p(W64), d, _p(U64), bits, int(bool(sym)), _p(cg), gs.shape[1],
                                       _p(gs), _p(gz), block, _p(codes), _p(w_at_q), _p(err))
    if st != 0:
        raise ValueError(f"oracle_gptq_pass_fixed failed ({st})")
    return dict(codes=codes, w_at_q=w_at_q, err=err)


def tensor_grid(W: np.ndarray, bits: int, sym: bool):
    """The one grid of a whole matrix: the per-row grid of W flattened into a single row."""
    r = rtn(np.reshape(np.asarray(W, dtype=np.float32), (1, -1)), bits, sym, 0)
    return float(r["scales"][0, 0]), float(r["zeros"][0, 0])


def gptq(W: np.ndarray, H: np.ndarray, bits: int, sym: bool, group: int, damp_rel: float,
         act_order: bool = False, block: int = 0, rows=None, hdiag=None, grid: str = "dynamic"):
    """Whole-layer GPTQ.  Codes are returned in the original column order.

    ``rows`` (optional) selects the output rows to quantize: rows are
    independent given U (and given the grids, which are fitted on the whole
    matrix first when ``grid`` is "tensor"), so a sample of rows gives exact
    per-row results.  ``hdiag`` (optional) is the fp64 diag(H) used as the
    ordering key.  ``grid``: "dynamic" fits each group when the pass reaches
    it (groups in processing order); "static" fits every group of the
    original W before the pass (groups in original column order, so
    g_idx[c] = c // group under act-order too); "tensor" fits one grid on the
    whole original W (group must be 0; scales/zeros [rows][1] all equal).
    """
    W = np.asarray(W)
    d = W.shape[1]
    g = group if group > 0 else d
    if grid not in ("dynamic", "static", "tensor"):
        raise ValueError(f"unknown grid {grid!r}")
    if grid == "tensor" and group != 0:
        raise ValueError("a per-tensor grid has no groups (group must be 0)")
    ts = tensor_grid(W, bits, sym) if grid == "tensor" else None
    if rows is not None:
        W = W[np.asarray(rows)]
    perm = np.arange(d, dtype=np.int32)
    Hp = H
    if act_order:
        perm = act_order_perm(np.diag(H) if hdiag is None else hdiag)
        Hp = H[np.ix_(perm, perm)]
    Hd = damp(Hp, damp_rel)
    U = inv_chol_upper(Hd)
    g_idx = np.empty(d, dtype=np.int32)
    if grid == "dynamic":
        out = gptq_pass(W[:, perm], U, bits, sym, group, block)
        g_idx[perm] = np.arange(d, dtype=np.int32) // g
    else:
        n = W.shape[0]
        if grid == "static":
            r = rtn(W, bits, sym, group)
            gs, gz = r["scales"], r["zeros"]
            col_grid = perm.astype(np.int64) // g
        else:
            gs = np.full((n, 1), ts[0], dtype=np.float32)
            gz = np.full((n, 1), ts[1], dtype=np.float32)
            col_grid = np.zeros(d, dtype=np.int64)
        out = gptq_pass_fixed(W[:, perm], U, bits, sym, col_grid, gs, gz, block)
        out.update(scales=gs, zeros=gz)
        g_idx[:] = np.arange(d, dtype=np.int32) // g
    codes = np.empty_like(out["codes"])
    codes[:, perm] = out["codes"]
    out.update(codes_perm=out["codes"], codes=codes, g_idx=g_idx, perm=perm, U=U, Hd=Hd)
    return out


def rtn(W: np.ndarray, bits: int, sym: bool, group: int, grid: str = "dynamic"):
    """Round-to-nearest baseline with the same grids as the column pass.

    RTN fits every grid on the original W, so "static" is "dynamic" here;
    "tensor" rounds on the one grid of the whole matrix (scales [d_out][1]).
    """
    W32 = np.ascontiguousarray(W, dtype=np.float32)
    n, d = W32.shape
    if grid == "tensor":
        if group != 0:
            raise ValueError("a per-tensor grid has no groups (group must be 0)")
        r = rtn(np.reshape(W32, (1, n * d)), bits, sym, 0)
        return dict(codes=np.reshape(r["codes"], (n, d)), scales=np.full((n, 1), r["scales"][0, 0], dtype=np.float32),
                    zeros=np.full((n, 1), r["zeros"][0, 0], dtype=np.float32))
    if grid not in ("dynamic", "static"):
        raise ValueError(f"unknown grid {grid!r}")
    g = group if group > 0 else d
    codes = np.zeros((n, d), dtype=np.uint8)
    scales = np.zeros((n, d // g), dtype=np.float32)
    zeros = np.zeros((n, d // g), dtype=np.float32)
    st = _lib().oracle_rtn(n, d, _p(W32), bits, int(bool(sym)), group, _p(codes), _p(scales), _p(zeros))
    if st != 0:
        raise ValueError(f"oracle_rtn failed ({st})")
    return dict(codes=codes, scales=scales, zeros=zeros)


# ----------------------------------------------------------------------------
# step 6: dequantization and loss
# ----------------------------------------------------------------------------
def dequant(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int, g_idx=None) -> np.ndarray:
    """W_hat = (code - zero) * scale in fp32 (the stored format), as fp64."""
    d = codes.shape[1]
    g = group if group > 0 else d
    gi = np.arange(d) // g if g_idx is None else np.asarray(g_idx)
    s = scales[:, gi]
    z = zeros[:, gi]
    return ((codes.astype(np.float32) - z) * s).astype(np.float64)


# ----------------------------------------------------------------------------
# before the pass: per-channel scaling (AWQ search, SmoothQuant migration)
# ----------------------------------------------------------------------------
def channel_stats(X: np.ndarray):
    """Per input channel over the tokens: (max |x|, mean |x|), X [d_in][n_tok] (bf16 bits or fp32)."""
    A = np.abs(widen(X))
    return A.max(axis=1), A.mean(axis=1)


def weight_stats(W: np.ndarray):
    """Per input column over the output rows: (max |w|, mean |w|)."""
    A = np.abs(np.asarray(W, dtype=np.float64))
    return A.max(axis=0), A.mean(axis=0)


def awq_scales(act_mean, w_mean, alpha: float) -> np.ndarray:
    """s_j = (mean|X_j| / mean|W_j|)^alpha in fp32 (page "LLM 量化方法原理与实现详解", §4.2, the
    printed AWQ sketch), kept at least 1e-5; a column whose weights are all zero gets s = 1."""
    a = np.asarray(act_mean, dtype=np.float32)
    w = np.asarray(w_mean, dtype=np.float32)
    r = np.where(w > 0, a / np.where(w > 0, w, np.float32(1)), np.float32(1)).astype(np.float32)
    s = np.power(r, np.float32(alpha), dtype=np.float32)
    return np.maximum(s, np.float32(1e-5)).astype(np.float32)


def smooth_scales(act_max, w_max, alpha: float = 0.5) -> np.ndarray:
    """s_j = max|X_j|^alpha / max|W_j|^(1 - alpha), kept at least 1e-5 (§4.3, SmoothQuant sketch), fp32."""
    a = np.asarray(act_max, dtype=np.float32)
    w = np.asarray(w_max, dtype=np.float32)
    num = np.power(a, np.float32(alpha), dtype=np.float32)
    den = np.power(w, np.float32(1.0 - alpha), dtype=np.float32)
    s = np.where(den > 0, num / np.where(den > 0, den, np.float32(1)), np.float32(1)).astype(np.float32)
    return np.maximum(s, np.float32(1e-5)).astype(np.float32)


def scale_layer(W: np.ndarray, H: np.ndarray, s):
    """The equivalent problem after X' = X diag(s)^-1, W' = W diag(s): W' in fp32 (the scaled weights
    are what gets quantized), H' = diag(s)^-1 H diag(s)^-1 = 2 X' X'^T in fp64."""
    s32 = np.asarray(s, dtype=np.float32)
    Ws = (np.asarray(W, dtype=np.float32) * s32[None, :]).astype(np.float32)
    inv = 1.0 / s32.astype(np.float64)
    return Ws, np.asarray(H, dtype=np.float64) * np.outer(inv, inv)


def awq_search(W: np.ndarray, H: np.ndarray, act_mean, bits: int, sym: bool, group: int, n_grid: int = 20):
    """AWQ's scale search (§4.2): for alpha = i / n_grid, i < n_grid, quantize W diag(s) to the nearest
    grid point and measure ||(Q(W diag(s)) diag(s)^-1 - W) X||^2 through H; the smallest loss wins
    (the first on ties).  Returns (alphas, losses, best index, s of the best)."""
    _, w_mean = weight_stats(W)
    alphas = [i / n_grid for i in range(n_grid)]
    losses = []
    for a in alphas:
        s = awq_scales(act_mean, w_mean, a)
        Ws, Hs = scale_layer(W, H, s)
        r = rtn(Ws, bits, sym, group)
        losses.append(layer_loss(Ws, dequant(r["codes"], r["scales"], r["zeros"], group), Hs))
    best = int(np.argmin(losses))
    return alphas, np.array(losses), best, awq_scales(act_mean, w_mean, alphas[best])


# ----------------------------------------------------------------------------
# after the pass: packed codes and the W4A16 product that consumes them
# ----------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int, perm=None) -> np.ndarray:
    """Rows of codes as little-endian bit streams in 32-bit words.

    Column k of the packed row (k-th code of the stream) is codes[o][perm[k]]
    (codes[o][k] without perm) at bits [bits*k, bits*k + bits); the stream is
    padded with zero bits to whole words.  The pages print no storage format
    for low-bit weights (page "量化经典：LLM.int8 / GPTQ / AWQ", GPTQ section:
    3/4-bit weights plus scales); this is the plainest dense one.
    """
    c = np.asarray(codes, dtype=np.uint8)
    if perm is not None:
        c = c[:, np.asarray(perm)]
    n, d = c.shape
    if np.any(c >> bits):
        raise ValueError("a code does not fit in the bit width")
    words = (d * bits + 31) // 32
    bitplane = ((c[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).reshape(n, d * bits)
    stream = np.zeros((n, words * 32), dtype=np.uint8)
    stream[:, :d * bits] = bitplane
    return np.packbits(stream, axis=1, bitorder="little").view("<u4").reshape(n, words)


def unpack_codes(packed: np.ndarray, bits: int, d_in: int) -> np.ndarray:
    """Inverse of pack_codes (in packed column order)."""
    p = np.ascontiguousarray(packed, dtype="<u4")
    n = p.shape[0]
    stream = np.unpackbits(p.view(np.uint8), axis=1, bitorder="little")[:, :d_in * bits].reshape(n, d_in, bits)
    return (stream.astype(np.uint32) << np.arange(bits, dtype=np.uint32)).sum(axis=2).astype(np.uint8)


def w4a16_matmul(X: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int,
                 kperm=None) -> np.ndarray:
    """Y = X' W_hat^T in fp64 with 4-bit packed weights.

    X [M][d_in] (fp16 values); X' = X[:, kperm] (X without kperm): column k of
    X' meets packed column k.  W_hat[o][k] = (code - zero) * scale of group
    k // group (groups contiguous in packed order), taken exactly
    (page "LLM 量化方法原理与实现详解", §2.2 dequantization; weight-only
    4-bit with 16-bit activations: page "量化经典", GPTQ section).
    """
    X64 = np.asarray(X, dtype=np.float64)
    d = X64.shape[1]
    g = group if group > 0 else d
    q = unpack_codes(packed, 4, d).astype(np.float64)
    gi = np.arange(d) // g
    What = (q - np.asarray(zeros, dtype=np.float64)[:, gi]) * np.asarray(scales, dtype=np.float64)[:, gi]
    Xp = X64 if kperm is None else X64[:, np.asarray(kperm)]
    return Xp @ What.T


def layer_loss(W: np.ndarray, What: np.ndarray, H: np.ndarray) -> float:
    """||(W - W_hat) X||_F^2 written through H = 2 X X^T: 1/2 sum_r D_r H D_r^T."""
    D = np.asarray(What, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    return 0.5 * float(np.sum((D @ H) * D))


def layer_loss_from_x(W: np.ndarray, What: np.ndarray, X: np.ndarray) -> float:
    """||W X - W_hat X||_F^2 computed directly from the activations."""
    D = np.asarray(What, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    R = D @ widen(X)
    return float(np.sum(R * R))
