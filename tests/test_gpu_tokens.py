"""GPU parity of the Hessian from token-major activations (calibration inputs as they arrive).

The token-major SYRK loads [n_tok][ldx] tiles itself and transposes them in
registers into the same LDS image the channel-major SYRK loads directly, so for
bf16 it must equal the channel-major entry point on the transposed activations
bit for bit, and the oracle within the H bound |H - H_ref| <= 2e-5 sqrt(H_ii H_jj)
of the channel-major parity tests.  The fp64 diagonal comes from a pass per
layout that sums in its own order: equal to fp64 rounding (and to the oracle's
within 1e-12).
"""
import ctypes

import numpy as np
import pytest

import datagen
import post_weight_quantization_21_amd as gq
from gpu_util import dev_x, host, log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _token_major(X: np.ndarray, ld: int = 0):
    """[n_tok][d] device view of the same values (bf16 bit patterns or fp32), rows `ld` elements apart
    (default: d rounded up to a multiple of 4)."""
    torch = torch_mod()
    d, n = X.shape
    ld = ld or (d + 3) // 4 * 4
    buf = np.zeros((n, ld), dtype=X.dtype)
    buf[:, :d] = X.T
    if X.dtype == np.uint16:
        t = torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(buf).cuda()
    return t[:, :d]


def _oracle_check(oracle_mod, X, Hg, hd):
    ref = oracle_mod.hessian(X)
    dg = np.sqrt(np.diag(ref))
    tol = 2e-5 * np.outer(dg, dg)
    iu = np.triu_indices(X.shape[0])
    assert np.all(np.abs(Hg.astype(np.float64) - ref)[iu] <= tol[iu] + 1e-30)
    assert not Hg[np.tril_indices(X.shape[0], -1)].any()
    assert np.allclose(hd, oracle_mod.hessian_diag(X), rtol=1e-12)


# (d, n_tok, extra row padding): ragged channel tiles, a partial last stage,
# a call that is only a partial stage, token splits, rows longer than d.
BF16_CASES = [(64, 512, 0), (300, 2000, 0), (129, 1000, 0), (8, 70, 0), (256, 31, 0), (256, 32, 0),
              (256, 69, 12), (1024, 8192, 0), (1300, 3000, 4), (512, 140000, 0), (130, 131072 + 45, 0),
              (4100, 600, 0)]


@pytest.mark.parametrize("d,n,pad", BF16_CASES)
def test_token_major_equals_channel_major(oracle_mod, d, n, pad):
    torch = torch_mod()
    log(f"tokens d={d} n={n} pad={pad}")
    X = datagen.make_layer("q_proj_7b", d_out=4, d_in=d, n_tok=n, seed=d)["X"]
    assert X.dtype == np.uint16
    H1 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g1 = torch.zeros(d, dtype=torch.float64, device="cuda")
    gq.hessian_accumulate_tokens(H1, _token_major(X, (d + 3) // 4 * 4 + pad), g1)
    H2 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g2 = torch.zeros(d, dtype=torch.float64, device="cuda")
    gq.hessian_accumulate(H2, dev_x(X), g2)
    torch.cuda.synchronize()
    a, b = host(H1), host(H2)
    assert np.array_equal(a, b)
    assert np.allclose(host(g1), host(g2), rtol=1e-13, atol=0)
    _oracle_check(oracle_mod, X, a, host(g1))


def test_token_major_without_diagonal(oracle_mod):
    """The kernel without the fp64 diagonal gives the same H."""
    torch = torch_mod()
    d, n = 520, 5000
    X = datagen.make_layer("q_proj_7b", d_out=4, d_in=d, n_tok=n, seed=7)["X"]
    Xt = _token_major(X)
    H1 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    gq.hessian_accumulate_tokens(H1, Xt)
    H2 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g2 = torch.zeros(d, dtype=torch.float64, device="cuda")
    gq.hessian_accumulate_tokens(H2, Xt, g2)
    torch.cuda.synchronize()
    assert np.array_equal(host(H1), host(H2))


@pytest.mark.parametrize("d,n", [(64, 512), (77, 301), (256, 4000)])
def test_token_major_f32(oracle_mod, d, n):
    torch = torch_mod()
    X = datagen.make_layer("tiny", d_out=4, d_in=d, n_tok=n, seed=d)["X"]
    assert X.dtype == np.float32
    H = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g = torch.zeros(d, dtype=torch.float64, device="cuda")
    gq.hessian_accumulate_tokens(H, _token_major(X), g)
    torch.cuda.synchronize()
    _oracle_check(oracle_mod, X, host(H), host(g))


def test_token_chunks_accumulate(oracle_mod):
    """Calls over consecutive token chunks add up to the sums over all tokens."""
    torch = torch_mod()
    d, n = 136, 3 * 20000
    X = datagen.make_layer("q_proj_7b", d_out=4, d_in=d, n_tok=n, seed=3)["X"]
    Xt = _token_major(X)
    H = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g = torch.zeros(d, dtype=torch.float64, device="cuda")
    for t0 in range(0, n, 20000):
        gq.hessian_accumulate_tokens(H, Xt[t0:t0 + 20000], g)
    torch.cuda.synchronize()
    _oracle_check(oracle_mod, X, host(H), host(g))


def test_token_major_arguments():
    torch = torch_mod()
    H = torch.zeros(8, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        gq.hessian_accumulate_tokens(H, torch.zeros(4, 8, dtype=torch.float16, device="cuda"))
    lib = gq.load_library()
    p = ctypes.c_void_p(H.data_ptr())
    # ldx below the channel count, and a workspace that is too small
    assert lib.gptq_hessian_accumulate_tokens(p, None, p, gq.DT_F32, 8, 4, 4, p, 1 << 20, None) == gq.ERR_INVALID_ARG
    assert lib.gptq_hessian_accumulate_tokens(p, None, p, gq.DT_F32, 8, 0, 8, None, 0, None) == gq.OK
    n = 200000
    need = gq.workspace_bytes(gq.OP_HESSIAN_TOKENS, 0, 512, n)
    assert need > 0
    X = torch.zeros(1, dtype=torch.float32, device="cuda")
    px = ctypes.c_void_p(X.data_ptr())
    assert lib.gptq_hessian_accumulate_tokens(p, None, px, gq.DT_BF16, 512, n, 512, p, need - 1, None) == \
        gq.ERR_WORKSPACE
    # bf16 token rows are read 4 channels (8 bytes) at a time
    assert lib.gptq_hessian_accumulate_tokens(p, None, px, gq.DT_BF16, 8, 4, 10, None, 0, None) == gq.ERR_INVALID_ARG
    px2 = ctypes.c_void_p(X.data_ptr() + 4)
    assert lib.gptq_hessian_accumulate_tokens(p, None, px2, gq.DT_BF16, 8, 4, 8, None, 0, None) == gq.ERR_INVALID_ARG
    assert b"8-byte" in lib.gptq_last_error()
