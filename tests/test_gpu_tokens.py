"""GPU parity of the Hessian from token-major activations (calibration inputs as they arrive).

The token-major entry point transposes blocks of 65536 tokens and runs the
channel-major SYRK on each, so it must equal, bit for bit, the channel-major
entry point called once per such block; and the oracle within the H bound
|H - H_ref| <= 2e-5 sqrt(H_ii H_jj) of the channel-major parity tests.
"""
import numpy as np
import pytest

import datagen
import post_weight_quantization_21_amd as gq
from gpu_util import cuda, dev_x, host, log, torch_mod

pytestmark = pytest.mark.gpu

BLOCK = 65536


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _token_major(X: np.ndarray):
    """[n_tok][d] device tensor of the same values (bf16 bit patterns or fp32)."""
    torch = torch_mod()
    Xt = np.ascontiguousarray(X.T)
    if Xt.dtype == np.uint16:
        return torch.from_numpy(Xt.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(Xt).cuda()


@pytest.mark.parametrize("d,n,dt", [(64, 512, "f32"), (300, 2000, "bf16"), (129, 1000, "bf16"),
                                    (512, 140000, "bf16"), (130, 2 * BLOCK, "bf16"), (8, 70, "bf16")])
def test_token_major_equals_channel_major_blocks(oracle_mod, d, n, dt):
    torch = torch_mod()
    log(f"tokens d={d} n={n} {dt}")
    name = "tiny" if dt == "f32" else "q_proj_7b"
    X = datagen.make_layer(name, d_out=4, d_in=d, n_tok=n, seed=d)["X"]
    assert (X.dtype == np.float32) == (dt == "f32")
    H1 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g1 = torch.zeros(d, dtype=torch.float64, device="cuda")
    gq.hessian_accumulate_tokens(H1, _token_major(X), g1)
    H2 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    g2 = torch.zeros(d, dtype=torch.float64, device="cuda")
    for t0 in range(0, n, BLOCK):
        gq.hessian_accumulate(H2, dev_x(np.ascontiguousarray(X[:, t0:t0 + BLOCK])), g2)
    torch.cuda.synchronize()
    a, b = np.triu(host(H1)), np.triu(host(H2))
    assert np.array_equal(a, b)
    assert np.array_equal(host(g1), host(g2))
    ref = oracle_mod.hessian(X)
    dg = np.sqrt(np.diag(ref))
    tol = 2e-5 * np.outer(dg, dg)
    assert np.all(np.abs(a - np.triu(ref)) <= np.triu(tol) + 1e-30)
    assert np.allclose(host(g1), oracle_mod.hessian_diag(X), rtol=1e-12)


def test_token_chunks_accumulate():
    """Two calls of one block each equal one call over both blocks (the same block sums)."""
    torch = torch_mod()
    d, n = 136, 2 * BLOCK
    X = datagen.make_layer("q_proj_7b", d_out=4, d_in=d, n_tok=n, seed=3)["X"]
    Xt = _token_major(X)
    H1 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    gq.hessian_accumulate_tokens(H1, Xt)
    H2 = torch.zeros(d, d, dtype=torch.float32, device="cuda")
    gq.hessian_accumulate_tokens(H2, Xt[:BLOCK])
    gq.hessian_accumulate_tokens(H2, Xt[BLOCK:])
    torch.cuda.synchronize()
    assert np.array_equal(np.triu(host(H1)), np.triu(host(H2)))


def test_token_major_arguments():
    torch = torch_mod()
    H = torch.zeros(8, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        gq.hessian_accumulate_tokens(H, torch.zeros(4, 8, dtype=torch.float16, device="cuda"))
    lib = gq.load_library()
    import ctypes
    p = ctypes.c_void_p(H.data_ptr())
    # ldx below the channel count, and a workspace that is too small
    assert lib.gptq_hessian_accumulate_tokens(p, None, p, gq.DT_F32, 8, 4, 4, p, 1 << 20, None) == gq.ERR_INVALID_ARG
    assert lib.gptq_hessian_accumulate_tokens(p, None, p, gq.DT_F32, 8, 4, 8, p, 0, None) == gq.ERR_WORKSPACE
    assert lib.gptq_hessian_accumulate_tokens(p, None, p, gq.DT_F32, 8, 0, 8, None, 0, None) == gq.OK
