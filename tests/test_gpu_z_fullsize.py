"""Full-size parity on the four large workloads, in the launch configuration bench.py times.

The GPU runs the whole layer (all rows) through the C ABI.  The fp64 oracle
computes H and the inverse factor in full, then the column pass on a seeded
sample of rows (rows are independent given U and the order, so a sampled row is
an exact per-row expectation).  Checked:
  * H: every upper entry, |H - H_ref| <= 2e-5 sqrt(H_ii H_jj);
  * order (act-order workload): identical permutation;
  * sampled rows: >= 99.9 % identical codes, scales within 1e-5 relative on the
    groups fitted before a row's first code flip (zeros identical there), and
    the sampled rows' loss 1/2 sum_r D_r H D_r^T within 1e-3 relative.
"""
import time

import numpy as np
import pytest

import datagen
import post_weight_quantization_21_amd as gq
from gpu_util import compare_layer, cuda, host, log, torch_mod, assert_grid_parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_ROWS = 48


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _gpu_layer(lay):
    """Same calls and buffers as bench.py's step."""
    torch = torch_mod()
    d_out, d_in, n = lay["d_out"], lay["d_in"], lay["n_tok"]
    cfg = gq.config(lay["bits"], lay["sym"], lay["group"], lay["block"], lay["damp"], lay["act_order"])
    X = torch.from_numpy(lay["X"].view(np.int16)).cuda().view(torch.bfloat16)
    H = torch.zeros(d_in, d_in, dtype=torch.float32, device="cuda")
    hdiag = torch.zeros(d_in, dtype=torch.float64, device="cuda") if lay["act_order"] else None
    gq.hessian_accumulate(H, X, hdiag)
    del X
    W = cuda(lay["W"])
    res, H, U = gq.gptq_layer(W, None, cfg, H=H, hdiag=hdiag)
    torch.cuda.synchronize()
    return res, H, cfg


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", ["q_proj_7b", "down_proj_7b", "o_proj_70b", "up_proj_70b"])
def test_full_size_layer(oracle_mod, name):
    torch = torch_mod()
    t0 = time.time()
    log(f"full-size {name}: generating")
    lay = datagen.make_layer(name)
    d_out, d_in = lay["d_out"], lay["d_in"]
    res, Hd_gpu, cfg = _gpu_layer(lay)
    assert int(host(res.info)[0]) == 0
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(d_out, N_ROWS, replace=False))
    # GPU loss of the sampled rows, through the C ABI
    rows_t = torch.from_numpy(rows).cuda()
    lg = gq.layer_loss(cuda(lay["W"][rows]), res.codes[rows_t].contiguous(), res.scales[rows_t].contiguous(),
                       res.zeros[rows_t].contiguous(), Hd_gpu, lay["group"], g_idx=res.g_idx)
    gout = dict(codes=host(res.codes)[rows], scales=host(res.scales)[rows], zeros=host(res.zeros)[rows],
                perm=host(res.perm), g_idx=host(res.g_idx), loss=float(host(lg)[0]))
    H_gpu = host(Hd_gpu)
    del res, Hd_gpu, lg
    torch.cuda.empty_cache()
    log(f"  gpu done {time.time() - t0:.0f}s; oracle H")

    H = oracle_mod.hessian(lay["X"], chunk=16384)
    log(f"  oracle H {time.time() - t0:.0f}s")
    iu = np.triu_indices(d_in)
    dg = np.sqrt(np.diag(H))
    bad = 0
    for i0 in range(0, d_in, 1024):  # blockwise to bound host memory
        blk = np.abs(H_gpu[i0:i0 + 1024].astype(np.float64) - H[i0:i0 + 1024])
        tol = 2e-5 * dg[i0:i0 + 1024, None] * dg[None, :]
        mask = np.triu(np.ones_like(blk, dtype=bool), k=i0)
        bad += int(((blk > tol) & mask).sum())
    assert bad == 0, f"{bad} H entries out of tolerance"
    del H_gpu, iu

    hdiag = np.diag(H).copy()
    ref = oracle_mod.gptq(lay["W"], H, lay["bits"], lay["sym"], lay["group"], lay["damp"],
                          act_order=lay["act_order"], rows=rows, hdiag=hdiag)
    What = oracle_mod.dequant(ref["codes"], ref["scales"], ref["zeros"], lay["group"], ref["g_idx"])
    ref["loss"] = oracle_mod.layer_loss(lay["W"][rows], What, H)
    log(f"  oracle pass {time.time() - t0:.0f}s")
    assert np.array_equal(gout["perm"], ref["perm"])
    assert np.array_equal(gout["g_idx"], ref["g_idx"])
    st = compare_layer(gout, ref, lay["group"], d_in)
    rel_loss = abs(gout["loss"] - ref["loss"]) / ref["loss"]
    log(f"  {name}: {st} loss gpu={gout['loss']:.6e} ref={ref['loss']:.6e} rel={rel_loss:.2e} ({time.time() - t0:.0f}s)")
    assert st["match"] >= 0.999
    assert_grid_parity(st)
    assert rel_loss <= 1e-3
