"""Layers whose superblock updates take the split-bf16 product (K >= 512, N >= 512, at least 64
tiles of 256 x 256), with ragged row and column tiles: right-looking and left-looking inner
updates (with their catch-up products: every 512 columns, and before a grid is fitted from a
group that spans batches), K = 1024 and K = 512 superblocks, with and without a column order.

Rows are independent given U and the order, so the oracle's pass on sampled rows (the last rows,
which sit in the partial row tile, included) is an exact per-row expectation: >= 99.9 % identical
codes and the grid bars of the other parity tests.  (Against the oracle the weights each column is
quantized at differ by the same amounts whether these updates run split or on the fp32 matrix cores:
max 7.4e-8, median 4.4e-9 at |w| <= 0.11 on the first layer.)  The whole layer's loss through the C ABI must
match the oracle's loss of the GPU's own outputs within 1e-3 (the bar of the other sampled-row tests).
"""
import numpy as np
import pytest

import post_weight_quantization_21_amd as gq
from gpu_util import assert_grid_parity, compare_layer, gpu_pipeline, log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


# d_out, d_in, super_cols, act_order, bits, symmetric, group
CASES = [
    # one split update (superblock 0, N = 1664: 6.5 column tiles; 4100 rows: a 4-row last tile)
    (4100, 2688, 0, False, 4, False, 128),
    # K = 512 superblocks: four split updates, the last two through the fp32 product
    (4100, 2688, 512, True, 3, True, 64),
    # tall layer: left-looking inner updates, one split update with N = 512
    (16388, 1536, 0, False, 4, True, 128),
    # 113 x 8 = 904 tiles in the first superblock update, a ragged last row tile of 4 rows
    (28676, 3072, 0, False, 4, True, 128),
    # tall layer, dynamic groups of 256 over batches of 128: before each group's grid is
    # fitted the rest of the superblock is brought up to date (left-looking catch-up)
    (16388, 2048, 0, False, 4, False, 256),
]


@pytest.mark.parametrize("d_out,d_in,sc,act,bits,sym,group", CASES)
def test_split_superblock_updates(oracle_mod, d_out, d_in, sc, act, bits, sym, group):
    log(f"split updates d_out={d_out} d_in={d_in} super_cols={sc} act_order={act}")
    rng = np.random.default_rng(d_out + d_in + sc)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    X = rng.standard_normal((d_in, 4096)).astype(np.float32)
    X[rng.choice(d_in, 16, replace=False)] *= 8.0
    cfg = gq.config(bits, sym, group, 128, 0.01, act, super_cols=sc)
    out = gpu_pipeline(W, X, cfg)
    assert out["info"] == 0
    H = oracle_mod.hessian(X)
    # every eighth row (at most about 512) and the partial tile's: enough rows that one row whose code flips (a weight
    # within fp32 rounding of a grid boundary, after which the row follows its own trajectory) stays
    # under the 0.1 % bar
    step = max(8, d_out // 512)
    rows = np.unique(np.concatenate([np.arange(0, d_out, step), np.arange(d_out - 4, d_out)]))
    ref = oracle_mod.gptq(W[rows], H, bits, sym, group, 0.01, act_order=act)
    gout = dict(codes=out["codes"][rows], scales=out["scales"][rows], zeros=out["zeros"][rows])
    assert np.array_equal(out["perm"], ref["perm"])
    st = compare_layer(gout, ref, group, d_in)
    log(f"  {st}")
    assert st["match"] >= 0.999
    assert_grid_parity(st)
    What = oracle_mod.dequant(out["codes"], out["scales"], out["zeros"], group, out["g_idx"])
    ref_loss = oracle_mod.layer_loss(W, What, H)
    assert abs(out["loss"] - ref_loss) <= 1e-3 * ref_loss
