"""Kernel timing of the column pass: launches of each kind and their flops add up to the pass's.

A 4096 x 2048 layer with superblocks of 1024 columns has one superblock update wide enough for the
split-bf16 product (K = 1024, N = 1024: 64 tiles of 256 x 256), the rest on the fp32 matrix cores
(each batch's update of the rest of its superblock).  Every product is 2 M N K flops, so the two kinds
sum to d_out d_in (d_in - B), and the split kind to 2 d_out 1024 1024.
"""
import numpy as np
import pytest

import post_weight_quantization_21_amd as gq
from gpu_util import cuda, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def test_timed_kinds_and_flops():
    torch = torch_mod()
    d_out, d_in, B = 4096, 2048, 128
    rng = np.random.default_rng(5)
    W = cuda((rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32))
    U = torch.triu(torch.from_numpy(rng.standard_normal((d_in, d_in)).astype(np.float32) * 0.01)).cuda()
    U.diagonal().copy_(torch.ones(d_in) + torch.rand(d_in))
    cfg = gq.config(4, False, 128, B, 0.01, False)
    ng = d_in // 128
    codes = torch.empty(d_out, d_in, dtype=torch.uint8, device="cuda")
    scales = torch.empty(d_out, ng, dtype=torch.float32, device="cuda")
    zeros = torch.empty(d_out, ng, dtype=torch.float32, device="cuda")
    gq.timing_enable(True)
    try:
        for op in (gq.TIMED_LAZY, gq.TIMED_LAZY_SPLIT, gq.TIMED_BATCH):
            gq.timing_read(op)
        gq.quantize_layer(W, U, cfg, codes, scales, zeros)
        torch.cuda.synchronize()
        f_ms, f_n, f_fl = gq.timing_read(gq.TIMED_LAZY, with_flops=True)
        s_ms, s_n, s_fl = gq.timing_read(gq.TIMED_LAZY_SPLIT, with_flops=True)
        b_ms, b_n, b_fl = gq.timing_read(gq.TIMED_BATCH, with_flops=True)
    finally:
        gq.timing_enable(False)
    assert b_n == d_in // B and b_fl == 0.0
    assert s_n == 1 and s_fl == 2.0 * d_out * 1024 * 1024
    assert f_n == 2 * (1024 // B - 1)  # each superblock: every batch but the last updates the rest
    assert f_fl + s_fl == float(d_out) * d_in * (d_in - B)
    assert min(f_ms, s_ms, b_ms) > 0.0
    # nothing left once read
    assert gq.timing_read(gq.TIMED_LAZY_SPLIT) == (0.0, 0)
