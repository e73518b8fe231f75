"""Helpers shared by the GPU parity tests: device transfer, library calls, comparisons."""
from __future__ import annotations

import sys

import numpy as np

import post_weight_quantization_21_amd as gq


def torch_mod():
    import torch
    return torch


def dev_x(X: np.ndarray, pad_to: int = 8):
    """X ([d][n] bf16 bits or fp32) on the device; rows padded to a multiple of `pad_to` elements."""
    torch = torch_mod()
    d, n = X.shape
    ld = (n + pad_to - 1) // pad_to * pad_to
    if X.dtype == np.uint16:
        buf = np.zeros((d, ld), dtype=np.uint16)
        buf[:, :n] = X
        t = torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        buf = np.zeros((d, ld), dtype=np.float32)
        buf[:, :n] = X
        t = torch.from_numpy(buf).cuda()
    return t[:, :n]


def cuda(a: np.ndarray):
    return torch_mod().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_pipeline(W: np.ndarray, X: np.ndarray, cfg, n_sample_rows=None):
    """Steps 1-4 on the GPU through the C ABI.  Returns host arrays."""
    torch = torch_mod()
    d_out, d_in = W.shape
    Xd = dev_x(X)
    H = torch.zeros(d_in, d_in, dtype=torch.float32, device="cuda")
    hdiag = torch.zeros(d_in, dtype=torch.float64, device="cuda") if cfg.act_order else None
    gq.hessian_accumulate(H, Xd, hdiag)
    del Xd
    Wd = cuda(W.astype(np.float32))
    res, H, U = gq.gptq_layer(Wd, None, cfg, H=H, hdiag=hdiag)
    Wo = cuda(W.astype(np.float32))
    loss = gq.layer_loss(Wo, res.codes, res.scales, res.zeros, H, cfg.group_size, g_idx=res.g_idx)
    torch.cuda.synchronize()
    out = dict(codes=host(res.codes), scales=host(res.scales), zeros=host(res.zeros), g_idx=host(res.g_idx),
               perm=host(res.perm), info=int(host(res.info)[0]), loss=float(host(loss)[0]), w_at_q=host(Wd))
    return out


def first_mismatch(a_codes_perm: np.ndarray, b_codes_perm: np.ndarray) -> np.ndarray:
    """Per row, processing position of the first differing code (d if none)."""
    diff = a_codes_perm != b_codes_perm
    d = diff.shape[1]
    has = diff.any(axis=1)
    first = np.where(has, diff.argmax(axis=1), d)
    return first


def compare_layer(gpu: dict, ref: dict, group: int, d_in: int):
    """Parity statistics of GPTQ outputs: code agreement, scale/zero errors."""
    g = group if group > 0 else d_in
    perm = ref["perm"]
    match = float(np.mean(gpu["codes"] == ref["codes"]))
    gp = gpu["codes"][:, perm]
    rp = ref["codes"][:, perm]
    first = first_mismatch(gp, rp)
    ng = ref["scales"].shape[1]
    starts = np.arange(ng) * g
    clean = starts[None, :] <= first[:, None]  # groups fitted before the row's first flip
    rs = np.abs(gpu["scales"] - ref["scales"]) / np.abs(ref["scales"])
    rz = np.abs(gpu["zeros"] - ref["zeros"]) / np.maximum(np.abs(ref["zeros"]), 1.0)
    return dict(match=match, scale_rel_all=float(rs.max()), scale_rel_clean=float(rs[clean].max()),
                zero_rel_clean=float(rz[clean].max()), zero_rel_all=float(rz.max()),
                rows_with_flip=int((first < d_in).sum()))


def assert_grid_parity(st: dict) -> None:
    """Grid bars: scales within 1e-5 relative and zeros identical on every group fitted before the
    row's first code flip; in a layer with no flip that is every group (the strict reading).  After a
    flip the row's later weights follow another trajectory, so its later grids are not compared."""
    assert st["scale_rel_clean"] <= 1e-5 and st["zero_rel_clean"] == 0.0
    if st["rows_with_flip"] == 0:
        assert st["scale_rel_all"] <= 1e-5 and st["zero_rel_all"] == 0.0
