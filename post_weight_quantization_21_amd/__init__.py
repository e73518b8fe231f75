"""Python binding of libgptq (GPTQ layer quantization on MI355X / gfx950).

Thin argument marshalling over the C ABI declared in ``include/gptq.h``:
every step of the method runs in the library's HIP kernels.  PyTorch only
provides device memory (tensors, workspaces) and the current HIP stream.
The binding refuses to run without the built library: there is no fallback.

Names follow the C ABI: ``hessian_accumulate``, ``prepare_hinv``,
``quantize_layer``, ``rtn_quantize``, ``layer_loss``, ``workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgptq.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
DT_F32, DT_BF16, DT_F16 = 0, 1, 2
OP_HESSIAN, OP_PREPARE, OP_QUANTIZE, OP_LOSS, OP_W4A16, OP_HESSIAN_TOKENS, OP_SMOOTH, OP_AWQ = 0, 1, 2, 3, 4, 5, 6, 7
OP_CALIBRATE = 8

EXPORTED = (
    "gptq_hessian_accumulate", "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_rtn_quantize",
    "gptq_layer_loss", "gptq_workspace_bytes", "gptq_status_string", "gptq_last_error",
    "gptq_pack_codes", "gptq_w4a16_gemm", "gptq_hessian_accumulate_tokens",
    "gptq_channel_stats", "gptq_smooth_scales", "gptq_awq_search", "gptq_scale_layer",
    "gptq_quantize_layer_noalloc", "gptq_timing_enable", "gptq_timing_read",
    "gptq_linear_forward", "gptq_calibrate_hessian", "gptq_calibrate_chunk_tokens",
)
TIMED_LAZY, TIMED_BATCH, TIMED_LAZY_SPLIT = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20  # GPTQ_NOALLOC_SCRATCH_BYTES


class GptqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gptq status {status}: {message}")
        self.status = status


class Config(ctypes.Structure):
    """Mirror of ``gptq_config``."""
    _fields_ = [("bits", ctypes.c_int32), ("symmetric", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("damp_rel", ctypes.c_float), ("act_order", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("super_cols", ctypes.c_int32)]


# gptq_grid: when the quantization grids are fitted
GRIDS = {"dynamic": 0, "static": 1, "tensor": 2}


def config(bits: int = 4, symmetric: bool = False, group_size: int = 128, block_size: int = 128,
           damp_rel: float = 0.01, act_order: bool = False, grid: str = "dynamic", super_cols: int = 0) -> Config:
    return Config(int(bits), int(bool(symmetric)), int(group_size), int(block_size), float(damp_rel),
                  int(bool(act_order)), GRIDS[grid], int(super_cols))


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgptq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m post_weight_quantization_21_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(Config)
    sig = {
        "gptq_hessian_accumulate": [vp, vp, vp, i32, i64, i64, i64, vp, sz, vp],
        "gptq_prepare_hinv": [vp, vp, i64, cfgp, vp, vp, vp, vp, sz, vp],
        "gptq_quantize_layer": [vp, i64, i64, vp, vp, cfgp, vp, vp, vp, vp, vp, sz, vp],
        "gptq_quantize_layer_noalloc": [vp, i64, i64, vp, vp, cfgp, vp, vp, vp, vp, vp],
        "gptq_rtn_quantize": [vp, i64, i64, cfgp, vp, vp, vp, vp],
        "gptq_layer_loss": [vp, vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, sz, vp],
        "gptq_workspace_bytes": [ctypes.c_int, i64, i64, i64, cfgp, ctypes.POINTER(sz)],
        "gptq_pack_codes": [vp, i64, i64, i32, vp, vp, vp],
        "gptq_channel_stats": [vp, i32, i64, i64, i64, vp, vp, vp],
        "gptq_smooth_scales": [vp, vp, i64, i64, ctypes.c_float, vp, vp, sz, vp],
        "gptq_awq_search": [vp, i64, i64, vp, vp, i64, cfgp, i32, vp, vp, vp, vp, sz, vp],
        "gptq_scale_layer": [vp, i64, i64, vp, vp, vp, vp],
        "gptq_hessian_accumulate_tokens": [vp, vp, vp, i32, i64, i64, i64, vp, sz, vp],
        "gptq_w4a16_gemm": [vp, i32, i64, i64, i64, vp, vp, vp, vp, i32, i64, vp, i64, vp, sz, vp],
        "gptq_linear_forward": [vp, i64, vp, i64, vp, i64, i64, i64, i64, vp],
        "gptq_calibrate_hessian": [vp, vp, vp, i64, vp, i64, i64, i64, i64, vp, sz, vp],
        "gptq_calibrate_chunk_tokens": [i64],
        "gptq_timing_enable": [i32],
        "gptq_timing_read": [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)],
        "gptq_status_string": [ctypes.c_int],
        "gptq_last_error": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = (ctypes.c_char_p if name in ("gptq_status_string", "gptq_last_error")
                     else ctypes.c_int64 if name == "gptq_calibrate_chunk_tokens" else ctypes.c_int)
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        msg = load_library().gptq_last_error().decode(errors="replace")
        raise GptqError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def timing_enable(on: bool = True) -> None:
    """Record HIP events around the column pass's update products and batch kernels (benchmarks)."""
    _check(load_library().gptq_timing_enable(int(bool(on))))


def timing_read(op: int, with_flops: bool = False):
    """(summed milliseconds, launches[, fp32 flops]) of the recorded kernels of one kind, then forget them."""
    ms, n, fl = ctypes.c_double(0.0), ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(load_library().gptq_timing_read(int(op), ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl)))
    return (ms.value, n.value, fl.value) if with_flops else (ms.value, n.value)


def workspace_bytes(op: int, d_out: int, d_in: int, n_tok: int = 0, cfg: Config | None = None) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().gptq_workspace_bytes(op, d_out, d_in, n_tok, ctypes.byref(cfg) if cfg else None,
                                               ctypes.byref(out)))
    return int(out.value)


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def hessian_accumulate(H, X, hdiag=None, ws=None, stream=None) -> None:
    """H (fp32 [d,d], upper) += 2 X X^T; hdiag (fp64 [d]) += 2 sum x^2.  X: bf16 or fp32 [d][n]."""
    import torch
    _need_cuda(H, hdiag)
    if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D device tensor with unit stride along tokens")
    if X.dtype == torch.bfloat16:
        dt = DT_BF16
    elif X.dtype == torch.float32:
        dt = DT_F32
    else:
        raise ValueError("X must be bfloat16 or float32")
    d, n = X.shape
    if ws is None:
        ws = _workspace(workspace_bytes(OP_HESSIAN, 0, d, n), X.device)
    _check(load_library().gptq_hessian_accumulate(_ptr(H), _ptr(hdiag), _ptr(X), dt, d, n, X.stride(0), _ptr(ws),
                                                  ws.numel(), _stream(stream)))


def hessian_accumulate_tokens(H, X, hdiag=None, ws=None, stream=None) -> None:
    """H (fp32 [d,d], upper) += 2 X^T X for token-major X: bf16 or fp32 [n_tok][d], one row per token.
    bf16 rows must be a multiple of 4 elements apart (X.stride(0) % 4 == 0) and 8-byte aligned."""
    import torch
    _need_cuda(H, hdiag)
    if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D device tensor with unit stride along channels")
    if X.dtype == torch.bfloat16:
        dt = DT_BF16
    elif X.dtype == torch.float32:
        dt = DT_F32
    else:
        raise ValueError("X must be bfloat16 or float32")
    n, d = X.shape
    if ws is None:
        ws = _workspace(workspace_bytes(OP_HESSIAN_TOKENS, 0, d, n), X.device)
    _check(load_library().gptq_hessian_accumulate_tokens(_ptr(H), _ptr(hdiag), _ptr(X), dt, d, n, X.stride(0),
                                                         _ptr(ws), ws.numel(), _stream(stream)))


def _bf16_rows(t, name):
    import torch
    if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1 or t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a 2-D bfloat16 device tensor with unit stride along its rows")


def linear_forward(Y, X, W, stream=None) -> None:
    """Y [n_tok][d_out] (bf16) = bf16(X W^T): X bf16 [n_tok][d_prev] token-major, W bf16 [d_out][d_prev]."""
    for t, n in ((Y, "Y"), (X, "X"), (W, "W")):
        _bf16_rows(t, n)
    n, dp = X.shape
    do = W.shape[0]
    if W.shape[1] != dp or tuple(Y.shape) != (n, do):
        raise ValueError("shapes: X [n][d_prev], W [d_out][d_prev], Y [n][d_out]")
    _check(load_library().gptq_linear_forward(_ptr(Y), Y.stride(0), _ptr(X), X.stride(0), _ptr(W), W.stride(0), n, dp,
                                              do, _stream(stream)))


def calibrate_chunk_tokens(d_in: int) -> int:
    return int(load_library().gptq_calibrate_chunk_tokens(d_in))


def calibrate_hessian(H, X, W, hdiag=None, ws=None, stream=None) -> None:
    """H (fp32 [d_in,d_in], upper) += 2 Y^T Y with Y = bf16(X W^T) made chunk by chunk on the device:
    X bf16 [n_tok][d_prev] (the previous layer's inputs), W bf16 [d_in][d_prev]."""
    _need_cuda(H, hdiag)
    _bf16_rows(X, "X")
    _bf16_rows(W, "W")
    n, dp = X.shape
    di = W.shape[0]
    if W.shape[1] != dp or tuple(H.shape) != (di, di):
        raise ValueError("shapes: X [n][d_prev], W [d_in][d_prev], H [d_in][d_in]")
    if ws is None:
        ws = _workspace(workspace_bytes(OP_CALIBRATE, 0, di, n), X.device)
    _check(load_library().gptq_calibrate_hessian(_ptr(H), _ptr(hdiag), _ptr(X), X.stride(0), _ptr(W), W.stride(0), n,
                                                 dp, di, _ptr(ws), ws.numel(), _stream(stream)))


def prepare_hinv(H, cfg: Config, U, perm=None, info=None, hdiag=None, ws=None, stream=None):
    """U = upper Cholesky factor of the damped (and ordered) inverse Hessian.  Returns the info tensor."""
    import torch
    _need_cuda(H, U, perm, info, hdiag)
    d = H.shape[0]
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=H.device)
    if ws is None:
        ws = _workspace(workspace_bytes(OP_PREPARE, 0, d, 0, cfg), H.device)
    _check(load_library().gptq_prepare_hinv(_ptr(H), _ptr(hdiag), d, ctypes.byref(cfg), _ptr(U), _ptr(perm),
                                            _ptr(info), _ptr(ws), ws.numel(), _stream(stream)))
    return info


def quantize_layer(W, U, cfg: Config, codes, scales, zeros, perm=None, g_idx=None, ws=None, stream=None) -> None:
    """GPTQ column pass (in place on W); writes codes/scales/zeros/g_idx."""
    _need_cuda(W, U, codes, scales, zeros, perm, g_idx)
    d_out, d_in = W.shape
    if ws is None:
        ws = _workspace(workspace_bytes(OP_QUANTIZE, d_out, d_in, 0, cfg), W.device)
    _check(load_library().gptq_quantize_layer(_ptr(W), d_out, d_in, _ptr(U), _ptr(perm), ctypes.byref(cfg),
                                              _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx), _ptr(ws),
                                              ws.numel(), _stream(stream)))


def quantize_layer_noalloc(W, U, cfg: Config, codes, scales, zeros, perm=None, g_idx=None, stream=None) -> None:
    """quantize_layer without a workspace: the library's fixed scratch array (NOALLOC_SCRATCH_BYTES)."""
    _need_cuda(W, U, codes, scales, zeros, perm, g_idx)
    d_out, d_in = W.shape
    _check(load_library().gptq_quantize_layer_noalloc(_ptr(W), d_out, d_in, _ptr(U), _ptr(perm), ctypes.byref(cfg),
                                                      _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                                      _stream(stream)))


def rtn_quantize(W, cfg: Config, codes, scales, zeros, stream=None) -> None:
    _need_cuda(W, codes, scales, zeros)
    d_out, d_in = W.shape
    _check(load_library().gptq_rtn_quantize(_ptr(W), d_out, d_in, ctypes.byref(cfg), _ptr(codes), _ptr(scales),
                                            _ptr(zeros), _stream(stream)))


def layer_loss(W, codes, scales, zeros, H, group_size: int, g_idx=None, out=None, ws=None, stream=None):
    """||W X - W_hat X||^2 through H (device fp64 scalar tensor)."""
    import torch
    _need_cuda(W, codes, scales, zeros, H, g_idx, out)
    d_out, d_in = W.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=W.device)
    if ws is None:
        ws = _workspace(workspace_bytes(OP_LOSS, d_out, d_in), W.device)
    _check(load_library().gptq_layer_loss(_ptr(W), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx), _ptr(H),
                                          d_out, d_in, int(group_size), _ptr(out), _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return out


def channel_stats(X, absmax=None, abssum=None, stream=None):
    """Per input channel of X ([d][n], bf16 or fp32): (max |x| fp32, sum |x| fp64), accumulated."""
    import torch
    if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D device tensor with unit stride along tokens")
    dt = DT_BF16 if X.dtype == torch.bfloat16 else DT_F32
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("X must be bfloat16 or float32")
    d, n = X.shape
    if absmax is None:
        absmax = torch.zeros(d, dtype=torch.float32, device=X.device)
    if abssum is None:
        abssum = torch.zeros(d, dtype=torch.float64, device=X.device)
    _need_cuda(absmax, abssum)
    _check(load_library().gptq_channel_stats(_ptr(X), dt, d, n, X.stride(0), _ptr(absmax), _ptr(abssum),
                                             _stream(stream)))
    return absmax, abssum


def smooth_scales(act_absmax, W, alpha: float = 0.5, s=None, ws=None, stream=None):
    """SmoothQuant scales s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)."""
    import torch
    _need_cuda(act_absmax, W, s)
    d_out, d_in = W.shape
    if s is None:
        s = torch.empty(d_in, dtype=torch.float32, device=W.device)
    if ws is None:
        ws = _workspace(workspace_bytes(OP_SMOOTH, d_out, d_in), W.device)
    _check(load_library().gptq_smooth_scales(_ptr(act_absmax), _ptr(W), d_out, d_in, float(alpha), _ptr(s), _ptr(ws),
                                             ws.numel(), _stream(stream)))
    return s


def awq_search(W, H, act_abssum, n_tok: int, cfg: Config, n_grid: int = 20, ws=None, stream=None):
    """AWQ's grid search; returns device tensors (s [d_in], losses [n_grid] fp64, best [1] int32)."""
    import torch
    _need_cuda(W, H, act_abssum)
    d_out, d_in = W.shape
    s = torch.empty(d_in, dtype=torch.float32, device=W.device)
    losses = torch.empty(n_grid, dtype=torch.float64, device=W.device)
    best = torch.empty(1, dtype=torch.int32, device=W.device)
    if ws is None:
        ws = _workspace(workspace_bytes(OP_AWQ, d_out, d_in, 0, cfg), W.device)
    _check(load_library().gptq_awq_search(_ptr(W), d_out, d_in, _ptr(H), _ptr(act_abssum), int(n_tok), ctypes.byref(cfg),
                                          int(n_grid), _ptr(s), _ptr(losses), _ptr(best), _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return s, losses, best


def scale_layer(s, W=None, H=None, hdiag=None, stream=None) -> None:
    """In place: W <- W diag(s), H <- diag(s)^-1 H diag(s)^-1 (upper), hdiag <- hdiag / s^2."""
    _need_cuda(s, W, H, hdiag)
    d_in = s.shape[0]
    d_out = W.shape[0] if W is not None else 0
    _check(load_library().gptq_scale_layer(_ptr(W), d_out, d_in, _ptr(H), _ptr(hdiag), _ptr(s), _stream(stream)))


def packed_words(d_in: int, bits: int) -> int:
    """32-bit words per packed row."""
    return (d_in * bits + 31) // 32


def pack_codes(codes, bits: int, packed=None, perm=None, stream=None):
    """Codes [d_out][d_in] u8 -> rows of little-endian bit streams (u32 [d_out][words])."""
    import torch
    _need_cuda(codes, packed, perm)
    d_out, d_in = codes.shape
    if packed is None:
        packed = torch.empty(d_out, packed_words(d_in, bits), dtype=torch.int32, device=codes.device)
    _check(load_library().gptq_pack_codes(_ptr(codes), d_out, d_in, int(bits), _ptr(perm), _ptr(packed),
                                          _stream(stream)))
    return packed


def w4a16_gemm(X, packed, scales, zeros, group_size: int, d_out: int, kperm=None, Y=None, ws=None, stream=None):
    """Y = X' W_hat^T with fp16 X [M][d_in] and 4-bit packed weights; Y fp32 [M][d_out]."""
    import torch
    _need_cuda(packed, scales, zeros, kperm, Y)
    if not X.is_cuda:
        raise ValueError("X must be a device tensor")
    if X.dtype != torch.float16:
        raise TypeError("X must be float16")
    M, d_in = X.shape
    if X.stride(1) != 1:  # rows may sit at any pitch (ldx = X.stride(0)); within a row, contiguous
        raise ValueError("X rows must be contiguous")
    if Y is None:
        Y = torch.empty(M, d_out, dtype=torch.float32, device=X.device)
    if ws is None:
        ws = _workspace(workspace_bytes(OP_W4A16, d_out, d_in, M), X.device)
    _check(load_library().gptq_w4a16_gemm(_ptr(X), DT_F16, M, d_in, X.stride(0), _ptr(kperm), _ptr(packed),
                                          _ptr(scales), _ptr(zeros), int(group_size), d_out, _ptr(Y), Y.stride(0),
                                          _ptr(ws), ws.numel(), _stream(stream)))
    return Y


@dataclass
class LayerResult:
    codes: object
    scales: object
    zeros: object
    g_idx: object
    perm: object
    info: object


def n_groups(d_in: int, group_size: int) -> int:
    return d_in // group_size if group_size > 0 else 1


def gptq_layer(W, X, cfg: Config, H=None, hdiag=None):
    """Convenience: all four steps on device tensors (W is overwritten)."""
    import torch
    dev = W.device
    d_out, d_in = W.shape
    if H is None:
        H = torch.zeros(d_in, d_in, dtype=torch.float32, device=dev)
        if cfg.act_order and hdiag is None:
            hdiag = torch.zeros(d_in, dtype=torch.float64, device=dev)
        hessian_accumulate(H, X, hdiag)
    U = torch.empty(d_in, d_in, dtype=torch.float32, device=dev)
    perm = torch.empty(d_in, dtype=torch.int32, device=dev)
    info = prepare_hinv(H, cfg, U, perm, hdiag=hdiag)
    ng = n_groups(d_in, cfg.group_size)
    codes = torch.empty(d_out, d_in, dtype=torch.uint8, device=dev)
    scales = torch.empty(d_out, ng, dtype=torch.float32, device=dev)
    zeros = torch.empty(d_out, ng, dtype=torch.float32, device=dev)
    g_idx = torch.empty(d_in, dtype=torch.int32, device=dev)
    quantize_layer(W, U, cfg, codes, scales, zeros, perm, g_idx)
    return LayerResult(codes, scales, zeros, g_idx, perm, info), H, U
