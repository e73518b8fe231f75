"""GPTQ layer-quantization benchmark on one MI355X.

One step = the whole hot path over one synthetic layer with every input
resident in HBM: H = 2 X X^T over all calibration tokens, damping + inverse
factor, and the column pass with lazy batch updates (W restored from a pristine
device copy first).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload up_proj_70b] [--no-cpu-baseline]

The default workload is the largest single-GPU one, up_proj_70b (W 28672 x 8192, X 8192 x 131072 bf16,
4-bit symmetric groups of 128, Hessian column order).  Kernel times for the roofline objects come from HIP
events recorded on the streams the kernels run on: around the Hessian call, and (library timing, see
gptq_timing_enable) around every lazy-update product and batch kernel of the column pass.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GPTQ ms/layer + TFLOP/s (XXᵀ, lazy update) vs MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak (AMD published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix peak (AMD published)
# fp32 products through the exact three-term bf16 split take six bf16 matrix-core
# products each: their fp32-equivalent ceiling is the bf16 dense peak / 6.
PEAK_SPLIT_TFLOPS = PEAK_BF16_TFLOPS / 6


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(workload: str, kind: str):
    """HBM bytes per launch (kind "hessian": one hessian_accumulate call; "lazy": the lazy-update products
    of one layer) from the committed counter runs, if they were taken on this workload with the current
    kernel sources; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    srcs = rec.get("kernel_sources") or [rec["kernel_source"]]
    shas = rec.get("kernel_sources_sha256") or [rec["kernel_source_sha256"]]
    for src, want in zip(srcs, shas):
        with open(os.path.join(ROOT, src), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != want:
                return None
    if rec.get("workload") != workload:
        return None
    return int(rec["traffic_bytes_per_launch"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(lay: dict, cfg_d: dict) -> dict:
    """The oracle as it stands, timed on a bounded sample of the same workload and scaled to one layer:
    H on the first tokens (fp64 X X^T scales linearly in tokens), the full factor, the column pass on the
    first rows (rows are independent given U)."""
    import oracle
    d_out, d_in, n = lay["d_out"], lay["d_in"], lay["n_tok"]
    n_s = min(n, max(4096, int(262144 * (4096 / d_in) ** 2 / 4)))  # about 10 s of fp64 products
    rows = min(d_out, max(128, int(1024 * (4096 / d_in) ** 2)))
    t0 = time.perf_counter()
    H = oracle.hessian(lay["X"][:, :n_s])
    t_h = time.perf_counter() - t0
    Hf = H * (n / n_s)  # stand-in Hessian of the right scale for the factor step
    t0 = time.perf_counter()
    perm = np.arange(d_in)
    if cfg_d["act_order"]:
        perm = oracle.act_order_perm(np.diag(Hf))
        Hf = Hf[np.ix_(perm, perm)]
    U = oracle.inv_chol_upper(oracle.damp(Hf, cfg_d["damp"]))
    t_p = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gptq_pass(lay["W"][:rows][:, perm], U, cfg_d["bits"], cfg_d["sym"], cfg_d["group"])
    t_q = time.perf_counter() - t0
    est_ms = 1e3 * (t_h * n / n_s + t_p + t_q * d_out / rows)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(est_ms, 1), "unit": "ms/layer", "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "sample": (f"H on {n_s} of {n} tokens (x{n / n_s:g}), full {d_in}x{d_in} factor, column pass on "
                       f"{rows} of {d_out} rows (x{d_out / rows:g}); measured {t_h:.2f}+{t_p:.2f}+{t_q:.2f} s")}


def bench_w4a16(args) -> int:
    """The product of M fp16 tokens with the 4-bit packed up_proj_70b layer (28672 x 8192, groups of 128).

    Codes, scales and zeros are seeded synthetic values of the quantizer's
    ranges.  Reported: microseconds per product, the weight stream against HBM
    bandwidth, a dense fp16 product of the dequantized weights for context, and
    the oracle on a sample of rows.
    """
    import numpy as np
    import torch

    import post_weight_quantization_21_amd as gq

    gq.load_library()
    dev = torch.device("cuda:0")
    M, d_out, d_in, g = args.w4a16, 28672, 8192, 128
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(d_out, d_in), dtype=np.uint8)
    scales = rng.uniform(1e-3, 2e-2, size=(d_out, d_in // g)).astype(np.float32)
    zeros = rng.integers(0, 16, size=(d_out, d_in // g)).astype(np.float32)
    X = rng.standard_normal((M, d_in)).astype(np.float16)
    cd, sd, zd, xd = (torch.from_numpy(a).to(dev) for a in (codes, scales, zeros, X))
    packed = gq.pack_codes(cd, 4)
    Y = torch.empty(M, d_out, dtype=torch.float32, device=dev)
    ws = torch.empty(max(gq.workspace_bytes(gq.OP_W4A16, d_out, d_in, M), 1), dtype=torch.uint8, device=dev)
    run = lambda: gq.w4a16_gemm(xd, packed, sd, zd, g, d_out, Y=Y, ws=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    Wd = ((cd.float() - zd.repeat_interleave(g, 1)) * sd.repeat_interleave(g, 1)).half()
    del cd
    for _ in range(2):
        torch.matmul(xd, Wd.t())
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        torch.matmul(xd, Wd.t())
    b.record()
    torch.cuda.synchronize()
    us_dense = a.elapsed_time(b) * 1e3 / args.steps
    nbytes = d_out * d_in // 2 + 2 * 4 * d_out * (d_in // g) + 2 * M * d_in + 4 * M * d_out  # weights, grids, X, Y
    flops = 2 * M * d_out * d_in
    if flops / nbytes > 2500.0 / 8.0:  # past the ridge of fp16 matrix cores (2.5 PFLOP/s) over HBM (8 TB/s)
        achieved = flops / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(achieved / 2500.0, 4), "traffic": None}
    else:
        achieved = nbytes / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(achieved / 8000.0, 4), "traffic": None}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = 2048
        pk = oracle.pack_codes(codes[:rows], 4)
        t0 = time.perf_counter()
        oracle.w4a16_matmul(X, pk, scales[:rows], zeros[:rows], g)
        dt = time.perf_counter() - t0
        cpu = {"value": round(dt * 1e6 * d_out / rows, 1), "unit": "us", "cores": torch.get_num_threads(),
               "kind": "oracle", "sample": f"{rows} of {d_out} weight rows (unpack, dequantize, fp64 matmul), scaled x{d_out // rows}"}
    out = {"metric": "w4a16_product_us", "value": round(us, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None, "dtype": "f16",
           "data": "synthetic", "config": {"workload": "w4a16_up_proj_70b", "tokens": M, "d_out": d_out, "d_in": d_in,
                                           "group": g},
           "dense_fp16_us": round(us_dense, 2),
           "roofline": roof,
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)
    return 0


def bench_tokens(args) -> int:
    """H from token-major activations ([n_tok][d_in] bf16, one row per token, as a layer's inputs
    arrive) on the workload's shape: the matrix-core SYRK reading token-major tiles.  Timed per
    call with X resident; H accumulates across calls."""
    import torch

    import datagen
    import post_weight_quantization_21_amd as gq

    gq.load_library()
    dev = torch.device("cuda:0")
    lay = datagen.make_layer(args.workload)
    d_in, n = lay["d_in"], lay["n_tok"]
    if lay["X"].dtype != np.uint16:
        print(f"bench.py --tokens: the {args.workload} workload has fp32 activations; use a bf16 workload", file=sys.stderr)
        return 2
    Xt = torch.from_numpy(lay["X"].view(np.int16)).to(dev).view(torch.bfloat16).t().contiguous()  # [n][d]
    del lay
    H = torch.zeros(d_in, d_in, dtype=torch.float32, device=dev)
    ws = torch.empty(max(gq.workspace_bytes(gq.OP_HESSIAN_TOKENS, 0, d_in, n), 1), dtype=torch.uint8, device=dev)
    run = lambda: gq.hessian_accumulate_tokens(H, Xt, ws=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = float(d_in) * (d_in + 1) * n  # the SYRK's multiply-adds (upper triangle incl. diagonal), x2
    tf = flops / (ms * 1e-3) / 1e12
    out = {"metric": "hessian_tokens_ms", "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None, "dtype": "bf16->f32",
           "data": "synthetic", "config": {"workload": args.workload + "_token_major", "d_in": d_in, "n_tok": n,
                                           "x_layout": "token-major [n_tok][d_in]"},
           "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "note": "SYRK flops over the whole call (split-K reduce included)"},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)
    return 0


def bench_calib(args) -> int:
    """The calibration pass of one layer on the workload's shape: a synthetic layer before it
    (W_prev [d_in][d_in] bf16, N(0, 1/d_in)) runs forward on token-major inputs X_prev
    ([n_tok][d_in] bf16, the workload's activations) chunk by chunk, each chunk of outputs
    accumulated into H on the device (gptq_calibrate_hessian)."""
    import torch

    import datagen
    import post_weight_quantization_21_amd as gq

    gq.load_library()
    dev = torch.device("cuda:0")
    lay = datagen.make_layer(args.workload)
    d_in, n = lay["d_in"], lay["n_tok"]
    if lay["X"].dtype != np.uint16:
        print(f"bench.py --calib: the {args.workload} workload has fp32 activations; use a bf16 workload", file=sys.stderr)
        return 2
    Xp = torch.from_numpy(lay["X"].view(np.int16)).to(dev).view(torch.bfloat16).t().contiguous()  # [n][d_in]
    del lay
    gen = torch.Generator(device=dev).manual_seed(0)
    Wp = (torch.randn(d_in, d_in, generator=gen, device=dev) * d_in ** -0.5).to(torch.bfloat16)
    H = torch.zeros(d_in, d_in, dtype=torch.float32, device=dev)
    ws = torch.empty(max(gq.workspace_bytes(gq.OP_CALIBRATE, 0, d_in, n), 1), dtype=torch.uint8, device=dev)
    run = lambda: gq.calibrate_hessian(H, Xp, Wp, ws=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    fwd = 2.0 * n * d_in * d_in
    syrk = float(d_in) * (d_in + 1) * n
    tf = (fwd + syrk) / (ms * 1e-3) / 1e12
    out = {"metric": "calibrate_hessian_ms", "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None, "dtype": "bf16->f32",
           "data": "synthetic", "config": {"workload": args.workload + "_calibrate", "d_prev": d_in, "d_in": d_in,
                                           "n_tok": n, "chunk_tokens": gq.calibrate_chunk_tokens(d_in)},
           "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "note": "forward GEMM and SYRK flops over the whole pass"},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)
    return 0


def bench_awq(args) -> int:
    """AWQ's scale search on the workload's layer: per-channel |x| statistics (outside the timed
    region, like H), then 20 alphas of scale, RTN and loss through the scaled H."""
    import torch

    import datagen
    import post_weight_quantization_21_amd as gq

    gq.load_library()
    dev = torch.device("cuda:0")
    lay = datagen.make_layer(args.workload)
    d_out, d_in, n = lay["d_out"], lay["d_in"], lay["n_tok"]
    cfg = gq.config(lay["bits"], lay["sym"], lay["group"], lay["block"], lay["damp"], False)
    Xd = torch.from_numpy(lay["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    _, asum = gq.channel_stats(Xd)
    H = torch.zeros(d_in, d_in, dtype=torch.float32, device=dev)
    gq.hessian_accumulate(H, Xd)
    del Xd
    Wd = torch.from_numpy(lay["W"]).to(dev)
    n_grid = 20
    ws = torch.empty(gq.workspace_bytes(gq.OP_AWQ, d_out, d_in, 0, cfg), dtype=torch.uint8, device=dev)
    run = lambda: gq.awq_search(Wd, H, asum, n, cfg, n_grid, ws=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        s, losses, best = run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    loss_flops = n_grid * 2.0 * d_out * d_in * d_in  # the loss's (W' - Q(W')) H' products, per search
    tf = loss_flops / (ms * 1e-3) / 1e12
    lv = losses.cpu().numpy()
    out = {"metric": "awq_search_ms", "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None, "dtype": "f32",
           "data": "synthetic", "config": {"workload": args.workload + "_awq", "d_out": d_out, "d_in": d_in,
                                           "n_grid": n_grid, "bits": lay["bits"], "group_size": lay["group"]},
           "best_alpha": int(best.cpu()[0]) / n_grid, "loss_rtn": float(lv[0]), "loss_best": float(lv.min()),
           "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": 157.3, "unit": "TFLOP/s",
                        "frac": round(tf / 157.3, 4), "traffic": None,
                        "note": "loss flops over the whole search time (scaling and RTN included): a lower bound"},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="up_proj_70b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--super-cols", type=int, default=0,
                    help="columns per superblock of the two-level lazy update (0: the library default, 1024)")
    ap.add_argument("--w4a16", type=int, default=0, metavar="M",
                    help="instead: time the W4A16 product of M tokens with the packed 28672x8192 layer")
    ap.add_argument("--awq", action="store_true",
                    help="instead: time the AWQ scale search (20 alphas) on the workload's layer")
    ap.add_argument("--tokens", action="store_true",
                    help="instead: time H from the workload's activations laid out token-major")
    ap.add_argument("--calib", action="store_true",
                    help="instead: time a synthetic layer's forward feeding H chunk by chunk")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this benchmark runs GPTQ on one GPU only "
              f"(sharding the layer: an all-reduce of H over token slices, then the column pass split by output rows, is not built).", file=sys.stderr)
        return 2

    if args.w4a16 > 0:
        return bench_w4a16(args)
    if args.awq:
        return bench_awq(args)
    if args.tokens:
        return bench_tokens(args)
    if args.calib:
        return bench_calib(args)

    import torch

    import datagen
    import post_weight_quantization_21_amd as gq

    gq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    lay = datagen.make_layer(args.workload)
    log(f"generated {args.workload}: W {lay['W'].shape} X {lay['X'].shape} {lay['X'].dtype} in {time.perf_counter() - t0:.1f}s")
    d_out, d_in, n = lay["d_out"], lay["d_in"], lay["n_tok"]
    cfg_d = dict(bits=lay["bits"], sym=lay["sym"], group=lay["group"], block=lay["block"], damp=lay["damp"],
                 act_order=lay["act_order"])
    cfg = gq.config(lay["bits"], lay["sym"], lay["group"], lay["block"], lay["damp"], lay["act_order"],
                    super_cols=args.super_cols)

    if lay["X"].dtype == np.uint16:
        X = torch.from_numpy(lay["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        X = torch.from_numpy(lay["X"]).to(dev)
    W0 = torch.from_numpy(lay["W"]).to(dev)
    W = torch.empty_like(W0)
    H = torch.zeros(d_in, d_in, dtype=torch.float32, device=dev)
    hdiag = torch.zeros(d_in, dtype=torch.float64, device=dev) if lay["act_order"] else None
    U = torch.empty(d_in, d_in, dtype=torch.float32, device=dev)
    perm = torch.empty(d_in, dtype=torch.int32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    ng = gq.n_groups(d_in, lay["group"])
    codes = torch.empty(d_out, d_in, dtype=torch.uint8, device=dev)
    scales = torch.empty(d_out, ng, dtype=torch.float32, device=dev)
    zeros = torch.empty(d_out, ng, dtype=torch.float32, device=dev)
    g_idx = torch.empty(d_in, dtype=torch.int32, device=dev)
    ws_h = torch.empty(max(1, gq.workspace_bytes(gq.OP_HESSIAN, 0, d_in, n)), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(gq.workspace_bytes(gq.OP_PREPARE, 0, d_in, 0, cfg), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(gq.workspace_bytes(gq.OP_QUANTIZE, d_out, d_in, 0, cfg), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        H.zero_()
        if hdiag is not None:
            hdiag.zero_()
        if ev:
            ev[0].record(stream)
        gq.hessian_accumulate(H, X, hdiag, ws=ws_h)
        if ev:
            ev[1].record(stream)
        gq.prepare_hinv(H, cfg, U, perm, info, hdiag=hdiag, ws=ws_p)
        if ev:
            ev[2].record(stream)
        W.copy_(W0)
        if ev:
            ev[3].record(stream)
        gq.quantize_layer(W, U, cfg, codes, scales, zeros, perm, g_idx, ws=ws_q)
        if ev:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        log(f"factorization reported info={int(info.item())}")
        return 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    ph = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])  # ms
    t_h, t_p, t_c, t_q = ph.mean(axis=0)
    log(f"phases (ms): hessian {t_h:.3f}  prepare {t_p:.3f}  copy {t_c:.3f}  quantize {t_q:.3f}  step {ms_step:.3f}")

    # Kernel times of the column pass: the same steps again with the library's event timing on
    # (two event records per launch, on the launch's own stream).
    gq.timing_enable(True)
    for op in (gq.TIMED_LAZY, gq.TIMED_LAZY_SPLIT, gq.TIMED_BATCH):
        gq.timing_read(op)
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    f32_ms, f32_n, f32_fl = gq.timing_read(gq.TIMED_LAZY, with_flops=True)
    spl_ms, spl_n, spl_fl = gq.timing_read(gq.TIMED_LAZY_SPLIT, with_flops=True)
    batch_ms, batch_n = gq.timing_read(gq.TIMED_BATCH)
    gq.timing_enable(False)
    f32_ms, spl_ms, batch_ms = f32_ms / args.steps, spl_ms / args.steps, batch_ms / args.steps
    f32_fl, spl_fl = f32_fl / args.steps, spl_fl / args.steps
    lazy_ms, lazy_n = f32_ms + spl_ms, f32_n + spl_n
    log(f"column pass kernels per step: lazy-update products {lazy_ms:.3f} ms ({lazy_n // args.steps} launches: "
        f"{spl_n // args.steps} split-bf16 {spl_ms:.3f} ms, {f32_n // args.steps} fp32 {f32_ms:.3f} ms), "
        f"batch kernels {batch_ms:.3f} ms ({batch_n // args.steps} launches)")

    syrk_flops = float(d_in) * (d_in + 1) * n
    lazy_flops = float(d_out) * d_in * max(0, d_in - lay["block"])
    syrk_tf = syrk_flops / (t_h * 1e-3) / 1e12
    lazy_tf = lazy_flops / (lazy_ms * 1e-3) / 1e12 if lazy_ms > 0 else 0.0
    roof_syrk = {"bound": "mfma", "achieved": round(syrk_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(syrk_tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(args.workload, "hessian"),
                 "kernel": "hessian_accumulate (mma_bf16_kernel<0>: the SYRK, + syrk_reduce_kernel" +
                           (" + diag_rows_kernel)" if lay["act_order"] else ")"),
                 "flops_per_launch": syrk_flops, "ms_per_launch": round(t_h, 3)}
    # Ceiling of the mix: each kind's flops at its own peak (the library counts 2 M N K per product,
    # which sums to the algorithmic d_out d_in (d_in - B)).
    t_peak_ms = (spl_fl / PEAK_SPLIT_TFLOPS + f32_fl / PEAK_F32_TFLOPS) / 1e9
    lazy_peak = (spl_fl + f32_fl) / t_peak_ms / 1e9 if t_peak_ms > 0 else PEAK_F32_TFLOPS

    def kind(fl, ms, peak):
        tf = fl / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
        return {"flops": fl, "ms": round(ms, 3), "achieved": round(tf, 1), "peak": round(peak, 1),
                "frac": round(tf / peak, 4)}

    roof_lazy = {"bound": "mfma", "achieved": round(lazy_tf, 1), "peak": round(lazy_peak, 1), "unit": "TFLOP/s",
                 "frac": round(lazy_tf / lazy_peak, 4), "traffic": measured_traffic(args.workload, "lazy"),
                 "kernel": "the column pass's lazy-update products, all launches of one layer: gemm_split_kernel "
                           "(superblock updates, fp32 operands split into three bf16 terms, six bf16 products each) "
                           "and the fp32 matrix-core GEMM (in-superblock updates)",
                 "peak_basis": "fp32-equivalent ceiling of the mix: split launches at the bf16 dense peak / 6 "
                               f"({PEAK_SPLIT_TFLOPS:.1f}), fp32 launches at {PEAK_F32_TFLOPS}, weighted by their flops",
                 "split_bf16": kind(spl_fl, spl_ms, PEAK_SPLIT_TFLOPS), "f32": kind(f32_fl, f32_ms, PEAK_F32_TFLOPS),
                 "flops_per_launch": lazy_flops, "ms_per_launch": round(lazy_ms, 3),
                 "launches_per_layer": lazy_n // args.steps}
    dominant = roof_lazy if lazy_ms > t_h else roof_syrk
    out = {
        "metric": METRIC,
        "value": round(ms_step, 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->f32 (XX^T), f32 (lazy update: f32 operands as exact bf16 triples)",
        "data": "synthetic",
        "config": {"workload": args.workload, "d_out": d_out, "d_in": d_in, "n_tok": n, "x_dtype": lay["x_dtype"],
                   "bits": lay["bits"], "symmetric": lay["sym"], "group_size": lay["group"],
                   "block_size": lay["block"], "damp_rel": lay["damp"], "act_order": lay["act_order"],
                   "super_cols": args.super_cols or 1024, "parallelism": "none (1 GPU)"},
        "roofline": dominant,
        "rooflines": {"xxt_syrk": roof_syrk, "lazy_update": roof_lazy},
        "phases_ms": {"hessian": round(t_h, 3), "prepare": round(t_p, 3), "restore_w": round(t_c, 3),
                      "quantize": round(t_q, 3), "quantize_batch_kernels": round(batch_ms, 3),
                      "quantize_lazy_products": round(lazy_ms, 3)},
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(lay, cfg_d)
        log(f"cpu baseline took {time.perf_counter() - t0:.1f}s")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
