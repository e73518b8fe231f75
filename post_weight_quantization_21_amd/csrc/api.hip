// C ABI entry points: argument checks, workspace sizing, dispatch.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

namespace {

thread_local char g_last_error[512] = "";

gptq_status fail(gptq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

gptq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return GPTQ_OK;
    return fail(GPTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a = 16) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gptq_status check_cfg(const gptq_config *c, int64_t d_in, const char *fn) {
    if (!c) return fail(GPTQ_ERR_INVALID_ARG, "%s: cfg is NULL", fn);
    if (c->bits < 2 || c->bits > 8) return fail(GPTQ_ERR_INVALID_ARG, "%s: bits=%d outside 2..8", fn, c->bits);
    if (c->group_size < 0 || (c->group_size > 0 && d_in % c->group_size != 0))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: group_size=%d does not divide d_in=%lld", fn, c->group_size, (long long)d_in);
    if (!(c->damp_rel >= 0.0f)) return fail(GPTQ_ERR_INVALID_ARG, "%s: damp_rel must be >= 0", fn);
    if (c->grid != GPTQ_GRID_DYNAMIC && c->grid != GPTQ_GRID_STATIC && c->grid != GPTQ_GRID_TENSOR)
        return fail(GPTQ_ERR_INVALID_ARG, "%s: unknown grid %d", fn, c->grid);
    if (c->super_cols < 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: super_cols must be >= 0", fn);
    if (c->grid == GPTQ_GRID_TENSOR && c->group_size != 0)
        return fail(GPTQ_ERR_INVALID_ARG, "%s: a per-tensor grid needs group_size 0", fn);
    return GPTQ_OK;
}

gptq_status check_quantize(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                           const gptq_config *cfg, uint8_t *codes, float *scales, float *zeros, int32_t *g_idx,
                           const char *fn) {
    if (d_out <= 0 || d_in <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    gptq_status st = check_cfg(cfg, d_in, fn);
    if (st != GPTQ_OK) return st;
    if (!W || !U || !codes || !scales || !zeros) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (cfg->act_order && !perm) return fail(GPTQ_ERR_INVALID_ARG, "%s: act_order needs perm", fn);
    if (!aligned(W) || !aligned(U) || !aligned(scales, 4) || !aligned(zeros, 4) || (perm && !aligned(perm, 4)) ||
        (g_idx && !aligned(g_idx, 4)))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (!gptq::quantize_supported(*cfg, d_in))
        return fail(GPTQ_ERR_UNSUPPORTED, "%s: block_size=%d group_size=%d not supported", fn, cfg->block_size, cfg->group_size);
    if (d_out > ((int64_t)1 << 21)) return fail(GPTQ_ERR_UNSUPPORTED, "%s: d_out above 2^21", fn);  // 64-row tiles on grid y
    return GPTQ_OK;
}

// Scratch memory of gptq_quantize_layer_noalloc: one fixed array per device,
// part of the library's device image (the runtime places it on each device
// the library runs on, for the life of the process).  In host code `scratch`
// names a host-side stand-in: the device copy's address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[GPTQ_NOALLOC_SCRATCH_BYTES];

hipError_t scratch_address(void **out) {
    constexpr int kMaxDevices = 64;
    static void *addr[kMaxDevices] = {};
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *gptq_status_string(gptq_status st) {
    switch (st) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case GPTQ_ERR_WORKSPACE: return "workspace missing or too small";
    case GPTQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *gptq_last_error(void) { return g_last_error; }

gptq_status gptq_timing_enable(int32_t on) {
    gptq::timing_set(on != 0);
    return GPTQ_OK;
}

gptq_status gptq_timing_read(int32_t op, double *ms, int64_t *count, double *flops) {
    const char *fn = "gptq_timing_read";
    if (op < 0 || op >= gptq::kTimedOps) return fail(GPTQ_ERR_INVALID_ARG, "%s: unknown op %d", fn, op);
    if (!ms || !count) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    double w = 0.0;
    const hipError_t e = gptq::timing_read(static_cast<gptq::TimedOp>(op), ms, count, &w);
    if (flops) *flops = w;
    return hip_status(e, fn);
}

gptq_status gptq_workspace_bytes(int op, int64_t d_out, int64_t d_in, int64_t n_tok, const gptq_config *cfg, size_t *out) {
    if (!out) return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: out is NULL");
    if (d_in <= 0 || d_out < 0 || n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: bad sizes");
    switch (op) {
    case GPTQ_OP_HESSIAN:
        *out = gptq::hessian_ws_bytes(d_in, n_tok, GPTQ_DT_BF16);
        return GPTQ_OK;
    case GPTQ_OP_PREPARE:
        *out = gptq::prepare_ws_bytes(d_in);
        return GPTQ_OK;
    case GPTQ_OP_QUANTIZE: {
        if (!cfg) return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: quantize needs cfg");
        if (cfg->block_size <= 0) return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: block_size must be > 0");
        if (cfg->super_cols < 0) return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: super_cols must be >= 0");
        *out = gptq::quantize_ws_bytes(d_out, d_in, *cfg);
        return GPTQ_OK;
    }
    case GPTQ_OP_LOSS:
        *out = gptq::loss_ws_bytes(d_out, d_in);
        return GPTQ_OK;
    case GPTQ_OP_HESSIAN_TOKENS:
        *out = gptq::hessian_ws_bytes(d_in, n_tok, GPTQ_DT_BF16);
        return GPTQ_OK;
    case GPTQ_OP_CALIBRATE:
        *out = gptq::calibrate_ws_bytes(d_in, n_tok);
        return GPTQ_OK;
    case GPTQ_OP_SMOOTH:
        *out = gptq::smooth_ws_bytes(d_out, d_in);
        return GPTQ_OK;
    case GPTQ_OP_AWQ: {
        if (!cfg) return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: the AWQ search needs cfg");
        gptq_status st = check_cfg(cfg, d_in, "gptq_workspace_bytes");
        if (st != GPTQ_OK) return st;
        *out = gptq::awq_ws_bytes(d_out, d_in, *cfg);
        return GPTQ_OK;
    }
    case GPTQ_OP_W4A16:  // the largest plan over the group sizes (the plan depends on g only through 32, 64, 128 | g)
        *out = std::max(gptq::w4a16_ws_bytes(n_tok, d_in, d_out, 32),
                        std::max(gptq::w4a16_ws_bytes(n_tok, d_in, d_out, 64), gptq::w4a16_ws_bytes(n_tok, d_in, d_out, 128)));
        return GPTQ_OK;
    }
    return fail(GPTQ_ERR_INVALID_ARG, "gptq_workspace_bytes: unknown op %d", op);
}

gptq_status gptq_hessian_accumulate(float *H, double *hdiag, const void *X, gptq_dtype x_dtype, int64_t d_in,
                                    int64_t n_tok, int64_t ldx, void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_hessian_accumulate";
    if (d_in <= 0 || n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: d_in must be > 0 and n_tok >= 0", fn);
    if (x_dtype != GPTQ_DT_F32 && x_dtype != GPTQ_DT_BF16) return fail(GPTQ_ERR_INVALID_ARG, "%s: unknown dtype", fn);
    if (ldx < n_tok) return fail(GPTQ_ERR_INVALID_ARG, "%s: ldx < n_tok", fn);
    const int64_t esz = x_dtype == GPTQ_DT_BF16 ? 2 : 4;
    if (!H || (n_tok > 0 && !X)) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(H) || (X && !aligned(X)) || (hdiag && !aligned(hdiag, 8)) || (ldx * esz) % 16 != 0)
        return fail(GPTQ_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned and ldx*elem a multiple of 16", fn);
    if (n_tok == 0) return GPTQ_OK;
    const size_t need = gptq::hessian_ws_bytes(d_in, n_tok, x_dtype);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_hessian(H, hdiag, X, x_dtype, d_in, n_tok, ldx, false, ws, stream), fn);
}

gptq_status gptq_hessian_accumulate_tokens(float *H, double *hdiag, const void *X, gptq_dtype x_dtype, int64_t d_in,
                                           int64_t n_tok, int64_t ldx, void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_hessian_accumulate_tokens";
    if (d_in <= 0 || n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: d_in must be > 0 and n_tok >= 0", fn);
    if (x_dtype != GPTQ_DT_F32 && x_dtype != GPTQ_DT_BF16) return fail(GPTQ_ERR_INVALID_ARG, "%s: unknown dtype", fn);
    if (ldx < d_in) return fail(GPTQ_ERR_INVALID_ARG, "%s: ldx < d_in", fn);
    if (!H || (n_tok > 0 && !X)) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(H) || (hdiag && !aligned(hdiag, 8)))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    // bf16: each lane loads 4 channels of a token as one 8-byte word
    if (x_dtype == GPTQ_DT_BF16 && ((X && !aligned(X, 8)) || ldx % 4 != 0))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: bf16 X must be 8-byte aligned with ldx a multiple of 4", fn);
    if (x_dtype == GPTQ_DT_F32 && X && !aligned(X, 4)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned X", fn);
    if (n_tok == 0) return GPTQ_OK;
    const size_t need = gptq::hessian_ws_bytes(d_in, n_tok, x_dtype);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_hessian(H, hdiag, X, x_dtype, d_in, n_tok, ldx, true, ws, stream), fn);
}

gptq_status gptq_linear_forward(void *Y, int64_t ldy, const void *X, int64_t ldx, const void *W, int64_t ldw,
                                int64_t n_tok, int64_t d_prev, int64_t d_out, hipStream_t stream) {
    const char *fn = "gptq_linear_forward";
    if (n_tok < 0 || d_out < 0 || d_prev <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: bad sizes", fn);
    if (n_tok == 0 || d_out == 0) return GPTQ_OK;
    if (!Y || !X || !W) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (ldx < d_prev || ldw < d_prev || ldy < d_out) return fail(GPTQ_ERR_INVALID_ARG, "%s: leading dimension too small", fn);
    if (!aligned(X) || !aligned(W) || ldx % 8 != 0 || ldw % 8 != 0 || !aligned(Y, 2))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: X and W must be 16-byte aligned with ldx, ldw multiples of 8", fn);
    return hip_status(gptq::run_linear_forward(static_cast<uint16_t *>(Y), ldy, static_cast<const uint16_t *>(X), ldx,
                                               static_cast<const uint16_t *>(W), ldw, n_tok, d_prev, d_out, stream),
                      fn);
}

gptq_status gptq_calibrate_hessian(float *H, double *hdiag, const void *X, int64_t ldx, const void *W, int64_t ldw,
                                   int64_t n_tok, int64_t d_prev, int64_t d_in, void *ws, size_t ws_bytes,
                                   hipStream_t stream) {
    const char *fn = "gptq_calibrate_hessian";
    if (n_tok < 0 || d_in <= 0 || d_prev <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: bad sizes", fn);
    if (n_tok == 0) return GPTQ_OK;
    if (!H || !X || !W) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (ldx < d_prev || ldw < d_prev) return fail(GPTQ_ERR_INVALID_ARG, "%s: leading dimension too small", fn);
    if (!aligned(H) || (hdiag && !aligned(hdiag, 8)) || !aligned(X) || !aligned(W) || ldx % 8 != 0 || ldw % 8 != 0)
        return fail(GPTQ_ERR_INVALID_ARG, "%s: X and W must be 16-byte aligned with ldx, ldw multiples of 8", fn);
    const size_t need = gptq::calibrate_ws_bytes(d_in, n_tok);
    if (!ws || ws_bytes < need || !aligned(ws))
        return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_calibrate(H, hdiag, static_cast<const uint16_t *>(X), ldx,
                                          static_cast<const uint16_t *>(W), ldw, n_tok, d_prev, d_in, ws, stream),
                      fn);
}

int64_t gptq_calibrate_chunk_tokens(int64_t d_in) { return d_in > 0 ? gptq::calibrate_chunk_tokens(d_in) : 0; }

gptq_status gptq_prepare_hinv(const float *H, const double *hdiag, int64_t d_in, const gptq_config *cfg, float *U,
                              int32_t *perm, int32_t *info_dev, void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_prepare_hinv";
    if (d_in <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: d_in must be > 0", fn);
    if (!cfg) return fail(GPTQ_ERR_INVALID_ARG, "%s: cfg is NULL", fn);
    if (!(cfg->damp_rel >= 0.0f)) return fail(GPTQ_ERR_INVALID_ARG, "%s: damp_rel must be >= 0", fn);
    if (!H || !U || !info_dev) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (cfg->act_order && !perm) return fail(GPTQ_ERR_INVALID_ARG, "%s: act_order needs perm", fn);
    if (!aligned(H) || !aligned(U) || (perm && !aligned(perm, 4)) || !aligned(info_dev, 4) || (hdiag && !aligned(hdiag, 8)))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (d_in > (int64_t)1 << 20) return fail(GPTQ_ERR_UNSUPPORTED, "%s: d_in too large", fn);
    const size_t need = gptq::prepare_ws_bytes(d_in);
    if (!ws || ws_bytes < need) return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    if (!aligned(ws)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned workspace", fn);
    return hip_status(gptq::run_prepare(H, hdiag, d_in, cfg->damp_rel, cfg->act_order ? 1 : 0, U, perm, info_dev, ws, stream), fn);
}

gptq_status gptq_quantize_layer(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                                const gptq_config *cfg, uint8_t *codes, float *scales, float *zeros, int32_t *g_idx,
                                void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_quantize_layer";
    gptq_status st = check_quantize(W, d_out, d_in, U, perm, cfg, codes, scales, zeros, g_idx, fn);
    if (st != GPTQ_OK) return st;
    const size_t need = gptq::quantize_ws_bytes(d_out, d_in, *cfg);
    if (!ws || ws_bytes < need) return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    if (need > 0 && !aligned(ws)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned workspace", fn);
    return hip_status(gptq::run_quantize(W, d_out, d_in, U, perm, *cfg, codes, scales, zeros, g_idx, ws, stream), fn);
}

gptq_status gptq_quantize_layer_noalloc(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                                        const gptq_config *cfg, uint8_t *codes, float *scales, float *zeros,
                                        int32_t *g_idx, hipStream_t stream) {
    const char *fn = "gptq_quantize_layer_noalloc";
    gptq_status st = check_quantize(W, d_out, d_in, U, perm, cfg, codes, scales, zeros, g_idx, fn);
    if (st != GPTQ_OK) return st;
    const size_t need = gptq::quantize_ws_bytes(d_out, d_in, *cfg);
    if (need > GPTQ_NOALLOC_SCRATCH_BYTES)
        return fail(GPTQ_ERR_WORKSPACE, "%s: this layer needs %zu scratch bytes, above the fixed %zu of the entry point",
                    fn, need, (size_t)GPTQ_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    st = hip_status(scratch_address(&ws), fn);
    if (st != GPTQ_OK) return st;
    return hip_status(gptq::run_quantize(W, d_out, d_in, U, perm, *cfg, codes, scales, zeros, g_idx, ws, stream), fn);
}

gptq_status gptq_rtn_quantize(const float *W, int64_t d_out, int64_t d_in, const gptq_config *cfg, uint8_t *codes,
                              float *scales, float *zeros, hipStream_t stream) {
    const char *fn = "gptq_rtn_quantize";
    if (d_out <= 0 || d_in <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    gptq_status st = check_cfg(cfg, d_in, fn);
    if (st != GPTQ_OK) return st;
    if (!W || !codes || !scales || !zeros) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(W, 4) || !aligned(scales, 4) || !aligned(zeros, 4)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return hip_status(gptq::run_rtn(W, d_out, d_in, *cfg, codes, scales, zeros, stream), fn);
}

gptq_status gptq_layer_loss(const float *W, const uint8_t *codes, const float *scales, const float *zeros,
                            const int32_t *g_idx, const float *H, int64_t d_out, int64_t d_in, int32_t group_size,
                            double *loss_dev, void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_layer_loss";
    if (d_out <= 0 || d_in <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    if (group_size < 0 || (group_size > 0 && d_in % group_size != 0))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: group_size does not divide d_in", fn);
    if (!W || !codes || !scales || !zeros || !H || !loss_dev) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(W, 4) || !aligned(H, 4) || !aligned(loss_dev, 8)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    const size_t need = gptq::loss_ws_bytes(d_out, d_in);
    if (!ws || ws_bytes < need) return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_loss(W, codes, scales, zeros, g_idx, H, d_out, d_in, group_size, loss_dev, ws, stream), fn);
}

gptq_status gptq_channel_stats(const void *X, gptq_dtype x_dtype, int64_t d_in, int64_t n_tok, int64_t ldx, float *absmax,
                               double *abssum, hipStream_t stream) {
    const char *fn = "gptq_channel_stats";
    if (d_in <= 0 || n_tok < 0 || ldx < n_tok) return fail(GPTQ_ERR_INVALID_ARG, "%s: bad sizes", fn);
    if (x_dtype != GPTQ_DT_F32 && x_dtype != GPTQ_DT_BF16) return fail(GPTQ_ERR_INVALID_ARG, "%s: unknown dtype", fn);
    if ((n_tok > 0 && !X) || !absmax || !abssum) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if ((X && !aligned(X, 4)) || !aligned(absmax, 4) || !aligned(abssum, 8)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return hip_status(gptq::run_channel_stats(X, x_dtype, d_in, n_tok, ldx, absmax, abssum, stream), fn);
}

gptq_status gptq_smooth_scales(const float *act_absmax, const float *W, int64_t d_out, int64_t d_in, float alpha, float *s,
                               void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_smooth_scales";
    if (d_out <= 0 || d_in <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(GPTQ_ERR_INVALID_ARG, "%s: alpha outside [0, 1]", fn);
    if (!act_absmax || !W || !s) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(act_absmax, 4) || !aligned(W, 4) || !aligned(s, 4)) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    const size_t need = gptq::smooth_ws_bytes(d_out, d_in);
    if (!ws || ws_bytes < need) return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_smooth_scales(act_absmax, W, d_out, d_in, alpha, s, ws, stream), fn);
}

gptq_status gptq_awq_search(const float *W, int64_t d_out, int64_t d_in, const float *H, const double *act_abssum,
                            int64_t n_tok, const gptq_config *cfg, int32_t n_grid, float *s, double *losses,
                            int32_t *best, void *ws, size_t ws_bytes, hipStream_t stream) {
    const char *fn = "gptq_awq_search";
    if (d_out <= 0 || d_in <= 0 || n_tok <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    gptq_status st = check_cfg(cfg, d_in, fn);
    if (st != GPTQ_OK) return st;
    if (n_grid < 1 || n_grid > 64) return fail(GPTQ_ERR_INVALID_ARG, "%s: n_grid outside 1..64", fn);
    if (!W || !H || !act_abssum || !s || !losses || !best) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(W, 4) || !aligned(H, 4) || !aligned(act_abssum, 8) || !aligned(s, 4) || !aligned(losses, 8) || !aligned(best, 4))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    const size_t need = gptq::awq_ws_bytes(d_out, d_in, *cfg);
    if (!ws || ws_bytes < need) return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_awq_search(W, d_out, d_in, H, act_abssum, n_tok, *cfg, n_grid, s, losses, best, ws, stream), fn);
}

gptq_status gptq_scale_layer(float *W, int64_t d_out, int64_t d_in, float *H, double *hdiag, const float *s,
                             hipStream_t stream) {
    const char *fn = "gptq_scale_layer";
    if (d_in <= 0 || (W && d_out <= 0)) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    if (!s) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if ((W && !aligned(W, 4)) || (H && !aligned(H, 4)) || (hdiag && !aligned(hdiag, 8)) || !aligned(s, 4))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return hip_status(gptq::run_scale_layer(W, d_out, d_in, H, hdiag, s, stream), fn);
}

gptq_status gptq_pack_codes(const uint8_t *codes, int64_t d_out, int64_t d_in, int32_t bits, const int32_t *perm,
                            uint32_t *packed, hipStream_t stream) {
    const char *fn = "gptq_pack_codes";
    if (d_out <= 0 || d_in <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    if (bits < 2 || bits > 8) return fail(GPTQ_ERR_INVALID_ARG, "%s: bits=%d outside 2..8", fn, bits);
    if (!codes || !packed) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(packed, 4) || (perm && !aligned(perm, 4))) return fail(GPTQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    return hip_status(gptq::run_pack(codes, d_out, d_in, bits, perm, packed, stream), fn);
}

gptq_status gptq_w4a16_gemm(const void *X, gptq_dtype x_dtype, int64_t M, int64_t d_in, int64_t ldx,
                            const int32_t *kperm, const uint32_t *packed, const float *scales, const float *zeros,
                            int32_t group_size, int64_t d_out, float *Y, int64_t ldy, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
    const char *fn = "gptq_w4a16_gemm";
    if (M <= 0 || d_in <= 0 || d_out <= 0) return fail(GPTQ_ERR_INVALID_ARG, "%s: sizes must be > 0", fn);
    if (x_dtype != GPTQ_DT_F16) return fail(GPTQ_ERR_UNSUPPORTED, "%s: activations must be fp16", fn);
    if (group_size < 0 || (group_size > 0 && d_in % group_size != 0))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: group_size does not divide d_in", fn);
    const int64_t g = group_size > 0 ? group_size : d_in;
    if (g % 32 != 0) return fail(GPTQ_ERR_UNSUPPORTED, "%s: group_size (or d_in when 0) must be a multiple of 32", fn);
    if (!X || !packed || !scales || !zeros || !Y) return fail(GPTQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (ldx < d_in || ldy < d_out) return fail(GPTQ_ERR_INVALID_ARG, "%s: ldx < d_in or ldy < d_out", fn);
    if (!aligned(X) || ldx % 8 != 0 || !aligned(packed) || !aligned(scales, 4) || !aligned(zeros, 4) || !aligned(Y, 4) ||
        (kperm && !aligned(kperm, 4)))
        return fail(GPTQ_ERR_INVALID_ARG, "%s: X and packed must be 16-byte aligned, ldx a multiple of 8; other pointers 4-byte aligned", fn);
    const size_t need = gptq::w4a16_ws_bytes(M, d_in, d_out, g);
    if (!ws || ws_bytes < need) return fail(GPTQ_ERR_WORKSPACE, "%s: need %zu workspace bytes, got %zu", fn, need, ws ? ws_bytes : (size_t)0);
    return hip_status(gptq::run_w4a16(X, M, d_in, ldx, kperm, packed, scales, zeros, g, d_out, Y, ldy, ws, stream), fn);
}

}  // extern "C"
