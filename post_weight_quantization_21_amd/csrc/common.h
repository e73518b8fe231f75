// Internal declarations of the gfx950 GPTQ library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "gptq.h"

namespace gptq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Matrix-core output layout of the 32x32 MFMA family (v_mfma_f32_32x32x*):
// accumulator register r of lane l holds D[row][col] with
//   col = l % 32, row = 8 * (r / 4) + 4 * (l / 32) + (r % 4).
__device__ __forceinline__ int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int mfma32_col(int lane) { return lane & 31; }

// ---------------------------------------------------------------------------
// fp32 matrix-core GEMM:  C = alpha * op(A) op(B) + beta * C   (see gemm_f32.hip)
// ---------------------------------------------------------------------------
enum GemmEpilogue { EPI_STORE = 0, EPI_DOT = 1 };

struct GemmDesc {
    int64_t M = 0, N = 0, K = 0;
    const float *A = nullptr;
    int64_t lda = 0;
    int a_trans = 0;  // 0: A[m][k] = A[m*lda+k];  1: A[m][k] = A[k*lda+m]
    const float *B = nullptr;
    int64_t ldb = 0;
    int b_trans = 0;  // 0: B[k][n] = B[k*ldb+n];  1: B[k][n] = B[n*ldb+k]
    float *C = nullptr;
    int64_t ldc = 0;
    float alpha = 1.0f, beta = 0.0f;
    int upper_only = 0;  // write only C[m][n] with m <= n (skip tiles below the diagonal)
    int a_upper = 0;     // A upper triangular: A[m][k] == 0 for k < m (K range trimmed)
    int b_upper = 0;     // B upper triangular: B[k][n] == 0 for k > n (K range trimmed)
    int batch = 1;       // blockIdx.z; operands advance by the strides below
    int max_wgs = 0;     // > 0: at most this many workgroups, each looping over tiles (leaves CUs to other streams)
    int64_t strideA = 0, strideB = 0, strideC = 0;
    // EPI_DOT: instead of storing, partial[tile] = sum over the tile of
    // (op(A) op(B))[m][n] * Dm[m*ldd+n] in fp64 (one double per workgroup).
    int epilogue = EPI_STORE;
    const float *Dm = nullptr;
    int64_t ldd = 0;
    double *partial = nullptr;
};

constexpr int kGemmTile = 128;
int64_t gemm_num_tiles(const GemmDesc &g);
hipError_t launch_gemm_f32(const GemmDesc &g, hipStream_t s);
// The same product on the bf16 matrix cores through an exact three-term split
// of each fp32 operand (gemm_split.hip): upper_only only for a square C, no
// batch, K a multiple of 32, 16-byte aligned operands, lda and ldb multiples
// of 4, and M (N) a multiple of 4 when A (B) is stored K-major.
bool gemm_split_supported(const GemmDesc &g);
hipError_t launch_gemm_split(const GemmDesc &g, hipStream_t s);

// ---------------------------------------------------------------------------
// Hessian (hessian.hip)
// ---------------------------------------------------------------------------
// Workspace of run_hessian, the same for both layouts.
size_t hessian_ws_bytes(int64_t d_in, int64_t n_tok, gptq_dtype dt);
// token_major: X is [n_tok][ldx] (channels contiguous), else [d_in][ldx].
hipError_t run_hessian(float *H, double *hdiag, const void *X, gptq_dtype dt, int64_t d_in, int64_t n_tok,
                       int64_t ldx, bool token_major, void *ws, hipStream_t s);
// Y[t][o] = bf16(sum_i X[t][i] W[o][i]) on the bf16 matrix cores (hessian.hip).
hipError_t run_linear_forward(uint16_t *Y, int64_t ldy, const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                              int64_t n_tok, int64_t d_prev, int64_t d_out, hipStream_t s);
// Forward of a layer in token chunks, each chunk's outputs accumulated into H.
int64_t calibrate_chunk_tokens(int64_t d_in);
size_t calibrate_ws_bytes(int64_t d_in, int64_t n_tok);
hipError_t run_calibrate(float *H, double *hdiag, const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                         int64_t n_tok, int64_t d_prev, int64_t d_in, void *ws, hipStream_t s);

// ---------------------------------------------------------------------------
// Prepare (prepare.hip)
// ---------------------------------------------------------------------------
size_t prepare_ws_bytes(int64_t d_in);
hipError_t run_prepare(const float *H, const double *hdiag, int64_t d, float damp_rel, int act_order, float *U,
                       int32_t *perm, int32_t *info, void *ws, hipStream_t s);

// ---------------------------------------------------------------------------
// Quantization (quantize.hip)
// ---------------------------------------------------------------------------
size_t quantize_ws_bytes(int64_t d_out, int64_t d_in, const gptq_config &c);
int quantize_supported(const gptq_config &c, int64_t d_in);
hipError_t run_quantize(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                        const gptq_config &c, uint8_t *codes, float *scales, float *zeros, int32_t *g_idx,
                        void *ws, hipStream_t s);
hipError_t run_rtn(const float *W, int64_t d_out, int64_t d_in, const gptq_config &c, uint8_t *codes,
                   float *scales, float *zeros, hipStream_t s);

// ---------------------------------------------------------------------------
// Loss (loss.hip)
// ---------------------------------------------------------------------------
size_t loss_ws_bytes(int64_t d_out, int64_t d_in);
hipError_t run_loss(const float *W, const uint8_t *codes, const float *scales, const float *zeros,
                    const int32_t *g_idx, const float *H, int64_t d_out, int64_t d_in, int32_t group_size,
                    double *loss, void *ws, hipStream_t s);

// ---------------------------------------------------------------------------
// Packed codes and the W4A16 product (w4a16.hip)
// ---------------------------------------------------------------------------
hipError_t run_pack(const uint8_t *codes, int64_t d_out, int64_t d_in, int bits, const int32_t *perm,
                    uint32_t *packed, hipStream_t s);
size_t w4a16_ws_bytes(int64_t M, int64_t d_in, int64_t d_out, int64_t g);
hipError_t run_w4a16(const void *X, int64_t M, int64_t d_in, int64_t ldx, const int32_t *kperm,
                     const uint32_t *packed, const float *scales, const float *zeros, int64_t g, int64_t d_out,
                     float *Y, int64_t ldy, void *ws, hipStream_t s);

// ---------------------------------------------------------------------------
// Per-channel scaling before the pass (prepass.hip)
// ---------------------------------------------------------------------------
hipError_t run_channel_stats(const void *X, gptq_dtype dt, int64_t d_in, int64_t n_tok, int64_t ldx, float *absmax,
                             double *abssum, hipStream_t s);
size_t smooth_ws_bytes(int64_t d_out, int64_t d_in);
hipError_t run_smooth_scales(const float *act_absmax, const float *W, int64_t d_out, int64_t d_in, float alpha,
                             float *s_out, void *ws, hipStream_t s);
hipError_t run_scale_layer(float *W, int64_t d_out, int64_t d_in, float *H, double *hdiag, const float *sv,
                           hipStream_t s);
size_t awq_ws_bytes(int64_t d_out, int64_t d_in, const gptq_config &c);
hipError_t run_awq_search(const float *W, int64_t d_out, int64_t d_in, const float *H, const double *act_abssum,
                          int64_t n_tok, const gptq_config &c, int n_grid, float *s_out, double *loss_out,
                          int32_t *best_out, void *ws, hipStream_t s);

// ---------------------------------------------------------------------------
// Second streams (streams.hip): one per device and purpose, created on first
// use (default priority).  A call holds `mu` over its whole enqueue sequence
// on the side stream, so the shared events are recorded and waited on in one
// host thread's order at a time.
// ---------------------------------------------------------------------------
enum SidePurpose { kSidePrepare = 0, kSidePurposes = 1 };
struct SideStream {
    static constexpr int kEvents = 4;
    hipStream_t st = nullptr, st2 = nullptr;
    hipEvent_t ev[kEvents] = {};
    std::mutex mu;
};
hipError_t side_stream(SidePurpose purpose, SideStream *&out);
// `to` continues once `from` has reached this point.
hipError_t signal_wait(hipEvent_t ev, hipStream_t from, hipStream_t to);

// Optional event timing of kernel groups (gptq_timing_enable / gptq_timing_read).
enum TimedOp { kTimedLazy = 0, kTimedBatch = 1, kTimedLazySplit = 2, kTimedOps = 3 };
void timing_set(bool on);
// Summed milliseconds, launches and work (the `work` of each scope, e.g. flops).
hipError_t timing_read(TimedOp op, double *ms, int64_t *count, double *work);
class TimedScope {
  public:
    TimedScope(TimedOp op, hipStream_t s, double work = 0.0);
    ~TimedScope();
    TimedScope(const TimedScope &) = delete;
    TimedScope &operator=(const TimedScope &) = delete;

  private:
    TimedOp op_;
    hipStream_t s_;
    double work_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace gptq
