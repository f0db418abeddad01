// Shared definitions for the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "ptq.h"

namespace ptq {

// ---------------------------------------------------------------- errors --
// Thread-local message of the last failure (read through ptq_last_error()).
void set_error(const char* fmt, ...);

struct Status {
    int code;
};

#define PTQ_HIP(expr)                                                              \
    do {                                                                           \
        hipError_t _e = (expr);                                                    \
        if (_e != hipSuccess) {                                                    \
            ::ptq::set_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(_e), \
                             __FILE__, __LINE__);                                  \
            return PTQ_EHIP;                                                       \
        }                                                                          \
    } while (0)

#define PTQ_LAUNCH_CHECK()                                                         \
    do {                                                                           \
        hipError_t _e = hipGetLastError();                                         \
        if (_e != hipSuccess) {                                                    \
            ::ptq::set_error("kernel launch failed: %s (%s:%d)", hipGetErrorString(_e), \
                             __FILE__, __LINE__);                                  \
            return PTQ_EHIP;                                                       \
        }                                                                          \
    } while (0)

#define PTQ_TRY(expr)                 \
    do {                              \
        int _s = (expr);              \
        if (_s != PTQ_OK) return _s;  \
    } while (0)

// -------------------------------------------------------------- vectors --
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 round-to-nearest-even (inputs here are finite).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_as_float(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_float<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_float<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_bits_to_float(p[i]);
}

// --------------------------------------------------------- workspace ----
// Bump allocator over the caller's workspace (256-byte aligned slices).
struct Arena {
    char* base;
    size_t size;
    size_t used;
    explicit Arena(void* p, size_t n) : base((char*)p), size(n), used(0) {}
    template <typename T>
    T* take(size_t count) {
        size_t off = (used + 255) & ~(size_t)255;
        used = off + count * sizeof(T);
        return (base && used <= size) ? (T*)(base + off) : nullptr;
    }
    bool ok() const { return used <= size && (used == 0 || base != nullptr); }
};

// Size accounting with the same alignment rule as Arena.
struct Sizer {
    size_t used = 0;
    template <typename T>
    void take(size_t count) {
        size_t off = (used + 255) & ~(size_t)255;
        used = off + count * sizeof(T);
    }
    size_t bytes() const { return (used + 255) & ~(size_t)255; }
};

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ profiling --
// Optional per-kernel timing with hipEvents on the launch stream (see
// ptq_profile_enable in ptq.h). Kernel classes:
enum ProfKernel {
    PROF_XTX_GEMM = 0,      // bf16 MFMA X^T X tiles
    PROF_FACTOR_GEMM = 1,   // fp32 MFMA GEMMs of the Cholesky / inverse recursion
    PROF_FACTOR_BASE = 2,   // diagonal-block factor + inverse kernels
    PROF_BLOCK_LOOP = 3,    // GPTQ in-block column loop
    PROF_TRAIL_GEMM = 4,    // GPTQ trailing fp32 MFMA update
    PROF_AWQ_GEMM = 5,      // AWQ error GEMM
    PROF_INNER_GEMM = 6,    // GPTQ update inside a super-block
    PROF_SPLIT3_GEMM = 7,   // fp32 GEMM as bf16 MFMAs on three-term splits (main loop only)
    PROF_NKERNELS = 8
};
// mfma_flops: the MFMA flops the bracketed launch executes (whole tiles,
// padding included; 0 where not counted), summed by ptq_profile_flops.
void prof_begin(int kernel, hipStream_t st, double mfma_flops = 0.0);
void prof_end(int kernel, hipStream_t st);

// ------------------------------------------------------------ launchers --
// (defined in the .hip files; all enqueue on `st` and return PTQ_* codes)

// K1: H (+)= X^T X (bf16 or fp32 X), full symmetric; d (+)= colsumsq (fp64).
size_t xtx_workspace_bytes(int64_t n, int64_t rows);
int launch_xtx(float* H, double* d, int64_t n, const void* X, int x_dtype, int64_t rows,
               int64_t ldx, void* ws, size_t ws_bytes, hipStream_t st);
// The same within a fixed scratch of scratch_bytes (device memory the caller
// owns): rows go in chunks sized to fit it; EINVAL when not even 64 rows fit.
int launch_xtx_bounded(float* H, double* d, int64_t n, const void* X, int x_dtype, int64_t rows,
                       int64_t ldx, void* scratch, size_t scratch_bytes, hipStream_t st);
// Argument checks of hessian_accumulate (api.cpp); no HIP call.
int check_hessian_args(const char* fn, const float* H, const double* d, int64_t in, const void* X, int x_dtype,
                       int64_t rows, int64_t ldx);
// Rows per chunk of launch_xtx_bounded for a scratch of scratch_bytes (0: none fit).
int64_t xtx_bounded_chunk(int64_t n, size_t scratch_bytes);

// fp32 MFMA GEMM: C = alpha * op(A) op(B) + beta * C, see gemm_f32.hip.
enum GemmLayoutA { A_MK = 0, A_KM = 1 };   // A row-major [M,K] or stored as [K,M]
enum GemmLayoutB { B_KN = 0, B_NK = 1 };   // B row-major [K,N] or stored as [N,K]
enum GemmTri {
    TRI_NONE = 0,
    TRI_A_UPPER = 1,     // A[i][k] == 0 for k < i (skip those k per row tile)
    TRI_B_UPPER_KN = 2,  // B[k][j] == 0 for k > j (B_KN upper triangular)
    TRI_B_UPPER_NK = 3   // stored B[j][k] == 0 for k < j (B_NK holding an upper matrix)
};
struct GemmArgs {
    int64_t M, N, K;
    const float* A; int64_t lda;
    const float* B; int64_t ldb;
    float* C; int64_t ldc;
    float alpha;      // +1 or -1 in this library
    int beta_one;     // 1: C += ..., 0: C = ...
    int layout_a;     // GemmLayoutA
    int layout_b;     // GemmLayoutB
    int tri;          // GemmTri
    int upper_only;   // only output tiles with tile_row <= tile_col (SYRK-style)
};
int launch_gemm_f32(const GemmArgs& a, hipStream_t st);
// Two products in one launch when both take the direct kernel at the same
// tile and ring shape, the first with B stored [N][K] and the second with B
// stored [K][N]; otherwise two launches. Same results as launch_gemm_f32 on
// each.
int launch_gemm_f32_pair(const GemmArgs& a0, const GemmArgs& a1, hipStream_t st);
// The same GEMM on the bf16 MFMA from three-term bf16 splits of both
// operands (gemm_bf16.hip): pa and pb hold gemm_f32_split3_elems(M, K) and
// (N, K) bf16 elements of scratch (pb is unused when B is A's transpose view).
size_t gemm_f32_split3_elems(int64_t rows, int64_t K);
int launch_gemm_f32_split3(const GemmArgs& a, uint16_t* pa, uint16_t* pb, hipStream_t st);
// Two such products in one launch: a0 = A op(A)^T (its planes in pa serve
// both operands) and a1 with the same A (rows, depth, layout) and its own B
// (planes in pb). EINVAL when the products do not fit that pattern.
int launch_gemm_f32_split3_pair(const GemmArgs& a0, const GemmArgs& a1, uint16_t* pa, uint16_t* pb, hipStream_t st);

// Stage 2 helpers (chol.hip)
size_t factor_workspace_bytes(int64_t n);
int run_inverse_factor(const float* H, const double* d, int64_t n, double damp, int act_order,
                       float* U, int32_t* perm, double* lambda_host, void* ws, size_t ws_bytes,
                       hipStream_t st);

// Stage 3 (gptq.hip)
size_t columns_workspace_bytes(int64_t out, int64_t n, int block);
int run_quantize_columns(const void* W, int w_dtype, int64_t out, int64_t n, int64_t ldw,
                         const float* U, const int32_t* perm, int bits, int g, int block,
                         int8_t* codes, float* scales, int8_t* zeros, int32_t* g_idx, double* stats_host,
                         void* ws, size_t ws_bytes, hipStream_t st);

// AWQ scaling composed with GPTQ (awq_gptq.hip)
size_t awq_gptq_workspace_bytes(int64_t out, int64_t n, int block);
int run_awq_gptq(const void* W, int w_dtype, int64_t out, int64_t n, int64_t ldw, const float* H, const double* d,
                 const float* s, int bits, int g, double damp, int act_order, int block, int8_t* codes,
                 float* scales, int32_t* g_idx, int32_t* perm, double* stats, void* ws, size_t ws_bytes,
                 hipStream_t st);

// INT4 storage (pack.hip)
int launch_pack_int4(const int8_t* codes, int64_t out, int64_t in, uint32_t* packed, hipStream_t st);
int launch_dequant_int4(const uint32_t* packed, const float* scales, const int32_t* g_idx, const int8_t* zeros,
                        int64_t out, int64_t in, int g, int out_dtype, void* What, int64_t ldo, hipStream_t st);

// Stage 4 (awq.hip)
size_t awq_ws_bytes(int64_t out, int64_t n, int64_t rows, int n_alpha);
size_t output_error_ws_bytes(int64_t out, int64_t n, int64_t rows, int x_dtype);
int run_output_error(const void* X, int x_dtype, int64_t rows, int64_t ldx, const void* W, int w_dtype, int64_t out,
                     int64_t n, int64_t ldw, const int8_t* codes, const float* scales, const int32_t* g_idx,
                     const int8_t* zeros, const float* s, int g, double* out2, void* ws, size_t ws_bytes,
                     hipStream_t st);
int run_awq(const void* W, int w_dtype, int64_t out, int64_t n, int64_t ldw, const void* X,
            int x_dtype, int64_t rows, int64_t ldx, const float* alphas, int n_alpha, int bits,
            int g, float* alpha_best, double* err_per_alpha, float* s, int8_t* codes,
            float* scales, void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace ptq
