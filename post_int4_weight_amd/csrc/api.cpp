// C ABI of libptq.so (declared in include/ptq.h): argument validation and
// stage orchestration. Every argument is checked before the first HIP call;
// a bad argument returns PTQ_EINVAL with a thread-local message.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace ptq {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

static int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool dtype_ok(int t) { return t == PTQ_BF16 || t == PTQ_F32; }
static int64_t elems16(int dtype) { return dtype == PTQ_BF16 ? 8 : 4; }  // elements per 16 bytes

static int check_gptq_common(int64_t out, int64_t in, int bits, int g, int block, const char* fn) {
    if (out < 0) return fail(PTQ_EINVAL, "%s: out = %lld < 0", fn, (long long)out);
    if (in < 1) return fail(PTQ_EINVAL, "%s: in = %lld < 1", fn, (long long)in);
    if (in % 8) return fail(PTQ_EINVAL, "%s: in = %lld must be a multiple of 8", fn, (long long)in);
    if (bits < 2 || bits > 8) return fail(PTQ_EINVAL, "%s: bits = %d outside [2, 8]", fn, bits);
    if (block != 32 && block != 64 && block != 128)
        return fail(PTQ_EINVAL, "%s: block_size = %d not in {32, 64, 128}", fn, block);
    if (g < 1) return fail(PTQ_EINVAL, "%s: group_size = %d < 1", fn, g);
    const bool wide = (g % block == 0);
    const bool narrow = (block % g == 0) && (g % 8 == 0);
    if (!wide && !narrow)
        return fail(PTQ_EINVAL,
                    "%s: group_size %d and block_size %d: need group %% block == 0, or block %% group == 0 "
                    "with group a multiple of 8",
                    fn, g, block);
    if ((int64_t)out * in > ((int64_t)1 << 40)) return fail(PTQ_EINVAL, "%s: layer too large", fn);
    return PTQ_OK;
}

// ------------------------------------------------------------ profiling --
// Event pairs recorded around launches of the selected kernel classes. The
// pool grows on demand and is reused across enable() calls; reading
// synchronises on the recorded events only.
struct ProfRec {
    hipEvent_t a, b;
    int kernel;
    double flops;   // MFMA flops the launch executes (0: not counted)
};
static std::mutex g_prof_mu;
static std::vector<ProfRec> g_prof_pool;
static size_t g_prof_used = 0;
static unsigned g_prof_mask = 0;
static int g_prof_open[PROF_NKERNELS];

void prof_begin(int kernel, hipStream_t st, double mfma_flops) {
    if (!(g_prof_mask & (1u << kernel))) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_used == g_prof_pool.size()) {
        ProfRec r{};
        if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
        g_prof_pool.push_back(r);
    }
    ProfRec& r = g_prof_pool[g_prof_used];
    r.kernel = kernel;
    r.flops = mfma_flops;
    if (hipEventRecord(r.a, st) != hipSuccess) return;
    g_prof_open[kernel] = (int)g_prof_used;
    ++g_prof_used;
}

void prof_end(int kernel, hipStream_t st) {
    if (!(g_prof_mask & (1u << kernel))) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    const int i = g_prof_open[kernel];
    if (i >= 0 && (size_t)i < g_prof_used) (void)hipEventRecord(g_prof_pool[i].b, st);
    g_prof_open[kernel] = -1;
}

}  // namespace ptq

using namespace ptq;

extern "C" {

const char* ptq_last_error(void) { return g_err; }

const char* ptq_status_string(int s) {
    switch (s) {
        case PTQ_OK: return "PTQ_OK";
        case PTQ_EINVAL: return "PTQ_EINVAL";
        case PTQ_ENOTPD: return "PTQ_ENOTPD";
        case PTQ_ENONFINITE: return "PTQ_ENONFINITE";
        case PTQ_EWORKSPACE: return "PTQ_EWORKSPACE";
        case PTQ_EHIP: return "PTQ_EHIP";
        default: return "PTQ_UNKNOWN";
    }
}

int ptq_abi_version(void) { return 1; }

int ptq_profile_enable(unsigned kernel_mask) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_mask = kernel_mask & ((1u << PROF_NKERNELS) - 1);
    g_prof_used = 0;
    for (int k = 0; k < PROF_NKERNELS; ++k) g_prof_open[k] = -1;
    return PTQ_OK;
}

int ptq_profile_read(int kernel, double* total_ms, int64_t* launches) {
    if (kernel < 0 || kernel >= PROF_NKERNELS || !total_ms || !launches)
        return fail(PTQ_EINVAL, "ptq_profile_read: bad arguments");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double tot = 0.0;
    int64_t cnt = 0;
    for (size_t i = 0; i < g_prof_used; ++i) {
        const ProfRec& r = g_prof_pool[i];
        if (r.kernel != kernel) continue;
        PTQ_HIP(hipEventSynchronize(r.b));
        float ms = 0.f;
        PTQ_HIP(hipEventElapsedTime(&ms, r.a, r.b));
        tot += ms;
        ++cnt;
    }
    *total_ms = tot;
    *launches = cnt;
    return PTQ_OK;
}

int ptq_profile_flops(int kernel, double* mfma_flops) {
    if (kernel < 0 || kernel >= PROF_NKERNELS || !mfma_flops) return fail(PTQ_EINVAL, "ptq_profile_flops: bad arguments");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double tot = 0.0;
    for (size_t i = 0; i < g_prof_used; ++i)
        if (g_prof_pool[i].kernel == kernel) tot += g_prof_pool[i].flops;
    *mfma_flops = tot;
    return PTQ_OK;
}

size_t hessian_workspace_bytes(int64_t in, int64_t rows) {
    if (in < 1 || rows < 0) return 0;
    return xtx_workspace_bytes(in, rows);
}

}  // extern "C"

namespace ptq {
int check_hessian_args(const char* fn, const float* H, const double* d, int64_t in, const void* X, int x_dtype,
                       int64_t rows, int64_t ldx) {
    if (in < 1) return fail(PTQ_EINVAL, "%s: in = %lld < 1", fn, (long long)in);
    if (in % 4) return fail(PTQ_EINVAL, "%s: in = %lld must be a multiple of 4 (16-byte rows of H)", fn, (long long)in);
    if (rows < 0) return fail(PTQ_EINVAL, "%s: rows = %lld < 0", fn, (long long)rows);
    if (!dtype_ok(x_dtype)) return fail(PTQ_EINVAL, "%s: x_dtype = %d", fn, x_dtype);
    if (ldx < in) return fail(PTQ_EINVAL, "%s: ldx = %lld < in", fn, (long long)ldx);
    if (ldx % elems16(x_dtype)) return fail(PTQ_EINVAL, "%s: ldx must keep rows 16-byte aligned", fn);
    if (!H) return fail(PTQ_EINVAL, "%s: H is NULL", fn);
    if (rows > 0 && !X) return fail(PTQ_EINVAL, "%s: X is NULL", fn);
    if (!aligned16(H) || (X && !aligned16(X)) || (d && ((uintptr_t)d & 7u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    return PTQ_OK;
}
}  // namespace ptq

extern "C" {

int hessian_accumulate(float* H, double* d, int64_t in, const void* X, int x_dtype, int64_t rows, int64_t ldx,
                       void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "hessian_accumulate";
    PTQ_TRY(check_hessian_args(fn, H, d, in, X, x_dtype, rows, ldx));
    if (workspace_bytes > 0 && !workspace) return fail(PTQ_EINVAL, "%s: workspace NULL with nonzero size", fn);
    if (workspace && !aligned16(workspace)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);
    if (rows == 0) return PTQ_OK;
    return launch_xtx(H, d, in, X, x_dtype, rows, ldx, workspace, workspace_bytes, (hipStream_t)stream);
}

size_t gptq_factor_workspace_bytes(int64_t in) { return in < 1 ? 0 : factor_workspace_bytes(in); }

static int check_factor(const float* H, const double* d, int64_t in, double damp, int act_order, float* U,
                        int32_t* perm, void* ws, size_t ws_bytes, const char* fn) {
    if (in < 1) return fail(PTQ_EINVAL, "%s: in = %lld < 1", fn, (long long)in);
    if (in % 4) return fail(PTQ_EINVAL, "%s: in = %lld must be a multiple of 4", fn, (long long)in);
    if (!(damp >= 0.0) || !std::isfinite(damp)) return fail(PTQ_EINVAL, "%s: damp = %g", fn, damp);
    if (act_order != 0 && act_order != 1) return fail(PTQ_EINVAL, "%s: act_order = %d", fn, act_order);
    if (!H || !U) return fail(PTQ_EINVAL, "%s: H or U is NULL", fn);
    if (!aligned16(H) || !aligned16(U) || (d && ((uintptr_t)d & 7u)) || (perm && ((uintptr_t)perm & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    if (!ws || ws_bytes < factor_workspace_bytes(in))
        return fail(PTQ_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, factor_workspace_bytes(in));
    if (!aligned16(ws)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);
    return PTQ_OK;
}

int gptq_inverse_factor(const float* H, const double* d, int64_t in, double damp, int act_order, float* U,
                        int32_t* perm, double* lambda_out, void* workspace, size_t workspace_bytes, void* stream) {
    PTQ_TRY(check_factor(H, d, in, damp, act_order, U, perm, workspace, workspace_bytes, "gptq_inverse_factor"));
    if (act_order && !perm) return fail(PTQ_EINVAL, "gptq_inverse_factor: act_order needs perm");
    return run_inverse_factor(H, d, in, damp, act_order, U, perm, lambda_out, workspace, workspace_bytes,
                              (hipStream_t)stream);
}

size_t gptq_columns_workspace_bytes(int64_t out, int64_t in, int block_size) {
    if (out < 0 || in < 1 || (block_size != 32 && block_size != 64 && block_size != 128)) return 0;
    return columns_workspace_bytes(out, in, block_size);
}

static int check_columns(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw, const float* U, int bits,
                         int g, int block, int8_t* codes, float* scales, int32_t* g_idx, void* ws, size_t ws_bytes,
                         const char* fn) {
    PTQ_TRY(check_gptq_common(out, in, bits, g, block, fn));
    if (!dtype_ok(w_dtype)) return fail(PTQ_EINVAL, "%s: w_dtype = %d", fn, w_dtype);
    if (ldw < in || ldw % elems16(w_dtype)) return fail(PTQ_EINVAL, "%s: bad ldw = %lld", fn, (long long)ldw);
    if (out > 0 && (!W || !codes || !scales)) return fail(PTQ_EINVAL, "%s: W, codes or scales is NULL", fn);
    if (!U) return fail(PTQ_EINVAL, "%s: U is NULL", fn);
    if ((W && !aligned16(W)) || !aligned16(U) || (codes && !aligned16(codes)) || (scales && ((uintptr_t)scales & 3u)) ||
        (g_idx && ((uintptr_t)g_idx & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    if (!ws || ws_bytes < columns_workspace_bytes(out, in, block))
        return fail(PTQ_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes,
                    columns_workspace_bytes(out, in, block));
    if (!aligned16(ws)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);
    return PTQ_OK;
}

int gptq_quantize_columns(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw, const float* U,
                          const int32_t* perm, int bits, int group_size, int block_size, int8_t* codes, float* scales,
                          int32_t* g_idx, double* stats, void* workspace, size_t workspace_bytes, void* stream) {
    PTQ_TRY(check_columns(W, w_dtype, out, in, ldw, U, bits, group_size, block_size, codes, scales, g_idx, workspace,
                          workspace_bytes, "gptq_quantize_columns"));
    if (perm && ((uintptr_t)perm & 3u)) return fail(PTQ_EINVAL, "gptq_quantize_columns: misaligned perm");
    return run_quantize_columns(W, w_dtype, out, in, ldw, U, perm, bits, group_size, block_size, codes, scales, nullptr,
                                g_idx, stats, workspace, workspace_bytes, (hipStream_t)stream);
}

size_t gptq_workspace_bytes(int64_t out, int64_t in, int block_size) {
    if (out < 0 || in < 1 || (block_size != 32 && block_size != 64 && block_size != 128)) return 0;
    Sizer z;
    z.take<char>(factor_workspace_bytes(in));
    z.take<float>((size_t)in * in);     // U
    z.take<int32_t>((size_t)in);        // perm (when the caller passes none)
    z.take<char>(columns_workspace_bytes(out, in, block_size));
    return z.bytes();
}

}  // extern "C"

// Stages 2 + 3; zeros == nullptr: symmetric grid, else zero-point groups.
static int quantize_layer(const char* fn, const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                          const float* H, const double* d, int bits, int group_size, double damp, int act_order,
                          int block_size, int8_t* codes, float* scales, int8_t* zeros, int32_t* g_idx, int32_t* perm,
                          double* stats, void* workspace, size_t workspace_bytes, void* stream) {
    PTQ_TRY(check_gptq_common(out, in, bits, group_size, block_size, fn));
    if (!dtype_ok(w_dtype)) return fail(PTQ_EINVAL, "%s: w_dtype = %d", fn, w_dtype);
    if (ldw < in || ldw % elems16(w_dtype)) return fail(PTQ_EINVAL, "%s: bad ldw", fn);
    if (!(damp >= 0.0) || !std::isfinite(damp)) return fail(PTQ_EINVAL, "%s: damp = %g", fn, damp);
    if (act_order != 0 && act_order != 1) return fail(PTQ_EINVAL, "%s: act_order = %d", fn, act_order);
    if (!H) return fail(PTQ_EINVAL, "%s: H is NULL", fn);
    if (out > 0 && (!W || !codes || !scales)) return fail(PTQ_EINVAL, "%s: W, codes or scales is NULL", fn);
    if (!aligned16(H) || (W && !aligned16(W)) || (codes && !aligned16(codes)) || (d && ((uintptr_t)d & 7u)) ||
        (scales && ((uintptr_t)scales & 3u)) || (g_idx && ((uintptr_t)g_idx & 3u)) || (perm && ((uintptr_t)perm & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    const size_t need = gptq_workspace_bytes(out, in, block_size);
    if (!workspace || workspace_bytes < need)
        return fail(PTQ_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);

    hipStream_t st = (hipStream_t)stream;
    Arena ar(workspace, workspace_bytes);
    void* fws = ar.take<char>(factor_workspace_bytes(in));
    float* U = ar.take<float>((size_t)in * in);
    int32_t* ptmp = ar.take<int32_t>((size_t)in);
    void* cws = ar.take<char>(columns_workspace_bytes(out, in, block_size));
    int32_t* p = perm ? perm : ptmp;
    double lam = 0.0;
    PTQ_TRY(run_inverse_factor(H, d, in, damp, act_order, U, p, &lam, fws, factor_workspace_bytes(in), st));
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    PTQ_TRY(run_quantize_columns(W, w_dtype, out, in, ldw, U, act_order ? p : nullptr, bits, group_size, block_size,
                                 codes, scales, zeros, g_idx, s, cws, columns_workspace_bytes(out, in, block_size),
                                 st));
    if (stats) {
        stats[0] = s[0];
        stats[1] = lam;
        stats[2] = s[2];
        stats[3] = s[0] - lam * s[2];
    }
    return PTQ_OK;
}

extern "C" {

int gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw, const float* H,
                        const double* d, int bits, int group_size, double damp, int act_order, int block_size,
                        int8_t* codes, float* scales, int32_t* g_idx, int32_t* perm, double* stats, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return quantize_layer("gptq_quantize_layer", W, w_dtype, out, in, ldw, H, d, bits, group_size, damp, act_order,
                          block_size, codes, scales, nullptr, g_idx, perm, stats, workspace, workspace_bytes, stream);
}

int gptq_quantize_layer_zp(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw, const float* H,
                           const double* d, int bits, int group_size, double damp, int act_order, int block_size,
                           int8_t* codes, float* scales, int8_t* zeros, int32_t* g_idx, int32_t* perm, double* stats,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "gptq_quantize_layer_zp";
    if (bits < 2 || bits > 7) return fail(PTQ_EINVAL, "%s: bits = %d outside [2, 7] (codes are int8)", fn, bits);
    if (out > 0 && !zeros) return fail(PTQ_EINVAL, "%s: zeros is NULL", fn);
    return quantize_layer(fn, W, w_dtype, out, in, ldw, H, d, bits, group_size, damp, act_order, block_size, codes,
                          scales, zeros, g_idx, perm, stats, workspace, workspace_bytes, stream);
}

int ptq_test_gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int layout_a, const float* B,
                      int64_t ldb, int layout_b, float* C, int64_t ldc, float alpha, int beta_one, int tri,
                      int upper_only, void* stream) {
    if (M < 0 || N < 0 || K < 0 || !A || !B || !C || (layout_a != 0 && layout_a != 1) ||
        (layout_b != 0 && layout_b != 1) || tri < 0 || tri > 3 || lda % 4 || ldb % 4 || !aligned16(A) ||
        !aligned16(B))
        return fail(PTQ_EINVAL, "ptq_test_gemm_f32: bad arguments");
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layout_a = layout_a;
    g.B = B; g.ldb = ldb; g.layout_b = layout_b;
    g.C = C; g.ldc = ldc;
    g.alpha = alpha; g.beta_one = beta_one; g.tri = tri; g.upper_only = upper_only;
    return launch_gemm_f32(g, (hipStream_t)stream);
}

int ptq_test_gemm_f32_pair(int64_t M0, int64_t N0, int64_t K0, const float* A0, int64_t lda0, const float* B0,
                           int64_t ldb0, float* C0, int64_t ldc0, float alpha0, int beta_one0, int tri0,
                           int upper_only0, int64_t M1, int64_t N1, int64_t K1, const float* A1, int64_t lda1,
                           const float* B1, int64_t ldb1, float* C1, int64_t ldc1, float alpha1, int beta_one1,
                           int tri1, int upper_only1, void* stream) {
    if (M0 < 0 || N0 < 0 || K0 < 0 || M1 < 0 || N1 < 0 || K1 < 0 || !A0 || !B0 || !C0 || !A1 || !B1 || !C1 ||
        tri0 < 0 || tri0 > 3 || tri1 < 0 || tri1 > 3 || K0 % 4 || K1 % 4 || lda0 % 4 || ldb0 % 4 || lda1 % 4 ||
        ldb1 % 4 || !aligned16(A0) || !aligned16(B0) || !aligned16(A1) || !aligned16(B1))
        return fail(PTQ_EINVAL, "ptq_test_gemm_f32_pair: bad arguments");
    GemmArgs g0{}, g1{};
    g0.M = M0; g0.N = N0; g0.K = K0;
    g0.A = A0; g0.lda = lda0; g0.layout_a = A_MK;
    g0.B = B0; g0.ldb = ldb0; g0.layout_b = B_NK;
    g0.C = C0; g0.ldc = ldc0;
    g0.alpha = alpha0; g0.beta_one = beta_one0; g0.tri = tri0; g0.upper_only = upper_only0;
    g1.M = M1; g1.N = N1; g1.K = K1;
    g1.A = A1; g1.lda = lda1; g1.layout_a = A_MK;
    g1.B = B1; g1.ldb = ldb1; g1.layout_b = B_KN;
    g1.C = C1; g1.ldc = ldc1;
    g1.alpha = alpha1; g1.beta_one = beta_one1; g1.tri = tri1; g1.upper_only = upper_only1;
    return launch_gemm_f32_pair(g0, g1, (hipStream_t)stream);
}

size_t ptq_test_gemm_f32_split3_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    Sizer z;
    z.take<uint16_t>(gemm_f32_split3_elems(M, K));
    z.take<uint16_t>(gemm_f32_split3_elems(N, K));
    return z.bytes();
}

int ptq_test_gemm_f32_split3(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int layout_a,
                             const float* B, int64_t ldb, int layout_b, float* C, int64_t ldc, float alpha,
                             int beta_one, int tri, int upper_only, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (M < 0 || N < 0 || K < 0 || !A || !B || !C || (layout_a != 0 && layout_a != 1) ||
        (layout_b != 0 && layout_b != 1) || tri < 0 || tri > 3)
        return fail(PTQ_EINVAL, "ptq_test_gemm_f32_split3: bad arguments");
    const size_t need = ptq_test_gemm_f32_split3_workspace_bytes(M, N, K);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(PTQ_EWORKSPACE, "ptq_test_gemm_f32_split3: workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    Arena ar(workspace, workspace_bytes);
    uint16_t* pa = ar.take<uint16_t>(gemm_f32_split3_elems(M, K));
    uint16_t* pb = ar.take<uint16_t>(gemm_f32_split3_elems(N, K));
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layout_a = layout_a;
    g.B = B; g.ldb = ldb; g.layout_b = layout_b;
    g.C = C; g.ldc = ldc;
    g.alpha = alpha; g.beta_one = beta_one; g.tri = tri; g.upper_only = upper_only;
    return launch_gemm_f32_split3(g, pa, pb, (hipStream_t)stream);
}

size_t awq_workspace_bytes(int64_t out, int64_t in, int64_t rows, int n_alpha) {
    if (out < 1 || in < 1 || rows < 1 || n_alpha < 1) return 0;
    return awq_ws_bytes(out, in, rows, n_alpha);
}

int awq_search_alpha(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw, const void* X, int x_dtype,
                     int64_t rows, int64_t ldx, const float* alphas, int n_alpha, int bits, int group_size,
                     float* alpha_best, double* err_per_alpha, float* s, int8_t* codes, float* scales, void* workspace,
                     size_t workspace_bytes, void* stream) {
    const char* fn = "awq_search_alpha";
    if (out < 1 || in < 1 || rows < 1) return fail(PTQ_EINVAL, "%s: empty layer (out, in, rows >= 1 required)", fn);
    if (in % 8) return fail(PTQ_EINVAL, "%s: in must be a multiple of 8", fn);
    if (!dtype_ok(w_dtype) || !dtype_ok(x_dtype)) return fail(PTQ_EINVAL, "%s: bad dtype", fn);
    if (ldw < in || ldw % elems16(w_dtype) || ldx < in || ldx % elems16(x_dtype))
        return fail(PTQ_EINVAL, "%s: bad ldw/ldx", fn);
    if (bits < 2 || bits > 8) return fail(PTQ_EINVAL, "%s: bits = %d", fn, bits);
    if (group_size < 1) return fail(PTQ_EINVAL, "%s: group_size = %d", fn, group_size);
    if (n_alpha < 1 || n_alpha > 64 || !alphas) return fail(PTQ_EINVAL, "%s: n_alpha = %d", fn, n_alpha);
    for (int a = 0; a < n_alpha; ++a)
        if (!std::isfinite(alphas[a])) return fail(PTQ_EINVAL, "%s: alpha[%d] not finite", fn, a);
    if (!W || !X || !codes || !scales) return fail(PTQ_EINVAL, "%s: NULL array", fn);
    if (!aligned16(W) || !aligned16(X) || !aligned16(codes) || ((uintptr_t)scales & 3u) || (s && ((uintptr_t)s & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    const size_t need = awq_ws_bytes(out, in, rows, n_alpha);
    if (!workspace || workspace_bytes < need)
        return fail(PTQ_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);
    return run_awq(W, w_dtype, out, in, ldw, X, x_dtype, rows, ldx, alphas, n_alpha, bits, group_size, alpha_best,
                   err_per_alpha, s, codes, scales, workspace, workspace_bytes, (hipStream_t)stream);
}

size_t awq_gptq_quantize_layer_workspace_bytes(int64_t out, int64_t in, int block_size) {
    if (out < 0 || in < 1) return 0;
    return awq_gptq_workspace_bytes(out, in, block_size);
}

int awq_gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw, const float* H,
                            const double* d, const float* s, int bits, int group_size, double damp, int act_order,
                            int block_size, int8_t* codes, float* scales, int32_t* g_idx, int32_t* perm,
                            double* stats, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "awq_gptq_quantize_layer";
    PTQ_TRY(check_gptq_common(out, in, bits, group_size, block_size, fn));
    if (!dtype_ok(w_dtype)) return fail(PTQ_EINVAL, "%s: w_dtype = %d", fn, w_dtype);
    if (ldw < in || ldw % elems16(w_dtype)) return fail(PTQ_EINVAL, "%s: bad ldw", fn);
    if (!(damp >= 0.0) || !std::isfinite(damp)) return fail(PTQ_EINVAL, "%s: damp = %g", fn, damp);
    if (act_order != 0 && act_order != 1) return fail(PTQ_EINVAL, "%s: act_order = %d", fn, act_order);
    if (!H || !s) return fail(PTQ_EINVAL, "%s: H or s is NULL", fn);
    if (out > 0 && (!W || !codes || !scales)) return fail(PTQ_EINVAL, "%s: W, codes or scales is NULL", fn);
    if (!aligned16(H) || (W && !aligned16(W)) || (codes && !aligned16(codes)) || (d && ((uintptr_t)d & 7u)) ||
        ((uintptr_t)s & 3u) || (scales && ((uintptr_t)scales & 3u)) || (g_idx && ((uintptr_t)g_idx & 3u)) ||
        (perm && ((uintptr_t)perm & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    const size_t need = awq_gptq_workspace_bytes(out, in, block_size);
    if (!workspace || workspace_bytes < need)
        return fail(PTQ_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);
    return run_awq_gptq(W, w_dtype, out, in, ldw, H, d, s, bits, group_size, damp, act_order, block_size, codes,
                        scales, g_idx, perm, stats, workspace, workspace_bytes, (hipStream_t)stream);
}

int pack_int4(const int8_t* codes, int64_t out, int64_t in, int bits, uint32_t* packed, void* stream) {
    const char* fn = "pack_int4";
    if (out < 0 || in < 0) return fail(PTQ_EINVAL, "%s: negative size", fn);
    if (in % 8) return fail(PTQ_EINVAL, "%s: in = %lld must be a multiple of 8", fn, (long long)in);
    if (bits < 2 || bits > 4) return fail(PTQ_EINVAL, "%s: bits = %d: only codes of 2 to 4 bits fit a nibble", fn, bits);
    if (out * in > 0 && (!codes || !packed)) return fail(PTQ_EINVAL, "%s: codes or packed is NULL", fn);
    if ((codes && !aligned16(codes)) || (packed && !aligned16(packed)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    return launch_pack_int4(codes, out, in, packed, (hipStream_t)stream);
}

int dequantize_int4(const uint32_t* packed, const float* scales, const int32_t* g_idx, const int8_t* zeros,
                    int64_t out, int64_t in, int group_size, int out_dtype, void* What, int64_t ldo, void* stream) {
    const char* fn = "dequantize_int4";
    if (out < 0 || in < 0) return fail(PTQ_EINVAL, "%s: negative size", fn);
    if (in > ((int64_t)1 << 30)) return fail(PTQ_EINVAL, "%s: in = %lld too large", fn, (long long)in);
    if (in % 8) return fail(PTQ_EINVAL, "%s: in = %lld must be a multiple of 8", fn, (long long)in);
    if (group_size < 1) return fail(PTQ_EINVAL, "%s: group_size = %d < 1", fn, group_size);
    if (!dtype_ok(out_dtype)) return fail(PTQ_EINVAL, "%s: out_dtype = %d", fn, out_dtype);
    if (ldo < in || ldo % 8) return fail(PTQ_EINVAL, "%s: ldo = %lld (need >= in, multiple of 8)", fn, (long long)ldo);
    if (out * in > 0 && (!packed || !scales || !What)) return fail(PTQ_EINVAL, "%s: NULL pointer", fn);
    if ((packed && !aligned16(packed)) || (What && !aligned16(What)) || (scales && ((uintptr_t)scales & 3u)) ||
        (g_idx && ((uintptr_t)g_idx & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    return launch_dequant_int4(packed, scales, g_idx, zeros, out, in, group_size, out_dtype, What, ldo,
                               (hipStream_t)stream);
}

size_t layer_output_error_workspace_bytes(int64_t out, int64_t in, int64_t rows, int x_dtype) {
    if (out < 1 || in < 1 || rows < 1 || !dtype_ok(x_dtype)) return 0;
    return output_error_ws_bytes(out, in, rows, x_dtype);
}

int layer_output_error(const void* X, int x_dtype, int64_t rows, int64_t ldx, const void* W, int w_dtype, int64_t out,
                       int64_t in, int64_t ldw, const int8_t* codes, const float* scales, const int32_t* g_idx,
                       const int8_t* zeros, const float* s, int group_size, double* out2, void* workspace,
                       size_t workspace_bytes, void* stream) {
    const char* fn = "layer_output_error";
    if (out < 1 || in < 1 || rows < 1) return fail(PTQ_EINVAL, "%s: empty layer (out, in, rows >= 1 required)", fn);
    if (in % 8) return fail(PTQ_EINVAL, "%s: in must be a multiple of 8", fn);
    if (!dtype_ok(w_dtype) || !dtype_ok(x_dtype)) return fail(PTQ_EINVAL, "%s: bad dtype", fn);
    if (ldw < in || ldw % elems16(w_dtype) || ldx < in || ldx % elems16(x_dtype))
        return fail(PTQ_EINVAL, "%s: bad ldw/ldx", fn);
    if (group_size < 1) return fail(PTQ_EINVAL, "%s: group_size = %d", fn, group_size);
    if (!X || !W || !codes || !scales || !out2) return fail(PTQ_EINVAL, "%s: NULL array", fn);
    if (!aligned16(W) || !aligned16(X) || ((uintptr_t)scales & 3u) || (g_idx && ((uintptr_t)g_idx & 3u)) ||
        (s && ((uintptr_t)s & 3u)))
        return fail(PTQ_EINVAL, "%s: misaligned pointer", fn);
    const size_t need = output_error_ws_bytes(out, in, rows, x_dtype);
    if (!workspace || workspace_bytes < need)
        return fail(PTQ_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PTQ_EINVAL, "%s: misaligned workspace", fn);
    return run_output_error(X, x_dtype, rows, ldx, W, w_dtype, out, in, ldw, codes, scales, g_idx, zeros, s,
                            group_size, out2, workspace, workspace_bytes, (hipStream_t)stream);
}

}  // extern "C"
