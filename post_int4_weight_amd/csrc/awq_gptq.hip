// AWQ's scaling first, GPTQ's rounding after.
//
// "GPTQ versus AWQ objectives" (inferenceinterviews.com), "A strong answer":
// for 3-bit or aggressive targets the two compose, AWQ's per-channel scaling
// applied first and GPTQ's rounding after. With X' = X diag(s)^-1 and
// W' = W diag(s) the layer output is unchanged, so GPTQ runs on the scaled
// layer as on any other: H0' = X'^T X' = diag(s)^-1 H0 diag(s)^-1, d' = d / s^2
// (the fp64 act-order key), damping taken on H0'. The codes and scales
// quantize W'; the caller folds 1/s into the previous operator, as for AWQ.
//
// Three streaming kernels build W' (fp32), H0' and d' in the workspace; the
// factor and the column loop are the GPTQ stages unchanged.
#include "common.hpp"

#include <algorithm>

namespace ptq {
namespace {

template <typename T>
__global__ void scale_columns_kernel(const T* __restrict__ W, int64_t ldw, int64_t out, int64_t n,
                                     const float* __restrict__ s, float* __restrict__ Ws) {
    const int64_t total = out * n;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = e / n, c = e % n;
        Ws[e] = (float)((double)load_as_float<T>(W, r * ldw + c) * (double)s[c]);
    }
}

// H'[i][j] = H[i][j] / (s_i s_j), in fp64 then rounded once
__global__ void scale_hessian_kernel(const float* __restrict__ H, int64_t n, const float* __restrict__ s,
                                     float* __restrict__ Hs) {
    const int64_t i = blockIdx.y;
    const double si = (double)s[i];
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x)
        Hs[i * n + j] = (float)((double)H[i * n + j] / (si * (double)s[j]));
}

__global__ void scale_key_kernel(const double* __restrict__ d, int64_t n, const float* __restrict__ s,
                                 double* __restrict__ ds) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < n) ds[j] = d[j] / ((double)s[j] * (double)s[j]);
}

}  // namespace

size_t awq_gptq_workspace_bytes(int64_t out, int64_t n, int block) {
    Sizer z;
    z.take<float>((size_t)out * n);          // W'
    z.take<float>((size_t)n * n);            // H0'
    z.take<double>((size_t)n);               // d'
    z.take<float>((size_t)n * n);            // U
    z.take<int32_t>((size_t)n);              // perm (when the caller passes none)
    z.take<char>(factor_workspace_bytes(n));
    z.take<char>(columns_workspace_bytes(out, n, block));
    return z.bytes();
}

int run_awq_gptq(const void* W, int w_dtype, int64_t out, int64_t n, int64_t ldw, const float* H, const double* d,
                 const float* s, int bits, int g, double damp, int act_order, int block, int8_t* codes,
                 float* scales, int32_t* g_idx, int32_t* perm, double* stats, void* ws, size_t ws_bytes,
                 hipStream_t st) {
    Arena ar(ws, ws_bytes);
    float* Ws = ar.take<float>((size_t)out * n);
    float* Hs = ar.take<float>((size_t)n * n);
    double* ds = ar.take<double>((size_t)n);
    float* U = ar.take<float>((size_t)n * n);
    int32_t* ptmp = ar.take<int32_t>((size_t)n);
    void* fws = ar.take<char>(factor_workspace_bytes(n));
    void* cws = ar.take<char>(columns_workspace_bytes(out, n, block));
    if (!Hs || !ds || !U || !ptmp || !fws || !cws || (out > 0 && !Ws)) {
        set_error("awq_gptq_quantize_layer: workspace of %zu bytes, %zu needed", ws_bytes,
                  awq_gptq_workspace_bytes(out, n, block));
        return PTQ_EWORKSPACE;
    }
    if (out > 0) {
        const unsigned grid = (unsigned)std::min<int64_t>(cdiv(out * n, 256), 16384);
        if (w_dtype == PTQ_BF16)
            hipLaunchKernelGGL(scale_columns_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, (const uint16_t*)W, ldw,
                               out, n, s, Ws);
        else
            hipLaunchKernelGGL(scale_columns_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)W, ldw, out,
                               n, s, Ws);
        PTQ_LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(scale_hessian_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)n),
                       dim3(256), 0, st, H, n, s, Hs);
    PTQ_LAUNCH_CHECK();
    if (d) {
        hipLaunchKernelGGL(scale_key_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, d, n, s, ds);
        PTQ_LAUNCH_CHECK();
    }
    int32_t* p = perm ? perm : ptmp;
    double lam = 0.0;
    PTQ_TRY(run_inverse_factor(Hs, d ? ds : nullptr, n, damp, act_order, U, p, &lam, fws, factor_workspace_bytes(n),
                               st));
    double sv[4] = {0.0, 0.0, 0.0, 0.0};
    PTQ_TRY(run_quantize_columns(Ws, PTQ_F32, out, n, n, U, act_order ? p : nullptr, bits, g, block, codes, scales,
                                 nullptr, g_idx, sv, cws, columns_workspace_bytes(out, n, block), st));
    if (stats) {
        stats[0] = sv[0];
        stats[1] = lam;
        stats[2] = sv[2];
        stats[3] = sv[0] - lam * sv[2];
    }
    return PTQ_OK;
}

}  // namespace ptq
