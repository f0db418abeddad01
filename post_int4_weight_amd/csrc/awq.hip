// Stage 4: AWQ's per-layer alpha grid search on the calibration output error.
//
// "GPTQ versus AWQ objectives", "A strong answer", AWQ paragraph: scale input
// channel j of W up by s_j = mean|x_j|^alpha (the activation is scaled down by
// the same factor in the previous operator), round to nearest, and grid-search
// the single exponent alpha per layer on the calibration output error; no
// reconstruction and no backprop. "A Comprehensive Analysis of Post-Training
// Quantization Strategies for LLMs: GPTQ, AWQ and GGUF", section 3.2: the
// equivalent transform y = (W s)(X / s), then uniform quantization of the
// scaled matrix.
//
// All alphas are evaluated in one batch: awq_quant_kernel writes, per alpha,
// dW = W - Q(W diag s) diag(s)^-1 as a bf16 high part plus a bf16 residual;
// the bf16 MFMA GEMM of gemm_bf16.hip then forms X dW^T tile by tile and keeps
// only each tile's sum of squares (E is never written). fp32 calibration
// inputs take an fp32 path (E through the fp32 MFMA GEMM, then a reduction).
#include "common.hpp"

#include <algorithm>
#include <cmath>
#include <vector>

namespace ptq {

int launch_awq_error_gemm(const uint16_t* X, int64_t ldx, int64_t rows, int64_t n, const uint16_t* hi,
                          const uint16_t* lo, int64_t ldw, int64_t out, int64_t batch_stride, int nbatch,
                          double* partial, int64_t* ntiles_out, hipStream_t st);

namespace {

constexpr double MEAN_ABS_FLOOR = 1e-12;
constexpr int AWQ_ROWS = 2;   // rows per wave of the batched search kernel

// m_j (+)= sum over a slab of rows of |x_ij| (fp64); slabs reduced later.
template <typename T>
__global__ void col_abs_sum_kernel(const T* __restrict__ X, int64_t ldx, int64_t rows, int64_t n,
                                   int64_t slab_rows, double* __restrict__ part) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n) return;
    const int64_t r0 = (int64_t)blockIdx.y * slab_rows, r1 = std::min<int64_t>(rows, r0 + slab_rows);
    double s = 0.0;
    for (int64_t r = r0; r < r1; ++r) s += fabs((double)load_as_float<T>(X, r * ldx + c));
    part[(int64_t)blockIdx.y * n + c] = s;
}

// m = mean|x| with the floor; one workgroup computes the max for the floor.
__global__ void mean_abs_finish_kernel(const double* part, int nslab, int64_t n, int64_t rows, double* m) {
    __shared__ double red[256];
    double mx = 0.0;
    for (int64_t c = threadIdx.x; c < n; c += 256) {
        double s = 0.0;
        for (int q = 0; q < nslab; ++q) s += part[(int64_t)q * n + c];
        s /= (double)rows;
        m[c] = s;
        mx = fmax(mx, s);
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    const double floor_v = MEAN_ABS_FLOOR * red[0];
    for (int64_t c = threadIdx.x; c < n; c += 256) m[c] = fmax(m[c], floor_v);
}

// s[a][j] = m_j ^ alpha_a in fp64 (the rounding decisions below are taken in
// fp64, the precision of the pages' NumPy reference), and 1 / s[a][j]
__global__ void scales_kernel(const double* m, int64_t n, const float* alphas, int na, double* s, double* rs) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int a = blockIdx.y;
    if (c < n && a < na) {
        const double v = pow(m[c], (double)alphas[a]);
        s[(int64_t)a * n + c] = v;
        rs[(int64_t)a * n + c] = 1.0 / v;
    }
}

__global__ void s_to_f32_kernel(const double* s64, int64_t n, float* s) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c < n) s[c] = (float)s64[c];
}

// RTN of one group of W diag(s), decided in fp64. Returns the fp64 scale;
// emit(c, w, q) is called per column with the fp64 code.
template <typename T, typename F>
__device__ __forceinline__ double awq_group(const T* W, int64_t row_off, int64_t c0, int64_t c1, const double* s,
                                            double qmax, F emit) {
    double mx = 0.0;
    for (int64_t c = c0; c < c1; ++c) mx = fmax(mx, fabs((double)load_as_float<T>(W, row_off + c) * s[c]));
    const double scale = mx / qmax;
    for (int64_t c = c0; c < c1; ++c) {
        const double w = (double)load_as_float<T>(W, row_off + c);
        double q = 0.0;
        if (scale > 0.0) q = fmin(fmax(rint((w * s[c]) / scale), -qmax - 1.0), qmax);
        emit(c, w, q, scale);
    }
    return scale;
}

// One wave per (alpha, row, group), lanes across the group's columns (so
// loads and stores are coalesced): the group max of |W diag(s)| by a wave
// reduction, then the RTN of every column, decided in fp64 with the same
// operations as awq_group; either the hi/lo split of dW = W - Q(W diag s)
// diag(s)^-1 (search) or the codes and scales of W diag(s) (final).
template <typename T>
__global__ __launch_bounds__(256) void awq_quant_kernel(const T* __restrict__ W, int64_t ldw, int64_t out, int64_t n,
                                                        int g, float qmax, const double* __restrict__ s_all, int na,
                                                        uint16_t* __restrict__ hi, uint16_t* __restrict__ lo,
                                                        int8_t* __restrict__ codes, float* __restrict__ scales,
                                                        int64_t ngroups) {
    const int lane = threadIdx.x & 63;
    const int64_t per_a = out * ngroups;
    const int64_t id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (id >= per_a * na) return;   // whole waves
    const int a = (int)(id / per_a);
    const int64_t rem = id % per_a;
    const int64_t r = rem / ngroups, grp = rem % ngroups;
    const double* s = s_all + (int64_t)a * n;
    const int64_t c0 = grp * g, c1 = std::min<int64_t>(n, c0 + g);
    const double qm = (double)qmax;
    double mx = 0.0;
    for (int64_t c = c0 + lane; c < c1; c += 64)
        mx = fmax(mx, fabs((double)load_as_float<T>(W, r * ldw + c) * s[c]));
    for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off, 64));
    const double scale = mx / qm;
    for (int64_t c = c0 + lane; c < c1; c += 64) {
        const double w = (double)load_as_float<T>(W, r * ldw + c);
        double q = 0.0;
        if (scale > 0.0) q = fmin(fmax(rint((w * s[c]) / scale), -qm - 1.0), qm);
        if (codes) {
            codes[r * n + c] = (int8_t)(int)q;
        } else {
            const float dw = (float)(w - (q * scale) / s[c]);
            const uint16_t h = float_to_bf16_bits(dw);
            const int64_t o = (int64_t)a * out * n + r * n + c;
            hi[o] = h;
            lo[o] = float_to_bf16_bits(dw - bf16_bits_to_float(h));
        }
    }
    if (scales && lane == 0) scales[r * ngroups + grp] = (float)scale;
}

// Distance from a half-integer below which the product w s (1/scale) is
// re-decided by the division: that product lies within 2^-52 relative of the
// exact quotient, |quotient| <= 128 for bits <= 8, so 1e-12 covers it.
constexpr double TIE_EPS = 1e-12;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Search-mode RTN for every alpha in one pass over W. Each lane owns 8
// consecutive columns (one 16-byte load of bf16 W), L = g/8 lanes form a
// group and a wave covers 64/L groups of R rows. W stays in registers across
// the alpha loop, so only s and 1/s are re-read (from L2), and every store is
// 16 bytes. The decisions are those of awq_group: the group max of |w s| and
// scale = max / qmax in fp64, and q = rint(w s / scale), taken here as
// rint((w s) (1/scale)) unless that product lies within TIE_EPS of a
// half-integer, where the exact division decides. dW = w - q scale (1/s)
// differs from w - q scale / s by an fp64 rounding, far below its bf16
// hi + lo representation.
template <typename T, int L, int R>
__global__ __launch_bounds__(256) void awq_dw_batch_kernel(const T* __restrict__ W, int64_t ldw, int64_t out,
                                                           int64_t n, float qmax, const double* __restrict__ s_all,
                                                           const double* __restrict__ rs_all, int na,
                                                           uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
    constexpr int COLS = 512;   // columns per wave: 64 lanes x 8
    const int lane = threadIdx.x & 63;
    const int64_t csets = cdiv(n, (int64_t)COLS);
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t r0 = (wid / csets) * R;
    if (r0 >= out) return;   // whole waves
    const int64_t c = (wid % csets) * COLS + (int64_t)lane * 8;
    const bool live = c < n;   // n is a multiple of 8: a lane is all in or all out
    const double qm = (double)qmax;
    float wv[R][8];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (live && r0 + j < out) {
            load8<T>(W + (r0 + j) * ldw + c, wv[j]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) wv[j][k] = 0.0f;
        }
    }
    for (int a = 0; a < na; ++a) {
        double sv[8], rv[8];
        if (live) {
            const double2* sp = reinterpret_cast<const double2*>(s_all + (int64_t)a * n + c);
            const double2* rp = reinterpret_cast<const double2*>(rs_all + (int64_t)a * n + c);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const double2 x = sp[k], y = rp[k];
                sv[2 * k] = x.x; sv[2 * k + 1] = x.y;
                rv[2 * k] = y.x; rv[2 * k + 1] = y.y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) sv[k] = rv[k] = 0.0;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t r = r0 + j;
            double mx = 0.0;
#pragma unroll
            for (int k = 0; k < 8; ++k) mx = fmax(mx, fabs((double)wv[j][k] * sv[k]));
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off, 64));
            const double scale = mx / qm;
            const double rsc = scale > 0.0 ? 1.0 / scale : 0.0;
            uint32_t hp[4], lp[4];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const double w = (double)wv[j][k];
                const double ws = w * sv[k];
                const double t = ws * rsc;
                double q = rint(t);
                const double u = fabs(t);
                if (fabs(u - floor(u) - 0.5) < TIE_EPS && scale > 0.0) q = rint(ws / scale);
                q = fmin(fmax(q, -qm - 1.0), qm);
                const float dw = (float)(w - (q * scale) * rv[k]);
                const uint32_t h = float_to_bf16_bits(dw);
                const uint32_t l = float_to_bf16_bits(dw - bf16_bits_to_float((uint16_t)h));
                if (k & 1) {
                    hp[k >> 1] |= h << 16;
                    lp[k >> 1] |= l << 16;
                } else {
                    hp[k >> 1] = h;
                    lp[k >> 1] = l;
                }
            }
            if (live && r < out) {
                const int64_t o = (int64_t)a * out * n + r * n + c;
                *reinterpret_cast<uint4*>(hi + o) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
                *reinterpret_cast<uint4*>(lo + o) = make_uint4(lp[0], lp[1], lp[2], lp[3]);
            }
        }
    }
}

// fp32 path: dW as fp32 for one alpha (no split)
template <typename T>
__global__ void awq_dw_f32_kernel(const T* __restrict__ W, int64_t ldw, int64_t out, int64_t n, int g, float qmax,
                                  const double* __restrict__ s, float* __restrict__ dW, int64_t ngroups) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= out * ngroups) return;
    const int64_t r = id / ngroups, grp = id % ngroups;
    const int64_t c0 = grp * g, c1 = std::min<int64_t>(n, c0 + g);
    awq_group<T>(W, r * ldw, c0, c1, s, (double)qmax, [&](int64_t c, double w, double q, double sc) {
        dW[r * n + c] = (float)(w - (q * sc) / s[c]);
    });
}

// sum of squares of a dense buffer (fp64, one workgroup per slice, fixed order)
__global__ void sumsq_slices_kernel(const float* E, int64_t count, int64_t slice, double* part) {
    __shared__ double red[256];
    const int64_t b = (int64_t)blockIdx.x * slice, e = std::min<int64_t>(count, b + slice);
    double s = 0.0;
    for (int64_t i = b + threadIdx.x; i < e; i += 256) s += (double)E[i] * (double)E[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// err[a] = sum over tiles of partial[a][tile], fixed order
__global__ void reduce_err_kernel(const double* partial, int64_t ntiles, double* err) {
    __shared__ double red[256];
    const int a = blockIdx.x;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < ntiles; i += 256) s += partial[(int64_t)a * ntiles + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) err[a] = red[0];
}

// Calibration output error of a quantized layer: per element of W,
// What = (code - zero) * scale[gi] / s (fp64) and dW = W - What. Batch 0 of
// the outputs gets dW, batch 1 gets W itself: as bf16 high and residual parts
// (hi, lo) for the bf16 MFMA error GEMM, or as fp32 (f32). A group index
// outside [0, ngroups) makes What NaN.
template <typename T>
__global__ void eval_prep_kernel(const T* __restrict__ W, int64_t ldw, int64_t out, int64_t n,
                                 const int8_t* __restrict__ codes, const float* __restrict__ scales,
                                 const int32_t* __restrict__ g_idx, const int8_t* __restrict__ zeros,
                                 const float* __restrict__ s, int g, int64_t ngroups, uint16_t* __restrict__ hi,
                                 uint16_t* __restrict__ lo, float* __restrict__ f32) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= out * n) return;
    const int64_t r = id / n, c = id % n;
    const int64_t gi = g_idx ? (int64_t)g_idx[c] : c / g;
    const double w = (double)load_as_float<T>(W, r * ldw + c);
    double what = __builtin_nan("");
    if (gi >= 0 && gi < ngroups) {
        const double q = (double)codes[r * n + c] - (zeros ? (double)zeros[r * ngroups + gi] : 0.0);
        what = q * (double)scales[r * ngroups + gi];
        if (s) what /= (double)s[c];
    }
    const float v[2] = {(float)(w - what), (float)w};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t o = b * out * n + id;
        if (f32) {
            f32[o] = v[b];
        } else {
            const uint16_t h = float_to_bf16_bits(v[b]);
            hi[o] = h;
            lo[o] = float_to_bf16_bits(v[b] - bf16_bits_to_float(h));
        }
    }
}

constexpr int64_t SLAB = 1024;
constexpr int64_t F32_SLICE = 1 << 16;

struct AwqLayout {
    int64_t nslab, ntiles;
};

AwqLayout awq_layout(int64_t out, int64_t n, int64_t rows) {
    AwqLayout l;
    l.nslab = std::max<int64_t>(1, cdiv(rows, SLAB));
    l.ntiles = cdiv(rows, 256) * cdiv(out, 256);
    return l;
}

}  // namespace

size_t awq_ws_bytes(int64_t out, int64_t n, int64_t rows, int n_alpha) {
    AwqLayout l = awq_layout(out, n, rows);
    Sizer z;
    z.take<double>((size_t)l.nslab * n);        // column |x| partials
    z.take<double>((size_t)n);                  // m
    z.take<double>((size_t)n_alpha * n);        // s per alpha (fp64)
    z.take<double>((size_t)n_alpha * n);        // 1 / s per alpha
    z.take<float>((size_t)n_alpha);             // alphas (device copy)
    z.take<double>((size_t)n_alpha);            // err
    // bf16 path: hi + lo for every alpha, one partial per tile and alpha
    Sizer b = z;
    b.take<uint16_t>((size_t)n_alpha * out * n);
    b.take<uint16_t>((size_t)n_alpha * out * n);
    b.take<double>((size_t)n_alpha * l.ntiles);
    // fp32 path: dW and E for one alpha, slice partials
    Sizer f = z;
    f.take<float>((size_t)out * n);
    f.take<float>((size_t)rows * out);
    f.take<double>((size_t)cdiv(rows * out, F32_SLICE) + 1);
    return std::max(b.bytes(), f.bytes());
}

int run_awq(const void* W, int w_dtype, int64_t out, int64_t n, int64_t ldw, const void* X, int x_dtype,
            int64_t rows, int64_t ldx, const float* alphas, int n_alpha, int bits, int g, float* alpha_best,
            double* err_per_alpha, float* s_out, int8_t* codes, float* scales, void* ws, size_t ws_bytes,
            hipStream_t st) {
    AwqLayout l = awq_layout(out, n, rows);
    Arena ar(ws, ws_bytes);
    double* cpart = ar.take<double>((size_t)l.nslab * n);
    double* m = ar.take<double>((size_t)n);
    double* s_all = ar.take<double>((size_t)n_alpha * n);
    double* rs_all = ar.take<double>((size_t)n_alpha * n);
    float* al_dev = ar.take<float>((size_t)n_alpha);
    double* err = ar.take<double>((size_t)n_alpha);
    const int64_t ngroups = cdiv(n, g);
    const float qmax = (float)((1 << (bits - 1)) - 1);
    const bool bf = (x_dtype == PTQ_BF16);
    uint16_t *hi = nullptr, *lo = nullptr;
    double* partial = nullptr;
    float *dW = nullptr, *E = nullptr;
    if (bf) {
        hi = ar.take<uint16_t>((size_t)n_alpha * out * n);
        lo = ar.take<uint16_t>((size_t)n_alpha * out * n);
        partial = ar.take<double>((size_t)n_alpha * l.ntiles);
    } else {
        dW = ar.take<float>((size_t)out * n);
        E = ar.take<float>((size_t)rows * out);
        partial = ar.take<double>((size_t)cdiv(rows * out, F32_SLICE) + 1);
    }
    if (!cpart || !m || !s_all || !rs_all || !al_dev || !err || !partial || (bf && (!hi || !lo)) || (!bf && (!dW || !E))) {
        set_error("awq_search_alpha: workspace of %zu bytes, %zu needed", ws_bytes,
                  awq_ws_bytes(out, n, rows, n_alpha));
        return PTQ_EWORKSPACE;
    }
    PTQ_HIP(hipMemcpyAsync(al_dev, alphas, sizeof(float) * n_alpha, hipMemcpyHostToDevice, st));

    // m_j = mean |x_j|
    {
        dim3 grid((unsigned)cdiv(n, 256), (unsigned)l.nslab);
        if (bf)
            hipLaunchKernelGGL(col_abs_sum_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)X, ldx, rows, n,
                               SLAB, cpart);
        else
            hipLaunchKernelGGL(col_abs_sum_kernel<float>, grid, dim3(256), 0, st, (const float*)X, ldx, rows, n, SLAB,
                               cpart);
        PTQ_LAUNCH_CHECK();
        hipLaunchKernelGGL(mean_abs_finish_kernel, dim3(1), dim3(256), 0, st, cpart, (int)l.nslab, n, rows, m);
        PTQ_LAUNCH_CHECK();
        hipLaunchKernelGGL(scales_kernel, dim3((unsigned)cdiv(n, 256), (unsigned)n_alpha), dim3(256), 0, st, m, n,
                           al_dev, n_alpha, s_all, rs_all);
        PTQ_LAUNCH_CHECK();
    }

    if (bf) {
        const int64_t nth = cdiv(out * ngroups * n_alpha, 4) * 256;   // one wave per (alpha, row, group)
        const int wbytes = w_dtype == PTQ_BF16 ? 2 : 4;
        const bool vec = g % 8 == 0 && g >= 32 && g <= 512 && (g & (g - 1)) == 0 && n % 8 == 0 &&
                         (ldw * wbytes) % 16 == 0 && ((uintptr_t)W & 15) == 0;
        if (vec) {
            constexpr int R = AWQ_ROWS;
            const int64_t waves = cdiv(out, (int64_t)R) * cdiv(n, (int64_t)512);
            const dim3 grid((unsigned)cdiv(waves, 4));
#define PTQ_AWQ_VEC(T, LL)                                                                                          \
    hipLaunchKernelGGL((awq_dw_batch_kernel<T, LL, R>), grid, dim3(256), 0, st, (const T*)W, ldw, out, n, qmax,   \
                       s_all, rs_all, n_alpha, hi, lo)
#define PTQ_AWQ_VEC_T(T)              \
    switch (g / 8) {                  \
        case 4: PTQ_AWQ_VEC(T, 4); break;   \
        case 8: PTQ_AWQ_VEC(T, 8); break;   \
        case 16: PTQ_AWQ_VEC(T, 16); break; \
        case 32: PTQ_AWQ_VEC(T, 32); break; \
        default: PTQ_AWQ_VEC(T, 64); break; \
    }
            if (w_dtype == PTQ_BF16) {
                PTQ_AWQ_VEC_T(uint16_t)
            } else {
                PTQ_AWQ_VEC_T(float)
            }
#undef PTQ_AWQ_VEC_T
#undef PTQ_AWQ_VEC
        } else if (w_dtype == PTQ_BF16)
            hipLaunchKernelGGL(awq_quant_kernel<uint16_t>, dim3((unsigned)cdiv(nth, 256)), dim3(256), 0, st,
                               (const uint16_t*)W, ldw, out, n, g, qmax, s_all, n_alpha, hi, lo, (int8_t*)nullptr,
                               (float*)nullptr, ngroups);
        else
            hipLaunchKernelGGL(awq_quant_kernel<float>, dim3((unsigned)cdiv(nth, 256)), dim3(256), 0, st,
                               (const float*)W, ldw, out, n, g, qmax, s_all, n_alpha, hi, lo, (int8_t*)nullptr,
                               (float*)nullptr, ngroups);
        PTQ_LAUNCH_CHECK();
        int64_t ntiles = 0;
        PTQ_TRY(launch_awq_error_gemm((const uint16_t*)X, ldx, rows, n, hi, lo, n, out, out * n, n_alpha, partial,
                                      &ntiles, st));
        hipLaunchKernelGGL(reduce_err_kernel, dim3((unsigned)n_alpha), dim3(256), 0, st, partial, ntiles, err);
        PTQ_LAUNCH_CHECK();
    } else {
        const int64_t nslice = cdiv(rows * out, F32_SLICE);
        for (int a = 0; a < n_alpha; ++a) {
            if (w_dtype == PTQ_BF16)
                hipLaunchKernelGGL(awq_dw_f32_kernel<uint16_t>, dim3((unsigned)cdiv(out * ngroups, 256)), dim3(256), 0,
                                   st, (const uint16_t*)W, ldw, out, n, g, qmax, s_all + (int64_t)a * n, dW, ngroups);
            else
                hipLaunchKernelGGL(awq_dw_f32_kernel<float>, dim3((unsigned)cdiv(out * ngroups, 256)), dim3(256), 0, st,
                                   (const float*)W, ldw, out, n, g, qmax, s_all + (int64_t)a * n, dW, ngroups);
            PTQ_LAUNCH_CHECK();
            // E = X dW^T  [rows, out]
            GemmArgs ga{};
            ga.M = rows; ga.N = out; ga.K = n;
            ga.A = (const float*)X; ga.lda = ldx; ga.layout_a = A_MK;
            ga.B = dW; ga.ldb = n; ga.layout_b = B_NK;
            ga.C = E; ga.ldc = out; ga.alpha = 1.f; ga.beta_one = 0; ga.tri = TRI_NONE; ga.upper_only = 0;
            PTQ_TRY(launch_gemm_f32(ga, st));
            hipLaunchKernelGGL(sumsq_slices_kernel, dim3((unsigned)nslice), dim3(256), 0, st, E, rows * out, F32_SLICE,
                               partial);
            PTQ_LAUNCH_CHECK();
            hipLaunchKernelGGL(reduce_err_kernel, dim3(1), dim3(256), 0, st, partial, nslice, err + a);
            PTQ_LAUNCH_CHECK();
        }
    }

    std::vector<double> eh(n_alpha);
    PTQ_HIP(hipMemcpyAsync(eh.data(), err, sizeof(double) * n_alpha, hipMemcpyDeviceToHost, st));
    PTQ_HIP(hipStreamSynchronize(st));
    int best = 0;
    for (int a = 1; a < n_alpha; ++a)
        if (eh[a] < eh[best]) best = a;
    if (err_per_alpha)
        for (int a = 0; a < n_alpha; ++a) err_per_alpha[a] = eh[a];
    if (alpha_best) *alpha_best = alphas[best];

    // final codes / scales of W diag(s) at alpha*
    const double* sb = s_all + (int64_t)best * n;
    if (s_out) {
        hipLaunchKernelGGL(s_to_f32_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, sb, n, s_out);
        PTQ_LAUNCH_CHECK();
    }
    const int64_t nth = cdiv(out * ngroups, 4) * 256;
    if (w_dtype == PTQ_BF16)
        hipLaunchKernelGGL(awq_quant_kernel<uint16_t>, dim3((unsigned)cdiv(nth, 256)), dim3(256), 0, st,
                           (const uint16_t*)W, ldw, out, n, g, qmax, sb, 1, (uint16_t*)nullptr, (uint16_t*)nullptr,
                           codes, scales, ngroups);
    else
        hipLaunchKernelGGL(awq_quant_kernel<float>, dim3((unsigned)cdiv(nth, 256)), dim3(256), 0, st, (const float*)W,
                           ldw, out, n, g, qmax, sb, 1, (uint16_t*)nullptr, (uint16_t*)nullptr, codes, scales, ngroups);
    PTQ_LAUNCH_CHECK();
    PTQ_HIP(hipStreamSynchronize(st));
    return PTQ_OK;
}

// ---------------------------------------------------------------------------
// ||X (W - What)^T||^2 and ||X W^T||^2 (the objective of "A strong answer" and
// its normaliser) for a quantized layer. bf16 X: both through the bf16 MFMA
// error GEMM (W and dW as hi + lo bf16 pairs, E never written). fp32 X: E in
// row chunks through the fp32 MFMA GEMM, then fp64 sums of squares.
constexpr int64_t EVAL_ROWS = 4096;   // fp32 path: rows of X per GEMM

size_t output_error_ws_bytes(int64_t out, int64_t n, int64_t rows, int x_dtype) {
    Sizer z;
    z.take<double>(2);
    if (x_dtype == PTQ_BF16) {
        z.take<uint16_t>((size_t)2 * out * n);
        z.take<uint16_t>((size_t)2 * out * n);
        z.take<double>((size_t)2 * cdiv(rows, 256) * cdiv(out, 256));
    } else {
        const int64_t rc = std::min<int64_t>(rows, EVAL_ROWS);
        z.take<float>((size_t)2 * out * n);
        z.take<float>((size_t)rc * out);
        z.take<double>((size_t)2 * cdiv(rows, EVAL_ROWS) * cdiv(rc * out, F32_SLICE));
    }
    return z.bytes();
}

int run_output_error(const void* X, int x_dtype, int64_t rows, int64_t ldx, const void* W, int w_dtype, int64_t out,
                     int64_t n, int64_t ldw, const int8_t* codes, const float* scales, const int32_t* g_idx,
                     const int8_t* zeros, const float* s, int g, double* out2, void* ws, size_t ws_bytes,
                     hipStream_t st) {
    Arena ar(ws, ws_bytes);
    double* err = ar.take<double>(2);
    const int64_t ngroups = cdiv(n, g);
    const bool bf = (x_dtype == PTQ_BF16);
    uint16_t *hi = nullptr, *lo = nullptr;
    float *f32 = nullptr, *E = nullptr;
    double* partial = nullptr;
    const int64_t rc = std::min<int64_t>(rows, EVAL_ROWS);
    const int64_t nchunk = cdiv(rows, EVAL_ROWS), per_chunk = cdiv(rc * out, F32_SLICE);
    if (bf) {
        hi = ar.take<uint16_t>((size_t)2 * out * n);
        lo = ar.take<uint16_t>((size_t)2 * out * n);
        partial = ar.take<double>((size_t)2 * cdiv(rows, 256) * cdiv(out, 256));
    } else {
        f32 = ar.take<float>((size_t)2 * out * n);
        E = ar.take<float>((size_t)rc * out);
        partial = ar.take<double>((size_t)2 * nchunk * per_chunk);
    }
    if (!err || !partial || (bf && (!hi || !lo)) || (!bf && (!f32 || !E))) {
        set_error("layer_output_error: workspace of %zu bytes, %zu needed", ws_bytes,
                  output_error_ws_bytes(out, n, rows, x_dtype));
        return PTQ_EWORKSPACE;
    }
    const unsigned blocks = (unsigned)cdiv(out * n, 256);
    if (w_dtype == PTQ_BF16)
        hipLaunchKernelGGL(eval_prep_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t*)W, ldw, out, n,
                           codes, scales, g_idx, zeros, s, g, ngroups, hi, lo, f32);
    else
        hipLaunchKernelGGL(eval_prep_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)W, ldw, out, n,
                           codes, scales, g_idx, zeros, s, g, ngroups, hi, lo, f32);
    PTQ_LAUNCH_CHECK();
    if (bf) {
        int64_t ntiles = 0;
        PTQ_TRY(launch_awq_error_gemm((const uint16_t*)X, ldx, rows, n, hi, lo, n, out, out * n, 2, partial, &ntiles,
                                      st));
        hipLaunchKernelGGL(reduce_err_kernel, dim3(2), dim3(256), 0, st, partial, ntiles, err);
        PTQ_LAUNCH_CHECK();
    } else {
        // slice partials packed densely: full chunks first, then the last
        const int64_t last = rows - (nchunk - 1) * EVAL_ROWS;
        const int64_t total = (nchunk - 1) * per_chunk + cdiv(last * out, F32_SLICE);
        for (int b = 0; b < 2; ++b) {
            for (int64_t k = 0; k < nchunk; ++k) {
                const int64_t r0 = k * EVAL_ROWS, nr = std::min<int64_t>(EVAL_ROWS, rows - r0);
                GemmArgs ga{};
                ga.M = nr; ga.N = out; ga.K = n;
                ga.A = (const float*)X + r0 * ldx; ga.lda = ldx; ga.layout_a = A_MK;
                ga.B = f32 + (int64_t)b * out * n; ga.ldb = n; ga.layout_b = B_NK;
                ga.C = E; ga.ldc = out; ga.alpha = 1.f; ga.beta_one = 0; ga.tri = TRI_NONE; ga.upper_only = 0;
                PTQ_TRY(launch_gemm_f32(ga, st));
                hipLaunchKernelGGL(sumsq_slices_kernel, dim3((unsigned)cdiv(nr * out, F32_SLICE)), dim3(256), 0, st, E,
                                   nr * out, F32_SLICE, partial + b * total + k * per_chunk);
                PTQ_LAUNCH_CHECK();
            }
        }
        hipLaunchKernelGGL(reduce_err_kernel, dim3(2), dim3(256), 0, st, partial, total, err);
        PTQ_LAUNCH_CHECK();
    }
    PTQ_HIP(hipMemcpyAsync(out2, err, sizeof(double) * 2, hipMemcpyDeviceToHost, st));
    PTQ_HIP(hipStreamSynchronize(st));
    return PTQ_OK;
}

}  // namespace ptq
