// Stage 3: GPTQ's column-by-column error-feedback loop, in lazy blocks.
//
// "GPTQ versus AWQ objectives", "A strong answer": at each group start the
// per-row scale is max |W| over the group's columns divided by qmax, taken
// from the CURRENT (error-updated) weights; each column is rounded to nearest
// and clipped to [-qmax-1, qmax]; its error divided by U_jj is subtracted from
// every later column through row j of U. The page's lazy-batch remark: the
// updates are batched over blocks of columns so the work runs as GEMMs.
//
// Rows are independent (each row's feedback only touches that row), so per
// block of B columns:
//  * gptq_block_kernel: 16 lanes per row, 8 columns per lane, the row's block
//    in registers and U's B x B diagonal block in LDS. Step j: every lane
//    rounds its copy of column j, the owner lane's error is broadcast across
//    the row's 16 lanes (a DPP row broadcast), and each lane updates its 8
//    columns with one LDS read of U[j][..] (U's strictly lower part is zero,
//    so columns <= j are untouched). Group maxima are lane-group reductions.
//  * the trailing update W[:, b1:] -= E U[b0:b1, b1:], E being the block's
//    errors, batched twice more: the block's errors update the rest of its
//    512-column mid-block at once and a mid-block's errors the rest of its
//    2048-column super-block (fp32 MFMA, gemm_f32.hip); the columns past the
//    super-block get all of its errors in one K = 2048 GEMM (on the bf16 MFMA
//    from three-term operand splits when large, gemm_bf16.hip).
// Act-order is a gather of W's columns into processing order up front; codes
// are written straight back to their original column positions.
#include "common.hpp"

#include <algorithm>
#include <type_traits>
#include <vector>

namespace ptq {
namespace {

constexpr int CPL = 8;     // columns per lane

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
// Super-block of the two-level lazy batch (a multiple of every block size).
// On the 8192 x 28672 down_proj shape the column stage takes 75.0 ms at 512,
// 63.8 at 1024 and 60.4 at 2048: the trailing GEMMs get 4x the depth per pass
// over W while the in-super-block updates (out * in * SB flops) stay small.
constexpr int64_t SB_COLS = 2048;
constexpr int NTH = 256;
// |w/scale| <= 128.5 for bits <= 8, where one fp32 ulp is <= 2^-16: a band of
// 2^-15 around each half-integer holds every fp32 quotient whose rounding
// could differ from the fp64 one.
constexpr float TIE_BAND = 1.0f / 32768.0f;

// Wc[r][k] = W[r][perm[k]] as fp32
template <typename T>
__global__ void gather_columns_kernel(const T* __restrict__ W, int64_t ldw, int64_t out, int64_t n,
                                      const int32_t* __restrict__ perm, float* __restrict__ Wc) {
    const int64_t r = blockIdx.y;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = perm ? perm[k] : k;
        Wc[r * n + k] = load_as_float<T>(W, r * ldw + c);
    }
}

// The same without a permutation, for bf16 W with 16-byte aligned rows and
// n % 8 == 0: Wc[r][8q .. 8q+7] from one 16-byte load, two 16-byte stores
__global__ void widen_rows_bf16_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t n,
                                       float* __restrict__ Wc) {
    const int64_t r = blockIdx.y, n8 = n / 8;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n8; q += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = *(const uint4*)(W + r * ldw + 8 * q);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = bf16_bits_to_float((uint16_t)(w[e] & 0xFFFFu));
            f[2 * e + 1] = bf16_bits_to_float((uint16_t)(w[e] >> 16));
        }
        float4* o = (float4*)(Wc + r * n + 8 * q);
        o[0] = make_float4(f[0], f[1], f[2], f[3]);
        o[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
}

// Zero-point group parameters from the group's range [lo, hi] (0 included):
// scale = (hi - lo) / maxq in fp32; zero = round(-lo / scale), decided in
// fp64 like the codes.
__device__ __forceinline__ void zp_params(float hi, float lo, float maxq, float& scale, float& zero) {
    scale = (hi - lo) / maxq;
    zero = (hi > lo) ? (float)rint(-(double)lo / (((double)hi - (double)lo) / (double)maxq)) : 0.f;
}

// ZP = false: symmetric grid, qmax = 2^(bits-1) - 1, codes in [-qmax-1, qmax].
// ZP = true: zero-point grid, qmax = maxq = 2^bits - 1, codes in [0, maxq],
// one zero-point per (row, group) in `zeros`.
template <int B, bool ZP>
__global__ __launch_bounds__(NTH) void gptq_block_kernel(float* __restrict__ Wc, int64_t out, int64_t n,
                                                          const float* __restrict__ U, int64_t b0, int bc,
                                                          int g, float qmax, const int32_t* __restrict__ perm,
                                                          int8_t* __restrict__ codes, float* __restrict__ scales,
                                                          int8_t* __restrict__ zeros,
                                                          int64_t ngroups, float* __restrict__ gmaxes,
                                                          float* __restrict__ E, int lde,
                                                          float* __restrict__ err2, int64_t nblocks,
                                                          int* __restrict__ flag, uint64_t gs_lo, uint64_t gs_hi) {
    // gs_lo / gs_hi: bit j (j < 64 / j - 64) set where a group of g <= B
    // columns starts at block column j (no bits when groups span blocks)
    constexpr int LPR = B / CPL;          // lanes per row
    constexpr int RPW = NTH / LPR;        // rows per workgroup
    __shared__ float Us[B][B + 4];
    __shared__ float rdiag[B];            // 1 / U[j][j]

    const int t = threadIdx.x;
    // stage U[b0:b0+bc, b0:b0+bc] (upper; zero elsewhere and outside bc):
    // all of this thread's loads in flight before the first LDS store
    {
        constexpr int PT = B * B / NTH;
        float sv[PT];
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int e = t + q * NTH, i = e / B, j = e % B;
            sv[q] = (i < bc && j < bc && j >= i) ? U[(b0 + i) * n + (b0 + j)] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int e = t + q * NTH;
            Us[e / B][e % B] = sv[q];
        }
    }
    __syncthreads();
    if (t < B) rdiag[t] = 1.f / ((t < bc) ? Us[t][t] : 1.f);
    __syncthreads();

    const int lr = t % LPR;                       // lane within row
    const int64_t r = (int64_t)blockIdx.x * RPW + t / LPR;
    const bool live = r < out;
    const int c0 = lr * CPL;                      // first column of this lane (within block)

    float w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) w[c] = (live && c0 + c < bc) ? Wc[r * n + b0 + c0 + c] : 0.f;

    float cq[CPL], ce[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) { cq[c] = 0.f; ce[c] = 0.f; }

    const int row_lane0 = (t & 63) - lr;          // first lane of this row in the wave
    // 1 / U[j][j] of this lane's own columns (only the owner's error is kept)
    float rd[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) rd[c] = rdiag[c0 + c];
    float scale = 0.f;
    float rscale = 0.f;     // 1 / scale (0 while scale is 0)
    float gmax = 0.f;       // symmetric: the group's max |w| (scale = gmax / qmax); zero-point: hi
    float glo = 0.f;        // zero-point: lo
    float zero = 0.f;       // zero-point: the group's zero

    if (g > B) {
        // groups span several blocks and start on block boundaries
        if (b0 % g == 0) {
            // new group: max over its columns of the current weights (all
            // earlier feedback has been applied to them)
            const int64_t j1 = std::min<int64_t>(n, b0 + g);
            float mx = 0.f, mn = 0.f;
            if (live)
                for (int64_t k = b0 + lr; k < j1; k += LPR) {
                    const float v = Wc[r * n + k];
                    if (ZP) {
                        mx = fmaxf(mx, v);
                        mn = fminf(mn, v);
                    } else {
                        mx = fmaxf(mx, fabsf(v));
                    }
                }
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) {
                mx = fmaxf(mx, __shfl_xor(mx, off, 64));
                if (ZP) mn = fminf(mn, __shfl_xor(mn, off, 64));
            }
            gmax = mx;
            glo = mn;
            if (ZP) zp_params(mx, mn, qmax, scale, zero);
            else scale = mx / qmax;
            rscale = (scale > 0.f) ? 1.f / scale : 0.f;
            if (live && lr == 0) {
                scales[r * ngroups + b0 / g] = scale;
                gmaxes[2 * (r * ngroups + b0 / g)] = mx;
                gmaxes[2 * (r * ngroups + b0 / g) + 1] = mn;
                if (ZP) zeros[r * ngroups + b0 / g] = (int8_t)(int)zero;
            }
        } else if (live) {
            scale = scales[r * ngroups + b0 / g];  // written by an earlier block
            gmax = gmaxes[2 * (r * ngroups + b0 / g)];
            glo = gmaxes[2 * (r * ngroups + b0 / g) + 1];
            if (ZP) zero = (float)zeros[r * ngroups + b0 / g];
            rscale = (scale > 0.f) ? 1.f / scale : 0.f;
        }
    }

    // Column j = CPL o + c belongs to lane o of its row (segment o). Group
    // starts and the block's end fall on segment starts (groups of g <= B
    // columns are multiples of 8, and bc is), so those checks run once per
    // segment; the segments are unrolled at compile time, which makes the
    // owner lane a constant (the DPP broadcast needs one).
    int64_t gnext = (b0 + g - 1) / g;             // index of the next group to start in this block
    // U[j][c0..c0+8) of the next column, read one column ahead (off the
    // dependency chain of the error broadcast)
    float4 un0 = *(const float4*)&Us[0][c0];
    float4 un1 = *(const float4*)&Us[0][c0 + 4];
    static_for<0, LPR>([&](auto oc) {
        constexpr int o = decltype(oc)::value;
        if (CPL * o >= bc) return;
        if (((o * CPL < 64 ? (gs_lo >> ((o * CPL) & 63)) : (gs_hi >> ((o * CPL) & 63))) & 1) != 0) {
            // the group [j, j+g) lies inside this block: lanes whose columns fall in it
            const int j = CPL * o;
            float loc = 0.f, lmn = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int col = c0 + c;
                if (col >= j && col < j + g && col < bc) {
                    if (ZP) {
                        loc = fmaxf(loc, w[c]);
                        lmn = fminf(lmn, w[c]);
                    } else {
                        loc = fmaxf(loc, fabsf(w[c]));
                    }
                }
            }
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) {
                loc = fmaxf(loc, __shfl_xor(loc, off, 64));
                if (ZP) lmn = fminf(lmn, __shfl_xor(lmn, off, 64));
            }
            gmax = loc;
            glo = lmn;
            if (ZP) zp_params(loc, lmn, qmax, scale, zero);
            else scale = loc / qmax;
            rscale = (scale > 0.f) ? 1.f / scale : 0.f;
            if (live && lr == 0) {
                scales[r * ngroups + gnext] = scale;
                if (ZP) zeros[r * ngroups + gnext] = (int8_t)(int)zero;
            }
            ++gnext;
        }
        const bool own = lr == o;
        // The segment's 8 columns run first without the fp64 recheck (a
        // branch on every column of the dependency chain), noting whether an
        // owner's quotient fell within TIE_BAND of a half-integer. If one did
        // (rare: the band is 2^-14 wide per half-integer), the wave restores
        // the segment's starting state and runs it again with the recheck,
        // so every result is the rechecked one.
        float wsave[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) wsave[c] = w[c];
        auto columns = [&](auto exact_c) {
            constexpr bool EXACT = decltype(exact_c)::value;
            float near = 1.f;   // least distance of this lane's quotients to a half-integer
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int j = CPL * o + c;
                const float4 u0 = un0, u1 = un1;
                if (j + 1 < B) {
                    un0 = *(const float4*)&Us[j + 1][c0];
                    un1 = *(const float4*)&Us[j + 1][c0 + 4];
                }
                // round this lane's copy of column j (the owner's copy is the
                // real one). The rounding decision is the fp64 one,
                // x / (gmax / qmax) in double: the fp32 x * (1 / scale) is
                // within 3 ulp of it, so only quotients that close to a
                // half-integer (TIE_BAND, far wider) are recomputed in fp64.
                // Scale 0 gives code 0 with no test on the chain: rscale is 0
                // then, so the quotient of a finite weight is 0 (and zero is
                // 0), never a tie.
                const float x = w[c];
                const float tq = x * rscale;
                float rq = rintf(tq);
                const float dist = fabsf(fabsf(tq - rq) - 0.5f);
                if constexpr (EXACT) {
                    if (dist < TIE_BAND) {
                        const double s64 =
                            ZP ? ((double)gmax - (double)glo) / (double)qmax : (double)gmax / (double)qmax;
                        rq = (float)rint((double)x / s64);
                    }
                } else {
                    near = fminf(near, dist);
                }
                // the clip as one median-of-three (the same value as
                // min(max()) for every finite rq)
                const float q = ZP ? __builtin_amdgcn_fmed3f(rq + zero, 0.f, qmax)
                                   : __builtin_amdgcn_fmed3f(rq, -qmax - 1.f, qmax);
                const float e = (x - (q - zero) * scale) * rd[c];
                // the owner's error to the row's lanes: with 16 lanes per row
                // a DPP broadcast of lane o within each 16-lane row
                // (row_newbcast), no LDS round trip; else a bpermute
                float eb;
                if constexpr (LPR == 16)
                    eb = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(e), 0x150 + o, 0xF, 0xF, false));
                else
                    eb = __shfl(e, row_lane0 + o, 64);
                cq[c] = own ? q : cq[c];
                ce[c] = own ? e : ce[c];
                w[0] = fmaf(-eb, u0.x, w[0]);
                w[1] = fmaf(-eb, u0.y, w[1]);
                w[2] = fmaf(-eb, u0.z, w[2]);
                w[3] = fmaf(-eb, u0.w, w[3]);
                w[4] = fmaf(-eb, u1.x, w[4]);
                w[5] = fmaf(-eb, u1.y, w[5]);
                w[6] = fmaf(-eb, u1.z, w[6]);
                w[7] = fmaf(-eb, u1.w, w[7]);
            }
            return near;
        };
        const float near = columns(std::false_type{});
        // the replay is marked unlikely, so the compiler lays it out of the
        // fast path's straight line (5.9 against 6.2 ms per down_proj layer)
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(own && near < TIE_BAND) != 0, 0)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) w[c] = wsave[c];
            un0 = *(const float4*)&Us[CPL * o][c0];
            un1 = *(const float4*)&Us[CPL * o][c0 + 4];
            columns(std::true_type{});
        }
    });

    // the sum of this lane's own squared errors, in column order
    float e2 = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) e2 = fmaf(ce[c], ce[c], e2);
    if (!live) return;
    // errors for the trailing GEMM, codes, per-(row, block) sum of err^2
    bool bad = false;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int col = c0 + c;
        if (col < bc) {
            E[r * lde + col] = ce[c];
            bad |= !isfinite(ce[c]);
            const int64_t k = b0 + col;
            const int64_t oc = perm ? perm[k] : k;
            codes[r * n + oc] = (int8_t)(int)cq[c];
        }
    }
    float s = e2;
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off, 64);
    if (lr == 0) err2[r * nblocks + b0 / B] = s;
    if (bad) atomicOr(flag, 1);
}

// g_idx[perm[k]] = k / g
__global__ void g_idx_kernel(const int32_t* perm, int64_t n, int g, int32_t* g_idx) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < n) g_idx[perm ? perm[k] : k] = (int32_t)(k / g);
}

// Per-row ||W - What||^2 and sum of err^2 (fp64, fixed order).
template <typename T>
__global__ void row_stats_kernel(const T* __restrict__ W, int64_t ldw, int64_t out, int64_t n,
                                 const int8_t* __restrict__ codes, const float* __restrict__ scales,
                                 const int8_t* __restrict__ zeros,
                                 int64_t ngroups, const int32_t* __restrict__ perm, const float* __restrict__ err2,
                                 int64_t nblocks, int g, double* __restrict__ row_out) {
    // one workgroup per row; position of column c in processing order is needed for
    // its group: pos[c] is not stored, so walk processing order k and read W[perm[k]]
    const int64_t r = blockIdx.x;
    __shared__ double red[2][256];
    double dw = 0.0, ee = 0.0;
    for (int64_t k = threadIdx.x; k < n; k += 256) {
        const int64_t c = perm ? perm[k] : k;
        const float z = zeros ? (float)zeros[r * ngroups + k / g] : 0.f;
        const float wh = ((float)codes[r * n + c] - z) * scales[r * ngroups + k / g];
        const double dv = (double)load_as_float<T>(W, r * ldw + c) - (double)wh;
        dw += dv * dv;
    }
    for (int64_t b = threadIdx.x; b < nblocks; b += 256) ee += (double)err2[r * nblocks + b];
    red[0][threadIdx.x] = dw;
    red[1][threadIdx.x] = ee;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            red[0][threadIdx.x] += red[0][threadIdx.x + w];
            red[1][threadIdx.x] += red[1][threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        row_out[2 * r] = red[1][0];
        row_out[2 * r + 1] = red[0][0];
    }
}

__global__ void sum_rows_kernel(const double* row_out, int64_t out, double* tot) {
    __shared__ double red[2][256];
    double a = 0.0, b = 0.0;
    for (int64_t r = threadIdx.x; r < out; r += 256) {
        a += row_out[2 * r];
        b += row_out[2 * r + 1];
    }
    red[0][threadIdx.x] = a;
    red[1][threadIdx.x] = b;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            red[0][threadIdx.x] += red[0][threadIdx.x + w];
            red[1][threadIdx.x] += red[1][threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        tot[0] = red[0][0];
        tot[1] = red[1][0];
    }
}

__global__ void zero_int_kernel(int* p) { *p = 0; }

// Trailing updates with at least this many rows and columns run on the bf16
// MFMA from three-term bf16 splits of E and U's rows (fp32 accuracy,
// gemm_bf16.hip); smaller ones on the fp32 MFMA GEMM.
constexpr int64_t TRAIL_SPLIT3_MIN = 2048;
// Mid-blocks of the three-level lazy batch: inside a super-block, a block's
// errors update only the rest of its mid-block (depth B); at each mid-block's
// end its errors update the rest of the super-block at depth MID_COLS. On the
// down_proj shape the column stage takes about 1.3 ms less than with two
// levels (256- and 1024-column mid-blocks: 0.5 ms more than 512; the
// mid-block updates on the split-operand GEMM: no faster than on fp32).
constexpr int64_t MID_COLS = 512;

template <int B, bool ZP>
int run_blocks(float* Wc, int64_t out, int64_t n, const float* U, int g, float qmax, const int32_t* perm,
               int8_t* codes, float* scales, int8_t* zeros, int64_t ngroups, float* gmaxes, float* E, float* err2,
               int64_t nblocks, int* flag, uint16_t* Pa, uint16_t* Pb, hipStream_t st) {
    constexpr int RPW = NTH / (B / CPL);
    const unsigned grid = (unsigned)cdiv(out, RPW);
    // W_cur[:, c1:] -= Err[:, 0:K] U[k0:k0+K, c1:c2]
    // Three levels of lazy batching: inside a mid-block of MB columns each
    // block's errors update only the rest of the mid-block; at a mid-block's
    // end its errors update the rest of its super-block of SB columns; the
    // columns past a super-block receive all of its errors in one GEMM with
    // K = SB (the same sums, regrouped). A group that spans blocks must not
    // straddle a super-block or a mid-block (its scale reads columns ahead), so
    // such group sizes that do not divide SB_COLS fall back to single blocks,
    // and those that do not divide MID_COLS to two levels.
    const int64_t SB = (g > B && SB_COLS % g != 0) ? B : SB_COLS;
    // the same for mid-blocks (without them: two levels)
    const int64_t MB = (g > B && MID_COLS % g != 0) ? SB : std::min<int64_t>(MID_COLS, SB);
    auto update = [&](int64_t k0, int64_t K, int64_t c1, int64_t c2, int kernel) {
        GemmArgs a{};
        a.M = out; a.N = c2 - c1; a.K = K;
        a.A = E + (k0 % SB); a.lda = SB; a.layout_a = A_MK;
        a.B = U + k0 * n + c1; a.ldb = n; a.layout_b = B_KN;
        a.C = Wc + c1; a.ldc = n;
        a.alpha = -1.f; a.beta_one = 1; a.tri = TRI_NONE; a.upper_only = 0;
        const bool split = Pa && kernel == PROF_TRAIL_GEMM && a.M >= TRAIL_SPLIT3_MIN && a.N >= TRAIL_SPLIT3_MIN;
        prof_begin(kernel, st);
        const int s = split ? launch_gemm_f32_split3(a, Pa, Pb, st) : launch_gemm_f32(a, st);
        prof_end(kernel, st);
        return s;
    };
    for (int64_t s0 = 0; s0 < n; s0 += SB) {
        const int64_t s1 = std::min<int64_t>(n, s0 + SB);
        for (int64_t m0 = s0; m0 < s1; m0 += MB) {
            const int64_t m1 = std::min<int64_t>(s1, m0 + MB);
            for (int64_t b0 = m0; b0 < m1; b0 += B) {
                const int bc = (int)std::min<int64_t>(B, m1 - b0);
                prof_begin(PROF_BLOCK_LOOP, st);
                uint64_t gs[2] = {0, 0};   // group starts inside the block (groups of g <= B)
                if (g <= B)
                    for (int j = 0; j < bc; j += g) gs[j >> 6] |= (uint64_t)1 << (j & 63);
                hipLaunchKernelGGL((gptq_block_kernel<B, ZP>), dim3(grid), dim3(NTH), 0, st, Wc, out, n, U, b0, bc,
                                   g, qmax, perm, codes, scales, zeros, ngroups, gmaxes, E + (b0 - s0), (int)SB,
                                   err2, nblocks, flag, gs[0], gs[1]);
                prof_end(PROF_BLOCK_LOOP, st);
                PTQ_LAUNCH_CHECK();
                const int64_t b1 = b0 + bc;
                if (b1 < m1) PTQ_TRY(update(b0, bc, b1, m1, PROF_INNER_GEMM));
            }
            if (m1 < s1) PTQ_TRY(update(m0, m1 - m0, m1, s1, PROF_INNER_GEMM));
        }
        if (s1 < n) PTQ_TRY(update(s0, s1 - s0, s1, n, PROF_TRAIL_GEMM));
    }
    return PTQ_OK;
}

}  // namespace

size_t columns_workspace_bytes(int64_t out, int64_t n, int block) {
    Sizer z;
    const int64_t nblocks = cdiv(n, block);
    z.take<float>((size_t)out * n);          // Wc
    z.take<float>((size_t)out * SB_COLS);    // E (errors of one super-block)
    z.take<float>((size_t)out * nblocks);    // err2
    z.take<float>((size_t)out * 2 * cdiv(n, 8)); // group range ends (groups of >= 8 columns)
    z.take<double>((size_t)out * 2);         // per-row stats
    z.take<double>(2);                       // totals
    z.take<int>(1);                          // flag
    if (out >= TRAIL_SPLIT3_MIN && n >= TRAIL_SPLIT3_MIN) {   // split planes of E and of U's rows
        z.take<uint16_t>(gemm_f32_split3_elems(out, SB_COLS));
        z.take<uint16_t>(gemm_f32_split3_elems(n, SB_COLS));
    }
    return z.bytes();
}

int run_quantize_columns(const void* W, int w_dtype, int64_t out, int64_t n, int64_t ldw, const float* U,
                         const int32_t* perm, int bits, int g, int block, int8_t* codes, float* scales,
                         int8_t* zeros, int32_t* g_idx, double* stats_host, void* ws, size_t ws_bytes,
                         hipStream_t st) {
    Arena ar(ws, ws_bytes);
    const int64_t nblocks = cdiv(n, block);
    const int64_t ngroups = cdiv(n, g);
    float* Wc = ar.take<float>((size_t)out * n);
    float* E = ar.take<float>((size_t)out * SB_COLS);
    float* err2 = ar.take<float>((size_t)out * nblocks);
    float* gmaxes = ar.take<float>((size_t)out * 2 * cdiv(n, 8));
    double* rowst = ar.take<double>((size_t)out * 2);
    double* tot = ar.take<double>(2);
    int* flag = ar.take<int>(1);
    const bool split = out >= TRAIL_SPLIT3_MIN && n >= TRAIL_SPLIT3_MIN;
    uint16_t* Pa = split ? ar.take<uint16_t>(gemm_f32_split3_elems(out, SB_COLS)) : nullptr;
    uint16_t* Pb = split ? ar.take<uint16_t>(gemm_f32_split3_elems(n, SB_COLS)) : nullptr;
    if (!Wc || !E || !err2 || !gmaxes || !rowst || !tot || !flag || (split && (!Pa || !Pb))) {
        set_error("gptq_quantize_columns: workspace of %zu bytes, %zu needed", ws_bytes,
                  columns_workspace_bytes(out, n, block));
        return PTQ_EWORKSPACE;
    }
    // symmetric: qmax = 2^(bits-1) - 1; zero-point: maxq = 2^bits - 1
    const float qmax = zeros ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
    hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, st, flag);
    PTQ_LAUNCH_CHECK();
    if (out > 0) {
        dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)out);
        if (w_dtype == PTQ_BF16 && !perm && n % 8 == 0 && ldw % 8 == 0 && ((uintptr_t)W & 15u) == 0)
            hipLaunchKernelGGL(widen_rows_bf16_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n / 8, 256), 64), (unsigned)out),
                               dim3(256), 0, st, (const uint16_t*)W, ldw, n, Wc);
        else if (w_dtype == PTQ_BF16)
            hipLaunchKernelGGL(gather_columns_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)W, ldw, out,
                               n, perm, Wc);
        else
            hipLaunchKernelGGL(gather_columns_kernel<float>, grid, dim3(256), 0, st, (const float*)W, ldw, out, n,
                               perm, Wc);
        PTQ_LAUNCH_CHECK();
        auto blocks = [&](auto zp) {
            constexpr bool Z = decltype(zp)::value;
            if (block == 128)
                return run_blocks<128, Z>(Wc, out, n, U, g, qmax, perm, codes, scales, zeros, ngroups, gmaxes, E, err2,
                                          nblocks, flag, Pa, Pb, st);
            if (block == 64)
                return run_blocks<64, Z>(Wc, out, n, U, g, qmax, perm, codes, scales, zeros, ngroups, gmaxes, E, err2,
                                         nblocks, flag, Pa, Pb, st);
            return run_blocks<32, Z>(Wc, out, n, U, g, qmax, perm, codes, scales, zeros, ngroups, gmaxes, E, err2,
                                     nblocks, flag, Pa, Pb, st);
        };
        if (zeros) PTQ_TRY(blocks(std::true_type{}));
        else PTQ_TRY(blocks(std::false_type{}));
    }

    if (g_idx) {
        hipLaunchKernelGGL(g_idx_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, perm, n, g, g_idx);
        PTQ_LAUNCH_CHECK();
    }
    if (stats_host && out == 0) {
        stats_host[0] = 0.0;
        stats_host[2] = 0.0;
    } else if (stats_host) {
        if (w_dtype == PTQ_BF16)
            hipLaunchKernelGGL(row_stats_kernel<uint16_t>, dim3((unsigned)out), dim3(256), 0, st, (const uint16_t*)W,
                               ldw, out, n, codes, scales, zeros, ngroups, perm, err2, nblocks, g, rowst);
        else
            hipLaunchKernelGGL(row_stats_kernel<float>, dim3((unsigned)out), dim3(256), 0, st, (const float*)W, ldw,
                               out, n, codes, scales, zeros, ngroups, perm, err2, nblocks, g, rowst);
        PTQ_LAUNCH_CHECK();
        hipLaunchKernelGGL(sum_rows_kernel, dim3(1), dim3(256), 0, st, rowst, out, tot);
        PTQ_LAUNCH_CHECK();
        double h[2];
        int fl = 0;
        PTQ_HIP(hipMemcpyAsync(h, tot, sizeof(h), hipMemcpyDeviceToHost, st));
        PTQ_HIP(hipMemcpyAsync(&fl, flag, sizeof(int), hipMemcpyDeviceToHost, st));
        PTQ_HIP(hipStreamSynchronize(st));
        stats_host[0] = h[0];
        stats_host[2] = h[1];
        if (fl) {
            set_error("gptq_quantize_columns: non-finite error term (NaN/Inf in W or U)");
            return PTQ_ENONFINITE;
        }
    }
    return PTQ_OK;
}

}  // namespace ptq
