// kda_ops.hip -- the two operations next to KDA in its layer, forward and
// backward: the short causal depthwise convolution before it and the gated
// output RMS norm after it.  Both are streaming, HBM-bound kernels.
//
// Short convolution ("Pure KDA 300M on Primus" guide, Overview: kernel size 4,
// depthwise, on the concatenated q/k/v channels; Troubleshooting: [B, T, D]
// is the native layout; torchtitan PR #4347, description: with document
// offsets the window resets at every document start):
//   z[t, c] = sum_{i < W} w[c, i] x[t - (W-1) + i, c]   (same document only)
//             + bias[c];        y = z, or SiLU(z) with KDA_CONV_SILU.
// Thread (channel group of 8, 4 in the backward; run of kConvRun tokens): the window of the last
// W inputs (and, in the backward, of the last W dz values) slides through the
// run in registers, so each input row is read once plus a W - 1 row halo.
// Loads are 16 bytes per lane (8 in the backward) along the channel axis (coalesced token rows).
// The backward forms dz = dy * act'(z) on the fly; dx is the anti-causal
// correlation of dz with w; dw and dbias are summed per run, then over the
// runs of a workgroup in LDS, then over the workgroups by a fixed tree
// (deterministic, no atomics).
//
// Gated norm (openkimi README, Profiling and H100 acceptance: the KDA output
// uses a fused RMSNorm plus a sigmoid gate; Primus guide, Overview: RMSNorm
// eps 1e-6, per-head output gate):
//   per row of dv values (one token and head): r = (mean(o^2) + eps)^{-1/2},
//   y = o r * weight * sigmoid(gate).
// dv / 8 consecutive lanes own a row (8 values each); the row sums are DPP
// reductions within those lanes.  dweight is summed like dw above.
#include "../../include/kda.h"
#include "kda_device.cuh"
#include "kda_internal.h"

namespace kda {

constexpr int kOpsThreads = 256;
constexpr int kConvRun = 16;          // tokens per thread
constexpr int kConvCG = 32;           // channel groups (of 8) per workgroup
constexpr int kConvRuns = kOpsThreads / kConvCG;  // runs per workgroup
constexpr int kBwdCPT = 4;            // channels per thread in the backward (8 in the forward): its
                                      // windows of x and dz and its dw partials then fit four waves per SIMD

__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }
__device__ __forceinline__ float dsilu_f(float z) {
    const float s = sigmoid_f(z);
    return s * (1.f + z * (1.f - s));
}

// Document index of position p (monotone queries): -1 outside [0, T).
struct DocCursor {
    const int32_t* cu;
    int T, d, de;
    __device__ __forceinline__ void start(const int32_t* cu_, int N, int T_, int p) {
        cu = cu_;
        T = T_;
        d = 0;
        de = T_;
        if (cu && p > 0) {
            // the last document with cu[d] <= p (binary search; empty documents skipped by the loop in at())
            int lo = 0, hi = N - 1;
            const int q = p < T_ ? p : T_ - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (cu[mid] <= q) lo = mid;
                else hi = mid - 1;
            }
            d = lo;
        }
        if (cu) de = cu[d + 1];
    }
    __device__ __forceinline__ int at(int p) {
        if (p < 0 || p >= T) return -1;
        if (cu) {
            while (p >= de) {
                ++d;
                de = cu[d + 1];
            }
        }
        return d;
    }
};

// ============================================================== convolution
template <int W, typename TIn, typename TOut, bool SILU>
__global__ void __launch_bounds__(kOpsThreads) conv_fwd_kernel(ConvArgs a) {
    const int cg = blockIdx.x * kConvCG + (threadIdx.x % kConvCG);
    const int run = blockIdx.y * kConvRuns + threadIdx.x / kConvCG;
    const int rpr = (a.T + kConvRun - 1) / kConvRun;  // runs per row
    if (cg * 8 >= a.D || run >= a.B * rpr) return;
    const int b = run / rpr, t0 = (run % rpr) * kConvRun;
    const int c0 = cg * 8;
    const TIn* x = (const TIn*)a.x + (size_t)b * a.T * a.D + c0;
    TOut* y = (TOut*)a.y + (size_t)b * a.T * a.D + c0;
    float w[W][8], bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int i = 0; i < W; ++i) w[i][j] = a.w[(size_t)(c0 + j) * W + i];
        bias[j] = a.bias ? a.bias[c0 + j] : 0.f;
    }
    float xw[W][8];
    int xd[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
        xd[i] = -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[i][j] = 0.f;
    }
    DocCursor dc;
    dc.start(a.cu, a.N, a.T, t0 - (W - 1));
#pragma unroll
    for (int k = 0; k < kConvRun + W - 1; ++k) {
        const int p = t0 - (W - 1) + k;
        const int dp = dc.at(p);
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            xd[i] = xd[i + 1];
#pragma unroll
            for (int j = 0; j < 8; ++j) xw[i][j] = xw[i + 1][j];
        }
        xd[W - 1] = dp;
        if (dp >= 0) load8<TIn>(x + (size_t)p * a.D, xw[W - 1]);
        if (k >= W - 1 && dp >= 0) {
            float z[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) z[j] = bias[j];
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const bool same = xd[i] == dp;
#pragma unroll
                for (int j = 0; j < 8; ++j) z[j] = fmaf(w[i][j], same ? xw[i][j] : 0.f, z[j]);
            }
            if (SILU) {
#pragma unroll
                for (int j = 0; j < 8; ++j) z[j] = silu_f(z[j]);
            }
            store8<TOut>(y + (size_t)p * a.D, z);
        }
    }
}

template <int W, typename TIn, typename TOut, bool SILU>
__global__ void __launch_bounds__(kOpsThreads) conv_bwd_kernel(ConvArgs a) {
    __shared__ float red[kConvRuns][kConvCG][(W + 1) * kBwdCPT + 1];
    const int cl = threadIdx.x % kConvCG, rl = threadIdx.x / kConvCG;
    const int cg = blockIdx.x * kConvCG + cl;
    const int run = blockIdx.y * kConvRuns + rl;
    const int rpr = (a.T + kConvRun - 1) / kConvRun;
    const bool active = cg * kBwdCPT < a.D && run < a.B * rpr;
    float dwp[W][kBwdCPT], dbp[kBwdCPT];
#pragma unroll
    for (int j = 0; j < kBwdCPT; ++j) {
        dbp[j] = 0.f;
#pragma unroll
        for (int i = 0; i < W; ++i) dwp[i][j] = 0.f;
    }
    if (active) {
        const int b = run / rpr, t0 = (run % rpr) * kConvRun;
        const int t1 = t0 + kConvRun < a.T ? t0 + kConvRun : a.T;
        const int c0 = cg * kBwdCPT;
        const size_t rowoff = (size_t)b * a.T * a.D + c0;
        const TIn* x = (const TIn*)a.x + rowoff;
        const TIn* dy = (const TIn*)a.dy + rowoff;
        TOut* dx = (TOut*)a.dx + rowoff;
        float w[W][kBwdCPT], bias[kBwdCPT];
#pragma unroll
        for (int j = 0; j < kBwdCPT; ++j) {
#pragma unroll
            for (int i = 0; i < W; ++i) w[i][j] = a.w[(size_t)(c0 + j) * W + i];
            bias[j] = a.bias ? a.bias[c0 + j] : 0.f;
        }
        // windows over positions p - (W-1) .. p: inputs (with their documents) and dz
        float xw[W][kBwdCPT], zw[W][kBwdCPT];
        int xd[W];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            xd[i] = -1;
#pragma unroll
            for (int j = 0; j < kBwdCPT; ++j) xw[i][j] = zw[i][j] = 0.f;
        }
        DocCursor dc;
        dc.start(a.cu, a.N, a.T, t0 - (W - 1));
#pragma unroll
        for (int k = 0; k < kConvRun + 2 * (W - 1); ++k) {
            const int p = t0 - (W - 1) + k;
            const int dp = dc.at(p);
#pragma unroll
            for (int i = 0; i < W - 1; ++i) {
                xd[i] = xd[i + 1];
#pragma unroll
                for (int j = 0; j < kBwdCPT; ++j) {
                    xw[i][j] = xw[i + 1][j];
                    zw[i][j] = zw[i + 1][j];
                }
            }
            xd[W - 1] = dp;
            if (dp >= 0) load4<TIn>(x + (size_t)p * a.D, xw[W - 1]);
            // dz at p, for p in [t0, t1 + W - 1): the window then holds x[p - (W-1) .. p]
            float dz[kBwdCPT] = {};
            if (k >= W - 1 && dp >= 0 && p < t1 + W - 1) {
                load4<TIn>(dy + (size_t)p * a.D, dz);
                if (SILU) {
                    float z[kBwdCPT];
#pragma unroll
                    for (int j = 0; j < kBwdCPT; ++j) z[j] = bias[j];
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const bool same = xd[i] == dp;
#pragma unroll
                        for (int j = 0; j < kBwdCPT; ++j) z[j] = fmaf(w[i][j], same ? xw[i][j] : 0.f, z[j]);
                    }
#pragma unroll
                    for (int j = 0; j < kBwdCPT; ++j) dz[j] *= dsilu_f(z[j]);
                }
                if (p < t1) {  // this run's own positions: dw and dbias
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const bool same = xd[i] == dp;
#pragma unroll
                        for (int j = 0; j < kBwdCPT; ++j) dwp[i][j] = fmaf(dz[j], same ? xw[i][j] : 0.f, dwp[i][j]);
                    }
#pragma unroll
                    for (int j = 0; j < kBwdCPT; ++j) dbp[j] += dz[j];
                }
            }
#pragma unroll
            for (int j = 0; j < kBwdCPT; ++j) zw[W - 1][j] = dz[j];
            // dx at s = p - (W-1): sum_i w[i] dz[s + lag_i], lag_i = W-1-i, same document as s
            const int s = p - (W - 1);
            if (s >= t0 && s < t1 && xd[0] >= 0) {
                float g[kBwdCPT] = {};
#pragma unroll
                for (int i = 0; i < W; ++i) {
                    const bool same = xd[W - 1 - i] == xd[0];
#pragma unroll
                    for (int j = 0; j < kBwdCPT; ++j) g[j] = fmaf(w[i][j], same ? zw[W - 1 - i][j] : 0.f, g[j]);
                }
                store4<TOut>(dx + (size_t)s * a.D, g);
            }
        }
    }
    // dw, dbias: this workgroup's runs in LDS, summed in a fixed order
#pragma unroll
    for (int j = 0; j < kBwdCPT; ++j) {
#pragma unroll
        for (int i = 0; i < W; ++i) red[rl][cl][i * kBwdCPT + j] = dwp[i][j];
        red[rl][cl][W * kBwdCPT + j] = dbp[j];
    }
    __syncthreads();
    constexpr int NV = kConvCG * (W + 1) * kBwdCPT;  // partial values of this workgroup
    for (int e = threadIdx.x; e < NV; e += kOpsThreads) {
        const int c = e / ((W + 1) * kBwdCPT), v = e % ((W + 1) * kBwdCPT);
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < kConvRuns; ++r) s += red[r][c][v];
        const int ch = (blockIdx.x * kConvCG + c) * kBwdCPT + v % kBwdCPT;
        if (ch < a.D) {
            const int i = v / kBwdCPT;  // tap, or W for the bias
            a.part[((size_t)blockIdx.y * a.D + ch) * (W + 1) + i] = s;
        }
    }
}

// sum over k < nblk of part[k * M + e], by a whole workgroup: thread t adds
// k = t, t + 256, ... in order, then a fixed tree over the threads, so the
// result does not depend on scheduling.  Every thread gets the sum.
__device__ __forceinline__ float block_col_sum(const float* __restrict__ part, int nblk, int M, int e) {
    __shared__ float red[kOpsThreads];
    float s = 0.f;
    for (int k = threadIdx.x; k < nblk; k += kOpsThreads) s += part[(size_t)k * M + e];
    red[threadIdx.x] = s;
    __syncthreads();
#pragma unroll
    for (int off = kOpsThreads / 2; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    return red[0];
}

// dw[c][i] and dbias[c] (i == W): one workgroup per value, over the row blocks' partials.
template <int W>
__global__ void __launch_bounds__(kOpsThreads) conv_wsum_kernel(ConvArgs a, int nblk) {
    const int e = blockIdx.x;  // < D * (W + 1)
    const float s = block_col_sum(a.part, nblk, a.D * (W + 1), e);
    if (threadIdx.x == 0) {
        const int c = e / (W + 1), i = e % (W + 1);
        if (i < W) a.dw[c * W + i] = s;
        else if (a.dbias) a.dbias[c] = s;
    }
}

size_t conv_bwd_workspace(int B, int T, int D) {
    const int rpr = (T + kConvRun - 1) / kConvRun;
    const size_t nblk = ((size_t)B * rpr + kConvRuns - 1) / kConvRuns;
    return nblk * D * 5 * sizeof(float);  // W <= 4 taps + bias per channel and row block
}

template <int W, typename TIn, typename TOut, bool SILU>
static hipError_t conv_launch(const ConvArgs& a, bool backward, hipStream_t s) {
    const int rpr = (a.T + kConvRun - 1) / kConvRun;
    const dim3 grid((a.D / 8 + kConvCG - 1) / kConvCG, (a.B * rpr + kConvRuns - 1) / kConvRuns);
    if (grid.y == 0) {  // no tokens: nothing to convolve; the weight gradients are zero
        if (backward)
            KDA_LAUNCH("conv_wsum", (conv_wsum_kernel<W>), dim3(a.D * (W + 1)), dim3(kOpsThreads), s, a, 0);
        return hipSuccess;
    }
    if (!backward) {
        KDA_LAUNCH("conv_fwd", (conv_fwd_kernel<W, TIn, TOut, SILU>), grid, dim3(kOpsThreads), s, a);
        return hipSuccess;
    }
    const dim3 gridb((a.D / kBwdCPT + kConvCG - 1) / kConvCG, grid.y);
    KDA_LAUNCH("conv_bwd", (conv_bwd_kernel<W, TIn, TOut, SILU>), gridb, dim3(kOpsThreads), s, a);
    KDA_LAUNCH("conv_wsum", (conv_wsum_kernel<W>), dim3(a.D * (W + 1)), dim3(kOpsThreads), s, a, (int)grid.y);
    return hipSuccess;
}

template <int W>
static hipError_t conv_dispatch_w(const ConvArgs& a, bool backward, hipStream_t s) {
    if (a.in_bf16) {
        if (a.out_bf16)
            return a.silu ? conv_launch<W, uint16_t, uint16_t, true>(a, backward, s)
                          : conv_launch<W, uint16_t, uint16_t, false>(a, backward, s);
        return a.silu ? conv_launch<W, uint16_t, float, true>(a, backward, s)
                      : conv_launch<W, uint16_t, float, false>(a, backward, s);
    }
    if (a.out_bf16)
        return a.silu ? conv_launch<W, float, uint16_t, true>(a, backward, s)
                      : conv_launch<W, float, uint16_t, false>(a, backward, s);
    return a.silu ? conv_launch<W, float, float, true>(a, backward, s) : conv_launch<W, float, float, false>(a, backward, s);
}

hipError_t launch_conv(const ConvArgs& a, bool backward, hipStream_t s) {
    switch (a.W) {
        case 1: return conv_dispatch_w<1>(a, backward, s);
        case 2: return conv_dispatch_w<2>(a, backward, s);
        case 3: return conv_dispatch_w<3>(a, backward, s);
        case 4: return conv_dispatch_w<4>(a, backward, s);
        default: return hipErrorInvalidValue;
    }
}

// ============================================================== gated norm
constexpr int kGnPasses = 8;  // row groups per workgroup

template <int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kOpsThreads) gnorm_fwd_kernel(GnormArgs a) {
    constexpr int TPR = DV / 8, RPP = kOpsThreads / TPR;  // threads per row, rows per pass
    const int part = threadIdx.x % TPR;
    float wt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wt[j] = a.weight[8 * part + j];
#pragma unroll 2
    for (int ps = 0; ps < kGnPasses; ++ps) {
        const int64_t row = ((int64_t)blockIdx.x * kGnPasses + ps) * RPP + threadIdx.x / TPR;
        const bool in = row < a.rows;
        const size_t off = (size_t)(in ? row : 0) * DV + 8 * part;
        float o[8], g[8];
        load8<TIn>((const TIn*)a.o + off, o);
        load8<TIn>((const TIn*)a.gate + off, g);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(o[j], o[j], ss);
        ss = row_group_sum<TPR>(ss);
        const float r = 1.0f / sqrtf(ss * (1.0f / DV) + a.eps);
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = o[j] * r * wt[j] * sigmoid_f(g[j]);
        if (in) store8<TOut>((TOut*)a.y + off, y);
    }
}

template <int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kOpsThreads) gnorm_bwd_kernel(GnormArgs a) {
    constexpr int TPR = DV / 8, RPP = kOpsThreads / TPR;
    __shared__ float red[kOpsThreads / 64][DV];
    const int part = threadIdx.x % TPR;
    float wt[8], dwp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        wt[j] = a.weight[8 * part + j];
        dwp[j] = 0.f;
    }
#pragma unroll 2
    for (int ps = 0; ps < kGnPasses; ++ps) {
        const int64_t row = ((int64_t)blockIdx.x * kGnPasses + ps) * RPP + threadIdx.x / TPR;
        const bool in = row < a.rows;
        const size_t off = (size_t)(in ? row : 0) * DV + 8 * part;
        float o[8], g[8], dy[8];
        load8<TIn>((const TIn*)a.o + off, o);
        load8<TIn>((const TIn*)a.gate + off, g);
        load8<TIn>((const TIn*)a.dy + off, dy);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(o[j], o[j], ss);
        ss = row_group_sum<TPR>(ss);
        const float r = 1.0f / sqrtf(ss * (1.0f / DV) + a.eps);
        float n[8], sg[8], dn[8], dgt[8], dot = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            n[j] = o[j] * r;
            sg[j] = sigmoid_f(g[j]);
            dn[j] = dy[j] * wt[j] * sg[j];
            dgt[j] = dn[j] * n[j] * (1.f - sg[j]);
            dot = fmaf(dn[j], n[j], dot);
            if (in) dwp[j] = fmaf(dy[j] * n[j], sg[j], dwp[j]);
        }
        dot = row_group_sum<TPR>(dot) * (1.0f / DV);
        float dox[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) dox[j] = r * (dn[j] - n[j] * dot);
        if (in) {
            store8<TOut>((TOut*)a.d_o + off, dox);
            store8<TOut>((TOut*)a.dgate + off, dgt);
        }
    }
    // dweight: over the rows of this wave (lanes with the same part), then over the waves
#pragma unroll
    for (int j = 0; j < 8; ++j) dwp[j] = rows_of_wave_sum<TPR>(dwp[j]);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane < TPR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wave][8 * lane + j] = dwp[j];
    }
    __syncthreads();
    if (threadIdx.x < DV) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kOpsThreads / 64; ++w) s += red[w][threadIdx.x];
        a.part[(size_t)blockIdx.x * DV + threadIdx.x] = s;
    }
}

// dweight[c]: one workgroup per channel, over the workgroups' partials.
__global__ void __launch_bounds__(kOpsThreads) gnorm_wsum_kernel(GnormArgs a, int nblk) {
    const int c = blockIdx.x;  // < dv
    const float s = block_col_sum(a.part, nblk, a.dv, c);
    if (threadIdx.x == 0) a.dweight[c] = s;
}

static int gnorm_blocks(int64_t rows, int dv) {
    const int64_t rpb = (int64_t)kGnPasses * (kOpsThreads / (dv / 8));
    return (int)((rows + rpb - 1) / rpb);
}

size_t gnorm_bwd_workspace(int64_t rows, int dv) { return (size_t)gnorm_blocks(rows, dv) * dv * sizeof(float); }

template <int DV, typename TIn, typename TOut>
static hipError_t gnorm_launch(const GnormArgs& a, bool backward, hipStream_t s) {
    const int nblk = gnorm_blocks(a.rows, DV);
    if (nblk == 0) {  // no rows: the weight gradient is zero
        if (backward) KDA_LAUNCH("gnorm_wsum", gnorm_wsum_kernel, dim3(DV), dim3(kOpsThreads), s, a, 0);
        return hipSuccess;
    }
    if (!backward) {
        KDA_LAUNCH("gnorm_fwd", (gnorm_fwd_kernel<DV, TIn, TOut>), dim3(nblk), dim3(kOpsThreads), s, a);
        return hipSuccess;
    }
    KDA_LAUNCH("gnorm_bwd", (gnorm_bwd_kernel<DV, TIn, TOut>), dim3(nblk), dim3(kOpsThreads), s, a);
    KDA_LAUNCH("gnorm_wsum", gnorm_wsum_kernel, dim3(DV), dim3(kOpsThreads), s, a, nblk);
    return hipSuccess;
}

template <int DV>
static hipError_t gnorm_dispatch(const GnormArgs& a, bool backward, hipStream_t s) {
    if (a.in_bf16)
        return a.out_bf16 ? gnorm_launch<DV, uint16_t, uint16_t>(a, backward, s)
                          : gnorm_launch<DV, uint16_t, float>(a, backward, s);
    return a.out_bf16 ? gnorm_launch<DV, float, uint16_t>(a, backward, s) : gnorm_launch<DV, float, float>(a, backward, s);
}

hipError_t launch_gnorm(const GnormArgs& a, bool backward, hipStream_t s) {
    switch (a.dv) {
        case 32: return gnorm_dispatch<32>(a, backward, s);
        case 64: return gnorm_dispatch<64>(a, backward, s);
        case 128: return gnorm_dispatch<128>(a, backward, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
