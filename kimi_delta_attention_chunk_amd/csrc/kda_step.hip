// kda_step.hip -- one-token recurrent decode (memory-bound).
//
// One iteration of the per-channel-gated delta rule on a caller-held fp32
// state (Primus guide, Overview: delta-rule recurrence with a decay gate;
// openkimi README, What is implemented: fp32 recurrent state):
//   a = exp(g); S' = Diag(a) S; r = v - S'^T k; S = S' + beta k r^T; o = scale S^T q.
//
// One workgroup per (sequence, head).  Thread (rg, j) owns column j of the
// state and the rows rg*RPT .. rg*RPT+RPT-1, so for a fixed row the 64-wide
// wave reads consecutive columns (coalesced 256-byte rows of the fp32 state).
// The state loads are issued first, so they overlap the staging of q, k and
// the decay; the two column sums (S'^T k and S^T q) are reduced across row
// groups in LDS (three barriers per step).
#include "kda_device.cuh"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads) step_kernel(
    int BH, int H, float scale, uint32_t flags, const TIn* __restrict__ q,
    const TIn* __restrict__ k, const TIn* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, float* __restrict__ h, TOut* __restrict__ o) {
    static_assert(kThreads % DV == 0, "DV must divide the workgroup");
    constexpr int RG = kThreads / DV;  // row groups
    static_assert(DK % RG == 0, "DK must split over the row groups");
    constexpr int RPT = DK / RG;       // rows per thread
    static_assert(DK <= kThreads, "one thread per key channel");

    const int bh = blockIdx.x;
    if (bh >= BH) return;
    const int head = bh % H;
    const int tid = threadIdx.x;
    const int j = tid % DV, rg = tid / DV;

    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ float s_p[RG][DV], s_o[RG][DV];
    __shared__ float s_norm[2][kThreads / 64];

    // this thread's state entries, first
    float* hs = h + (size_t)bh * DK * DV;
    float S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = hs[(rg * RPT + i) * DV + j];
    const float vj = Elem<TIn>::load(v, (size_t)bh * DV + j);
    float b = beta[bh];
    if (flags & 4u) b = sigmoid_f(b);

    // q, k and the decay of this (sequence, head): thread c < DK holds channel c
    float qc = 0.f, kc = 0.f, ac = 0.f;
    if (tid < DK) {
        const size_t base = (size_t)bh * DK + tid;
        qc = Elem<TIn>::load(q, base);
        kc = Elem<TIn>::load(k, base);
        float gg = g[base];
        if (flags & 2u) gg = -expf(A_log[head]) * softplus_f(gg + dt_bias[head * DK + tid]);
        ac = expf(gg);
    }
    if (flags & 1u) {
        // L2 norms of q and k over the DK channels (whole waves; lanes past DK hold 0)
        const float sq = wave_sum(qc * qc), sk = wave_sum(kc * kc);
        float tq = sq, tk = sk;
        if constexpr (DK > 64) {
            if ((tid & 63) == 0) { s_norm[0][tid >> 6] = sq; s_norm[1][tid >> 6] = sk; }
            __syncthreads();
            tq = 0.f;
            tk = 0.f;
#pragma unroll
            for (int w = 0; w < DK / 64; ++w) { tq += s_norm[0][w]; tk += s_norm[1][w]; }
        }
        qc *= 1.0f / sqrtf(tq + kL2Eps);
        kc *= 1.0f / sqrtf(tk + kL2Eps);
    }
    if (tid < DK) { s_q[tid] = qc; s_k[tid] = kc; s_a[tid] = ac; }
    __syncthreads();

    // decay, prediction p_j = (S'^T k)_j
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg * RPT + i;
        S[i] *= s_a[c];
        p = fmaf(S[i], s_k[c], p);
    }
    s_p[rg][j] = p;
    __syncthreads();
    float pj = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) pj += s_p[r][j];
    const float rj = b * (vj - pj);
    // delta-rule write, then the output read o_j = scale (S^T q)_j
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg * RPT + i;
        S[i] = fmaf(s_k[c], rj, S[i]);
        hs[c * DV + j] = S[i];
        acc = fmaf(S[i], s_q[c], acc);
    }
    s_o[rg][j] = acc;
    __syncthreads();
    if (rg == 0) {
        float oj = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) oj += s_o[r][j];
        Elem<TOut>::store(o, (size_t)bh * DV + j, scale * oj);
    }
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t s) {
    KDA_LAUNCH("step", (step_kernel<DK, DV, TIn, TOut>), dim3(a.B * a.H), dim3(kThreads), s,
               a.B * a.H, a.H, a.scale, a.flags, (const TIn*)a.q, (const TIn*)a.k,
                       (const TIn*)a.v, a.g, a.beta, a.A_log, a.dt_bias, a.h, (TOut*)a.o);
    return hipSuccess;
}

template <int DK, int DV>
static hipError_t launch_step_dims(const StepArgs& a, hipStream_t s) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_step_t<DK, DV, uint16_t, uint16_t>(a, s)
                          : launch_step_t<DK, DV, uint16_t, float>(a, s);
    return a.out_bf16 ? launch_step_t<DK, DV, float, uint16_t>(a, s)
                      : launch_step_t<DK, DV, float, float>(a, s);
}

hipError_t launch_step(const StepArgs& a, hipStream_t s) {
    if (a.dk == 32 && a.dv == 64) return launch_step_dims<32, 64>(a, s);
    if (a.dk == 64 && a.dv == 64) return launch_step_dims<64, 64>(a, s);
    if (a.dk == 128 && a.dv == 128) return launch_step_dims<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
