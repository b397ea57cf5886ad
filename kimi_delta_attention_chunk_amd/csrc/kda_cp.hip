// kda_cp.hip -- the building blocks of context parallelism (the maps for dk = 32
// here; for dk = dv >= 64 the forward state pass forms them, kda_scan.cuh): the
// affine map of a segment of chunks, and the short scan that chains segments.
//
// A chunk maps the state entering it to the state leaving it affinely,
// h' = P h + hh (kda_pscan.cuh), so a segment of chunks -- a rank's share of a
// long row, or any run of chunks -- does too: h_out = M h_in + c with
// M = P_last ... P_first (dk x dk) and c = the segment's final state from a
// zero entering state (kda_fwd's hT with h0 = 0).  Segments can therefore be
// computed independently and chained afterwards:
//   forward   h_in[0] = h0;  h_in[r+1] = M_r h_in[r] + c_r      (hT = h_out of the last)
//   backward  D[R-1] = dhT;  D[r-1] = M_r^T D[r] + e_r          (dh0 = M_0^T D[0] + e_0)
// where e_r is the gradient with respect to the segment's entering state from
// its own outputs (kda_bwd's dh0 with dhT = 0) and D[r] = dL/dh_out[r].  A
// second pass of each segment with its h_in (and D) then gives the same outputs
// and gradients as one pass over the whole row.
//
// seg_map_kernel: one workgroup of four waves per (segment, head); the 32 x 32
// product X = P X runs chunk after chunk from X = I with the same fragment
// scheme as the state pass (P's rows as register fragments from the intra
// kernel's fragment-form array, prefetched four chunks ahead; X^T in a
// double-buffered LDS tile, one barrier per chunk).
// state_scan_kernel: one workgroup per (head, 32 state columns); fp32 MFMA over
// the segments in order, M_r staged in LDS (transposed for the backward), the
// next segments' operands in flight while the current one is applied.
#include "../../include/kda.h"
#include "kda_chunk.cuh"
#include "kda_internal.h"
#include "kda_mma.cuh"
#include "kda_pscan.cuh"

namespace kda {

template <Prec P>
__global__ void __launch_bounds__(kPsThreads) seg_map_kernel(Prm p, float* __restrict__ M) {
    constexpr int DK = kPsDK, LK = DK + 8, PD = 4;
    __shared__ __attribute__((aligned(16))) float sX[2][DK * LK];
    static_assert(STile<Prec::F32, DK>::ld == LK, "tile footprint");
    const STile<P, DK> XT[2] = {STile<P, DK>(sX[0], DK), STile<P, DK>(sX[1], DK)};
    const int nh = blockIdx.x;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const int tc = wave >> 1, tj = wave & 1;  // this wave's 16x16 tile of X
    const int crow = 16 * tc + frag_row(0), jcol = 16 * tj + lr;
    f32x4 S;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[r] = crow + r == jcol ? 1.f : 0.f;
    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    auto slot_of = [&](int cc) { return (size_t)(cc < c1 ? cc : c1 - 1) * p.H + h; };
    auto load = [&](int cc, AFrag<P>& f) {
        load_afrag(f, frag_rec(p.pm + slot_of(cc) * DK * DK, 16 * tc + lr, 0, 1));
    };
    XT[0].put4(jcol, crow, S);
    if (c0 < c1) {
        AFrag<P> R[PD];
#pragma unroll
        for (int i = 0; i < PD; ++i) load(c0 + i, R[i]);
        auto step = [&](int buf, const AFrag<P>& pm) {
            __syncthreads();  // X^T of this chunk complete; the other buffer's readers are done
            AFrag<P> fb;
            load_frag(fb, XT[buf].sub(16 * tj), 0);
            S = mma_ff(pm, fb, f32x4{0.f, 0.f, 0.f, 0.f});
            XT[buf ^ 1].put4(jcol, crow, S);
        };
        int c = c0;
        for (; c + PD - 1 < c1; c += PD) {
#pragma unroll
            for (int i = 0; i < PD; ++i) {
                step(i & 1, R[i]);
                load(c + PD + i, R[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < PD - 1; ++i)
            if (c + i < c1) step(i & 1, R[i]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) M[((size_t)nh * DK + crow + r) * DK + jcol] = S[r];
}

// X <- A_r X + c_r over the segments (A_r = M_r, or M_r^T in reverse order for
// the backward); out[r] receives X before segment r's step.  The chain is
// latency-bound (R dependent steps of a small product): the 32 x 32 block of X
// is four 16x16 tiles held as fp32 MFMA accumulators, one per wave, and each
// step is eight v_mfma_f32_16x16x4_f32 on operands read from double-buffered
// LDS tiles (one barrier per segment), while the next four segments' A and c
// are in flight in registers.
template <int DK>
__global__ void __launch_bounds__(kThreads) state_scan_kernel(int R, int H, int DV, int transpose,
                                                              const float* __restrict__ M,
                                                              const float* __restrict__ c,
                                                              const float* __restrict__ x0, float* __restrict__ out,
                                                              float* __restrict__ xfinal) {
    constexpr int BV = 32, LX = BV + 4, LM = DK + 1;
    constexpr int MPT = DK * DK / kThreads;  // entries of A staged per thread
    static_assert(DK == 32 && kThreads == 256 && DK * DK % kThreads == 0, "four 16x16 tiles, one per wave");
    __shared__ __attribute__((aligned(16))) float sX[2][DK * LX];
    __shared__ float sA[2][DK * LM];
    const int h = blockIdx.x, jb = blockIdx.y * BV;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int tm = wave >> 1, tn = wave & 1;  // this wave's tile: rows 16 tm .., columns 16 tn ..
    const int lr = lane & 15, lg = lane >> 4;
    const int col = jb + 16 * tn + lr;         // this lane's column of X (D fragment)
    const int row0 = 16 * tm + 4 * lg;         // and its four rows row0 .. row0 + 3
    f32x4 X;
#pragma unroll
    for (int i = 0; i < 4; ++i) X[i] = x0 ? x0[((size_t)h * DK + row0 + i) * DV + col] : 0.f;
    // PD segments' A and c in flight (a register ring; slot = segment index mod PD)
    constexpr int PD = 4;
    float mreg[PD][MPT];
    f32x4 creg[PD];
    auto seg_of = [&](int s) { return (size_t)(transpose ? R - 1 - s : s) * H + h; };
    auto fetch = [&](int s, int slot) {  // A and c of the s-th segment in scan order
        const size_t seg = seg_of(s < R ? s : R - 1);
#pragma unroll
        for (int i = 0; i < MPT; ++i) mreg[slot][i] = M[seg * DK * DK + tid + kThreads * i];
#pragma unroll
        for (int i = 0; i < 4; ++i) creg[slot][i] = c[(seg * DK + row0 + i) * DV + col];
    };
    auto step = [&](int s, int slot) {
        const int b = s & 1;
        const size_t seg = seg_of(s);
#pragma unroll
        for (int i = 0; i < MPT; ++i) {
            const int e = tid + kThreads * i, a = e / DK, bb = e - a * DK;
            if (transpose) sA[b][bb * LM + a] = mreg[slot][i];
            else sA[b][a * LM + bb] = mreg[slot][i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sX[b][(row0 + i) * LX + 16 * tn + lr] = X[i];
            out[(seg * DK + row0 + i) * DV + col] = X[i];
        }
        // One barrier per segment: buffer b was last read in step s - 2, and every
        // thread passed step s - 1's barrier after finishing that step.
        __syncthreads();
        f32x4 acc = creg[slot];
#pragma unroll
        for (int k = 0; k < DK; k += 4) {
            const float a = sA[b][(16 * tm + lr) * LM + k + lg];   // A(row 16 tm + lr, k + lg)
            const float x = sX[b][(k + lg) * LX + 16 * tn + lr];   // X(k + lg, column 16 tn + lr)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, x, acc, 0, 0, 0);
        }
        X = acc;
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) fetch(i, i);
    // The loop body issues the same loads on every path (past the end it reloads
    // the last segment), so each wait on the memory counter covers one batch.
    int s = 0;
    for (; s + PD <= R; s += PD) {
#pragma unroll
        for (int i = 0; i < PD; ++i) {
            step(s + i, i);
            fetch(s + i + PD, i);
        }
    }
#pragma unroll
    for (int i = 0; i < PD - 1; ++i)
        if (s + i < R) step(s + i, i);
    if (xfinal) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xfinal[((size_t)h * DK + row0 + i) * DV + col] = X[i];
    }
}

// The same chain for dk = dv in {64, 128}: one workgroup of eight waves per
// (head, 32 columns of X); wave w holds the D fragments of X's tiles in row block
// 16 tm (tm = w at dk = 128, with both column tiles; w >> 1 at dk = 64, column
// tile w & 1).  A (dk x dk) is too large to stage per segment, so each lane
// reads its rows of A straight from memory as fp32 MFMA A operands, four
// consecutive k at once: step e of k-block kb takes k = 16 kb + 4 g + e from lane
// group g, for A and for X alike (any assignment of k to steps gives the same
// sum).  X^T sits in double-buffered LDS ([column][k], one barrier per segment);
// the next segment's A and c are in flight while the current one is applied.
constexpr int kWideThreads = 512;
template <int DK, bool TR>
__global__ void __launch_bounds__(kWideThreads) state_scan_wide_kernel(int R, int H, const float* __restrict__ M,
                                                                      const float* __restrict__ c,
                                                                      const float* __restrict__ x0,
                                                                      float* __restrict__ out,
                                                                      float* __restrict__ xfinal) {
    constexpr int DV = DK, BV = 32, TPW = DK / 64, KB = DK / 16, LX = DK + 4, PD = 2;
    static_assert((DK == 64 || DK == 128) && kWideThreads == 512, "two or one tiles per wave, eight waves");
    __shared__ __attribute__((aligned(16))) float sX[2][BV * LX];  // X^T [column][k]
    const int h = blockIdx.x, jb = blockIdx.y * BV;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int tm = TPW == 2 ? wave : wave >> 1;  // this wave's row block
    const int tn0 = TPW == 2 ? 0 : (wave & 1);   // its first column tile
    const int row0 = 16 * tm + 4 * lg;           // this lane's four rows of X (D fragment)
    const int arow = 16 * tm + lr;               // and its row of A (A fragment)
    f32x4 X[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int col = jb + 16 * (tn0 + t) + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) X[t][i] = x0 ? x0[((size_t)h * DK + row0 + i) * DV + col] : 0.f;
    }
    f32x4 areg[PD][KB], creg[PD][TPW];
    auto seg_of = [&](int s) { return (size_t)(TR ? R - 1 - s : s) * H + h; };
    auto fetch = [&](int s, int slot) {  // A and c of the s-th segment in scan order (past the end: the last)
        const size_t seg = seg_of(s < R ? s : R - 1);
        const float* Ms = M + seg * DK * DK;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if constexpr (TR) {  // A = M^T: A[arow][k] = M[k][arow]
#pragma unroll
                for (int e = 0; e < 4; ++e) areg[slot][kb][e] = Ms[(size_t)(16 * kb + 4 * lg + e) * DK + arow];
            } else {
                areg[slot][kb] = *(const f32x4*)(Ms + (size_t)arow * DK + 16 * kb + 4 * lg);
            }
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) creg[slot][t][i] = c[(seg * DK + row0 + i) * DV + jb + 16 * (tn0 + t) + lr];
    };
    auto step = [&](int s, int slot) {
        const int b = s & 1;
        const size_t seg = seg_of(s);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int cl = 16 * (tn0 + t) + lr;
            *(f32x4*)&sX[b][cl * LX + row0] = X[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(seg * DK + row0 + i) * DV + jb + cl] = X[t][i];
        }
        // One barrier per segment: buffer b was last read in step s - 2, and every
        // thread passed step s - 1's barrier after finishing that step.
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int cl = 16 * (tn0 + t) + lr;
            f32x4 acc = creg[slot][t];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f32x4 xv = *(const f32x4*)&sX[b][cl * LX + 16 * kb + 4 * lg];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(areg[slot][kb][e], xv[e], acc, 0, 0, 0);
            }
            X[t] = acc;
        }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) fetch(i, i);
    int s = 0;
    for (; s + PD <= R; s += PD) {
#pragma unroll
        for (int i = 0; i < PD; ++i) {
            step(s + i, i);
            fetch(s + i + PD, i);
        }
    }
#pragma unroll
    for (int i = 0; i < PD - 1; ++i)
        if (s + i < R) step(s + i, i);
    if (xfinal) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) xfinal[((size_t)h * DK + row0 + i) * DV + jb + 16 * (tn0 + t) + lr] = X[t][i];
    }
}

hipError_t launch_segment_maps(const ChunkArgs& a, float* M, hipStream_t s) {
    if (a.dk != 32) return launch_segmaps_wide(a, M, s);  // dk = dv >= 64: the direct form's state pass
    // (the forward arrays lead both layouts, so a saved forward's P is read at the same offset)
    const Prm p = make_prm(a, ws_layout(a, false));
    if (!(a.flags & (1u << 4))) {  // not KDA_F_FWD_SAVED: form the chunks' P first
        const hipError_t e = launch_recompute_intra(p, a, s);
        if (e != hipSuccess) return e;
    }
    if (a.in_bf16)
        KDA_LAUNCH("seg_map", seg_map_kernel<Prec::BF3>, dim3(a.N * a.H), dim3(kPsThreads), s, p, M);
    else
        KDA_LAUNCH("seg_map", seg_map_kernel<Prec::F32>, dim3(a.N * a.H), dim3(kPsThreads), s, p, M);
    return hipSuccess;
}

hipError_t launch_state_scan(int R, int H, int dk, int dv, bool transpose, const float* M, const float* c,
                             const float* x0, float* out, float* xfinal, hipStream_t s) {
    if ((dk == 64 || dk == 128) && dv == dk) {
        const dim3 grid(H, dv / 32);
        if (dk == 64) {
            if (transpose)
                KDA_LAUNCH("state_scan", (state_scan_wide_kernel<64, true>), grid, dim3(kWideThreads), s, R, H, M, c, x0, out, xfinal);
            else
                KDA_LAUNCH("state_scan", (state_scan_wide_kernel<64, false>), grid, dim3(kWideThreads), s, R, H, M, c, x0, out, xfinal);
        } else {
            if (transpose)
                KDA_LAUNCH("state_scan", (state_scan_wide_kernel<128, true>), grid, dim3(kWideThreads), s, R, H, M, c, x0, out, xfinal);
            else
                KDA_LAUNCH("state_scan", (state_scan_wide_kernel<128, false>), grid, dim3(kWideThreads), s, R, H, M, c, x0, out, xfinal);
        }
        return hipSuccess;
    }
    if (dk != 32 || dv % 32 != 0) return hipErrorInvalidValue;
    KDA_LAUNCH("state_scan", state_scan_kernel<32>, dim3(H, dv / 32), dim3(kThreads), s, R, H, dv, transpose ? 1 : 0,
               M, c, x0, out, xfinal);
    return hipSuccess;
}

}  // namespace kda
