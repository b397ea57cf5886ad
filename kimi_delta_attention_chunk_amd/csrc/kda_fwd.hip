// kda_fwd.hip -- chunked forward: intra-chunk, inter-chunk state passing, output.
//
// Three launches per call (the in-chunk algebra is in kda_chunk.cuh):
//   fwd_intra   one workgroup per (chunk, head): gate preparation, in-chunk
//               cumulative decay, Gram matrices, UT inverse, w and u, Aqk;
//   fwd_state   one workgroup per (sequence, head, 32-column block of dv):
//               the only sequential part, chunk after chunk with the fp32
//               state in LDS; stores the state entering every chunk and v_new;
//   fwd_output  one workgroup per (chunk, head, column block): o.
// All products are fp32 MFMA (v_mfma_f32_16x16x4_f32); decays are exact.
#include <type_traits>

#include "kda_chunk.cuh"
#include "kda_internal.h"
#include "kda_intra.cuh"
#include "kda_pscan.cuh"
#include "kda_scan.cuh"

namespace kda {

// ============================================================== state passing
template <int DK, int DV, typename TIn>
__global__ void __launch_bounds__(kThreads) fwd_state_kernel(Prm p, int total_wg) {
    constexpr int LS = kBV + 4;
    __shared__ float S[DK * LS];        // state block, [c][j]
    __shared__ float KhT[DK * kLD];     // k . exp(G_L - G), transposed
    __shared__ float GT[DK * kLD];
    __shared__ float WL[kChunk * (DK + 4)];
    __shared__ float VN[kChunk * LS];
    __shared__ float gL[DK];
    __shared__ float rn[kChunk];

    constexpr int NV = DV / kBV;
    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int vb = lid % NV;
    const int nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = vb * kBV;
    const bool l2 = p.flags & 1u;

    for (int e = threadIdx.x; e < DK * kBV; e += kThreads) {
        const int cc = e / kBV, j = e - cc * kBV;
        S[cc * LS + j] = p.h0 ? p.h0[((size_t)nh * DK + cc) * DV + jb + j] : 0.f;
    }
    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    for (int c = c0; c < c1; ++c) {
        const ChunkRef cr = p.seq.chunk(c);
        const size_t slot = (size_t)c * p.H + h;
        __syncthreads();  // S of the previous chunk complete
        stage_qk<DK, TIn>((const TIn*)p.k, cr, h, p.H, l2, KhT, rn);
        stage_g<DK>(p, cr, h, GT, nullptr);
        float* hs = p.hs + slot * DK * DV;
        for (int e = threadIdx.x; e < DK * kBV; e += kThreads) {
            const int cc = e / kBV, j = e - cc * kBV;
            hs[cc * DV + jb + j] = S[cc * LS + j];
        }
        const int last = cr.len - 1;
        for (int e = threadIdx.x; e < DK * kChunk; e += kThreads) {
            const int cc = e / kChunk, t = e - cc * kChunk;
            KhT[cc * kLD + t] *= __expf(GT[cc * kLD + last] - GT[cc * kLD + t]);
        }
        if (threadIdx.x < DK) gL[threadIdx.x] = __expf(GT[threadIdx.x * kLD + last]);
        const float* wi = p.w + slot * kChunk * DK;
        for (int e = threadIdx.x; e < kChunk * DK; e += kThreads) {
            const int t = e / DK, cc = e - t * DK;
            WL[t * (DK + 4) + cc] = wi[t * DK + cc];
        }
        __syncthreads();
        // v_new = u - w S
        const float* ui = p.u + slot * kChunk * DV;
        float* vo = p.vn + slot * kChunk * DV;
        wg_gemm<kChunk, kBV>(WL, DK + 4, 1, S, LS, 1, DK, FullK(), [&](int t, int j, float x) {
            const float val = ui[t * DV + jb + j] - x;
            VN[t * LS + j] = val;
            vo[t * DV + jb + j] = val;
        });
        __syncthreads();
        // S = Diag(exp G_L) S + Kh^T v_new
        wg_gemm<DK, kBV>(KhT, kLD, 1, VN, LS, 1, kChunk, FullK(), [&](int cc, int j, float x) {
            S[cc * LS + j] = gL[cc] * S[cc * LS + j] + x;
        });
    }
    __syncthreads();
    if (p.hT) {
        for (int e = threadIdx.x; e < DK * kBV; e += kThreads) {
            const int cc = e / kBV, j = e - cc * kBV;
            p.hT[((size_t)nh * DK + cc) * DV + jb + j] = S[cc * LS + j];
        }
    }
}

// ============================================================== output
template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kThreads) fwd_output_kernel(Prm p) {
    constexpr int OB = DV < 64 ? DV : 64;  // output columns per workgroup
    constexpr int LO = OB + 4;
    __shared__ float QT[DK * kLD];
    __shared__ float GT[DK * kLD];
    __shared__ float Hs[DK * LO];
    __shared__ float VN[kChunk * LO];
    __shared__ float AQ[kChunk * kLD];
    __shared__ float rn[kChunk];

    const int c = blockIdx.x, h = blockIdx.y, jb = blockIdx.z * OB;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;

    stage_qk<DK, TIn>((const TIn*)p.q, cr, h, p.H, p.flags & 1u, QT, rn);
    stage_g<DK>(p, cr, h, GT, nullptr);
    const float* hs = p.hs + slot * DK * DV;
    const float* vn = p.vn + slot * kChunk * DV;
    const float* aq = p.aqk + slot * kChunk * kChunk;
    for (int e = threadIdx.x; e < DK * OB; e += kThreads) {
        const int cc = e / OB, j = e - cc * OB;
        Hs[cc * LO + j] = hs[cc * DV + jb + j];
    }
    for (int e = threadIdx.x; e < kChunk * OB; e += kThreads) {
        const int t = e / OB, j = e - t * OB;
        VN[t * LO + j] = vn[t * DV + jb + j];
    }
    for (int e = threadIdx.x; e < kChunk * kChunk; e += kThreads) {
        const int t = e >> 6, s = e & 63;
        AQ[t * kLD + s] = aq[e];
    }
    for (int e = threadIdx.x; e < DK * kChunk; e += kThreads) {
        const int cc = e / kChunk, t = e - cc * kChunk;
        QT[cc * kLD + t] *= __expf(GT[cc * kLD + t]);
    }
    __syncthreads();
    TOut* o = (TOut*)p.o;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    constexpr int TN = OB / 16, TILES = (kChunk / 16) * TN;
    for (int tile = wave; tile < TILES; tile += kWaves) {
        const int tm = tile / TN, tn = tile % TN;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma16_f32(QT + tm * 16, 1, kLD, Hs + tn * 16, LO, 1, 0, DK, acc);
        acc = mma16_f32(AQ + tm * 16 * kLD, kLD, 1, VN + tn * 16, LO, 1, 0, 16 * (tm + 1), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tm * 16 + 4 * (lane >> 4) + i, j = tn * 16 + (lane & 15);
            if (t < cr.len) Elem<TOut>::store(o, tok_index(cr.t0 + t, h, p.H, DV) + jb + j, p.scale * acc[i]);
        }
    }
}

// ============================================================== host side
Prm make_prm(const ChunkArgs& a, const WsLayout& L) {
    Prm p{};
    p.B = a.B; p.T = a.T; p.H = a.H; p.N = a.N;
    p.scale = a.scale; p.flags = a.flags;
    p.seq.B = a.B; p.seq.T = a.T; p.seq.N = a.N;
    p.seq.cu = a.cu; p.seq.cidx = a.cidx; p.seq.coff = a.coff; p.seq.nc_dense = a.nc_dense;
    p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta;
    p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.h0 = a.h0;
    p.o = a.o; p.hT = a.hT; p.d_o = a.d_o; p.dhT = a.dhT;
    p.dq = a.dq; p.dk = a.dk_; p.dv = a.dv_; p.dg = a.dg; p.dbeta = a.dbeta; p.dh0 = a.dh0;
    p.dA_log = a.dA_log; p.ddt_bias = a.ddt_bias;
    char* base = (char*)a.ws;
    auto at = [&](size_t off) { return off ? (float*)(base + off) : (float*)nullptr; };
    p.w = at(L.w);
    p.u = at(L.u); p.aqk = at(L.aqk); p.tm = at(L.tm); p.hs = at(L.hs); p.vn = at(L.vn);
    p.qg = at(L.qg); p.khT = at(L.khT); p.gl = at(L.gl);
    p.dhs = at(L.dhs); p.dvn = at(L.dvn);
    p.dqt = at(L.dqt); p.dkh = at(L.dkh); p.dwv = at(L.dwv); p.daq = at(L.daq); p.dtv = at(L.dtv);
    p.dgl = at(L.dgl); p.dbv = at(L.dbv);
    p.dkt = at(L.dkt); p.dxq = at(L.dxq); p.dxk = at(L.dxk); p.part_a = at(L.part_a); p.part_dt = at(L.part_dt);
    p.pm = at(L.pm); p.pmT = at(L.pmT); p.hh = at(L.hh); p.qh = at(L.qh); p.qhT = at(L.qhT); p.ol = at(L.ol);
    p.aqT = at(L.aqT);
    p.sink = (float*)base;
    return p;
}

WsLayout ws_layout(const ChunkArgs& a, bool backward) {
    WsLayout L{};
    const size_t slots = (size_t)a.n_chunks_bound * a.H;
    const size_t C = kChunk, dk = a.dk, dv = a.dv;
    auto bytes = [](size_t n) { return (n * sizeof(float) + 255) & ~(size_t)255; };
    // The first 256 bytes hold no array: offset 0 means "array absent" (null
    // pointer in the kernel parameters), and masked-out lanes of branch-free
    // stores write there (Prm::sink).
    size_t off = 256;
    auto take = [&](size_t& field, size_t n) { field = off; off += bytes(n ? n : 1); };
    if (dk == 32 && dv == 64) {
        // affine chunk form: only what its kernels read
        take(L.hs, slots * dk * dv);
        take(L.pm, slots * dk * dk);
        take(L.pmT, slots * dk * dk);
        take(L.hh, slots * dk * dv);
        take(L.qh, slots * C * dk);
        take(L.qhT, slots * C * dk);
        take(L.ol, slots * C * dv);
        if (backward) {
            take(L.aqT, slots * C * C);
            take(L.tm, slots * C * C);
            take(L.dhs, slots * dk * dv);
            take(L.part_a, slots);
            take(L.part_dt, slots * dk);
        }
        L.total = off;
        return L;
    }
    take(L.w, slots * C * dk);
    take(L.u, slots * C * dv);
    take(L.aqk, slots * C * C);
    take(L.hs, slots * dk * dv);
    take(L.vn, slots * C * dv);
    take(L.qg, slots * C * dk);
    take(L.khT, slots * C * dk);
    take(L.gl, slots * dk);
    if (backward) {
        take(L.tm, slots * C * C);
        take(L.dhs, slots * dk * dv);
        take(L.dvn, slots * C * dv);
        take(L.dqt, slots * C * dk);
        take(L.dkh, slots * C * dk);
        take(L.dwv, slots * C * dk);
        take(L.daq, slots * C * C);
        take(L.dtv, slots * C * C);
        take(L.dgl, slots * dk);
        take(L.dbv, slots * C);
        take(L.dkt, slots * C * dk);
        take(L.dxq, slots * C * dk);
        take(L.dxk, slots * C * dk);
        take(L.part_a, slots);
        take(L.part_dt, slots * dk);
    }
    L.total = off;
    return L;
}

bool dims_supported(int dk, int dv) {
    return (dk == 32 && dv == 64) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128);
}

// Intra-chunk kernel, then the sequential pass.  `write_o`: produce o (the
// forward); `store` : keep the state entering each chunk and v_new (the
// backward's recompute).  dk <= 64 uses the precomputed-operand scan; dk = 128
// keeps the staging state and output kernels above (the scan's tiles would
// exceed the 160 KB of LDS).
template <int DK, int DV, typename TIn, typename TOut>
hipError_t launch_fwd_pipeline(const Prm& p, const ChunkArgs& a, hipStream_t s, bool write_o, bool store) {
    constexpr Prec P = std::is_same<TIn, uint16_t>::value ? Prec::BF3 : Prec::F32;
    if constexpr (DK == 32 && DV == 64) {
        // every array these kernels write must be in the workspace layout
        if (!p.hs || !p.pm || !p.pmT || !p.hh || !p.qh || !p.qhT || !p.ol) return hipErrorInvalidValue;
        if (store && (!p.tm || !p.aqT)) return hipErrorInvalidValue;
    }
    if (a.n_chunks_bound > 0)
        KDA_LAUNCH("fwd_intra", (intra_kernel<DK, DV, TIn, P>), dim3(a.n_chunks_bound, a.H), dim3(kThreads), s, p);
    if constexpr (DK == 32 && DV == 64) {
        const int total = a.N * a.H * (DV / kPsBV);
        if (write_o && store)
            KDA_LAUNCH("fwd_scan", (fwd_pscan_kernel<TOut, P, kPsBV, true, true>), dim3(total), dim3(kPsThreads), s, p, total);
        else if (write_o)
            KDA_LAUNCH("fwd_scan", (fwd_pscan_kernel<TOut, P, kPsBV, true, false>), dim3(total), dim3(kPsThreads), s, p, total);
        else if (store)
            KDA_LAUNCH("fwd_scan", (fwd_pscan_kernel<TOut, P, kPsBV, false, true>), dim3(total), dim3(kPsThreads), s, p, total);
        else
            KDA_LAUNCH("fwd_scan", (fwd_pscan_kernel<TOut, P, kPsBV, false, false>), dim3(total), dim3(kPsThreads), s, p, total);
    } else if constexpr (DK <= 64) {
        const int total = a.N * a.H * (DV / 32);
        KDA_LAUNCH("fwd_scan", (fwd_scan_kernel<DK, DV, TOut, P>), dim3(total), dim3(kScanThreads), s, p, total,
                   write_o ? 1 : 0, store ? 1 : 0);
    } else {
        const int total = a.N * a.H * (DV / kBV);
        KDA_LAUNCH("fwd_state", (fwd_state_kernel<DK, DV, TIn>), dim3(total), dim3(kThreads), s, p, total);
        if (write_o && a.n_chunks_bound > 0) {
            constexpr int OB = DV < 64 ? DV : 64;
            KDA_LAUNCH("fwd_output", (fwd_output_kernel<DK, DV, TIn, TOut>), dim3(a.n_chunks_bound, a.H, DV / OB),
                       dim3(kThreads), s, p);
        }
    }
    return hipSuccess;
}

hipError_t launch_recompute(const Prm& p, const ChunkArgs& a, hipStream_t s) {
    // the output dtype is irrelevant without o
    if (a.dk == 32 && a.dv == 64)
        return a.in_bf16 ? launch_fwd_pipeline<32, 64, uint16_t, float>(p, a, s, false, true)
                         : launch_fwd_pipeline<32, 64, float, float>(p, a, s, false, true);
    if (a.dk == 64 && a.dv == 64)
        return a.in_bf16 ? launch_fwd_pipeline<64, 64, uint16_t, float>(p, a, s, false, true)
                         : launch_fwd_pipeline<64, 64, float, float>(p, a, s, false, true);
    if (a.dk == 128 && a.dv == 128)
        return a.in_bf16 ? launch_fwd_pipeline<128, 128, uint16_t, float>(p, a, s, false, true)
                         : launch_fwd_pipeline<128, 128, float, float>(p, a, s, false, true);
    return hipErrorInvalidValue;
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_fwd_t(const ChunkArgs& a, hipStream_t s) {
    const bool save = a.flags & (1u << 3);
    const WsLayout L = ws_layout(a, save);
    const Prm p = make_prm(a, L);
    return launch_fwd_pipeline<DK, DV, TIn, TOut>(p, a, s, true, save || DK > 64);
}

template <int DK, int DV>
static hipError_t launch_fwd_dims(const ChunkArgs& a, hipStream_t s) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_fwd_t<DK, DV, uint16_t, uint16_t>(a, s)
                          : launch_fwd_t<DK, DV, uint16_t, float>(a, s);
    return a.out_bf16 ? launch_fwd_t<DK, DV, float, uint16_t>(a, s)
                      : launch_fwd_t<DK, DV, float, float>(a, s);
}

hipError_t launch_fwd(const ChunkArgs& a, hipStream_t s) {
    if (a.dk == 32 && a.dv == 64) return launch_fwd_dims<32, 64>(a, s);
    if (a.dk == 64 && a.dv == 64) return launch_fwd_dims<64, 64>(a, s);
    if (a.dk == 128 && a.dv == 128) return launch_fwd_dims<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
