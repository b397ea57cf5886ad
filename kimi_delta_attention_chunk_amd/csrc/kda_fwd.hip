// kda_fwd.hip -- chunked forward: intra-chunk, then the sequential pass.
//
// Two launches per call (the in-chunk algebra is in kda_chunk.cuh):
//   fwd_intra   one workgroup per (chunk, head): gate preparation, in-chunk
//               cumulative decay, Gram matrices, UT inverse, w and u, Aqk
//               (kda_intra.cuh); dk = 32: the chunk's affine form instead, by
//               a workgroup of eight waves (kda_intra32.cuh);
//   fwd_scan    one workgroup per (sequence, head, block of state columns):
//               chunk after chunk with the fp32 state in registers, the state
//               update and the output o (kda_pscan.cuh for dk = 32,
//               kda_scan.cuh otherwise).
// Products are MFMA: fp32 operands for fp32 inputs, bf16 hi/lo split (three
// bf16 MFMAs per product) for bf16 inputs; decays are exact.
#include <type_traits>

#include "kda_chunk.cuh"
#include "kda_internal.h"
#include "kda_intra.cuh"
#include "kda_intra32.cuh"
#include "kda_pscan.cuh"
#include "kda_scan.cuh"

namespace kda {

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
    p.qgT = at(L.qgT); p.khb = at(L.khb); p.wT = at(L.wT); p.gcs = at(L.gcs);
    p.dhs = at(L.dhs); p.dvn = at(L.dvn);
    p.dqt = at(L.dqt); p.dkh = at(L.dkh); p.dwv = at(L.dwv); p.daq = at(L.daq); p.dtv = at(L.dtv);
    p.dgl = at(L.dgl); p.dbv = at(L.dbv);
    p.dkt = at(L.dkt); p.dxq = at(L.dxq); p.dxk = at(L.dxk); p.part_a = at(L.part_a); p.part_dt = at(L.part_dt);
    p.pm = at(L.pm); p.pmT = at(L.pmT); p.hh = at(L.hh); p.qh = at(L.qh); p.qhT = at(L.qhT); p.ol = at(L.ol);
    p.aqT = at(L.aqT);
    p.sink = (float*)base;
    return p;
}

WsLayout ws_layout(const ChunkArgs& a, bool backward, WsRecord rec, void* ctx) {
    WsLayout L{};
    const size_t slots = (size_t)a.n_chunks_bound * a.H;
    const size_t C = kChunk, dk = a.dk, dv = a.dv;
    auto bytes = [](size_t n) { return (n * sizeof(float) + 255) & ~(size_t)255; };
    // The first 256 bytes hold no array: offset 0 means "array absent" (null
    // pointer in the kernel parameters), and masked-out lanes of branch-free
    // stores write there (Prm::sink).
    size_t off = 256;
    auto take_named = [&](size_t& field, size_t n, const char* name) {
        field = off;
        if (rec) rec(ctx, name, off, bytes(n ? n : 1));
        off += bytes(n ? n : 1);
    };
#define take(field, n) take_named(field, n, &(#field)[2])  // the array's name without "L."
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
            take(L.tm, slots * kTPacked);
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
        take(L.tm, slots * kTPacked);
        take(L.aqT, slots * C * C);
        take(L.qgT, slots * C * dk);
        take(L.khb, slots * C * dk);
        take(L.wT, slots * C * dk);
        take(L.gcs, slots * C * dk);
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
#undef take
}

bool dims_supported(int dk, int dv) {
    return (dk == 32 && dv == 64) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128);
}

// Intra-chunk kernel, then the sequential pass.  `write_o`: produce o (the
// forward); `store` : keep the state entering each chunk and v_new (the
// backward's recompute).
template <int DK, int DV, typename TIn, typename TOut>
hipError_t launch_fwd_pipeline(const Prm& p, const ChunkArgs& a, hipStream_t s, bool write_o, bool store,
                               bool run_intra = true) {
    constexpr Prec P = std::is_same<TIn, uint16_t>::value ? Prec::BF3 : Prec::F32;
    if constexpr (DK == 32 && DV == 64) {
        // every array these kernels write must be in the workspace layout
        if (!p.hs || !p.pm || !p.pmT || !p.hh || !p.qh || !p.qhT || !p.ol) return hipErrorInvalidValue;
        if (store && (!p.tm || !p.aqT)) return hipErrorInvalidValue;
    }
    if (run_intra && a.n_chunks_bound > 0) {
        if constexpr (DK == 32 && DV == 64)
            KDA_LAUNCH("fwd_intra", (intra32_kernel<TIn, P>), dim3(a.n_chunks_bound, a.H), dim3(kI32Threads), s, p);
        else
            KDA_LAUNCH("fwd_intra", (intra_kernel<DK, DV, TIn, P>), dim3(a.n_chunks_bound, a.H), dim3(kThreads), s, p);
    }
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
    } else {
        constexpr int BV = DK <= 32 ? 32 : 16;  // dk >= 64: 16 columns per workgroup (kda_scan.cuh)
        const int total = a.N * a.H * (DV / BV);
        KDA_LAUNCH("fwd_scan", (fwd_scan_kernel<DK, DV, BV, TOut, P>), dim3(total), dim3(kScanThreads), s, p, total,
                   write_o ? 1 : 0, store ? 1 : 0);
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

// The intra-chunk kernel alone (dk = 32: the affine form of every chunk), into
// the forward workspace layout.
hipError_t launch_recompute_intra(const Prm& p, const ChunkArgs& a, hipStream_t s) {
    if (a.dk != 32 || a.dv != 64 || !p.pm || !p.pmT || !p.hh || !p.qh || !p.qhT || !p.ol) return hipErrorInvalidValue;
    if (a.n_chunks_bound == 0) return hipSuccess;
    if (a.in_bf16)
        KDA_LAUNCH("fwd_intra", (intra32_kernel<uint16_t, Prec::BF3>), dim3(a.n_chunks_bound, a.H), dim3(kI32Threads),
                   s, p);
    else
        KDA_LAUNCH("fwd_intra", (intra32_kernel<float, Prec::F32>), dim3(a.n_chunks_bound, a.H), dim3(kI32Threads), s,
                   p);
    return hipSuccess;
}

// The transition map M of every sequence at dk = dv >= 64 (context parallelism):
// the intra-chunk kernel (unless the workspace holds a saved forward), then the
// forward state pass in its SEGMAP mode, which runs the chunks' transitions from
// the identity and writes M where the final state would go.
template <int DK, typename TIn>
static hipError_t launch_segmaps_t(Prm p, const ChunkArgs& a, float* M, bool saved, hipStream_t s) {
    constexpr Prec P = std::is_same<TIn, uint16_t>::value ? Prec::BF3 : Prec::F32;
    if (!p.w || !p.khT || !p.gl) return hipErrorInvalidValue;
    if (!saved && a.n_chunks_bound > 0)
        KDA_LAUNCH("fwd_intra", (intra_kernel<DK, DK, TIn, P>), dim3(a.n_chunks_bound, a.H), dim3(kThreads), s, p);
    p.hT = M;
    p.h0 = nullptr;
    p.o = nullptr;
    p.hs = nullptr;
    p.vn = nullptr;
    constexpr int BV = 16;  // as the forward pass at dk >= 64
    const int total = a.N * a.H * (DK / BV);
    KDA_LAUNCH("seg_map", (fwd_scan_kernel<DK, DK, BV, float, P, true>), dim3(total), dim3(kScanThreads), s, p, total,
               0, 0);
    return hipSuccess;
}

hipError_t launch_segmaps_wide(const ChunkArgs& a, float* M, hipStream_t s) {
    const Prm p = make_prm(a, ws_layout(a, false));
    const bool saved = a.flags & (1u << 4);  // KDA_F_FWD_SAVED: the forward arrays lead both layouts
    if (a.dk == 64 && a.dv == 64)
        return a.in_bf16 ? launch_segmaps_t<64, uint16_t>(p, a, M, saved, s) : launch_segmaps_t<64, float>(p, a, M, saved, s);
    if (a.dk == 128 && a.dv == 128)
        return a.in_bf16 ? launch_segmaps_t<128, uint16_t>(p, a, M, saved, s)
                         : launch_segmaps_t<128, float>(p, a, M, saved, s);
    return hipErrorInvalidValue;
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_fwd_t(const ChunkArgs& a, hipStream_t s) {
    const bool save = a.flags & (1u << 3), saved = a.flags & (1u << 4);
    // (with KDA_F_FWD_SAVED the intra-chunk quantities are already in the save layout)
    const WsLayout L = ws_layout(a, save || saved);
    const Prm p = make_prm(a, L);
    return launch_fwd_pipeline<DK, DV, TIn, TOut>(p, a, s, true, save, !saved);
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
