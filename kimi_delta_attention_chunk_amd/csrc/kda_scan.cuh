// kda_scan.cuh -- the sequential part of the forward: state passing and output.
//
// One workgroup per (sequence, head, BV columns of the state).  For every
// chunk of the sequence, in order, with h the fp32 state entering it:
//   v_new = u - w h                         (64 x BV)
//   o     = scale (exp(G) q h + Aqk v_new)  (64 x BV, written if requested)
//   h    <- Diag(exp G_L) h + (k exp(G_L - G))^T v_new
// All operands of a chunk come precomputed from the intra-chunk kernel in
// fragment form (kda_mma.cuh), so each lane loads its MFMA A fragments straight
// into registers, two or three chunks ahead, and the loop body is
// three products with two barriers.  Only the operands that depend on the
// state pass through LDS: the fp32 state stays in the registers of the lanes
// that own its 16x16 tiles, and an MFMA copy hT[j][c] is written each chunk,
// double buffered so that the output product (reading h) and the state update
// run in the same phase; v_new^T likewise.
// BV = 32 (dk = 64): each wave forms one v_new tile and the output tile at the
// same place.  BV = 16 (dk = 128: twice the state rows, so half the columns
// per workgroup keeps the registers and puts N*H*8 workgroups on the chip):
// there are only four 64 x 16 tiles, so waves 0-3 form v_new and waves 4-7 the
// output, each wave holding only the row operand its product needs.
// Optional stores for the backward: the state entering each chunk and v_new.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kScanThreads = 512, kScanWaves = 8;  // two waves per SIMD

// One chunk's operands for this lane, loaded straight from the fragment-form
// workspace arrays into MFMA A fragments.
template <int DK, int BV, Prec P>
struct ScanFrags {
    static constexpr int KB = DK / 32;
    static constexpr int TN = BV / 16;                               // 16-column tiles of the block
    static constexpr int VT = 4 * TN;                                // v_new / output tiles (64 x BV)
    static constexpr bool SPLIT = VT < kScanWaves;                   // v_new and output on separate waves
    static_assert(VT == kScanWaves || 2 * VT == kScanWaves, "block width");
    static constexpr int TH = (DK / 16) * TN;                        // state tiles (DK x BV)
    static constexpr int HPW = (TH + kScanWaves - 1) / kScanWaves;   // state tiles per wave
    // x: this wave's row operand over the state rows -- w (v_new tile), or
    // exp(G) q on the output waves of a split block; q: exp(G) q when the
    // same wave forms both products.
    AFrag<P> x[KB], q[SPLIT ? 1 : KB], a[2], k[HPW][2];
    float u[4];        // u at this lane's v_new fragment positions
    float g[4 * HPW];  // exp(G_L) at this lane's state rows
    // this wave's v_new / output tile (row block tm, column tile tn)
    __device__ __forceinline__ static int vtile(int wave) { return SPLIT && wave >= VT ? wave - VT : wave; }
    __device__ __forceinline__ static bool forms_vnew(int wave) { return !SPLIT || wave < VT; }
    __device__ __forceinline__ static bool forms_out(int wave) { return !SPLIT || wave >= VT; }
};

template <int DK, int DV, int BV, Prec P, bool SEGMAP>
__device__ __forceinline__ void scan_load(const Prm& p, size_t slot, int jb, ScanFrags<DK, BV, P>& R) {
    using F = ScanFrags<DK, BV, P>;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const int vt = F::vtile(wave), tm = vt / F::TN, tn = vt % F::TN;
    const char* w = (const char*)(p.w + slot * kChunk * DK);       // rows t, DK/32 k-blocks
    const char* q = (const char*)(p.qg + slot * kChunk * DK);      // [t][DK/32]
    const char* a = (const char*)(p.aqk + slot * kChunk * kChunk); // [t][2]
    const char* k = (const char*)(p.khT + slot * DK * kChunk);     // [c][2]
    const char* xs = F::forms_vnew(wave) ? w : q;
    const int row = 16 * tm + lr;
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb) {
        // (SEGMAP: no output, so the output waves' exp(G) q is not loaded)
        if (!SEGMAP || F::forms_vnew(wave)) load_afrag(R.x[kb], frag_rec(xs, row, kb, F::KB));
        if constexpr (!F::SPLIT && !SEGMAP) load_afrag(R.q[kb], frag_rec(q, row, kb, F::KB));
    }
    // A wave loads only the fragments its own products use (the conditions are
    // wave-uniform): the operand bytes each CU fetches per chunk bound this pass.
    // Aqk: the output waves, only its blocks below the diagonal.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        if (!SEGMAP && F::forms_out(wave) && kb <= (tm >> 1)) load_afrag(R.a[kb], frag_rec(a, row, kb, 2));
#pragma unroll
    for (int i = 0; i < F::HPW; ++i) {
        const int tile = wave + kScanWaves * i;
        if (tile < F::TH) {
        const int crow = 16 * (tile / F::TN) + lr;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) load_afrag(R.k[i][kb], frag_rec(k, crow, kb, 2));
        }
    }
    const float* u = p.u + slot * kChunk * DV + jb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (SEGMAP) R.u[r] = 0.f;  // (u = 0: the recurrence applies the transitions alone)
        else if (F::forms_vnew(wave)) R.u[r] = u[(size_t)(tm * 16 + frag_row(r)) * DV + tn * 16 + frag_col()];
    }
#pragma unroll
    for (int i = 0; i < F::HPW; ++i) {
        const int tile = wave + kScanWaves * i;
        {
            const int tmh = (tile < F::TH ? tile : 0) / F::TN;
#pragma unroll
            for (int r = 0; r < 4; ++r) R.g[4 * i + r] = p.gl[slot * DK + tmh * 16 + frag_row(r)];
        }
    }
}

// SEGMAP: the transition map of every sequence instead (dv = dk): from h = I with
// u = 0 the recurrence gives M = P_last ... P_first, P = Diag(exp G_L) - Kh^T w,
// written to p.hT; nothing else is written.
template <int DK, int DV, int BV, typename TOut, Prec P, bool SEGMAP = false>
__global__ void __launch_bounds__(kScanThreads) fwd_scan_kernel(Prm p, int total_wg, int write_o, int store_states) {
    static_assert(!SEGMAP || DK == DV, "a transition map is dk x dk");
    using F = ScanFrags<DK, BV, P>;
    constexpr int LK = DK + 8, LA = kChunk + 8, NV = DV / BV, TN = F::TN;
    constexpr int TH = F::TH, HPW = F::HPW, NWV = kScanWaves;
    __shared__ __attribute__((aligned(16))) float sH[2][BV * LK];
    __shared__ __attribute__((aligned(16))) float sV[BV * LA];
    const Tile<P> vnT(sV, BV, LA);
    const Tile<P> hT0(sH[0], BV, LK), hT1(sH[1], BV, LK);

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int vb = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = vb * BV;
    const int wave = wave_id();
    const int tm = F::vtile(wave) / TN, tn = F::vtile(wave) % TN;  // this wave's v_new / output tile

    // fp32 state: this lane's elements of its state tiles (rows c, column j)
    f32x4 S[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int tile = wave + NWV * i;
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < TH) {
            const int tmh = tile / TN, tnh = tile % TN, j = tnh * 16 + frag_col();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cc = tmh * 16 + frag_row(r);
                if constexpr (SEGMAP) S[i][r] = cc == jb + j ? 1.f : 0.f;
                else S[i][r] = p.h0 ? p.h0[((size_t)nh * DK + cc) * DV + jb + j] : 0.f;
            }
            hT0.put4(j, tmh * 16 + frag_row(0), S[i]);
        }
    }
    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    int64_t s0;
    int slen;
    p.seq.seq_tokens(n, s0, slen);
    TOut* o = (TOut*)p.o;
    // operand batches in flight: three at dk = 64; at dk = 128 the registers of two
    // waves per SIMD hold two
    constexpr int PD = DK <= 64 ? 3 : 2;
    F R[PD];
    // Prefetches are unconditional (past the last chunk they reload it), so the
    // control flow around them is uniform and each wait covers one chunk only.
    auto slot_of = [&](int cc) { return (size_t)(cc < c1 ? cc : c1 - 1) * p.H + h; };

    // One chunk: v_new = u - w h; h' = Diag(exp G_L) h + Kh^T v_new; o = scale (Qg h + Aqk v_new).
    auto step = [&](int c, F& Rc) {
        const ChunkRef cr = SeqLayout::chunk_of(n, c - c0, s0, slen);
        const size_t slot = (size_t)c * p.H + h;
        const bool odd = (c - c0) & 1;
        const Tile<P> hb = odd ? hT1 : hT0;
        const Tile<P> hn = odd ? hT0 : hT1;
        __syncthreads();  // h of this chunk is in hb; the previous chunk is done with vnT
        if (store_states) {
            float* hs = p.hs + slot * DK * DV;
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int tile = wave + NWV * i;
                if (tile < TH) {
                    const int tmh = tile / TN, tnh = tile % TN;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        hs[(size_t)(tmh * 16 + frag_row(r)) * DV + jb + tnh * 16 + frag_col()] = S[i][r];
                }
            }
        }
        if (F::forms_vnew(wave)) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < F::KB; ++kb) acc = mma_frag(Rc.x[kb], hb.sub(tn * 16), 32 * kb, acc);
            f32x4 val;
#pragma unroll
            for (int r = 0; r < 4; ++r) val[r] = Rc.u[r] - acc[r];
            const int j = tn * 16 + frag_col();
            vnT.put4(j, tm * 16 + frag_row(0), val);
            if (store_states) {
                float* vno = p.vn + slot * kChunk * DV;
#pragma unroll
                for (int r = 0; r < 4; ++r) vno[(size_t)(tm * 16 + frag_row(r)) * DV + jb + j] = val[r];
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + NWV * i;
            if (tile < TH) {
                const int tmh = tile / TN, tnh = tile % TN;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_frag(Rc.k[i][0], vnT.sub(tnh * 16), 0, acc);
                acc = mma_frag(Rc.k[i][1], vnT.sub(tnh * 16), 32, acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = Rc.g[4 * i + r] * S[i][r] + acc[r];
                hn.put4(tnh * 16 + frag_col(), tmh * 16 + frag_row(0), S[i]);
            }
        }
        if (write_o && F::forms_out(wave)) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < F::KB; ++kb) {
                if constexpr (F::SPLIT) acc = mma_frag(Rc.x[kb], hb.sub(tn * 16), 32 * kb, acc);
                else acc = mma_frag(Rc.q[kb], hb.sub(tn * 16), 32 * kb, acc);
            }
            acc = mma_frag(Rc.a[0], vnT.sub(tn * 16), 0, acc);
            if (tm >= 2) acc = mma_frag(Rc.a[1], vnT.sub(tn * 16), 32, acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tm * 16 + frag_row(r), j = tn * 16 + frag_col();
                if (t < cr.len) Elem<TOut>::store(o, tok_index(cr.t0 + t, h, p.H, DV) + jb + j, p.scale * acc[r]);
            }
        }
    };
    if (c0 < c1) {
        // (scheduling barriers keep the batches in issue order: the waits count
        // completions in order)
#pragma unroll
        for (int i = 0; i < PD; ++i) scan_load<DK, DV, BV, P, SEGMAP>(p, slot_of(c0 + i), jb, R[i]);
        __builtin_amdgcn_sched_barrier(0);
        for (int c = c0; c < c1; c += PD) {
#pragma unroll
            for (int i = 0; i < PD; ++i)
                if (i == 0 || c + i < c1) {
                    step(c + i, R[i]);
                    scan_load<DK, DV, BV, P, SEGMAP>(p, slot_of(c + i + PD), jb, R[i]);
                }
        }
    }
    if (p.hT) {
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + NWV * i;
            if (tile < TH) {
                const int tmh = tile / TN, tnh = tile % TN;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.hT[((size_t)nh * DK + tmh * 16 + frag_row(r)) * DV + jb + tnh * 16 + frag_col()] = S[i][r];
            }
        }
    }
}

}  // namespace kda
