// kda_scan.cuh -- the sequential part of the forward: state passing and output.
//
// One workgroup per (sequence, head, 32 columns of the state).  For every
// chunk of the sequence, in order, with h the fp32 state entering it:
//   v_new = u - w h                         (64 x 32)
//   o     = scale (exp(G) q h + Aqk v_new)  (64 x 32, written if requested)
//   h    <- Diag(exp G_L) h + (k exp(G_L - G))^T v_new
// All operands of a chunk come precomputed from the intra-chunk kernel, so the
// loop body is three MFMA products; the operands of chunk n+1 are loaded into
// registers while chunk n is computed.  The fp32 state stays in the registers
// of the lanes that own its 16x16 tiles (the same lanes every chunk); an MFMA
// operand copy hT[j][c] is written each chunk, double buffered so that the
// output product (reading h) and the state update run in the same phase.
// Optional stores for the backward: the state entering each chunk and v_new.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

template <int DK>
struct ScanRegs {
    static constexpr int NW = kChunk * DK / 4 / kThreads;          // float4 of w (and of qg, khT)
    static constexpr int NA = kChunk * kChunk / 4 / kThreads;      // float4 of aqk
    f32x4 w[NW], q[NW], k[NW], a[NA];
    float u[8];   // u at this lane's v_new fragment positions (2 tiles x 4 rows)
    float g[4 * ((DK / 16) * 2 + kWaves - 1) / kWaves];  // exp(G_L) at this lane's state rows
};

template <int DK, int DV>
__device__ __forceinline__ void scan_load(const Prm& p, size_t slot, int jb, ScanRegs<DK>& R) {
    const int tid = threadIdx.x, wave = tid >> 6;
    const f32x4* w = (const f32x4*)(p.w + slot * kChunk * DK);
    const f32x4* q = (const f32x4*)(p.qg + slot * kChunk * DK);
    const f32x4* k = (const f32x4*)(p.khT + slot * DK * kChunk);
    const f32x4* a = (const f32x4*)(p.aqk + slot * kChunk * kChunk);
#pragma unroll
    for (int i = 0; i < ScanRegs<DK>::NW; ++i) {
        R.w[i] = w[tid + kThreads * i];
        R.q[i] = q[tid + kThreads * i];
        R.k[i] = k[tid + kThreads * i];
    }
#pragma unroll
    for (int i = 0; i < ScanRegs<DK>::NA; ++i) R.a[i] = a[tid + kThreads * i];
    const float* u = p.u + slot * kChunk * DV + jb;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // v_new tiles wave and wave + 4 of 8: (tm, tn) = (tile >> 1, tile & 1)
        const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) R.u[4 * i + r] = u[(size_t)(tm * 16 + frag_row(r)) * DV + tn * 16 + frag_col()];
    }
    constexpr int TH = (DK / 16) * 2;
#pragma unroll
    for (int i = 0; i < (TH + kWaves - 1) / kWaves; ++i) {
        const int tile = wave + kWaves * i;
        if (tile < TH) {
            const int tm = tile >> 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) R.g[4 * i + r] = p.gl[slot * DK + tm * 16 + frag_row(r)];
        }
    }
}

template <int DK, int DV, typename TOut, Prec P>
__global__ void __launch_bounds__(kThreads) fwd_scan_kernel(Prm p, int total_wg, int write_o, int store_states) {
    constexpr int BV = 32, LK = DK + 8, LA = kChunk + 8, NV = DV / BV;
    constexpr int TH = (DK / 16) * 2;                         // state tiles (DK x 32)
    constexpr int HPW = (TH + kWaves - 1) / kWaves;           // state tiles per wave
    __shared__ __attribute__((aligned(16))) float sW[kChunk * LK];
    __shared__ __attribute__((aligned(16))) float sQ[kChunk * LK];
    __shared__ __attribute__((aligned(16))) float sA[kChunk * LA];
    __shared__ __attribute__((aligned(16))) float sK[DK * LA];
    __shared__ __attribute__((aligned(16))) float sH[2][BV * LK];
    __shared__ __attribute__((aligned(16))) float sV[BV * LA];
    const Tile<P> Wl(sW, kChunk, LK), Ql(sQ, kChunk, LK), Al(sA, kChunk, LA), KhT(sK, DK, LA), vnT(sV, BV, LA);
    const Tile<P> hT0(sH[0], BV, LK), hT1(sH[1], BV, LK);

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int vb = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = vb * BV;
    const int tid = threadIdx.x, wave = tid >> 6;

    // fp32 state: this lane's elements of its state tiles (rows c, column j)
    f32x4 S[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int tile = wave + kWaves * i;
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < TH) {
            const int tm = tile >> 1, tn = tile & 1, j = tn * 16 + frag_col();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cc = tm * 16 + frag_row(r);
                S[i][r] = p.h0 ? p.h0[((size_t)nh * DK + cc) * DV + jb + j] : 0.f;
            }
            hT0.put4(j, tm * 16 + frag_row(0), S[i]);
        }
    }
    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    ScanRegs<DK> R;
    if (c0 < c1) scan_load<DK, DV>(p, (size_t)c0 * p.H + h, jb, R);
    TOut* o = (TOut*)p.o;
    for (int c = c0; c < c1; ++c) {
        const ChunkRef cr = p.seq.chunk(c);
        const size_t slot = (size_t)c * p.H + h;
        __syncthreads();  // the previous chunk is done with the operand tiles
#pragma unroll
        for (int i = 0; i < ScanRegs<DK>::NW; ++i) {
            const int e4 = 4 * (tid + kThreads * i);
            const int t = e4 / DK, cc = e4 - t * DK;
            Wl.put4(t, cc, R.w[i]);
            Ql.put4(t, cc, R.q[i]);
            const int kc = e4 / kChunk, kt = e4 - kc * kChunk;
            KhT.put4(kc, kt, R.k[i]);
        }
#pragma unroll
        for (int i = 0; i < ScanRegs<DK>::NA; ++i) {
            const int e4 = 4 * (tid + kThreads * i);
            Al.put4(e4 >> 6, e4 & 63, R.a[i]);
        }
        float u[8], gl[4 * HPW];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = R.u[i];
#pragma unroll
        for (int i = 0; i < 4 * HPW; ++i) gl[i] = R.g[i];
        __syncthreads();
        if (c + 1 < c1) scan_load<DK, DV>(p, slot + p.H, jb, R);
        const bool odd = (c - c0) & 1;
        const Tile<P> hb = odd ? hT1 : hT0;
        const Tile<P> hn = odd ? hT0 : hT1;
        if (store_states) {
            float* hs = p.hs + slot * DK * DV;
#pragma unroll
            for (int i = 0; i < HPW; ++i) {
                const int tile = wave + kWaves * i;
                if (tile < TH) {
                    const int tm = tile >> 1, tn = tile & 1;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        hs[(size_t)(tm * 16 + frag_row(r)) * DV + jb + tn * 16 + frag_col()] = S[i][r];
                }
            }
        }
        // v_new = u - w h
        float* vno = p.vn + slot * kChunk * DV;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_tile(Wl.sub(tm * 16), hb.sub(tn * 16), 0, DK, acc);
            f32x4 val;
#pragma unroll
            for (int r = 0; r < 4; ++r) val[r] = u[4 * i + r] - acc[r];
            const int j = tn * 16 + frag_col();
            vnT.put4(j, tm * 16 + frag_row(0), val);
            if (store_states) {
#pragma unroll
                for (int r = 0; r < 4; ++r) vno[(size_t)(tm * 16 + frag_row(r)) * DV + jb + j] = val[r];
            }
        }
        __syncthreads();
        // h' = Diag(exp G_L) h + Kh^T v_new (the state tiles of this wave)
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + kWaves * i;
            if (tile < TH) {
                const int tm = tile >> 1, tn = tile & 1;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_tile(KhT.sub(tm * 16), vnT.sub(tn * 16), 0, kChunk, acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = gl[4 * i + r] * S[i][r] + acc[r];
                hn.put4(tn * 16 + frag_col(), tm * 16 + frag_row(0), S[i]);
            }
        }
        // o = scale (Qg h + Aqk v_new)
        if (write_o) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_tile(Ql.sub(tm * 16), hb.sub(tn * 16), 0, DK, acc);
                int k0 = 0, k1 = 16 * (tm + 1);
                widen<P>(k0, k1);
                acc = mma_tile(Al.sub(tm * 16), vnT.sub(tn * 16), k0, k1, acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = tm * 16 + frag_row(r), j = tn * 16 + frag_col();
                    if (t < cr.len) Elem<TOut>::store(o, tok_index(cr.t0 + t, h, p.H, DV) + jb + j, p.scale * acc[r]);
                }
            }
        }
    }
    if (p.hT) {
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + kWaves * i;
            if (tile < TH) {
                const int tm = tile >> 1, tn = tile & 1;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.hT[((size_t)nh * DK + tm * 16 + frag_row(r)) * DV + jb + tn * 16 + frag_col()] = S[i][r];
            }
        }
    }
}

}  // namespace kda
