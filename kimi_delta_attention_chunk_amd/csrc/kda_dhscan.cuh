// kda_dhscan.cuh -- the sequential part of the backward: the state gradient.
//
// One workgroup per (sequence, head, BV columns of the state: 32 for dk <= 64,
// 16 for dk = 128 so that the operand tiles fit the 160 KB of LDS), chunks in
// reverse.  With D = dL/dS at the end of the chunk (dhT, or 0, at the end of
// the sequence), per chunk:
//   dv_new = scale Aqk^T dO + Kh D                       (64 x 32)
//   D     <- scale (exp(G) q)^T dO + Diag(exp G_L) D - w^T dv_new
// (the reverse of v_new = u - w h, o = scale (Qg h + Aqk v_new),
// h' = Diag(exp G_L) h + Kh^T v_new).  D at every chunk end and dv_new are
// stored for the per-chunk gradient kernel; D after the first chunk is dh0.
// Operands come from the intra-chunk kernel (aqk, khT, qg, w, gl) and from dO,
// loaded one chunk ahead into registers, then transposed into MFMA tiles.
// The fp32 D stays in the registers of the lanes that own its tiles.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kDhThreads = 512, kDhWaves = 8;  // two waves per SIMD

// One chunk's operands, as loaded: 8-value chunks of the k-block arrays
// (kda_mma.cuh) -- w, exp(G) q [t][c], (k exp(G_L - G))^T [c][t] and Aqk [t][s] --
// plus dO and exp(G_L).
template <int DK, int BV, typename TIn, Prec P>
struct DhRegs {
    static constexpr int TN = BV / 16;                                          // 16-column tiles of the block
    static constexpr int CW = (kChunk * DK / 8 + kDhThreads - 1) / kDhThreads;  // chunks of w, qg, khT
    static constexpr int CA = kChunk * kChunk / 8 / kDhThreads;                 // chunks of aqk
    static constexpr int HPW = ((DK / 16) * TN + kDhWaves - 1) / kDhWaves;      // D tiles per wave
    static constexpr int ND = BV / 8;                                           // dO values per thread
    KChunk<P> w[CW], q[CW], k[CW], a[CA];
    float d[ND];  // dO[t][jb + ND part + i] for t = tid >> 3
    float g[4 * HPW];
};

template <int DK, int DV, int BV, typename TIn, Prec P>
__device__ __forceinline__ void dh_load(const Prm& p, size_t slot, const ChunkRef& cr, int h, int jb,
                                        DhRegs<DK, BV, TIn, P>& R) {
    using Rg = DhRegs<DK, BV, TIn, P>;
    const int tid = threadIdx.x, wave = wave_id();
    const char* w = (const char*)(p.w + slot * kChunk * DK);
    const char* q = (const char*)(p.qg + slot * kChunk * DK);
    const char* k = (const char*)(p.khT + slot * DK * kChunk);
    const char* a = (const char*)(p.aqk + slot * kChunk * kChunk);
#pragma unroll
    for (int i = 0; i < Rg::CW; ++i) {
        const int c8 = tid + kDhThreads * i;
        if (c8 < kChunk * DK / 8) {
            const int t = c8 / (DK / 8), k0 = 8 * (c8 % (DK / 8));  // w, qg: row t, index k0
            load_kchunk(R.w[i], w + (size_t)(t * (DK / 32) + (k0 >> 5)) * kKBlockBytes, (k0 >> 3) & 3);
            load_kchunk(R.q[i], q + (size_t)(t * (DK / 32) + (k0 >> 5)) * kKBlockBytes, (k0 >> 3) & 3);
            const int cc = c8 >> 3, t0 = 8 * (c8 & 7);                // khT: row c, index t0
            load_kchunk(R.k[i], k + (size_t)(cc * 2 + (t0 >> 5)) * kKBlockBytes, (t0 >> 3) & 3);
        }
    }
#pragma unroll
    for (int i = 0; i < Rg::CA; ++i) {
        const int c8 = tid + kDhThreads * i;
        const int t = c8 >> 3, s0 = 8 * (c8 & 7);
        load_kchunk(R.a[i], a + (size_t)(t * 2 + (s0 >> 5)) * kKBlockBytes, (s0 >> 3) & 3);
    }
    const int t = tid >> 3, part = tid & 7;
    {
        // rows past the chunk end read row 0 (always valid) and are zeroed
        const TIn* src = (const TIn*)p.d_o + tok_index(cr.t0 + (t < cr.len ? t : 0), h, p.H, DV) + jb + Rg::ND * part;
        if constexpr (Rg::ND == 4) {
            load4<TIn>(src, R.d);
        } else {
#pragma unroll
            for (int i = 0; i < Rg::ND; ++i) R.d[i] = Elem<TIn>::load(src, i);
        }
#pragma unroll
        for (int i = 0; i < Rg::ND; ++i) R.d[i] = t < cr.len ? R.d[i] : 0.f;
    }
    constexpr int TH = (DK / 16) * Rg::TN;
#pragma unroll
    for (int i = 0; i < Rg::HPW; ++i) {
        const int tile = wave + kDhWaves * i;
        if (tile < TH) {
            const int tm = tile / Rg::TN;
#pragma unroll
            for (int r = 0; r < 4; ++r) R.g[4 * i + r] = p.gl[slot * DK + tm * 16 + frag_row(r)];
        }
    }
}

template <int DK, int DV, int BV, typename TIn, Prec P>
__global__ void __launch_bounds__(kDhThreads) bwd_dh_scan_kernel(Prm p, int total_wg) {
    using Rg = DhRegs<DK, BV, TIn, P>;
    constexpr int LK = DK + 8, LA = kChunk + 8, NV = DV / BV, TN = Rg::TN;
    constexpr int TH = (DK / 16) * TN, VT = 4 * TN;  // D tiles; dv_new tiles (64 x BV)
    static_assert(VT <= kDhWaves, "one dv_new tile per wave");
    constexpr int HPW = Rg::HPW;
    constexpr int NTH = kDhThreads, NWV = kDhWaves;
    __shared__ __attribute__((aligned(16))) float sAq[kChunk * LA];   // Aqk^T [t][s]
    __shared__ __attribute__((aligned(16))) float sKh[kChunk * LK];   // Kh [t][c]
    __shared__ __attribute__((aligned(16))) float sQ[DK * LA];        // Qg^T [c][t]
    __shared__ __attribute__((aligned(16))) float sW[DK * LA];        // w^T [c][t]
    __shared__ __attribute__((aligned(16))) float sO[BV * LA];        // dO^T [j][t]
    __shared__ __attribute__((aligned(16))) float sD[2][BV * LK];     // D^T [j][c]
    __shared__ __attribute__((aligned(16))) float sV[BV * LA];        // dv_new^T [j][t]
    const Tile<P> AqT(sAq, kChunk, LA), Kh(sKh, kChunk, LK), QgT(sQ, DK, LA), WT(sW, DK, LA), dOT(sO, BV, LA),
        dvnT(sV, BV, LA);
    const Tile<P> DT0(sD[0], BV, LK), DT1(sD[1], BV, LK);

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int vb = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = vb * BV;
    const int tid = threadIdx.x, wave = wave_id();
    const float scale = p.scale;

    f32x4 D[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int tile = wave + NWV * i;
        D[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < TH) {
            const int tm = tile / TN, tn = tile % TN, j = tn * 16 + frag_col();
#pragma unroll
            for (int r = 0; r < 4; ++r)
                D[i][r] = p.dhT ? p.dhT[((size_t)nh * DK + tm * 16 + frag_row(r)) * DV + jb + j] : 0.f;
            DT0.put4(j, tm * 16 + frag_row(0), D[i]);
        }
    }
    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    int64_t s0;
    int slen;
    p.seq.seq_tokens(n, s0, slen);
    Rg R;
    // The prefetch is unconditional (at the first chunk it reloads it), so the
    // control flow around it is uniform and the wait covers one chunk only.
    if (c0 < c1) dh_load<DK, DV, BV, TIn, P>(p, (size_t)(c1 - 1) * p.H + h, SeqLayout::chunk_of(n, c1 - 1 - c0, s0, slen), h, jb, R);
    for (int c = c1 - 1; c0 < c1 && c >= c0; --c) {
        const size_t slot = (size_t)c * p.H + h;
        __syncthreads();  // the previous chunk is done with the operand tiles
#pragma unroll
        for (int i = 0; i < Rg::CW; ++i) {
            const int c8 = tid + NTH * i;
            if (c8 < kChunk * DK / 8) {
                const int t = c8 / (DK / 8), k0 = 8 * (c8 % (DK / 8));
                put_kchunk_t(WT, k0, t, R.w[i]);   // w^T [c][t]
                put_kchunk_t(QgT, k0, t, R.q[i]);  // Qg^T [c][t]
                const int cc = c8 >> 3, t0 = 8 * (c8 & 7);
                put_kchunk_t(Kh, t0, cc, R.k[i]);  // Kh [t][c]
            }
        }
#pragma unroll
        for (int i = 0; i < Rg::CA; ++i) {
            const int c8 = tid + NTH * i;
            put_kchunk_t(AqT, 8 * (c8 & 7), c8 >> 3, R.a[i]);  // Aqk^T [s][t]
        }
        {
            const int t = tid >> 3, part = tid & 7;
#pragma unroll
            for (int i = 0; i < Rg::ND; ++i) dOT.put(Rg::ND * part + i, t, R.d[i]);
        }
        float gl[4 * HPW];
#pragma unroll
        for (int i = 0; i < 4 * HPW; ++i) gl[i] = R.g[i];
        __syncthreads();
        {
            const int cn = c - 1 >= c0 ? c - 1 : c0;
            dh_load<DK, DV, BV, TIn, P>(p, (size_t)cn * p.H + h, SeqLayout::chunk_of(n, cn - c0, s0, slen), h, jb, R);
        }
        const bool odd = (c1 - 1 - c) & 1;
        const Tile<P> Db = odd ? DT1 : DT0;
        const Tile<P> Dn = odd ? DT0 : DT1;
        // D at the end of this chunk
        float* dhs = p.dhs + slot * DK * DV;
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + NWV * i;
            if (tile < TH) {
                const int tm = tile / TN, tn = tile % TN;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dhs[(size_t)(tm * 16 + frag_row(r)) * DV + jb + tn * 16 + frag_col()] = D[i][r];
            }
        }
        // dv_new = scale Aqk^T dO + Kh D
        float* dvo = p.dvn + slot * kChunk * DV;
        if (wave < VT) {
            const int tm = wave / TN, tn = wave % TN;
            int k0 = 16 * tm, k1 = kChunk;
            widen<P>(k0, k1);
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
            a1 = mma_tile(AqT.sub(tm * 16), dOT.sub(tn * 16), k0, k1, a1);
            a2 = mma_tile(Kh.sub(tm * 16), Db.sub(tn * 16), 0, DK, a2);
            f32x4 val;
#pragma unroll
            for (int r = 0; r < 4; ++r) val[r] = scale * a1[r] + a2[r];
            const int j = tn * 16 + frag_col();
            dvnT.put4(j, tm * 16 + frag_row(0), val);
#pragma unroll
            for (int r = 0; r < 4; ++r) dvo[(size_t)(tm * 16 + frag_row(r)) * DV + jb + j] = val[r];
        }
        __syncthreads();
        // D <- scale Qg^T dO + Diag(exp G_L) D - w^T dv_new
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + NWV * i;
            if (tile < TH) {
                const int tm = tile / TN, tn = tile % TN;
                f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
                a1 = mma_tile(QgT.sub(tm * 16), dOT.sub(tn * 16), 0, kChunk, a1);
                a2 = mma_tile(WT.sub(tm * 16), dvnT.sub(tn * 16), 0, kChunk, a2);
#pragma unroll
                for (int r = 0; r < 4; ++r) D[i][r] = gl[4 * i + r] * D[i][r] + scale * a1[r] - a2[r];
                Dn.put4(tn * 16 + frag_col(), tm * 16 + frag_row(0), D[i]);
            }
        }
    }
    if (p.dh0) {
#pragma unroll
        for (int i = 0; i < HPW; ++i) {
            const int tile = wave + NWV * i;
            if (tile < TH) {
                const int tm = tile / TN, tn = tile % TN;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.dh0[((size_t)nh * DK + tm * 16 + frag_row(r)) * DV + jb + tn * 16 + frag_col()] = D[i][r];
            }
        }
    }
}

}  // namespace kda
