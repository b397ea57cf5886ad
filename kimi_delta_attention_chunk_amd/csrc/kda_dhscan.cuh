// kda_dhscan.cuh -- the sequential part of the backward: the state gradient
// (dk = 64 and 128; dk = 32 uses the affine form in kda_pscan.cuh).
//
// One workgroup per (sequence, head, BV columns of the state), chunks in
// reverse.  With D = dL/dS at the end of the chunk (dhT, or 0, at the end of
// the sequence), per chunk:
//   dv_new = scale Aqk^T dO + Kh D                       (64 x BV)
//   D     <- scale (exp(G) q)^T dO + Diag(exp G_L) D - w^T dv_new
// (the reverse of v_new = u - w h, o = scale (Qg h + Aqk v_new),
// h' = Diag(exp G_L) h + Kh^T v_new).  D at every chunk end and dv_new are
// stored for the per-chunk gradient kernels; D after the first chunk is dh0.
//
// Every state-independent operand is an MFMA A fragment loaded straight from
// the fragment-form arrays the intra-chunk kernel writes for the reverse pass --
// Aqk^T and Kh (rows t), (exp(G) q)^T and w^T (rows c) -- two chunks ahead,
// double buffered, as in the forward scan.  Only dO^T, D^T and dv_new^T pass
// through LDS: the fp32 D stays in the registers of the lanes that own its
// 16x16 tiles.  dO^T of the next chunk is staged during the current one (its
// values arrive with the operand batch of the chunk before), so a chunk costs
// two barriers.
// BV = 32 (dk = 64): every wave forms one dv_new tile and one D tile.  BV = 16
// (dk = 128): four dv_new tiles on waves 0-3, eight D tiles on all waves.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kDhThreads = 512, kDhWaves = 8;  // two waves per SIMD

template <int DK, int BV, Prec P>
struct DhFrags {
    static constexpr int KB = DK / 32;
    static constexpr int TN = BV / 16;                             // 16-column tiles of the block
    static constexpr int VT = 4 * TN;                              // dv_new tiles (64 x BV)
    static constexpr int TH = (DK / 16) * TN;                      // D tiles (DK x BV)
    static constexpr int HPW = (TH + kDhWaves - 1) / kDhWaves;     // D tiles per wave
    static constexpr int ND = BV / 8;                              // dO values per thread
    static_assert(VT <= kDhWaves, "one dv_new tile per wave");
    AFrag<P> aq[2], kh[KB];          // Aqk^T, Kh rows of this wave's dv_new tile
    AFrag<P> qt[HPW][2], wt[HPW][2]; // (exp(G) q)^T, w^T rows of its D tiles
    float g[4 * HPW];                // exp(G_L) at its D rows
    float d[ND];                     // dO of the chunk processed after this one
};

// Operands of chunk slot `slot` and dO of the chunk `crd` (the one processed
// next, or a clamped repeat).
template <int DK, int DV, int BV, typename TIn, Prec P>
__device__ __forceinline__ void dh_load(const Prm& p, size_t slot, const ChunkRef& crd, int h, int jb,
                                        DhFrags<DK, BV, P>& R) {
    using F = DhFrags<DK, BV, P>;
    const int wave = wave_id(), lr = threadIdx.x & 15, tid = threadIdx.x;
    const int vt = wave < F::VT ? wave : 0, tm = vt / F::TN;
    const char* aq = (const char*)(p.aqT + slot * kChunk * kChunk);  // [t][2]
    const char* kh = (const char*)(p.khb + slot * kChunk * DK);      // [t][DK/32]
    const char* qt = (const char*)(p.qgT + slot * DK * kChunk);      // [c][2]
    const char* wt = (const char*)(p.wT + slot * DK * kChunk);       // [c][2]
    const int row = 16 * tm + lr;
    // A wave loads only the fragments its own products use (the conditions are
    // wave-uniform): the operand bytes each CU fetches per chunk bound this pass.
    if (wave < F::VT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) load_afrag(R.aq[kb], frag_rec(aq, row, kb, 2));
#pragma unroll
        for (int kb = 0; kb < F::KB; ++kb) load_afrag(R.kh[kb], frag_rec(kh, row, kb, F::KB));
    }
#pragma unroll
    for (int i = 0; i < F::HPW; ++i) {
        const int tile = wave + kDhWaves * i;
        const int c16 = 16 * ((tile < F::TH ? tile : 0) / F::TN);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {  // (a wave without a D tile reads tile 0's: a branch here costs more)
            load_afrag(R.qt[i][kb], frag_rec(qt, c16 + lr, kb, 2));
            load_afrag(R.wt[i][kb], frag_rec(wt, c16 + lr, kb, 2));
        }
        const f32x4 g4 = *(const f32x4*)&p.gl[slot * DK + c16 + frag_row(0)];
#pragma unroll
        for (int r = 0; r < 4; ++r) R.g[4 * i + r] = g4[r];
    }
    {
        // dO rows t = tid >> 3, columns jb + ND part ..; rows past the end read row 0 and are zeroed
        const int t = tid >> 3, part = tid & 7;
        const TIn* src = (const TIn*)p.d_o + tok_index(crd.t0 + (t < crd.len ? t : 0), h, p.H, DV) + jb + F::ND * part;
        if constexpr (F::ND == 4) {
            load4<TIn>(src, R.d);
        } else {
#pragma unroll
            for (int i = 0; i < F::ND; ++i) R.d[i] = Elem<TIn>::load(src, i);
        }
#pragma unroll
        for (int i = 0; i < F::ND; ++i) R.d[i] = t < crd.len ? R.d[i] : 0.f;
    }
}

template <int DK, int DV, int BV, typename TIn, Prec P>
__global__ void __launch_bounds__(kDhThreads) bwd_dh_scan_kernel(Prm p, int total_wg) {
    using F = DhFrags<DK, BV, P>;
    constexpr int LK = DK + 8, LA = kChunk + 8, NV = DV / BV, TN = F::TN, TH = F::TH, VT = F::VT, HPW = F::HPW;
    __shared__ __attribute__((aligned(16))) float sO[2][BV * LA];  // dO^T [j][t], double buffered
    __shared__ __attribute__((aligned(16))) float sD[2][BV * LK];  // D^T [j][c], double buffered
    __shared__ __attribute__((aligned(16))) float sV[BV * LA];     // dv_new^T [j][t]
    const Tile<P> dOT0(sO[0], BV, LA), dOT1(sO[1], BV, LA), DT0(sD[0], BV, LK), DT1(sD[1], BV, LK),
        dvnT(sV, BV, LA);

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int vb = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = vb * BV;
    const int tid = threadIdx.x, wave = wave_id();
    const float scale = p.scale;
    const int tmv = (wave < VT ? wave : 0) / TN, tnv = (wave < VT ? wave : 0) % TN;  // this wave's dv_new tile

    f32x4 D[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int tile = wave + kDhWaves * i;
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
    auto clamp = [&](int cc) { return cc >= c0 ? cc : c0; };
    auto ref = [&](int cc) { return SeqLayout::chunk_of(n, clamp(cc) - c0, s0, slen); };
    auto slot_of = [&](int cc) { return (size_t)clamp(cc) * p.H + h; };
    // Chunk c, the i-th from the end (i = c1 - 1 - c): dO^T of c is in dOb, D^T (at
    // its end) in Db; stages dO^T of c - 1 (in Rc.d) into dOn and D^T at the chunk
    // start into Dn.  Every global store is issued on every wave and path (stores
    // a wave does not make go to p.sink), so the waits on the memory counter count
    // exactly the operand batches in flight.
    auto step = [&](int c, const F& Rc) {
        const size_t slot = (size_t)c * p.H + h;
        const bool odd = (c1 - 1 - c) & 1;
        const Tile<P> dOb = odd ? dOT1 : dOT0, dOn = odd ? dOT0 : dOT1;
        const Tile<P> Db = odd ? DT1 : DT0, Dn = odd ? DT0 : DT1;
        __syncthreads();  // dO^T and D^T of this chunk staged; the previous chunk is done with dv_new^T
        {
            float* dhs = p.dhs + slot * DK * DV;
#pragma unroll
            for (int k = 0; k < HPW; ++k) {
                const int tile = wave + kDhWaves * k;
                const bool has = tile < TH;
                const int tm = (has ? tile : 0) / TN, tn = (has ? tile : 0) % TN;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *(has ? dhs + (size_t)(tm * 16 + frag_row(r)) * DV + jb + tn * 16 + frag_col() : p.sink) = D[k][r];
            }
        }
        f32x4 val = {0.f, 0.f, 0.f, 0.f};
        if (wave < VT) {
            // dv_new = scale Aqk^T dO + Kh D (Aqk^T rows 16 tm .. are zero before index 16 tm)
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
            if (tmv < 2) a1 = mma_frag(Rc.aq[0], dOb.sub(tnv * 16), 0, a1);
            a1 = mma_frag(Rc.aq[1], dOb.sub(tnv * 16), 32, a1);
#pragma unroll
            for (int kb = 0; kb < F::KB; ++kb) a2 = mma_frag(Rc.kh[kb], Db.sub(tnv * 16), 32 * kb, a2);
#pragma unroll
            for (int r = 0; r < 4; ++r) val[r] = scale * a1[r] + a2[r];
            dvnT.put4(tnv * 16 + frag_col(), tmv * 16 + frag_row(0), val);
        }
        {
            float* dvo = p.dvn + slot * kChunk * DV;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *(wave < VT ? dvo + (size_t)(tmv * 16 + frag_row(r)) * DV + jb + tnv * 16 + frag_col() : p.sink) = val[r];
        }
        {
            // dO^T of the chunk processed next
            const int t = tid >> 3, part = tid & 7;
#pragma unroll
            for (int k = 0; k < F::ND; ++k) dOn.put(F::ND * part + k, t, Rc.d[k]);
        }
        __syncthreads();
        // D <- scale Qg^T dO + Diag(exp G_L) D - w^T dv_new
#pragma unroll
        for (int k = 0; k < HPW; ++k) {
            const int tile = wave + kDhWaves * k;
            if (tile < TH) {
                const int tm = tile / TN, tn = tile % TN;
                f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    a1 = mma_frag(Rc.qt[k][kb], dOb.sub(tn * 16), 32 * kb, a1);
                    a2 = mma_frag(Rc.wt[k][kb], dvnT.sub(tn * 16), 32 * kb, a2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) D[k][r] = Rc.g[4 * k + r] * D[k][r] + scale * a1[r] - a2[r];
                Dn.put4(tn * 16 + frag_col(), tm * 16 + frag_row(0), D[k]);
            }
        }
    };

    if (c0 < c1) {
        {
            // dO^T of the last chunk, staged before the loop
            const ChunkRef cr = ref(c1 - 1);
            const int t = tid >> 3, part = tid & 7;
            const TIn* src = (const TIn*)p.d_o + tok_index(cr.t0 + (t < cr.len ? t : 0), h, p.H, DV) + jb + F::ND * part;
#pragma unroll
            for (int k = 0; k < F::ND; ++k) {
                const float x = Elem<TIn>::load(src, k);
                dOT0.put(F::ND * part + k, t, t < cr.len ? x : 0.f);
            }
        }
        // the operand batch of chunk c carries dO of chunk c - 1; PD batches in flight
        constexpr int PD = 2;
        F R[PD];
#pragma unroll
        for (int k = 0; k < PD; ++k) dh_load<DK, DV, BV, TIn, P>(p, slot_of(c1 - 1 - k), ref(c1 - 2 - k), h, jb, R[k]);
        int c = c1 - 1;
        for (; c - (PD - 1) >= c0; c -= PD) {
#pragma unroll
            for (int k = 0; k < PD; ++k) {
                step(c - k, R[k]);
                dh_load<DK, DV, BV, TIn, P>(p, slot_of(c - k - PD), ref(c - k - PD - 1), h, jb, R[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < PD - 1; ++k)
            if (c - k >= c0) step(c - k, R[k]);
    }
    if (p.dh0) {
#pragma unroll
        for (int k = 0; k < HPW; ++k) {
            const int tile = wave + kDhWaves * k;
            if (tile < TH) {
                const int tm = tile / TN, tn = tile % TN;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.dh0[((size_t)nh * DK + tm * 16 + frag_row(r)) * DV + jb + tn * 16 + frag_col()] = D[k][r];
            }
        }
    }
}

}  // namespace kda
