// kda_bwdchunk.cuh -- the per-chunk backward (everything but the state
// gradient recurrence), one workgroup of 8 waves per (chunk, head), dk = 32.
//
// Given, for the chunk, the state h entering it and D = dL/dS at its end (from
// the forward and the reverse scan), v_new and dv_new, it forms the gradients
// of the chunk form (kda_chunk.cuh) with respect to q, k, v, beta and the
// log-decay, then the preparation chain.  With Qg = exp(G) q, Kg = exp(G) k,
// Kh = k exp(G_L - G), u = T beta V, w = T beta Kg:
//   P1  dQg = scale dO h^T, dAqk = scale dO vn^T (s <= t), dKh = vn D^T,
//       dw = -dvn h^T, dT_v = dvn (beta V)^T, and through u:
//       dV = beta (T^T dvn), dbeta += rowsum((T^T dvn) V); dGamma_L = rowsum(h D)
//   P2  dT = dT_v + dw (beta Kg)^T, and through w:
//       dKg = beta (T^T dw), dbeta += rowsum((T^T dw) Kg)
//   P3  dA = -T^T dT T^T, strictly lower (T = (I + A)^{-1})
//   P4  the decayed pair sums of Akk = beta_t sum k_t k_s e^{G_t-G_s} and
//       Aqk = sum q_t k_s e^{G_t-G_s}: for rows t (partner s <= t) and columns s
//       (partner t >= s).  Off-diagonal 16x16 blocks (t in block I, s in J < I)
//       are MFMA products with the decay split at the first row of I and the
//       last row of J (three factors, each at most 1): the outer two scale the
//       operands, one staged copy each, the middle one each block pair's
//       product.  In the bf16 path the diagonal blocks are split the same way
//       into 4-token sub-blocks (4-deep fp32 products between sub-blocks, exact
//       decays for the pairs inside one); the fp32 path takes the exact exp of
//       every difference in the diagonal blocks.
//   P5  the explicit factors (Qg, Kg, Kh, exp(G_L)) are folded in as they are
//       produced; dg is the reverse in-chunk cumulative sum of dG; then the
//       gate, sigmoid and L2-norm chains.
// Gradient accumulators DQ, DK, DG live in LDS (fp32); every element is owned
// by one lane in each phase, so no atomics are used.
//
// Latency: the workgroup holds ~156 KB of LDS, so one runs per CU; 8 waves
// give two per SIMD to cover LDS and MFMA latency.  Epilogues read their LDS
// operands unconditionally (selects, not branches) so the reads issue
// together, and cross-lane sums use DPP / permlane swaps.
#pragma once

#include "kda_chunk.cuh"
#include "kda_intra.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kBcThreads = 512, kBcWaves = 8;

// Staging of T's values as loaded (fp32, or with bf16 inputs the hi/lo split
// words of tpk_load4_split carried as raw bits): four consecutive values of a
// row, or value m of such a group.
template <int C>
__device__ __forceinline__ void put_t4(const STile<Prec::F32, C>& T, int r, int k, f32x4 x) { T.put4(r, k, x); }
template <int C>
__device__ __forceinline__ void put_t4(const STile<Prec::BF3, C>& T, int r, int k, f32x4 x) {
    const tpk_words w = __builtin_bit_cast(tpk_words, x);
    T.put4_split(r, k, u32x2v{w[0], w[1]}, u32x2v{w[2], w[3]});
}
template <int C>
__device__ __forceinline__ void put_t1(const STile<Prec::F32, C>& T, int r, int k, f32x4 x, int m) { T.put(r, k, x[m]); }
template <int C>
__device__ __forceinline__ void put_t1(const STile<Prec::BF3, C>& T, int r, int k, f32x4 x, int m) {
    const tpk_words w = __builtin_bit_cast(tpk_words, x);
    const int sh = 16 * (m & 1);
    T.put_split(r, k, (uint16_t)(w[m >> 1] >> sh), (uint16_t)(w[2 + (m >> 1)] >> sh));
}

template <int DV, typename TIn, typename TOut, Prec P>
__global__ void __launch_bounds__(kBcThreads) bwd_chunk_kernel(Prm p) {
    constexpr int NTH = kBcThreads, NW = kBcWaves;
    constexpr int DK = 32, NVB = DV / 32, LR = DK + 1;  // odd stride: lanes over tokens hit distinct banks
    constexpr int GV = DV / 16;
    using T32 = STile<P, 32>;  // operand tiles of 32 and 64 values per row
    using T64 = STile<P, 64>;
    constexpr int NT4 = kChunk * kChunk / 4 / NTH;  // float4 of T per thread
    constexpr int NH4 = DK * DV / 4 / NTH;          // float4 of h (and D)
    constexpr int NV4 = kChunk * DV / 4 / NTH;      // float4 of vn (and dvn)
    static_assert(NT4 >= 1 && NH4 >= 1 && NV4 >= 1, "shapes");
    __shared__ __attribute__((aligned(16))) float Ks[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float Qs[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float Gs[kChunk * LR];
    // gradient accumulators DQ, DKa, DG, one array (P0 uses it as fp32 staging
    // before the first accumulator is written)
    __shared__ __attribute__((aligned(16))) float ACC[3 * kChunk * LR];
    float* const DQ = ACC;
    float* const DKa = ACC + kChunk * LR;
    float* const DG = ACC + 2 * kChunk * LR;
    __shared__ float dAd[4 * 16 * 17], dAqd[4 * 16 * 17];  // diagonal blocks of dA, dAq
    __shared__ __attribute__((aligned(16))) float bet[kChunk];
    __shared__ float rnq[kChunk], rnk[kChunk];
    __shared__ float wsum[NW];
    __shared__ float GL[DK], dgl[DK], colp[NW * DK];
    __shared__ float dbv[kChunk * GV], dbw[kChunk * 2], dba[kChunk * 2], rowp[NW * kChunk];
    constexpr int PH = 23040;
    __shared__ __attribute__((aligned(16))) float ph[PH];

    const int c = blockIdx.x, h = blockIdx.y;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int tr = tid >> 3, part = tid & 7;  // row-wise work: token tr, channels 4 part .. 4 part + 3
    const bool l2 = p.flags & 1u, gate = p.flags & 2u;
    const TIn* qin = (const TIn*)p.q;
    const TIn* kin = (const TIn*)p.k;
    const TIn* vin = (const TIn*)p.v;
    const TIn* doin = (const TIn*)p.d_o;
    const int last = cr.len - 1;
    const bool in = tr < cr.len;
    const float scale = p.scale;

    // ------------------------------------------------ the inputs' global loads, up front
    // (the gate parameters first, so that no later load waits behind the rest)
    float braw = 0.f, alog = 0.f, dtb[4] = {0.f, 0.f, 0.f, 0.f};
    if (gate) {
        alog = p.A_log[h];
        load4<float>(p.dt_bias + h * DK + 4 * part, dtb);
    }
    // rows past the chunk end load row 0 (always valid) and are zeroed after the loads
    const int trc = in ? tr : 0;
    if (tid < kChunk) braw = p.beta[(size_t)(cr.t0 + (tid < cr.len ? tid : 0)) * p.H + h];
    float kx[4], qx[4], G[4], graw[4], vx[NVB][4], dox[NVB][4];
    {
        const size_t base = tok_index(cr.t0 + trc, h, p.H, DK) + 4 * part;
        load4<TIn>(kin + base, kx);
        load4<TIn>(qin + base, qx);
        load4<float>(p.g + base, graw);
    }
    f32x4 Tr[NT4], Hr[NH4], Dr[NH4];
    AFrag<P> fa[2];  // Aqk^T rows 16 (w >> 1) .., k-blocks (w >> 2) .. 1 (P0)
    if (tid < kChunk && tid >= cr.len) braw = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kx[i] = in ? kx[i] : 0.f;
        qx[i] = in ? qx[i] : 0.f;
        graw[i] = in ? graw[i] : 0.f;
    }

    // ------------------------------------------------ preparation (registers), resident tiles
    if (tid < kChunk) {
        const float b = (p.flags & 4u) ? (tid < cr.len ? sigmoid_f(braw) : 0.f) : braw;
        bet[tid] = b;
        dba[2 * tid] = 0.f;
        dba[2 * tid + 1] = 0.f;
    }
    if (l2) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) { sk += kx[i] * kx[i]; sq += qx[i] * qx[i]; }
        sk = sum8(sk);
        sq = sum8(sq);
        const float rk = rsqrt_hw(sk + kL2Eps), rq = rsqrt_hw(sq + kL2Eps);
#pragma unroll
        for (int i = 0; i < 4; ++i) { kx[i] *= rk; qx[i] *= rq; }
        if (part == 0) { rnk[tr] = rk; rnq[tr] = rq; }
    }
    const float graw_f[4] = {graw[0], graw[1], graw[2], graw[3]};  // the raw gate input f (gate flag)
    const float eA = exp_hw(alog);
    if (gate && in) {
#pragma unroll
        for (int i = 0; i < 4; ++i) graw[i] = -eA * softplus_f(graw[i] + dtb[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int cc = 4 * part + i;
        Ks[tr * LR + cc] = kx[i];
        Qs[tr * LR + cc] = qx[i];
        Gs[tr * LR + cc] = graw[i] * kLog2e;  // base-2 log-decay (cumulated in place below)
    }
    __syncthreads();
    // v, dO and the chunk's intermediates (Aqk^T, T, h, D'), issued once the
    // preparation's inputs have arrived: issued with them, they shared the
    // bandwidth of the start of every round (every CU loads at once) and
    // delayed the preparation.
#pragma unroll
    for (int b = 0; b < NVB; ++b) {  // v and dO (rows past the end: zeroed in P0)
        const size_t vb = tok_index(cr.t0 + trc, h, p.H, DV) + 32 * b + 4 * part;
        load4<TIn>(vin + vb, vx[b]);
        load4<TIn>(doin + vb, dox[b]);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)  // Aqk^T row block tm reaches t >= 16 tm: k-blocks tm >> 1 .. 1
        if (kb >= (wave >> 2))
            load_afrag(fa[kb], frag_rec(p.aqT + slot * kChunk * kChunk, 16 * (wave >> 1) + (lane & 15), kb, 2));
    {
        const float* tpk = p.tm + slot * kTPacked;
        const f32x4* h4 = (const f32x4*)(p.hs + slot * DK * DV);
        const f32x4* d4 = (const f32x4*)(p.dhs + slot * DK * DV);
#pragma unroll
        for (int i = 0; i < NT4; ++i) {
            const int e4 = 4 * (tid + NTH * i);
            if constexpr (P == Prec::BF3)  // (the hi/lo split words, kept as raw bits)
                Tr[i] = __builtin_bit_cast(f32x4, tpk_load4_split(tpk, e4 >> 6, e4 & 63));
            else
                Tr[i] = tpk_load4(tpk, e4 >> 6, e4 & 63);
        }
#pragma unroll
        for (int i = 0; i < NH4; ++i) { Hr[i] = h4[tid + NTH * i]; Dr[i] = d4[tid + NTH * i]; }
    }
    {
        // in-chunk cumulative log-decay G, in place in Gs: wave w scans columns 4 w .. 4 w + 3
        static_assert(NW * 4 == DK, "four columns per wave");
        float x[4];
        const int col = 4 * wave + (lane >> 4), s = lane & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = Gs[(4 * s + i) * LR + col];
        col_scan16<false>(x, Gs, LR, col, s);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) G[i] = Gs[tr * LR + 4 * part + i];
    if (tr == last) {
#pragma unroll
        for (int i = 0; i < 4; ++i) GL[4 * part + i] = G[i];
    }
    // (h and D', loaded last, are first needed here: the barrier above and the
    // scan did not wait for them)
    // dGamma_L (read in P5) = rowsum(h . D): 16 consecutive lanes share one row c per float4 slot
#pragma unroll
    for (int i = 0; i < NH4; ++i) {
        const int e4 = 4 * (tid + NTH * i);
        const int cc = e4 / DV;
        const float s = sum16(Hr[i][0] * Dr[i][0] + Hr[i][1] * Dr[i][1] + Hr[i][2] * Dr[i][2] + Hr[i][3] * Dr[i][3]);
        static_assert(DV == 64, "one row of h per 16 lanes");
        if ((lane & 15) == 0) dgl[cc] = s;
    }
    // h and D' again, rows 16 (w & 1) + (lane & 15), as the register fragments of P1's
    // products: issued now, so that they arrive during P0
    f32x4 hraw[2][2], draw[2][2];  // this lane's 8 values of h / D' rows 16 an + (lane & 15), per k-block
    {
        const int row = 16 * (wave & 1) + (lane & 15), c8 = 8 * (lane >> 4);
        const float* hs = p.hs + slot * DK * DV + (size_t)row * DV + c8;
        const float* ds = p.dhs + slot * DK * DV + (size_t)row * DV + c8;
#pragma unroll
        for (int kb = 0; kb < NVB; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                hraw[kb][q] = *(const f32x4*)(hs + 32 * kb + 4 * q);
                draw[kb][q] = *(const f32x4*)(ds + 32 * kb + 4 * q);
            }
    }

    // ------------------------------------------------ P0: v_new and dv_new of the chunk
    //   v_new  = T (beta V - (beta Kg) h)      (= u - w h)
    //   dv_new = Kh D' + scale Aqk^T dO         (D' = dL/dS at the chunk end)
    // Aqk^T comes as row fragments from the intra-chunk kernel's fragment-form array;
    // T, beta Kg, Kh, h^T, D'^T and dO^T are staged in LDS from registers.  Wave w
    // forms 64x64 tiles (w >> 1, 2 (w & 1) + e), e = 0, 1; the results pass
    // through fp32 LDS staging into the row-major registers Vn, dVn that the
    // dv-side phase stages from.
    f32x4 Vn[NV4], dVn[NV4];
    {
        const int tm = wave >> 1, tn0 = 2 * (wave & 1);
        const int lr = lane & 15, lg = lane >> 4;
        // ph: [0, 4608) T;  [4608, 7168) beta Kg;  [7168, 9728) Kh;  [9728, 12288) h^T;
        //     [12288, 14848) D'^T;  [14848, 19456) dO^T;  then Z^T over [4608, 9216) and
        //     v_new (fp32 [t][68]) over [9728, 14080).  ACC: V, then dv_new (fp32 [t][68]).
        const T64 TRW(ph, kChunk), DOT(ph + 14848, DV);
        const T32 BKG(ph + 4608, kChunk), KHt(ph + 7168, kChunk), HTt(ph + 9728, DV), DTt(ph + 12288, DV);
        float* const VS = ACC;  // V, overwritten in place by dv_new
        float* const VNs = ph + 9728;
        static_assert(14848 + DV * 72 <= PH && 9728 + kChunk * 68 <= 14848 && kChunk * 68 <= 3 * kChunk * LR,
                      "P0 staging must fit");
        {
            const float b = bet[tr];
            f32x4 xg, xh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gL = Gs[last * LR + 4 * part + i];  // in-chunk decay at the last token
                xg[i] = b * exp2_hw(G[i]) * kx[i];
                xh[i] = kx[i] * exp2_hw(gL - G[i]);
            }
            BKG.put4(tr, 4 * part, xg);
            KHt.put4(tr, 4 * part, xh);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vx[vb][i] = in ? vx[vb][i] : 0.f;
                    dox[vb][i] = in ? dox[vb][i] : 0.f;
                }
                *(f32x4*)&VS[tr * 68 + 32 * vb + 4 * part] = f32x4{vx[vb][0], vx[vb][1], vx[vb][2], vx[vb][3]};
#pragma unroll
                for (int m = 0; m < 4; ++m) DOT.put_hi(32 * vb + 4 * part + m, tr, dox[vb][m]);  // dO: bf16 numbers
            }
        }
#pragma unroll
        for (int i = 0; i < NT4; ++i) {
            const int e4 = 4 * (tid + NTH * i);
            put_t4(TRW, e4 >> 6, e4 & 63, Tr[i]);
        }
#pragma unroll
        for (int i = 0; i < NH4; ++i) {  // h and D' rows c, columns j .. j + 3 -> h^T, D'^T [j][c]
            const int e4 = 4 * (tid + NTH * i);
            const int cc = e4 / DV, j = e4 - cc * DV;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                HTt.put(j + m, cc, Hr[i][m]);
                DTt.put(j + m, cc, Dr[i][m]);
            }
        }
        __syncthreads();
        f32x4 z[2];
        AFrag<P> fbk, fkh;  // this wave's rows of beta Kg and Kh, shared by both column tiles
        load_frag(fbk, BKG.sub(16 * tm), 0);
        load_frag(fkh, KHt.sub(16 * tm), 0);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int tn = tn0 + e;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            AFrag<P> fy;
            load_frag(fy, HTt.sub(16 * tn), 0);
            const f32x4 y = mma_ff(fbk, fy, zero);
            load_frag(fy, DTt.sub(16 * tn), 0);
            const f32x4 x1 = mma_ff(fkh, fy, zero);
            f32x4 x2 = zero;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb >= (tm >> 1)) {
                    load_frag_hi(fy, DOT.sub(16 * tn), 32 * kb);
                    x2 = mma_ff_bh(fa[kb], fy, x2);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tm + 4 * lg + r;
                float* vd = &VS[t * 68 + 16 * tn + lr];  // V here, replaced by dv_new
                z[e][r] = bet[t] * (*vd) - y[r];
                *vd = x1[r] + scale * x2[r];
            }
        }
        __syncthreads();  // beta Kg, Kh, h^T, D'^T consumed
        const T64 ZT(ph + 4608, DV);  // Z^T [j][s]
#pragma unroll
        for (int e = 0; e < 2; ++e) ZT.put4(16 * (tn0 + e) + lr, 16 * tm + 4 * lg, z[e]);
        __syncthreads();
        {
            AFrag<P> ft[2], fy;  // this wave's rows of T (lower triangular: k-blocks 0 .. tm >> 1)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb <= (tm >> 1)) load_frag(ft[kb], TRW.sub(16 * tm), 32 * kb);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int tn = tn0 + e;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb <= (tm >> 1)) {
                        load_frag(fy, ZT.sub(16 * tn), 32 * kb);
                        acc = mma_ff(ft[kb], fy, acc);
                    }
#pragma unroll
                for (int r = 0; r < 4; ++r) VNs[(16 * tm + 4 * lg + r) * 68 + 16 * tn + lr] = acc[r];
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int e4 = 4 * (tid + NTH * i);
            const int t = e4 / DV, j = e4 - t * DV;
            Vn[i] = *(const f32x4*)&VNs[t * 68 + j];
            dVn[i] = *(const f32x4*)&VS[t * 68 + j];
        }
    }

    // ------------------------------------------------ P1: contractions over dv
    const T64 TT(ph, kChunk);  // T^T [t][s], phases 1-3
#pragma unroll
    for (int i = 0; i < NT4; ++i) {
        const int e4 = 4 * (tid + NTH * i);
        const int s = e4 >> 6, t = e4 & 63;  // T[s][t .. t+3]
#pragma unroll
        for (int m = 0; m < 4; ++m) put_t1(TT, t + m, s, Tr[i], m);
    }
    // [64 x 32] results: wave w owns tile (w >> 1, w & 1); [64 x 64]: tiles w, w + 8 -> (tile >> 2, tile & 3)
    const int am = wave >> 1, an = wave & 1;
    f32x4 aQ = {0.f, 0.f, 0.f, 0.f}, aKh = aQ, aW = aQ, aAq[2], aT[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) aAq[i] = aT[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        // All dv columns at once (two k-blocks per product).  ph: T^T, v_new, dv_new,
        // dv_new^T, dO; ACC (not yet accumulating): v.  dO and v are bf16 numbers:
        // hi parts only.  h and D' (rows c, columns j, row-major fp32) come
        // as register fragments from their fp32 arrays.
        const T64 vnb(ph + 4608, kChunk), dvnb(ph + 9216, kChunk), dvnT(ph + 13824, DV), dOb(ph + 18432, kChunk);
        const T64 Vh(ACC, kChunk);
        static_assert(18432 + kChunk * (DV + 8) <= PH && kChunk * (DV + 8) <= 3 * kChunk * LR, "P1 staging must fit");
        __syncthreads();  // P0's readers of ph and ACC are done
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
            dOb.put4_hi(tr, 32 * vb + 4 * part, f32x4{dox[vb][0], dox[vb][1], dox[vb][2], dox[vb][3]});
            Vh.put4_hi(tr, 32 * vb + 4 * part, f32x4{vx[vb][0], vx[vb][1], vx[vb][2], vx[vb][3]});
        }
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int e4 = 4 * (tid + NTH * i);
            const int t = e4 / DV, j = e4 - t * DV;
            vnb.put4(t, j, Vn[i]);
            dvnb.put4(t, j, dVn[i]);
#pragma unroll
            for (int m = 0; m < 4; ++m) dvnT.put(j + m, t, dVn[i][m]);
        }
        __syncthreads();
        // dQg = dO h^T, dw = -dvn h^T, dKh = vn D^T: this wave's tile (am, an)
#pragma unroll
        for (int kb = 0; kb < NVB; ++kb) {
            AFrag<P> fh, fa, fb;
            {
                const float xh[8] = {hraw[kb][0][0], hraw[kb][0][1], hraw[kb][0][2], hraw[kb][0][3],
                                     hraw[kb][1][0], hraw[kb][1][1], hraw[kb][1][2], hraw[kb][1][3]};
                const float xd[8] = {draw[kb][0][0], draw[kb][0][1], draw[kb][0][2], draw[kb][0][3],
                                     draw[kb][1][0], draw[kb][1][1], draw[kb][1][2], draw[kb][1][3]};
                make_frag(fh, xh);
                make_frag(fb, xd);
            }
            load_frag_hi(fa, dOb.sub(16 * am), 32 * kb);
            aQ = mma_ff_ah(fa, fh, aQ);
            load_frag(fa, dvnb.sub(16 * am), 32 * kb);
            aW = mma_ff(fa, fh, aW);
            load_frag(fa, vnb.sub(16 * am), 32 * kb);
            aKh = mma_ff(fa, fb, aKh);
        }
        // dAqk = dO vn^T: tiles w, w + 8, which share the column tile w & 3; and
        // dT_v = dvn (beta V)^T = (dvn V^T) diag(beta), held transposed (aT: tiles (w & 3,
        // w >> 2 + 2 i) of dT^T), so that a lane's four values are consecutive s of a row
        // t of dT when it is staged
        {
            const int tn = wave & 3;
#pragma unroll
            for (int kb = 0; kb < NVB; ++kb) {
                AFrag<P> fv, fvh, fa;
                load_frag(fv, vnb.sub(16 * tn), 32 * kb);
                load_frag_hi(fvh, Vh.sub(16 * tn), 32 * kb);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tm = (wave + NW * i) >> 2;
                    load_frag_hi(fa, dOb.sub(16 * tm), 32 * kb);
                    aAq[i] = mma_ff_ah(fa, fv, aAq[i]);
                    load_frag(fa, dvnb.sub(16 * tm), 32 * kb);
                    aT[i] = mma_ff_ah(fvh, fa, aT[i]);
                }
            }
            const f32x4 bs = *(const f32x4*)&bet[16 * tn + frag_row(0)];  // beta of this lane's rows s
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) aT[i][r] *= bs[r];
        }
        // X_u = T^T dvn, formed transposed: tiles (an + 2 e, am) of X_u^T = dvn^T T, so
        // that a lane holds four consecutive columns j of one row t of dV = beta X_u
        // (one 8-byte store); dbeta_v = rowsum(X_u V)
        {
            TOut* dvout = (TOut*)p.dv;
            AFrag<P> ft[2], fy;  // T^T rows am: zero before index 16 am, so k-blocks (am >> 1) .. 1
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb >= (am >> 1)) load_frag(ft[kb], TT.sub(16 * am), 32 * kb);
            const int t = 16 * am + frag_col();
            const float bt = bet[t];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int jt = an + 2 * e;  // 16-column tile of dv
                const int j0 = 16 * jt + frag_row(0);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb >= (am >> 1)) {
                        load_frag(fy, dvnT.sub(16 * jt), 32 * kb);
                        acc = mma_ff(fy, ft[kb], acc);
                    }
                const f32x4 vv = Vh.get4_hi(t, j0);
                const float part_v = sum_rows((acc[0] * vv[0] + acc[1] * vv[1]) + (acc[2] * vv[2] + acc[3] * vv[3]));
                if (lane < 16) dbv[t * GV + jt] = part_v;
                const float o[4] = {bt * acc[0], bt * acc[1], bt * acc[2], bt * acc[3]};
                if (t < cr.len) store4<TOut>(dvout + tok_index(cr.t0 + t, h, p.H, DV) + j0, o);
            }
        }
    }

    // ------------------------------------------------ P2: through w
    {
        const T32 dwt(ph + 4608, kChunk), bKg(ph + 7168, kChunk);
        const T64 dwT(ph + 9728, DK);
        __syncthreads();  // P1 tiles consumed (and ACC free for the accumulators)
        // explicit factors of Qg and Kh, as the dQg and dKh tiles come out
        {
            const int cc = 16 * an + frag_col();
            const float glc = GL[cc];
            float gt[4], kt[4], qt[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * am + frag_row(r);
                gt[r] = Gs[t * LR + cc];
                kt[r] = Ks[t * LR + cc];
                qt[r] = Qs[t * LR + cc];
            }
            float colsum = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * am + frag_row(r);
                const float gam = exp2_hw(gt[r]), eL = exp2_hw(glc - gt[r]);
                const float dqg = scale * aQ[r], dkh = aKh[r];
                const float kh = kt[r] * eL;
                DQ[t * LR + cc] = gam * dqg;
                DKa[t * LR + cc] = eL * dkh;
                DG[t * LR + cc] = qt[r] * gam * dqg - kh * dkh;
                colsum += t < cr.len ? kh * dkh : 0.f;
            }
            colsum = sum_rows(colsum);
            if (lane < 16) colp[am * DK + cc] = colsum;
        }
        {
            const float b = bet[tr];
            f32x4 v0;
#pragma unroll
            for (int m = 0; m < 4; ++m) v0[m] = b * exp2_hw(G[m]) * kx[m];
            bKg.put4(tr, 4 * part, v0);
        }
        {
            const int cc = 16 * an + frag_col();
            f32x4 dw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dw[r] = -aW[r];
                dwt.put(16 * am + frag_row(r), cc, dw[r]);
            }
            dwT.put4(cc, 16 * am + frag_row(0), dw);
        }
        __syncthreads();
        // dT = dT_v + dw (beta Kg)^T, transposed as aT   (dT_v already carries beta_s: it was
        // formed with beta V)
        {
            AFrag<P> fb, fa;  // both tiles w, w + 8 share the column tile w & 3
            load_frag(fb, bKg.sub(16 * (wave & 3)), 0);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                load_frag(fa, dwt.sub(16 * ((wave + NW * i) >> 2)), 0);
                aT[i] = mma_ff(fb, fa, aT[i]);
            }
        }
        // X_w = T^T dw: dKg = beta X_w, dbeta_w = rowsum(X_w Kg)
        {
            int k0 = 16 * am, k1 = kChunk;
            widen<P>(k0, k1);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_tile(TT.sub(16 * am), dwT.sub(16 * an), k0, k1, acc);
            const int cc = 16 * an + frag_col();
            float gt[4], kt[4], bt[4], dk0[4], dg0[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * am + frag_row(r);
                gt[r] = Gs[t * LR + cc];
                kt[r] = Ks[t * LR + cc];
                bt[r] = bet[t];
                dk0[r] = DKa[t * LR + cc];
                dg0[r] = DG[t * LR + cc];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * am + frag_row(r);
                const float gam = exp2_hw(gt[r]);
                const float kg = gam * kt[r], dkg = bt[r] * acc[r];
                DKa[t * LR + cc] = dk0[r] + gam * dkg;
                DG[t * LR + cc] = dg0[r] + kt[r] * gam * dkg;
                const float pb = row16_sum(acc[r] * kg);
                if (frag_col() == 0) dbw[t * 2 + an] = pb;
            }
        }
    }

    // ------------------------------------------------ P3: dA = -T^T dT T^T
    f32x4 dAr[2];
    {
        const T64 Trow(ph + 4608, kChunk), dTt(ph + 9216, kChunk), YT(ph + 13824, kChunk);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NT4; ++i) {
            const int e4 = 4 * (tid + NTH * i);
            put_t4(Trow, e4 >> 6, e4 & 63, Tr[i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + NW * i, tm = tile >> 2, tn = tile & 3;
            dTt.put4(16 * tm + frag_col(), 16 * tn + frag_row(0), aT[i]);  // row t, s .. s + 3
        }
        __syncthreads();
        // Y = dT T^T, stored transposed: YT[b][t].  This wave's tiles w, w + 8 share
        // the column tile tn = w & 3, whose T rows are zero past index 16 tn + 15.
        const int tn = wave & 3, nkb = (16 * tn + 47) / 32;  // k-blocks of T rows tn that can be nonzero
        {
            AFrag<P> fb[2], fa;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (kb < nkb) load_frag(fb[kb], Trow.sub(16 * tn), 32 * kb);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tm = (wave + NW * i) >> 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb < nkb) {
                        load_frag(fa, dTt.sub(16 * tm), 32 * kb);
                        acc = mma_ff(fa, fb[kb], acc);
                    }
                YT.put4(16 * tn + frag_col(), 16 * tm + frag_row(0), acc);
            }
        }
        __syncthreads();
        {
            // dA tile (tm, tn) = -(T^T rows tm) Y^T: T^T rows tm are zero before index 16 tm,
            // so tiles w (tm < 2) take k-blocks 0 and 1, tiles w + 8 (tm >= 2) k-block 1 only
            AFrag<P> fy1, fa;
            load_frag(fy1, YT.sub(16 * tn), 32);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tm = (wave + NW * i) >> 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (tn <= tm) {
                    if (i == 0) {
                        AFrag<P> fy0;
                        load_frag(fy0, YT.sub(16 * tn), 0);
                        load_frag(fa, TT.sub(16 * tm), 0);
                        acc = mma_ff(fa, fy0, acc);
                    }
                    load_frag(fa, TT.sub(16 * tm), 32);
                    acc = mma_ff(fa, fy1, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = 16 * tm + frag_row(r), bb = 16 * tn + frag_col();
                    dAr[i][r] = bb < a ? -acc[r] : 0.f;
                }
            }
        }
    }
    // scale and mask dAqk (s <= t)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tile = wave + NW * i, tm = tile >> 2, tn = tile & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tm + frag_row(r), s = 16 * tn + frag_col();
            aAq[i][r] = s <= t ? scale * aAq[i][r] : 0.f;
        }
    }

    // ------------------------------------------------ P4: decayed pair sums
    // Off-diagonal 16x16 blocks (t in block I, s in block J < I) split the decay
    // at the first row a_I = 16 I of I and the last row b_J = 16 J + 15 of J:
    //   exp(G_t - G_s) = exp(G_t - G_{a_I}) exp(G_{a_I} - G_{b_J}) exp(G_{b_J} - G_s),
    // each factor at most 1 (s <= b_J < a_I <= t).  The outer factors scale one
    // staged copy of each operand (every token by its own block's reference);
    // the middle factor, one number per channel and block pair, scales that
    // pair's 16-deep product.
    if constexpr (P == Prec::BF3) {
        // All seven operand tiles fit in LDS at once, so one staging phase serves both
        // sums, and wave (block b, channels 16 tn ..) forms the row sums of b (over the
        // blocks J < b) and its column sums (over the blocks I > b): b + (3 - b) = three
        // 16-deep block products on every wave, and each wave alone owns the
        // accumulator rows it updates.  The same wave then takes the pairs of its
        // diagonal block b, so these sums are complete when they are added in.
        const T64 dAt(ph, kChunk), dAqt(ph + 4096, kChunk), bdAT(ph + 8192, kChunk), dAqT(ph + 12288, kChunk);
        const T64 KcT(ph + 16384, DK);  // [c][s] = k_s e^{G_{b(s)} - G_s}, b(s) the last row of s's block
        // [c][t] = k_t e^{G_t - G_{a(t)}} and q_t e^{..}, a(t) the first row of t's block
        const T64 KxT(ph + 18432, DK), QxT(ph + 20480, DK);
        static_assert(20480 + 2048 <= PH, "P4 tiles must fit (bf16 hi/lo tiles)");
        __syncthreads();  // P3 tiles consumed
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + NW * i, tm = tile >> 2, tn = tile & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tm + frag_row(r), s = 16 * tn + frag_col();
                dAt.put(t, s, dAr[i][r]);
                dAqt.put(t, s, aAq[i][r]);
                if (tm == tn) {
                    dAd[tm * 272 + (t & 15) * 17 + (s & 15)] = dAr[i][r];
                    dAqd[tm * 272 + (t & 15) * 17 + (s & 15)] = aAq[i][r];
                }
            }
            const int s = 16 * tn + frag_col();
            f32x4 bd;
#pragma unroll
            for (int r = 0; r < 4; ++r) bd[r] = bet[16 * tm + frag_row(r)] * dAr[i][r];
            bdAT.put4(s, 16 * tm + frag_row(0), bd);
            dAqT.put4(s, 16 * tm + frag_row(0), aAq[i]);
        }
        {
            // channel c, tokens t0 .. t0 + 3 of one 16-token block, read down the columns of
            // the fp32 rows (odd stride: no bank conflicts), so that each tile row takes four
            // consecutive tokens in one store
            static_assert(NTH == DK * kChunk / 4, "one four-token group per thread");
            const int c = tid & 31, t0 = 4 * (tid >> 5), b0 = t0 & ~15;
            const float gend = Gs[(b0 + 15) * LR + c], gst = Gs[b0 * LR + c];
            f32x4 kc4, kx4, qx4;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int t = t0 + m;
                const float g = Gs[t * LR + c], kv = Ks[t * LR + c], qv = Qs[t * LR + c];
                kc4[m] = kv * exp2_hw(gend - g);
                const float e = exp2_hw(g - gst);
                kx4[m] = kv * e;
                qx4[m] = qv * e;
            }
            KcT.put4(c, t0, kc4);
            KxT.put4(c, t0, kx4);
            QxT.put4(c, t0, qx4);
        }
        __syncthreads();
        {
            // Wave (block bk, channels 16 tn ..).  Lane l holds rows 16 bk + 4 g + r
            // (r = 0..3) of column cc: the whole 4-token sub-block g = l >> 4.  The
            // decays are split at this sub-block's first row a (row sums) and last
            // row b (column sums), so the outer factors below are per row and
            // every middle factor is per lane.
            const int bk = wave >> 1, tn = wave & 1;
            const int g4 = lane >> 4, n = lane & 15;
            const int cc = 16 * tn + n;
            const int ra = 16 * bk + 4 * g4;
            const float gA = Gs[ra * LR + cc];        // G at the sub-block's first row
            const float gB = Gs[(ra + 3) * LR + cc];  // and at its last row
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 ak = zero, aq = zero, ck = zero, cq = zero;
#pragma unroll
            for (int J = 0; J < 3; ++J)
                if (J < bk) {  // row sums: partners in the earlier block J (16-deep products)
                    const f32x4 pk = mma_tile_k16(dAt.sub(16 * bk), KcT.sub(16 * tn), 16 * J, zero);
                    const f32x4 pq = mma_tile_k16(dAqt.sub(16 * bk), KcT.sub(16 * tn), 16 * J, zero);
                    const float m = exp2_hw(gA - Gs[(16 * J + 15) * LR + cc]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ak[r] = fmaf(m, pk[r], ak[r]);
                        aq[r] = fmaf(m, pq[r], aq[r]);
                    }
                }
#pragma unroll
            for (int I = 1; I < 4; ++I)
                if (I > bk) {  // column sums: partners in the later block I
                    const f32x4 pk = mma_tile_k16(bdAT.sub(16 * bk), KxT.sub(16 * tn), 16 * I, zero);
                    const f32x4 pq = mma_tile_k16(dAqT.sub(16 * bk), QxT.sub(16 * tn), 16 * I, zero);
                    const float m = exp2_hw(Gs[(16 * I) * LR + cc] - gB);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ck[r] = fmaf(m, pk[r], ck[r]);
                        cq[r] = fmaf(m, pq[r], cq[r]);
                    }
                }
            // The diagonal block bk, by its 4-token sub-blocks: pairs in different
            // sub-blocks as 4-deep fp32 products (v_mfma_f32_16x16x4_f32: lane l
            // gives A[l & 15][l >> 4] and B[l >> 4][l & 15]) with the decay split
            // at the sub-blocks' boundary rows, each factor at most 1; the middle
            // factor is zero where the partner sub-block is not on the summed side.
            const float* dAb = dAd + bk * 272;   // dA[16 bk + i][16 bk + j] at i * 17 + j
            const float* dAqb = dAqd + bk * 272;
#pragma unroll
            for (int J = 0; J < 3; ++J) {  // row sums: partner sub-block J < g
                const int s = 16 * bk + 4 * J + g4;  // this lane's B row (k index l >> 4)
                const float gbJ = Gs[(16 * bk + 4 * J + 3) * LR + cc];
                const float b = Ks[s * LR + cc] * exp2_hw(gbJ - Gs[s * LR + cc]);
                const f32x4 pk = __builtin_amdgcn_mfma_f32_16x16x4f32(dAb[n * 17 + 4 * J + g4], b, zero, 0, 0, 0);
                const f32x4 pq = __builtin_amdgcn_mfma_f32_16x16x4f32(dAqb[n * 17 + 4 * J + g4], b, zero, 0, 0, 0);
                const float m = J < g4 ? exp2_hw(gA - gbJ) : 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ak[r] = fmaf(m, pk[r], ak[r]);
                    aq[r] = fmaf(m, pq[r], aq[r]);
                }
            }
#pragma unroll
            for (int I = 1; I < 4; ++I) {  // column sums: partner sub-block I > g
                const int ti = 4 * I + g4;  // this lane's B row within the block
                const float gaI = Gs[(16 * bk + 4 * I) * LR + cc];
                const float e = exp2_hw(Gs[(16 * bk + ti) * LR + cc] - gaI);
                const float bk_ = Ks[(16 * bk + ti) * LR + cc] * e, bq = Qs[(16 * bk + ti) * LR + cc] * e;
                const float a1 = bet[16 * bk + ti] * dAb[ti * 17 + n];  // beta_t dA[t][s], s = 16 bk + n
                const f32x4 pk = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bk_, zero, 0, 0, 0);
                const f32x4 pq = __builtin_amdgcn_mfma_f32_16x16x4f32(dAqb[ti * 17 + n], bq, zero, 0, 0, 0);
                const float m = I > g4 ? exp2_hw(gaI - gB) : 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ck[r] = fmaf(m, pk[r], ck[r]);
                    cq[r] = fmaf(m, pq[r], cq[r]);
                }
            }
            float gt[4], kt[4], qt[4], bt[4], dk0[4], dq0[4], dg0[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = ra + r;
                gt[r] = Gs[t * LR + cc];
                kt[r] = Ks[t * LR + cc];
                qt[r] = Qs[t * LR + cc];
                bt[r] = bet[t];
                dk0[r] = DKa[t * LR + cc];
                dq0[r] = DQ[t * LR + cc];
                dg0[r] = DG[t * LR + cc];
            }
            // pairs inside the sub-block (all in this lane): exact decays
            float rkx[4], rqx[4], ckx[4], cqx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float aqd = dAqb[(4 * g4 + i) * 17 + 4 * g4 + i];  // dAq[t][t], decay 1
                rkx[i] = 0.f;
                rqx[i] = aqd * kt[i];
                ckx[i] = 0.f;
                cqx[i] = aqd * qt[i];
            }
#pragma unroll
            for (int i = 1; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < i; ++j) {  // t = row i, s = row j < i
                    const float da = dAb[(4 * g4 + i) * 17 + 4 * g4 + j], daq = dAqb[(4 * g4 + i) * 17 + 4 * g4 + j];
                    const float e = exp2_hw(gt[i] - gt[j]);
                    const float kse = kt[j] * e, kte = kt[i] * e;
                    rkx[i] = fmaf(da, kse, rkx[i]);
                    rqx[i] = fmaf(daq, kse, rqx[i]);
                    ckx[j] = fmaf(bt[i] * da, kte, ckx[j]);
                    cqx[j] = fmaf(daq, qt[i] * e, cqx[j]);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = ra + r;
                const float e = exp2_hw(gt[r] - gA), e2 = exp2_hw(gB - gt[r]);
                const float rkv = fmaf(e, ak[r], rkx[r]), rqv = fmaf(e, aq[r], rqx[r]);
                const float cs = fmaf(e2, ck[r] + cq[r], ckx[r] + cqx[r]);
                DKa[t * LR + cc] = dk0[r] + bt[r] * rkv + cs;
                DQ[t * LR + cc] = dq0[r] + rqv;
                DG[t * LR + cc] = dg0[r] + bt[r] * kt[r] * rkv + qt[r] * rqv - kt[r] * cs;
                const float pb = row16_sum(kt[r] * rkv);
                if (n == 0) dba[t * 2 + tn] = pb;
            }
        }
        __syncthreads();
    } else {
    {
        // row sums: R'k[t] = sum_{s<t} dA[t][s] k_s e^{G_t-G_s},  Rq[t] = sum_{s<=t} dAq[t][s] k_s e^{..}
        const T64 dAt(ph, kChunk), dAqt(ph + 4608, kChunk);
        const T64 KcT(ph + 9216, DK);  // [c][s] = k_s e^{G_{b(s)} - G_s}, b(s) the last row of s's block
        float gend[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gend[i] = Gs[(16 * (tr >> 4) + 15) * LR + 4 * part + i];
        __syncthreads();  // P3 tiles consumed
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + NW * i, tm = tile >> 2, tn = tile & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tm + frag_row(r), s = 16 * tn + frag_col();
                dAt.put(t, s, dAr[i][r]);
                dAqt.put(t, s, aAq[i][r]);
                if (tm == tn) {
                    dAd[tm * 272 + (t & 15) * 17 + (s & 15)] = dAr[i][r];
                    dAqd[tm * 272 + (t & 15) * 17 + (s & 15)] = aAq[i][r];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) KcT.put(4 * part + i, tr, kx[i] * exp2_hw(gend[i] - G[i]));
        __syncthreads();
        // 6 tasks: (I, column tile of c), on waves 0..5
        if (wave < 6) {
            const int I = 1 + (wave >> 1), tn = wave & 1;
            const int cc = 16 * tn + frag_col();
            const float gr = Gs[(16 * I) * LR + cc];  // G at a_I
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < 3; ++J)
                if (J < I) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 pk = mma_tile_k16(dAt.sub(16 * I), KcT.sub(16 * tn), 16 * J, zero);
                    const f32x4 pq = mma_tile_k16(dAqt.sub(16 * I), KcT.sub(16 * tn), 16 * J, zero);
                    const float m = exp2_hw(gr - Gs[(16 * J + 15) * LR + cc]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ak[r] = fmaf(m, pk[r], ak[r]);
                        aq[r] = fmaf(m, pq[r], aq[r]);
                    }
                }
            float gt[4], kt[4], qt[4], bt[4], dk0[4], dq0[4], dg0[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + frag_row(r);
                gt[r] = Gs[t * LR + cc];
                kt[r] = Ks[t * LR + cc];
                qt[r] = Qs[t * LR + cc];
                bt[r] = bet[t];
                dk0[r] = DKa[t * LR + cc];
                dq0[r] = DQ[t * LR + cc];
                dg0[r] = DG[t * LR + cc];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + frag_row(r);
                const float e = exp2_hw(gt[r] - gr);
                const float rkv = e * ak[r], rqv = e * aq[r];
                DKa[t * LR + cc] = dk0[r] + bt[r] * rkv;
                DQ[t * LR + cc] = dq0[r] + rqv;
                DG[t * LR + cc] = dg0[r] + bt[r] * kt[r] * rkv + qt[r] * rqv;
                const float pb = row16_sum(kt[r] * rkv);
                if (frag_col() == 0) dba[t * 2 + tn] = pb;
            }
        }
    }
    {
        // column sums: Ck[s] = sum_{t>s} beta_t dA[t][s] k_t e^{G_t-G_s}, Cq[s] = sum_{t>=s} dAq[t][s] q_t e^{..}
        const T64 bdAT(ph, kChunk), dAqT(ph + 4608, kChunk);
        // [c][t] = k_t e^{G_t - G_{a(t)}} and q_t e^{..}, a(t) the first row of t's block
        const T64 KxT(ph + 9216, DK), QxT(ph + 9216 + 2304, DK);
        float gst[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gst[i] = Gs[(16 * (tr >> 4)) * LR + 4 * part + i];
        __syncthreads();  // row-sum tiles consumed
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + NW * i, tm = tile >> 2, tn = tile & 3;
            const int s = 16 * tn + frag_col();
            f32x4 bd;
#pragma unroll
            for (int r = 0; r < 4; ++r) bd[r] = bet[16 * tm + frag_row(r)] * dAr[i][r];
            bdAT.put4(s, 16 * tm + frag_row(0), bd);
            dAqT.put4(s, 16 * tm + frag_row(0), aAq[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 4 * part + i;
            const float e = exp2_hw(G[i] - gst[i]);
            KxT.put(cc, tr, kx[i] * e);
            QxT.put(cc, tr, qx[i] * e);
        }
        __syncthreads();
        if (wave < 6) {
            const int J = wave >> 1, tn = wave & 1;
            const int cc = 16 * tn + frag_col();
            const float gr = Gs[(16 * J + 15) * LR + cc];  // G at b_J
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = 1; I < 4; ++I)
                if (I > J) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 pk = mma_tile_k16(bdAT.sub(16 * J), KxT.sub(16 * tn), 16 * I, zero);
                    const f32x4 pq = mma_tile_k16(dAqT.sub(16 * J), QxT.sub(16 * tn), 16 * I, zero);
                    const float m = exp2_hw(Gs[(16 * I) * LR + cc] - gr);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ak[r] = fmaf(m, pk[r], ak[r]);
                        aq[r] = fmaf(m, pq[r], aq[r]);
                    }
                }
            float gs[4], ks[4], dk0[4], dg0[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * J + frag_row(r);
                gs[r] = Gs[s * LR + cc];
                ks[r] = Ks[s * LR + cc];
                dk0[r] = DKa[s * LR + cc];
                dg0[r] = DG[s * LR + cc];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * J + frag_row(r);
                const float e = exp2_hw(gr - gs[r]);
                const float cs = e * (ak[r] + aq[r]);
                DKa[s * LR + cc] = dk0[r] + cs;
                DG[s * LR + cc] = dg0[r] - ks[r] * cs;
            }
        }
        __syncthreads();
    }
    // diagonal blocks (fp32 path), exact pairwise decays; lane = token t (row t >> 4 of the
    // wave = diagonal block), each wave four channels.  The partner token s of
    // the same block sits in lane s of the same 16-lane row, so its values come
    // by DPP row broadcast from this lane's registers; the dA entries of (t, s)
    // and (s, t) are read once per partner for all four channels.
    {
        const int t = lane, blk = t >> 4, tl = t & 15;
        const float bt = bet[t];
        float gtv[DK / NW], ktv[DK / NW], qtv[DK / NW];
        float rkv[DK / NW], rqv[DK / NW], ck[DK / NW], cq[DK / NW];
#pragma unroll
        for (int jc = 0; jc < DK / NW; ++jc) {
            const int cc = wave + NW * jc;
            gtv[jc] = Gs[t * LR + cc];
            ktv[jc] = Ks[t * LR + cc];
            qtv[jc] = Qs[t * LR + cc];
            rkv[jc] = rqv[jc] = ck[jc] = cq[jc] = 0.f;
        }
        const float* dAr_ = dAd + blk * 272;
        const float* dAqr = dAqd + blk * 272;
        static_for16([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            const float ad_ts = dAr_[tl * 17 + u], aq_ts = dAqr[tl * 17 + u];  // dA[t][s], dAq[t][s]
            const float ad_st = dAr_[u * 17 + tl], aq_st = dAqr[u * 17 + tl];  // dA[s][t], dAq[s][t]
            const float bad = row_bcast<u>(bt) * ad_st;                         // beta_s dA[s][t]
            const bool lower = u <= tl;
#pragma unroll
            for (int jc = 0; jc < DK / NW; ++jc) {
                const float gs = row_bcast<u>(gtv[jc]), ks = row_bcast<u>(ktv[jc]), qs = row_bcast<u>(qtv[jc]);
                // One exp per pair: e^{G_t - G_s} for s <= t, e^{G_s - G_t} for s >= t.  The
                // stored diagonal blocks are zero outside their triangles (dA strictly lower,
                // dAq lower), so each product below only counts on its own side.
                const float x = gtv[jc] - gs;
                const float e = exp2_hw(lower ? x : -x);
                const float ek = e * ks;
                rkv[jc] = fmaf(ad_ts, ek, rkv[jc]);
                rqv[jc] = fmaf(aq_ts, ek, rqv[jc]);
                ck[jc] = fmaf(bad, ek, ck[jc]);
                cq[jc] = fmaf(aq_st * qs, e, cq[jc]);
            }
        });
        float r_dbA = 0.f;  // this lane's share of dbeta from Akk
#pragma unroll
        for (int jc = 0; jc < DK / NW; ++jc) {
            const int cc = wave + NW * jc;
            const float kt = ktv[jc], qt = qtv[jc];
            const float dk0 = DKa[t * LR + cc], dq0 = DQ[t * LR + cc], dg0 = DG[t * LR + cc];
            DKa[t * LR + cc] = dk0 + (bt * rkv[jc] + ck[jc] + cq[jc]);
            DQ[t * LR + cc] = dq0 + rqv[jc];
            DG[t * LR + cc] = dg0 + (bt * kt * rkv[jc] + qt * rqv[jc] - kt * (ck[jc] + cq[jc]));
            r_dbA += kt * rkv[jc];
        }
        rowp[wave * kChunk + lane] = r_dbA;
    }
    __syncthreads();
    }  // (diagonal blocks: fp32 path)

    // ------------------------------------------------ P5: dg, gate chain, outputs
    // (a) dG_L into the last row, rows past the end zeroed, reverse cumulative sum -> DG holds dg
    {
        // (wave w scans columns 4 w .. 4 w + 3; the scan's closing barrier also orders
        // these reads of colp before its reuse below)
        const int cs = 4 * wave + (lane >> 4), s = lane & 15;
        const float extra = ((colp[cs] + colp[DK + cs]) + (colp[2 * DK + cs] + colp[3 * DK + cs])) +
                            exp2_hw(GL[cs]) * dgl[cs];
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * s + i;
            const float v = DG[t * LR + cs];
            x[i] = t < cr.len ? v + (t == last ? extra : 0.f) : 0.f;
        }
        col_scan16<true>(x, DG, LR, cs, s);
    }
    // (b) row-wise pass, thread = (token tr, 4 channels): gate, sigmoid and L2 chains, stores
    {
        const int t = tr;
        float dgv[4], dqv[4], dkv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 4 * part + i;
            dgv[i] = DG[t * LR + cc];
            dqv[i] = DQ[t * LR + cc];
            dkv[i] = DKa[t * LR + cc];
        }
        float pa = 0.f;
        if (gate) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = in ? graw_f[i] + dtb[i] : 0.f;
                const float df = in ? dgv[i] * (-eA) * dsoftplus_f(x) : 0.f;
                pa += dgv[i] * graw[i];  // graw: the log-decay -e^A softplus(x) (zero past the end)
                dgv[i] = df;
            }
            // column sums of df over this wave's 8 rows (lanes 8 apart), per wave
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float cs = sum_rows(sum_x8(dgv[i]));
                if (lane < 8) colp[wave * DK + 4 * part + i] = cs;
            }
        }
        if (l2) {
            float dotq = 0.f, dotk = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { dotq += qx[i] * dqv[i]; dotk += kx[i] * dkv[i]; }
            dotq = sum8(dotq);
            dotk = sum8(dotk);
            const float r_q = rnq[t], r_k = rnk[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dqv[i] = r_q * (dqv[i] - dotq * qx[i]);
                dkv[i] = r_k * (dkv[i] - dotk * kx[i]);
            }
        }
        if (in) {
            const size_t gi = tok_index(cr.t0 + t, h, p.H, DK) + 4 * part;
            store4<TOut>((TOut*)p.dq + gi, dqv);
            store4<TOut>((TOut*)p.dk + gi, dkv);
            store4<float>(p.dg + gi, dgv);
        }
        if (gate) {
            const float pw = wave_sum(pa);
            if (lane == 0) wsum[wave] = pw;
        }
    }
    if (tid < kChunk) {
        const int t = tid;
        float db = 0.f;
        if constexpr (P != Prec::BF3) {  // the fp32 path's diagonal blocks
#pragma unroll
            for (int w = 0; w < NW; ++w) db += rowp[w * kChunk + t];
        }
        db += dba[t * 2] + dba[t * 2 + 1] + dbw[t * 2] + dbw[t * 2 + 1];
#pragma unroll
        for (int g = 0; g < GV; ++g) db += dbv[t * GV + g];
        if (t < cr.len) {
            if (p.flags & 4u) db *= bet[t] * (1.f - bet[t]);
            p.dbeta[(size_t)(cr.t0 + t) * p.H + h] = db;
        }
    }
    if (gate) {
        __syncthreads();
        if (tid < DK) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) s += colp[w * DK + tid];
            p.part_dt[slot * DK + tid] = s;
        }
        if (tid == 0) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) s += wsum[w];
            p.part_a[slot] = s;
        }
    }
}

}  // namespace kda
