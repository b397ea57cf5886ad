// kda_bwdchunk.cuh -- the per-chunk backward (everything but the state
// gradient recurrence), one workgroup per (chunk, head), dk = 32.
//
// Given, for the chunk, the state h entering it and D = dL/dS at its end (from
// the forward recompute and the reverse scan), v_new and dv_new, it forms the
// gradients of the chunk form (kda_chunk.cuh) with respect to q, k, v, beta
// and the log-decay, then the preparation chain.  With Qg = exp(G) q,
// Kg = exp(G) k, Kh = k exp(G_L - G), u = T beta V, w = T beta Kg:
//   P1  dQg = scale dO h^T, dAqk = scale dO vn^T (s <= t), dKh = vn D^T,
//       dw = -dvn h^T, dT_v = dvn (beta V)^T, and through u:
//       dV = beta (T^T dvn), dbeta += rowsum((T^T dvn) V); dGamma_L = rowsum(h D)
//   P2  dT = dT_v + dw (beta Kg)^T, and through w:
//       dKg = beta (T^T dw), dbeta += rowsum((T^T dw) Kg)
//   P3  dA = -T^T dT T^T, strictly lower (T = (I + A)^{-1})
//   P4  the decayed pair sums of Akk = beta_t sum k_t k_s e^{G_t-G_s} and
//       Aqk = sum q_t k_s e^{G_t-G_s}: for rows t (partner s <= t) and columns s
//       (partner t >= s).  Off-diagonal 16x16 blocks are MFMA products with
//       the decay factored through a reference row r between the pair
//       (exp(G_t - G_r) exp(G_r - G_s), both at most 1): r = the first row of
//       the row block for the row sums, the last row of the column block for
//       the column sums.  Diagonal blocks use the exact exp of each difference.
//   P5  the explicit factors (Qg, Kg, Kh, exp(G_L)) are folded in as they are
//       produced; dg is the reverse in-chunk cumulative sum of dG; then the
//       gate, sigmoid and L2-norm chains.
// Gradient accumulators DQ, DK, DG live in LDS (fp32); every element is owned
// by one lane in each phase, so no atomics are used.
#pragma once

#include "kda_chunk.cuh"
#include "kda_intra.cuh"
#include "kda_mma.cuh"

namespace kda {

template <int DV, typename TIn, typename TOut, Prec P>
__global__ void __launch_bounds__(kThreads) bwd_chunk_kernel(Prm p) {
    constexpr int DK = 32, NVB = DV / 32, LR = DK + 1;  // odd stride: lanes over tokens hit distinct banks
    constexpr int L40 = 40, L72 = 72, GV = DV / 16;
    constexpr int NT4 = kChunk * kChunk / 4 / kThreads;  // float4 of T per thread
    constexpr int NH4 = DK * DV / 4 / kThreads;          // float4 of h (and D)
    constexpr int NV4 = kChunk * DV / 4 / kThreads;      // float4 of vn (and dvn)
    __shared__ __attribute__((aligned(16))) float Ks[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float Qs[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float Gs[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float DQ[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float DKa[kChunk * LR];
    __shared__ __attribute__((aligned(16))) float DG[kChunk * LR];
    __shared__ float dAd[4 * 16 * 17], dAqd[4 * 16 * 17];  // diagonal blocks of dA, dAq
    __shared__ float bet[kChunk], rnq[kChunk], rnk[kChunk];
    __shared__ float wsum[4 * 32];
    __shared__ float GL[DK], dgl[DK], colp[4 * DK];
    __shared__ float dbv[kChunk * GV], dbw[kChunk * 2], dba[kChunk * 2], rowp[kWaves * kChunk];
    constexpr int PH = 23040;
    __shared__ __attribute__((aligned(16))) float ph[PH];

    const int c = blockIdx.x, h = blockIdx.y;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tr = tid >> 2, part = tid & 3;
    const bool l2 = p.flags & 1u, gate = p.flags & 2u;
    const TIn* qin = (const TIn*)p.q;
    const TIn* kin = (const TIn*)p.k;
    const TIn* vin = (const TIn*)p.v;
    const TIn* doin = (const TIn*)p.d_o;
    const int last = cr.len - 1;
    const bool in = tr < cr.len;
    const float scale = p.scale;

    // ------------------------------------------------ every global load, up front
    float braw = 0.f;
    if (tid < kChunk && tid < cr.len) braw = p.beta[(size_t)(cr.t0 + tid) * p.H + h];
    float kx[8], qx[8], G[8], graw[8], vx[NVB][8], dox[NVB][8];
    if (in) {
        const size_t base = tok_index(cr.t0 + tr, h, p.H, DK) + 8 * part;
        load8<TIn>(kin + base, kx);
        load8<TIn>(qin + base, qx);
        load8<float>(p.g + base, graw);
#pragma unroll
        for (int b = 0; b < NVB; ++b) {
            const size_t vb = tok_index(cr.t0 + tr, h, p.H, DV) + 32 * b + 8 * part;
            load8<TIn>(vin + vb, vx[b]);
            load8<TIn>(doin + vb, dox[b]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kx[i] = qx[i] = graw[i] = 0.f;
#pragma unroll
            for (int b = 0; b < NVB; ++b) vx[b][i] = dox[b][i] = 0.f;
        }
    }
    f32x4 Tr[NT4], Hr[NH4], Dr[NH4], Vn[NV4], dVn[NV4];
    {
        const f32x4* t4 = (const f32x4*)(p.tm + slot * kChunk * kChunk);
        const f32x4* h4 = (const f32x4*)(p.hs + slot * DK * DV);
        const f32x4* d4 = (const f32x4*)(p.dhs + slot * DK * DV);
        const f32x4* v4 = (const f32x4*)(p.vn + slot * kChunk * DV);
        const f32x4* w4 = (const f32x4*)(p.dvn + slot * kChunk * DV);
#pragma unroll
        for (int i = 0; i < NT4; ++i) Tr[i] = t4[tid + kThreads * i];
#pragma unroll
        for (int i = 0; i < NH4; ++i) { Hr[i] = h4[tid + kThreads * i]; Dr[i] = d4[tid + kThreads * i]; }
#pragma unroll
        for (int i = 0; i < NV4; ++i) { Vn[i] = v4[tid + kThreads * i]; dVn[i] = w4[tid + kThreads * i]; }
    }

    // ------------------------------------------------ preparation (registers), resident tiles
    if (tid < kChunk) {
        const float b = (p.flags & 4u) ? (tid < cr.len ? sigmoid_f(braw) : 0.f) : braw;
        bet[tid] = b;
        dba[2 * tid] = 0.f;
        dba[2 * tid + 1] = 0.f;
    }
    float rk = 1.f, rq = 1.f;
    if (l2) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) { sk += kx[i] * kx[i]; sq += qx[i] * qx[i]; }
        sk += __shfl_xor(sk, 1, 64); sk += __shfl_xor(sk, 2, 64);
        sq += __shfl_xor(sq, 1, 64); sq += __shfl_xor(sq, 2, 64);
        rk = 1.0f / sqrtf(sk + kL2Eps);
        rq = 1.0f / sqrtf(sq + kL2Eps);
#pragma unroll
        for (int i = 0; i < 8; ++i) { kx[i] *= rk; qx[i] *= rq; }
        if (part == 0) { rnk[tr] = rk; rnq[tr] = rq; }
    }
    float graw_f[8];  // the raw gate input f (with the gate flag)
#pragma unroll
    for (int i = 0; i < 8; ++i) graw_f[i] = graw[i];
    if (gate && in) {
        const float eA = expf(p.A_log[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) graw[i] = -eA * softplus_f(graw[i] + p.dt_bias[h * DK + 8 * part + i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) G[i] = graw[i];
    cumsum_rows(G, wsum);  // barriers inside
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int cc = 8 * part + i;
        Ks[tr * LR + cc] = kx[i];
        Qs[tr * LR + cc] = qx[i];
        Gs[tr * LR + cc] = G[i];
        DQ[tr * LR + cc] = 0.f;
        DKa[tr * LR + cc] = 0.f;
        DG[tr * LR + cc] = 0.f;
        if (tr == last) GL[cc] = G[i];
    }
    // dGamma_L = rowsum(h . D): 16 consecutive lanes share one row c per float4 slot
    {
#pragma unroll
        for (int i = 0; i < NH4; ++i) {
            const int e4 = 4 * (tid + kThreads * i);
            const int cc = e4 / DV;
            float s = Hr[i][0] * Dr[i][0] + Hr[i][1] * Dr[i][1] + Hr[i][2] * Dr[i][2] + Hr[i][3] * Dr[i][3];
            constexpr int LPR = DV / 4;  // lanes per row of h
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off, 64);
            if ((tid % LPR) == 0) dgl[cc] = s;
        }
    }
    __syncthreads();

    // ------------------------------------------------ P1: contractions over dv
    const Tile<P> TT(ph, kChunk, L72);  // T^T [t][s], phases 1-3
#pragma unroll
    for (int i = 0; i < NT4; ++i) {
        const int e4 = 4 * (tid + kThreads * i);
        const int s = e4 >> 6, t = e4 & 63;  // T[s][t .. t+3]
#pragma unroll
        for (int m = 0; m < 4; ++m) TT.put(t + m, s, Tr[i][m]);
    }
    f32x4 aQ[2], aKh[2], aW[2], aAq[4], aT[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) aQ[i] = aKh[i] = aW[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) aAq[i] = aT[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const Tile<P> dOb(ph + 4608, kChunk, L40), vnb(ph + 7168, kChunk, L40), dvnb(ph + 9728, kChunk, L40),
            bVb(ph + 12288, kChunk, L40), hb(ph + 14848, DK, L40), Db(ph + 16128, DK, L40),
            dvnT(ph + 17408, 32, L72);
        float* Vf = ph + 19712;  // fp32 v of the column block [t][j], stride 36
        TOut* dvout = (TOut*)p.dv;
#pragma unroll
        for (int vbk = 0; vbk < NVB; ++vbk) {
            const int jb = 32 * vbk;
            __syncthreads();  // previous block's tiles consumed
            dOb.put4(tr, 8 * part, f32x4{dox[vbk][0], dox[vbk][1], dox[vbk][2], dox[vbk][3]});
            dOb.put4(tr, 8 * part + 4, f32x4{dox[vbk][4], dox[vbk][5], dox[vbk][6], dox[vbk][7]});
            {
                const float b = bet[tr];
                bVb.put4(tr, 8 * part, f32x4{b * vx[vbk][0], b * vx[vbk][1], b * vx[vbk][2], b * vx[vbk][3]});
                bVb.put4(tr, 8 * part + 4, f32x4{b * vx[vbk][4], b * vx[vbk][5], b * vx[vbk][6], b * vx[vbk][7]});
                *(f32x4*)&Vf[tr * 36 + 8 * part] = f32x4{vx[vbk][0], vx[vbk][1], vx[vbk][2], vx[vbk][3]};
                *(f32x4*)&Vf[tr * 36 + 8 * part + 4] = f32x4{vx[vbk][4], vx[vbk][5], vx[vbk][6], vx[vbk][7]};
            }
#pragma unroll
            for (int i = 0; i < NV4; ++i) {
                const int e4 = 4 * (tid + kThreads * i);
                const int t = e4 / DV, j = e4 - t * DV;
                if (j >= jb && j < jb + 32) {
                    vnb.put4(t, j - jb, Vn[i]);
                    dvnb.put4(t, j - jb, dVn[i]);
#pragma unroll
                    for (int m = 0; m < 4; ++m) dvnT.put(j - jb + m, t, dVn[i][m]);
                }
            }
#pragma unroll
            for (int i = 0; i < NH4; ++i) {
                const int e4 = 4 * (tid + kThreads * i);
                const int cc = e4 / DV, j = e4 - cc * DV;
                if (j >= jb && j < jb + 32) {
                    hb.put4(cc, j - jb, Hr[i]);
                    Db.put4(cc, j - jb, Dr[i]);
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 2; ++i) {  // [64 x 32] tiles
                const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
                aQ[i] = mma_tile(dOb.sub(16 * tm), hb.sub(16 * tn), 0, 32, aQ[i]);
                aKh[i] = mma_tile(vnb.sub(16 * tm), Db.sub(16 * tn), 0, 32, aKh[i]);
                aW[i] = mma_tile(dvnb.sub(16 * tm), hb.sub(16 * tn), 0, 32, aW[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // [64 x 64] tiles
                const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
                aAq[i] = mma_tile(dOb.sub(16 * tm), vnb.sub(16 * tn), 0, 32, aAq[i]);
                aT[i] = mma_tile(dvnb.sub(16 * tm), bVb.sub(16 * tn), 0, 32, aT[i]);
            }
            // X_u = T^T dvn: dV = beta X_u, dbeta_v = rowsum(X_u V)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
                int k0 = 16 * tm, k1 = kChunk;
                widen<P>(k0, k1);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_tile(TT.sub(16 * tm), dvnT.sub(16 * tn), k0, k1, acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tm + frag_row(r), j = 16 * tn + frag_col();
                    const float bt = bet[t];
                    if (t < cr.len) Elem<TOut>::store(dvout, tok_index(cr.t0 + t, h, p.H, DV) + jb + j, bt * acc[r]);
                    const float part_v = row16_sum(acc[r] * Vf[t * 36 + j]);
                    if (frag_col() == 0) dbv[t * GV + 2 * vbk + tn] = part_v;
                }
            }
        }
    }
    // explicit factors of Qg and Kh, as the dQg and dKh tiles come out
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
        const int cc = 16 * tn + frag_col();
        float colsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tm + frag_row(r);
            const float gt = Gs[t * LR + cc], kt = Ks[t * LR + cc], qt = Qs[t * LR + cc];
            const float gam = __expf(gt), eL = __expf(GL[cc] - gt);
            const float dqg = scale * aQ[i][r], dkh = aKh[i][r];
            const float kh = kt * eL;
            DQ[t * LR + cc] = gam * dqg;
            DKa[t * LR + cc] = eL * dkh;
            DG[t * LR + cc] = qt * gam * dqg - kh * dkh;
            colsum += t < cr.len ? kh * dkh : 0.f;
        }
        colsum += __shfl_xor(colsum, 16, 64);
        colsum += __shfl_xor(colsum, 32, 64);
        if (lane < 16) colp[tm * DK + cc] = colsum;
    }

    // ------------------------------------------------ P2: through w
    {
        const Tile<P> dwt(ph + 4608, kChunk, L40), bKg(ph + 7168, kChunk, L40), dwT(ph + 9728, DK, L72);
        __syncthreads();  // P1 tiles consumed
        {
            const float b = bet[tr];
            f32x4 v0, v1;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                v0[m] = b * __expf(G[m]) * kx[m];
                v1[m] = b * __expf(G[4 + m]) * kx[4 + m];
            }
            bKg.put4(tr, 8 * part, v0);
            bKg.put4(tr, 8 * part + 4, v1);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
            const int cc = 16 * tn + frag_col();
            f32x4 dw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dw[r] = -aW[i][r];
                dwt.put(16 * tm + frag_row(r), cc, dw[r]);
            }
            dwT.put4(cc, 16 * tm + frag_row(0), dw);
        }
        __syncthreads();
        // dT = dT_v + dw (beta Kg)^T   (dT_v already carries beta_s: it was formed with beta V)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
            aT[i] = mma_tile(dwt.sub(16 * tm), bKg.sub(16 * tn), 0, DK, aT[i]);
        }
        // X_w = T^T dw: dKg = beta X_w, dbeta_w = rowsum(X_w Kg)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 1, tn = tile & 1;
            int k0 = 16 * tm, k1 = kChunk;
            widen<P>(k0, k1);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_tile(TT.sub(16 * tm), dwT.sub(16 * tn), k0, k1, acc);
            const int cc = 16 * tn + frag_col();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tm + frag_row(r);
                const float gam = __expf(Gs[t * LR + cc]), kt = Ks[t * LR + cc];
                const float kg = gam * kt, dkg = bet[t] * acc[r];
                DKa[t * LR + cc] += gam * dkg;
                DG[t * LR + cc] += kt * gam * dkg;
                const float pb = row16_sum(acc[r] * kg);
                if (frag_col() == 0) dbw[t * 2 + tn] = pb;
            }
        }
    }

    // ------------------------------------------------ P3: dA = -T^T dT T^T
    f32x4 dAr[4];
    {
        const Tile<P> Trow(ph + 4608, kChunk, L72), dTt(ph + 9216, kChunk, L72), YT(ph + 13824, kChunk, L72);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NT4; ++i) {
            const int e4 = 4 * (tid + kThreads * i);
            Trow.put4(e4 >> 6, e4 & 63, Tr[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) dTt.put(16 * tm + frag_row(r), 16 * tn + frag_col(), aT[i][r]);
        }
        __syncthreads();
        // Y = dT T^T, stored transposed: YT[b][t]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
            int k0 = 0, k1 = 16 * (tn + 1);
            widen<P>(k0, k1);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_tile(dTt.sub(16 * tm), Trow.sub(16 * tn), k0, k1, acc);
            YT.put4(16 * tn + frag_col(), 16 * tm + frag_row(0), acc);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (tn <= tm) {
                int k0 = 16 * tm, k1 = kChunk;
                widen<P>(k0, k1);
                acc = mma_tile(TT.sub(16 * tm), YT.sub(16 * tn), k0, k1, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int a = 16 * tm + frag_row(r), bb = 16 * tn + frag_col();
                dAr[i][r] = bb < a ? -acc[r] : 0.f;
            }
        }
    }
    // scale and mask dAqk (s <= t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tm + frag_row(r), s = 16 * tn + frag_col();
            aAq[i][r] = s <= t ? scale * aAq[i][r] : 0.f;
        }
    }

    // ------------------------------------------------ P4: decayed pair sums
    float r_dbA = 0.f;  // this lane's share of dbeta from Akk (rows t = lane, this wave's channels)
    {
        // row sums: R'k[t] = sum_{s<t} dA[t][s] k_s e^{G_t-G_s},  Rq[t] = sum_{s<=t} dAq[t][s] k_s e^{..}
        const Tile<P> dAt(ph, kChunk, L72), dAqt(ph + 4608, kChunk, L72);
        auto KcT = [&](int i) { return Tile<P>(ph + 9216 + 2304 * i, DK, L72); };
        __syncthreads();  // P3 tiles consumed
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
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
        // KcT_I[c][s] = k_s e^{G_{16 I} - G_s} for s < 16 I, else 0
#pragma unroll
        for (int I = 1; I <= 3; ++I) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int cc = 8 * part + i;
                const float v = tr < 16 * I ? kx[i] * __expf(Gs[(16 * I) * LR + cc] - G[i]) : 0.f;
                KcT(I - 1).put(cc, tr, v);
            }
        }
        __syncthreads();
        // 6 tasks: (I, column tile of c)
        for (int task = wave; task < 6; task += kWaves) {
            const int I = 1 + task / 2, tn = task & 1;
            int k0 = 0, k1 = 16 * I;
            widen<P>(k0, k1);
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
            const Tile<P> kc = KcT(I - 1);
            ak = mma_tile(dAt.sub(16 * I), kc.sub(16 * tn), k0, k1, ak);
            aq = mma_tile(dAqt.sub(16 * I), kc.sub(16 * tn), k0, k1, aq);
            const int cc = 16 * tn + frag_col();
            const float gr = Gs[(16 * I) * LR + cc];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + frag_row(r);
                const float e = __expf(Gs[t * LR + cc] - gr);
                const float rkv = e * ak[r], rqv = e * aq[r];
                const float kt = Ks[t * LR + cc], qt = Qs[t * LR + cc], bt = bet[t];
                DKa[t * LR + cc] += bt * rkv;
                DQ[t * LR + cc] += rqv;
                DG[t * LR + cc] += bt * kt * rkv + qt * rqv;
                const float pb = row16_sum(kt * rkv);
                if (frag_col() == 0) dba[t * 2 + tn] = pb;
            }
        }
    }
    {
        // column sums: Ck[s] = sum_{t>s} beta_t dA[t][s] k_t e^{G_t-G_s}, Cq[s] = sum_{t>=s} dAq[t][s] q_t e^{..}
        const Tile<P> bdAT(ph, kChunk, L72), dAqT(ph + 4608, kChunk, L72);
        auto KxT = [&](int j) { return Tile<P>(ph + 9216 + 2304 * j, DK, L72); };
        auto QxT = [&](int j) { return Tile<P>(ph + 16128 + 2304 * j, DK, L72); };
        __syncthreads();  // row-sum tiles consumed
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tile = wave + kWaves * i, tm = tile >> 2, tn = tile & 3;
            const int s = 16 * tn + frag_col();
            f32x4 bd;
#pragma unroll
            for (int r = 0; r < 4; ++r) bd[r] = bet[16 * tm + frag_row(r)] * dAr[i][r];
            bdAT.put4(s, 16 * tm + frag_row(0), bd);
            dAqT.put4(s, 16 * tm + frag_row(0), aAq[i]);
        }
        // KxT_J[c][t] = k_t e^{G_t - G_{16 J + 15}} for t > 16 J + 15, else 0 (QxT_J likewise)
#pragma unroll
        for (int J = 0; J < 3; ++J) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int cc = 8 * part + i;
                const bool after = tr > 16 * J + 15;
                const float e = after ? __expf(G[i] - Gs[(16 * J + 15) * LR + cc]) : 0.f;
                KxT(J).put(cc, tr, kx[i] * e);
                QxT(J).put(cc, tr, qx[i] * e);
            }
        }
        __syncthreads();
        for (int task = wave; task < 6; task += kWaves) {
            const int J = task / 2, tn = task & 1;
            int k0 = 16 * J + 16, k1 = kChunk;
            widen<P>(k0, k1);
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
            ak = mma_tile(bdAT.sub(16 * J), KxT(J).sub(16 * tn), k0, k1, ak);
            aq = mma_tile(dAqT.sub(16 * J), QxT(J).sub(16 * tn), k0, k1, aq);
            const int cc = 16 * tn + frag_col();
            const float gr = Gs[(16 * J + 15) * LR + cc];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * J + frag_row(r);
                const float e = __expf(gr - Gs[s * LR + cc]);
                const float cs = e * (ak[r] + aq[r]);
                DKa[s * LR + cc] += cs;
                DG[s * LR + cc] -= Ks[s * LR + cc] * cs;
            }
        }
        __syncthreads();
    }
    // diagonal blocks, exact pairwise decays; lane = token t, waves take channels
    {
        const int t = lane, blk = t >> 4, t0b = blk * 16;
        for (int cc = wave; cc < DK; cc += kWaves) {
            const float gt = Gs[t * LR + cc], kt = Ks[t * LR + cc], qt = Qs[t * LR + cc];
            float rkv = 0.f, rqv = 0.f, ck = 0.f, cq = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int s = t0b + u;
                const float gs = Gs[s * LR + cc], ks = Ks[s * LR + cc], qs = Qs[s * LR + cc];
                const float ad_ts = dAd[blk * 272 + (t & 15) * 17 + u];   // dA[t][s]
                const float aq_ts = dAqd[blk * 272 + (t & 15) * 17 + u];  // dAq[t][s]
                const float ad_st = dAd[blk * 272 + u * 17 + (t & 15)];   // dA[s][t]
                const float aq_st = dAqd[blk * 272 + u * 17 + (t & 15)];  // dAq[s][t]
                if (s <= t) {
                    const float e = __expf(gt - gs) * ks;
                    rkv += ad_ts * e;
                    rqv += aq_ts * e;
                }
                if (s >= t) {
                    const float e = __expf(gs - gt);
                    ck += bet[s] * ad_st * ks * e;
                    cq += aq_st * qs * e;
                }
            }
            const float bt = bet[t];
            DKa[t * LR + cc] += bt * rkv + ck + cq;
            DQ[t * LR + cc] += rqv;
            DG[t * LR + cc] += bt * kt * rkv + qt * rqv - kt * (ck + cq);
            r_dbA += kt * rkv;
        }
    }
    rowp[wave * kChunk + lane] = r_dbA;
    __syncthreads();

    // ------------------------------------------------ P5: dg, gate chain, outputs
    // (a) lane = token: add dG_L to the last row, reverse in-chunk cumsum -> DG holds dg
    {
        const int t = lane;
        for (int cc = wave; cc < DK; cc += kWaves) {
            float dG = DG[t * LR + cc];
            if (t == last) {
                float sl = 0.f;
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) sl += colp[tm * DK + cc];
                dG += sl + __expf(GL[cc]) * dgl[cc];
            }
            if (t >= cr.len) dG = 0.f;
            float sfx = dG;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_down(sfx, off, 64);
                if (t + off < 64) sfx += o;
            }
            DG[t * LR + cc] = sfx;
        }
    }
    __syncthreads();
    // (b) coalesced pass, thread = (row tr, 8 channels): gate, sigmoid and L2 chains, stores
    {
        const int t = tr;
        float dgv[8], dqv[8], dkv[8], qh[8], kh[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int cc = 8 * part + i;
            dgv[i] = DG[t * LR + cc];
            dqv[i] = DQ[t * LR + cc];
            dkv[i] = DKa[t * LR + cc];
            qh[i] = Qs[t * LR + cc];
            kh[i] = Ks[t * LR + cc];
        }
        float pa = 0.f;
        if (gate) {
            const float eA = expf(p.A_log[h]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // graw still holds this row's raw f (the staging layout is the same)
                const float x = in ? graw_f[i] + p.dt_bias[h * DK + 8 * part + i] : 0.f;
                const float df = in ? dgv[i] * (-eA) * dsoftplus_f(x) : 0.f;
                pa += in ? dgv[i] * (-eA * softplus_f(x)) : 0.f;
                dgv[i] = df;
            }
            // column sums of df over the chunk: 16 rows per wave (lanes 4 apart), then waves
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float cs = dgv[i];
#pragma unroll
                for (int off = 4; off < 64; off <<= 1) cs += __shfl_xor(cs, off, 64);
                if (lane < 4) colp[wave * DK + 8 * part + i] = cs;
            }
        }
        float dotq = 0.f, dotk = 0.f;
        if (l2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) { dotq += qh[i] * dqv[i]; dotk += kh[i] * dkv[i]; }
            dotq += __shfl_xor(dotq, 1, 64); dotq += __shfl_xor(dotq, 2, 64);
            dotk += __shfl_xor(dotk, 1, 64); dotk += __shfl_xor(dotk, 2, 64);
            const float r_q = rnq[t], r_k = rnk[t];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                dqv[i] = r_q * (dqv[i] - dotq * qh[i]);
                dkv[i] = r_k * (dkv[i] - dotk * kh[i]);
            }
        }
        if (in) {
            const size_t gi = tok_index(cr.t0 + t, h, p.H, DK) + 8 * part;
            store8<TOut>((TOut*)p.dq + gi, dqv);
            store8<TOut>((TOut*)p.dk + gi, dkv);
            store8<float>(p.dg + gi, dgv);
        }
        if (gate) {
            const float pw = wave_sum(pa);
            if (lane == 0) wsum[wave] = pw;
        }
    }
    if (tid < kChunk) {
        const int t = tid;
        float db = 0.f;
        for (int w = 0; w < kWaves; ++w) db += rowp[w * kChunk + t];
        db += dba[t * 2] + dba[t * 2 + 1] + dbw[t * 2] + dbw[t * 2 + 1];
        for (int g = 0; g < GV; ++g) db += dbv[t * GV + g];
        if (t < cr.len) {
            if (p.flags & 4u) db *= bet[t] * (1.f - bet[t]);
            p.dbeta[(size_t)(cr.t0 + t) * p.H + h] = db;
        }
    }
    if (gate) {
        __syncthreads();
        if (tid < DK) p.part_dt[slot * DK + tid] = (colp[tid] + colp[DK + tid]) + (colp[2 * DK + tid] + colp[3 * DK + tid]);
        if (tid == 0) p.part_a[slot] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    }
}

}  // namespace kda
