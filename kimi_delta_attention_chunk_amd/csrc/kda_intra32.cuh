// kda_intra32.cuh -- the intra-chunk kernel for dk = 32, dv = 64, eight waves
// per workgroup.
//
// It computes what intra_kernel (kda_intra.cuh) computes for this shape, the
// chunk as an affine map of the state entering it, from the same algebra:
//   pass 1: k, q (L2-normalised if flagged), the gate and the in-chunk
//     cumulative decay G; the Gram matrices Akk and Aqk (off-diagonal 16x16
//     blocks as MFMA products of operands scaled through the block's first
//     row, diagonal blocks from exact pairwise decays);
//   solve: T = (I + Akk)^{-1} (kda_chunk.cuh);
//   pass 2: w = T beta exp(G) k and u = T beta v;
//   pass 3: P = Diag(exp G_L) - Kh^T w, hh = Kh^T u, qh = scale (Qg - Aqk w),
//     ol = scale Aqk u (and Aqk^T, T for the backward if requested).
// The difference is the split of the work over 512 threads instead of 256:
// eight threads per token row (four channels each) in the staging steps, one
// diagonal pair per thread, three w / u tiles per wave and pass 3's products
// over eight waves.  The LDS plan is unchanged (about 78 KB), so two
// workgroups still share a CU, now with four waves per SIMD instead of two:
// the kernel is bound by latency, and the extra waves hide more of it.
#pragma once

#include "kda_intra.cuh"

namespace kda {

constexpr int kI32Threads = 512;
constexpr int kI32Waves = kI32Threads / 64;

template <typename TIn, Prec P>
__global__ void __launch_bounds__(kI32Threads, 2) intra32_kernel(Prm p) {  // two workgroups per CU
    constexpr int DK = 32, DV = 64, NVB = DV / 32;
    // LDS, as in intra_kernel:
    //   KQG  Kb | Qb | Gb   fp32 [t][c]; after pass 1: Aqk staging, BT tiles, w^T / u^T
    //   S1   Kr | Qr | Kc   MFMA tiles of the off-diagonal Gram blocks; then Akk; then T (tile); then Qg, Kh^T
    //   Tm   T, fp32 (the solve)
    constexpr int LB8 = kCB32 + 8, LA = kChunk + 8, LQ = kChunk + 1;
    constexpr int S1F = (48 + 48 + 96) * LB8;
    __shared__ __attribute__((aligned(16))) float KQG[3 * kChunk * kLB];
    __shared__ __attribute__((aligned(16))) float S1[S1F];
    __shared__ __attribute__((aligned(16))) float Tm[kChunk * kLD];
    __shared__ __attribute__((aligned(16))) float bet[kChunk];
    __shared__ float seg[16 * 32];  // column-scan segment totals (4 rows per thread)
    __shared__ float glS[DK];       // exp(G_L)
    static_assert(kChunk * kLD <= S1F && kChunk * LA <= S1F, "Akk and the T tile must fit in S1");
    static_assert(kCB32 * LA <= 3 * kChunk * kLB, "a BT tile must fit in KQG");
    static_assert(kChunk * LQ <= 3 * kChunk * kLB, "the Aqk staging must fit in KQG");
    static_assert(kI32Threads == 8 * kChunk, "eight threads per token row");
    static_assert(P != Prec::BF3 || sizeof(TIn) == 2, "the bf16 path has bf16 inputs (v is a bf16 number)");

    float* Kb = KQG;
    float* Qb = KQG + kChunk * kLB;
    float* Gb = KQG + 2 * kChunk * kLB;
    using T32 = STile<P, 32>;
    using T64 = STile<P, 64>;
    static_assert(STile<Prec::F32, 32>::ld == LB8 && STile<Prec::F32, 64>::ld == LA, "tile footprints");
    const T32 Kr(S1, 48);
    const T32 Qr(S1 + 48 * LB8, 48);
    const T32 Kc(S1 + 96 * LB8, 96);
    float* A = S1;             // fp32 Akk, after pass 1
    const T64 Tt(S1, kChunk);  // T as an MFMA operand, after the solve

    const int c = blockIdx.x, h = blockIdx.y;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int tr = threadIdx.x >> 3, ch = 4 * (threadIdx.x & 7);  // token row, first of its four channels
    const bool l2 = p.flags & 1u;
    const TIn* qin = (const TIn*)p.q;
    const TIn* kin = (const TIn*)p.k;
    const TIn* vin = (const TIn*)p.v;
    const int last = cr.len - 1;
    const bool in = tr < cr.len;

    // ---- the chunk's global loads, the gate parameters first
    const bool gate = p.flags & 2u;
    float kx[4], qx[4], G[4], vx[NVB][4], dtb[4];
    float braw = 0.f, alog = 0.f;
    if (gate) {
        alog = p.A_log[h];
        load4<float>(p.dt_bias + h * DK + ch, dtb);
    }
    // rows past the chunk end load row 0 (always valid) and are zeroed after the loads
    const int trc = in ? tr : 0;
    if (threadIdx.x < kChunk) braw = p.beta[(size_t)(cr.t0 + (threadIdx.x < cr.len ? threadIdx.x : 0)) * p.H + h];
    {
        const size_t base = tok_index(cr.t0 + trc, h, p.H, DK) + ch;
        load4<TIn>(kin + base, kx);
        load4<TIn>(qin + base, qx);
        load4<float>(p.g + base, G);
    }
    if (threadIdx.x < kChunk && threadIdx.x >= cr.len) braw = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kx[i] = in ? kx[i] : 0.f;
        qx[i] = in ? qx[i] : 0.f;
        G[i] = in ? G[i] : 0.f;
    }
    // ---- preparation in registers: beta, L2 norms (eight lanes per row), gate
    if (threadIdx.x < kChunk) bet[threadIdx.x] = (p.flags & 4u) ? (threadIdx.x < cr.len ? sigmoid_f(braw) : 0.f) : braw;
    if (l2) {
        float sk = (kx[0] * kx[0] + kx[1] * kx[1]) + (kx[2] * kx[2] + kx[3] * kx[3]);
        float sq = (qx[0] * qx[0] + qx[1] * qx[1]) + (qx[2] * qx[2] + qx[3] * qx[3]);
        sk = sum8(sk);
        sq = sum8(sq);
        const float rk = rsqrt_hw(sk + kL2Eps), rq = rsqrt_hw(sq + kL2Eps);
#pragma unroll
        for (int i = 0; i < 4; ++i) { kx[i] *= rk; qx[i] *= rq; }
    }
    if (gate && in) {
        const float eA = exp_hw(alog);
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i] = -eA * softplus_f(G[i] + dtb[i]);
    }
    // v, first needed in pass 2: issued once the preparation's inputs have arrived
    // (rows past the chunk end are zeroed where v is used)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) load4<TIn>(vin + tok_index(cr.t0 + trc, h, p.H, DV) + 32 * vb + ch, vx[vb]);

    // ---- pass 1: stage, scan G, scaled operands, Gram blocks
    *(f32x4*)&Kb[tr * kLB + ch] = f32x4{kx[0], kx[1], kx[2], kx[3]};
    *(f32x4*)&Qb[tr * kLB + ch] = f32x4{qx[0], qx[1], qx[2], qx[3]};
    *(f32x4*)&Gb[tr * kLB + ch] = f32x4{G[0] * kLog2e, G[1] * kLog2e, G[2] * kLog2e, G[3] * kLog2e};  // base 2
    __syncthreads();
    {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = Gb[(4 * (threadIdx.x >> 5) + i) * kLB + (threadIdx.x & 31)];
        col_scan_regs<false>(x, Gb, kLB, seg);  // in-chunk cumulative sum G; ends with a barrier
    }
    {
        const f32x4 g4 = *(const f32x4*)&Gb[tr * kLB + ch];
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i] = g4[i];
    }
    // Kh = k exp(G_L - G) (kept for pass 3) and the scaled Gram operands: rows of
    // block I >= 1 scaled by exp(G_t - G_{16 I}), and for each column block's
    // reference row r = 16 J the rows s < r scaled by exp(G_r - G_s)
    float khs[4];
    {
        const int I = tr >> 4;
        f32x4 kr, qr, kc[3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = ch + i;
            const float gt = G[i];
            khs[i] = kx[i] * exp2_hw(Gb[last * kLB + cc] - gt);
            const float e = exp2_hw(gt - Gb[16 * (I >= 1 ? I : 1) * kLB + cc]);
            kr[i] = kx[i] * e;
            qr[i] = qx[i] * e;
#pragma unroll
            for (int J = 1; J <= 3; ++J) kc[J - 1][i] = kx[i] * exp2_hw(Gb[16 * J * kLB + cc] - gt);
        }
        if (I >= 1) {
            Kr.put4(tr - 16, ch, kr);
            Qr.put4(tr - 16, ch, qr);
        }
#pragma unroll
        for (int J = 1; J <= 3; ++J)
            if (tr < 16 * J) Kc.put4(kc_off(J) + tr, ch, kc[J - 1]);
    }
    __syncthreads();
    // off-diagonal Gram tiles: 12 (6 of Akk, 6 of Aqk), one or two per wave
    f32x4 gacc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        gacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tau = wave + kI32Waves * i;
        if (tau < 12) {
            const int pr = tau % 6, kind = tau / 6;  // kind 0: Akk, 1: Aqk
            int I, J;
            gram_pair(pr, I, J);
            const T32 Aop = (kind == 0 ? Kr : Qr).sub((I - 1) * 16);
            gacc[i] = mma_tile(Aop, Kc.sub(kc_off(I) + 16 * J), 0, kCB32, gacc[i]);
        }
    }
    // diagonal blocks, exact pairwise decays: the 4 x 120 pairs s < t, one per
    // thread; then Aqk[t][t] = q_t . k_t (no decay) over the row's eight lanes
    float dkk = 0.f, dqk = 0.f;
    const int pidx = threadIdx.x;
    int pt = 0, ps = 0;
    if (pidx < kDiagPairs) {
        diag_pair(pidx, pt, ps);
        f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aqv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c4 = 0; c4 < kCB32; c4 += 4) {
            const f32x4 gt = *(const f32x4*)&Gb[pt * kLB + c4];
            const f32x4 gs = *(const f32x4*)&Gb[ps * kLB + c4];
            const f32x4 ks = *(const f32x4*)&Kb[ps * kLB + c4];
            const f32x4 kt = *(const f32x4*)&Kb[pt * kLB + c4];
            const f32x4 qt = *(const f32x4*)&Qb[pt * kLB + c4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float e = ks[m] * exp2_hw(gt[m] - gs[m]);
                ak[m] += kt[m] * e;
                aqv[m] += qt[m] * e;
            }
        }
        dkk = (ak[0] + ak[1]) + (ak[2] + ak[3]);
        dqk = (aqv[0] + aqv[1]) + (aqv[2] + aqv[3]);
    }
    const float dqd = sum8((qx[0] * kx[0] + qx[1] * kx[1]) + (qx[2] * kx[2] + qx[3] * kx[3]));
    __syncthreads();  // the pass-1 tiles are overwritten next

    // ---- assemble Akk (fp32, rows times beta, over S1; strictly lower part only, as
    // the solve reads it) and Aqk (fp32 staging over KQG; zero above the diagonal by index below)
    float* AqL = KQG;  // [t][s], stride LQ (odd: its row-wise and column-wise reads are free of bank conflicts)
    if (pidx < kDiagPairs) {
        A[pt * kLD + ps] = bet[pt] * dkk;
        AqL[pt * LQ + ps] = dqk;
    }
    if ((threadIdx.x & 7) == 0) AqL[tr * (LQ + 1)] = dqd;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tau = wave + kI32Waves * i;
        if (tau < 12) {
            const int pr = tau % 6, kind = tau / 6;
            int I, J;
            gram_pair(pr, I, J);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + frag_row(r), s = 16 * J + frag_col();
                if (kind == 0) A[t * kLD + s] = bet[t] * gacc[i][r];
                else AqL[t * LQ + s] = gacc[i][r];
            }
        }
    }
    __syncthreads();
    // The Aqk rows of pass 3's row tile tt = wave >> 1 (k-blocks 0 .. tt >> 1, zero
    // above the diagonal), kept as register fragments through the solve and pass 2.
    const int tt = wave >> 1, hf = wave & 1;
    const int nq = (tt >> 1) + 1;
    AFrag<P> fQ[2];
    {
        const int r = 16 * tt + (lane & 15), s8 = 8 * (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            if (kb < nq) {
                float x[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int s = 32 * kb + s8 + m;
                    x[m] = s > r ? 0.f : AqL[r * LQ + s];
                }
                make_frag(fQ[kb], x);
            }
    }
    if (p.aqT) {
        // Aqk^T (row s, indices t; zero for t < s) for the backward, eight entries per thread
        static_assert(kChunk * kChunk / 8 == kI32Threads, "one group of eight per thread");
        const int sr = threadIdx.x >> 3, t0 = 8 * (threadIdx.x & 7);
        float x[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) x[m] = t0 + m < sr ? 0.f : AqL[(t0 + m) * LQ + sr];
        // (the block of rows s >= 32, t < 32 is zero and never read: not written)
        if (sr < 32 || t0 >= 32)
            store_frag8<P>(frag_rec((char*)(p.aqT + slot * kChunk * kChunk), sr, t0 >> 5, 2), sr, x, (t0 >> 3) & 3);
    }
    solve_unit_lower(A, Tm);  // (waves 0-3; ends with a barrier)
    if (p.tm) {
        // the 10 blocks on and below the diagonal, packed (tpk_index)
        f32x4* to = (f32x4*)(p.tm + slot * kTPacked);
        for (int e = threadIdx.x; e < kTPacked / 4; e += kI32Threads) {
            const int b = e >> 6, I = b < 1 ? 0 : (b < 3 ? 1 : (b < 6 ? 2 : 3)), J = b - I * (I + 1) / 2;
            const int t = 16 * I + ((e & 63) >> 2), s = 16 * J + 4 * (e & 3);
            const f32x4 x = *(const f32x4*)&Tm[t * kLD + s];
            if constexpr (P == Prec::BF3) {  // stored as its hi/lo split (tpk_load4_split)
                const float v[4] = {x[0], x[1], x[2], x[3]};
                u32x2v hw, lw;
                split4(v, hw, lw);
                *(tpk_words*)&to[e] = tpk_words{hw[0], hw[1], lw[0], lw[1]};
            } else {
                to[e] = x;
            }
        }
    }

    // ---- pass 2: w = (T Diag(beta)) (exp(G) k) and u = (T Diag(beta)) v, one round of
    // three [32 x 64] operand blocks in KQG.  beta is folded into T's columns, so that v
    // (a bf16 number for bf16 inputs) is an operand as it stands: hi part only, two
    // MFMAs per k-block for u.
    for (int e = threadIdx.x; e < kChunk * kChunk / 4; e += kI32Threads) {
        const int t = e >> 4, s4 = (e & 15) * 4;
        const f32x4 tb = *(const f32x4*)&Tm[t * kLD + s4] * *(const f32x4*)&bet[s4];
        Tt.put4(t, s4, (s4 >> 4) > (t >> 4) ? f32x4{0.f, 0.f, 0.f, 0.f} : tb);
    }
    static_assert(3 * kCB32 * LA <= 3 * kChunk * kLB, "three operand blocks must fit in KQG");
    {
        const T64 B0(KQG, kCB32), B1(KQG + kCB32 * LA, kCB32), B2(KQG + 2 * kCB32 * LA, kCB32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            B0.put(ch + i, tr, exp2_hw(G[i]) * kx[i]);
            B1.put_hi(ch + i, tr, in ? vx[0][i] : 0.f);
            B2.put_hi(ch + i, tr, in ? vx[1][i] : 0.f);
        }
    }
    __syncthreads();
    // 24 tiles (3 blocks x 4 row tiles x 2 column tiles), three per wave: column
    // tile hf, row tiles m, 3 - m and m ^ 1 (m = wave >> 1) of blocks 0, 1, 2, which
    // evens out the triangular contraction lengths (16 (tm + 1)) between waves
    f32x4 pacc[3];
    const int m3[3] = {tt, 3 - tt, tt ^ 1};
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        const int tm = m3[g];
        const T64 BTg(KQG + g * kCB32 * LA, kCB32);
        int k0 = 0, k1 = 16 * (tm + 1);
        widen<P>(k0, k1);
        pacc[g] = g == 0 ? mma_tile(Tt.sub(tm * 16), BTg.sub(hf * 16), k0, k1, f32x4{0.f, 0.f, 0.f, 0.f})
                         : mma_tile_bh(Tt.sub(tm * 16), BTg.sub(hf * 16), k0, k1, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();  // pass-2 operand tiles (KQG, S1) consumed

    // ---- pass 3: the chunk as an affine map of the state entering it.
    //   P   = Diag(exp G_L) - Kh^T w      (32 x 32)   h'     = P h + hh
    //   hh  = Kh^T u                      (32 x 64)
    //   qh  = scale (Qg - Aqk w)          (64 x 32)   o      = ol + qh h
    //   ol  = scale Aqk u                 (64 x 64)
    // and for the reverse pass D = P^T D' + qh^T dO.  w^T and u^T are staged in
    // LDS from pass 2's tiles and Kh^T from the pass-1 registers.  A D fragment
    // holds four consecutive rows of one column, so each fragment-form array is
    // written from the product of its transpose: P from P^T's tiles and P^T from
    // P's, qh from qh^T's and qh^T from qh's.  hh and ol are kept in fragment
    // order ([32-column block][16x16 tile][lane][4]) for the state pass to add to
    // its accumulators directly.
    const T64 WT(KQG, DK), UT(KQG + DK * LA, DV);
    static_assert(DK * LA + DV * LA <= 3 * kChunk * kLB, "w^T and u^T must fit in KQG");
    float* Qgs = S1;  // exp(G) q, fp32 [t][c], stride kLB
    const T64 KHT(S1 + kChunk * kLB, DK);  // Kh^T [c][t]
    static_assert(kChunk * kLB + DK * LA <= S1F, "Qg and Kh^T must fit in S1");
#pragma unroll
    for (int i = 0; i < 4; ++i) KHT.put(ch + i, tr, khs[i]);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        const int tm = m3[g];
        if (g == 0) WT.put4(hf * 16 + frag_col(), tm * 16 + frag_row(0), pacc[g]);
        else UT.put4((g - 1) * 32 + hf * 16 + frag_col(), tm * 16 + frag_row(0), pacc[g]);
    }
    {
        f32x4 qv;
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = exp2_hw(G[i]) * qx[i];
        *(f32x4*)&Qgs[tr * kLB + ch] = qv;
        if (tr == last) {
#pragma unroll
            for (int i = 0; i < 4; ++i) glS[ch + i] = exp2_hw(G[i]);
        }
    }
    const int lr = lane & 15, lg = lane >> 4;
    const float scale = p.scale;
    __syncthreads();
    // waves 0, 1: P and P^T; waves 2, 3: hh rows 16 (wave - 2) ..; every wave:
    // qh, qh^T (column tile hf) and ol (column tiles 2 hf, 2 hf + 1) of row tile tt
    AFrag<P> fb;
    if (wave < 2) {
        AFrag<P> fK[2][2];  // Kh^T: row tiles ta, k-blocks kb
#pragma unroll
        for (int ta = 0; ta < 2; ++ta)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) load_frag(fK[ta][kb], KHT.sub(16 * ta), 32 * kb);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ta = q >> 1, tb = q & 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (wave == 0) {
                    load_frag(fb, WT.sub(16 * tb), 32 * kb);
                    acc = mma_ff(fK[ta][kb], fb, acc);
                } else {
                    load_frag(fb, WT.sub(16 * ta), 32 * kb);
                    acc = mma_ff(fb, fK[tb][kb], acc);
                }
            }
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ra = 16 * ta + 4 * lg + i, cb = 16 * tb + lr;
                x[i] = (ra == cb ? glS[ra] : 0.f) - acc[i];
            }
            float* dst = wave == 0 ? p.pmT : p.pm;
            store_frag4<P>(frag_rec(dst + slot * DK * DK, 16 * tb + lr, 0, 1), 16 * tb + lr, x, 16 * ta + 4 * lg);
        }
    } else if (wave < 4) {
        const int ta = wave - 2;
        AFrag<P> fK[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) load_frag(fK[kb], KHT.sub(16 * ta), 32 * kb);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                load_frag(fb, UT.sub(16 * tj), 32 * kb);
                acc = mma_ff(fK[kb], fb, acc);
            }
            *(f32x4*)(p.hh + slot * DK * DV + (size_t)(((tj >> 1) * 4 + ta * 2 + (tj & 1)) * 64 + lane) * 4) = acc;
        }
    }
    {
        // qh tile (tt, hf) -> qh^T (row c, indices t), and qh^T tile (hf, tt) -> qh
        const int tc = hf;
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb < nq) {
                load_frag(fb, WT.sub(16 * tc), 32 * kb);
                a1 = mma_ff(fQ[kb], fb, a1);
                a2 = mma_ff(fb, fQ[kb], a2);
            }
        }
        f32x4 x1, x2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a = 4 * lg + i;
            x1[i] = scale * (Qgs[(16 * tt + a) * kLB + 16 * tc + lr] - a1[i]);
            x2[i] = scale * (Qgs[(16 * tt + lr) * kLB + 16 * tc + a] - a2[i]);
        }
        store_frag4<P>(frag_rec(p.qhT + slot * kChunk * DK, 16 * tc + lr, tt >> 1, 2), 16 * tc + lr, x1,
                       (16 * tt + 4 * lg) & 31);
        store_frag4<P>(frag_rec(p.qh + slot * kChunk * DK, 16 * tt + lr, 0, 1), 16 * tt + lr, x2, 16 * tc + 4 * lg);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        // ol tile (tt, tj)
        const int tj = 2 * hf + j;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb < nq) {
                load_frag(fb, UT.sub(16 * tj), 32 * kb);
                acc = mma_ff(fQ[kb], fb, acc);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= scale;
        *(f32x4*)(p.ol + slot * kChunk * DV + (size_t)(((tj >> 1) * 8 + tt * 2 + (tj & 1)) * 64 + lane) * 4) = acc;
    }
}

}  // namespace kda
