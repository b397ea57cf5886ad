// kda_intra.cuh -- the intra-chunk kernel: everything of a chunk that does not
// depend on the state entering it.
//
// Per (chunk, head), 256 threads, channels processed in blocks of 32:
//   pass 1 (per channel block): stage k, q (L2-normalised if flagged; the row
//     norms are taken first over all channels), the per-token log-decay g
//     (from f, A_log, dt_bias if flagged) and its in-chunk cumulative sum G
//     (a scan over the 64 tokens in registers and cross-lane shuffles); write
//     exp(G) q and (k exp(G_L - G))^T and exp(G_L); accumulate the Gram
//     matrices Akk and Aqk.
//   Gram matrices by 16x16 blocks: for a row block I and an earlier column
//     block J, the decay is factored through r = 16 I (the first row of I):
//       exp(G_t - G_s) = exp(G_t - G_r) * exp(G_r - G_s),   s < r <= t,
//     both factors at most 1, so the block is an MFMA product of two scaled
//     operands.  Diagonal blocks take the exact exp of each (t, s) difference.
//   solve: T = (I + Akk)^{-1} (kda_chunk.cuh, fp32).
//   pass 2: w = T beta exp(G) k  (per channel block) and u = T beta v (per
//     32-column block of v), as MFMA products; beta is folded into T's columns,
//     so that v (a bf16 number for bf16 inputs) is an operand as it stands.
// Outputs (fp32 workspace, slot = chunk * H + head): w [64][DK], u [64][DV],
// qg = exp(G) q^ [64][DK], khT = (k^ exp(G_L - G))^T [DK][64], gl = exp(G_L)
// [DK], aqk [64][64] (zero above the diagonal), and T [64][64] if requested.
// dk = 32 (dv = 64) keeps the chunk's affine form instead and has a kernel of
// its own with eight waves (kda_intra32.cuh), which shares the helpers below.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kCB32 = 32;        // channels per block
constexpr int kLB = kCB32 + 4;   // row stride of [token][channel-block] tiles

// The p-th pair (t, s), s < t, of the four 16x16 diagonal blocks (120 each),
// enumerated in integer arithmetic: within a block, rows a = g + 1 and 15 - g
// (g = 0..6) have 16 partners together, so group g = q >> 4 takes row a's
// partners and then row 15 - g's; group 7 is row 8's eight partners.
__device__ __forceinline__ void diag_pair(int p, int& t, int& s) {
    const int I = p / 120, q = p - 120 * I;
    const int g = q >> 4, u = q & 15, a = g + 1;
    const bool first = u < a;  // (always in group 7: a = 8, u < 8)
    t = 16 * I + (first ? a : 15 - g);
    s = 16 * I + (first ? u : u - a);
}
constexpr int kDiagPairs = 4 * 120;

// Gram tile list: pairs (I, J), J < I, of 16x16 blocks below the diagonal.
__device__ __forceinline__ void gram_pair(int p, int& I, int& J) {
    // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    I = p < 1 ? 1 : (p < 3 ? 2 : 3);
    J = p - (I * (I - 1)) / 2;
}
// row offset of the column-factor rows for row block I inside Kc
__device__ __forceinline__ int kc_off(int I) { return (I - 1) * I * 8; }  // 0, 16, 48

template <int DK, int DV, typename TIn, Prec P>
__global__ void __launch_bounds__(kThreads, 2) intra_kernel(Prm p) {  // two workgroups per CU
    static_assert(DK >= 64, "dk = 32: intra32_kernel");
    constexpr int NB = DK / kCB32, NVB = DV / 32;
    // LDS (about 77 KB, two workgroups per CU):
    //   KQG  Kb | Qb | Gb   one channel block, fp32 [t][c]; after pass 1: Aqk staging, BT tiles
    //   S1   Kr | Qr | Kc   MFMA tiles of the off-diagonal Gram blocks; then Akk (fp32); then T (tile)
    //   Tm   T, fp32 (the solve)
    constexpr int LB8 = kCB32 + 8, LA = kChunk + 8, LQ = kChunk + 1;
    constexpr int S1F = (48 + 48 + 96) * LB8;
    __shared__ __attribute__((aligned(16))) float KQG[3 * kChunk * kLB];
    __shared__ __attribute__((aligned(16))) float S1[S1F];
    __shared__ __attribute__((aligned(16))) float Tm[kChunk * kLD];
    __shared__ __attribute__((aligned(16))) float bet[kChunk];
    __shared__ float seg[8 * 32];        // column-scan segment totals
    static_assert(kChunk * kLD <= S1F && kChunk * LA <= S1F, "Akk and the T tile must fit in S1");
    static_assert(kCB32 * LA <= 3 * kChunk * kLB, "a BT tile must fit in KQG");
    static_assert(kChunk * LQ <= 3 * kChunk * kLB, "the Aqk staging must fit in KQG");

    float* Kb = KQG;
    float* Qb = KQG + kChunk * kLB;
    float* Gb = KQG + 2 * kChunk * kLB;
    using T32 = STile<P, 32>;  // operand tiles of 32 and 64 values per row
    using T64 = STile<P, 64>;
    static_assert(STile<Prec::F32, 32>::ld == LB8 && STile<Prec::F32, 64>::ld == LA, "tile footprints");
    const T32 Kr(S1, 48);
    const T32 Qr(S1 + 48 * LB8, 48);
    const T32 Kc(S1 + 96 * LB8, 96);
    float* A = S1;                  // fp32 Akk, after pass 1
    const T64 Tt(S1, kChunk);       // T as an MFMA operand, after the solve

    // w, exp(G) q, (k exp(G_L - G))^T and Aqk go to the workspace in fragment form
    // (kda_mma.cuh) for the sequential kernels, which load MFMA fragments from it
    // directly.
    constexpr Prec WP = P;
    const int c = blockIdx.x, h = blockIdx.y;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;
    const int wave = wave_id();
    const int tr = threadIdx.x >> 2, part = threadIdx.x & 3;  // staging row / channel group
    const bool l2 = p.flags & 1u;
    const TIn* qin = (const TIn*)p.q;
    const TIn* kin = (const TIn*)p.k;
    const TIn* vin = (const TIn*)p.v;
    const int last = cr.len - 1;
    const bool in = tr < cr.len;

    // ---- every global load of the chunk, issued up front (the gate parameters
    // too, so that no later load waits behind the bulk of them)
    const bool gate = p.flags & 2u;
    float kx[NB][8], qx[NB][8], G[NB][8], vx[NVB][8], dtb[NB][8];
    float braw = 0.f, alog = 0.f;
    (void)Gb;
    if (gate) {
        alog = p.A_log[h];
#pragma unroll
        for (int b = 0; b < NB; ++b) load8<float>(p.dt_bias + h * DK + b * kCB32 + 8 * part, dtb[b]);
    }
    // Rows past the chunk end load row 0 (always valid) and are zeroed after the
    // loads: unconditional loads keep every wait after the whole batch.
    const int trc = in ? tr : 0;
    if (threadIdx.x < kChunk) braw = p.beta[(size_t)(cr.t0 + (threadIdx.x < cr.len ? threadIdx.x : 0)) * p.H + h];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const size_t base = tok_index(cr.t0 + trc, h, p.H, DK) + b * kCB32 + 8 * part;
        load8<TIn>(kin + base, kx[b]);
        load8<TIn>(qin + base, qx[b]);
        load8<float>(p.g + base, G[b]);
    }
    if (threadIdx.x < kChunk && threadIdx.x >= cr.len) braw = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            kx[b][i] = in ? kx[b][i] : 0.f;
            qx[b][i] = in ? qx[b][i] : 0.f;
            G[b][i] = in ? G[b][i] : 0.f;
        }
    }
    // ---- preparation in registers: beta, L2 norms, gate, in-chunk cumulative decay
    if (threadIdx.x < kChunk) bet[threadIdx.x] = (p.flags & 4u) ? (threadIdx.x < cr.len ? sigmoid_f(braw) : 0.f) : braw;
    if (l2) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) { sk += kx[b][i] * kx[b][i]; sq += qx[b][i] * qx[b][i]; }
        sk += __shfl_xor(sk, 1, 64); sk += __shfl_xor(sk, 2, 64);
        sq += __shfl_xor(sq, 1, 64); sq += __shfl_xor(sq, 2, 64);
        const float rk = rsqrt_hw(sk + kL2Eps), rq = rsqrt_hw(sq + kL2Eps);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) { kx[b][i] *= rk; qx[b][i] *= rq; }
    }
    if (gate && in) {
        const float eA = exp_hw(alog);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) G[b][i] = -eA * softplus_f(G[b][i] + dtb[b][i]);
    }

    // v, first needed in pass 2: issued once the preparation's inputs have arrived
    // (rows past the chunk end are zeroed where v is used)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) load8<TIn>(vin + tok_index(cr.t0 + trc, h, p.H, DV) + 32 * vb + 8 * part, vx[vb]);

    // Gram accumulators: 12 off-diagonal tiles (6 of Akk, 6 of Aqk), 3 per wave,
    // and this thread's 4 diagonal-block entries of each.
    f32x4 gacc[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) gacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dkk[2] = {0.f, 0.f}, dqk[2] = {0.f, 0.f}, dqd = 0.f;

    char* qg = (char*)(p.qg + slot * kChunk * DK);    // rows t, DK/32 k-blocks
    char* khT = (char*)(p.khT + slot * DK * kChunk);  // rows c, 2 k-blocks
    float* KhS = Tm;                                   // (k exp(G_L - G))^T staging, [c][t], pass 1 only
    float* QgS = Tm + kCB32 * kLD;                     // (exp(G) q)^T staging, [c][t], pass 1 only (dk >= 64)
    const bool rev_ops = p.qgT != nullptr;  // transposed operands for the reverse scan
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int cb = b * kCB32;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            Kb[tr * kLB + 8 * part + i] = kx[b][i];
            Qb[tr * kLB + 8 * part + i] = qx[b][i];
            Gb[tr * kLB + 8 * part + i] = G[b][i] * kLog2e;  // base-2 log-decay; scanned in place below
        }
        __syncthreads();
        {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = Gb[(8 * (threadIdx.x >> 5) + i) * kLB + (threadIdx.x & 31)];
            col_scan_regs<false>(x, Gb, kLB, seg);  // in-chunk cumulative sum G; ends with a barrier
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) G[b][i] = Gb[tr * kLB + 8 * part + i];
        if (p.gcs) {  // the backward's dk-side kernel reads G instead of forming it again
            f32x4* gd = (f32x4*)(p.gcs + (slot * kChunk + tr) * DK + cb + 8 * part);
            gd[0] = f32x4{G[b][0], G[b][1], G[b][2], G[b][3]};
            gd[1] = f32x4{G[b][4], G[b][5], G[b][6], G[b][7]};
        }
        // G at the reference rows 16 I and at the last row come straight from the scanned tile
        // scaled operands for the off-diagonal Gram blocks, exp(G) q, k exp(G_L - G)
        {
            const int I = tr >> 4;
            float qgv[8], khv[8], kr[8], qr[8], kc[3][8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int cc = 8 * part + i;
                const float gt = G[b][i];
                qgv[i] = exp2_hw(gt) * qx[b][i];
                khv[i] = kx[b][i] * exp2_hw(Gb[last * kLB + cc] - gt);
                KhS[cc * kLD + tr] = khv[i];
                if (rev_ops) QgS[cc * kLD + tr] = qgv[i];
                const float e = exp2_hw(gt - Gb[16 * (I >= 1 ? I : 1) * kLB + cc]);
                kr[i] = kx[b][i] * e;
                qr[i] = qx[b][i] * e;
#pragma unroll
                for (int J = 1; J <= 3; ++J) kc[J - 1][i] = kx[b][i] * exp2_hw(Gb[16 * J * kLB + cc] - gt);
            }
            if (I >= 1) {
                Kr.put8(tr - 16, 8 * part, kr);
                Qr.put8(tr - 16, 8 * part, qr);
            }
#pragma unroll
            for (int J = 1; J <= 3; ++J)
                if (tr < 16 * J) Kc.put8(kc_off(J) + tr, 8 * part, kc[J - 1]);
            store_frag8<WP>(frag_rec(qg, tr, b, DK / 32), tr, qgv, part);
            if (rev_ops)  // Kh rows t, channels of this block
                store_frag8<WP>(frag_rec(p.khb + slot * kChunk * DK, tr, b, DK / 32), tr, khv, part);
        }
        if (tr == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) p.gl[slot * DK + cb + 8 * part + i] = exp2_hw(Gb[last * kLB + 8 * part + i]);
        }
        __syncthreads();
        {
            // (k exp(G_L - G))^T of this channel block to the workspace: row c = cb + tid / 8
            const int cr8 = threadIdx.x >> 3, w8 = threadIdx.x & 7;
            float x[8];
            const f32x4 a0 = *(const f32x4*)&KhS[cr8 * kLD + 8 * w8], a1 = *(const f32x4*)&KhS[cr8 * kLD + 8 * w8 + 4];
            x[0] = a0[0]; x[1] = a0[1]; x[2] = a0[2]; x[3] = a0[3]; x[4] = a1[0]; x[5] = a1[1]; x[6] = a1[2]; x[7] = a1[3];
            store_frag8<WP>(frag_rec(khT, cb + cr8, w8 >> 2, 2), cb + cr8, x, w8 & 3);
            if (rev_ops) {  // (exp(G) q)^T rows c, tokens as indices
                const f32x4 b0 = *(const f32x4*)&QgS[cr8 * kLD + 8 * w8], b1 = *(const f32x4*)&QgS[cr8 * kLD + 8 * w8 + 4];
                x[0] = b0[0]; x[1] = b0[1]; x[2] = b0[2]; x[3] = b0[3]; x[4] = b1[0]; x[5] = b1[1]; x[6] = b1[2]; x[7] = b1[3];
                store_frag8<WP>(frag_rec(p.qgT + slot * DK * kChunk, cb + cr8, w8 >> 2, 2), cb + cr8, x, w8 & 3);
            }
        }
        // off-diagonal Gram tiles
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int tau = wave + 4 * i;         // 0..11
            const int pr = tau % 6, kind = tau / 6;  // kind 0: Akk, 1: Aqk
            int I, J;
            gram_pair(pr, I, J);
            const T32 Aop = (kind == 0 ? Kr : Qr).sub((I - 1) * 16);
            gacc[i] = mma_tile(Aop, Kc.sub(kc_off(I) + 16 * J), 0, kCB32, gacc[i]);
        }
        // diagonal blocks, exact pairwise decays: the 4 x 120 pairs s < t of the 16x16
        // diagonal blocks, two per thread (the last 32 threads have one); then the
        // diagonal itself, Aqk[t][t] = q_t . k_t (no decay), four threads per token
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pidx = threadIdx.x + kThreads * i;
            if (pidx < kDiagPairs) {
                int t, s;
                diag_pair(pidx, t, s);
                f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aqv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c4 = 0; c4 < kCB32; c4 += 4) {
                    const f32x4 gt = *(const f32x4*)&Gb[t * kLB + c4];
                    const f32x4 gs = *(const f32x4*)&Gb[s * kLB + c4];
                    const f32x4 ks = *(const f32x4*)&Kb[s * kLB + c4];
                    const f32x4 kt = *(const f32x4*)&Kb[t * kLB + c4];
                    const f32x4 qt = *(const f32x4*)&Qb[t * kLB + c4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float e = ks[m] * exp2_hw(gt[m] - gs[m]);
                        ak[m] += kt[m] * e;
                        aqv[m] += qt[m] * e;
                    }
                }
                dkk[i] += (ak[0] + ak[1]) + (ak[2] + ak[3]);
                dqk[i] += (aqv[0] + aqv[1]) + (aqv[2] + aqv[3]);
            }
        }
        {
            static_assert(kThreads == 4 * kChunk && kCB32 == 32, "four threads of 8 channels per token");
            const int t = threadIdx.x >> 2, c8 = 8 * (threadIdx.x & 3);
            const f32x4 q0 = *(const f32x4*)&Qb[t * kLB + c8], q1 = *(const f32x4*)&Qb[t * kLB + c8 + 4];
            const f32x4 k0 = *(const f32x4*)&Kb[t * kLB + c8], k1 = *(const f32x4*)&Kb[t * kLB + c8 + 4];
            const float a = ((q0[0] * k0[0] + q0[1] * k0[1]) + (q0[2] * k0[2] + q0[3] * k0[3])) +
                            ((q1[0] * k1[0] + q1[1] * k1[1]) + (q1[2] * k1[2] + q1[3] * k1[3]));
            dqd += sum4(a);
        }
        __syncthreads();  // channel-block tiles are rewritten next
    }

    // ---- assemble Akk (fp32, rows times beta, over S1) and Aqk (fp32 staging over KQG).
    // Only the parts that are read are written: the solve reads the strictly lower part of
    // Akk; the Aqk copy below writes zeros above the diagonal by index.
    float* AqL = KQG;  // [t][s], stride LQ (odd: its row-wise and column-wise reads are free of bank conflicts)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pidx = threadIdx.x + kThreads * i;
        if (pidx < kDiagPairs) {
            int t, s;
            diag_pair(pidx, t, s);
            A[t * kLD + s] = bet[t] * dkk[i];
            AqL[t * LQ + s] = dqk[i];
        }
    }
    if ((threadIdx.x & 3) == 0) AqL[(threadIdx.x >> 2) * (LQ + 1)] = dqd;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int tau = wave + 4 * i;
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
    __syncthreads();
    {
        // Aqk to the workspace in fragment form, zero above the diagonal: 8 entries per thread and pass
        char* aq = (char*)(p.aqk + slot * kChunk * kChunk);
#pragma unroll
        for (int i = 0; i < kChunk * kChunk / 8 / kThreads; ++i) {
            const int q8 = threadIdx.x + kThreads * i;
            const int t = q8 >> 3, s0 = 8 * (q8 & 7);
            float x[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) x[m] = s0 + m > t ? 0.f : AqL[t * LQ + s0 + m];
            // (the block of rows t < 32, s >= 32 is zero and never read: not written)
            if (t >= 32 || s0 < 32) store_frag8<WP>(frag_rec(aq, t, s0 >> 5, 2), t, x, (s0 >> 3) & 3);
        }
    }
    if (p.aqT) {
        // Aqk^T (row s, indices t; zero for t < s) for the backward
        char* aqt = (char*)(p.aqT + slot * kChunk * kChunk);
#pragma unroll
        for (int i = 0; i < kChunk * kChunk / 8 / kThreads; ++i) {
            const int q8 = threadIdx.x + kThreads * i;
            const int sr = q8 >> 3, t0 = 8 * (q8 & 7);
            float x[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) x[m] = t0 + m < sr ? 0.f : AqL[(t0 + m) * LQ + sr];
            // (the block of rows s >= 32, t < 32 is zero and never read: not written)
            if (sr < 32 || t0 >= 32) store_frag8<WP>(frag_rec(aqt, sr, t0 >> 5, 2), sr, x, (t0 >> 3) & 3);
        }
    }
    solve_unit_lower(A, Tm);  // ends with a barrier
    if (p.tm) {
        // the 10 blocks on and below the diagonal, packed (tpk_index)
        f32x4* to = (f32x4*)(p.tm + slot * kTPacked);
        for (int e = threadIdx.x; e < kTPacked / 4; e += kThreads) {
            const int b = e >> 6, I = b < 1 ? 0 : (b < 3 ? 1 : (b < 6 ? 2 : 3)), J = b - I * (I + 1) / 2;
            const int t = 16 * I + ((e & 63) >> 2), s = 16 * J + 4 * (e & 3);
            to[e] = *(const f32x4*)&Tm[t * kLD + s];
        }
    }

    // ---- pass 2: w = (T Diag(beta)) (exp(G) k) per channel block, u = (T Diag(beta)) v per
    // column block (v: hi parts only, two MFMAs per k-block), as many blocks per barrier as
    // fit in KQG
    static_assert(P != Prec::BF3 || sizeof(TIn) == 2, "the bf16 path has bf16 inputs (v is a bf16 number)");
    for (int e = threadIdx.x; e < kChunk * kChunk / 4; e += kThreads) {
        const int t = e >> 4, s4 = (e & 15) * 4;
        const f32x4 tb = *(const f32x4*)&Tm[t * kLD + s4] * *(const f32x4*)&bet[s4];
        Tt.put4(t, s4, (s4 >> 4) > (t >> 4) ? f32x4{0.f, 0.f, 0.f, 0.f} : tb);
    }
    constexpr int NBLK = NB + NVB;
    constexpr int GRP = (3 * kChunk * kLB) / (kCB32 * LA);  // blocks per round
    static_assert(GRP >= 1, "one operand block must fit in KQG");
    float* wo = p.w + slot * kChunk * DK;
    float* uo = p.u + slot * kChunk * DV;
#pragma unroll
    for (int b0 = 0; b0 < NBLK; b0 += GRP) {
        if (b0 > 0) __syncthreads();  // the previous round's operand tiles are consumed
#pragma unroll
        for (int g = 0; g < GRP; ++g) {
            const int b = b0 + g;
            if (b < NBLK) {
                const T64 BTg(KQG + g * kCB32 * LA, kCB32);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (b < NB) BTg.put(8 * part + i, tr, exp2_hw(G[b < NB ? b : 0][i]) * kx[b < NB ? b : 0][i]);
                    else BTg.put_hi(8 * part + i, tr, in ? vx[b < NB ? 0 : b - NB][i] : 0.f);
                }
            }
        }
        __syncthreads();
        constexpr int TPB = 8;  // [64 x 32] tiles per block
        const int nb = NBLK - b0 < GRP ? NBLK - b0 : GRP;
#pragma unroll
        for (int kt = 0; kt < (TPB * GRP + kWaves - 1) / kWaves; ++kt) {
            const int tile = wave + kWaves * kt;
            if (tile >= TPB * nb) break;
            const int g = tile / TPB, tl = tile % TPB, tm = tl >> 1, tn = tl & 1;
            const int b = b0 + g;
            const T64 BTg(KQG + g * kCB32 * LA, kCB32);
            int k0 = 0, k1 = 16 * (tm + 1);
            widen<P>(k0, k1);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = b < NB ? mma_tile(Tt.sub(tm * 16), BTg.sub(tn * 16), k0, k1, acc)
                         : mma_tile_bh(Tt.sub(tm * 16), BTg.sub(tn * 16), k0, k1, acc);
            if (rev_ops && b < NB) {  // w^T rows c, tokens as indices: four consecutive t per lane
                const int t0 = tm * 16 + frag_row(0), cw = b * kCB32 + tn * 16 + frag_col();
                store_frag4<WP>(frag_rec(p.wT + slot * DK * kChunk, cw, t0 >> 5, 2), cw, acc, t0 & 31);
            }
            if (DK <= 64 && b < NB) {  // w: staged in Tm [t][c] (stride kLD), written out below
#pragma unroll
                for (int r = 0; r < 4; ++r) Tm[(tm * 16 + frag_row(r)) * kLD + b * kCB32 + tn * 16 + frag_col()] = acc[r];
            } else if (b < NB) {  // w (dk > 64): k-block b of rows 16 tm .., straight from the fragment
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    store_frag1<WP>(frag_rec(wo, tm * 16 + frag_row(r), b, NB), tm * 16 + frag_row(r), acc[r],
                                    tn * 16 + frag_col());
            } else {
                float* out = uo + (b - NB) * 32;
#pragma unroll
                for (int r = 0; r < 4; ++r) out[(size_t)(tm * 16 + frag_row(r)) * DV + tn * 16 + frag_col()] = acc[r];
            }
        }
    }
    if constexpr (DK == 64) {
        __syncthreads();
        char* wk = (char*)wo;  // rows t, DK/32 k-blocks
#pragma unroll
        for (int i = 0; i < (kChunk * DK / 8 + kThreads - 1) / kThreads; ++i) {
            const int q8 = threadIdx.x + kThreads * i;
            if (q8 < kChunk * DK / 8) {
                const int t = q8 / (DK / 8), k0 = 8 * (q8 % (DK / 8));
                float x[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = Tm[t * kLD + k0 + m];
                store_frag8<WP>(frag_rec(wk, t, k0 >> 5, DK / 32), t, x, (k0 >> 3) & 3);
            }
        }
    }
}

}  // namespace kda
