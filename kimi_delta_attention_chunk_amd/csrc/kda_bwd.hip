// kda_bwd.hip -- chunked backward.
//
// Reverse-mode of the chunk form in kda_chunk.cuh (derived by hand from the
// recurrence; the pages only name the FLA backward kernels and their
// "diagonal phases": openkimi README, the paragraph on the guarded midpoint
// change, and the Primus guide's autotune paragraph on
// chunk_kda_bwd_kernel_intra).  Launch sequence:
//   1. forward recompute: intra (w, u, Aqk, T) and state pass (h_n, v_new);
//   2. bwd_dh   one workgroup per (sequence, head, 32 or 16 state columns),
//               chunks in reverse (kda_dhscan.cuh): D = dL/dS at each chunk end, and
//               dv_new = scale Aqk^T dO + Kh D,
//               D     <- scale Qg^T dO + Diag(exp G_L) D - w^T dv_new;
//   3. bwd_dv   one workgroup per (chunk, head): the products that contract
//               over dv (register accumulators over 32-column blocks):
//               dQg = scale dO h^T, dAqk = scale dO vn^T, dKh = vn D^T,
//               dw = -dvn h^T, dT_v = dvn (beta V)^T, dGamma_L = rowsum(h . D),
//               and through u = T beta V: dV = beta . (T^T dvn), dbeta_v;
//   4. bwd_dk   one workgroup per (chunk, head): dT += dw (beta Kg)^T,
//               dKg = beta . (T^T dw), dA = -T^T dT T^T (strictly lower), the
//               decayed pair terms of Akk and Aqk (exact exp of each
//               non-positive difference), the explicit factors exp(G) Q,
//               exp(G) K, K exp(G_L - G), exp(G_L), the reverse in-chunk
//               cumulative sum dg, and the preparation chain;
//   5. (gate in kernel) a fixed-order reduction of dA_log and dt_bias.
// Every reduction has a fixed order: no floating-point atomics anywhere.
#include <type_traits>

#include "kda_chunk.cuh"
#include "kda_bwdchunk.cuh"
#include "kda_dhscan.cuh"
#include "kda_pscan.cuh"
#include "kda_internal.h"

namespace kda {

// ============================================================== dv-side contractions
// The per-chunk kernels of dk = 64 and 128 run 8 waves (two per SIMD): their
// tiles take most of the LDS, so one workgroup fits per CU.
constexpr int kGThreads = 512, kGWaves = kGThreads / 64;

// acc += A B^T over [k0, k1) on swizzled tiles (origins at their view rows).
// AH / BH: that operand holds bf16 numbers, stored with put_hi (no lo part).
template <bool AH, bool BH, Prec P, int CA, int CB>
__device__ __forceinline__ f32x4 mma_st(const STile<P, CA>& A, const STile<P, CB>& B, int k0, int k1, f32x4 acc) {
    static_assert(!(AH && BH), "at most one operand without a lo part");
    if constexpr (P == Prec::F32) {
        return mma_tile(A, B, k0, k1, acc);
    } else {
        for (int kb = k0; kb < k1; kb += 32) {
            AFrag<P> a, b;
            if constexpr (AH) load_frag_hi(a, A, kb); else load_frag(a, A, kb);
            if constexpr (BH) load_frag_hi(b, B, kb); else load_frag(b, B, kb);
            if constexpr (AH) acc = mma_ff_ah(a, b, acc);
            else if constexpr (BH) acc = mma_ff_bh(a, b, acc);
            else acc = mma_ff(a, b, acc);
        }
        return acc;
    }
}
// The same product into every tile of a TileSet that this wave owns.
template <bool AH, bool BH, class TS, Prec P, int CA, int CB>
__device__ __forceinline__ void tiles_mma(TS& ts, const STile<P, CA>& A, const STile<P, CB>& B, int k0, int k1) {
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < TS::PER; ++i) {
        const int tile = wave + i * TS::NWAVES;
        if (tile < TS::TILES) {
            const int tm = tile / TS::TN, tn = tile % TS::TN;
            ts.acc[i] = mma_st<AH, BH>(A.sub(16 * tm), B.sub(16 * tn), k0, k1, ts.acc[i]);
        }
    }
}

// Per 32-column block jb of v: the products over the block's columns, accumulated
// in registers across the blocks (P: bf16x3 MFMA for bf16 inputs, fp32 MFMA for
// fp32 inputs; dO and v are input values, so for bf16 inputs their lo parts are
// zero and those products take two MFMAs):
//   dQg += dO h^T, dKh += vn D^T, dw += dvn h^T, dAqk += dO vn^T, dT_v += dvn V^T
// and X_u = T^T dvn (dV = beta X_u, dbeta_v = rowsum(X_u V)); dGamma_L = rowsum(h D).
template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kGThreads) bwd_dv_kernel(Prm p) {
    constexpr int VB = 32, NG = DV / 16;
    constexpr Prec P = std::is_same<TIn, uint16_t>::value ? Prec::BF3 : Prec::F32;
    using T32 = STile<P, 32>;
    using T64 = STile<P, 64>;
    constexpr int F32R = P == Prec::F32 ? 40 : 32, F64R = P == Prec::F32 ? 72 : 64;  // floats per tile row
    __shared__ __attribute__((aligned(16))) float sT[kChunk * F64R];     // T^T [t][s]
    __shared__ __attribute__((aligned(16))) float sDVT[VB * F64R];       // dvn^T [j][s]
    __shared__ __attribute__((aligned(16))) float sH[DK * F32R], sD[DK * F32R];
    __shared__ __attribute__((aligned(16))) float sDO[kChunk * F32R], sV[kChunk * F32R];
    __shared__ __attribute__((aligned(16))) float sVN[kChunk * F32R], sDVN[kChunk * F32R];
    __shared__ float bet[kChunk];
    __shared__ float dbv_part[kChunk * NG];
    const T64 TT(sT, kChunk), DVT(sDVT, VB);
    const T32 Hs(sH, DK), Ds(sD, DK), DOs(sDO, kChunk), Vs(sV, kChunk), VNs(sVN, kChunk), DVNs(sDVN, kChunk);

    const int c = blockIdx.x, h = blockIdx.y;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;
    const TIn* dO = (const TIn*)p.d_o;
    const TIn* vin = (const TIn*)p.v;
    TOut* dvout = (TOut*)p.dv;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;

    {
        // T^T: row t of the tile holds T[s][t] over s (T is unit lower triangular)
        const float* tmi = p.tm + slot * kTPacked;
#pragma unroll
        for (int i = 0; i < kChunk * kChunk / 4 / kGThreads; ++i) {
            const int e4 = tid + i * kGThreads;
            const int s_ = e4 / (kChunk / 4), t4 = 4 * (e4 % (kChunk / 4));
            const f32x4 x = tpk_load4(tmi, s_, t4);
#pragma unroll
            for (int r = 0; r < 4; ++r) TT.put(t4 + r, s_, x[r]);
        }
    }
    if (tid < kChunk) {
        const int t = tid;
        float b = 0.f;
        if (t < cr.len) {
            b = p.beta[(size_t)(cr.t0 + t) * p.H + h];
            if (p.flags & 4u) b = sigmoid_f(b);
        }
        bet[t] = b;
    }

    TileSet<kChunk, DK, kGWaves> aQ, aKh, aW;
    TileSet<kChunk, kChunk, kGWaves> aAq, aT;
    aQ.zero(); aKh.zero(); aW.zero(); aAq.zero(); aT.zero();

    const float* hs = p.hs + slot * DK * DV;
    const float* dhs = p.dhs + slot * DK * DV;
    const float* vn = p.vn + slot * kChunk * DV;
    const float* dvn = p.dvn + slot * kChunk * DV;
    // thread's float4 of the h / D block (fixed rows over the blocks) and its row-sum partials
    constexpr int HQ = DK * VB / 4 / kGThreads;
    static_assert(HQ >= 1 && kChunk * VB / 4 == kGThreads, "one float4 of each token block per thread");
    float hd[HQ];
#pragma unroll
    for (int i = 0; i < HQ; ++i) hd[i] = 0.f;
    const int tt = tid / (VB / 4), j4 = 4 * (tid % (VB / 4));  // token block: (token, 4 columns)
    const bool tin = tt < cr.len;
    const size_t tok = tok_index(cr.t0 + (tin ? tt : 0), h, p.H, DV);
    // One block's global values for this thread, as loaded: the next block's loads
    // are issued once this block is staged, so that they arrive during its products
    // (converted or masked right after the load, a value would be waited for there).
    using Raw4 = typename std::conditional<std::is_same<TIn, uint16_t>::value, u32x2v, f32x4>::type;
    struct Blk {
        f32x4 xh[HQ], xd[HQ], xn, xdn;
        Raw4 xo, xv;
    };
    auto load_blk = [&](int jb, Blk& B) {
#pragma unroll
        for (int i = 0; i < HQ; ++i) {
            const int e4 = tid + i * kGThreads;
            const int cc = e4 / (VB / 4), q4 = 4 * (e4 % (VB / 4));
            B.xh[i] = *(const f32x4*)(hs + cc * DV + jb + q4);
            B.xd[i] = *(const f32x4*)(dhs + cc * DV + jb + q4);
        }
        B.xo = *(const Raw4*)(dO + tok + jb + j4);
        B.xv = *(const Raw4*)(vin + tok + jb + j4);
        B.xn = *(const f32x4*)(vn + tt * DV + jb + j4);
        B.xdn = *(const f32x4*)(dvn + tt * DV + jb + j4);
    };
    auto raw_at = [](const Raw4& x, int r) -> float {
        if constexpr (std::is_same<TIn, uint16_t>::value) {
            const uint32_t w = x[r >> 1];
            return __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return x[r];
        }
    };
    Blk B;
    load_blk(0, B);
    for (int jb = 0; jb < DV; jb += VB) {
        __syncthreads();  // the previous block's readers are done
#pragma unroll
        for (int i = 0; i < HQ; ++i) {
            const int e4 = tid + i * kGThreads;
            const int cc = e4 / (VB / 4), q4 = 4 * (e4 % (VB / 4));
            const f32x4 xh = B.xh[i], xd = B.xd[i];
            Hs.put4(cc, q4, xh);
            Ds.put4(cc, q4, xd);
            hd[i] += xh[0] * xd[0] + xh[1] * xd[1] + xh[2] * xd[2] + xh[3] * xd[3];
        }
        {
            const f32x4 xn = B.xn, xdn = B.xdn;
            f32x4 o4, v4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o4[r] = tin ? raw_at(B.xo, r) : 0.f;
                v4[r] = tin ? raw_at(B.xv, r) : 0.f;
                DVT.put(j4 + r, tt, xdn[r]);
            }
            DOs.put4_hi(tt, j4, o4);
            Vs.put4_hi(tt, j4, v4);
            VNs.put4(tt, j4, xn);
            DVNs.put4(tt, j4, xdn);
        }
        // the next block (past the last one: the last again, unused), with no branch around the loads
        load_blk(jb + VB < DV ? jb + VB : jb, B);
        __syncthreads();
        tiles_mma<true, false>(aQ, DOs, Hs, 0, VB);
        tiles_mma<false, false>(aKh, VNs, Ds, 0, VB);
        tiles_mma<false, false>(aW, DVNs, Hs, 0, VB);
        tiles_mma<true, false>(aAq, DOs, VNs, 0, VB);
        tiles_mma<false, true>(aT, DVNs, Vs, 0, VB);
        // X_u = T^T dvn  ->  dV = beta . X_u,  dbeta_v = rowsum(X_u . V)
        {
            constexpr int TN = VB / 16, TILES = (kChunk / 16) * TN;
            for (int tile = wave; tile < TILES; tile += kGWaves) {
                const int tm = tile / TN, tn = tile % TN;
                int k0 = 16 * tm, k1 = kChunk;
                widen<P>(k0, k1);
                const f32x4 acc = mma_st<false, false>(TT.sub(16 * tm), DVT.sub(16 * tn), k0, k1,
                                                       f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tm * 16 + 4 * (lane >> 4) + i, j = tn * 16 + (lane & 15);
                    if (t < cr.len)
                        Elem<TOut>::store(dvout, tok_index(cr.t0 + t, h, p.H, DV) + jb + j, bet[t] * acc[i]);
                    const float part = row16_sum(acc[i] * Vs.get_hi(t, j));
                    if ((lane & 15) == 0) dbv_part[t * NG + (jb >> 4) + tn] = part;
                }
            }
        }
    }
    const float scale = p.scale;
    float* o_q = p.dqt + slot * kChunk * DK;
    float* o_kh = p.dkh + slot * kChunk * DK;
    float* o_w = p.dwv + slot * kChunk * DK;
    float* o_aq = p.daq + slot * kChunk * kChunk;
    float* o_t = p.dtv + slot * kChunk * kChunk;
    aQ.store([&](int t, int cc, float x) { o_q[t * DK + cc] = scale * x; });
    aKh.store([&](int t, int cc, float x) { o_kh[t * DK + cc] = x; });
    aW.store([&](int t, int cc, float x) { o_w[t * DK + cc] = -x; });
    aAq.store([&](int t, int s, float x) { o_aq[t * kChunk + s] = s <= t ? scale * x : 0.f; });
    aT.store([&](int t, int s, float x) { o_t[t * kChunk + s] = bet[s] * x; });
    // dGamma_L: the VB / 4 = 8 consecutive lanes sharing a row of h hold its partial sums
#pragma unroll
    for (int i = 0; i < HQ; ++i) {
        const float sum = sum8(hd[i]);
        const int e4 = tid + i * kGThreads;
        if ((e4 % (VB / 4)) == 0) p.dgl[slot * DK + e4 / (VB / 4)] = sum;
    }
    __syncthreads();
    if (tid < kChunk) {
        const int t = tid;
        float acc = 0.f;
        for (int gidx = 0; gidx < NG; ++gidx) acc += dbv_part[t * NG + gidx];
        p.dbv[slot * kChunk + t] = acc;
    }
}

// ============================================================== dk-side
constexpr int kCB = 32;  // channels per block in the dk-side kernel

// Channel blocks [cb, cb + kCB) are staged in two steps, so that a block's
// global loads can be issued one block ahead: load_* brings this thread's
// values into registers as they are stored in memory, put_* converts them and
// writes them to LDS.  (A conversion or mask right after a load would make the
// compiler wait for that load there, a block early.)
// q or k: thread element e = tid + NTH i is (token e / kCB, channel e % kCB).
template <int NTH, typename TIn>
struct QkBlock {
    TIn x[kChunk * kCB / NTH];
};
template <int DK, typename TIn, int NTH>
__device__ __forceinline__ void load_qk_block(const TIn* __restrict__ src, const ChunkRef& cr, int h, int H, int cb,
                                              QkBlock<NTH, TIn>& r) {
#pragma unroll
    for (int i = 0; i < kChunk * kCB / NTH; ++i) {
        const int e = threadIdx.x + i * NTH;
        const int t = e / kCB, cc = e - t * kCB;  // rows past the chunk end read row 0, zeroed in put_qk_block
        r.x[i] = src[tok_index(cr.t0 + (t < cr.len ? t : 0), h, H, DK) + cb + cc];
    }
}
// XT[c][t] = x (times the row's inverse norm if `rn` is given; zero past the chunk end)
template <int NTH, typename TIn>
__device__ __forceinline__ void put_qk_block(const QkBlock<NTH, TIn>& r, int len, const float* rn, float* XT) {
#pragma unroll
    for (int i = 0; i < kChunk * kCB / NTH; ++i) {
        const int e = threadIdx.x + i * NTH;
        const int t = e / kCB, cc = e - t * kCB;
        const float x = t < len ? Elem<TIn>::cvt(r.x[i]) : 0.f;
        XT[cc * kLD + t] = rn ? x * rn[t] : x;
    }
}

// The in-chunk cumulative log-decay G of channels [cb, cb + kCB), in base 2 as
// the intra-chunk kernel formed and saved it (flat past the chunk end, so every
// decay factor between a row and a later reference row stays at most 1): thread
// (sg, c) = (tid >> 5, tid & 31) holds R consecutive tokens of channel c.
template <int NTH>
struct GBlock {
    static constexpr int R = kChunk * kCB / NTH;
    float x[R];
};
template <int DK, int NTH>
__device__ __forceinline__ void load_g_block(const Prm& p, size_t slot, int cb, GBlock<NTH>& r) {
    constexpr int R = GBlock<NTH>::R;
    const int c = threadIdx.x & 31, sg = threadIdx.x >> 5;
    const float* gs = p.gcs + slot * kChunk * DK + cb + c;
#pragma unroll
    for (int i = 0; i < R; ++i) r.x[i] = gs[(size_t)(R * sg + i) * DK];
}
// GT[c][t] = G; ends with a barrier.
template <int NTH>
__device__ __forceinline__ void put_g_block(const GBlock<NTH>& r, float* GT) {
    constexpr int R = GBlock<NTH>::R;
    const int c = threadIdx.x & 31, sg = threadIdx.x >> 5;
#pragma unroll
    for (int i = 0; i < R; ++i) GT[c * kLD + R * sg + i] = r.x[i];
    __syncthreads();
}

// Inverse L2 norms of the raw rows of q or k (NTH / 64 threads per token).
template <int DK, typename TIn, int NTH>
__device__ __forceinline__ void row_rnorm(const TIn* __restrict__ src, const ChunkRef& cr, int h, int H, float* rn) {
    constexpr int PT = NTH / kChunk, CPT = DK / PT;  // threads per token, channels per thread
    static_assert((PT == 4 || PT == 8) && CPT % 4 == 0, "threads per token");
    const int t = threadIdx.x / PT, part = threadIdx.x % PT;
    float ss = 0.f;
    if (t < cr.len) {
        const TIn* row = src + tok_index(cr.t0 + t, h, H, DK) + CPT * part;
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
            float x[4];
            load4<TIn>(row + c, x);
            ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        }
    }
#pragma unroll
    for (int off = 1; off < PT; off <<= 1) ss += __shfl_xor(ss, off, 64);
    if (part == 0) rn[t] = 1.0f / sqrtf(ss + kL2Eps);
}

template <int DK, int DV, typename TIn, typename TOut>
__global__ void __launch_bounds__(kGThreads) bwd_dk_kernel(Prm p) {
    constexpr int LC = kCB + 4, LS = kCB + 1, NB = DK / kCB, NG = DK / 16;
    __shared__ float Tm[kChunk * kLD];   // T, later dAqk^T
    __shared__ float dT[kChunk * kLD];
    __shared__ float dAq[kChunk * kLD];  // scale * dAqk (lower incl. diagonal)
    __shared__ float dA[kChunk * kLD];   // dAkk (strictly lower)
    __shared__ float Y[kChunk * kLD];    // dT T^T, later dAkk^T
    __shared__ float QTb[kCB * kLD];
    __shared__ float KTb[kCB * kLD];
    __shared__ float GTb[kCB * kLD];
    __shared__ float X1[kChunk * LC];
    __shared__ float X2[kChunk * LC];
    __shared__ float X3[kChunk * LC];
    __shared__ float STk[kChunk * LS];  // Kt of the off-diagonal row sums
    __shared__ float bet[kChunk], rnq[kChunk], rnk[kChunk];
    __shared__ float dbw_part[kChunk * NG];
    __shared__ float wpart[kGWaves * kChunk];   // per-wave row partials
    __shared__ float dbA[kChunk], dotq[kChunk], dotk[kChunk];
    __shared__ float pa_part[kGWaves * NB];
    __shared__ float dgl[DK];

    const int c = blockIdx.x, h = blockIdx.y;
    const ChunkRef cr = p.seq.chunk(c);
    if (cr.len == 0) return;
    const size_t slot = (size_t)c * p.H + h;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const bool l2 = p.flags & 1u, gate = p.flags & 2u;
    const TIn* qin = (const TIn*)p.q;
    const TIn* kin = (const TIn*)p.k;
    const int last = cr.len - 1;

    // ---- load the chunk matrices and row scalars
    {
        const float* tmi = p.tm + slot * kTPacked;
        const float* dti = p.dtv + slot * kChunk * kChunk;
        const float* dai = p.daq + slot * kChunk * kChunk;
        #pragma unroll
    for (int e_i = 0; e_i < (kChunk * kChunk) / kGThreads; ++e_i) {
        const int e = threadIdx.x + e_i * kGThreads;
            const int idx = (e >> 6) * kLD + (e & 63);
            {
                const int t = e >> 6, s = e & 63;  // T packed: zero above the block diagonal
                const float x = tmi[tpk_index(t, (s >> 4) > (t >> 4) ? t : s)];
                Tm[idx] = (s >> 4) > (t >> 4) ? 0.f : x;
            }
            dT[idx] = dti[e];
            dAq[idx] = dai[e];
        }
    }
    if (threadIdx.x < kChunk) {
        const int t = threadIdx.x;
        float b = 0.f;
        if (t < cr.len) {
            b = p.beta[(size_t)(cr.t0 + t) * p.H + h];
            if (p.flags & 4u) b = sigmoid_f(b);
        }
        bet[t] = b;
        dbA[t] = 0.f; dotq[t] = 0.f; dotk[t] = 0.f;
        rnq[t] = 1.f; rnk[t] = 1.f;
    }
    if (threadIdx.x < DK) dgl[threadIdx.x] = p.dgl[slot * DK + threadIdx.x];
    __syncthreads();
    // channel block 0 of k, the log-decay and dw, for phase 3
    QkBlock<kGThreads, TIn> qr, kr;
    GBlock<kGThreads> gr;
    constexpr int NE = kChunk * kCB / kGThreads;
    float dwr[NE];
    const float* dwi = p.dwv + slot * kChunk * DK;
    auto load_dw = [&](int cb) {
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = threadIdx.x + i * kGThreads;
            const int t = e / kCB, cc = e - t * kCB;
            dwr[i] = dwi[t * DK + cb + cc];
        }
    };
    load_qk_block<DK, TIn, kGThreads>(kin, cr, h, p.H, 0, kr);
    load_g_block<DK, kGThreads>(p, slot, 0, gr);
    load_dw(0);
    if (l2) {
        row_rnorm<DK, TIn, kGThreads>(qin, cr, h, p.H, rnq);
        row_rnorm<DK, TIn, kGThreads>(kin, cr, h, p.H, rnk);
    }
    __syncthreads();

    // ---- phase 3: dT += dw (beta Kg)^T ; dKg = beta . (T^T dw) ; dbeta_w
    // (each block's global loads are issued during the block before)
    for (int b = 0; b < NB; ++b) {
        const int cb = b * kCB;
        put_qk_block(kr, cr.len, l2 ? rnk : nullptr, KTb);
        put_g_block<kGThreads>(gr, GTb);  // its barrier covers KTb
        if (b + 1 < NB) {
            load_qk_block<DK, TIn, kGThreads>(kin, cr, h, p.H, cb + kCB, kr);
            load_g_block<DK, kGThreads>(p, slot, cb + kCB, gr);
        } else {  // the first block of the pair-sum phase
            load_qk_block<DK, TIn, kGThreads>(qin, cr, h, p.H, 0, qr);
            load_qk_block<DK, TIn, kGThreads>(kin, cr, h, p.H, 0, kr);
            load_g_block<DK, kGThreads>(p, slot, 0, gr);
        }
#pragma unroll
        for (int e_i = 0; e_i < NE; ++e_i) {
            const int e = threadIdx.x + e_i * kGThreads;
            const int t = e / kCB, cc = e - t * kCB;
            X1[t * LC + cc] = dwr[e_i];
            const float kg = KTb[cc * kLD + t] * exp2_hw(GTb[cc * kLD + t]);
            X2[t * LC + cc] = kg;                 // Kg[t][c]
            QTb[cc * kLD + t] = bet[t] * kg;      // (beta Kg)^T, reusing the q tile
        }
        if (b + 1 < NB) load_dw(cb + kCB);
        __syncthreads();
        {
            constexpr int TILES = 16;  // 64 x 64 tiles of dT
            for (int tile = wave; tile < TILES; tile += kGWaves) {
                const int tm = tile >> 2, tn = tile & 3;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma16_f32(X1 + tm * 16 * LC, LC, 1, QTb + tn * 16, kLD, 1, 0, kCB, acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tm * 16 + 4 * (lane >> 4) + i, s = tn * 16 + (lane & 15);
                    dT[t * kLD + s] += acc[i];
                }
            }
            constexpr int TN = kCB / 16, T2 = (kChunk / 16) * TN;
            float* dkt = p.dkt + slot * kChunk * DK;
            for (int tile = wave; tile < T2; tile += kGWaves) {
                const int tm = tile / TN, tn = tile % TN;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma16_f32(Tm + tm * 16, 1, kLD, X1 + tn * 16, LC, 1, 16 * tm, kChunk, acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tm * 16 + 4 * (lane >> 4) + i, cc = tn * 16 + (lane & 15);
                    dkt[t * DK + cb + cc] = bet[t] * acc[i];
                    const float part = row16_sum(acc[i] * X2[t * LC + cc]);
                    if ((lane & 15) == 0) dbw_part[t * NG + (cb >> 4) + tn] = part;
                }
            }
        }
        __syncthreads();
    }

    // ---- phase 4: Y = dT T^T ; dA = -T^T Y (strictly lower)
    {
        for (int tile = wave; tile < 16; tile += kGWaves) {
            const int tm = tile >> 2, tn = tile & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma16_f32(dT + tm * 16 * kLD, kLD, 1, Tm + tn * 16 * kLD, 1, kLD, 0, 16 * (tn + 1), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) Y[(tm * 16 + 4 * (lane >> 4) + i) * kLD + tn * 16 + (lane & 15)] = acc[i];
        }
        __syncthreads();
        for (int tile = wave; tile < 16; tile += kGWaves) {
            const int tm = tile >> 2, tn = tile & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (tn <= tm) acc = mma16_f32(Tm + tm * 16, 1, kLD, Y + tn * 16, kLD, 1, 16 * tm, kChunk, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = tm * 16 + 4 * (lane >> 4) + i, bb = tn * 16 + (lane & 15);
                dA[a * kLD + bb] = bb < a ? -acc[i] : 0.f;
            }
        }
        __syncthreads();
        // transposed copies for the column sums (A operands with rows s)
        #pragma unroll
    for (int e_i = 0; e_i < (kChunk * kChunk) / kGThreads; ++e_i) {
        const int e = threadIdx.x + e_i * kGThreads;
            const int t = e >> 6, s = e & 63;
            Y[s * kLD + t] = dA[t * kLD + s];
            Tm[s * kLD + t] = dAq[t * kLD + s];
        }
        __syncthreads();
    }

    // ---- phases 5-6: pair terms, explicit factors, dg, preparation chain
    const float eA = gate ? expf(p.A_log[h]) : 0.f;
    const int t = lane;
    float pa_acc = 0.f;               // sum of dg * g over this wave's (t, c)
    float r_dbA = 0.f, r_dq = 0.f, r_dk = 0.f;  // per-row partials of this wave
    // Pair sums of Akk = beta_t sum_c k_t k_s e^{G_t - G_s} and Aqk = sum_c q_t k_s e^{G_t - G_s}
    // per channel block, split by 16-token blocks:
    //   off-diagonal blocks (I > J) as MFMA products, the decay factored through a
    //   reference row r between the pair, e^{G_t - G_r} e^{G_r - G_s} (both at most 1):
    //     row sums    (t in I, partners s in J)  r = 16 J + 15, the last row of J:
    //                 P[t][c] = sum_{s in J} dA[t][s] Kt[s][c],  Kt[s][c] = k_s e^{G_r - G_s}
    //     column sums (s in J, partners t in I)  r = 16 I, the first row of I:
    //                 C[s][c] = sum_{t in I} dA[t][s] Kb[t][c],  Kb[t][c] = beta_t k_t e^{G_t - G_r}
    //                 (and q_t e^{G_t - G_r} with dAq)
    //   so one scaled operand per side serves every block pair; the results are
    //   scaled by the other factor and gathered in LDS ([t][c]: ODk, ODq, ODc);
    //   diagonal blocks: split the same way into 4-token sub-blocks (4-deep
    //   products between sub-blocks), exact exps for the pairs inside one.
    float* const STa = dT;                 // Kb  [64][LS] (dT is free after phase 4)
    float* const STb = dT + kChunk * LS;   // Qb  [64][LS]
    float* const ODk = X1;                 // off-diagonal row sums with dA  [t][c]
    float* const ODq = X2;                 // off-diagonal row sums with dAq
    float* const ODc = X3;                 // off-diagonal column sums (dA and dAq)
    static_assert(2 * kChunk * LS <= kChunk * kLD && kChunk * LS <= kChunk * LC, "pair-sum staging must fit");
    for (int b = 0; b < NB; ++b) {
        const int cb = b * kCB;
        put_qk_block(qr, cr.len, l2 ? rnq : nullptr, QTb);
        put_qk_block(kr, cr.len, l2 ? rnk : nullptr, KTb);
        // this lane's epilogue operands (token t = lane, channels cb + CPW wave .. + CPW - 1, one
        // 16-byte access per array), issued now so that they arrive during the pair sums
        constexpr int CPW = kCB / kGWaves;
        static_assert(CPW == 4, "one float4 of channels per lane");
        const int c4 = CPW * wave;  // this wave's first channel in the block
        float dq_r[CPW], dkh_r[CPW], dkt_r[CPW], f_r[CPW] = {0.f, 0.f, 0.f, 0.f}, db_r[CPW] = {0.f, 0.f, 0.f, 0.f};
        const size_t wrow = slot * kChunk * DK + (size_t)t * DK + cb + c4;
        const size_t grow = tok_index(cr.t0 + (t < cr.len ? t : 0), h, p.H, DK) + cb + c4;
        load4<float>(p.dqt + wrow, dq_r);
        load4<float>(p.dkh + wrow, dkh_r);
        load4<float>(p.dkt + wrow, dkt_r);
        if (gate) {
            load4<float>(p.g + grow, f_r);
            load4<float>(p.dt_bias + h * DK + cb + c4, db_r);
        }
        put_g_block<kGThreads>(gr, GTb);  // ends with a barrier
        if (b + 1 < NB) {
            load_qk_block<DK, TIn, kGThreads>(qin, cr, h, p.H, cb + kCB, qr);
            load_qk_block<DK, TIn, kGThreads>(kin, cr, h, p.H, cb + kCB, kr);
            load_g_block<DK, kGThreads>(p, slot, cb + kCB, gr);
        }
        // -- off-diagonal row and column sums: the scaled operands of both, then both products
#pragma unroll
        for (int e_i = 0; e_i < kChunk * kCB / kGThreads; ++e_i) {
            const int e = threadIdx.x + e_i * kGThreads;
            const int sr = e >> 5, cc = e & 31, r = (sr | 15), r0 = sr & ~15;
            const float gs = GTb[cc * kLD + sr], ks = KTb[cc * kLD + sr];
            const float x = ks * exp2_hw(GTb[cc * kLD + r] - gs);  // row sums: partner s = sr, r its block's last row
            const float y = exp2_hw(gs - GTb[cc * kLD + r0]);       // column sums: t = sr, r0 its block's first row
            STk[sr * LS + cc] = sr < 48 ? x : 0.f;
            STa[sr * LS + cc] = sr >= 16 ? bet[sr] * ks * y : 0.f;
            STb[sr * LS + cc] = sr >= 16 ? QTb[cc * kLD + sr] * y : 0.f;
            if (sr >= 48) ODc[sr * LS + cc] = 0.f;
            if (sr < 16) { ODk[sr * LS + cc] = 0.f; ODq[sr * LS + cc] = 0.f; }
        }
        __syncthreads();
        if (wave < 6) {
            // row tile (I, tn), I = 1 .. 3, over J < I; column tile (J, tn), J = 0 .. 2, over I > J:
            // I + (3 - J) = 4 block products per wave
            const int tn = wave & 1, c = 16 * tn + frag_col();
            {
                const int I = 1 + (wave >> 1);
                f32x4 rk = {0.f, 0.f, 0.f, 0.f}, rq = rk;
                for (int J = 0; J < I; ++J) {
                    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
                    pk = mma16_f32(dA + 16 * I * kLD + 16 * J, kLD, 1, STk + 16 * J * LS + 16 * tn, LS, 1, 0, 16, pk);
                    pq = mma16_f32(dAq + 16 * I * kLD + 16 * J, kLD, 1, STk + 16 * J * LS + 16 * tn, LS, 1, 0, 16, pq);
                    const float gr = GTb[c * kLD + 16 * J + 15];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = exp2_hw(GTb[c * kLD + 16 * I + frag_row(i)] - gr);
                        rk[i] = fmaf(e, pk[i], rk[i]);
                        rq[i] = fmaf(e, pq[i], rq[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ODk[(16 * I + frag_row(i)) * LS + c] = rk[i];
                    ODq[(16 * I + frag_row(i)) * LS + c] = rq[i];
                }
            }
            {
                const int J = wave >> 1;
                f32x4 cs = {0.f, 0.f, 0.f, 0.f};
                for (int I = J + 1; I < 4; ++I) {
                    f32x4 pk = {0.f, 0.f, 0.f, 0.f};
                    pk = mma16_f32(Y + 16 * J * kLD + 16 * I, kLD, 1, STa + 16 * I * LS + 16 * tn, LS, 1, 0, 16, pk);
                    pk = mma16_f32(Tm + 16 * J * kLD + 16 * I, kLD, 1, STb + 16 * I * LS + 16 * tn, LS, 1, 0, 16, pk);
                    const float gr = GTb[c * kLD + 16 * I];
#pragma unroll
                    for (int i = 0; i < 4; ++i) cs[i] = fmaf(exp2_hw(gr - GTb[c * kLD + 16 * J + frag_row(i)]), pk[i], cs[i]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) ODc[(16 * J + frag_row(i)) * LS + c] = cs[i];
            }
        }
        __syncthreads();
        // -- diagonal blocks, by 4-token sub-blocks.  Wave (block bk, channels 16 tn ..):
        // lane l holds rows 16 bk + 4 g + r (r = 0..3) of column cc, the whole sub-block
        // g = l >> 4.  Pairs in different sub-blocks are 4-deep fp32 products
        // (v_mfma_f32_16x16x4_f32: lane l gives A[l & 15][l >> 4] and B[l >> 4][l & 15])
        // with the decay split at the sub-blocks' boundary rows (three factors, each at
        // most 1; the middle one zero where the partner sub-block is not on the summed
        // side); the pairs inside a sub-block take the exact exp of their difference.
        {
            const int bk = wave >> 1, tn = wave & 1;
            const int g4 = lane >> 4, n = lane & 15;
            const int cc = 16 * tn + n;
            const int ra = 16 * bk + 4 * g4, r0 = 16 * bk;
            const float* Gc = GTb + cc * kLD;  // G[.][cc], k[.][cc], q[.][cc]
            const float* Kc = KTb + cc * kLD;
            const float* Qc = QTb + cc * kLD;
            const float gA = Gc[ra], gB = Gc[ra + 3];  // G at the sub-block's first and last rows
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 ak = zero, aq = zero, ac = zero;
#pragma unroll
            for (int J = 0; J < 3; ++J) {  // row sums: partner sub-block J < g
                const int s = r0 + 4 * J + g4;  // this lane's B row (k index l >> 4)
                const float gbJ = Gc[r0 + 4 * J + 3];
                const float b = Kc[s] * exp2_hw(gbJ - Gc[s]);
                const int ai = (r0 + n) * kLD + r0 + 4 * J + g4;  // dA[16 bk + n][s]
                const f32x4 pk = __builtin_amdgcn_mfma_f32_16x16x4f32(dA[ai], b, zero, 0, 0, 0);
                const f32x4 pq = __builtin_amdgcn_mfma_f32_16x16x4f32(dAq[ai], b, zero, 0, 0, 0);
                const float m = J < g4 ? exp2_hw(gA - gbJ) : 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ak[r] = fmaf(m, pk[r], ak[r]);
                    aq[r] = fmaf(m, pq[r], aq[r]);
                }
            }
#pragma unroll
            for (int I = 1; I < 4; ++I) {  // column sums: partner sub-block I > g
                const int tI = r0 + 4 * I + g4;  // this lane's B row
                const float gaI = Gc[r0 + 4 * I];
                const float e = exp2_hw(Gc[tI] - gaI);
                const int ai = tI * kLD + r0 + n;  // dA[t][16 bk + n]
                f32x4 pc = __builtin_amdgcn_mfma_f32_16x16x4f32(dA[ai], bet[tI] * Kc[tI] * e, zero, 0, 0, 0);
                pc = __builtin_amdgcn_mfma_f32_16x16x4f32(dAq[ai], Qc[tI] * e, pc, 0, 0, 0);
                const float m = I > g4 ? exp2_hw(gaI - gB) : 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) ac[r] = fmaf(m, pc[r], ac[r]);
            }
            float gt[4], kt[4], qt[4], bt[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                gt[r] = Gc[ra + r];
                kt[r] = Kc[ra + r];
                qt[r] = Qc[ra + r];
                bt[r] = bet[ra + r];
            }
            // pairs inside the sub-block (all in this lane)
            float rkx[4], rqx[4], cx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float aqd = dAq[(ra + i) * kLD + ra + i];  // scale dAqk[t][t], decay 1
                rkx[i] = 0.f;
                rqx[i] = aqd * kt[i];
                cx[i] = aqd * qt[i];
            }
#pragma unroll
            for (int i = 1; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < i; ++j) {  // t = row i, s = row j < i
                    const float da = dA[(ra + i) * kLD + ra + j], daq = dAq[(ra + i) * kLD + ra + j];
                    const float e = exp2_hw(gt[i] - gt[j]);
                    const float kse = kt[j] * e;
                    rkx[i] = fmaf(da, kse, rkx[i]);
                    rqx[i] = fmaf(daq, kse, rqx[i]);
                    cx[j] = fmaf(bt[i] * da, kt[i] * e, cx[j]);
                    cx[j] = fmaf(daq, qt[i] * e, cx[j]);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (ra + r) * LS + cc;
                const float e = exp2_hw(gt[r] - gA), e2 = exp2_hw(gB - gt[r]);
                ODk[o] += fmaf(e, ak[r], rkx[r]);
                ODq[o] += fmaf(e, aq[r], rqx[r]);
                ODc[o] += fmaf(e2, ac[r], cx[r]);
            }
        }
        __syncthreads();
        // -- the per-token epilogue: lane = token t, CPW channels per wave
        float dg_o[CPW], dq_o[CPW], dk_o[CPW];
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int cc = c4 + j;
            const float gt = GTb[cc * kLD + t], kt = KTb[cc * kLD + t], qt = QTb[cc * kLD + t];
            const float rk = ODk[t * LS + cc], rq = ODq[t * LS + cc], ck = ODc[t * LS + cc], cq = 0.f;
            const float gam = exp2_hw(gt);
            const float gl_c = GTb[cc * kLD + last];
            const float eL = exp2_hw(gl_c - gt);
            const float dqt = dq_r[j], dkh = dkh_r[j], dkg = dkt_r[j];
            const float bt = bet[t];
            const float kh = kt * eL;
            float dQ = rq + gam * dqt;
            float dK = bt * rk + ck + cq + gam * dkg + eL * dkh;
            float dG = bt * kt * rk + qt * rq - kt * (ck + cq) + qt * gam * dqt + kt * gam * dkg - kh * dkh;
            // dG_L collects sum_t Kh . dKh and exp(G_L) dGamma_L
            const float sl = wave_sum(t < cr.len ? kh * dkh : 0.f);
            if (t == last) dG += sl + exp2_hw(gl_c) * dgl[cb + cc];
            if (t >= cr.len) { dQ = 0.f; dK = 0.f; dG = 0.f; }
            r_dbA += kt * rk;
            r_dq += qt * dQ;
            r_dk += kt * dK;
            // reverse in-chunk cumulative sum: dg_t = sum_{u >= t} dG_u
            const float sfx = wave_suffix_sum(dG);
            float dgo = sfx;
            if (gate) {
                float dfv = 0.f;
                if (t < cr.len) {
                    const float x = f_r[j] + db_r[j];
                    dfv = sfx * (-eA) * dsoftplus_f(x);
                    pa_acc += sfx * ((-eA) * softplus_f(x));
                }
                dgo = dfv;
                const float colsum = wave_sum(dfv);
                if (lane == 0) p.part_dt[slot * DK + cb + cc] = colsum;
            }
            dg_o[j] = dgo;
            dq_o[j] = dQ;
            dk_o[j] = dK;
        }
        if (t < cr.len) {
            store4<float>(p.dg + grow, dg_o);
            if (l2) {
                store4<float>(p.dxq + wrow, dq_o);
                store4<float>(p.dxk + wrow, dk_o);
            } else {
                store4<TOut>((TOut*)p.dq + grow, dq_o);
                store4<TOut>((TOut*)p.dk + grow, dk_o);
            }
        }
        __syncthreads();  // tiles of this block are reused by the next
    }

    // ---- row results: dbeta, and the second pass of the L2-norm chain
    wpart[wave * kChunk + t] = r_dbA;
    const float pa_w = wave_sum(pa_acc);
    if (lane == 0) pa_part[wave] = pa_w;
    __syncthreads();
    if (threadIdx.x < kChunk) {
        float acc = 0.f;
        for (int w = 0; w < kGWaves; ++w) acc += wpart[w * kChunk + t];
        dbA[t] = acc;
    }
    __syncthreads();
    wpart[wave * kChunk + t] = r_dq;
    __syncthreads();
    if (threadIdx.x < kChunk) {
        float acc = 0.f;
        for (int w = 0; w < kGWaves; ++w) acc += wpart[w * kChunk + t];
        dotq[t] = acc;
    }
    __syncthreads();
    wpart[wave * kChunk + t] = r_dk;
    __syncthreads();
    if (threadIdx.x < kChunk) {
        float acc = 0.f;
        for (int w = 0; w < kGWaves; ++w) acc += wpart[w * kChunk + t];
        dotk[t] = acc;
        if (t < cr.len) {
            float db = p.dbv[slot * kChunk + t] + dbA[t];
            for (int gidx = 0; gidx < NG; ++gidx) db += dbw_part[t * NG + gidx];
            if (p.flags & 4u) db *= bet[t] * (1.f - bet[t]);
            p.dbeta[(size_t)(cr.t0 + t) * p.H + h] = db;
        }
    }
    if (gate && threadIdx.x == 0) {
        float acc = 0.f;
        for (int w = 0; w < kGWaves; ++w) acc += pa_part[w];
        p.part_a[slot] = acc;
    }
    if (l2) {
        __syncthreads();
        // dx = r (dx^ - (x^ . dx^) x^), x^ the normalised row
        // four consecutive channels per thread and access
#pragma unroll
        for (int e_i = 0; e_i < kChunk * DK / 4 / kGThreads; ++e_i) {
            const int e = threadIdx.x + e_i * kGThreads;
            const int tt = e / (DK / 4), cc = 4 * (e - tt * (DK / 4));
            if (tt >= cr.len) continue;
            const size_t gi = tok_index(cr.t0 + tt, h, p.H, DK) + cc;
            const size_t wi = slot * kChunk * DK + (size_t)tt * DK + cc;
            float xq[4], xk[4], dxq[4], dxk[4], oq[4], ok[4];
            load4<TIn>(qin + gi, xq);
            load4<TIn>(kin + gi, xk);
            load4<float>(p.dxq + wi, dxq);
            load4<float>(p.dxk + wi, dxk);
            const float rq = rnq[tt], rk = rnk[tt], sq = dotq[tt], sk = dotk[tt];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                oq[i] = rq * (dxq[i] - sq * (xq[i] * rq));
                ok[i] = rk * (dxk[i] - sk * (xk[i] * rk));
            }
            store4<TOut>((TOut*)p.dq + gi, oq);
            store4<TOut>((TOut*)p.dk + gi, ok);
        }
    }
}

// ============================================================== gate parameter sums
// dA_log[h] = sum over chunks of part_a, ddt_bias[h][c] = sum of part_dt.  One
// workgroup per (head, column; column -1 = A_log): thread i takes chunks
// i, i + 256, ... and the 256 partial sums are added by a fixed tree, so the
// result does not depend on scheduling.
template <int DK>
__global__ void __launch_bounds__(kThreads) bwd_gate_sum_kernel(Prm p, int n_chunks) {
    __shared__ float red[kThreads];
    const int h = blockIdx.x, col = (int)blockIdx.y - 1, tid = threadIdx.x;
    float acc = 0.f;
    for (int c = tid; c < n_chunks; c += kThreads) {
        if (p.seq.chunk(c).len == 0) continue;
        const size_t slot = (size_t)c * p.H + h;
        acc += col < 0 ? p.part_a[slot] : p.part_dt[slot * DK + col];
    }
    red[tid] = acc;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off) red[tid] += red[tid + off];
        __syncthreads();
    }
    if (tid == 0) {
        if (col < 0) p.dA_log[h] = red[0];
        else p.ddt_bias[h * DK + col] = red[0];
    }
}

// ============================================================== host side
template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_bwd_t(const ChunkArgs& a, hipStream_t s) {
    const WsLayout L = ws_layout(a, true);
    Prm p = make_prm(a, L);
    p.hT = nullptr;
    p.o = nullptr;
    if constexpr (DK == 32 && DV == 64) {
        // every array the dk = 32 backward reads or writes must be in the workspace layout
        if (!p.tm || !p.hs || !p.dhs || !p.aqT || !p.pmT || !p.qhT || !p.part_a || !p.part_dt)
            return hipErrorInvalidValue;
    } else {
        // the reverse scan's operands (written by the intra-chunk kernel) and its outputs
        if (!p.tm || !p.hs || !p.vn || !p.dhs || !p.dvn || !p.aqT || !p.khb || !p.qgT || !p.wT || !p.gcs)
            return hipErrorInvalidValue;
    }
    if (!(a.flags & (1u << 4))) {  // no forward saved in ws: recompute it
        hipError_t e = launch_recompute(p, a, s);
        if (e != hipSuccess) return e;
    }
    constexpr Prec P = std::is_same<TIn, uint16_t>::value ? Prec::BF3 : Prec::F32;
    if constexpr (DK == 32 && DV == 64) {
        const int tot16 = a.N * a.H * (DV / kPsBV);
        KDA_LAUNCH("bwd_dh", (bwd_pdh_kernel<TIn, P, kPsBV>), dim3(tot16), dim3(kPsThreads), s, p, tot16);
    } else {
        constexpr int BV = DK <= 32 ? 32 : 16;  // dk >= 64: more workgroups; dk = 128: the operand tiles fill the LDS
        const int total = a.N * a.H * (DV / BV);
        KDA_LAUNCH("bwd_dh", (bwd_dh_scan_kernel<DK, DV, BV, TIn, P>), dim3(total), dim3(kDhThreads), s, p, total);
    }
    if (a.flags & (1u << 5)) return hipSuccess;  // KDA_F_DH0_ONLY: the state pass alone
    if (a.n_chunks_bound > 0) {
        if constexpr (DK == 32 && DV == 64) {
            KDA_LAUNCH("bwd_chunk", (bwd_chunk_kernel<DV, TIn, TOut, P>), dim3(a.n_chunks_bound, a.H), dim3(kBcThreads),
                       s, p);
        } else {
            KDA_LAUNCH("bwd_dv", (bwd_dv_kernel<DK, DV, TIn, TOut>), dim3(a.n_chunks_bound, a.H), dim3(kGThreads), s,
                       p);
            KDA_LAUNCH("bwd_dk", (bwd_dk_kernel<DK, DV, TIn, TOut>), dim3(a.n_chunks_bound, a.H), dim3(kGThreads), s,
                       p);
        }
    }
    if (a.flags & 2u) {
        KDA_LAUNCH("bwd_gate_sum", (bwd_gate_sum_kernel<DK>), dim3(a.H, DK + 1), dim3(kThreads), s, p,
                   a.n_chunks_bound);
    }
    return hipSuccess;
}

template <int DK, int DV>
static hipError_t launch_bwd_dims(const ChunkArgs& a, hipStream_t s) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_bwd_t<DK, DV, uint16_t, uint16_t>(a, s)
                          : launch_bwd_t<DK, DV, uint16_t, float>(a, s);
    return a.out_bf16 ? launch_bwd_t<DK, DV, float, uint16_t>(a, s) : launch_bwd_t<DK, DV, float, float>(a, s);
}

hipError_t launch_bwd(const ChunkArgs& a, hipStream_t s) {
    if (a.dk == 32 && a.dv == 64) return launch_bwd_dims<32, 64>(a, s);
    if (a.dk == 64 && a.dv == 64) return launch_bwd_dims<64, 64>(a, s);
    if (a.dk == 128 && a.dv == 128) return launch_bwd_dims<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
