// kda_chunk.cuh -- staging and in-chunk algebra shared by the forward and
// backward chunk kernels.
//
// The chunked form is the exact algebraic rewrite of the token recurrence
// over a chunk of L <= 64 tokens entering with state h (the pages name the
// chunked FLA kernels -- Primus guide, the autotune paragraph of the training
// step; openkimi README, What is implemented -- but print no formulas; these
// are derived from the recurrence):
//   G_t      = sum_{s<=t} g_s                          (in-chunk, per channel)
//   Akk[t,s] = beta_t sum_c k_tc k_sc exp(G_tc - G_sc)     s <  t
//   Aqk[t,s] =        sum_c q_tc k_sc exp(G_tc - G_sc)     s <= t
//   T        = (I + Akk)^{-1}                          (unit lower triangular)
//   w = T Diag(beta) (exp(G) . K),   u = T Diag(beta) V
//   v_new    = u - w h
//   o        = scale ((exp(G) . Q) h + Aqk v_new)
//   h'       = Diag(exp(G_L)) h + (K . exp(G_L - G))^T v_new
// Decay factors are only ever formed as exp of a non-positive difference
// G_t - G_s (t >= s), so nothing overflows; the cumulative sum restarts at
// every chunk.
//
// LDS layout: per-chunk token tiles are stored transposed, X^T[c][t] with a
// padded row stride kLD, so a wave reading one channel for 64 tokens hits 64
// consecutive words.
#pragma once

#include "kda_device.cuh"
#include "kda_internal.h"

namespace kda {

constexpr int kLD = kChunk + 4;  // padded stride of [channel][token] tiles

// Logical workgroup id such that consecutive logical ids run on the same XCD
// (hardware deals workgroups round-robin over the 8 XCDs, each with its own
// L2).  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_local_id(int wg, int total) {
    if ((total & 7) != 0) return wg;
    return (wg & 7) * (total >> 3) + (wg >> 3);
}

// Kernel parameters (device view of one call).
struct Prm {
    int B, T, H, N;
    float scale;
    uint32_t flags;
    SeqLayout seq;
    const void *q, *k, *v;
    const float *g, *beta, *A_log, *dt_bias, *h0;
    void* o;
    float* hT;
    const void* d_o;
    const float* dhT;
    void *dq, *dk, *dv;
    float *dg, *dbeta, *dh0;
    float *dA_log, *ddt_bias;
    // workspace arrays (fp32), indexed by slot = chunk * H + head
    float *w, *u, *aqk, *tm, *hs, *vn;   // forward recompute (tm only for the backward)
    float *qg, *khT, *gl;                // exp(G) q, (k exp(G_L - G))^T, exp(G_L)
    float *qgT, *khb, *wT;               // (exp(G) q)^T, k exp(G_L - G), w^T: the reverse scan (dk >= 64)
    float* gcs;                          // in-chunk cumulative log-decay G (base 2, [t][c]) for the dk-side kernel (dk >= 64)
    float *dhs, *dvn;                    // backward state pass
    float *dqt, *dkh, *dwv, *daq, *dtv, *dgl, *dbv;
    float *dkt, *dxq, *dxk, *part_a, *part_dt;
    // affine form of a chunk (dk = 32): h' = P h + hh, o = ol + qh h, and for
    // the backward D = P^T D' + qh^T dO (fragment-form or fragment-order arrays, see
    // the intra-chunk kernel); aqT = Aqk^T for the backward chunk kernel
    float *pm, *pmT, *hh, *qh, *qhT, *ol, *aqT;
    // the workspace's first 256 bytes, never read: lanes whose store is masked
    // out write here instead, so a store is issued on every path
    float* sink;
};

__device__ __forceinline__ size_t tok_index(int64_t t, int h, int H, int d) {
    return ((size_t)t * H + h) * d;
}

// T = (I + A)^{-1} is unit lower triangular: in the workspace only its 10 blocks
// (I, J), J <= I, of 16x16 are kept, each row-major, in the order (0,0) (1,0)
// (1,1) (2,0) ... (3,3): 10 KB per chunk instead of 16.
constexpr int kTPacked = 10 * 256;  // floats per chunk
__host__ __device__ constexpr int tpk_index(int t, int s) {
    return ((((t >> 4) * ((t >> 4) + 1)) / 2 + (s >> 4)) << 8) + ((t & 15) << 4) + (s & 15);
}
// T[t][s .. s + 3] (s a multiple of 4) from the packed form: zero above the block
// diagonal (the load is issued on every lane, from the diagonal block there).
__device__ __forceinline__ f32x4 tpk_load4(const float* T, int t, int s) {
    const bool upper = (s >> 4) > (t >> 4);
    const f32x4 x = *(const f32x4*)(T + tpk_index(t, upper ? t : s));
    return upper ? f32x4{0.f, 0.f, 0.f, 0.f} : x;
}
// With bf16 inputs the dk = 32 kernels keep each group of four values in the
// packed form as its bf16 hi/lo split (the operand form of every product T
// enters): words (hi 0-1, hi 2-3, lo 0-1, lo 2-3), 16 bytes as in fp32.
typedef uint32_t tpk_words __attribute__((ext_vector_type(4)));
__device__ __forceinline__ tpk_words tpk_load4_split(const float* T, int t, int s) {
    const bool upper = (s >> 4) > (t >> 4);
    const tpk_words x = *(const tpk_words*)(T + tpk_index(t, upper ? t : s));
    return upper ? tpk_words{0u, 0u, 0u, 0u} : x;  // (the split of zeros is zero)
}

// T = (I + A)^{-1} for strictly lower-triangular A (64x64, stride kLD), by
// 16x16 blocks: diagonal blocks by forward substitution, then the off-diagonal
// blocks level by level,
//   T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ.
// Only the blocks on and below the diagonal of Tm are written (those above are
// zero by definition; readers of Tm mask them).  Only A's entries strictly below
// the diagonal enter the result (the others are read and discarded by
// selection).  Waves 0-3 compute; a workgroup of more waves passes the others
// through the barriers.  Ends with a barrier.
//
// Level LVL: wave w forms block (I, J) = (LVL + w, w).  Both products are MFMA
// chains whose operands are all read from LDS before the first product.  The
// sum X = sum_K A_IK T_KJ stays in its accumulator registers: in the product
// T_II X the contraction index is visited in a permuted order, lane group g
// taking index 4 g + s at step s, which is exactly the row that the lane's
// accumulator register s of X holds, so X is the B operand as it stands.
template <int LVL>
__device__ __forceinline__ void solve_level(const float* A, float* Tm, int wave, int lane) {
    const int I = LVL + wave, J = wave;
    if (I >= 4) return;
    const int r = lane & 15, kq = lane >> 4;
    constexpr int NS = 4 * LVL;  // steps of 4 over the contraction range [16 J, 16 I)
    float a[NS], b[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        a[s] = A[(16 * I + r) * kLD + 16 * J + 4 * s + kq];
        b[s] = Tm[(16 * J + 4 * s + kq) * kLD + 16 * J + r];
    }
    const f32x4 t = *(const f32x4*)&Tm[(16 * I + r) * kLD + 16 * I + 4 * kq];  // T_II, row r, columns 4 kq ..
    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], x, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) y = __builtin_amdgcn_mfma_f32_16x16x4f32(t[s], x[s], y, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) Tm[(16 * I + 4 * kq + i) * kLD + 16 * J + r] = -y[i];
}
__device__ __forceinline__ void solve_unit_lower(const float* A, float* Tm) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    if (wave < 4) {
        // diagonal block I = wave, right-looking: lane (column j = lane >> 2, quad
        // position q = lane & 3) holds rows 4 q .. 4 q + 3 of column j.  Once row k
        // is final it is x_k: its owner (quad position k >> 2) broadcasts it to its
        // quad by DPP, and every row t > k takes -A[t][k] x_k.  The lane's four rows
        // of A's block are read whole before the chain starts.
        const int I = wave, j = lane >> 2, q = lane & 3;
        const float* Ab = A + (16 * I + 4 * q) * kLD + 16 * I;  // this lane's first row of the block
        f32x4 ar[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) ar[i][c] = *(const f32x4*)(Ab + i * kLD + 4 * c);
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (4 * q + i == j) ? 1.f : 0.f;
        static_for16([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            constexpr int qk = k >> 2;
            constexpr int ctl = qk | (qk << 2) | (qk << 4) | (qk << 6);  // quad_perm [qk, qk, qk, qk]
            const float xk = dpp_f<ctl>(r[k & 3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = (4 * q + i > k) ? ar[i][k >> 2][k & 3] : 0.f;  // strictly below the diagonal only
                r[i] = fmaf(-a, xk, r[i]);
            }
        });
#pragma unroll
        for (int i = 0; i < 4; ++i) Tm[(16 * I + 4 * q + i) * kLD + 16 * I + j] = r[i];
    }
    __syncthreads();
    solve_level<1>(A, Tm, wave, lane);
    __syncthreads();
    solve_level<2>(A, Tm, wave, lane);
    __syncthreads();
    solve_level<3>(A, Tm, wave, lane);
    __syncthreads();
}

// Inclusive cumulative sum over the 64 rows of a 64 x 32 LDS array A (row
// stride ld), forward or in reverse, by every thread of the workgroup:
// thread (sg, c) = (tid >> 5, tid & 31) brings in x, the R = 64 * 32
// / blockDim values of rows R sg .. R sg + R - 1 of column c, scans them, and
// adds the totals of the segments before (after) its own.  The results go
// back to A.  seg: LDS [64 / R][32].  Starts with the segment exchange and
// ends with a barrier.
template <bool REV, int R>
__device__ __forceinline__ void col_scan_regs(float (&x)[R], float* A, int ld, float* seg) {
    constexpr int NS = 64 / R;
    const int c = threadIdx.x & 31, sg = threadIdx.x >> 5;
    if (!REV) {
#pragma unroll
        for (int i = 1; i < R; ++i) x[i] += x[i - 1];
        seg[sg * 32 + c] = x[R - 1];
    } else {
#pragma unroll
        for (int i = R - 2; i >= 0; --i) x[i] += x[i + 1];
        seg[sg * 32 + c] = x[0];
    }
    __syncthreads();
    float off = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const float v = seg[j * 32 + c];
        off += (REV ? j > sg : j < sg) ? v : 0.f;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) A[(R * sg + i) * ld + c] = x[i] + off;
    __syncthreads();
}

// Inclusive cumulative sum over the 64 rows of a 64 x 32 LDS array A (row
// stride ld), forward or in reverse, by a workgroup of 8 waves without a
// segment exchange: wave w scans columns 4 w .. 4 w + 3, lane (row-of-16 r =
// lane >> 4, position s = lane & 15) holds in x rows 4 s .. 4 s + 3 of column
// col = 4 w + r.  Each lane scans its four rows; the totals of the 16 lanes
// of a DPP row are combined by a Hillis-Steele scan over the row (lane shifts
// of 1, 2, 4, 8), and every lane adds the total of the lanes before (after)
// it.  The results go back to A, each element by the lane that read it.  Ends
// with a barrier.
template <bool REV>
__device__ __forceinline__ void col_scan16(float (&x)[4], float* A, int ld, int col, int s) {
    if (!REV) {
#pragma unroll
        for (int i = 1; i < 4; ++i) x[i] += x[i - 1];
    } else {
#pragma unroll
        for (int i = 2; i >= 0; --i) x[i] += x[i + 1];
    }
    // exclusive scan of the lane totals: shift by one lane, then an inclusive scan
    // (lanes shifted in from outside the row read zero)
    const float tot = REV ? x[0] : x[3];
    float v;
    if (!REV) {
        v = dpp_f<0x111>(tot);  // row_shr:1
        v += dpp_f<0x111>(v);
        v += dpp_f<0x112>(v);   // row_shr:2
        v += dpp_f<0x114>(v);   // row_shr:4
        v += dpp_f<0x118>(v);   // row_shr:8
    } else {
        v = dpp_f<0x101>(tot);  // row_shl:1
        v += dpp_f<0x101>(v);
        v += dpp_f<0x102>(v);
        v += dpp_f<0x104>(v);
        v += dpp_f<0x108>(v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) A[(4 * s + i) * ld + col] = x[i] + v;
    __syncthreads();
}

// ----------------------------------------------------------------- host helpers
// (kda_fwd.hip) Kernel parameters of a call, and the forward recompute used
// by the backward: intra-chunk (w, u, Aqk and, if p.tm is set, T) then the
// state pass (states entering each chunk, v_new; hT if p.hT is set).
Prm make_prm(const ChunkArgs& a, const WsLayout& L);
hipError_t launch_recompute(const Prm& p, const ChunkArgs& a, hipStream_t s);
hipError_t launch_recompute_intra(const Prm& p, const ChunkArgs& a, hipStream_t s);

// Register-resident accumulators for the 16x16 tiles of an M x N result that
// this wave owns (tile = wave + i * NW, NW waves), so several products can be
// accumulated over blocks of their contraction index without LDS traffic.
template <int M, int N, int NW = kWaves>
struct TileSet {
    static constexpr int TN = N / 16, TILES = (M / 16) * TN, NWAVES = NW;
    static constexpr int PER = (TILES + NW - 1) / NW;
    f32x4 acc[PER];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    template <class F>
    __device__ __forceinline__ void store(F f) const {
        const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int tile = wave + i * NW;
            if (tile < TILES) {
                const int tm = tile / TN, tn = tile % TN;
#pragma unroll
                for (int r = 0; r < 4; ++r) f(tm * 16 + 4 * (lane >> 4) + r, tn * 16 + (lane & 15), acc[i][r]);
            }
        }
    }
};

// Sum over the 16 lanes that share the rows of an MFMA D fragment (lanes
// 16g .. 16g+15); every lane of the group gets the sum.
__device__ __forceinline__ float row16_sum(float x) { return sum16(x); }

}  // namespace kda

