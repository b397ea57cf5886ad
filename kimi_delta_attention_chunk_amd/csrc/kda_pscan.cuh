// kda_pscan.cuh -- the sequential passes of dk = 32 on the affine chunk form.
//
// A chunk maps the state entering it to the state leaving it by an affine
// map, and its output is affine in the entering state too (the intra-chunk
// kernel's pass 3 forms the coefficients):
//   h'  = P h + hh,           P  = Diag(exp G_L) - Kh^T w,   hh = Kh^T u
//   o   = ol + qh h,          qh = scale (Qg - Aqk w),       ol = scale Aqk u
// so the only work that must run chunk after chunk is one 32 x 32 x 32 product
// per chunk and 32 state columns; the output product hangs off that chain.
// The reverse pass is the transpose:
//   D   = P^T D' + qh^T dO    (D' = dL/dh', D = dL/dh)
// One workgroup of four waves per (sequence, head, 32 columns of the state):
// wave w owns state tile (w >> 1, w & 1) (rows c, columns j) in fp32
// registers, and output rows 16 w .. 16 w + 15.  The state is copied each
// chunk into a double-buffered LDS tile h^T[j][c], the B operand of every
// product of the chunk; everything else comes from memory as register
// fragments, prefetched two chunks ahead.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kPsThreads = 256;
constexpr int kPsDK = 32, kPsDV = 64;

// Fragment-order index of a 16x16 tile: [32-column block][tile][lane][4].
__device__ __forceinline__ size_t frag_order(int colblock, int tiles_per_block, int tile) {
    return ((size_t)(colblock * tiles_per_block + tile) * 64 + (threadIdx.x & 63)) * 4;
}

template <Prec P>
struct PsFwdOps {
    AFrag<P> pm, qh;   // rows of P (this wave's state tile), rows of qh (this wave's output rows)
    f32x4 hh, ol[2];   // hh tile, ol tiles (fragment order)
};

template <Prec P>
__device__ __forceinline__ void ps_fwd_load(const Prm& p, size_t slot, int jbk, int tc, int tj, PsFwdOps<P>& R) {
    const int wave = wave_id(), lr = threadIdx.x & 15;
    load_afrag(R.pm, (const char*)(p.pm + slot * kPsDK * kPsDK) + (size_t)(16 * tc + lr) * kKBlockBytes);
    load_afrag(R.qh, (const char*)(p.qh + slot * kChunk * kPsDK) + (size_t)(16 * wave + lr) * kKBlockBytes);
    R.hh = *(const f32x4*)(p.hh + slot * kPsDK * kPsDV + frag_order(jbk, 4, 2 * tc + tj));
#pragma unroll
    for (int j = 0; j < 2; ++j) R.ol[j] = *(const f32x4*)(p.ol + slot * kChunk * kPsDV + frag_order(jbk, 8, 2 * wave + j));
}

template <typename TOut, Prec P>
__global__ void __launch_bounds__(kPsThreads) fwd_pscan_kernel(Prm p, int total_wg, int write_o, int store_states) {
    constexpr int DK = kPsDK, DV = kPsDV, BV = 32, LK = DK + 8, NV = DV / BV;
    __shared__ __attribute__((aligned(16))) float sH[2][BV * LK];
    const Tile<P> HT[2] = {Tile<P>(sH[0], BV, LK), Tile<P>(sH[1], BV, LK)};

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int jbk = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = jbk * BV;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const int tc = wave >> 1, tj = wave & 1;  // state tile
    const int crow = 16 * tc + frag_row(0), jcol = 16 * tj + lr;

    f32x4 S;
#pragma unroll
    for (int r = 0; r < 4; ++r) S[r] = p.h0 ? p.h0[((size_t)nh * DK + crow + r) * DV + jb + jcol] : 0.f;

    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    int64_t s0;
    int slen;
    p.seq.seq_tokens(n, s0, slen);
    TOut* o = (TOut*)p.o;
    auto slot_of = [&](int cc) { return (size_t)(cc < c1 ? cc : c1 - 1) * p.H + h; };

    auto step = [&](int c, int buf, const PsFwdOps<P>& Rc) {
        const ChunkRef cr = SeqLayout::chunk_of(n, c - c0, s0, slen);
        const size_t slot = (size_t)c * p.H + h;
        HT[buf].put4(jcol, crow, S);
        if (store_states) {
            float* hs = p.hs + slot * DK * DV;
#pragma unroll
            for (int r = 0; r < 4; ++r) hs[(size_t)(crow + r) * DV + jb + jcol] = S[r];
        }
        __syncthreads();  // h^T of this chunk complete (the other buffer was read a chunk ago)
        AFrag<P> fb;
        load_frag(fb, HT[buf].sub(16 * tj), 0);
        S = mma_ff(Rc.pm, fb, Rc.hh);
        if (write_o) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                AFrag<P> fo;
                load_frag(fo, HT[buf].sub(16 * j), 0);
                const f32x4 acc = mma_ff(Rc.qh, fo, Rc.ol[j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * wave + frag_row(r);
                    if (t < cr.len) Elem<TOut>::store(o, tok_index(cr.t0 + t, h, p.H, DV) + jb + 16 * j + lr, acc[r]);
                }
            }
        }
    };
    if (c0 < c1) {
        PsFwdOps<P> R[2];
        ps_fwd_load<P>(p, slot_of(c0), jbk, tc, tj, R[0]);
        ps_fwd_load<P>(p, slot_of(c0 + 1), jbk, tc, tj, R[1]);
        for (int c = c0; c < c1; c += 2) {
            step(c, 0, R[0]);
            ps_fwd_load<P>(p, slot_of(c + 2), jbk, tc, tj, R[0]);
            if (c + 1 < c1) {
                step(c + 1, 1, R[1]);
                ps_fwd_load<P>(p, slot_of(c + 3), jbk, tc, tj, R[1]);
            }
        }
    }
    if (p.hT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.hT[((size_t)nh * DK + crow + r) * DV + jb + jcol] = S[r];
    }
}

// ============================================================== reverse pass
template <Prec P>
struct PsBwdOps {
    AFrag<P> pt, qt[2];  // rows of P^T and of qh^T (this wave's state tile rows)
    float d[8];          // dO[t][jb + 8 part .. + 7], t = tid >> 2
};

template <typename TIn, Prec P>
__device__ __forceinline__ void ps_bwd_load(const Prm& p, size_t slot, const ChunkRef& cr, int h, int jb, int tc,
                                            PsBwdOps<P>& R) {
    const int lr = threadIdx.x & 15;
    load_afrag(R.pt, (const char*)(p.pmT + slot * kPsDK * kPsDK) + (size_t)(16 * tc + lr) * kKBlockBytes);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        load_afrag(R.qt[kb], (const char*)(p.qhT + slot * kChunk * kPsDK) + (size_t)((16 * tc + lr) * 2 + kb) * kKBlockBytes);
    // rows past the chunk end read row 0 (always valid) and are zeroed
    const int t = threadIdx.x >> 2, part = threadIdx.x & 3;
    load8<TIn>((const TIn*)p.d_o + tok_index(cr.t0 + (t < cr.len ? t : 0), h, p.H, kPsDV) + jb + 8 * part, R.d);
#pragma unroll
    for (int i = 0; i < 8; ++i) R.d[i] = t < cr.len ? R.d[i] : 0.f;
}

// Chunks in reverse: store D' (dL/dh at the chunk end) for the chunk kernels,
// then D = P^T D' + qh^T dO.  dO^T is staged in LDS per chunk (double
// buffered with the state tile, one barrier per chunk).
template <typename TIn, Prec P>
__global__ void __launch_bounds__(kPsThreads) bwd_pdh_kernel(Prm p, int total_wg) {
    constexpr int DK = kPsDK, DV = kPsDV, BV = 32, LK = DK + 8, LA = kChunk + 8, NV = DV / BV;
    __shared__ __attribute__((aligned(16))) float sD[2][BV * LK];
    __shared__ __attribute__((aligned(16))) float sO[2][BV * LA];
    const Tile<P> DT[2] = {Tile<P>(sD[0], BV, LK), Tile<P>(sD[1], BV, LK)};
    const Tile<P> OT[2] = {Tile<P>(sO[0], BV, LA), Tile<P>(sO[1], BV, LA)};

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int jbk = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = jbk * BV;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const int tc = wave >> 1, tj = wave & 1;
    const int crow = 16 * tc + frag_row(0), jcol = 16 * tj + lr;
    const int tt = threadIdx.x >> 2, part = threadIdx.x & 3;  // dO staging: token, 8 columns

    f32x4 D;
#pragma unroll
    for (int r = 0; r < 4; ++r) D[r] = p.dhT ? p.dhT[((size_t)nh * DK + crow + r) * DV + jb + jcol] : 0.f;

    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    int64_t s0;
    int slen;
    p.seq.seq_tokens(n, s0, slen);
    auto cref = [&](int cc) { return SeqLayout::chunk_of(n, (cc >= c0 ? cc : c0) - c0, s0, slen); };
    auto slot_of = [&](int cc) { return (size_t)(cc >= c0 ? cc : c0) * p.H + h; };

    auto step = [&](int c, int buf, const PsBwdOps<P>& Rc) {
        const size_t slot = (size_t)c * p.H + h;
        float* dhs = p.dhs + slot * DK * DV;
#pragma unroll
        for (int r = 0; r < 4; ++r) dhs[(size_t)(crow + r) * DV + jb + jcol] = D[r];
        DT[buf].put4(jcol, crow, D);
#pragma unroll
        for (int i = 0; i < 8; ++i) OT[buf].put(8 * part + i, tt, Rc.d[i]);
        __syncthreads();  // D'^T and dO^T of this chunk complete (the other buffers were read a chunk ago)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        AFrag<P> fb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            load_frag(fb, OT[buf].sub(16 * tj), 32 * kb);
            acc = mma_ff(Rc.qt[kb], fb, acc);
        }
        load_frag(fb, DT[buf].sub(16 * tj), 0);
        D = mma_ff(Rc.pt, fb, acc);
    };
    if (c0 < c1) {
        PsBwdOps<P> R[2];
        ps_bwd_load<TIn, P>(p, slot_of(c1 - 1), cref(c1 - 1), h, jb, tc, R[0]);
        ps_bwd_load<TIn, P>(p, slot_of(c1 - 2), cref(c1 - 2), h, jb, tc, R[1]);
        for (int c = c1 - 1; c >= c0; c -= 2) {
            step(c, 0, R[0]);
            ps_bwd_load<TIn, P>(p, slot_of(c - 2), cref(c - 2), h, jb, tc, R[0]);
            if (c - 1 >= c0) {
                step(c - 1, 1, R[1]);
                ps_bwd_load<TIn, P>(p, slot_of(c - 3), cref(c - 3), h, jb, tc, R[1]);
            }
        }
    }
    if (p.dh0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.dh0[((size_t)nh * DK + crow + r) * DV + jb + jcol] = D[r];
    }
}

}  // namespace kda
