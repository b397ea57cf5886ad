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
// One workgroup of four waves per (sequence, head, BV columns of the state),
// BV = 16 or 32: the state's 16x16 tiles (rows c, columns j) are held in fp32
// registers by waves 0 .. 2 BV / 16 - 1, and wave w forms output rows
// 16 w .. 16 w + 15.  The state is copied each chunk into a double-buffered LDS
// tile h^T[j][c], the B operand of every product of the chunk; everything else
// comes from memory as register fragments, prefetched two chunks ahead.  With
// BV = 16 each (sequence, head) runs as four independent chains, which keeps
// more operand loads in flight per CU than two chains of 32 columns.
#pragma once

#include "kda_chunk.cuh"
#include "kda_mma.cuh"

namespace kda {

constexpr int kPsThreads = 256;
constexpr int kPsDK = 32, kPsDV = 64;
constexpr int kPsBV = 32;  // state columns per workgroup

// Fragment-order index of the 16x16 tile of columns j0 .. j0 + 15 (j0 a
// multiple of 16): [32-column block][tile][lane][4] with `tiles_per_block`
// tiles per 32-column block and `row_tile` the tile's row index.
__device__ __forceinline__ size_t frag_order(int j0, int tiles_per_block, int row_tile) {
    const int tile = 2 * row_tile + ((j0 >> 4) & 1);
    return ((size_t)((j0 >> 5) * tiles_per_block + tile) * 64 + (threadIdx.x & 63)) * 4;
}

template <Prec P, int NJ>
struct PsFwdOps {
    AFrag<P> pm, qh;   // rows of P (this wave's state tile), rows of qh (this wave's output rows)
    f32x4 hh, ol[NJ];  // hh tile, ol tiles (fragment order)
};

template <Prec P, int NJ>
__device__ __forceinline__ void ps_fwd_load(const Prm& p, size_t slot, int jb, int tc, int tj, PsFwdOps<P, NJ>& R) {
    const int wave = wave_id(), lr = threadIdx.x & 15;
    load_afrag(R.pm, (const char*)(p.pm + slot * kPsDK * kPsDK) + (size_t)(16 * tc + lr) * kKBlockBytes);
    load_afrag(R.qh, (const char*)(p.qh + slot * kChunk * kPsDK) + (size_t)(16 * wave + lr) * kKBlockBytes);
    R.hh = *(const f32x4*)(p.hh + slot * kPsDK * kPsDV + frag_order(jb + 16 * tj, 4, tc));
#pragma unroll
    for (int j = 0; j < NJ; ++j) R.ol[j] = *(const f32x4*)(p.ol + slot * kChunk * kPsDV + frag_order(jb + 16 * j, 8, wave));
}

template <typename TOut, Prec P, int BV>
__global__ void __launch_bounds__(kPsThreads) fwd_pscan_kernel(Prm p, int total_wg, int write_o, int store_states) {
    constexpr int DK = kPsDK, DV = kPsDV, LK = DK + 8, NV = DV / BV, NJ = BV / 16, NST = 2 * NJ;
    __shared__ __attribute__((aligned(16))) float sH[2][BV * LK];
    static_assert(STile<Prec::F32, DK>::ld == LK, "tile footprint");
    const STile<P, DK> HT[2] = {STile<P, DK>(sH[0], BV), STile<P, DK>(sH[1], BV)};

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int jbk = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = jbk * BV;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const bool owner = wave < NST;  // holds a state tile
    const int sw = owner ? wave : 0;
    const int tc = sw / NJ, tj = sw % NJ;  // state tile (waves past NST mirror wave 0's loads, unused)
    const int crow = 16 * tc + frag_row(0), jcol = 16 * tj + lr;

    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (owner && p.h0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = p.h0[((size_t)nh * DK + crow + r) * DV + jb + jcol];
    }

    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    int64_t s0;
    int slen;
    p.seq.seq_tokens(n, s0, slen);
    TOut* o = (TOut*)p.o;
    auto slot_of = [&](int cc) { return (size_t)(cc < c1 ? cc : c1 - 1) * p.H + h; };

    // Chunk c: the state entering it is in h^T buffer `buf`.  The chain work
    // comes first -- the state leaving the chunk, its copy into the other buffer
    // (read after the next barrier) and its store -- then the chunk's output,
    // which only reads `buf`.  Both buffers were last read before this step's
    // barrier, so one barrier per chunk suffices.
    auto put_state = [&](int c, int buf) {
        if (owner) {
            HT[buf].put4(jcol, crow, S);
            if (store_states) {
                float* hs = p.hs + ((size_t)c * p.H + h) * DK * DV;
#pragma unroll
                for (int r = 0; r < 4; ++r) hs[(size_t)(crow + r) * DV + jb + jcol] = S[r];
            }
        }
    };
    auto step = [&](int c, int buf, const PsFwdOps<P, NJ>& Rc) {
        const ChunkRef cr = SeqLayout::chunk_of(n, c - c0, s0, slen);
        __syncthreads();  // h^T of this chunk complete; the other buffer's readers are done
        if (owner) {
            AFrag<P> fb;
            load_frag(fb, HT[buf].sub(16 * tj), 0);
            S = mma_ff(Rc.pm, fb, Rc.hh);
        }
        if (c + 1 < c1) put_state(c + 1, buf ^ 1);
        if (write_o) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
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
        PsFwdOps<P, NJ> R[2];
        ps_fwd_load<P, NJ>(p, slot_of(c0), jb, tc, tj, R[0]);
        ps_fwd_load<P, NJ>(p, slot_of(c0 + 1), jb, tc, tj, R[1]);
        put_state(c0, 0);
        // Pairs of chunks with no branch inside the loop body: every path to the
        // loop latch issues both prefetch batches, so each wait covers one batch
        // (a skippable second half would make the waits drain the prefetch).
        int c = c0;
        for (; c + 1 < c1; c += 2) {
            step(c, 0, R[0]);
            ps_fwd_load<P, NJ>(p, slot_of(c + 2), jb, tc, tj, R[0]);
            step(c + 1, 1, R[1]);
            ps_fwd_load<P, NJ>(p, slot_of(c + 3), jb, tc, tj, R[1]);
        }
        if (c < c1) step(c, 0, R[0]);
    }
    if (owner && p.hT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.hT[((size_t)nh * DK + crow + r) * DV + jb + jcol] = S[r];
    }
}

// ============================================================== reverse pass
template <Prec P, int BV>
struct PsBwdOps {
    AFrag<P> pt, qt[2];  // rows of P^T and of qh^T (this wave's state tile rows)
    float d[BV / 4];     // dO[t][jb + (BV / 4) part ..], t = tid >> 2
};

template <typename TIn, Prec P, int BV>
__device__ __forceinline__ void ps_bwd_load(const Prm& p, size_t slot, const ChunkRef& cr, int h, int jb, int tc,
                                            PsBwdOps<P, BV>& R) {
    const int lr = threadIdx.x & 15;
    load_afrag(R.pt, (const char*)(p.pmT + slot * kPsDK * kPsDK) + (size_t)(16 * tc + lr) * kKBlockBytes);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        load_afrag(R.qt[kb], (const char*)(p.qhT + slot * kChunk * kPsDK) + (size_t)((16 * tc + lr) * 2 + kb) * kKBlockBytes);
    // rows past the chunk end read row 0 (always valid) and are zeroed
    const int t = threadIdx.x >> 2, part = threadIdx.x & 3;
    const TIn* src = (const TIn*)p.d_o + tok_index(cr.t0 + (t < cr.len ? t : 0), h, p.H, kPsDV) + jb + (BV / 4) * part;
    if constexpr (BV == 32) load8<TIn>(src, R.d);
    else load4<TIn>(src, R.d);
#pragma unroll
    for (int i = 0; i < BV / 4; ++i) R.d[i] = t < cr.len ? R.d[i] : 0.f;
}

// Chunks in reverse: store D' (dL/dh at the chunk end) for the chunk kernels,
// then D = P^T D' + qh^T dO.  dO^T is staged in LDS per chunk (double
// buffered with the state tile, one barrier per chunk).
template <typename TIn, Prec P, int BV>
__global__ void __launch_bounds__(kPsThreads) bwd_pdh_kernel(Prm p, int total_wg) {
    constexpr int DK = kPsDK, DV = kPsDV, LK = DK + 8, LA = kChunk + 8, NV = DV / BV, NJ = BV / 16, NST = 2 * NJ;
    __shared__ __attribute__((aligned(16))) float sD[2][BV * LK];
    __shared__ __attribute__((aligned(16))) float sO[2][BV * LA];
    static_assert(STile<Prec::F32, DK>::ld == LK && STile<Prec::F32, kChunk>::ld == LA, "tile footprints");
    const STile<P, DK> DT[2] = {STile<P, DK>(sD[0], BV), STile<P, DK>(sD[1], BV)};
    const STile<P, kChunk> OT[2] = {STile<P, kChunk>(sO[0], BV), STile<P, kChunk>(sO[1], BV)};

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int jbk = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = jbk * BV;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const bool owner = wave < NST;
    const int sw = owner ? wave : 0;
    const int tc = sw / NJ, tj = sw % NJ;
    const int crow = 16 * tc + frag_row(0), jcol = 16 * tj + lr;
    const int tt = threadIdx.x >> 2, part = threadIdx.x & 3;  // dO staging: token, BV / 4 columns

    f32x4 D = {0.f, 0.f, 0.f, 0.f};
    if (owner && p.dhT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) D[r] = p.dhT[((size_t)nh * DK + crow + r) * DV + jb + jcol];
    }

    int c0, c1;
    p.seq.seq_chunks(n, c0, c1);
    int64_t s0;
    int slen;
    p.seq.seq_tokens(n, s0, slen);
    auto cref = [&](int cc) { return SeqLayout::chunk_of(n, (cc >= c0 ? cc : c0) - c0, s0, slen); };
    auto slot_of = [&](int cc) { return (size_t)(cc >= c0 ? cc : c0) * p.H + h; };

    auto step = [&](int c, int buf, const PsBwdOps<P, BV>& Rc) {
        const size_t slot = (size_t)c * p.H + h;
        if (owner) {
            float* dhs = p.dhs + slot * DK * DV;
#pragma unroll
            for (int r = 0; r < 4; ++r) dhs[(size_t)(crow + r) * DV + jb + jcol] = D[r];
            DT[buf].put4(jcol, crow, D);
        }
#pragma unroll
        for (int i = 0; i < BV / 4; ++i) OT[buf].put((BV / 4) * part + i, tt, Rc.d[i]);
        __syncthreads();  // D'^T and dO^T of this chunk complete (the other buffers were read a chunk ago)
        if (owner) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            AFrag<P> fb;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                load_frag(fb, OT[buf].sub(16 * tj), 32 * kb);
                acc = mma_ff(Rc.qt[kb], fb, acc);
            }
            load_frag(fb, DT[buf].sub(16 * tj), 0);
            D = mma_ff(Rc.pt, fb, acc);
        }
    };
    if (c0 < c1) {
        PsBwdOps<P, BV> R[2];
        ps_bwd_load<TIn, P, BV>(p, slot_of(c1 - 1), cref(c1 - 1), h, jb, tc, R[0]);
        ps_bwd_load<TIn, P, BV>(p, slot_of(c1 - 2), cref(c1 - 2), h, jb, tc, R[1]);
        int c = c1 - 1;
        for (; c - 1 >= c0; c -= 2) {  // (no branch in the body, as in the forward pass)
            step(c, 0, R[0]);
            ps_bwd_load<TIn, P, BV>(p, slot_of(c - 2), cref(c - 2), h, jb, tc, R[0]);
            step(c - 1, 1, R[1]);
            ps_bwd_load<TIn, P, BV>(p, slot_of(c - 3), cref(c - 3), h, jb, tc, R[1]);
        }
        if (c >= c0) step(c, 0, R[0]);
    }
    if (owner && p.dh0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.dh0[((size_t)nh * DK + crow + r) * DV + jb + jcol] = D[r];
    }
}

}  // namespace kda
