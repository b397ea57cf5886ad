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
// comes from memory as register fragments, prefetched four chunks ahead (two
// in the reverse pass).  BV = 32 is the one launched: with BV = 16 each
// (sequence, head) runs as four independent chains instead of two, and at the
// layer shape that measured slower (every chain re-reads P and qh).
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
    load_afrag(R.pm, frag_rec(p.pm + slot * kPsDK * kPsDK, 16 * tc + lr, 0, 1));
    load_afrag(R.qh, frag_rec(p.qh + slot * kChunk * kPsDK, 16 * wave + lr, 0, 1));
    R.hh = *(const f32x4*)(p.hh + slot * kPsDK * kPsDV + frag_order(jb + 16 * tj, 4, tc));
#pragma unroll
    for (int j = 0; j < NJ; ++j) R.ol[j] = *(const f32x4*)(p.ol + slot * kChunk * kPsDV + frag_order(jb + 16 * j, 8, wave));
}

// WO: write o; SS: store the state entering every chunk (for the backward).
// Both are compile-time, and every store of the loop body is issued on every
// path (masked lanes write to p.sink), so the compiler's waits on the memory
// counter count exactly the operand batches in flight.
template <typename TOut, Prec P, int BV, bool WO, bool SS>
__global__ void __launch_bounds__(kPsThreads) fwd_pscan_kernel(Prm p, int total_wg) {
    constexpr int DK = kPsDK, DV = kPsDV, LK = DK + 8, NV = DV / BV, NJ = BV / 16, NST = 2 * NJ;
    __shared__ __attribute__((aligned(16))) float sH[2][BV * LK];
    static_assert(STile<Prec::F32, DK>::ld == LK, "tile footprint");
    const STile<P, DK> HT[2] = {STile<P, DK>(sH[0], BV), STile<P, DK>(sH[1], BV)};
    // the chunk's output rows, staged so that they leave as 16-byte words (double buffered
    // like h^T: chunk c's rows are written after the barrier of chunk c and stored after
    // the barrier of chunk c + 1); rows padded by 16 bytes
    constexpr int OE = 16 / (int)sizeof(TOut), OLD = BV + OE, OWR = BV / OE;
    static_assert(kChunk * OWR % kPsThreads == 0, "whole 16-byte words per thread");
    __shared__ __attribute__((aligned(16))) TOut sO[WO ? 2 : 1][WO ? kChunk * OLD : OE];

    const int lid = xcd_local_id(blockIdx.x, total_wg);
    const int jbk = lid % NV, nh = lid / NV;
    const int n = nh / p.H, h = nh % p.H;
    if (n >= p.N) return;
    const int jb = jbk * BV;
    const int wave = wave_id(), lr = threadIdx.x & 15;
    const bool owner = NST == kPsThreads / 64 || wave < NST;  // holds a state tile
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
    // (`valid` false: past the sequence end, the store goes to p.sink)
    auto put_state = [&](int c, int buf, bool valid) {
        if (owner) {
            HT[buf].put4(jcol, crow, S);
            if constexpr (SS) {
                float* hs = p.hs + ((size_t)c * p.H + h) * DK * DV;
#pragma unroll
                for (int r = 0; r < 4; ++r) *(valid ? hs + (size_t)(crow + r) * DV + jb + jcol : p.sink) = S[r];
            }
        }
    };
    // the staged rows of chunk c (buffer `buf`) to o; rows past the chunk end, and every row
    // when `valid` is false, go to p.sink
    auto flush_o = [&](int c, int buf, bool valid) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const int len = valid ? SeqLayout::chunk_of(n, c - c0, s0, slen).len : 0;
        const int64_t t0 = valid ? SeqLayout::chunk_of(n, c - c0, s0, slen).t0 : 0;
#pragma unroll
        for (int i = 0; i < kChunk * OWR / kPsThreads; ++i) {
            const int w = threadIdx.x + i * kPsThreads, t = w / OWR, cw = w % OWR;
            const u32x4 x = *(const u32x4*)&sO[buf][t * OLD + cw * OE];
            TOut* dst = t < len ? o + tok_index(t0 + t, h, p.H, DV) + jb + cw * OE : (TOut*)p.sink;
            *(u32x4*)dst = x;
        }
    };
    auto step = [&](int c, int buf, const PsFwdOps<P, NJ>& Rc) {
        __syncthreads();  // h^T of this chunk complete; the other buffer's readers are done
        if constexpr (WO) flush_o(c - 1, buf ^ 1, c > c0);
        if (owner) {
            AFrag<P> fb;
            load_frag(fb, HT[buf].sub(16 * tj), 0);
            S = mma_ff(Rc.pm, fb, Rc.hh);
        }
        put_state(c + 1, buf ^ 1, c + 1 < c1);
        if constexpr (WO) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                AFrag<P> fo;
                load_frag(fo, HT[buf].sub(16 * j), 0);
                const f32x4 acc = mma_ff(Rc.qh, fo, Rc.ol[j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) Elem<TOut>::store(sO[buf], (16 * wave + frag_row(r)) * OLD + 16 * j + lr, acc[r]);
            }
        }
    };
    if (c0 < c1) {
        // PD chunks' operands in flight.  The loop body has no branch: every path
        // to the latch issues the same loads and stores, so each wait on the
        // memory counter covers one chunk's batch (a skippable part would make
        // the waits drain the prefetch).
        constexpr int PD = 4;
        PsFwdOps<P, NJ> R[PD];
#pragma unroll
        for (int i = 0; i < PD; ++i) ps_fwd_load<P, NJ>(p, slot_of(c0 + i), jb, tc, tj, R[i]);
        put_state(c0, 0, true);
        int c = c0;
        for (; c + PD - 1 < c1; c += PD) {
#pragma unroll
            for (int i = 0; i < PD; ++i) {
                step(c + i, i & 1, R[i]);
                ps_fwd_load<P, NJ>(p, slot_of(c + PD + i), jb, tc, tj, R[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < PD - 1; ++i)
            if (c + i < c1) step(c + i, i & 1, R[i]);
        if constexpr (WO) {
            __syncthreads();
            flush_o(c1 - 1, (c1 - 1 - c0) & 1, true);
        }
    }
    if (owner && p.hT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.hT[((size_t)nh * DK + crow + r) * DV + jb + jcol] = S[r];
    }
}

// ============================================================== reverse pass
template <typename TIn, Prec P, int BV>
struct PsBwdOps {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    static constexpr int NW4 = BV / 4 * (int)sizeof(TIn) / 16;  // 16-byte words of dO per thread
    AFrag<P> pt, qt[2];  // rows of P^T and of qh^T (this wave's state tile rows)
    // dO[t][jb + (BV / 4) part ..], t = tid >> 2, as loaded: converted to fp32
    // where it is used, so that nothing waits for the load before then
    u32x4 d[NW4];
    __device__ __forceinline__ float at(int i) const {
        if constexpr (sizeof(TIn) == 2) {
            const uint32_t w = d[i >> 3][(i >> 1) & 3];
            return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return __uint_as_float(d[i >> 2][i & 3]);
        }
    }
};

template <typename TIn, Prec P, int BV>
__device__ __forceinline__ void ps_bwd_load(const Prm& p, size_t slot, const ChunkRef& cr, int h, int jb, int tc,
                                            PsBwdOps<TIn, P, BV>& R) {
    const int lr = threadIdx.x & 15;
    load_afrag(R.pt, frag_rec(p.pmT + slot * kPsDK * kPsDK, 16 * tc + lr, 0, 1));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        load_afrag(R.qt[kb], frag_rec(p.qhT + slot * kChunk * kPsDK, 16 * tc + lr, kb, 2));
    // rows past the chunk end read row 0 (always valid); they are zeroed where used
    const int t = threadIdx.x >> 2, part = threadIdx.x & 3;
    const TIn* src = (const TIn*)p.d_o + tok_index(cr.t0 + (t < cr.len ? t : 0), h, p.H, kPsDV) + jb + (BV / 4) * part;
    static_assert(PsBwdOps<TIn, P, BV>::NW4 >= 1, "whole 16-byte words of dO per thread");
#pragma unroll
    for (int i = 0; i < PsBwdOps<TIn, P, BV>::NW4; ++i)
        R.d[i] = ((const typename PsBwdOps<TIn, P, BV>::u32x4*)src)[i];
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
    const bool owner = NST == kPsThreads / 64 || wave < NST;
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

    auto step = [&](int c, int buf, const PsBwdOps<TIn, P, BV>& Rc) {
        const size_t slot = (size_t)c * p.H + h;
        const int len = cref(c).len;
        if (owner) {
            float* dhs = p.dhs + slot * DK * DV;
#pragma unroll
            for (int r = 0; r < 4; ++r) dhs[(size_t)(crow + r) * DV + jb + jcol] = D[r];
            DT[buf].put4(jcol, crow, D);
        }
        // dO is a bf16 number: its hi part alone (the lo part is zero and neither stored nor read)
#pragma unroll
        for (int i = 0; i < BV / 4; ++i) OT[buf].put_hi((BV / 4) * part + i, tt, tt < len ? Rc.at(i) : 0.f);
        __syncthreads();  // D'^T and dO^T of this chunk complete (the other buffers were read a chunk ago)
        if (owner) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            AFrag<P> fb;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                load_frag_hi(fb, OT[buf].sub(16 * tj), 32 * kb);
                acc = mma_ff_bh(Rc.qt[kb], fb, acc);
            }
            load_frag(fb, DT[buf].sub(16 * tj), 0);
            D = mma_ff(Rc.pt, fb, acc);
        }
    };
    if (c0 < c1) {
        // chunks of operands in flight (branch-free body, as in the forward pass).  Two are
        // as fast as four (memory latency is not what sets the time per chunk) and keep the
        // kernel at 112 VGPRs; four took 256 + 8 AGPRs, six spilled to AGPRs and ran slower.
        constexpr int PD = 2;
        PsBwdOps<TIn, P, BV> R[PD];
#pragma unroll
        for (int i = 0; i < PD; ++i) ps_bwd_load<TIn, P, BV>(p, slot_of(c1 - 1 - i), cref(c1 - 1 - i), h, jb, tc, R[i]);
        int c = c1 - 1;
        for (; c - (PD - 1) >= c0; c -= PD) {
#pragma unroll
            for (int i = 0; i < PD; ++i) {
                step(c - i, i & 1, R[i]);
                ps_bwd_load<TIn, P, BV>(p, slot_of(c - PD - i), cref(c - PD - i), h, jb, tc, R[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < PD - 1; ++i)
            if (c - i >= c0) step(c - i, i & 1, R[i]);
    }
    if (owner && p.dh0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.dh0[((size_t)nh * DK + crow + r) * DV + jb + jcol] = D[r];
    }
}

}  // namespace kda
