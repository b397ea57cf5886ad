// kda_mma.cuh -- MFMA tile products on LDS operands, in two precisions.
//
//   Prec::F32  v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulate
//              (used when the inputs are fp32).
//   Prec::BF3  v_mfma_f32_16x16x32_bf16 three times on a hi/lo bf16 split of
//              each fp32 operand: a*b ~ ah*bh + ah*bl + al*bh, with
//              x = xh + xl + O(2^-17 |x|).  Relative error per product about
//              3 * 2^-17, far inside the bf16-input tolerance, at 16x the
//              fp32 MFMA rate per instruction (used when the inputs are bf16).
//
// Operands live in LDS as `Tile<P>`: R rows of K contiguous values with a row
// stride `ld` (a multiple of 8).  For F32 the tile is an fp32 array; for BF3
// the same bytes hold two bf16 arrays, the hi parts then the lo parts, so a
// value is split once when it is stored and every fragment read is a single
// 16-byte load of 8 consecutive bf16.
//
// Product convention: C(16x16) += A(16 x K) * B(16 x K)^T where A row m is
// output row m and B row n is output column n (B is stored transposed).
// k ranges step by 4 (F32) or 32 (BF3); a triangular factor's range may be
// widened to the step (widen) because its entries outside the exact range are
// stored zeros.
//
// D fragment (result): lane l holds rows 4*(l>>4)+i (i = 0..3) of column l&15.
#pragma once

#include "kda_device.cuh"

namespace kda {

enum class Prec { F32, BF3 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The hi/lo split of two values as packed bf16 pairs: hi = x rounded to bf16,
// lo = the remainder x - hi (exact in fp32) rounded to bf16.  The remainder is
// taken from the packed hi word, so a pair costs one conversion for hi, two bit
// operations, two subtractions and one conversion for lo (element-wise code
// converts every value twice).
// (The low half is moved up with a byte permute: written as a shift, the
// compiler rebuilds it from a second conversion of x0.)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hp, uint32_t& lp) {
    hp = pack_bf16x2(x0, x1);
    const float h0 = __uint_as_float(__builtin_amdgcn_perm(hp, 0u, 0x05040c0cu));  // bytes 1:0 of hp -> 3:2
    lp = pack_bf16x2(x0 - h0, x1 - __uint_as_float(hp & 0xffff0000u));
}
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
// four values (hi and lo each as two words) and eight values (four words)
__device__ __forceinline__ void split4(const float* x, u32x2v& h, u32x2v& l) {
    uint32_t h0, l0, h1, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    h = u32x2v{h0, h1};
    l = u32x2v{l0, l1};
}
__device__ __forceinline__ void split8(const float* x, u32x4v& h, u32x4v& l) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], hw[i], lw[i]);
    h = u32x4v{hw[0], hw[1], hw[2], hw[3]};
    l = u32x4v{lw[0], lw[1], lw[2], lw[3]};
}

template <Prec P> struct KStep;
template <> struct KStep<Prec::F32> { static constexpr int value = 4; };
template <> struct KStep<Prec::BF3> { static constexpr int value = 32; };

template <Prec P> struct Tile;

template <> struct Tile<Prec::F32> {
    float* p;
    int ld;
    __device__ __forceinline__ Tile(float* base, int rows, int ld_) : p(base), ld(ld_) { (void)rows; }
    __device__ __forceinline__ void put(int r, int k, float x) const { p[r * ld + k] = x; }
    __device__ __forceinline__ void put4(int r, int k, f32x4 x) const { *(f32x4*)(p + r * ld + k) = x; }
    __device__ __forceinline__ float get(int r, int k) const { return p[r * ld + k]; }
    __device__ __forceinline__ Tile sub(int r) const {
        Tile t = *this;
        t.p += r * ld;
        return t;
    }
};

template <> struct Tile<Prec::BF3> {
    __bf16* hi;
    __bf16* lo;
    int ld;
    // `base` provides rows * ld floats of LDS: hi occupies the first half of the bytes
    __device__ __forceinline__ Tile(float* base, int rows, int ld_)
        : hi((__bf16*)base), lo((__bf16*)base + rows * ld_), ld(ld_) {}
    __device__ __forceinline__ Tile(__bf16* h, __bf16* l, int ld_) : hi(h), lo(l), ld(ld_) {}
    __device__ __forceinline__ void put(int r, int k, float x) const {
        const __bf16 h = (__bf16)x;
        hi[r * ld + k] = h;
        lo[r * ld + k] = (__bf16)(x - (float)h);
    }
    // four consecutive values (k a multiple of 4)
    __device__ __forceinline__ void put4(int r, int k, f32x4 x) const {
        const float v[4] = {x[0], x[1], x[2], x[3]};
        u32x2v h, l;
        split4(v, h, l);
        *(u32x2v*)(hi + r * ld + k) = h;
        *(u32x2v*)(lo + r * ld + k) = l;
    }
    __device__ __forceinline__ float get(int r, int k) const { return (float)hi[r * ld + k] + (float)lo[r * ld + k]; }
    __device__ __forceinline__ Tile sub(int r) const { return Tile(hi + r * ld, lo + r * ld, ld); }
};

// acc += A(16 x [k0,k1)) * B(16 x [k0,k1))^T; A, B at the tile origin rows.
__device__ __forceinline__ f32x4 mma_tile(const Tile<Prec::F32>& A, const Tile<Prec::F32>& B, int k0, int k1,
                                          f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    for (int k = k0; k < k1; k += 4) {
        const float a = A.p[r * A.ld + k + g];
        const float b = B.p[r * B.ld + k + g];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

__device__ __forceinline__ f32x4 mma_tile(const Tile<Prec::BF3>& A, const Tile<Prec::BF3>& B, int k0, int k1,
                                          f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    for (int k = k0; k < k1; k += 32) {
        const int ao = r * A.ld + k + 8 * g, bo = r * B.ld + k + 8 * g;
        const bf16x8 ah = *(const bf16x8*)(A.hi + ao);
        const bf16x8 al = *(const bf16x8*)(A.lo + ao);
        const bf16x8 bh = *(const bf16x8*)(B.hi + bo);
        const bf16x8 bl = *(const bf16x8*)(B.lo + bo);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    }
    return acc;
}

// ----------------------------------------------------------------- A fragments from memory
// Operands produced by one kernel and consumed by another are stored in
// "fragment" form: per 16-row tile and block of 32 contraction indices, one
// 2 KB record in the lane order of the MFMA operand -- lane l = 16 g + (r & 15)
// holds indices 8 g .. 8 g + 7 of row r -- first 64 x 16 bytes (BF3: the 8 hi
// parts; F32: values 0 .. 3), then 64 x 16 bytes (BF3: the 8 lo parts; F32:
// values 4 .. 7).  A wave loads a fragment straight into registers with two
// fully contiguous 1 KB reads (whole cache lines, in order).  mma_frag then
// contracts it with a B tile in LDS over the same 8 indices per lane: for F32
// the 16x16x4 instruction at step kk takes index 8 g + kk from lane group g
// (A and B agree, so the sum is over every index exactly once).
template <Prec P> struct AFrag;
template <> struct AFrag<Prec::BF3> { bf16x8 hi, lo; };
template <> struct AFrag<Prec::F32> { f32x4 a, b; };

constexpr int kFragRecBytes = 2048;
// The record of (the 16-row tile of) row `row` and k-block kb of an array of
// KB k-blocks per row.
__device__ __forceinline__ char* frag_rec(void* base, int row, int kb, int KB) {
    return (char*)base + ((size_t)(row >> 4) * KB + kb) * kFragRecBytes;
}
__device__ __forceinline__ const char* frag_rec(const void* base, int row, int kb, int KB) {
    return (const char*)base + ((size_t)(row >> 4) * KB + kb) * kFragRecBytes;
}

// This lane's share of a fragment (rows of the record's tile, lane & 15 the row).
__device__ __forceinline__ void load_afrag(AFrag<Prec::BF3>& f, const char* rec) {
    const int lane = threadIdx.x & 63;
    f.hi = *(const bf16x8*)(rec + 16 * lane);
    f.lo = *(const bf16x8*)(rec + 1024 + 16 * lane);
}
__device__ __forceinline__ void load_afrag(AFrag<Prec::F32>& f, const char* rec) {
    const int lane = threadIdx.x & 63;
    f.a = *(const f32x4*)(rec + 16 * lane);
    f.b = *(const f32x4*)(rec + 1024 + 16 * lane);
}

// acc += A(16 x [kb, kb+32)) * B(16 x [kb, kb+32))^T, A from registers, B a tile
// in LDS at its origin row.
__device__ __forceinline__ f32x4 mma_frag(const AFrag<Prec::BF3>& a, const Tile<Prec::BF3>& B, int kb, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int bo = (lane & 15) * B.ld + kb + 8 * (lane >> 4);
    const bf16x8 bh = *(const bf16x8*)(B.hi + bo);
    const bf16x8 bl = *(const bf16x8*)(B.lo + bo);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, bh, acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 mma_frag(const AFrag<Prec::F32>& a, const Tile<Prec::F32>& B, int kb, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const float* bp = B.p + (lane & 15) * B.ld + kb + 8 * (lane >> 4);
    const f32x4 b0 = *(const f32x4*)bp, b1 = *(const f32x4*)(bp + 4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[kk], b0[kk], acc, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[kk], b1[kk], acc, 0, 0, 0);
    return acc;
}

// A fragment from this lane's 8 values (indices 8 g .. 8 g + 7 of the k-block,
// g = lane >> 4), split as a store to and load from fragment form would.
__device__ __forceinline__ void make_frag(AFrag<Prec::BF3>& f, const float (&x)[8]) {
    u32x4v h, l;
    split8(x, h, l);
    f.hi = __builtin_bit_cast(bf16x8, h);
    f.lo = __builtin_bit_cast(bf16x8, l);
}
__device__ __forceinline__ void make_frag(AFrag<Prec::F32>& f, const float (&x)[8]) {
    f.a = f32x4{x[0], x[1], x[2], x[3]};
    f.b = f32x4{x[4], x[5], x[6], x[7]};
}

// Write 8 consecutive values (indices 8 w .. 8 w + 7 of a k-block, w = which)
// of row `row` into its fragment record `rec`.
template <Prec P>
__device__ __forceinline__ void store_frag8(char* rec, int row, const float (&x)[8], int which);
template <>
__device__ __forceinline__ void store_frag8<Prec::BF3>(char* rec, int row, const float (&x)[8], int which) {
    u32x4v h, l;
    split8(x, h, l);
    char* b = rec + 16 * (16 * which + (row & 15));
    *(u32x4v*)b = h;
    *(u32x4v*)(b + 1024) = l;
}
template <>
__device__ __forceinline__ void store_frag8<Prec::F32>(char* rec, int row, const float (&x)[8], int which) {
    char* b = rec + 16 * (16 * which + (row & 15));
    *(f32x4*)b = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(b + 1024) = f32x4{x[4], x[5], x[6], x[7]};
}

// ----------------------------------------------------------------- fragments in registers
// Either operand of a product may be held as a register fragment: for C = A B^T
// the B fragment of output column n has the same lane layout as the A fragment
// of row n (row = lane & 15, indices 8 g .. 8 g + 7 of the k-block, g = lane >> 4).
// A fragment of a tile in LDS (`T` at its origin row), k-block starting at kb.
__device__ __forceinline__ void load_frag(AFrag<Prec::BF3>& f, const Tile<Prec::BF3>& T, int kb) {
    const int lane = threadIdx.x & 63;
    const int o = (lane & 15) * T.ld + kb + 8 * (lane >> 4);
    f.hi = *(const bf16x8*)(T.hi + o);
    f.lo = *(const bf16x8*)(T.lo + o);
}
__device__ __forceinline__ void load_frag(AFrag<Prec::F32>& f, const Tile<Prec::F32>& T, int kb) {
    const int lane = threadIdx.x & 63;
    const float* q = T.p + (lane & 15) * T.ld + kb + 8 * (lane >> 4);
    f.a = *(const f32x4*)q;
    f.b = *(const f32x4*)(q + 4);
}
// acc += A B^T over one k-block, both operands as register fragments.
__device__ __forceinline__ f32x4 mma_ff(const AFrag<Prec::BF3>& a, const AFrag<Prec::BF3>& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 mma_ff(const AFrag<Prec::F32>& a, const AFrag<Prec::F32>& b, f32x4 acc) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[kk], b.a[kk], acc, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[kk], b.b[kk], acc, 0, 0, 0);
    return acc;
}

// Write one value (index k of a k-block) of row `row` into its fragment record.
template <Prec P>
__device__ __forceinline__ void store_frag1(char* rec, int row, float x, int k);
template <>
__device__ __forceinline__ void store_frag1<Prec::BF3>(char* rec, int row, float x, int k) {
    const __bf16 h = (__bf16)x;
    __bf16* b = (__bf16*)(rec + 16 * (16 * (k >> 3) + (row & 15))) + (k & 7);
    b[0] = h;
    b[512] = (__bf16)(x - (float)h);  // 1024 bytes on: the lo part
}
template <>
__device__ __forceinline__ void store_frag1<Prec::F32>(char* rec, int row, float x, int k) {
    *(float*)(rec + 16 * (16 * (k >> 3) + (row & 15)) + ((k & 4) ? 1024 : 0) + 4 * (k & 3)) = x;
}

// Write 4 consecutive values (indices k0 .. k0 + 3 of a k-block, k0 a multiple
// of 4) of row `row` into its fragment record.  A D fragment holds, per lane,
// four consecutive rows of one column, i.e. four consecutive k-block indices of
// a row of the transposed result.
template <Prec P>
__device__ __forceinline__ void store_frag4(char* rec, int row, const f32x4& x, int k0);
template <>
__device__ __forceinline__ void store_frag4<Prec::BF3>(char* rec, int row, const f32x4& x, int k0) {
    const float v[4] = {x[0], x[1], x[2], x[3]};
    u32x2v h, l;
    split4(v, h, l);
    char* b = rec + 16 * (16 * (k0 >> 3) + (row & 15)) + 2 * (k0 & 4);
    *(u32x2v*)b = h;
    *(u32x2v*)(b + 1024) = l;
}
template <>
__device__ __forceinline__ void store_frag4<Prec::F32>(char* rec, int row, const f32x4& x, int k0) {
    *(f32x4*)(rec + 16 * (16 * (k0 >> 3) + (row & 15)) + ((k0 & 4) ? 1024 : 0)) = x;
}

// ----------------------------------------------------------------- swizzled tiles
// STile<P, C>: an R x C operand tile (C = 32 or 64 values per row) laid out for
// the LDS banks of gfx950.  Measured bank behaviour: ds_read_b128 serves a
// half-wave per pass in two 8-byte halves over 64 banks of 8 bytes; ds_write_b64
// serves 16 lanes per pass and ds_write_b16 a half-wave, both over 32 banks of
// 4 bytes.  A padded row stride (C + 8 bf16) makes every fragment read a 2-way
// conflict and the transposed scalar stores 4- to 8-way ones.  For BF3 the rows
// are therefore dense (C bf16 each, hi then lo array as in Tile) and the 16-byte
// group j of row r is stored at group j ^ f(r), with f chosen so that fragment
// reads, row-wise stores and transposed stores from row-wise or linear thread
// layouts are all conflict-free (transposed stores from a linear layout keep a
// 2-way conflict at C = 32).  The F32 layout is the padded one of Tile.
// sub(r) moves the origin down r rows (the swizzle follows the absolute row).
template <int C>
__device__ __forceinline__ int stile_swz(int row) {
    static_assert(C == 32 || C == 64, "swizzled tiles hold 32 or 64 values per row");
    if constexpr (C == 64) return ((row >> 1) & 7) ^ ((row >> 4) & 1);
    else return ((row >> 1) & 2) ^ (((row >> 3) & 1) * 3);
}
template <Prec P, int C> struct STile;
template <int C> struct STile<Prec::F32, C> {
    static constexpr int ld = C + 8;
    float* p;
    __device__ __forceinline__ STile(float* base, int rows) : p(base) { (void)rows; }
    __device__ __forceinline__ void put(int r, int k, float x) const { p[r * ld + k] = x; }
    __device__ __forceinline__ void put4(int r, int k, f32x4 x) const { *(f32x4*)(p + r * ld + k) = x; }
    // eight consecutive values (k a multiple of 8)
    __device__ __forceinline__ void put8(int r, int k, const float (&x)[8]) const {
        *(f32x4*)(p + r * ld + k) = f32x4{x[0], x[1], x[2], x[3]};
        *(f32x4*)(p + r * ld + k + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
    // (the _hi forms are for values that are bf16 numbers; in fp32 tiles they are the plain ones)
    __device__ __forceinline__ void put_hi(int r, int k, float x) const { put(r, k, x); }
    __device__ __forceinline__ void put4_hi(int r, int k, f32x4 x) const { put4(r, k, x); }
    __device__ __forceinline__ float get_hi(int r, int k) const { return p[r * ld + k]; }
    __device__ __forceinline__ f32x4 get4_hi(int r, int k) const { return *(const f32x4*)(p + r * ld + k); }
    __device__ __forceinline__ STile sub(int r) const {
        STile t = *this;
        t.p += r * ld;
        return t;
    }
    __device__ __forceinline__ Tile<Prec::F32> plain() const { return Tile<Prec::F32>(p, 0, ld); }
};
template <int C> struct STile<Prec::BF3, C> {
    __bf16* hi;
    __bf16* lo;
    int r0;
    __device__ __forceinline__ STile(float* base, int rows) : hi((__bf16*)base), lo((__bf16*)base + rows * C), r0(0) {}
    // element offset of (row r of the view, value k) in either array
    __device__ __forceinline__ int at(int r, int k) const {
        const int row = r0 + r;
        return row * C + 8 * ((k >> 3) ^ stile_swz<C>(row)) + (k & 7);
    }
    __device__ __forceinline__ void put(int r, int k, float x) const {
        const __bf16 h = (__bf16)x;
        const int o = at(r, k);
        hi[o] = h;
        lo[o] = (__bf16)(x - (float)h);
    }
    __device__ __forceinline__ void put4(int r, int k, f32x4 x) const {
        const float v[4] = {x[0], x[1], x[2], x[3]};
        u32x2v h, l;
        split4(v, h, l);
        const int o = at(r, k);
        *(u32x2v*)(hi + o) = h;
        *(u32x2v*)(lo + o) = l;
    }
    // Values already split: four (k a multiple of 4) as two words each of hi and lo
    // parts, or one as its two halves.
    __device__ __forceinline__ void put4_split(int r, int k, u32x2v h, u32x2v l) const {
        const int o = at(r, k);
        *(u32x2v*)(hi + o) = h;
        *(u32x2v*)(lo + o) = l;
    }
    __device__ __forceinline__ void put_split(int r, int k, uint16_t h, uint16_t l) const {
        const int o = at(r, k);
        *(uint16_t*)(hi + o) = h;
        *(uint16_t*)(lo + o) = l;
    }
    // Values that are bf16 numbers (bf16 inputs): the lo part is zero and is
    // neither stored nor read (load_frag_hi, mma_ff_ah / mma_ff_bh).
    __device__ __forceinline__ void put_hi(int r, int k, float x) const { hi[at(r, k)] = (__bf16)x; }
    __device__ __forceinline__ float get_hi(int r, int k) const { return (float)hi[at(r, k)]; }
    // four consecutive values (k a multiple of 4), one 8-byte read
    __device__ __forceinline__ f32x4 get4_hi(int r, int k) const {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 h = *(const bf16x4*)(hi + at(r, k));
        return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    }
    __device__ __forceinline__ void put4_hi(int r, int k, f32x4 x) const {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (__bf16)x[i];
        *(bf16x4*)(hi + at(r, k)) = h;
    }
    // eight consecutive values (k a multiple of 8): one 16-byte group of each array
    __device__ __forceinline__ void put8(int r, int k, const float (&x)[8]) const {
        u32x4v h, l;
        split8(x, h, l);
        const int o = at(r, k);
        *(u32x4v*)(hi + o) = h;
        *(u32x4v*)(lo + o) = l;
    }
    __device__ __forceinline__ STile sub(int r) const {
        STile t = *this;
        t.r0 += r;
        return t;
    }
};

// acc += A(16 x [k0,k1)) * B(16 x [k0,k1))^T on swizzled tiles (origins at their view rows).
template <int CA, int CB>
__device__ __forceinline__ f32x4 mma_tile(const STile<Prec::F32, CA>& A, const STile<Prec::F32, CB>& B, int k0, int k1,
                                          f32x4 acc) {
    return mma_tile(A.plain(), B.plain(), k0, k1, acc);
}
template <int CA, int CB>
__device__ __forceinline__ f32x4 mma_tile(const STile<Prec::BF3, CA>& A, const STile<Prec::BF3, CB>& B, int k0, int k1,
                                          f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int ra = A.r0 + r, rb = B.r0 + r;
    const int fa = stile_swz<CA>(ra), fb = stile_swz<CB>(rb);
    for (int k = k0; k < k1; k += 32) {
        const int j = (k >> 3) + g;
        const int ao = ra * CA + 8 * (j ^ fa), bo = rb * CB + 8 * (j ^ fb);
        const bf16x8 ah = *(const bf16x8*)(A.hi + ao);
        const bf16x8 al = *(const bf16x8*)(A.lo + ao);
        const bf16x8 bh = *(const bf16x8*)(B.hi + bo);
        const bf16x8 bl = *(const bf16x8*)(B.lo + bo);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    }
    return acc;
}
// As mma_tile, for a B tile whose values are bf16 numbers (stored with put_hi):
// B's lo part is zero and is not read, two MFMAs per k-block.
template <int CA, int CB>
__device__ __forceinline__ f32x4 mma_tile_bh(const STile<Prec::BF3, CA>& A, const STile<Prec::BF3, CB>& B, int k0,
                                             int k1, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int ra = A.r0 + r, rb = B.r0 + r;
    const int fa = stile_swz<CA>(ra), fb = stile_swz<CB>(rb);
    for (int k = k0; k < k1; k += 32) {
        const int j = (k >> 3) + g;
        const int ao = ra * CA + 8 * (j ^ fa), bo = rb * CB + 8 * (j ^ fb);
        const bf16x8 ah = *(const bf16x8*)(A.hi + ao);
        const bf16x8 al = *(const bf16x8*)(A.lo + ao);
        const bf16x8 bh = *(const bf16x8*)(B.hi + bo);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    }
    return acc;
}
template <int CA, int CB>
__device__ __forceinline__ f32x4 mma_tile_bh(const STile<Prec::F32, CA>& A, const STile<Prec::F32, CB>& B, int k0,
                                             int k1, f32x4 acc) {
    return mma_tile(A.plain(), B.plain(), k0, k1, acc);
}
// acc += A(16 x [k0, k0+16)) * B(16 x [k0, k0+16))^T on swizzled tiles, k0 a
// multiple of 16: a 16-deep product (v_mfma_f32_16x16x16_bf16, three times on the
// hi/lo split; lane l holds indices k0 + 4 (l >> 4) .. + 3 of row l & 15).
template <int CA, int CB>
__device__ __forceinline__ f32x4 mma_tile_k16(const STile<Prec::F32, CA>& A, const STile<Prec::F32, CB>& B, int k0,
                                              f32x4 acc) {
    return mma_tile(A.plain(), B.plain(), k0, k0 + 16, acc);
}
template <int CA, int CB>
__device__ __forceinline__ f32x4 mma_tile_k16(const STile<Prec::BF3, CA>& A, const STile<Prec::BF3, CB>& B, int k0,
                                              f32x4 acc) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, k = k0 + 4 * (lane >> 4);
    const int ao = A.at(r, k), bo = B.at(r, k);
    const s16x4 ah = *(const s16x4*)(A.hi + ao), al = *(const s16x4*)(A.lo + ao);
    const s16x4 bh = *(const s16x4*)(B.hi + bo), bl = *(const s16x4*)(B.lo + bo);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
    return acc;
}
// A fragment (rows of the view, k-block starting at kb) of a swizzled tile.
template <int C>
__device__ __forceinline__ void load_frag(AFrag<Prec::BF3>& f, const STile<Prec::BF3, C>& T, int kb) {
    const int lane = threadIdx.x & 63;
    const int o = T.at(lane & 15, kb + 8 * (lane >> 4));
    f.hi = *(const bf16x8*)(T.hi + o);
    f.lo = *(const bf16x8*)(T.lo + o);
}
template <int C>
__device__ __forceinline__ void load_frag(AFrag<Prec::F32>& f, const STile<Prec::F32, C>& T, int kb) {
    load_frag(f, T.plain(), kb);
}
template <int C>
__device__ __forceinline__ f32x4 mma_frag(const AFrag<Prec::BF3>& a, const STile<Prec::BF3, C>& B, int kb, f32x4 acc) {
    AFrag<Prec::BF3> b;
    load_frag(b, B, kb);
    return mma_ff(a, b, acc);
}
template <int C>
__device__ __forceinline__ f32x4 mma_frag(const AFrag<Prec::F32>& a, const STile<Prec::F32, C>& B, int kb, f32x4 acc) {
    return mma_frag(a, B.plain(), kb, acc);
}

// Fragments of operands whose values are bf16 numbers (stored with put_hi /
// put4_hi): only the hi part is read, and the product with the other operand's
// split skips the term that would multiply a zero lo part.
template <int C>
__device__ __forceinline__ void load_frag_hi(AFrag<Prec::BF3>& f, const STile<Prec::BF3, C>& T, int kb) {
    const int lane = threadIdx.x & 63;
    f.hi = *(const bf16x8*)(T.hi + T.at(lane & 15, kb + 8 * (lane >> 4)));
}
template <int C>
__device__ __forceinline__ void load_frag_hi(AFrag<Prec::F32>& f, const STile<Prec::F32, C>& T, int kb) {
    load_frag(f, T, kb);
}
// acc += A B^T, A's values bf16 numbers
__device__ __forceinline__ f32x4 mma_ff_ah(const AFrag<Prec::BF3>& a, const AFrag<Prec::BF3>& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 mma_ff_ah(const AFrag<Prec::F32>& a, const AFrag<Prec::F32>& b, f32x4 acc) {
    return mma_ff(a, b, acc);
}
// acc += A B^T, B's values bf16 numbers
__device__ __forceinline__ f32x4 mma_ff_bh(const AFrag<Prec::BF3>& a, const AFrag<Prec::BF3>& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4 mma_ff_bh(const AFrag<Prec::F32>& a, const AFrag<Prec::F32>& b, f32x4 acc) {
    return mma_ff(a, b, acc);
}

// Round a k range outward to the step of P (for triangular factors whose
// entries outside the exact range are zero).
template <Prec P>
__device__ __forceinline__ void widen(int& k0, int& k1) {
    constexpr int S = KStep<P>::value;
    k0 = (k0 / S) * S;
    k1 = ((k1 + S - 1) / S) * S;
}

__device__ __forceinline__ int frag_row(int i) { return 4 * ((threadIdx.x & 63) >> 4) + i; }
__device__ __forceinline__ int frag_col() { return threadIdx.x & 15; }

}  // namespace kda
