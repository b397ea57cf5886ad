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
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = (__bf16)x[i];
            l[i] = (__bf16)(x[i] - (float)h[i]);
        }
        *(bf16x4*)(hi + r * ld + k) = h;
        *(bf16x4*)(lo + r * ld + k) = l;
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
