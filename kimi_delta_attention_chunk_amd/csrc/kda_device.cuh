// kda_device.cuh -- device helpers shared by the gfx950 KDA kernels.
//
// Wave64 everywhere.  Matrix products use the CDNA MFMA 16x16 tiles:
//   v_mfma_f32_16x16x4_f32 : A 16x4, B 4x16, C/D 16x16, fp32 in and out.
// Operand layout for one wave (lane l = 0..63):
//   A fragment: element (row = l & 15, k = l >> 4)
//   B fragment: element (k = l >> 4, col = l & 15)
//   D fragment: four floats, rows 4*(l >> 4) + i (i = 0..3), col = l & 15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace kda {

constexpr int kChunk = 64;     // chunk length (tokens)
constexpr int kThreads = 256;  // threads per workgroup of the chunk kernels
constexpr int kWaves = kThreads / 64;
constexpr float kL2Eps = 1e-6f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar)
// value: tile and row offsets derived from it stay in SGPRs instead of being
// recomputed per lane.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ----------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
    return __uint_as_float(((uint32_t)u) << 16);
}
// Round to nearest even; NaN stays NaN (the hardware conversion,
// v_cvt_pk_bf16_f32, in the default round-to-nearest-even mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values packed as a 32-bit word, a in the low half (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static float cvt(float x) { return x; }  // a value as loaded, to fp32
    __device__ __forceinline__ static void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static float cvt(uint16_t x) { return bf16_to_f32(x); }
    __device__ __forceinline__ static void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Four consecutive elements of a row (8- or 16-byte aligned) as fp32, and back.
template <typename TIn>
__device__ __forceinline__ void load4(const TIn* p, float (&x)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&x)[4]) {
    const f32x4 a = *(const f32x4*)p;
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float (&x)[4]) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = *(const u32x2*)p;
    x[0] = __uint_as_float(v[0] << 16);
    x[1] = __uint_as_float(v[0] & 0xffff0000u);
    x[2] = __uint_as_float(v[1] << 16);
    x[3] = __uint_as_float(v[1] & 0xffff0000u);
}
template <typename TOut>
__device__ __forceinline__ void store4(TOut* p, const float (&x)[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&x)[4]) {
    *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float (&x)[4]) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v;
    v[0] = pack_bf16x2(x[0], x[1]);
    v[1] = pack_bf16x2(x[2], x[3]);
    *(u32x2*)p = v;
}

// Load 8 consecutive elements of one token row (16-byte aligned) as fp32.
// Store 8 consecutive fp32 values to one token row (16-byte aligned) as TOut.
template <typename TOut>
__device__ __forceinline__ void store8(TOut* p, const float (&x)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
    *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float (&x)[8]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *(u32x4*)p = v;
}

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3]; x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}

// ----------------------------------------------------------------- prep math
// Hardware transcendentals (v_exp_f32, v_log_f32, v_rcp_f32: about 1 ulp),
// instead of the library's range-reduced versions: the preparation runs
// them per element in every chunk kernel.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
// The chunk kernels keep the in-chunk cumulative log-decay in base 2 (G log2 e),
// so each decay factor exp(G_t - G_s) is one v_exp_f32 of a difference.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
// log(1 + y) for y >= 0 to full relative precision: log(z) * y / (z - 1) with
// z = 1 + y rounded, which cancels the rounding of z (y when z rounds to 1).
// The correction factor y / (z - 1) is within an ulp or two of 1, so the
// hardware reciprocal (about 1 ulp) is as good as a division here.
__device__ __forceinline__ float log1p_hw(float y) {
    const float z = 1.f + y;
    const float l = __builtin_amdgcn_logf(z) * 0.6931471805599453f;
    return z == 1.f ? y : l * (y * __builtin_amdgcn_rcpf(z - 1.f));
}
// (x)^-1/2 by the hardware reciprocal square root (about 1 ulp), for the L2 norms.
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }
// softplus with the usual threshold: x for x > 20; else max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ float softplus_f(float x) {
    return x > 20.f ? x : fmaxf(x, 0.f) + log1p_hw(exp_hw(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.f + exp_hw(-x)); }
__device__ __forceinline__ float dsoftplus_f(float x) { return x > 20.f ? 1.f : sigmoid_f(x); }

// ----------------------------------------------------------------- cross-lane sums
// All of these run on the VALU (DPP lane permutes and the gfx950 permlane
// swaps), with no LDS round trip.  They must be called with every lane of the
// wave active.  Each lane of a group receives the same sum: pair sums are
// formed as x_a + x_b on both sides, which is exact commutation.
template <int CTL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTL, 0xF, 0xF, false));
}
// lanes l, l^1, l^2, l^3 (a quad)
__device__ __forceinline__ float sum4(float x) {
    x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
    return x + dpp_f<0x4E>(x);  // quad_perm [2,3,0,1]
}
// the 8 lanes 8m .. 8m+7
__device__ __forceinline__ float sum8(float x) { x = sum4(x); return x + dpp_f<0x141>(x); }   // row_half_mirror
// the 16 lanes 16m .. 16m+15 (one DPP row)
__device__ __forceinline__ float sum16(float x) { x = sum8(x); return x + dpp_f<0x140>(x); }  // row_mirror
// Sum over the N consecutive lanes (N = 4, 8 or 16) of this lane's group.
template <int N>
__device__ __forceinline__ float row_group_sum(float x) {
    if constexpr (N == 4) return sum4(x);
    else if constexpr (N == 8) return sum8(x);
    else {
        static_assert(N == 16, "groups of 4, 8 or 16 lanes");
        return sum16(x);
    }
}
// Sum over the lanes of this wave congruent to this lane modulo N (a butterfly
// in a fixed order).
template <int N>
__device__ __forceinline__ float rows_of_wave_sum(float x) {
#pragma unroll
    for (int off = N; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}
// lanes l and l^8
__device__ __forceinline__ float sum_x8(float x) { return x + dpp_f<0x128>(x); }  // row_ror:8
// lanes l, l^16, l^32, l^48
__device__ __forceinline__ float sum_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);   // even row + odd row
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);  // lower half + upper half
}
__device__ __forceinline__ float wave_sum(float x) { return sum_rows(sum16(x)); }

// Lane n of this lane's 16-lane row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}

// Inclusive suffix sum over the 64 lanes: lane t receives x_t + x_{t+1} + ... + x_63.
// Within each 16-lane row a shift-left scan (row_shl 1, 2, 4, 8; lanes past the
// row end read 0), then the totals of the later rows are added: a row's total is
// its first lane after the scan, and the permlane swaps bring the other rows'.
__device__ __forceinline__ float wave_suffix_sum(float x) {
    x += dpp_f<0x101>(x);  // row_shl:1
    x += dpp_f<0x102>(x);  // row_shl:2
    x += dpp_f<0x104>(x);  // row_shl:4
    x += dpp_f<0x108>(x);  // row_shl:8
    const float tot = row_bcast<0>(x);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(tot), __float_as_int(tot), false, false);
    const float odd = __int_as_float(a[1]);  // total of the odd row of this lane's pair (row 1 or 3)
    const float pair = __int_as_float(a[0]) + odd;
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(pair), __float_as_int(pair), false, false);
    const float upper = __int_as_float(b[1]);  // rows 2 + 3
    const int r = (threadIdx.x & 63) >> 4;
    const float later = r == 0 ? odd + upper : r == 1 ? upper : r == 2 ? odd : 0.f;
    return x + later;
}

// f(std::integral_constant<int, u>) for u = 0 .. 15, in order (for DPP
// controls and other immediates that must be compile-time constants).
template <class F, int... U>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, U...>) {
    (f(std::integral_constant<int, U>{}), ...);
}
template <class F>
__device__ __forceinline__ void static_for16(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, 16>{});
}

// ----------------------------------------------------------------- MFMA fp32 tiles
// acc(16x16) += A(16 x K) * B(K x 16) over k in [k0, k1), k1 - k0 a multiple of 4.
// A(m,k) = A[m*am + k*ak], B(k,n) = B[k*bk + n*bn]; pointers at the tile origin.
__device__ __forceinline__ f32x4 mma16_f32(const float* A, int am, int ak, const float* B, int bk,
                                           int bn, int k0, int k1, f32x4 acc) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    for (int k = k0; k < k1; k += 4) {
        const float a = A[r * am + (k + kq) * ak];
        const float b = B[(k + kq) * bk + r * bn];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

// ----------------------------------------------------------------- chunk addressing
// A chunk is a run of at most kChunk tokens of one sequence.  Dense rows:
// sequence n = row b, chunk i covers tokens [i*64, min(i*64+64, T)) of that
// row.  Packed rows: chunk c is (doc n, i) = chunk_indices[c], covering
// [cu[n] + i*64, min(cu[n] + i*64 + 64, cu[n+1])).  The global token index
// (into the [B*T] token axis) is returned in t0.
struct ChunkRef {
    int n;      // sequence
    int i;      // chunk index within the sequence
    int64_t t0; // first token (global)
    int len;    // tokens in the chunk, 1..64 (0 = no such chunk)
};

struct SeqLayout {
    int B, T, N;
    const int32_t* cu;       // null when dense
    const int32_t* cidx;     // [max,2]
    const int32_t* coff;     // [N+1]
    int nc_dense;            // chunks per row when dense

    __device__ __forceinline__ ChunkRef chunk(int c) const {
        ChunkRef r;
        if (cu == nullptr) {
            r.n = c / nc_dense;
            r.i = c - r.n * nc_dense;
            if (r.n >= B) { r.len = 0; r.t0 = 0; return r; }
            r.t0 = (int64_t)r.n * T + (int64_t)r.i * kChunk;
            const int rem = T - r.i * kChunk;
            r.len = rem < kChunk ? rem : kChunk;
        } else {
            if (c >= coff[N]) { r.n = 0; r.i = 0; r.len = 0; r.t0 = 0; return r; }
            r.n = cidx[2 * c];
            r.i = cidx[2 * c + 1];
            const int s = cu[r.n] + r.i * kChunk;
            const int rem = cu[r.n + 1] - s;
            r.t0 = s;
            r.len = rem < kChunk ? rem : kChunk;
        }
        return r;
    }
    // Range of global chunk ids belonging to sequence n.
    __device__ __forceinline__ void seq_chunks(int n, int& c0, int& c1) const {
        if (cu == nullptr) { c0 = n * nc_dense; c1 = c0 + nc_dense; }
        else { c0 = coff[n]; c1 = coff[n + 1]; }
    }
    // Token range [s0, s0 + len) of sequence n.
    __device__ __forceinline__ void seq_tokens(int n, int64_t& s0, int& len) const {
        if (cu == nullptr) { s0 = (int64_t)n * T; len = T; }
        else { s0 = cu[n]; len = cu[n + 1] - cu[n]; }
    }
    // Chunk i of sequence n whose tokens are [s0, s0 + len): the chunks of a
    // sequence are consecutive and each starts 64 tokens after the previous
    // one, so a sequential pass needs no per-chunk metadata loads.
    __device__ __forceinline__ static ChunkRef chunk_of(int n, int i, int64_t s0, int len) {
        ChunkRef r;
        r.n = n;
        r.i = i;
        r.t0 = s0 + (int64_t)i * kChunk;
        const int rem = len - i * kChunk;
        r.len = rem < kChunk ? rem : kChunk;
        return r;
    }
};

}  // namespace kda
