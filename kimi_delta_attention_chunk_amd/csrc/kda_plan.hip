// kda_plan.hip -- per-document chunk tables for packed rows (integer, exact).
//
// torchtitan PR #4347 ("[kimi k3] Support sample packing in KDA"): document
// offsets make the recurrent state restart at every document, and the
// chunk index tables derived from them should be built once per batch rather
// than in every layer.  Here they are built on the device, without a host
// round trip:
//   chunk_offsets[n] = sum_{m<n} ceil(L_m / C),   L_m = cu[m+1] - cu[m]
//   chunk_indices[chunk_offsets[n] + i] = (n, i),  i < ceil(L_n / C)
// and the rows past the real count are set to (-1, -1).
//
// One workgroup of 1024 threads scans the per-document counts in tiles of
// 1024 documents with a carried prefix.  Every store is bounds-checked against
// max_chunks, so even offsets that break the documented precondition cannot
// write out of range.
#include "kda_device.cuh"
#include "kda_internal.h"

namespace kda {

constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(const int32_t* __restrict__ cu, int N,
                                                            int chunk, int max_chunks,
                                                            int32_t* __restrict__ cidx,
                                                            int32_t* __restrict__ coff) {
    __shared__ int s_scan[kPlanThreads];
    __shared__ int s_carry;
    const int tid = threadIdx.x;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += kPlanThreads) {
        const int n = base + tid;
        int cnt = 0;
        if (n < N) {
            const int L = cu[n + 1] - cu[n];
            cnt = L > 0 ? (L + chunk - 1) / chunk : 0;
        }
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int excl = s_carry + s_scan[tid] - cnt;
        if (n < N) coff[n] = excl;
        for (int i = 0; i < cnt; ++i) {
            const int r = excl + i;
            if (r >= 0 && r < max_chunks) {
                cidx[2 * r] = n;
                cidx[2 * r + 1] = i;
            }
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) s_carry += s_scan[kPlanThreads - 1];
        __syncthreads();
    }
    const int total = s_carry;
    if (tid == 0) coff[N] = total;
    for (int r = (total > 0 ? total : 0) + tid; r < max_chunks; r += kPlanThreads) {
        cidx[2 * r] = -1;
        cidx[2 * r + 1] = -1;
    }
}

hipError_t launch_plan(const int32_t* cu, int N, int T, int chunk, int max_chunks,
                       int32_t* chunk_indices, int32_t* chunk_offsets, hipStream_t s) {
    (void)T;
    KDA_LAUNCH("plan", plan_kernel, dim3(1), dim3(kPlanThreads), s, cu, N, chunk, max_chunks,
               chunk_indices, chunk_offsets);
    return hipSuccess;
}

}  // namespace kda
