// kda_internal.h -- host-side launch interface between the C ABI (kda_api.hip)
// and the kernel files.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct StepArgs {
    int B, H, dk, dv;
    bool in_bf16, out_bf16;
    float scale;
    uint32_t flags;
    const void *q, *k, *v;
    const float *g, *beta, *A_log, *dt_bias;
    float* h;
    void* o;
};
hipError_t launch_step(const StepArgs& a, hipStream_t s);

// Short causal depthwise convolution over [B, T, D] rows (kda_ops.hip).
struct ConvArgs {
    int B, T, D, W, N;
    bool in_bf16, out_bf16, silu;
    const int32_t* cu;  // document offsets [N + 1] (B == 1), or null
    const void* x;
    const float *w, *bias;
    void* y;
    const void* dy;
    void* dx;
    float *dw, *dbias;
    float* part;  // workspace: per row-block partial sums of dw and dbias
};
hipError_t launch_conv(const ConvArgs& a, bool backward, hipStream_t s);
size_t conv_bwd_workspace(int B, int T, int D);

// Context parallelism (kda_cp.hip): the chain of segment maps, x <- M_r x + c_r
// over the segments (M_r^T, segments in reverse, with `transpose`).
hipError_t launch_state_scan(int R, int H, int dk, int dv, bool transpose, const float* M, const float* c,
                             const float* x0, float* out, float* xfinal, hipStream_t s);

// Gated RMS norm over rows of dv values (kda_ops.hip).
struct GnormArgs {
    int64_t rows;
    int dv;
    bool in_bf16, out_bf16;
    float eps;
    const void *o, *gate;
    const float* weight;
    void* y;
    const void* dy;
    void *d_o, *dgate;
    float* dweight;
    float* part;  // workspace: per workgroup partial sums of dweight
};
hipError_t launch_gnorm(const GnormArgs& a, bool backward, hipStream_t s);
size_t gnorm_bwd_workspace(int64_t rows, int dv);

hipError_t launch_plan(const int32_t* cu, int N, int T, int chunk, int max_chunks,
                       int32_t* chunk_indices, int32_t* chunk_offsets, hipStream_t s);

// Everything a chunked forward/backward launch needs.
struct ChunkArgs {
    int B, T, H, dk, dv, N;
    bool in_bf16, out_bf16;
    float scale;
    uint32_t flags;
    int n_chunks_bound;  // grid size over chunks (exact when dense)
    int nc_dense;        // chunks per row when dense
    const int32_t *cu, *cidx, *coff;
    const void *q, *k, *v;
    const float *g, *beta, *A_log, *dt_bias, *h0;
    // forward outputs
    void* o;
    float* hT;
    // backward inputs / outputs
    const void* d_o;
    const float* dhT;
    void *dq, *dk_, *dv_;
    float *dg, *dbeta, *dh0, *dA_log, *ddt_bias;
    // workspace
    void* ws;
    size_t ws_bytes;
};

// Workspace layout shared by the forward and backward launches.
// Byte offsets of the per-chunk fp32 arrays inside the caller's workspace;
// every array is indexed by slot = chunk * H + head.  The backward-only
// arrays are 0 (absent) in a forward layout.
struct WsLayout {
    size_t w, u, aqk, tm, hs, vn;                    // forward recompute
    size_t qg, khT, gl;                              // per-chunk operands of the scan
    size_t qgT, khb, wT;                             // transposed operands of the reverse scan (dk >= 64)
    size_t gcs;                                      // in-chunk cumulative log-decay (dk >= 64 backward)
    size_t dhs, dvn;                                 // backward state pass
    size_t dqt, dkh, dwv, daq, dtv, dgl, dbv;        // dv-side intermediates
    size_t dkt, dxq, dxk, part_a, part_dt;           // dk-side intermediates
    size_t pm, pmT, hh, qh, qhT, ol, aqT;            // affine chunk form (dk = 32)
    size_t total;
};
// `rec`, if set, is told the name, byte offset and byte size of every array the
// layout holds, in order (the introspection call kda_debug_ws_layout uses it).
typedef void (*WsRecord)(void* ctx, const char* name, size_t offset, size_t bytes);
WsLayout ws_layout(const ChunkArgs& a, bool backward, WsRecord rec = nullptr, void* ctx = nullptr);

bool dims_supported(int dk, int dv);
hipError_t launch_segmaps_wide(const ChunkArgs& a, float* M, hipStream_t s);  // dk = dv >= 64
hipError_t launch_fwd(const ChunkArgs& a, hipStream_t s);

// Opt-in per-kernel timing (kda_timing.hip): a pair of hipEvents around a launch.
void prof_begin(hipStream_t s);
void prof_end(hipStream_t s, const char* name);
// Launches `kernel` and returns its launch error from the enclosing function
// (which must return hipError_t); the error is read before the timing event
// is recorded so that event calls cannot mask it.
#define KDA_LAUNCH(name, kernel, grid, block, stream, ...)                     \
    do {                                                                       \
        ::kda::prof_begin(stream);                                             \
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);       \
        const hipError_t kda_launch_err_ = hipGetLastError();                  \
        ::kda::prof_end(stream, name);                                         \
        if (kda_launch_err_ != hipSuccess) return kda_launch_err_;             \
    } while (0)
hipError_t launch_bwd(const ChunkArgs& a, hipStream_t s);
// The transition matrix of every sequence of a call, dk = 32 (kda_cp.hip; runs
// the intra-chunk kernel into the forward workspace first).
hipError_t launch_segment_maps(const ChunkArgs& a, float* M, hipStream_t s);

}  // namespace kda
