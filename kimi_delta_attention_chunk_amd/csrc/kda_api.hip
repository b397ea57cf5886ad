// kda_api.hip -- the extern "C" entry points declared in include/kda.h.
//
// Every call validates its arguments from the descriptor and the pointer
// values alone (no device reads, no synchronisation), then enqueues its
// kernels on the caller's stream.  On an error nothing is launched and the
// thread-local message returned by kda_last_error() says what was wrong.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptr(const void* p, const char* name, bool required) {
    if (p == nullptr) return required ? fail(KDA_ERR_INVALID, "%s must not be null", name) : KDA_OK;
    if (!aligned16(p)) return fail(KDA_ERR_INVALID, "%s is not 16-byte aligned", name);
    return KDA_OK;
}

bool dtype_ok(int d) { return d == KDA_BF16 || d == KDA_FP32; }

const uint32_t kKnownFlags = KDA_F_QK_L2NORM | KDA_F_GATE_IN_KERNEL | KDA_F_BETA_LOGITS | KDA_F_SAVE_FOR_BWD |
                             KDA_F_FWD_SAVED | KDA_F_DH0_ONLY;
const uint32_t kStepFlags = KDA_F_QK_L2NORM | KDA_F_GATE_IN_KERNEL | KDA_F_BETA_LOGITS;

int validate_desc(const kda_desc* d) {
    if (d == nullptr) return fail(KDA_ERR_INVALID, "desc must not be null");
    if (d->B < 1 || d->T < 0 || d->H < 1 || d->N < 1)
        return fail(KDA_ERR_INVALID, "bad sizes B=%d T=%d H=%d N=%d", d->B, d->T, d->H, d->N);
    if (d->dk < 1 || d->dv < 1) return fail(KDA_ERR_INVALID, "bad head dims dk=%d dv=%d", d->dk, d->dv);
    if (!kda::dims_supported(d->dk, d->dv))
        return fail(KDA_ERR_UNSUPPORTED, "head dims (dk=%d, dv=%d) not supported; use (32,64), (64,64) or (128,128)",
                    d->dk, d->dv);
    if (d->chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk=%d not supported (64 only)", d->chunk);
    if (!dtype_ok(d->dtype) || !dtype_ok(d->out_dtype)) return fail(KDA_ERR_INVALID, "bad dtype");
    if (d->flags & ~kKnownFlags) return fail(KDA_ERR_INVALID, "unknown flag bits 0x%x", d->flags & ~kKnownFlags);
    if ((int64_t)d->B * d->T > INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "B*T exceeds 2^31-1 tokens");
    if ((int64_t)d->B * d->T * d->H * (d->dk > d->dv ? d->dk : d->dv) > ((int64_t)1 << 40))
        return fail(KDA_ERR_UNSUPPORTED, "tensor too large");
    return KDA_OK;
}

// Fill the parts of ChunkArgs that come from the descriptor and the varlen tables.
int make_args(const kda_desc* d, const int32_t* cu, const int32_t* cidx, const int32_t* coff,
              kda::ChunkArgs& a) {
    int rc = validate_desc(d);
    if (rc) return rc;
    const bool packed = cu != nullptr || cidx != nullptr || coff != nullptr;
    if (packed) {
        if (!cu || !cidx || !coff)
            return fail(KDA_ERR_INVALID, "packed rows need cu_seqlens, chunk_indices and chunk_offsets together");
        if (d->B != 1) return fail(KDA_ERR_INVALID, "packed rows require B == 1 (got B=%d)", d->B);
        if ((rc = check_ptr(cu, "cu_seqlens", true)) || (rc = check_ptr(cidx, "chunk_indices", true)) ||
            (rc = check_ptr(coff, "chunk_offsets", true)))
            return rc;
    } else if (d->N != d->B) {
        return fail(KDA_ERR_INVALID, "dense rows require N == B (got N=%d, B=%d)", d->N, d->B);
    }
    memset(&a, 0, sizeof a);
    a.B = d->B; a.T = d->T; a.H = d->H; a.dk = d->dk; a.dv = d->dv; a.N = d->N;
    a.in_bf16 = d->dtype == KDA_BF16;
    a.out_bf16 = d->out_dtype == KDA_BF16;
    a.scale = d->scale;
    a.flags = d->flags;
    a.cu = cu; a.cidx = cidx; a.coff = coff;
    if (packed) {
        a.nc_dense = 0;
        a.n_chunks_bound = kda_max_chunks(d->T, d->N, d->chunk);
    } else {
        a.nc_dense = (d->T + d->chunk - 1) / d->chunk;
        a.n_chunks_bound = a.nc_dense * d->B;
    }
    return KDA_OK;
}

// Sizes for the workspace queries: N != B means packed rows (B must be 1);
// a single packed document has the same chunk bound as one dense row.
int ws_args(const kda_desc* d, kda::ChunkArgs& a) {
    int rc = validate_desc(d);
    if (rc) return rc;
    const bool packed = d->N != d->B;
    if (packed && d->B != 1) return fail(KDA_ERR_INVALID, "packed rows require B == 1 (got B=%d)", d->B);
    memset(&a, 0, sizeof a);
    a.B = d->B; a.T = d->T; a.H = d->H; a.dk = d->dk; a.dv = d->dv; a.N = d->N;
    a.nc_dense = (d->T + d->chunk - 1) / d->chunk;
    a.n_chunks_bound = packed ? kda_max_chunks(d->T, d->N, d->chunk) : a.nc_dense * d->B;
    return KDA_OK;
}

int check_common_inputs(const kda_desc* d, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* A_log, const float* dt_bias, const float* h0) {
    int rc;
    const bool tok = d->T > 0;  // with no tokens the per-token arrays may be null
    if ((rc = check_ptr(q, "q", tok)) || (rc = check_ptr(k, "k", tok)) || (rc = check_ptr(v, "v", tok)) ||
        (rc = check_ptr(g, "g", tok)) || (rc = check_ptr(beta, "beta", tok)) || (rc = check_ptr(h0, "h0", false)))
        return rc;
    const bool gate = d->flags & KDA_F_GATE_IN_KERNEL;
    if ((rc = check_ptr(A_log, "A_log", gate)) || (rc = check_ptr(dt_bias, "dt_bias", gate))) return rc;
    return KDA_OK;
}

// Scratch of kda_fwd_noalloc: a file-scope device array, one copy per GPU, held
// until the process ends.  In host code its name is only a stand-in for the
// device symbol, never a device address: the address of each GPU's copy is
// looked up once per device (hipGetSymbolAddress, that device current) and
// only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The scratch address on the device that `stream` runs on, which must be the
// current device (so that the lookup resolves that device's copy).
int scratch_on_stream_device(hipStream_t stream, void** out) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (stream != nullptr) {
        hipDevice_t sd = -1;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sd != cur)
            return fail(KDA_ERR_INVALID, "the stream belongs to device %d but device %d is current; make the "
                                         "stream's device current", (int)sd, cur);
    }
    if (cur < 0 || cur >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "device index %d out of range", cur);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[cur] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", cur, hipGetErrorString(e));
        g_scratch_ptr[cur] = p;
    }
    *out = g_scratch_ptr[cur];
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_str(int s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

const char* kda_last_error(void) { return g_err; }

int32_t kda_max_chunks(int32_t T, int32_t N, int32_t chunk) {
    if (T < 0 || N < 0 || chunk < 1) return -1;
    const int64_t m = ((int64_t)T + (int64_t)N * (chunk - 1)) / chunk;
    return m > INT32_MAX ? -1 : (int32_t)m;
}

int kda_plan_varlen(const int32_t* cu_seqlens, int32_t N, int32_t T, int32_t chunk,
                    int32_t* chunk_indices, int32_t* chunk_offsets, kda_stream_t stream) {
    g_err[0] = 0;
    if (N < 1 || T < 0) return fail(KDA_ERR_INVALID, "bad sizes N=%d T=%d", N, T);
    if (chunk < 1) return fail(KDA_ERR_INVALID, "bad chunk %d", chunk);
    int rc;
    if ((rc = check_ptr(cu_seqlens, "cu_seqlens", true)) || (rc = check_ptr(chunk_offsets, "chunk_offsets", true)))
        return rc;
    const int32_t mc = kda_max_chunks(T, N, chunk);
    if (mc < 0) return fail(KDA_ERR_INVALID, "chunk bound overflows");
    if (mc > 0 && (rc = check_ptr(chunk_indices, "chunk_indices", true))) return rc;
    hipError_t e = kda::launch_plan(cu_seqlens, N, T, chunk, mc, chunk_indices, chunk_offsets, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

int kda_check_cu_seqlens(const int32_t* cu_seqlens, int32_t N, int32_t T, kda_stream_t stream) {
    g_err[0] = 0;
    if (N < 1 || cu_seqlens == nullptr) return fail(KDA_ERR_INVALID, "bad arguments");
    int32_t* host = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
    if (!host) return fail(KDA_ERR_INVALID, "host allocation failed");
    hipError_t e = hipMemcpyAsync(host, cu_seqlens, sizeof(int32_t) * (size_t)(N + 1), hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) { free(host); return fail(KDA_ERR_HIP, "copy: %s", hipGetErrorString(e)); }
    int rc = KDA_OK;
    if (host[0] != 0) rc = fail(KDA_ERR_INVALID, "cu_seqlens[0] = %d, expected 0", host[0]);
    for (int i = 0; rc == KDA_OK && i < N; ++i)
        if (host[i + 1] < host[i]) rc = fail(KDA_ERR_INVALID, "cu_seqlens decreases at %d", i);
    if (rc == KDA_OK && host[N] != T) rc = fail(KDA_ERR_INVALID, "cu_seqlens[N] = %d, expected T = %d", host[N], T);
    free(host);
    return rc;
}

size_t kda_fwd_workspace(const kda_desc* desc) {
    g_err[0] = 0;
    kda::ChunkArgs a;
    if (ws_args(desc, a)) return 0;
    return kda::ws_layout(a, false).total;
}

int kda_debug_ws_layout(const kda_desc* desc, int backward, const char** names, size_t* offsets, size_t* bytes,
                        int cap) {
    g_err[0] = 0;
    kda::ChunkArgs a;
    if (ws_args(desc, a)) return -1;
    struct Out {
        const char** names;
        size_t *offsets, *bytes;
        int cap, n;
    } out{names, offsets, bytes, cap, 0};
    kda::ws_layout(a, backward != 0, [](void* ctx, const char* name, size_t off, size_t nb) {
        Out& o = *(Out*)ctx;
        if (o.n < o.cap) {
            if (o.names) o.names[o.n] = name;
            if (o.offsets) o.offsets[o.n] = off;
            if (o.bytes) o.bytes[o.n] = nb;
        }
        ++o.n;
    }, &out);
    return out.n;
}

size_t kda_bwd_workspace(const kda_desc* desc) {
    g_err[0] = 0;
    kda::ChunkArgs a;
    if (ws_args(desc, a)) return 0;
    return kda::ws_layout(a, true).total;
}

int kda_fwd(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* A_log, const float* dt_bias, const float* h0,
            const int32_t* cu_seqlens, const int32_t* chunk_indices, const int32_t* chunk_offsets,
            void* o, float* hT, void* ws, size_t ws_bytes, kda_stream_t stream) {
    g_err[0] = 0;
    kda::ChunkArgs a;
    int rc = make_args(desc, cu_seqlens, chunk_indices, chunk_offsets, a);
    if (rc) return rc;
    if ((rc = check_common_inputs(desc, q, k, v, g, beta, A_log, dt_bias, h0))) return rc;
    if ((rc = check_ptr(o, "o", desc->T > 0)) || (rc = check_ptr(hT, "hT", false))) return rc;
    if (desc->flags & KDA_F_DH0_ONLY) return fail(KDA_ERR_INVALID, "KDA_F_DH0_ONLY is a backward flag");
    const size_t need = kda::ws_layout(a, (desc->flags & (KDA_F_SAVE_FOR_BWD | KDA_F_FWD_SAVED)) != 0).total;
    if (ws == nullptr || ws_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(KDA_ERR_INVALID, "ws is not 16-byte aligned");
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.A_log = A_log; a.dt_bias = dt_bias; a.h0 = h0;
    a.o = o; a.hT = hT; a.ws = ws; a.ws_bytes = ws_bytes;
    hipError_t e = kda::launch_fwd(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

// ---------------------------------------------------------------- allocation-free forward
int kda_fwd_noalloc(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, const float* A_log, const float* dt_bias, const float* h0,
                    const int32_t* cu_seqlens, const int32_t* chunk_indices, const int32_t* chunk_offsets,
                    void* o, float* hT, kda_stream_t stream) {
    g_err[0] = 0;
    if (desc != nullptr && (desc->flags & (KDA_F_SAVE_FOR_BWD | KDA_F_FWD_SAVED | KDA_F_DH0_ONLY)))
        return fail(KDA_ERR_INVALID, "kda_fwd_noalloc takes no save/saved/dh0 flag: its scratch does not "
                                     "outlive the call");
    kda::ChunkArgs a;
    int rc = make_args(desc, cu_seqlens, chunk_indices, chunk_offsets, a);
    if (rc) return rc;
    if ((rc = check_common_inputs(desc, q, k, v, g, beta, A_log, dt_bias, h0))) return rc;
    if ((rc = check_ptr(o, "o", desc->T > 0)) || (rc = check_ptr(hT, "hT", false))) return rc;
    const size_t need = kda::ws_layout(a, false).total;
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
        return fail(KDA_ERR_UNSUPPORTED,
                    "kda_fwd_noalloc: this problem needs %zu bytes of scratch, more than its fixed %zu "
                    "(use kda_fwd with a workspace)", need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((rc = scratch_on_stream_device((hipStream_t)stream, &ws))) return rc;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.A_log = A_log; a.dt_bias = dt_bias; a.h0 = h0;
    a.o = o; a.hT = hT; a.ws = ws; a.ws_bytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
    hipError_t e = kda::launch_fwd(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

int kda_bwd(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* A_log, const float* dt_bias, const float* h0,
            const int32_t* cu_seqlens, const int32_t* chunk_indices, const int32_t* chunk_offsets,
            const void* d_o, const float* dhT, void* dq, void* dk, void* dv, float* dg, float* dbeta,
            float* dh0, float* dA_log, float* ddt_bias, void* ws, size_t ws_bytes, kda_stream_t stream) {
    g_err[0] = 0;
    kda::ChunkArgs a;
    int rc = make_args(desc, cu_seqlens, chunk_indices, chunk_offsets, a);
    if (rc) return rc;
    if ((rc = check_common_inputs(desc, q, k, v, g, beta, A_log, dt_bias, h0))) return rc;
    if (desc->flags & KDA_F_SAVE_FOR_BWD) return fail(KDA_ERR_INVALID, "KDA_F_SAVE_FOR_BWD is a forward flag");
    // with KDA_F_DH0_ONLY only dh0 is produced: the per-token gradients may be null
    const bool only = desc->flags & KDA_F_DH0_ONLY;
    const bool gate = (desc->flags & KDA_F_GATE_IN_KERNEL) && !only;
    const bool tok = desc->T > 0, grads = tok && !only;  // with no tokens the per-token arrays may be null
    if ((rc = check_ptr(d_o, "d_o", tok)) || (rc = check_ptr(dhT, "dhT", false)) ||
        (rc = check_ptr(dq, "dq", grads)) || (rc = check_ptr(dk, "dk", grads)) || (rc = check_ptr(dv, "dv", grads)) ||
        (rc = check_ptr(dg, "dg", grads)) || (rc = check_ptr(dbeta, "dbeta", grads)) ||
        (rc = check_ptr(dh0, "dh0", only)) || (rc = check_ptr(dA_log, "dA_log", gate)) ||
        (rc = check_ptr(ddt_bias, "ddt_bias", gate)))
        return rc;
    const size_t need = kda::ws_layout(a, true).total;
    if (ws == nullptr || ws_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(KDA_ERR_INVALID, "ws is not 16-byte aligned");
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.A_log = A_log; a.dt_bias = dt_bias; a.h0 = h0;
    a.d_o = d_o; a.dhT = dhT; a.dq = dq; a.dk_ = dk; a.dv_ = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.dA_log = dA_log; a.ddt_bias = ddt_bias; a.ws = ws; a.ws_bytes = ws_bytes;
    hipError_t e = kda::launch_bwd(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

int kda_step(int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype dtype, kda_dtype out_dtype, float scale,
             uint32_t flags, const void* q, const void* k, const void* v, const float* g, const float* beta,
             const float* A_log, const float* dt_bias, float* h, void* o, kda_stream_t stream) {
    g_err[0] = 0;
    if (B < 1 || H < 1) return fail(KDA_ERR_INVALID, "bad sizes B=%d H=%d", B, H);
    if ((int64_t)B * H > INT32_MAX / 2) return fail(KDA_ERR_UNSUPPORTED, "B*H too large");
    if (!kda::dims_supported(dk, dv))
        return fail(KDA_ERR_UNSUPPORTED, "head dims (dk=%d, dv=%d) not supported", dk, dv);
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return fail(KDA_ERR_INVALID, "bad dtype");
    if (flags & ~kStepFlags) return fail(KDA_ERR_INVALID, "unknown flag bits");
    int rc;
    const bool gate = flags & KDA_F_GATE_IN_KERNEL;
    if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k, "k", true)) || (rc = check_ptr(v, "v", true)) ||
        (rc = check_ptr(g, "g", true)) || (rc = check_ptr(beta, "beta", true)) || (rc = check_ptr(h, "h", true)) ||
        (rc = check_ptr(o, "o", true)) || (rc = check_ptr(A_log, "A_log", gate)) ||
        (rc = check_ptr(dt_bias, "dt_bias", gate)))
        return rc;
    kda::StepArgs a;
    a.B = B; a.H = H; a.dk = dk; a.dv = dv;
    a.in_bf16 = dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.scale = scale; a.flags = flags;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.A_log = A_log; a.dt_bias = dt_bias; a.h = h; a.o = o;
    hipError_t e = kda::launch_step(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "step launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

// ---------------------------------------------------------------- context parallelism (dk = 32)
int kda_segment_maps(const kda_desc* desc, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                     const int32_t* chunk_indices, const int32_t* chunk_offsets, float* M, void* ws, size_t ws_bytes,
                     kda_stream_t stream) {
    g_err[0] = 0;
    kda::ChunkArgs a;
    int rc = make_args(desc, cu_seqlens, chunk_indices, chunk_offsets, a);
    if (rc) return rc;
    if (desc->flags & (KDA_F_SAVE_FOR_BWD | KDA_F_DH0_ONLY)) return fail(KDA_ERR_INVALID, "flag does not apply");
    if ((rc = check_common_inputs(desc, q, k, v, g, beta, A_log, dt_bias, nullptr))) return rc;
    if ((rc = check_ptr(M, "M", true))) return rc;
    const size_t need = kda::ws_layout(a, false).total;
    if (ws == nullptr || ws_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(KDA_ERR_INVALID, "ws is not 16-byte aligned");
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.A_log = A_log; a.dt_bias = dt_bias;
    a.ws = ws; a.ws_bytes = ws_bytes;
    hipError_t e = kda::launch_segment_maps(a, M, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "segment maps launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

int kda_state_scan(int32_t R, int32_t H, int32_t dk, int32_t dv, int32_t transpose, const float* M, const float* c,
                   const float* x0, float* x_in, float* x_out, kda_stream_t stream) {
    g_err[0] = 0;
    if (R < 1 || H < 1) return fail(KDA_ERR_INVALID, "bad sizes R=%d H=%d", R, H);
    if (!((dk == 32 && dv == 64) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128)))
        return fail(KDA_ERR_UNSUPPORTED, "state scan needs (dk, dv) in (32, 64), (64, 64), (128, 128) (got %d, %d)", dk, dv);
    if (transpose != 0 && transpose != 1) return fail(KDA_ERR_INVALID, "transpose must be 0 or 1");
    int rc;
    if ((rc = check_ptr(M, "M", true)) || (rc = check_ptr(c, "c", true)) || (rc = check_ptr(x0, "x0", false)) ||
        (rc = check_ptr(x_in, "x_in", true)) || (rc = check_ptr(x_out, "x_out", false)))
        return rc;
    hipError_t e = kda::launch_state_scan(R, H, dk, dv, transpose != 0, M, c, x0, x_in, x_out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "state scan launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

// ---------------------------------------------------------------- short convolution
static int conv_check(int32_t B, int32_t T, int32_t D, int32_t W, int dtype, int out_dtype, uint32_t flags,
                      const int32_t* cu, int32_t N) {
    if (B < 1 || T < 0 || D < 8 || D % 8 != 0)
        return fail(KDA_ERR_INVALID, "bad sizes B=%d T=%d D=%d (D a positive multiple of 8)", B, T, D);
    if (W < 1 || W > 4) return fail(KDA_ERR_UNSUPPORTED, "kernel width W=%d not supported (1..4)", W);
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return fail(KDA_ERR_INVALID, "bad dtype");
    if (flags & ~(uint32_t)KDA_CONV_SILU) return fail(KDA_ERR_INVALID, "unknown flag bits 0x%x", flags);
    if ((int64_t)B * T * D > ((int64_t)1 << 40)) return fail(KDA_ERR_UNSUPPORTED, "tensor too large");
    if (cu) {
        if (B != 1) return fail(KDA_ERR_INVALID, "document offsets require B == 1 (got B=%d)", B);
        if (N < 1) return fail(KDA_ERR_INVALID, "document offsets need N >= 1 (got N=%d)", N);
        int rc = check_ptr(cu, "cu_seqlens", true);
        if (rc) return rc;
    }
    return KDA_OK;
}

static kda::ConvArgs conv_args(int32_t B, int32_t T, int32_t D, int32_t W, int dtype, int out_dtype, uint32_t flags,
                               const void* x, const float* w, const float* bias, const int32_t* cu, int32_t N) {
    kda::ConvArgs a;
    memset(&a, 0, sizeof a);
    a.B = B; a.T = T; a.D = D; a.W = W; a.N = cu ? N : 1;
    a.in_bf16 = dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16; a.silu = flags & KDA_CONV_SILU;
    a.cu = cu; a.x = x; a.w = w; a.bias = bias;
    return a;
}

int kda_conv_fwd(int32_t B, int32_t T, int32_t D, int32_t W, kda_dtype dtype, kda_dtype out_dtype, uint32_t flags,
                 const void* x, const float* w, const float* bias, const int32_t* cu_seqlens, int32_t N, void* y,
                 kda_stream_t stream) {
    g_err[0] = 0;
    int rc = conv_check(B, T, D, W, dtype, out_dtype, flags, cu_seqlens, N);
    if (rc) return rc;
    const bool tok = T > 0;  // with no tokens x and y may be null
    if ((rc = check_ptr(x, "x", tok)) || (rc = check_ptr(w, "w", true)) || (rc = check_ptr(bias, "bias", false)) ||
        (rc = check_ptr(y, "y", tok)))
        return rc;
    kda::ConvArgs a = conv_args(B, T, D, W, dtype, out_dtype, flags, x, w, bias, cu_seqlens, N);
    a.y = y;
    hipError_t e = kda::launch_conv(a, false, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "conv_fwd launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

size_t kda_conv_bwd_workspace(int32_t B, int32_t T, int32_t D, int32_t W) {
    if (B < 1 || T < 0 || D < 8 || D % 8 != 0 || W < 1 || W > 4) return 0;
    const size_t n = kda::conv_bwd_workspace(B, T, D);
    return n ? n : 256;
}

int kda_conv_bwd(int32_t B, int32_t T, int32_t D, int32_t W, kda_dtype dtype, kda_dtype out_dtype, uint32_t flags,
                 const void* x, const float* w, const float* bias, const int32_t* cu_seqlens, int32_t N,
                 const void* dy, void* dx, float* dw, float* dbias, void* ws, size_t ws_bytes, kda_stream_t stream) {
    g_err[0] = 0;
    int rc = conv_check(B, T, D, W, dtype, out_dtype, flags, cu_seqlens, N);
    if (rc) return rc;
    const bool tok = T > 0;  // with no tokens x, dy and dx may be null
    if ((rc = check_ptr(x, "x", tok)) || (rc = check_ptr(w, "w", true)) || (rc = check_ptr(bias, "bias", false)) ||
        (rc = check_ptr(dy, "dy", tok)) || (rc = check_ptr(dx, "dx", tok)) || (rc = check_ptr(dw, "dw", true)) ||
        (rc = check_ptr(dbias, "dbias", false)) || (rc = check_ptr(ws, "ws", true)))
        return rc;
    const size_t need = kda_conv_bwd_workspace(B, T, D, W);
    if (ws_bytes < need) return fail(KDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    kda::ConvArgs a = conv_args(B, T, D, W, dtype, out_dtype, flags, x, w, bias, cu_seqlens, N);
    a.dy = dy; a.dx = dx; a.dw = dw; a.dbias = dbias; a.part = (float*)ws;
    hipError_t e = kda::launch_conv(a, true, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "conv_bwd launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

// ---------------------------------------------------------------- gated norm
static int gnorm_check(int64_t rows, int32_t dv, int dtype, int out_dtype, float eps) {
    if (rows < 0) return fail(KDA_ERR_INVALID, "rows=%lld must be >= 0", (long long)rows);
    if (dv != 32 && dv != 64 && dv != 128) return fail(KDA_ERR_UNSUPPORTED, "dv=%d not supported (32, 64, 128)", dv);
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return fail(KDA_ERR_INVALID, "bad dtype");
    if (!(eps > 0.f)) return fail(KDA_ERR_INVALID, "eps must be positive");
    if (rows > ((int64_t)1 << 34)) return fail(KDA_ERR_UNSUPPORTED, "too many rows");
    return KDA_OK;
}

int kda_gnorm_fwd(int64_t rows, int32_t dv, kda_dtype dtype, kda_dtype out_dtype, float eps, const void* o,
                  const void* gate, const float* weight, void* y, kda_stream_t stream) {
    g_err[0] = 0;
    int rc = gnorm_check(rows, dv, dtype, out_dtype, eps);
    if (rc) return rc;
    const bool any = rows > 0;  // with no rows the row arrays may be null
    if ((rc = check_ptr(o, "o", any)) || (rc = check_ptr(gate, "gate", any)) ||
        (rc = check_ptr(weight, "weight", true)) || (rc = check_ptr(y, "y", any)))
        return rc;
    kda::GnormArgs a;
    memset(&a, 0, sizeof a);
    a.rows = rows; a.dv = dv; a.in_bf16 = dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16; a.eps = eps;
    a.o = o; a.gate = gate; a.weight = weight; a.y = y;
    hipError_t e = kda::launch_gnorm(a, false, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "gnorm_fwd launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

size_t kda_gnorm_bwd_workspace(int64_t rows, int32_t dv) {
    if (rows < 0 || (dv != 32 && dv != 64 && dv != 128)) return 0;
    const size_t n = kda::gnorm_bwd_workspace(rows, dv);
    return n ? n : 256;
}

int kda_gnorm_bwd(int64_t rows, int32_t dv, kda_dtype dtype, kda_dtype out_dtype, float eps, const void* o,
                  const void* gate, const float* weight, const void* dy, void* d_o, void* dgate, float* dweight,
                  void* ws, size_t ws_bytes, kda_stream_t stream) {
    g_err[0] = 0;
    int rc = gnorm_check(rows, dv, dtype, out_dtype, eps);
    if (rc) return rc;
    const bool any = rows > 0;  // with no rows the row arrays may be null
    if ((rc = check_ptr(o, "o", any)) || (rc = check_ptr(gate, "gate", any)) ||
        (rc = check_ptr(weight, "weight", true)) || (rc = check_ptr(dy, "dy", any)) ||
        (rc = check_ptr(d_o, "d_o", any)) || (rc = check_ptr(dgate, "dgate", any)) ||
        (rc = check_ptr(dweight, "dweight", true)) || (rc = check_ptr(ws, "ws", true)))
        return rc;
    const size_t need = kda_gnorm_bwd_workspace(rows, dv);
    if (ws_bytes < need) return fail(KDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    kda::GnormArgs a;
    memset(&a, 0, sizeof a);
    a.rows = rows; a.dv = dv; a.in_bf16 = dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16; a.eps = eps;
    a.o = o; a.gate = gate; a.weight = weight; a.dy = dy; a.d_o = d_o; a.dgate = dgate; a.dweight = dweight;
    a.part = (float*)ws;
    hipError_t e = kda::launch_gnorm(a, true, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "gnorm_bwd launch: %s", hipGetErrorString(e));
    return KDA_OK;
}

}  // extern "C"
