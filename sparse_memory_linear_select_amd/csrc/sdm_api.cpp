// C ABI of libsdm: argument validation, workspace layout, stream-ordered
// launches.  Every check happens before the first HIP call, so invalid
// arguments never enqueue work.  See include/sdm.h for the contract.
#include "sdm.h"

#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <new>
#include <string>

#include "sdm_internal.h"

// Scratch of sdm_forward_noalloc: the workspace of one forward call, in a
// static device array (each GPU the library runs on holds its own copy
// until the process ends).  Host code never uses the name `scratch` as an
// address: it looks up each device's address once (scratch_on) and passes
// that to the kernels.
static __device__ __align__(256) unsigned char scratch[SDM_NOALLOC_MAX_BYTES];

struct sdm_ctx {
    const float *M0 = nullptr;
    int H = 0, sqrtN = 0, d_v = 0, W = 0, R = 0;
    sdm::StateFmt state;  // element type of M (and the E4M3 scale)
};

namespace {

thread_local std::string g_err;

sdm_status fail(sdm_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

sdm_status hip_fail(hipError_t e, const char *what)
{
    return fail(SDM_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

sdm::Shape shape_of(const sdm_ctx *h, int B, int64_t T)
{
    sdm::Shape s;
    s.B = B;
    s.T = T;
    s.H = h->H;
    s.sqrtN = h->sqrtN;
    s.d_v = h->d_v;
    s.W = h->W;
    s.R = h->R;
    return s;
}

sdm_status check_handle_call(const sdm_ctx *h, int B, int64_t T, sdm_dtype dtype)
{
    if (!h) return fail(SDM_ERR_ARG, "null handle");
    if (B < 1) return fail(SDM_ERR_ARG, "B must be >= 1 (got %d)", B);
    if (T < 1) return fail(SDM_ERR_ARG, "T must be >= 1 (got %lld)", (long long)T);
    if (dtype != SDM_F32 && dtype != SDM_BF16)
        return fail(SDM_ERR_ARG, "dtype must be SDM_F32 or SDM_BF16 (got %d)", (int)dtype);
    const double ht = (double)B * (double)T * (double)h->H;
    if (ht >= 2147483648.0) return fail(SDM_ERR_UNSUPPORTED, "B*T*H must be < 2^31");
    return SDM_OK;
}

// Workspace: token records for every (chain, token); the time-parallel
// schedule adds its sorted events, segments and read links after them.
size_t records_bytes(const sdm_ctx *h, int B, int64_t T)
{
    const sdm::RecLayout L(h->W, h->R);
    return round_up((size_t)B * h->H * (size_t)T * (size_t)L.dwords() * 4u);
}

// AUTO: the time-parallel schedule whenever it applies.  Its parallelism does
// not depend on the number of chains, and it merges repeated writes to a slot
// within an epoch.  Measured write+read on MI355X (time-parallel vs
// token-serial): 32 chains x 512 columns 7.8 ms vs 12.2, 8 x 1024 15.9 vs 43.3,
// 32 x 1024 31.8 vs 41.4, 1 x 2048 (2^20 tokens) 269 vs 1676.  The token-serial
// schedule remains for d_v % 4 != 0 (one column per lane) and on request.
sdm_variant resolve_variant(const sdm_ctx *h, int B, int64_t T, sdm_variant v)
{
    if (v != SDM_VARIANT_AUTO) return v;
    return sdm::tp_supported(shape_of(h, B, T)) ? SDM_VARIANT_TIMEPAR : SDM_VARIANT_SERIAL;
}

size_t ws_bytes_for(const sdm_ctx *h, int B, int64_t T, sdm_variant var)
{
    size_t n = records_bytes(h, B, T);
    if (var == SDM_VARIANT_TIMEPAR)
        n += round_up(sdm::tp_workspace_bytes(shape_of(h, B, T), h->state.type != sdm::kStateF32));
    return n;
}

sdm_status check_variant(const sdm_ctx *h, int B, int64_t T, sdm_variant variant,
                         sdm_variant *out)
{
    const sdm_variant var = resolve_variant(h, B, T, variant);
    if (var != SDM_VARIANT_SERIAL && var != SDM_VARIANT_TIMEPAR)
        return fail(SDM_ERR_ARG, "unknown variant %d", (int)variant);
    if (h->state.type != sdm::kStateF32 && var == SDM_VARIANT_SERIAL)
        return fail(SDM_ERR_UNSUPPORTED,
                    "a bfloat16 or E4M3 state needs the time-parallel schedule (d_v %% 4 == 0)");
    if (var == SDM_VARIANT_TIMEPAR && !sdm::tp_supported(shape_of(h, B, T)))
        return fail(SDM_ERR_UNSUPPORTED,
                    "time-parallel schedule needs d_v %% 4 == 0 and N*d_v*4 <= 2^31");
    *out = var;
    return SDM_OK;
}

sdm_status check_variant_and_ws(const sdm_ctx *h, int B, int64_t T, sdm_variant variant,
                                size_t ws_bytes, sdm_variant *out)
{
    sdm_status st = check_variant(h, B, T, variant, out);
    if (st != SDM_OK) return st;
    const size_t need = ws_bytes_for(h, B, T, *out);
    if (ws_bytes < need)
        return fail(SDM_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    return SDM_OK;
}

// Backward workspace with the sequence run in `chunks` chunks (0: the count
// that needs the least memory).
size_t bwd_ws_bytes(const sdm_ctx *h, int B, int64_t T, int chunks)
{
    const sdm::Shape s = shape_of(h, B, T);
    return records_bytes(h, B, T) + round_up(sdm::tp_workspace_bytes(s)) +
           round_up(sdm::tp_backward_workspace_bytes(s, chunks));
}

// The fewest chunks whose workspace fits in ws_bytes (0 if none does).
int bwd_chunks_for(const sdm_ctx *h, int B, int64_t T, size_t ws_bytes)
{
    const sdm::Shape s = shape_of(h, B, T);
    const int nep = sdm::tp_backward_epochs(s);
    const int cmin = sdm::tp_backward_min_chunks(s);
    for (int c = 1; c <= nep; c++)
        if (bwd_ws_bytes(h, B, T, c) <= ws_bytes) return c;
    return bwd_ws_bytes(h, B, T, cmin) <= ws_bytes ? cmin : 0;
}

sdm_status check_backward(const sdm_ctx *h, int B, int64_t T)
{
    if (h->state.type != sdm::kStateF32)
        return fail(SDM_ERR_UNSUPPORTED, "the backward needs a float32 state");
    if (!sdm::tp_supported(shape_of(h, B, T)))
        return fail(SDM_ERR_UNSUPPORTED,
                    "the backward runs on the time-parallel schedule: d_v %% 4 == 0 and "
                    "N*d_v*4 <= 2^31");
    return SDM_OK;
}

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

sdm_status scratch_on(hipStream_t stream, void **out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SDM_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "current device");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "set device");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_fail(e, "address of the static scratch");
        if (!p) return fail(SDM_ERR_HIP, "address of the static scratch: null");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SDM_OK;
}

}  // namespace

extern "C" {

const char *sdm_status_string(sdm_status s)
{
    switch (s) {
        case SDM_OK: return "ok";
        case SDM_ERR_ARG: return "invalid argument";
        case SDM_ERR_UNSUPPORTED: return "unsupported shape or option";
        case SDM_ERR_WORKSPACE: return "workspace too small";
        case SDM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *sdm_last_error(void) { return g_err.c_str(); }

sdm_status sdm_create_ex(const float *M0, int H, int sqrtN, int d_v, int W, int R,
                         sdm_dtype state_dtype, sdm_handle *out)
{
    if (!out) return fail(SDM_ERR_ARG, "null output handle pointer");
    *out = nullptr;
    if (!M0) return fail(SDM_ERR_ARG, "null M0");
    if (!aligned16(M0)) return fail(SDM_ERR_ARG, "M0 must be 16-byte aligned");
    if (H < 1 || sqrtN < 1 || d_v < 1 || W < 1 || R < 1)
        return fail(SDM_ERR_ARG, "H, sqrtN, d_v, W, R must be >= 1 (got %d %d %d %d %d)", H,
                    sqrtN, d_v, W, R);
    if (W > sqrtN || R > sqrtN)
        return fail(SDM_ERR_ARG, "W and R must not exceed sqrtN (got W=%d R=%d sqrtN=%d)", W, R,
                    sqrtN);
    if (sqrtN > sdm::kMaxSqrtN)
        return fail(SDM_ERR_UNSUPPORTED, "sqrtN > %d is not supported", sdm::kMaxSqrtN);
    if (W > sdm::kMaxK || R > sdm::kMaxK)
        return fail(SDM_ERR_UNSUPPORTED, "W, R > %d are not supported", sdm::kMaxK);
    if (state_dtype == SDM_FP8_E4M3)
        return fail(SDM_ERR_ARG, "an E4M3 state takes a scale: create it with sdm_create_fp8");
    if (state_dtype != SDM_F32 && state_dtype != SDM_BF16)
        return fail(SDM_ERR_ARG, "state dtype must be SDM_F32 or SDM_BF16 (got %d)",
                    (int)state_dtype);
    sdm_ctx *h = new (std::nothrow) sdm_ctx;
    if (!h) return fail(SDM_ERR_ARG, "out of host memory");
    h->M0 = M0;
    h->H = H;
    h->sqrtN = sqrtN;
    h->d_v = d_v;
    h->W = W;
    h->R = R;
    h->state.type = state_dtype == SDM_BF16 ? sdm::kStateBF16 : sdm::kStateF32;
    *out = h;
    return SDM_OK;
}

sdm_status sdm_create(const float *M0, int H, int sqrtN, int d_v, int W, int R, sdm_handle *out)
{
    return sdm_create_ex(M0, H, sqrtN, d_v, W, R, SDM_F32, out);
}

sdm_status sdm_create_fp8(const float *M0, int H, int sqrtN, int d_v, int W, int R,
                          int scale_log2, sdm_handle *out)
{
    if (out) *out = nullptr;
    if (scale_log2 < -64 || scale_log2 > 64)
        return fail(SDM_ERR_ARG, "scale_log2 must be in [-64, 64] (got %d)", scale_log2);
    sdm_status st = sdm_create_ex(M0, H, sqrtN, d_v, W, R, SDM_F32, out);
    if (st != SDM_OK) return st;
    (*out)->state.type = sdm::kStateFP8;
    (*out)->state.scale_log2 = scale_log2;
    return SDM_OK;
}

sdm_status sdm_destroy(sdm_handle h)
{
    delete h;
    return SDM_OK;
}

sdm_status sdm_workspace_size(sdm_handle h, int B, int64_t T, sdm_dtype dtype,
                              sdm_variant variant, size_t *bytes)
{
    if (!bytes) return fail(SDM_ERR_ARG, "null bytes pointer");
    *bytes = 0;
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    sdm_variant v;
    st = check_variant(h, B, T, variant, &v);
    if (st != SDM_OK) return st;
    *bytes = ws_bytes_for(h, B, T, v);
    return SDM_OK;
}

sdm_status sdm_select(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                      sdm_dtype dtype, int32_t *Iw, float *kw, int32_t *Ir, float *qw,
                      void *stream)
{
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!kp || !qp || !Iw || !kw || !Ir || !qw) return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(kp) || !aligned16(qp) || !aligned16(Iw) || !aligned16(kw) || !aligned16(Ir) ||
        !aligned16(qw))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    const sdm::Shape s = shape_of(h, B, T);
    hipError_t e = sdm::launch_select(s, kp, qp, dtype == SDM_BF16, Iw, kw, Ir, qw, nullptr,
                                      nullptr, nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    return SDM_OK;
}

sdm_status sdm_write_histogram(sdm_handle h, int B, int64_t T, const void *kp, sdm_dtype dtype,
                               uint32_t *counts, void *stream)
{
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!kp || !counts) return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(kp) || !aligned16(counts))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    const sdm::Shape s = shape_of(h, B, T);
    hipError_t e = sdm::launch_select(s, kp, kp, dtype == SDM_BF16, nullptr, nullptr, nullptr,
                                      nullptr, nullptr, nullptr, nullptr, (hipStream_t)stream,
                                      counts);
    if (e != hipSuccess) return hip_fail(e, "histogram launch");
    return SDM_OK;
}

sdm_status sdm_prepare(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                       const float *alpha, const float *beta, sdm_dtype dtype,
                       sdm_variant variant, unsigned flags, void *workspace, size_t ws_bytes,
                       void *M, void *stream)
{
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!kp || !qp || !alpha || !beta || !M || !workspace)
        return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(kp) || !aligned16(qp) || !aligned16(alpha) || !aligned16(beta) ||
        !aligned16(M) || !aligned16(workspace))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    if (flags & ~SDM_FLAG_CONTINUE) return fail(SDM_ERR_ARG, "unknown flags 0x%x", flags);
    sdm_variant var;
    st = check_variant_and_ws(h, B, T, variant, ws_bytes, &var);
    if (st != SDM_OK) return st;

    const sdm::Shape s = shape_of(h, B, T);
    const hipStream_t hs = (hipStream_t)stream;
    uint32_t *rec = static_cast<uint32_t *>(workspace);
    hipError_t e;
    // M <- M_0, inside the selection launch where its items cover M_0 (the
    // copy then runs under the selection's arithmetic), else on its own
    const bool init = !(flags & SDM_FLAG_CONTINUE);
    const bool fused_init =
        init && h->state.type != sdm::kStateFP8 && sdm::select_can_init(s);
    if (init && !fused_init) {
        e = sdm::launch_init(s, h->M0, M, h->state, hs);
        if (e != hipSuccess) return hip_fail(e, "init launch");
    }
    const sdm::SelInit si{h->M0, M, h->state.type == sdm::kStateBF16};
    e = sdm::launch_select(s, kp, qp, dtype == SDM_BF16, nullptr, nullptr, nullptr, nullptr, rec,
                           alpha, beta, hs, nullptr, 0, -1, fused_init ? &si : nullptr);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    if (var == SDM_VARIANT_TIMEPAR) {
        if (!sdm::decode_supported(s)) {  // one token: nothing to sort (see sdm_apply)
            char *tp = static_cast<char *>(workspace) + records_bytes(h, B, T);
            e = sdm::launch_tp_prepare(s, rec, tp, hs, 0, -1, true,
                                       h->state.type != sdm::kStateF32);
            if (e != hipSuccess) return hip_fail(e, "time-parallel sort launch");
        }
    } else if (sdm::rw_serial_supported(s)) {
        e = sdm::launch_plan(s, rec, sdm::rw_serial_depth(s), hs);
        if (e != hipSuccess) return hip_fail(e, "plan launch");
    }
    return SDM_OK;
}

sdm_status sdm_apply(sdm_handle h, int B, int64_t T, const void *v, sdm_dtype dtype,
                     sdm_variant variant, void *workspace, size_t ws_bytes, float *y, void *M,
                     void *stream)
{
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!v || !y || !M || !workspace) return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(v) || !aligned16(y) || !aligned16(M) || !aligned16(workspace))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    sdm_variant var;
    st = check_variant_and_ws(h, B, T, variant, ws_bytes, &var);
    if (st != SDM_OK) return st;

    const sdm::Shape s = shape_of(h, B, T);
    const hipStream_t hs = (hipStream_t)stream;
    const uint32_t *rec = static_cast<const uint32_t *>(workspace);
    if (var == SDM_VARIANT_TIMEPAR && sdm::decode_supported(s)) {
        // one token per sequence: its writes, then its reads, in one kernel
        const hipError_t e =
            sdm::launch_rw_decode(s, rec, v, dtype == SDM_BF16, y, M, h->state, hs);
        if (e != hipSuccess) return hip_fail(e, "one-token write/read launch");
        return SDM_OK;
    }
    if (var == SDM_VARIANT_TIMEPAR) {
        char *tp = static_cast<char *>(workspace) + records_bytes(h, B, T);
        const hipError_t e =
            sdm::launch_tp_apply(s, rec, tp, v, dtype == SDM_BF16, y, M, h->state, hs);
        if (e != hipSuccess) return hip_fail(e, "time-parallel write/read launch");
        return SDM_OK;
    }
    float *Mf = static_cast<float *>(M);  // the serial schedule keeps a float32 state
    const hipError_t e = sdm::rw_serial_supported(s)
                             ? sdm::launch_rw_serial(s, rec, v, dtype == SDM_BF16, y, Mf, hs)
                             : sdm::launch_rw_simple(s, rec, v, dtype == SDM_BF16, y, Mf, hs);
    if (e != hipSuccess) return hip_fail(e, "write/read launch");
    return SDM_OK;
}

sdm_status sdm_forward(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                       const void *v, const float *alpha, const float *beta, sdm_dtype dtype,
                       sdm_variant variant, unsigned flags, void *workspace, size_t ws_bytes,
                       float *y, void *M, void *stream)
{
    // validate everything before enqueueing either half
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!v || !y) return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(v) || !aligned16(y))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    if (!kp || !qp || !alpha || !beta || !M || !workspace)
        return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(kp) || !aligned16(qp) || !aligned16(alpha) || !aligned16(beta) ||
        !aligned16(M) || !aligned16(workspace))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    if (flags & ~SDM_FLAG_CONTINUE) return fail(SDM_ERR_ARG, "unknown flags 0x%x", flags);
    sdm_variant var;
    st = check_variant_and_ws(h, B, T, variant, ws_bytes, &var);
    if (st != SDM_OK) return st;
    const sdm::Shape s = shape_of(h, B, T);
    if (var == SDM_VARIANT_TIMEPAR && sdm::decode_fused_supported(s)) {
        // one token per sequence: selection, writes and reads in one launch
        // (the workspace is not used)
        const hipStream_t hs = (hipStream_t)stream;
        hipError_t e;
        if (!(flags & SDM_FLAG_CONTINUE)) {
            e = sdm::launch_init(s, h->M0, M, h->state, hs);
            if (e != hipSuccess) return hip_fail(e, "init launch");
        }
        e = sdm::launch_decode_fused(s, kp, qp, v, dtype == SDM_BF16, alpha, beta, y, M, h->state,
                                     hs);
        if (e != hipSuccess) return hip_fail(e, "one-token step launch");
        return SDM_OK;
    }
    st = sdm_prepare(h, B, T, kp, qp, alpha, beta, dtype, variant, flags, workspace, ws_bytes, M,
                     stream);
    if (st != SDM_OK) return st;
    return sdm_apply(h, B, T, v, dtype, variant, workspace, ws_bytes, y, M, stream);
}

sdm_status sdm_forward_noalloc(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                               const void *v, const float *alpha, const float *beta,
                               sdm_dtype dtype, sdm_variant variant, unsigned flags, float *y,
                               void *M, void *stream)
{
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!kp || !qp || !v || !alpha || !beta || !y || !M)
        return fail(SDM_ERR_ARG, "null tensor pointer");
    if (!aligned16(kp) || !aligned16(qp) || !aligned16(v) || !aligned16(alpha) ||
        !aligned16(beta) || !aligned16(y) || !aligned16(M))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    if (flags & ~SDM_FLAG_CONTINUE) return fail(SDM_ERR_ARG, "unknown flags 0x%x", flags);
    sdm_variant var;
    st = check_variant(h, B, T, variant, &var);
    if (st != SDM_OK) return st;
    const size_t need = ws_bytes_for(h, B, T, var);
    if (need > (size_t)SDM_NOALLOC_MAX_BYTES)
        return fail(SDM_ERR_UNSUPPORTED,
                    "this call needs %zu bytes of scratch; the static scratch holds %zu "
                    "(fewer sequences or tokens per call, or sdm_forward with a workspace)",
                    need, (size_t)SDM_NOALLOC_MAX_BYTES);
    void *ws = nullptr;
    st = scratch_on((hipStream_t)stream, &ws);
    if (st != SDM_OK) return st;
    return sdm_forward(h, B, T, kp, qp, v, alpha, beta, dtype, variant, flags, ws,
                       (size_t)SDM_NOALLOC_MAX_BYTES, y, M, stream);
}

}  // extern "C"

extern "C" {

sdm_status sdm_backward_workspace_size_ex(sdm_handle h, int B, int64_t T, sdm_dtype dtype,
                                          int chunks, size_t *bytes)
{
    if (!bytes) return fail(SDM_ERR_ARG, "null bytes pointer");
    *bytes = 0;
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    st = check_backward(h, B, T);
    if (st != SDM_OK) return st;
    if (chunks < 0) return fail(SDM_ERR_ARG, "chunks must be >= 0 (got %d)", chunks);
    *bytes = bwd_ws_bytes(h, B, T, chunks);
    return SDM_OK;
}

sdm_status sdm_backward_workspace_size(sdm_handle h, int B, int64_t T, sdm_dtype dtype,
                                       size_t *bytes)
{
    return sdm_backward_workspace_size_ex(h, B, T, dtype, 0, bytes);
}

sdm_status sdm_backward(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                        const void *v, const float *alpha, const float *beta, sdm_dtype dtype,
                        const float *Minit, const float *dy, const float *dMT, void *workspace,
                        size_t ws_bytes, float *dkp, float *dqp, float *dv, float *dalpha,
                        float *dbeta, float *dMinit, float *dM0, void *stream)
{
    sdm_status st = check_handle_call(h, B, T, dtype);
    if (st != SDM_OK) return st;
    if (!kp || !qp || !v || !alpha || !beta || !dy || !workspace || !dkp || !dqp || !dv ||
        !dalpha || !dbeta || !dMinit)
        return fail(SDM_ERR_ARG, "null tensor pointer");
    const void *ptrs[] = {kp, qp, v, alpha, beta, dy, workspace, dkp, dqp, dv, dalpha, dbeta,
                          dMinit};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    if ((Minit && !aligned16(Minit)) || (dMT && !aligned16(dMT)) || (dM0 && !aligned16(dM0)))
        return fail(SDM_ERR_ARG, "tensor pointers must be 16-byte aligned");
    st = check_backward(h, B, T);
    if (st != SDM_OK) return st;
    const int chunks = bwd_chunks_for(h, B, T, ws_bytes);
    if (chunks == 0)
        return fail(SDM_ERR_WORKSPACE, "workspace has %zu bytes, needs at least %zu", ws_bytes,
                    bwd_ws_bytes(h, B, T, 0));

    const sdm::Shape s = shape_of(h, B, T);
    const hipStream_t hs = (hipStream_t)stream;
    uint32_t *rec = static_cast<uint32_t *>(workspace);
    char *fwd = static_cast<char *>(workspace) + records_bytes(h, B, T);
    char *bwd = fwd + round_up(sdm::tp_workspace_bytes(s));
    hipError_t e = sdm::launch_select(s, kp, qp, dtype == SDM_BF16, nullptr, nullptr, nullptr,
                                      nullptr, rec, alpha, beta, hs);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    e = sdm::launch_tp_backward(s, chunks, rec, fwd, bwd, v, dtype == SDM_BF16, h->M0, Minit, dy,
                                dMT, alpha, beta, dkp, dqp, dv, dalpha, dbeta, dMinit, dM0, hs);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return SDM_OK;
}

}  // extern "C"
