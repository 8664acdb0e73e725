// api.cpp -- the C ABI of libssd.so (declared in include/ssd.h): argument
// validation with messages that name the offending argument and its values,
// then one launch on the caller's stream.  Nothing here touches device
// memory or calls HIP before validation has passed.
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/ssd.h"
#include "ssd_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return SSD_OK;
}

int hip_status(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(int dtype) { return dtype == SSD_F32 ? 4 : 2; }

constexpr int kMaxL = 1 << 30;   // tokens per batch row

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Shared size checks; returns SSD_OK or a failure with the message set.
int check_dims(const char* fn, int B, int L, int H, int P, int N, int G, int K, int dtype) {
    if (dtype != SSD_F32 && dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "%s: dtype=%d is not supported (only SSD_F32=0 and SSD_BF16=1; "
                    "fp16, fp64 and other types are refused, not converted)", fn, dtype);
    if (B < 0) return fail(SSD_ERR_BAD_SHAPE, "%s: B=%d must be >= 0", fn, B);
    if (L < 0) return fail(SSD_ERR_BAD_SHAPE, "%s: L=%d must be >= 0", fn, L);
    // the scans address a row's document ids with 32-bit byte offsets
    if (L > kMaxL) return fail(SSD_ERR_BAD_SHAPE, "%s: L=%d is above the %d tokens a row may hold", fn, L, kMaxL);
    if (H <= 0) return fail(SSD_ERR_BAD_SHAPE, "%s: H=%d must be > 0", fn, H);
    if (G <= 0) return fail(SSD_ERR_BAD_SHAPE, "%s: G=%d must be > 0", fn, G);
    if (H % G != 0) return fail(SSD_ERR_BAD_SHAPE, "%s: H=%d is not divisible by G=%d", fn, H, G);
    if (P != 64) return fail(SSD_ERR_UNSUPPORTED, "%s: P=%d is not supported (head dim must be 64)", fn, P);
    if (N != 16 && N != 32 && N != 64 && N != 128)
        return fail(SSD_ERR_UNSUPPORTED, "%s: N=%d is not supported (state dim must be 16, 32, 64 or 128)", fn, N);
    if (K != 4) return fail(SSD_ERR_UNSUPPORTED, "%s: K=%d is not supported (conv kernel must be 4)", fn, K);
    const long long total_heads = (long long)B * H;
    if (total_heads > 0x7fffffffLL)
        return fail(SSD_ERR_BAD_SHAPE, "%s: B*H=%lld is too large", fn, total_heads);
    // one batch row of the widest activation (the [x | B | C] columns in T, or y in fp32) must stay below
    // 2^31 bytes: longer rows are not validated (a scan over 4.4 GB rows gave wrong outputs past 2^31 bytes)
    const long long row_bytes = std::max((long long)(H * P + 2 * G * N) * esize(dtype), (long long)H * P * 4);
    if ((long long)L * row_bytes >= (1LL << 31))
        return fail(SSD_ERR_BAD_SHAPE, "%s: L=%d rows of %lld bytes reach 2^31 bytes per batch row (not supported)",
                    fn, L, row_bytes);
    return SSD_OK;
}

int check_tensor(const char* fn, const char* name, const void* p, int64_t stride, int64_t width, int es,
                 bool required) {
    if (!p) {
        if (required) return fail(SSD_ERR_NULL_ARG, "%s: %s is NULL", fn, name);
        return SSD_OK;
    }
    if (stride < width)
        return fail(SSD_ERR_BAD_SHAPE, "%s: %s row stride %lld is smaller than the row width %lld", fn, name,
                    (long long)stride, (long long)width);
    if (!aligned16(p))
        return fail(SSD_ERR_ALIGNMENT, "%s: %s=%p is not 16-byte aligned", fn, name, p);
    if ((stride * es) % 16 != 0)
        return fail(SSD_ERR_ALIGNMENT, "%s: %s row stride %lld elements is not a multiple of 16 bytes", fn, name,
                    (long long)stride);
    return SSD_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, bool required, bool need16) {
    if (!p) return required ? fail(SSD_ERR_NULL_ARG, "%s: %s is NULL", fn, name) : SSD_OK;
    if (need16 && !aligned16(p)) return fail(SSD_ERR_ALIGNMENT, "%s: %s=%p is not 16-byte aligned", fn, name, p);
    if (!need16 && (reinterpret_cast<uintptr_t>(p) & 3u))
        return fail(SSD_ERR_ALIGNMENT, "%s: %s=%p is not 4-byte aligned", fn, name, p);
    return SSD_OK;
}

#define TRY(expr)                     \
    do {                              \
        int _s = (expr);              \
        if (_s != SSD_OK) return _s;  \
    } while (0)

}  // namespace

extern "C" {

const char* ssd_last_error(void) { return g_err; }

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG";
        case SSD_ERR_BAD_SHAPE: return "SSD_ERR_BAD_SHAPE";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
        case SSD_ERR_ALIGNMENT: return "SSD_ERR_ALIGNMENT";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
        case SSD_ERR_HIP: return "SSD_ERR_HIP";
    }
    return "SSD_ERR_UNKNOWN";
}

int ssd_version(void) { return SSD_ABI_VERSION; }

int ssd_conv_fwd(int B, int L, int H, int P, int N, int G, int K, int dtype,
                 const void* xbc_raw, int64_t xbc_raw_row_stride,
                 const float* conv_w, const float* conv_b,
                 const void* dt_raw, int64_t dt_raw_row_stride,
                 const float* dt_bias, const int32_t* doc_ids,
                 const void* conv_state_in, void* conv_state_out, int act,
                 void* xbc_out, int64_t xbc_out_row_stride, float* dt_out,
                 void* stream) {
    const char* fn = "ssd_conv_fwd";
    TRY(check_dims(fn, B, L, H, P, N, G, K, dtype));
    if (act != SSD_ACT_SILU && act != SSD_ACT_NONE)
        return fail(SSD_ERR_UNSUPPORTED, "%s: act=%d is not supported (SSD_ACT_SILU=0, SSD_ACT_NONE=1)", fn, act);
    const int64_t C = (int64_t)H * P + 2LL * G * N;
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    TRY(check_tensor(fn, "xbc_raw", xbc_raw, xbc_raw_row_stride, C, es, work));
    TRY(check_tensor(fn, "xbc_out", xbc_out, xbc_out_row_stride, C, es, work));
    TRY(check_ptr(fn, "conv_w", conv_w, true, true));
    TRY(check_ptr(fn, "conv_b", conv_b, false, false));
    if (dt_raw) {
        if (dt_raw_row_stride < H)
            return fail(SSD_ERR_BAD_SHAPE, "%s: dt_raw row stride %lld is smaller than H=%d", fn,
                        (long long)dt_raw_row_stride, H);
        TRY(check_ptr(fn, "dt_raw", dt_raw, true, false));
        TRY(check_ptr(fn, "dt_out", dt_out, true, false));
    } else if (dt_out) {
        return fail(SSD_ERR_NULL_ARG, "%s: dt_out is given but dt_raw is NULL", fn);
    }
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    TRY(check_ptr(fn, "conv_state_in", conv_state_in, false, true));
    TRY(check_ptr(fn, "conv_state_out", conv_state_out, false, true));
    if (work && xbc_out == xbc_raw)
        return fail(SSD_ERR_BAD_SHAPE, "%s: xbc_out must not alias xbc_raw (halo rows are re-read)", fn);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        // nothing to convolve; the carried state passes through unchanged
        if (conv_state_out && B > 0)
            return hip_status(fn, ssd::launch_copy16(conv_state_in, conv_state_out, (size_t)B * 3 * C * es / 16, s));
        return ok();
    }
    ssd::ConvArgs a;
    a.B = B; a.L = L; a.C = (int)C; a.H = H; a.dtype = dtype; a.act = act;
    a.Lb_in = a.Lb_out = L;
    a.raw = xbc_raw; a.raw_stride = xbc_raw_row_stride;
    a.w = conv_w; a.bias = conv_b;
    a.dt_raw = dt_raw; a.dt_stride = dt_raw_row_stride; a.dt_bias = dt_bias;
    a.doc = doc_ids;
    a.state_in = conv_state_in; a.state_out = conv_state_out;
    a.out = xbc_out; a.out_stride = xbc_out_row_stride;
    a.dt_out = dt_out;
    return hip_status(fn, ssd::launch_conv(a, s));
}

size_t ssd_chunk_scan_workspace_size(int B, int L, int H, int P, int N, int G, int dtype) {
    (void)G; (void)dtype;
    if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0) return 0;
    return ssd::scan_workspace_bytes(B, L, H, P, N, G, dtype);
}

// The scan behind ssd_chunk_scan_fwd and ssd_chunk_scan_fwd_static.
// static_ws: take the split workspace from the library's static scratch.
static int chunk_scan_fwd(const char* fn, bool static_ws, int B, int L, int H, int P, int N, int G, int chunk,
                          int dtype, const void* x, int64_t x_row_stride, const void* Bm, int64_t B_row_stride,
                          const void* Cm, int64_t C_row_stride, const float* dt, int64_t dt_row_stride,
                          int dt_softplus, const float* dt_bias, const float* A, const float* D, const void* z,
                          int64_t z_row_stride, const int32_t* doc_ids, const int32_t* lengths,
                          const float* init_state, float* final_state, float* y, int64_t y_row_stride,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (lengths && (init_state || final_state))
        return fail(SSD_ERR_BAD_SHAPE, "%s: lengths cannot be combined with init_state / final_state", fn);
    TRY(check_ptr(fn, "lengths", lengths, false, false));
    TRY(check_dims(fn, B, L, H, P, N, G, 4, dtype));
    if (chunk != 64) return fail(SSD_ERR_UNSUPPORTED, "%s: chunk=%d is not supported (must be 64)", fn, chunk);
    if (dt_softplus != 0 && dt_softplus != 1)
        return fail(SSD_ERR_UNSUPPORTED, "%s: dt_softplus=%d must be 0 or 1", fn, dt_softplus);
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    TRY(check_tensor(fn, "x", x, x_row_stride, (int64_t)H * P, es, work));
    TRY(check_tensor(fn, "Bm", Bm, B_row_stride, (int64_t)G * N, es, work));
    TRY(check_tensor(fn, "Cm", Cm, C_row_stride, (int64_t)G * N, es, work));
    TRY(check_tensor(fn, "z", z, z_row_stride, (int64_t)H * P, es, false));
    TRY(check_tensor(fn, "y", y, y_row_stride, (int64_t)H * P, 4, work));
    if (work) {
        if (!dt) return fail(SSD_ERR_NULL_ARG, "%s: dt is NULL", fn);
        if (dt_row_stride < H)
            return fail(SSD_ERR_BAD_SHAPE, "%s: dt row stride %lld is smaller than H=%d", fn, (long long)dt_row_stride, H);
    }
    TRY(check_ptr(fn, "dt", dt, false, false));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "A", A, B > 0, false));
    TRY(check_ptr(fn, "D", D, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    TRY(check_ptr(fn, "init_state", init_state, false, true));
    TRY(check_ptr(fn, "final_state", final_state, false, true));
    // A workspace enables the sequence split (when these sizes call for one);
    // without one the scan is a single sequential pass over every (b, h).
    const size_t need = ssd_chunk_scan_workspace_size(B, L, H, P, N, G, dtype);
    if (static_ws && need > 0) {
        if (need > SSD_STATIC_SCRATCH_BYTES)
            return fail(SSD_ERR_WORKSPACE,
                        "%s: these sizes need %zu bytes of workspace, more than the %zu-byte static scratch "
                        "(use ssd_chunk_scan_fwd with a caller workspace, or none)",
                        fn, need, (size_t)SSD_STATIC_SCRATCH_BYTES);
        TRY(hip_status(fn, ssd::scan_static_scratch(&workspace, &workspace_bytes)));
    }
    const bool split = workspace != nullptr && need > 0;
    if (split && workspace_bytes < need)
        return fail(SSD_ERR_WORKSPACE, "%s: workspace_bytes=%zu is smaller than the required %zu", fn,
                    workspace_bytes, need);
    if (split && !aligned16(workspace))
        return fail(SSD_ERR_ALIGNMENT, "%s: workspace=%p is not 16-byte aligned", fn, workspace);
    if (work && (x_row_stride > (1 << 22) || B_row_stride > (1 << 22) || C_row_stride > (1 << 22) ||
                 z_row_stride > (1 << 22) || dt_row_stride > (1 << 22) ||
                 y_row_stride > (1 << 22)))
        return fail(SSD_ERR_BAD_SHAPE, "%s: row strides above 4194304 elements are not supported", fn);
    if (work && y == final_state)
        return fail(SSD_ERR_BAD_SHAPE, "%s: y must not alias final_state", fn);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        if (final_state && B > 0)
            return hip_status(fn, ssd::launch_copy16(init_state, final_state, (size_t)B * H * P * N * 4 / 16, s));
        return ok();
    }
    ssd::ScanArgs a{};
    a.B = B; a.L = L; a.H = H; a.P = P; a.N = N; a.G = G; a.dtype = dtype; a.Lb = L;
    a.x = x; a.x_stride = x_row_stride;
    a.Bm = Bm; a.B_stride = B_row_stride;
    a.Cm = Cm; a.C_stride = C_row_stride;
    a.dt = dt; a.dt_stride = dt_row_stride;
    a.dt_softplus = dt_softplus; a.dt_bias = dt_bias;
    a.A = A; a.D = D;
    a.z = z; a.z_stride = z_row_stride;
    a.doc = doc_ids;
    a.init_state = init_state; a.final_state = final_state;
    a.y = y; a.y_stride = y_row_stride;
    a.K = 1; a.S = ((L + 63) / 64) * 64; a.hloc = nullptr; a.dec = nullptr; a.h0 = nullptr;
    if (split) {
        ssd::scan_split(B, L, H, N, G, dtype, a.K, a.S);
        const size_t u = (size_t)B * H * (a.K - 1);
        a.hloc = static_cast<float*>(workspace);
        a.dec = a.hloc + u * (size_t)P * N;
        if (init_state) a.h0 = a.dec + ((u * sizeof(float) + 255) / 256) * 256 / sizeof(float);
    }
    TRY(hip_status(fn, ssd::launch_scan(a, s)));
    if (lengths) return hip_status(fn, ssd::launch_zero_rows(y, y_row_stride, B, L, H * P, lengths, s));
    return ok();
}

int ssd_chunk_scan_fwd(int B, int L, int H, int P, int N, int G, int chunk, int dtype,
                       const void* x, int64_t x_row_stride,
                       const void* Bm, int64_t B_row_stride,
                       const void* Cm, int64_t C_row_stride,
                       const float* dt, int64_t dt_row_stride,
                       int dt_softplus, const float* dt_bias,
                       const float* A, const float* D,
                       const void* z, int64_t z_row_stride,
                       const int32_t* doc_ids, const int32_t* lengths,
                       const float* init_state, float* final_state,
                       float* y, int64_t y_row_stride,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_scan_fwd("ssd_chunk_scan_fwd", false, B, L, H, P, N, G, chunk, dtype, x, x_row_stride, Bm,
                          B_row_stride, Cm, C_row_stride, dt, dt_row_stride, dt_softplus, dt_bias, A, D, z,
                          z_row_stride, doc_ids, lengths, init_state, final_state, y, y_row_stride, workspace,
                          workspace_bytes, stream);
}

int ssd_chunk_scan_fwd_static(int B, int L, int H, int P, int N, int G, int chunk, int dtype,
                              const void* x, int64_t x_row_stride,
                              const void* Bm, int64_t B_row_stride,
                              const void* Cm, int64_t C_row_stride,
                              const float* dt, int64_t dt_row_stride,
                              int dt_softplus, const float* dt_bias,
                              const float* A, const float* D,
                              const void* z, int64_t z_row_stride,
                              const int32_t* doc_ids, const int32_t* lengths,
                              const float* init_state, float* final_state,
                              float* y, int64_t y_row_stride, void* stream) {
    return chunk_scan_fwd("ssd_chunk_scan_fwd_static", true, B, L, H, P, N, G, chunk, dtype, x, x_row_stride, Bm,
                          B_row_stride, Cm, C_row_stride, dt, dt_row_stride, dt_softplus, dt_bias, A, D, z,
                          z_row_stride, doc_ids, lengths, init_state, final_state, y, y_row_stride, nullptr, 0,
                          stream);
}

size_t ssd_mixer_workspace_size(int B, int L, int H, int P, int N, int G, int dtype) {
    if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0) return 0;
    // the staged plan: the conv output [B][L][conv_dim] (T) and dt [B][L][H] (fp32), then the split state
    const size_t C = (size_t)H * P + 2 * (size_t)G * N;
    return round256((size_t)B * L * C * esize(dtype)) + round256((size_t)B * L * H * 4) +
           ssd::scan_workspace_bytes(B, L, H, P, N, G, dtype);
}

int ssd_mixer_fwd(int B, int L, int H, int P, int N, int G, int K, int chunk, int dtype,
                  const void* xbc_raw, int64_t xbc_raw_row_stride,
                  const float* conv_w, const float* conv_b,
                  const void* dt_raw, int64_t dt_raw_row_stride, const float* dt_bias,
                  const float* A, const float* D,
                  const void* z, int64_t z_row_stride,
                  const int32_t* doc_ids, const int32_t* lengths,
                  const void* conv_state_in, void* conv_state_out,
                  const float* init_state, float* final_state,
                  int act, float* y, int64_t y_row_stride,
                  void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_mixer_fwd";
    if (lengths && (init_state || final_state || conv_state_in || conv_state_out))
        return fail(SSD_ERR_BAD_SHAPE, "%s: lengths cannot be combined with carried states", fn);
    TRY(check_ptr(fn, "lengths", lengths, false, false));
    TRY(check_dims(fn, B, L, H, P, N, G, K, dtype));
    if (chunk != 64) return fail(SSD_ERR_UNSUPPORTED, "%s: chunk=%d is not supported (must be 64)", fn, chunk);
    if (act != SSD_ACT_SILU && act != SSD_ACT_NONE)
        return fail(SSD_ERR_UNSUPPORTED, "%s: act=%d is not supported (SSD_ACT_SILU=0, SSD_ACT_NONE=1)", fn, act);
    const int64_t C = (int64_t)H * P + 2LL * G * N;
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    TRY(check_tensor(fn, "xbc_raw", xbc_raw, xbc_raw_row_stride, C, es, work));
    TRY(check_tensor(fn, "z", z, z_row_stride, (int64_t)H * P, es, false));
    TRY(check_tensor(fn, "y", y, y_row_stride, (int64_t)H * P, 4, work));
    if (work) {
        if (!dt_raw) return fail(SSD_ERR_NULL_ARG, "%s: dt_raw is NULL", fn);
        if (dt_raw_row_stride < H)
            return fail(SSD_ERR_BAD_SHAPE, "%s: dt_raw row stride %lld is smaller than H=%d", fn,
                        (long long)dt_raw_row_stride, H);
        if (dtype == SSD_BF16 && (dt_raw_row_stride & 1))
            return fail(SSD_ERR_ALIGNMENT, "%s: dt_raw row stride %lld must be even for bf16 (4-byte reads)", fn,
                        (long long)dt_raw_row_stride);
    }
    TRY(check_ptr(fn, "dt_raw", dt_raw, false, false));
    TRY(check_ptr(fn, "conv_w", conv_w, work, true));
    TRY(check_ptr(fn, "conv_b", conv_b, false, false));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "A", A, B > 0, false));
    TRY(check_ptr(fn, "D", D, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    TRY(check_ptr(fn, "conv_state_in", conv_state_in, false, true));
    TRY(check_ptr(fn, "conv_state_out", conv_state_out, false, true));
    TRY(check_ptr(fn, "init_state", init_state, false, true));
    TRY(check_ptr(fn, "final_state", final_state, false, true));
    if (conv_state_in && conv_state_out) {
        const uintptr_t i0 = reinterpret_cast<uintptr_t>(conv_state_in), o0 = reinterpret_cast<uintptr_t>(conv_state_out);
        const uintptr_t n = (uintptr_t)B * 3 * (uintptr_t)C * es;
        if (i0 < o0 + n && o0 < i0 + n)
            return fail(SSD_ERR_BAD_SHAPE, "%s: conv_state_out must not overlap conv_state_in (several workgroups "
                        "read the incoming B/C history while others write the outgoing one)", fn);
    }
    if (work && (xbc_raw_row_stride > (1 << 22) || z_row_stride > (1 << 22) || dt_raw_row_stride > (1 << 22) ||
                 y_row_stride > (1 << 22)))
        return fail(SSD_ERR_BAD_SHAPE, "%s: row strides above 4194304 elements are not supported", fn);
    if (work && y == final_state)
        return fail(SSD_ERR_BAD_SHAPE, "%s: y must not alias final_state", fn);
    // Plan: staged (the conv kernel into the workspace, then the scan) when the workspace holds
    // ssd_mixer_workspace_size() bytes; otherwise (bf16 only) fused, with the sequence split when the
    // workspace holds the scan's split state.
    const size_t need = ssd_mixer_workspace_size(B, L, H, P, N, G, dtype);
    const size_t need_split = ssd::scan_workspace_bytes(B, L, H, P, N, G, dtype);
    if (workspace == nullptr) workspace_bytes = 0;
    const bool staged = work && workspace_bytes >= need;
    if (work && dtype == SSD_F32 && !staged)
        return fail(SSD_ERR_WORKSPACE, "%s: fp32 needs a workspace of ssd_mixer_workspace_size()=%zu bytes (the "
                    "conv output is staged there), got %zu", fn, need, workspace_bytes);
    if (workspace_bytes > 0 && !aligned16(workspace))
        return fail(SSD_ERR_ALIGNMENT, "%s: workspace=%p is not 16-byte aligned", fn, workspace);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        // nothing to scan; both carried states pass through unchanged
        if (B > 0 && conv_state_out) {
            hipError_t e = ssd::launch_copy16(conv_state_in, conv_state_out, (size_t)B * 3 * C * es / 16, s);
            if (e != hipSuccess) return hip_status(fn, e);
        }
        if (B > 0 && final_state)
            return hip_status(fn, ssd::launch_copy16(init_state, final_state, (size_t)B * H * P * N * 4 / 16, s));
        return ok();
    }

    ssd::ScanArgs a{};
    a.B = B; a.L = L; a.H = H; a.P = P; a.N = N; a.G = G; a.dtype = dtype; a.Lb = L;
    a.A = A; a.D = D;
    a.z = z; a.z_stride = z_row_stride;
    a.doc = doc_ids;
    a.init_state = init_state; a.final_state = final_state;
    a.y = y; a.y_stride = y_row_stride;
    a.dt_bias = dt_bias;
    a.K = 1; a.S = ((L + 63) / 64) * 64;
    char* ws = static_cast<char*>(workspace);
    size_t ws_left = workspace_bytes;
    if (staged) {
        // conv into the workspace, then the scan over it
        char* xbc = ws;
        float* dtw = reinterpret_cast<float*>(ws + round256((size_t)B * L * C * es));
        const size_t used = round256((size_t)B * L * C * es) + round256((size_t)B * L * H * 4);
        ws += used;
        ws_left -= used;
        ssd::ConvArgs c;
        c.B = B; c.L = L; c.C = (int)C; c.H = H; c.dtype = dtype; c.act = act;
        c.Lb_in = c.Lb_out = L;
        c.raw = xbc_raw; c.raw_stride = xbc_raw_row_stride;
        c.w = conv_w; c.bias = conv_b;
        c.dt_raw = dt_raw; c.dt_stride = dt_raw_row_stride; c.dt_bias = dt_bias;
        c.doc = doc_ids;
        c.state_in = conv_state_in; c.state_out = conv_state_out;
        c.out = xbc; c.out_stride = C;
        c.dt_out = dtw;
        hipError_t e = ssd::launch_conv(c, s);
        if (e != hipSuccess) return hip_status(fn, e);
        a.x = xbc; a.x_stride = C;
        a.Bm = xbc + (size_t)H * P * es; a.B_stride = C;
        a.Cm = xbc + ((size_t)H * P + (size_t)G * N) * es; a.C_stride = C;
        a.dt = dtw; a.dt_stride = H; a.dt_softplus = 0;
    } else {
        const char* raw = static_cast<const char*>(xbc_raw);
        a.x = raw; a.x_stride = xbc_raw_row_stride;
        a.Bm = raw + (size_t)H * P * es; a.B_stride = xbc_raw_row_stride;
        a.Cm = raw + ((size_t)H * P + (size_t)G * N) * es; a.C_stride = xbc_raw_row_stride;
        a.dt16 = static_cast<const uint16_t*>(dt_raw); a.dt16_stride = dt_raw_row_stride; a.dt_softplus = 1;
        a.conv = 1; a.act = act;
        a.conv_w = conv_w; a.conv_b = conv_b;
        a.cstate_in = conv_state_in; a.cstate_out = conv_state_out;
    }
    if (need_split > 0 && ws_left >= need_split) {
        ssd::scan_split(B, L, H, N, G, dtype, a.K, a.S);
        const size_t u = (size_t)B * H * (a.K - 1);
        a.hloc = reinterpret_cast<float*>(ws);
        a.dec = a.hloc + u * (size_t)P * N;
        if (init_state) a.h0 = a.dec + ((u * sizeof(float) + 255) / 256) * 256 / sizeof(float);
    }
    TRY(hip_status(fn, ssd::launch_scan(a, s)));
    if (lengths) return hip_status(fn, ssd::launch_zero_rows(y, y_row_stride, B, L, H * P, lengths, s));
    return ok();
}

int ssd_resume_fwd(int B, int H, int P, int N, int G, int K, int dtype, int pos, int n,
                   const void* xbc_raw, const void* dt_raw, const void* z,
                   const float* conv_w, const float* conv_b, const float* dt_bias,
                   const float* A, const float* D, int act,
                   void* conv_state, void* chunk_xbc, float* chunk_dt, void* chunk_z,
                   float* chunk_state, float* chunk_y, float* y, void* stream) {
    const char* fn = "ssd_resume_fwd";
    TRY(check_dims(fn, B, 1, H, P, N, G, K, dtype));
    if (act != SSD_ACT_SILU && act != SSD_ACT_NONE)
        return fail(SSD_ERR_UNSUPPORTED, "%s: act=%d is not supported (SSD_ACT_SILU=0, SSD_ACT_NONE=1)", fn, act);
    if (pos < 0 || pos > 63)
        return fail(SSD_ERR_BAD_SHAPE, "%s: pos=%d must lie in [0, 63] (tokens already in the working chunk)", fn, pos);
    if (n < 1 || pos + n > 64)
        return fail(SSD_ERR_BAD_SHAPE, "%s: n=%d must be >= 1 with pos + n = %d <= 64", fn, n, pos + n);
    const bool work = B > 0;
    const int64_t C = (int64_t)H * P + 2LL * G * N;
    const int es = esize(dtype);
    if (C > (1 << 22))   // the working chunk's rows are C elements apart
        return fail(SSD_ERR_BAD_SHAPE, "%s: conv_dim=%lld above 4194304 is not supported", fn, (long long)C);
    TRY(check_ptr(fn, "xbc_raw", xbc_raw, work, true));
    TRY(check_ptr(fn, "dt_raw", dt_raw, work, false));
    TRY(check_ptr(fn, "z", z, false, true));
    TRY(check_ptr(fn, "conv_w", conv_w, work, true));
    TRY(check_ptr(fn, "conv_b", conv_b, false, false));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "A", A, work, false));
    TRY(check_ptr(fn, "D", D, false, false));
    TRY(check_ptr(fn, "conv_state", conv_state, work, true));
    TRY(check_ptr(fn, "chunk_xbc", chunk_xbc, work, true));
    TRY(check_ptr(fn, "chunk_dt", chunk_dt, work, false));
    TRY(check_ptr(fn, "chunk_z", chunk_z, false, true));
    TRY(check_ptr(fn, "chunk_state", chunk_state, work, true));
    TRY(check_ptr(fn, "chunk_y", chunk_y, work, true));
    TRY(check_ptr(fn, "y", y, work, true));
    if ((z == nullptr) != (chunk_z == nullptr))
        return fail(SSD_ERR_NULL_ARG, "%s: z and chunk_z must be given together (z=%p, chunk_z=%p)", fn, z, chunk_z);
    if (!work) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t HP = (int64_t)H * P;

    // 1. conv of the new tokens into rows pos .. pos+n-1 of the working chunk;
    //    the rolling conv state advances in place
    ssd::ConvArgs c;
    c.B = B; c.L = n; c.C = (int)C; c.H = H; c.dtype = dtype; c.act = act;
    c.Lb_in = n; c.Lb_out = 64;
    c.raw = xbc_raw; c.raw_stride = C;
    c.w = conv_w; c.bias = conv_b;
    c.dt_raw = dt_raw; c.dt_stride = H; c.dt_bias = dt_bias;
    c.doc = nullptr;
    c.state_in = conv_state; c.state_out = conv_state;
    c.out = static_cast<char*>(chunk_xbc) + (size_t)pos * C * es; c.out_stride = C;
    c.dt_out = chunk_dt + (size_t)pos * H;
    hipError_t e = ssd::launch_conv(c, s);
    if (e != hipSuccess) return hip_status(fn, e);
    // 2. the gate rows
    if (z) {
        e = ssd::launch_copy_rows(z, HP * es, n * HP * es, static_cast<char*>(chunk_z) + (size_t)pos * HP * es,
                                  HP * es, 64 * HP * es, B, n, (int)(HP * es), s);
        if (e != hipSuccess) return hip_status(fn, e);
    }
    // 3. the scan over the working chunk from its starting state, as the
    //    sequential forward runs this chunk; a full chunk replaces the state
    ssd::ScanArgs a{};
    a.B = B; a.L = pos + n; a.H = H; a.P = P; a.N = N; a.G = G; a.dtype = dtype; a.Lb = 64;
    const char* xb = static_cast<const char*>(chunk_xbc);
    a.x = xb; a.x_stride = C;
    a.Bm = xb + (size_t)HP * es; a.B_stride = C;
    a.Cm = xb + ((size_t)HP + (size_t)G * N) * es; a.C_stride = C;
    a.dt = chunk_dt; a.dt_stride = H; a.dt_softplus = 0;
    a.A = A; a.D = D;
    a.z = chunk_z; a.z_stride = HP;
    a.doc = nullptr;
    a.init_state = chunk_state; a.final_state = pos + n == 64 ? chunk_state : nullptr;
    a.y = chunk_y; a.y_stride = HP;
    a.K = 1; a.S = 64;
    a.y_row0 = pos;   // rows before pos were output by earlier calls
    e = ssd::launch_scan(a, s);
    if (e != hipSuccess) return hip_status(fn, e);
    // 4. the new tokens' outputs
    return hip_status(fn, ssd::launch_copy_rows(chunk_y + (size_t)pos * HP, HP * 4, 64 * HP * 4, y, HP * 4,
                                                n * HP * 4, B, n, (int)(HP * 4), s));
}

static int check_bwd_dims(const char* fn, int B, int L, int H, int P, int N, int G, int dtype) {
    TRY(check_dims(fn, B, L, H, P, N, G, 4, dtype));
    return SSD_OK;
}

size_t ssd_chunk_scan_bwd_workspace_size(int B, int L, int H, int P, int N, int G, int dtype) {
    (void)G; (void)dtype;
    if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0) return 0;
    return ssd::scan_bwd_workspace_bytes(B, L, H, P, N);
}

// Shared by ssd_chunk_scan_bwd and ssd_mixer_bwd: the three backward passes,
// arguments already validated.
static int run_scan_bwd(const char* fn, ssd::BwdArgs& a, void* workspace, hipStream_t s) {
    const size_t nc = (size_t)(a.L + 63) / 64;
    const size_t st = round256((size_t)a.B * a.H * nc * a.N * a.P * sizeof(float));
    a.nc = (int)nc;
    a.S = static_cast<float*>(workspace);
    a.dS = a.S + st / sizeof(float);
    a.dec = a.dS + st / sizeof(float);
    a.part = a.dec + round256((size_t)a.B * a.H * nc * sizeof(float)) / sizeof(float);
    return hip_status(fn, ssd::launch_scan_bwd(a, s));
}

int ssd_chunk_scan_bwd(int B, int L, int H, int P, int N, int G, int chunk, int dtype,
                       const void* x, int64_t x_row_stride,
                       const void* Bm, int64_t B_row_stride,
                       const void* Cm, int64_t C_row_stride,
                       const float* dt, int64_t dt_row_stride,
                       int dt_softplus, const float* dt_bias,
                       const float* A, const float* D,
                       const void* z, int64_t z_row_stride,
                       const int32_t* doc_ids,
                       const float* grad_y, int64_t grad_y_row_stride,
                       float* dx, int64_t dx_row_stride,
                       float* dB, int64_t dB_row_stride,
                       float* dC, int64_t dC_row_stride,
                       float* ddt, int64_t ddt_row_stride,
                       float* ddt_bias, float* dA, float* dD,
                       float* dz, int64_t dz_row_stride,
                       void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_chunk_scan_bwd";
    TRY(check_bwd_dims(fn, B, L, H, P, N, G, dtype));
    if (chunk != 64) return fail(SSD_ERR_UNSUPPORTED, "%s: chunk=%d is not supported (must be 64)", fn, chunk);
    if (dt_softplus != 0 && dt_softplus != 1)
        return fail(SSD_ERR_UNSUPPORTED, "%s: dt_softplus=%d must be 0 or 1", fn, dt_softplus);
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N;
    TRY(check_tensor(fn, "x", x, x_row_stride, HP, es, work));
    TRY(check_tensor(fn, "Bm", Bm, B_row_stride, GN, es, work));
    TRY(check_tensor(fn, "Cm", Cm, C_row_stride, GN, es, work));
    TRY(check_tensor(fn, "z", z, z_row_stride, HP, es, false));
    TRY(check_tensor(fn, "grad_y", grad_y, grad_y_row_stride, HP, 4, work));
    TRY(check_tensor(fn, "dx", dx, dx_row_stride, HP, 4, work));
    TRY(check_tensor(fn, "dB", dB, dB_row_stride, GN, 4, work));
    TRY(check_tensor(fn, "dC", dC, dC_row_stride, GN, 4, work));
    TRY(check_tensor(fn, "dz", dz, dz_row_stride, HP, 4, false));
    if (work) {
        if (!dt) return fail(SSD_ERR_NULL_ARG, "%s: dt is NULL", fn);
        if (dt_row_stride < H)
            return fail(SSD_ERR_BAD_SHAPE, "%s: dt row stride %lld is smaller than H=%d", fn, (long long)dt_row_stride, H);
        if (!ddt) return fail(SSD_ERR_NULL_ARG, "%s: ddt is NULL", fn);
        if (ddt_row_stride < H)
            return fail(SSD_ERR_BAD_SHAPE, "%s: ddt row stride %lld is smaller than H=%d", fn,
                        (long long)ddt_row_stride, H);
    }
    if (dz && !z) return fail(SSD_ERR_NULL_ARG, "%s: dz is given but z is NULL", fn);
    TRY(check_ptr(fn, "dt", dt, false, false));
    TRY(check_ptr(fn, "ddt", ddt, false, false));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "A", A, B > 0, false));
    TRY(check_ptr(fn, "dA", dA, B > 0, false));
    TRY(check_ptr(fn, "D", D, false, false));
    TRY(check_ptr(fn, "dD", dD, false, false));
    TRY(check_ptr(fn, "ddt_bias", ddt_bias, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    if (work && (x_row_stride > (1 << 22) || B_row_stride > (1 << 22) || C_row_stride > (1 << 22) ||
                 z_row_stride > (1 << 22) || dt_row_stride > (1 << 22) || grad_y_row_stride > (1 << 22) ||
                 dx_row_stride > (1 << 22) || dB_row_stride > (1 << 22) || dC_row_stride > (1 << 22) ||
                 ddt_row_stride > (1 << 22) || dz_row_stride > (1 << 22)))
        return fail(SSD_ERR_BAD_SHAPE, "%s: row strides above 4194304 elements are not supported", fn);
    const size_t need = ssd_chunk_scan_bwd_workspace_size(B, L, H, P, N, G, dtype);
    if (work && (!workspace || workspace_bytes < need))
        return fail(SSD_ERR_WORKSPACE, "%s: workspace_bytes=%zu is smaller than the required %zu", fn,
                    workspace ? workspace_bytes : (size_t)0, need);
    if (work && !aligned16(workspace))
        return fail(SSD_ERR_ALIGNMENT, "%s: workspace=%p is not 16-byte aligned", fn, workspace);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {   // no tokens: every parameter gradient is zero
        if (B > 0) {
            TRY(hip_status(fn, ssd::launch_zero_f32(dA, (size_t)H, s)));
            TRY(hip_status(fn, ssd::launch_zero_f32(dD, (size_t)H, s)));
            TRY(hip_status(fn, ssd::launch_zero_f32(dt_softplus ? ddt_bias : nullptr, (size_t)H, s)));
        }
        return ok();
    }
    ssd::BwdArgs a{};
    a.B = B; a.L = L; a.H = H; a.P = P; a.N = N; a.G = G; a.dtype = dtype;
    a.x = x; a.x_stride = x_row_stride;
    a.Bm = Bm; a.B_stride = B_row_stride;
    a.Cm = Cm; a.C_stride = C_row_stride;
    a.dt = dt; a.dt_stride = dt_row_stride;
    a.dt_softplus = dt_softplus; a.chain_from_dt = 0; a.dt_bias = dt_bias;
    a.A = A; a.D = D;
    a.z = z; a.z_stride = z_row_stride;
    a.doc = doc_ids;
    a.gy = grad_y; a.gy_stride = grad_y_row_stride;
    a.dx = dx; a.dx_stride = dx_row_stride;
    a.dB = dB; a.dB_stride = dB_row_stride;
    a.dC = dC; a.dC_stride = dC_row_stride;
    a.ddt = ddt; a.ddt_stride = ddt_row_stride;
    a.dz = dz; a.dz_stride = dz_row_stride;
    a.ddt_bias = dt_softplus ? ddt_bias : nullptr; a.dA = dA; a.dD = D ? dD : nullptr;
    if (!D) TRY(hip_status(fn, ssd::launch_zero_f32(dD, (size_t)H, s)));
    return run_scan_bwd(fn, a, workspace, s);
}

size_t ssd_conv_bwd_workspace_size(int B, int L, int H, int P, int N, int G, int dtype) {
    (void)dtype;
    if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return 0;
    return ssd::conv_bwd_workspace_bytes(B, L, H * P + 2 * G * N);
}

static int run_conv_bwd(const char* fn, int B, int L, int C, int dtype, const void* raw, int64_t raw_stride,
                        const float* w, const float* bias, const int32_t* doc, int act, const float* dout,
                        int64_t dout_stride, float* draw, int64_t draw_stride, float* dw, float* dbias,
                        void* workspace, hipStream_t s) {
    ssd::ConvBwdArgs c{};
    c.B = B; c.L = L; c.C = C; c.dtype = dtype; c.act = act;
    c.raw = raw; c.raw_stride = raw_stride;
    c.w = w; c.bias = bias; c.doc = doc;
    c.dout = dout; c.dout_stride = dout_stride;
    c.draw = draw; c.draw_stride = draw_stride;
    c.dw = dw; c.dbias = dbias;
    c.ntc = (L + 63) / 64;
    c.part = static_cast<float*>(workspace);
    return hip_status(fn, ssd::launch_conv_bwd(c, s));
}

int ssd_conv_bwd(int B, int L, int H, int P, int N, int G, int K, int dtype,
                 const void* xbc_raw, int64_t xbc_raw_row_stride,
                 const float* conv_w, const float* conv_b, const int32_t* doc_ids, int act,
                 const float* grad_xbc, int64_t grad_xbc_row_stride,
                 float* dxbc_raw, int64_t dxbc_raw_row_stride,
                 float* dconv_w, float* dconv_b,
                 void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_conv_bwd";
    TRY(check_dims(fn, B, L, H, P, N, G, K, dtype));
    if (act != SSD_ACT_SILU && act != SSD_ACT_NONE)
        return fail(SSD_ERR_UNSUPPORTED, "%s: act=%d is not supported (SSD_ACT_SILU=0, SSD_ACT_NONE=1)", fn, act);
    const int64_t C = (int64_t)H * P + 2LL * G * N;
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    TRY(check_tensor(fn, "xbc_raw", xbc_raw, xbc_raw_row_stride, C, es, work));
    TRY(check_tensor(fn, "grad_xbc", grad_xbc, grad_xbc_row_stride, C, 4, work));
    TRY(check_tensor(fn, "dxbc_raw", dxbc_raw, dxbc_raw_row_stride, C, 4, work));
    TRY(check_ptr(fn, "conv_w", conv_w, true, true));
    TRY(check_ptr(fn, "dconv_w", dconv_w, true, false));
    TRY(check_ptr(fn, "conv_b", conv_b, false, false));
    TRY(check_ptr(fn, "dconv_b", dconv_b, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    const size_t need = ssd_conv_bwd_workspace_size(B, L, H, P, N, G, dtype);
    if (work && (!workspace || workspace_bytes < need))
        return fail(SSD_ERR_WORKSPACE, "%s: workspace_bytes=%zu is smaller than the required %zu", fn,
                    workspace ? workspace_bytes : (size_t)0, need);
    if (work && !aligned16(workspace))
        return fail(SSD_ERR_ALIGNMENT, "%s: workspace=%p is not 16-byte aligned", fn, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        TRY(hip_status(fn, ssd::launch_zero_f32(dconv_w, (size_t)C * 4, s)));
        TRY(hip_status(fn, ssd::launch_zero_f32(dconv_b, (size_t)C, s)));
        return ok();
    }
    return run_conv_bwd(fn, B, L, (int)C, dtype, xbc_raw, xbc_raw_row_stride, conv_w, conv_b, doc_ids, act, grad_xbc,
                        grad_xbc_row_stride, dxbc_raw, dxbc_raw_row_stride, dconv_w, dconv_b, workspace, s);
}

size_t ssd_mixer_bwd_workspace_size(int B, int L, int H, int P, int N, int G, int dtype) {
    if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return 0;
    const size_t C = (size_t)H * P + 2 * (size_t)G * N;
    return round256((size_t)B * L * C * esize(dtype)) + round256((size_t)B * L * H * 4) +
           round256((size_t)B * L * C * 4) + ssd_chunk_scan_bwd_workspace_size(B, L, H, P, N, G, dtype) +
           round256(ssd_conv_bwd_workspace_size(B, L, H, P, N, G, dtype));
}

int ssd_mixer_bwd(int B, int L, int H, int P, int N, int G, int K, int chunk, int dtype,
                  const void* xbc_raw, int64_t xbc_raw_row_stride,
                  const float* conv_w, const float* conv_b,
                  const void* dt_raw, int64_t dt_raw_row_stride, const float* dt_bias,
                  const float* A, const float* D,
                  const void* z, int64_t z_row_stride,
                  const int32_t* doc_ids, int act,
                  const float* grad_y, int64_t grad_y_row_stride,
                  float* dxbc_raw, int64_t dxbc_raw_row_stride,
                  float* dconv_w, float* dconv_b,
                  float* ddt_raw, int64_t ddt_raw_row_stride, float* ddt_bias,
                  float* dA, float* dD,
                  float* dz, int64_t dz_row_stride,
                  void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_mixer_bwd";
    TRY(check_bwd_dims(fn, B, L, H, P, N, G, dtype));
    if (K != 4) return fail(SSD_ERR_UNSUPPORTED, "%s: K=%d is not supported (conv kernel must be 4)", fn, K);
    if (chunk != 64) return fail(SSD_ERR_UNSUPPORTED, "%s: chunk=%d is not supported (must be 64)", fn, chunk);
    if (act != SSD_ACT_SILU && act != SSD_ACT_NONE)
        return fail(SSD_ERR_UNSUPPORTED, "%s: act=%d is not supported (SSD_ACT_SILU=0, SSD_ACT_NONE=1)", fn, act);
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N, C = HP + 2 * GN;
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    TRY(check_tensor(fn, "xbc_raw", xbc_raw, xbc_raw_row_stride, C, es, work));
    TRY(check_tensor(fn, "z", z, z_row_stride, HP, es, false));
    TRY(check_tensor(fn, "grad_y", grad_y, grad_y_row_stride, HP, 4, work));
    TRY(check_tensor(fn, "dxbc_raw", dxbc_raw, dxbc_raw_row_stride, C, 4, work));
    TRY(check_tensor(fn, "dz", dz, dz_row_stride, HP, 4, false));
    if (work) {
        if (!dt_raw) return fail(SSD_ERR_NULL_ARG, "%s: dt_raw is NULL", fn);
        if (!ddt_raw) return fail(SSD_ERR_NULL_ARG, "%s: ddt_raw is NULL", fn);
        if (dt_raw_row_stride < H || ddt_raw_row_stride < H)
            return fail(SSD_ERR_BAD_SHAPE, "%s: dt_raw / ddt_raw row strides (%lld, %lld) are smaller than H=%d", fn,
                        (long long)dt_raw_row_stride, (long long)ddt_raw_row_stride, H);
    }
    if (dz && !z) return fail(SSD_ERR_NULL_ARG, "%s: dz is given but z is NULL", fn);
    TRY(check_ptr(fn, "dt_raw", dt_raw, false, false));
    TRY(check_ptr(fn, "ddt_raw", ddt_raw, false, false));
    TRY(check_ptr(fn, "conv_w", conv_w, true, true));
    TRY(check_ptr(fn, "dconv_w", dconv_w, true, false));
    TRY(check_ptr(fn, "conv_b", conv_b, false, false));
    TRY(check_ptr(fn, "dconv_b", dconv_b, false, false));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "ddt_bias", ddt_bias, false, false));
    TRY(check_ptr(fn, "A", A, B > 0, false));
    TRY(check_ptr(fn, "dA", dA, B > 0, false));
    TRY(check_ptr(fn, "D", D, false, false));
    TRY(check_ptr(fn, "dD", dD, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    if (work && (xbc_raw_row_stride > (1 << 22) || z_row_stride > (1 << 22) || grad_y_row_stride > (1 << 22) ||
                 dxbc_raw_row_stride > (1 << 22) || dz_row_stride > (1 << 22) || dt_raw_row_stride > (1 << 22) ||
                 ddt_raw_row_stride > (1 << 22)))
        return fail(SSD_ERR_BAD_SHAPE, "%s: row strides above 4194304 elements are not supported", fn);
    const size_t need = ssd_mixer_bwd_workspace_size(B, L, H, P, N, G, dtype);
    if (work && (!workspace || workspace_bytes < need))
        return fail(SSD_ERR_WORKSPACE, "%s: workspace_bytes=%zu is smaller than the required %zu", fn,
                    workspace ? workspace_bytes : (size_t)0, need);
    if (work && !aligned16(workspace))
        return fail(SSD_ERR_ALIGNMENT, "%s: workspace=%p is not 16-byte aligned", fn, workspace);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        if (B > 0) {
            TRY(hip_status(fn, ssd::launch_zero_f32(dA, (size_t)H, s)));
            TRY(hip_status(fn, ssd::launch_zero_f32(dD, (size_t)H, s)));
            TRY(hip_status(fn, ssd::launch_zero_f32(ddt_bias, (size_t)H, s)));
        }
        TRY(hip_status(fn, ssd::launch_zero_f32(dconv_w, (size_t)C * 4, s)));
        TRY(hip_status(fn, ssd::launch_zero_f32(dconv_b, (size_t)C, s)));
        return ok();
    }
    // workspace: the recomputed conv output (T) and dt, the conv output's gradient, then the passes' scratch
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    void* xbc = ws;
    ws += round256((size_t)B * L * C * es);
    float* dtw = reinterpret_cast<float*>(ws);
    ws += round256((size_t)B * L * H * 4);
    float* dxbc = reinterpret_cast<float*>(ws);
    ws += round256((size_t)B * L * C * 4);
    void* scan_ws = ws;
    ws += ssd_chunk_scan_bwd_workspace_size(B, L, H, P, N, G, dtype);
    void* conv_ws = ws;

    ssd::ConvArgs cv{};
    cv.B = B; cv.L = L; cv.C = (int)C; cv.H = H; cv.dtype = dtype; cv.act = act;
    cv.Lb_in = cv.Lb_out = L;
    cv.raw = xbc_raw; cv.raw_stride = xbc_raw_row_stride;
    cv.w = conv_w; cv.bias = conv_b;
    cv.dt_raw = dt_raw; cv.dt_stride = dt_raw_row_stride; cv.dt_bias = dt_bias;
    cv.doc = doc_ids;
    cv.out = xbc; cv.out_stride = C;
    cv.dt_out = dtw;
    TRY(hip_status(fn, ssd::launch_conv(cv, s)));

    const unsigned char* xb = static_cast<const unsigned char*>(xbc);
    ssd::BwdArgs a{};
    a.B = B; a.L = L; a.H = H; a.P = P; a.N = N; a.G = G; a.dtype = dtype;
    a.x = xb; a.x_stride = C;
    a.Bm = xb + HP * es; a.B_stride = C;
    a.Cm = xb + (HP + GN) * es; a.C_stride = C;
    a.dt = dtw; a.dt_stride = H;
    a.dt_softplus = 0; a.chain_from_dt = 1; a.dt_bias = nullptr;   // dt = softplus(dt_raw + dt_bias)
    a.A = A; a.D = D;
    a.z = z; a.z_stride = z_row_stride;
    a.doc = doc_ids;
    a.gy = grad_y; a.gy_stride = grad_y_row_stride;
    a.dx = dxbc; a.dx_stride = C;
    a.dB = dxbc + HP; a.dB_stride = C;
    a.dC = dxbc + HP + GN; a.dC_stride = C;
    a.ddt = ddt_raw; a.ddt_stride = ddt_raw_row_stride;
    a.dz = dz; a.dz_stride = dz_row_stride;
    a.ddt_bias = ddt_bias; a.dA = dA; a.dD = D ? dD : nullptr;
    if (!D) TRY(hip_status(fn, ssd::launch_zero_f32(dD, (size_t)H, s)));
    TRY(run_scan_bwd(fn, a, scan_ws, s));
    return run_conv_bwd(fn, B, L, (int)C, dtype, xbc_raw, xbc_raw_row_stride, conv_w, conv_b, doc_ids, act, dxbc, C,
                        dxbc_raw, dxbc_raw_row_stride, dconv_w, dconv_b, conv_ws, s);
}

size_t ssd_s6_workspace_size(int B, int L, int D, int N, int dtype) {
    (void)dtype;
    if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 0;
    return ssd::s6_workspace_bytes(B, L, D, N);
}

int ssd_s6_scan_fwd(int B, int L, int D, int N, int dtype,
                    const void* x, int64_t x_row_stride,
                    const void* dt, int64_t dt_row_stride,
                    int dt_softplus, const float* dt_bias,
                    const float* A,
                    const void* Bm, int64_t B_row_stride,
                    const void* Cm, int64_t C_row_stride,
                    const float* D_skip,
                    const void* z, int64_t z_row_stride,
                    const int32_t* doc_ids,
                    const float* init_state, float* final_state,
                    float* y, int64_t y_row_stride,
                    void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "ssd_s6_scan_fwd";
    if (dtype != SSD_F32 && dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "%s: dtype=%d is not supported (only SSD_F32=0 and SSD_BF16=1; "
                    "fp16, fp64 and other types are refused, not converted)", fn, dtype);
    if (B < 0) return fail(SSD_ERR_BAD_SHAPE, "%s: B=%d must be >= 0", fn, B);
    if (L < 0) return fail(SSD_ERR_BAD_SHAPE, "%s: L=%d must be >= 0", fn, L);
    if (D <= 0) return fail(SSD_ERR_BAD_SHAPE, "%s: D=%d must be > 0", fn, D);
    if (N != 8 && N != 16 && N != 32)
        return fail(SSD_ERR_UNSUPPORTED, "%s: N=%d is not supported (state dim must be 8, 16 or 32)", fn, N);
    if ((long long)B * D > 0x7fffffffLL || (long long)B * L > 0x7fffffffLL)
        return fail(SSD_ERR_BAD_SHAPE, "%s: B*D or B*L is too large", fn);
    if (dt_softplus != 0 && dt_softplus != 1)
        return fail(SSD_ERR_UNSUPPORTED, "%s: dt_softplus=%d must be 0 or 1", fn, dt_softplus);
    const int es = esize(dtype);
    const bool work = B > 0 && L > 0;
    TRY(check_tensor(fn, "x", x, x_row_stride, D, es, work));
    TRY(check_tensor(fn, "dt", dt, dt_row_stride, D, es, work));
    TRY(check_tensor(fn, "Bm", Bm, B_row_stride, N, es, work));
    TRY(check_tensor(fn, "Cm", Cm, C_row_stride, N, es, work));
    TRY(check_tensor(fn, "z", z, z_row_stride, D, es, false));
    TRY(check_tensor(fn, "y", y, y_row_stride, D, 4, work));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "A", A, B > 0, false));
    TRY(check_ptr(fn, "D_skip", D_skip, false, false));
    TRY(check_ptr(fn, "doc_ids", doc_ids, false, false));
    TRY(check_ptr(fn, "init_state", init_state, false, true));
    TRY(check_ptr(fn, "final_state", final_state, false, true));
    if (work && (x_row_stride > (1 << 22) || dt_row_stride > (1 << 22) || B_row_stride > (1 << 22) ||
                 C_row_stride > (1 << 22) || z_row_stride > (1 << 22) || y_row_stride > (1 << 22)))
        return fail(SSD_ERR_BAD_SHAPE, "%s: row strides above 4194304 elements are not supported", fn);
    const size_t need = ssd_s6_workspace_size(B, L, D, N, dtype);
    const bool split = workspace != nullptr && need > 0;
    if (split && workspace_bytes < need)
        return fail(SSD_ERR_WORKSPACE, "%s: workspace_bytes=%zu is smaller than the required %zu", fn,
                    workspace_bytes, need);
    if (split && !aligned16(workspace))
        return fail(SSD_ERR_ALIGNMENT, "%s: workspace=%p is not 16-byte aligned", fn, workspace);
    if (work && y == final_state)
        return fail(SSD_ERR_BAD_SHAPE, "%s: y must not alias final_state", fn);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        if (final_state && B > 0)
            return hip_status(fn, ssd::launch_copy16(init_state, final_state, (size_t)B * D * N * 4 / 16, s));
        return ok();
    }
    ssd::S6Args a{};
    a.B = B; a.L = L; a.D = D; a.N = N; a.dtype = dtype;
    a.x = x; a.x_stride = x_row_stride;
    a.dt = dt; a.dt_stride = dt_row_stride;
    a.dt_softplus = dt_softplus; a.dt_bias = dt_bias;
    a.A = A;
    a.Bm = Bm; a.B_stride = B_row_stride;
    a.Cm = Cm; a.C_stride = C_row_stride;
    a.D_skip = D_skip;
    a.z = z; a.z_stride = z_row_stride;
    a.doc = doc_ids;
    a.init_state = init_state; a.final_state = final_state;
    a.y = y; a.y_stride = y_row_stride;
    a.K = 1; a.S = L;
    if (split) {
        ssd::s6_split(B, L, D, a.K, a.S);
        const size_t u = (size_t)B * D * (a.K - 1);
        a.hloc = static_cast<float*>(workspace);
        a.sdt = a.hloc + u * (size_t)N;
        if (init_state) a.h0 = a.sdt + round256(u * sizeof(float)) / sizeof(float);
    }
    return hip_status(fn, ssd::launch_s6(a, s));
}

int ssd_step(int B, int H, int P, int N, int G, int K, int dtype,
             const void* xbc_raw, const void* dt_raw, const void* z,
             const float* conv_w, const float* conv_b, const float* dt_bias,
             const float* A, const float* D,
             void* conv_state, float* ssm_state, int act, float* y, void* stream) {
    const char* fn = "ssd_step";
    TRY(check_dims(fn, B, 1, H, P, N, G, K, dtype));
    if (act != SSD_ACT_SILU && act != SSD_ACT_NONE)
        return fail(SSD_ERR_UNSUPPORTED, "%s: act=%d is not supported (SSD_ACT_SILU=0, SSD_ACT_NONE=1)", fn, act);
    const bool work = B > 0;
    const int64_t C = (int64_t)H * P + 2LL * G * N;
    TRY(check_ptr(fn, "xbc_raw", xbc_raw, work, true));
    TRY(check_ptr(fn, "dt_raw", dt_raw, work, false));
    TRY(check_ptr(fn, "z", z, false, true));      // read in 16-byte pieces
    TRY(check_ptr(fn, "conv_w", conv_w, work, true));
    TRY(check_ptr(fn, "conv_b", conv_b, false, false));
    TRY(check_ptr(fn, "dt_bias", dt_bias, false, false));
    TRY(check_ptr(fn, "A", A, work, false));
    TRY(check_ptr(fn, "D", D, false, false));
    TRY(check_ptr(fn, "conv_state", conv_state, work, true));
    TRY(check_ptr(fn, "ssm_state", ssm_state, work, true));
    TRY(check_ptr(fn, "y", y, work, false));
    const size_t lds = ssd::step_lds_bytes(H, P, N, G);
    if (lds > 64 * 1024)
        return fail(SSD_ERR_UNSUPPORTED, "%s: conv_dim=%lld plus H*P=%d plus 4*H=%d floats exceed the 64 KiB LDS budget",
                    fn, (long long)C, H * P, 4 * H);
    if (!work) return ok();
    ssd::StepArgs a;
    a.B = B; a.H = H; a.P = P; a.N = N; a.G = G; a.dtype = dtype; a.act = act;
    a.xbc_raw = xbc_raw; a.dt_raw = dt_raw; a.z = z;
    a.conv_w = conv_w; a.conv_b = conv_b; a.dt_bias = dt_bias; a.A = A; a.D = D;
    a.conv_state = conv_state; a.ssm_state = ssm_state; a.y = y;
    return hip_status(fn, ssd::launch_step(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
