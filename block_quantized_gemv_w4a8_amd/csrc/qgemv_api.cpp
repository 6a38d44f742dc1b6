// qgemv_api.cpp -- the C ABI of libqgemv: argument gates, status codes and
// kernel launches.  No allocation, no host synchronisation, no copies.
//
// Every entry point runs its gates in the same order -- NULL pointers,
// shapes, limits of this library, alignment, device -- and returns at the first
// failure without launching anything, so a failed call never leaves a partial
// result (colibri GPU backends, "Eligibility gates" and "Failure invariant").
// A refusal names its reason through qgemv_last_error() ("Backends and
// hardware", section "CUDA": decline at open with a message naming the reason
// rather than run a different path).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "qgemv.h"
#include "qgemv_launch.h"

static_assert(QGEMV_MULTI_MAX == qgemv::kMultiMax, "one limit for the multi-matrix entries");

namespace {

thread_local char g_last_error[256] = "";

qgemv_status fail(qgemv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

qgemv_status ok() { return QGEMV_OK; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Per-device cache of "is this device gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

qgemv_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(QGEMV_E_DEVICE, "no current HIP device");
    }
    if (dev >= kMaxDevices) return fail(QGEMV_E_DEVICE, "device index %d out of range", dev);
    int state = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(QGEMV_E_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
        }
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_dev_ok[dev].store(state, std::memory_order_relaxed);
        if (state == 2)
            return fail(QGEMV_E_DEVICE, "device %d is %s, this library targets gfx950", dev,
                        prop.gcnArchName);
    }
    if (state == 2) return fail(QGEMV_E_DEVICE, "device %d is not gfx950", dev);
    return QGEMV_OK;
}

qgemv_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(QGEMV_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return QGEMV_OK;
}

qgemv_status check_k(int64_t K) {
    if (K < 32 || K % 32 != 0)
        return fail(QGEMV_E_SHAPE, "K = %lld must be a positive multiple of 32", (long long)K);
    return QGEMV_OK;
}

qgemv_status check_act_align(const int8_t* q, const uint16_t* d, const int32_t* s) {
    if (!aligned(q, 16)) return fail(QGEMV_E_ALIGN, "q must be 16-byte aligned");
    if (!aligned(d, 2)) return fail(QGEMV_E_ALIGN, "d must be 2-byte aligned");
    if (!aligned(s, 4)) return fail(QGEMV_E_ALIGN, "s must be 4-byte aligned");
    return QGEMV_OK;
}

const char* fmt_name(int fmt) {
    switch (fmt) {
    case QGEMV_FMT_Q4_0: return "qgemv_q4_0";
    case QGEMV_FMT_Q4_K: return "qgemv_q4_k";
    case QGEMV_FMT_Q6_K: return "qgemv_q6_k";
    case QGEMV_FMT_Q8_0: return "qgemv_q8_0";
    case QGEMV_FMT_Q6_K_R8: return "qgemv_q6_k_r8";
    default: return "qgemv";
    }
}

qgemv_status gemv_common(int fmt, const void* w, int64_t N, int64_t K, const int8_t* q,
                         const uint16_t* d, const int32_t* s, float* y, qgemv_stream_t stream) {
    const char* name = fmt_name(fmt);
    if (N < 0) return fail(QGEMV_E_SHAPE, "%s: N = %lld is negative", name, (long long)N);
    if (N == 0) return ok();
    if (!w || !q || !d || !s || !y) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (N > INT32_MAX) return fail(QGEMV_E_SHAPE, "%s: N = %lld exceeds 2^31-1", name, (long long)N);
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX = %d", name,
                    (long long)K, QGEMV_K_MAX);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if (!aligned(y, 4)) return fail(QGEMV_E_ALIGN, "%s: y must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    const qgemv::GemvArgs a{w, N, K, q, d, s, y};
    return launched(qgemv::launch_gemv(fmt, a, (hipStream_t)stream), name);
}

qgemv_status small_m_common(int fmt, const char* name, const void* w, int64_t N, int64_t K,
                            int64_t M, const int8_t* q, const uint16_t* d, const int32_t* s,
                            float* y, int variant, qgemv_stream_t stream) {
    if (N < 0 || M < 0) return fail(QGEMV_E_SHAPE, "%s: negative N or M", name);
    if (N == 0 || M == 0) return ok();
    if (!w || !q || !d || !s || !y) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (N > INT32_MAX) return fail(QGEMV_E_SHAPE, "%s: N exceeds 2^31-1", name);
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX", name, (long long)K);
    if (M > QGEMV_M_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: M = %lld exceeds QGEMV_M_MAX = %d", name,
                    (long long)M, QGEMV_M_MAX);
    if (variant != QGEMV_VARIANT_AUTO && variant != QGEMV_VARIANT_DOT4 &&
        variant != QGEMV_VARIANT_MFMA && variant != QGEMV_VARIANT_MFMA_STAGED &&
        variant != QGEMV_VARIANT_MFMA_STREAM && variant != QGEMV_VARIANT_MFMA_RESIDENT)
        return fail(QGEMV_E_UNSUPPORTED, "%s: unknown variant %d", name, variant);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if (!aligned(y, 4)) return fail(QGEMV_E_ALIGN, "%s: y must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_small_m(fmt, w, N, K, M, q, d, s, y, variant,
                                          (hipStream_t)stream),
                    name);
}

// Gates shared by the two fused gate|up entries; x == NULL for the one whose
// activation codes are given.
qgemv_status swiglu_common(const char* name, const void* w, int64_t N, int64_t K,
                           const float* x, const int8_t* q, const uint16_t* d, const int32_t* s,
                           int8_t* q_out, uint16_t* d_out, int32_t* s_out, float* gu, float* h,
                           qgemv_stream_t stream) {
    if (N < 0) return fail(QGEMV_E_SHAPE, "%s: N = %lld is negative", name, (long long)N);
    if (N == 0) return ok();
    if (!w || !q || !d || !s || !q_out || !d_out || !s_out)
        return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (N % 32 != 0)
        return fail(QGEMV_E_SHAPE, "%s: N = %lld must be a multiple of 32", name, (long long)N);
    if (2 * N > INT32_MAX)
        return fail(QGEMV_E_SHAPE, "%s: 2N = %lld exceeds 2^31-1", name, (long long)(2 * N));
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX = %d", name,
                    (long long)K, QGEMV_K_MAX);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if (x && !aligned(x, 16)) return fail(QGEMV_E_ALIGN, "%s: x must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if ((st = check_act_align(q_out, d_out, s_out)) != QGEMV_OK) return st;
    if (gu && !aligned(gu, 4)) return fail(QGEMV_E_ALIGN, "%s: gu must be 4-byte aligned", name);
    if (h && !aligned(h, 4)) return fail(QGEMV_E_ALIGN, "%s: h must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    const qgemv::GemvArgs a{w, 2 * N, K, q, d, s, nullptr};
    const qgemv::SwigluOut so{N, q_out, d_out, s_out, gu, h};
    if (!x) return launched(qgemv::launch_q4k_swiglu(a, so, (hipStream_t)stream), name);
    const qgemv::ActIn ai{x, const_cast<int8_t*>(q), const_cast<uint16_t*>(d),
                          const_cast<int32_t*>(s)};
    return launched(qgemv::launch_quantize_q4k_swiglu(a, so, ai, (hipStream_t)stream), name);
}

// Gates shared by the two multi-matrix entries; x == NULL for the one whose
// activation codes are given (q, d, s inputs), else q, d, s are outputs.
qgemv_status multi_common(const char* name, int fmt, int count, const void* const* w,
                          const int64_t* n, int64_t K, const float* x, const int8_t* q,
                          const uint16_t* d, const int32_t* s, float* const* y,
                          qgemv_stream_t stream) {
    if (count < 0) return fail(QGEMV_E_SHAPE, "%s: count = %d is negative", name, count);
    if (count == 0) return ok();
    if (!w || !n || !y) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    int64_t total = 0;
    for (int i = 0; i < count; i++) {
        if (n[i] < 0)
            return fail(QGEMV_E_SHAPE, "%s: n[%d] = %lld is negative", name, i, (long long)n[i]);
        total += n[i];
        if (total > INT32_MAX)
            return fail(QGEMV_E_SHAPE, "%s: %lld rows in all exceed 2^31-1", name,
                        (long long)total);
    }
    if (total == 0) return ok();
    if (!q || !d || !s) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    for (int i = 0; i < count; i++)
        if (n[i] > 0 && (!w[i] || !y[i]))
            return fail(QGEMV_E_NULL, "%s: NULL weights or output of matrix %d", name, i);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (fmt < QGEMV_FMT_Q4_0 || fmt > QGEMV_FMT_Q6_K_R8)
        return fail(QGEMV_E_UNSUPPORTED, "%s: unknown format %d", name, fmt);
    if (count > QGEMV_MULTI_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: count = %d exceeds QGEMV_MULTI_MAX = %d", name,
                    count, QGEMV_MULTI_MAX);
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX = %d", name,
                    (long long)K, QGEMV_K_MAX);
    for (int i = 0; i < count; i++) {
        if (n[i] > 0 && !aligned(w[i], 16))
            return fail(QGEMV_E_ALIGN, "%s: weights of matrix %d must be 16-byte aligned", name, i);
        if (n[i] > 0 && !aligned(y[i], 4))
            return fail(QGEMV_E_ALIGN, "%s: output of matrix %d must be 4-byte aligned", name, i);
    }
    if (x && !aligned(x, 16)) return fail(QGEMV_E_ALIGN, "%s: x must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if ((st = check_device()) != QGEMV_OK) return st;
    qgemv::MultiRows mr{};
    mr.count = count;
    mr.start[0] = 0;
    for (int i = 0; i < count; i++) {
        mr.start[i + 1] = mr.start[i] + (int)n[i];
        mr.w[i] = w[i];
        mr.y[i] = y[i];
    }
    for (int i = count; i < qgemv::kMultiMax; i++) {
        mr.start[i + 1] = mr.start[count];
        mr.w[i] = nullptr;
        mr.y[i] = nullptr;
    }
    if (!x) return launched(qgemv::launch_multi(fmt, mr, K, q, d, s, (hipStream_t)stream), name);
    const qgemv::ActIn ai{x, const_cast<int8_t*>(q), const_cast<uint16_t*>(d),
                          const_cast<int32_t*>(s)};
    return launched(qgemv::launch_quantize_multi(fmt, mr, K, ai, (hipStream_t)stream), name);
}

}  // namespace

namespace qgemv {
LaunchTimer& next_launch_timer() {
    static thread_local LaunchTimer t;
    return t;
}
}  // namespace qgemv

extern "C" {

int qgemv_abi_version(void) { return QGEMV_ABI_VERSION; }

const char* qgemv_status_str(int status) {
    switch (status) {
    case QGEMV_OK: return "QGEMV_OK";
    case QGEMV_E_NULL: return "QGEMV_E_NULL: a required pointer is NULL";
    case QGEMV_E_SHAPE: return "QGEMV_E_SHAPE: invalid size or stride";
    case QGEMV_E_UNSUPPORTED: return "QGEMV_E_UNSUPPORTED: valid but declined by this library";
    case QGEMV_E_ALIGN: return "QGEMV_E_ALIGN: misaligned pointer";
    case QGEMV_E_DEVICE: return "QGEMV_E_DEVICE: no usable gfx950 device";
    case QGEMV_E_LAUNCH: return "QGEMV_E_LAUNCH: kernel launch failed";
    default: return "QGEMV_E_UNKNOWN: unknown status code";
    }
}

const char* qgemv_build_info(void) {
    return "libqgemv abi=1 arch=gfx950 formats=q4_0,q4_k,q6_k,q8_0,q6_k_r8(repacked) act=int8/32+fp16+int32sum "
           "gemv=v_dot4_i32_i8,lds-row-stream,lds-dynamic-rows(+row-pairs),direct-loads,lanes-per-row{4,8,16,32,64} "
           "small_m=q4_k{dot4,mfma_i8_16x16x32(staged,wave-stream,register-resident)},"
           "q6_k/q4_0{dot4_multirow(2|4),mfma_i8_16x16x32(staged,wave-stream)},"
           "two-block_tiles_mfma_i8_16x16x64(M<=8) "
           "block_dots=lds-rows,staged-stream,small_m_mfma_tiles "
           "fused=q4_k_swiglu_quantize,quantize_gemv,quantize_q4_k_swiglu multi=multi,quantize_multi(<=8) "
           "stream_read=calibration K_max=32768 M_max=64";
}

const char* qgemv_last_error(void) { return g_last_error; }

qgemv_status qgemv_time_next_launch(void* start, void* stop) {
    qgemv::next_launch_timer() = {(hipEvent_t)start, (hipEvent_t)stop};
    return QGEMV_OK;
}

qgemv_status qgemv_stream_read(const void* buf, int64_t bytes, int nontemporal, uint32_t* sink,
                               int wg_per_cu, qgemv_stream_t stream) {
    const char* name = "qgemv_stream_read";
    if (!buf || !sink) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    if (bytes < 16 || bytes % 16 != 0)
        return fail(QGEMV_E_SHAPE, "%s: bytes = %lld must be a positive multiple of 16", name,
                    (long long)bytes);
    if (wg_per_cu < 1 || wg_per_cu > 32)
        return fail(QGEMV_E_UNSUPPORTED, "%s: wg_per_cu = %d outside 1..32", name, wg_per_cu);
    if (!aligned(buf, 16)) return fail(QGEMV_E_ALIGN, "%s: buf must be 16-byte aligned", name);
    if (!aligned(sink, 4)) return fail(QGEMV_E_ALIGN, "%s: sink must be 4-byte aligned", name);
    qgemv_status st = check_device();
    if (st != QGEMV_OK) return st;
    return launched(qgemv::launch_stream_read(buf, bytes, nontemporal, sink, wg_per_cu,
                                              (hipStream_t)stream),
                    name);
}

qgemv_status qgemv_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                uint16_t* d, int32_t* s, qgemv_stream_t stream) {
    if (M < 0) return fail(QGEMV_E_SHAPE, "qgemv_quantize_act: M = %lld is negative", (long long)M);
    if (M == 0) return ok();
    if (!x || !q || !d || !s) return fail(QGEMV_E_NULL, "qgemv_quantize_act: NULL pointer argument");
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (ldx < K)
        return fail(QGEMV_E_SHAPE, "qgemv_quantize_act: ldx = %lld < K = %lld", (long long)ldx,
                    (long long)K);
    if (M > (int64_t)1 << 31 || ldx > (int64_t)1 << 40 || K > (int64_t)1 << 31)
        return fail(QGEMV_E_UNSUPPORTED, "qgemv_quantize_act: sizes beyond this library's range");
    const int64_t Kp = (K + 255) / 256 * 256;
    if (M * (Kp / 32) * 8 / 256 >= ((int64_t)1 << 31))
        return fail(QGEMV_E_UNSUPPORTED, "qgemv_quantize_act: M*K too large for one launch");
    if (!aligned(x, 4)) return fail(QGEMV_E_ALIGN, "qgemv_quantize_act: x must be 4-byte aligned");
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_quantize_act(x, M, K, ldx, q, d, s, (hipStream_t)stream),
                    "qgemv_quantize_act");
}

qgemv_status qgemv_q4_0(const void* w, int64_t N, int64_t K, const int8_t* q, const uint16_t* d,
                        const int32_t* s, float* y, qgemv_stream_t stream) {
    return gemv_common(QGEMV_FMT_Q4_0, w, N, K, q, d, s, y, stream);
}

qgemv_status qgemv_q4_k(const void* w, int64_t N, int64_t K, const int8_t* q, const uint16_t* d,
                        const int32_t* s, float* y, qgemv_stream_t stream) {
    return gemv_common(QGEMV_FMT_Q4_K, w, N, K, q, d, s, y, stream);
}

qgemv_status qgemv_q6_k(const void* w, int64_t N, int64_t K, const int8_t* q, const uint16_t* d,
                        const int32_t* s, float* y, qgemv_stream_t stream) {
    return gemv_common(QGEMV_FMT_Q6_K, w, N, K, q, d, s, y, stream);
}

qgemv_status qgemv_q8_0(const void* w, int64_t N, int64_t K, const int8_t* q, const uint16_t* d,
                        const int32_t* s, float* y, qgemv_stream_t stream) {
    return gemv_common(QGEMV_FMT_Q8_0, w, N, K, q, d, s, y, stream);
}

qgemv_status qgemv_q6_k_r8(const void* w_r, int64_t N, int64_t K, const int8_t* q,
                           const uint16_t* d, const int32_t* s, float* y, qgemv_stream_t stream) {
    return gemv_common(QGEMV_FMT_Q6_K_R8, w_r, N, K, q, d, s, y, stream);
}

qgemv_status qgemv_quantize_gemv(int fmt, const void* w, int64_t N, int64_t K, const float* x,
                                 int8_t* q, uint16_t* d, int32_t* s, float* y,
                                 qgemv_stream_t stream) {
    const char* name = "qgemv_quantize_gemv";
    if (N < 0) return fail(QGEMV_E_SHAPE, "%s: N = %lld is negative", name, (long long)N);
    if (N == 0) return ok();
    if (!w || !x || !q || !d || !s || !y)
        return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (N > INT32_MAX) return fail(QGEMV_E_SHAPE, "%s: N = %lld exceeds 2^31-1", name, (long long)N);
    if (fmt < QGEMV_FMT_Q4_0 || fmt > QGEMV_FMT_Q6_K_R8)
        return fail(QGEMV_E_UNSUPPORTED, "%s: unknown format %d", name, fmt);
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX = %d", name,
                    (long long)K, QGEMV_K_MAX);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if (!aligned(x, 16)) return fail(QGEMV_E_ALIGN, "%s: x must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if (!aligned(y, 4)) return fail(QGEMV_E_ALIGN, "%s: y must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    const qgemv::GemvArgs a{w, N, K, q, d, s, y};
    const qgemv::ActIn ai{x, q, d, s};
    return launched(qgemv::launch_quantize_gemv(fmt, a, ai, (hipStream_t)stream), name);
}

qgemv_status qgemv_q6_k_repack(const void* w, int64_t N, int64_t K, void* w_r,
                               qgemv_stream_t stream) {
    const char* name = "qgemv_q6_k_repack";
    if (N < 0) return fail(QGEMV_E_SHAPE, "%s: N = %lld is negative", name, (long long)N);
    if (N == 0) return ok();
    if (!w || !w_r) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (N > INT32_MAX) return fail(QGEMV_E_SHAPE, "%s: N = %lld exceeds 2^31-1", name, (long long)N);
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX = %d", name,
                    (long long)K, QGEMV_K_MAX);
    if (!aligned(w, 16) || !aligned(w_r, 16))
        return fail(QGEMV_E_ALIGN, "%s: w and w_r must be 16-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_q6k_repack(w, N, K, w_r, (hipStream_t)stream), name);
}

qgemv_status qgemm_q4_k_small_m(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                                const uint16_t* d, const int32_t* s, float* y, int variant,
                                qgemv_stream_t stream) {
    return small_m_common(QGEMV_FMT_Q4_K, "qgemm_q4_k_small_m", w, N, K, M, q, d, s, y, variant,
                          stream);
}

qgemv_status qgemm_q6_k_small_m(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                                const uint16_t* d, const int32_t* s, float* y, int variant,
                                qgemv_stream_t stream) {
    return small_m_common(QGEMV_FMT_Q6_K, "qgemm_q6_k_small_m", w, N, K, M, q, d, s, y, variant,
                          stream);
}

qgemv_status qgemm_q4_0_small_m(const void* w, int64_t N, int64_t K, int64_t M, const int8_t* q,
                                const uint16_t* d, const int32_t* s, float* y, int variant,
                                qgemv_stream_t stream) {
    return small_m_common(QGEMV_FMT_Q4_0, "qgemm_q4_0_small_m", w, N, K, M, q, d, s, y, variant,
                          stream);
}

qgemv_status qgemm_small_m_block_dots(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                                     const int8_t* q, const uint16_t* d, const int32_t* s,
                                     float* y, int variant, int32_t* dots,
                                     qgemv_stream_t stream) {
    const char* name = "qgemm_small_m_block_dots";
    if (N < 0 || M < 0) return fail(QGEMV_E_SHAPE, "%s: negative N or M", name);
    if (N == 0 || M == 0) return ok();
    if (!w || !q || !d || !s || !y || !dots)
        return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (N > INT32_MAX) return fail(QGEMV_E_SHAPE, "%s: N exceeds 2^31-1", name);
    if (fmt != QGEMV_FMT_Q4_K && fmt != QGEMV_FMT_Q6_K && fmt != QGEMV_FMT_Q4_0)
        return fail(QGEMV_E_UNSUPPORTED, "%s: format %d has no small-M product", name, fmt);
    if (K > QGEMV_K_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: K = %lld exceeds QGEMV_K_MAX", name, (long long)K);
    if (M > QGEMV_M_MAX)
        return fail(QGEMV_E_UNSUPPORTED, "%s: M = %lld exceeds QGEMV_M_MAX = %d", name,
                    (long long)M, QGEMV_M_MAX);
    if (variant != QGEMV_VARIANT_MFMA && variant != QGEMV_VARIANT_MFMA_STAGED &&
        variant != QGEMV_VARIANT_MFMA_RESIDENT)
        return fail(QGEMV_E_UNSUPPORTED,
                    "%s: variant %d: only the MFMA, MFMA_STAGED and MFMA_RESIDENT variants "
                    "have a dots mode", name, variant);
    if (variant != QGEMV_VARIANT_MFMA_STAGED && !qgemv::small_m_dots_supported(fmt, N, K, M, variant))
        return fail(QGEMV_E_UNSUPPORTED,
                    "%s: the kernel variant %d selects for this shape (the wave-stream "
                    "kernel) has no dots mode", name, variant);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if (!aligned(y, 4) || !aligned(dots, 4))
        return fail(QGEMV_E_ALIGN, "%s: y and dots must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_small_m_dots(fmt, w, N, K, M, q, d, s, y, variant, dots,
                                               (hipStream_t)stream),
                    name);
}

qgemv_status qgemv_silu_mul_quantize(const float* gu, int64_t N, int8_t* q, uint16_t* d,
                                     int32_t* s, float* h, qgemv_stream_t stream) {
    const char* name = "qgemv_silu_mul_quantize";
    if (N < 0) return fail(QGEMV_E_SHAPE, "%s: N is negative", name);
    if (N == 0) return ok();
    if (!gu || !q || !d || !s) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    if (N % 32 != 0)
        return fail(QGEMV_E_SHAPE, "%s: N = %lld must be a multiple of 32", name, (long long)N);
    if (N > (int64_t)1 << 31) return fail(QGEMV_E_UNSUPPORTED, "%s: N too large", name);
    if (!aligned(gu, 4)) return fail(QGEMV_E_ALIGN, "%s: gu must be 4-byte aligned", name);
    qgemv_status st = check_act_align(q, d, s);
    if (st != QGEMV_OK) return st;
    if (h && !aligned(h, 4)) return fail(QGEMV_E_ALIGN, "%s: h must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_silu_mul_quantize(gu, N, q, d, s, h, (hipStream_t)stream), name);
}

qgemv_status qgemv_q4_k_swiglu_quantize(const void* w, int64_t N, int64_t K, const int8_t* q,
                                        const uint16_t* d, const int32_t* s, int8_t* q_out,
                                        uint16_t* d_out, int32_t* s_out, float* gu, float* h,
                                        qgemv_stream_t stream) {
    return swiglu_common("qgemv_q4_k_swiglu_quantize", w, N, K, nullptr, q, d, s, q_out, d_out,
                         s_out, gu, h, stream);
}

qgemv_status qgemv_quantize_q4_k_swiglu(const void* w, int64_t N, int64_t K, const float* x,
                                        int8_t* q, uint16_t* d, int32_t* s, int8_t* q_out,
                                        uint16_t* d_out, int32_t* s_out, float* gu, float* h,
                                        qgemv_stream_t stream) {
    const char* name = "qgemv_quantize_q4_k_swiglu";
    if (N > 0 && !x) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    return swiglu_common(name, w, N, K, x, q, d, s, q_out, d_out, s_out, gu, h, stream);
}

qgemv_status qgemv_multi(int fmt, int count, const void* const* w, const int64_t* n, int64_t K,
                         const int8_t* q, const uint16_t* d, const int32_t* s, float* const* y,
                         qgemv_stream_t stream) {
    return multi_common("qgemv_multi", fmt, count, w, n, K, nullptr, q, d, s, y, stream);
}

qgemv_status qgemv_quantize_multi(int fmt, int count, const void* const* w, const int64_t* n,
                                  int64_t K, const float* x, int8_t* q, uint16_t* d, int32_t* s,
                                  float* const* y, qgemv_stream_t stream) {
    const char* name = "qgemv_quantize_multi";
    if (count > 0 && !x) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    return multi_common(name, fmt, count, w, n, K, x, q, d, s, y, stream);
}

qgemv_status qgemv_block_dots(int fmt, const void* w, int64_t N, int64_t K, int64_t row0,
                              int64_t nrows, const int8_t* q, int32_t* dots,
                              qgemv_stream_t stream) {
    const char* name = "qgemv_block_dots";
    if (N < 0 || row0 < 0 || nrows < 0 || row0 > N || nrows > N - row0)
        return fail(QGEMV_E_SHAPE, "%s: rows [%lld, %lld) outside [0, %lld)", name,
                    (long long)row0, (long long)(row0 + nrows), (long long)N);
    if (nrows == 0) return ok();
    if (!w || !q || !dots) return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (fmt < QGEMV_FMT_Q4_0 || fmt > QGEMV_FMT_Q6_K_R8)
        return fail(QGEMV_E_UNSUPPORTED, "%s: unknown format %d", name, fmt);
    if (K > QGEMV_K_MAX) return fail(QGEMV_E_UNSUPPORTED, "%s: K exceeds QGEMV_K_MAX", name);
    if (nrows * ((K + 255) / 64) / 256 >= ((int64_t)1 << 31))
        return fail(QGEMV_E_UNSUPPORTED, "%s: too many rows for one launch", name);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if (!aligned(q, 16)) return fail(QGEMV_E_ALIGN, "%s: q must be 16-byte aligned", name);
    if (!aligned(dots, 4)) return fail(QGEMV_E_ALIGN, "%s: dots must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_block_dots(fmt, w, K, row0, nrows, q, dots, (hipStream_t)stream),
                    name);
}

qgemv_status qgemv_block_dots_staged(int fmt, const void* w, int64_t N, int64_t K,
                                     int64_t row0, int64_t nrows, const int8_t* q,
                                     const uint16_t* d, const int32_t* s, int wk,
                                     int32_t* dots, qgemv_stream_t stream) {
    const char* name = "qgemv_block_dots_staged";
    if (N < 0 || row0 < 0 || nrows < 0 || row0 > N || nrows > N - row0)
        return fail(QGEMV_E_SHAPE, "%s: rows [%lld, %lld) outside [0, %lld)", name,
                    (long long)row0, (long long)(row0 + nrows), (long long)N);
    if (nrows == 0) return ok();
    if (!w || !q || !d || !s || !dots)
        return fail(QGEMV_E_NULL, "%s: NULL pointer argument", name);
    qgemv_status st = check_k(K);
    if (st != QGEMV_OK) return st;
    if (fmt < QGEMV_FMT_Q4_0 || fmt > QGEMV_FMT_Q6_K_R8)
        return fail(QGEMV_E_UNSUPPORTED, "%s: unknown format %d", name, fmt);
    if (K > QGEMV_K_MAX) return fail(QGEMV_E_UNSUPPORTED, "%s: K exceeds QGEMV_K_MAX", name);
    if (nrows * 4 >= ((int64_t)1 << 31))
        return fail(QGEMV_E_UNSUPPORTED, "%s: too many rows for one launch", name);
    if (!qgemv::block_dots_staged_supported(fmt, K, wk))
        return fail(QGEMV_E_UNSUPPORTED,
                    "%s: split-K width %d with K = %lld has no staged configuration (wk in "
                    "1, 2, 4; at most 128 units per slice)",
                    name, wk, (long long)K);
    if (!aligned(w, 16)) return fail(QGEMV_E_ALIGN, "%s: w must be 16-byte aligned", name);
    if ((st = check_act_align(q, d, s)) != QGEMV_OK) return st;
    if (!aligned(dots, 4)) return fail(QGEMV_E_ALIGN, "%s: dots must be 4-byte aligned", name);
    if ((st = check_device()) != QGEMV_OK) return st;
    return launched(qgemv::launch_block_dots_staged(fmt, w, K, row0, nrows, q, d, s, wk, dots,
                                                    (hipStream_t)stream),
                    name);
}

}  // extern "C"
