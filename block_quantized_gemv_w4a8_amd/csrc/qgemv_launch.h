// qgemv_launch.h -- internal interface between the C-ABI layer (qgemv_api.cpp)
// and the kernel translation units.  Arguments reaching these launchers have
// already passed every gate of the public entry points.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qgemv {

// Events that the next kernel launched from this host thread records at its
// start and end (set by qgemv_time_next_launch; both NULL when disarmed).
struct LaunchTimer {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTimer& next_launch_timer();

// Every kernel of the library is launched through here: a plain launch, or,
// when the calling thread is armed, one that records the timer's events
// around the kernel and disarms the thread.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned smem,
                          hipStream_t st, Args... args) {
    LaunchTimer& t = next_launch_timer();
    if (t.start || t.stop) {
        const LaunchTimer use = t;
        t = LaunchTimer{};
        hipExtLaunchKernelGGL(kernel, grid, block, smem, st, use.start, use.stop, 0u,
                              static_cast<KArgs>(args)...);
    } else {
        kernel<<<grid, block, smem, st>>>(static_cast<KArgs>(args)...);
    }
}

struct GemvArgs {
    const void* w;
    int64_t N, K;
    const int8_t* q;
    const uint16_t* d;
    const int32_t* s;
    float* y;
};

// Outputs of the fused gate|up -> SwiGLU -> quantise product: the activation
// of the next product (nh values, padded to whole super-blocks of 256) and,
// where not NULL, the fp32 [gate | up] products and h.
struct SwigluOut {
    int64_t nh;
    int8_t* q;
    uint16_t* d;
    int32_t* s;
    float* gu;
    float* h;
};

// An fp32 activation row x [K] (16-byte aligned) quantised inside the
// product's own launch: every workgroup forms the codes of x in its LDS and
// workgroup 0 also writes them to q [Kp], d [Kp/32], s [Kp/32], exactly as
// launch_quantize_act would.
struct ActIn {
    const float* x;
    int8_t* q;
    uint16_t* d;
    int32_t* s;
};

// Several matrices of one format and K that share one activation row, seen
// as one range of rows: matrix i holds rows start[i] .. start[i + 1] - 1.
constexpr int kMultiMax = 8;
struct MultiRows {
    int count;
    int start[kMultiMax + 1];
    const void* w[kMultiMax];
    float* y[kMultiMax];
};

hipError_t launch_gemv(int fmt, const GemvArgs& a, hipStream_t st);
// The GEMVs of mr on one activation row (q, d, s), in one launch where the
// rows take the lanes-per-row kernel, else one launch per matrix.
hipError_t launch_multi(int fmt, const MultiRows& mr, int64_t K, const int8_t* q,
                        const uint16_t* d, const int32_t* s, hipStream_t st);
// The same with the activation quantised from ai.x in the launch.
hipError_t launch_quantize_multi(int fmt, const MultiRows& mr, int64_t K, const ActIn& ai,
                                 hipStream_t st);
// launch_quantize_act on ai then launch_gemv on its codes, in one launch
// where the kernel's LDS also holds the quantised row (else in those two
// launches)
hipError_t launch_quantize_gemv(int fmt, const GemvArgs& a, const ActIn& ai, hipStream_t st);
hipError_t launch_q6k_repack(const void* w, int64_t N, int64_t K, void* wr, hipStream_t st);
hipError_t launch_q4k_swiglu(const GemvArgs& a, const SwigluOut& so, hipStream_t st);
// the same with the gate|up activation quantised from ai.x in the launch
hipError_t launch_quantize_q4k_swiglu(const GemvArgs& a, const SwigluOut& so, const ActIn& ai,
                                      hipStream_t st);
hipError_t launch_block_dots(int fmt, const void* w, int64_t K, int64_t row0, int64_t nrows,
                             const int8_t* q, int32_t* dots, hipStream_t st);
// The same through the LDS-streaming loaders with split-K width wk (1, 2,
// 4); supported says whether (fmt, K, wk) has a configuration.
bool block_dots_staged_supported(int fmt, int64_t K, int wk);
hipError_t launch_block_dots_staged(int fmt, const void* w, int64_t K, int64_t row0,
                                    int64_t nrows, const int8_t* q, const uint16_t* d,
                                    const int32_t* s, int wk, int32_t* dots, hipStream_t st);
hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               uint16_t* d, int32_t* s, hipStream_t st);
hipError_t launch_silu_mul_quantize(const float* gu, int64_t N, int8_t* q, uint16_t* d,
                                    int32_t* s, float* h, hipStream_t st);
// fmt: QGEMV_FMT_Q4_K, QGEMV_FMT_Q6_K or QGEMV_FMT_Q4_0
hipError_t launch_small_m(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                          const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                          int variant, hipStream_t st);

// The small-M product through the batch-1 dynamic-row streaming kernel with
// up to four activation rows per pass over the weights (fmt: QGEMV_FMT_Q4_K,
// QGEMV_FMT_Q6_K or QGEMV_FMT_Q4_0; M >= 2).  hipErrorNotSupported (nothing
// launched) for rows of more than 256 units or slices too long for its
// buffers.
hipError_t launch_small_m_rows(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                               const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                               hipStream_t st);

// The small-M product on int8 matrix cores with each wave's slice of the
// activation resident in registers (Q4_K, 1 <= M <= 16, K <= 16384: where
// small_m3_supported; else hipErrorNotSupported, nothing launched).
bool small_m3_supported(int fmt, int64_t K, int64_t M);
hipError_t launch_small_m3(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                           const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                           hipStream_t st);
// the same kernel also storing its raw int32 MFMA tiles to dots (validation)
hipError_t launch_small_m3_dots(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                                const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                                int32_t* dots, hipStream_t st);
// Validation: the small-M product of variant (MFMA, MFMA_STAGED or
// MFMA_RESIDENT) run by the kernel that variant selects, storing every raw
// int32 MFMA tile to dots [M][N][nb] as well as y; hipErrorNotSupported
// (nothing launched) where that kernel has no such mode.
bool small_m_dots_supported(int fmt, int64_t N, int64_t K, int64_t M, int variant);
hipError_t launch_small_m_dots(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                               const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                               int variant, int32_t* dots, hipStream_t st);

// The small-M product on int8 matrix cores with wave-private weight streams
// (fmt: QGEMV_FMT_Q4_K, QGEMV_FMT_Q6_K or QGEMV_FMT_Q4_0; 1 <= M <= 64).
hipError_t launch_small_m2(int fmt, const void* w, int64_t N, int64_t K, int64_t M,
                           const int8_t* q, const uint16_t* d, const int32_t* s, float* y,
                           hipStream_t st);

// Measurement aid: a plain streaming read of `bytes` (a multiple of 16) at
// buf with 16-byte loads (non-temporal if asked), wg_per_cu workgroups per
// compute unit.
hipError_t launch_stream_read(const void* buf, int64_t bytes, int nontemporal, uint32_t* sink,
                              int wg_per_cu, hipStream_t st);

}  // namespace qgemv
